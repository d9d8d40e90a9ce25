"""csa_sparse_attn_noalloc (the split partials in the library's static device
scratch, no workspace) against csa_sparse_attn with a caller workspace: the
same kernels run, so outputs and log-sum-exps must be bit-identical. Two
calls in a row, the second with a smaller batch, fewer entries and another
position, so the second reuses scratch the first left behind."""

from __future__ import annotations

import math

import pytest
import torch

import compressed_sparse_attention_compress_amd as csa
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def _world(seed, B, L, d, H, m, Hi, Di, Wcap=256):
    g = synth.generator(DEV, seed, "noalloc", B, L)
    kv = torch.randn(B, L, d, generator=g, device=DEV)
    gate = torch.randn(B, L, generator=g, device=DEV)
    cap = -(-L // m)
    codes = torch.empty(B, cap, d // 2, device=DEV, dtype=torch.uint8)
    scales = torch.empty(B, cap, d // 32, device=DEV, dtype=torch.uint8)
    csa.compress_quantize(kv, gate, 0, m, codes, scales)
    win = torch.zeros(B, Wcap, d, device=DEV, dtype=torch.bfloat16)
    t0 = max(0, L - Wcap)
    win[:, torch.arange(t0, L, device=DEV) % Wcap] = kv[:, t0:L].to(torch.bfloat16)
    q = (torch.randn(B, 1, H, d, generator=g, device=DEV) / math.sqrt(d)).to(torch.bfloat16)
    q_idx = torch.randint(-8, 8, (B, 1, Hi, Di), generator=g, device=DEV, dtype=torch.int8)
    w = torch.randint(0, 4, (B, 1, Hi), generator=g, device=DEV, dtype=torch.int8)
    keys = torch.randint(-8, 8, (B, cap, Di), generator=g, device=DEV, dtype=torch.int8)
    return dict(codes=codes, scales=scales, win=win, q=q, q_idx=q_idx, w=w, keys=keys)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_call(out_dtype):
    d, H, m, Hi, Di, W = 512, 64, 4, 8, 64, 128
    # (B, L, k, position offset from the end): the second call is smaller
    cases = [(8, 4 * 6000, 1024, 0), (3, 4 * 2500, 256, 7)]
    for i, (B, L, k, back) in enumerate(cases):
        say(f"noalloc call {i}: B={B} L={L} k={k} out={out_dtype}")
        x = _world(10 + i, B, L, d, H, m, Hi, Di)
        t = L - 1 - back
        idx = torch.empty(B, 1, k, device=DEV, dtype=torch.int32)
        csa.index_topk(x["q_idx"], x["w"], x["keys"], m, t, k, idx)
        need = csa.attn_workspace(B, 1, H, d, k + W)
        assert 0 < need <= csa.NOALLOC_SCRATCH_MAX
        ref = torch.empty(B, 1, H, d, device=DEV, dtype=out_dtype)
        ref_lse = torch.empty(B, 1, H, device=DEV, dtype=torch.float32)
        ws = torch.empty(need + 256, device=DEV, dtype=torch.uint8)
        csa.sparse_attn(x["q"], x["codes"], x["scales"], idx, x["win"], W, t, 1.0, ref,
                        lse=ref_lse, workspace=ws)
        got = torch.full_like(ref, 3.0)
        got_lse = torch.full_like(ref_lse, 3.0)
        csa.sparse_attn_noalloc(x["q"], x["codes"], x["scales"], idx, x["win"], W, t, 1.0, got,
                                lse=got_lse)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), i
        assert torch.equal(got_lse, ref_lse), i
        assert torch.isfinite(ref.float()).all()
        say(f"  call {i} bit-identical")


def test_noalloc_many_queries_no_split():
    """A run of 16 queries per sequence needs no scratch (one workgroup per
    query); the no-alloc call must still match."""
    B, L, d, H, m, Hi, Di, W, T, k = 2, 4 * 1500, 512, 64, 4, 8, 64, 128, 16, 128
    x = _world(20, B, L, d, H, m, Hi, Di)
    g = synth.generator(DEV, 21, "noalloc-q")
    q = (torch.randn(B, T, H, d, generator=g, device=DEV) / math.sqrt(d)).to(torch.bfloat16)
    q_idx = torch.randint(-8, 8, (B, T, Hi, Di), generator=g, device=DEV, dtype=torch.int8)
    w = torch.randint(0, 4, (B, T, Hi), generator=g, device=DEV, dtype=torch.int8)
    pos0 = L - T
    idx = torch.empty(B, T, k, device=DEV, dtype=torch.int32)
    csa.index_topk(q_idx, w, x["keys"], m, pos0, k, idx)
    assert csa.attn_workspace(B, T, H, d, k + W) == 0
    ref = torch.empty(B, T, H, d, device=DEV, dtype=torch.bfloat16)
    csa.sparse_attn(q, x["codes"], x["scales"], idx, x["win"], W, pos0, 1.0, ref)
    got = torch.zeros_like(ref)
    csa.sparse_attn_noalloc(q, x["codes"], x["scales"], idx, x["win"], W, pos0, 1.0, got)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
