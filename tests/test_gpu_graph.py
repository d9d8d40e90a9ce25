"""HIP graph capture of the decode path: a captured index_topk + sparse_attn
(and a pool-restricted index_topk + hca_dense_attn layer) replayed several
times, with unrelated eager work and synchronisations between the replays,
must reproduce the eager results bit for bit on every replay (every kernel
of the path is deterministic). The eager results are checked against the
oracle on a sample of queries."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import compressed_sparse_attention_compress_amd as csa
import oracle.csa_oracle as O
import synth
from parity_util import REL_TOL, attn_excess_error, bf16_bits, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def _world(seed, B, L, d, H, m, Hi, Di, Wcap=128):
    g = synth.generator(DEV, seed, "graph", B, L)
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


def test_graph_replay_decode():
    B, L, d, H, m, Hi, Di, k, pool_k, W = 4, 4 * 12000, 512, 64, 4, 8, 64, 384, 1024, 128
    t = L - 1
    x = _world(3, B, L, d, H, m, Hi, Di)
    hca_m = 64
    h_codes = torch.empty(B, -(-L // hca_m), d // 2, device=DEV, dtype=torch.uint8)
    h_scales = torch.empty(B, -(-L // hca_m), d // 32, device=DEV, dtype=torch.uint8)
    g = synth.generator(DEV, 4, "graph-hca")
    csa.compress_quantize(torch.randn(B, L, d, generator=g, device=DEV),
                          torch.randn(B, L, generator=g, device=DEV), 0, hca_m, h_codes, h_scales)
    ws, ws_a = csa.Workspace(DEV), csa.Workspace(DEV)
    idx = torch.empty(B, 1, k, device=DEV, dtype=torch.int32)
    pool = torch.empty(B, 1, pool_k, device=DEV, dtype=torch.int32)
    ridx = torch.empty(B, 1, k, device=DEV, dtype=torch.int32)
    out = torch.empty(B, 1, H, d, device=DEV, dtype=torch.bfloat16)
    rout = torch.empty(B, 1, H, d, device=DEV, dtype=torch.bfloat16)
    hout = torch.empty(B, 1, H, d, device=DEV, dtype=torch.float32)
    lse = torch.empty(B, 1, H, device=DEV, dtype=torch.float32)

    def step():
        csa.index_topk(x["q_idx"], x["w"], x["keys"], m, t, k, idx, workspace=ws)
        csa.sparse_attn(x["q"], x["codes"], x["scales"], idx, x["win"], W, t, 1.0, out, lse,
                        workspace=ws_a)
        csa.index_topk(x["q_idx"], x["w"], x["keys"], m, t, pool_k, pool, workspace=ws)
        csa.index_topk(x["q_idx"], x["w"], x["keys"], m, t, k, ridx, cand=pool, workspace=ws)
        csa.sparse_attn(x["q"], x["codes"], x["scales"], ridx, x["win"], W, t, 0.5, rout,
                        workspace=ws_a)
        csa.hca_dense_attn(x["q"], h_codes, h_scales, hca_m, x["win"], W, t, 1.0, hout,
                           workspace=ws_a)

    bufs = [idx, pool, ridx, out, rout, hout, lse]
    step()
    torch.cuda.synchronize()
    ref = [b.clone() for b in bufs]
    # the pool-restricted top-k of a pool that holds the whole top-k is the top-k
    assert torch.equal(ridx, idx)
    say("capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    other = _world(5, B, L, d, H, m, Hi, Di)
    o_idx = torch.empty_like(idx)
    o_out = torch.empty_like(out)
    for r in range(4):
        for b in bufs:
            b.fill_(-3)
        graph.replay()
        torch.cuda.synchronize()
        for name, b, e in zip(["idx", "pool", "ridx", "out", "rout", "hout", "lse"], bufs, ref):
            assert torch.equal(b, e), (r, name)
        # unrelated eager work on the same workspaces between replays
        csa.index_topk(other["q_idx"], other["w"], other["keys"], m, t - 5, k, o_idx,
                       workspace=ws)
        csa.sparse_attn(other["q"], other["codes"], other["scales"], o_idx, other["win"], W,
                        t - 5, 1.0, o_out, workspace=ws_a)
        torch.cuda.synchronize()
        say(f"  replay {r} identical")

    # the eager results against the oracle, first two sequences
    kn, cn, sn = x["keys"].cpu().numpy(), x["codes"].cpu().numpy(), x["scales"].cpu().numpy()
    hcn, hsn = h_codes.cpu().numpy(), h_scales.cpu().numpy()
    qin, wn = x["q_idx"].cpu().numpy(), x["w"].cpu().numpy()
    qb, winb = bf16_bits(x["q"]), bf16_bits(x["win"])
    for b in range(2):
        ri, _ = O.index_topk(qin[b, 0], wn[b, 0], kn[b], m, t, k)
        assert np.array_equal(ref[0][b, 0].cpu().numpy(), ri)
        rp, _ = O.index_topk(qin[b, 0], wn[b, 0], kn[b], m, t, pool_k)
        assert np.array_equal(ref[1][b, 0].cpu().numpy(), rp)
        o, _ = O.sparse_attn(qb[b, 0], cn[b], sn[b], ri, winb[b], winb.shape[1], W, t, 1.0)
        ex, _ = attn_excess_error(to_np(ref[3])[b, 0][None], o[None], True)
        assert ex <= REL_TOL, ex
        o, _ = O.hca_dense_attn(qb[b, 0], hcn[b], hsn[b], hca_m, winb[b], winb.shape[1], W, t, 1.0)
        ex, _ = attn_excess_error(to_np(ref[5])[b, 0][None], o[None], False)
        assert ex <= REL_TOL, ex


def test_prepared_calls_replay():
    """csa.prepare records a step's launches with their marshalled arguments;
    replaying them reproduces the eager results bit for bit, also after other
    calls have used the same workspaces, and recording issues nothing."""
    B, L, d, H, m, Hi, Di, k, W = 2, 4 * 6000, 512, 64, 4, 8, 64, 256, 128
    t = L - 1
    x = _world(6, B, L, d, H, m, Hi, Di)
    ws, ws_a = csa.Workspace(DEV), csa.Workspace(DEV)
    idx = torch.full((B, 1, k), -5, device=DEV, dtype=torch.int32)
    out = torch.zeros(B, 1, H, d, device=DEV, dtype=torch.bfloat16)

    def step():
        csa.index_topk(x["q_idx"], x["w"], x["keys"], m, t, k, idx, workspace=ws)
        csa.sparse_attn(x["q"], x["codes"], x["scales"], idx, x["win"], W, t, 1.0, out,
                        workspace=ws_a)

    run = csa.prepare(step)
    torch.cuda.synchronize()
    assert (idx == -5).all() and (out == 0).all()   # nothing was issued while recording
    step()
    torch.cuda.synchronize()
    ref_i, ref_o = idx.clone(), out.clone()
    other = _world(7, B, L, d, H, m, Hi, Di)
    o_idx = torch.empty_like(idx)
    for r in range(3):
        idx.fill_(-3)
        out.fill_(7)
        run()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_i) and torch.equal(out, ref_o), r
        csa.index_topk(other["q_idx"], other["w"], other["keys"], m, t - 9, k, o_idx, workspace=ws)
    kn, qin, wn = x["keys"].cpu().numpy(), x["q_idx"].cpu().numpy(), x["w"].cpu().numpy()
    for b in range(B):
        ri, _ = O.index_topk(qin[b, 0], wn[b, 0], kn[b], m, t, k)
        assert np.array_equal(ref_i[b, 0].cpu().numpy(), ri)


def test_prepared_replay_keeps_buffers_and_workspace_state():
    """A recording made with no attention workspace keeps its temporary
    alive; growing the index workspace afterwards, and an eager call at a
    different B*T on the recorded buffer (whose body then overlaps the
    recorded layout's head), leave every replay correct: the head is
    re-cleared for the recorded layout before the recorded index call."""
    B, L, d, H, m, Hi, Di, k, W = 4, 4 * 6000, 512, 64, 4, 8, 64, 256, 128
    t = L - 1
    x = _world(8, B, L, d, H, m, Hi, Di)
    ws = csa.Workspace(DEV)
    idx = torch.empty(B, 1, k, device=DEV, dtype=torch.int32)
    out = torch.empty(B, 1, H, d, device=DEV, dtype=torch.bfloat16)

    def step():
        csa.index_topk(x["q_idx"], x["w"], x["keys"], m, t, k, idx, workspace=ws)
        csa.sparse_attn(x["q"], x["codes"], x["scales"], idx, x["win"], W, t, 1.0, out)

    step()
    torch.cuda.synchronize()
    ref_i, ref_o = idx.clone(), out.clone()
    run = csa.prepare(step)
    buf0 = ws.buf
    # a longer context grows the workspace (a new buffer)
    big = _world(9, 3, 4 * 20000, d, H, m, Hi, Di)
    o_idx = torch.empty(3, 1, k, device=DEV, dtype=torch.int32)
    csa.index_topk(big["q_idx"], big["w"], big["keys"], m, 4 * 20000 - 1, k, o_idx, workspace=ws)
    assert ws.buf is not buf0
    # allocations that could reuse freed memory, then replays
    junk = [torch.full((1 << 20,), 7, device=DEV, dtype=torch.int32) for _ in range(8)]
    one = csa.Workspace(DEV)
    one.buf = buf0
    i1 = torch.empty(1, 1, k, device=DEV, dtype=torch.int32)
    for r in range(3):
        idx.fill_(-3)
        out.fill_(5)
        run()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_i) and torch.equal(out, ref_o), r
        # an eager call of one sequence (B*T = 1) on the recorded buffer
        csa.index_topk(x["q_idx"][:1].contiguous(), x["w"][:1].contiguous(),
                       x["keys"][:1].contiguous(), m, t - 3 * r, k, i1, workspace=one)
        assert one.buf is buf0
    del junk
