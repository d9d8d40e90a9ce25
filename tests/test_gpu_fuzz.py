"""Seeded random sweep of the indexer and attention calls over small shapes:
every combination the launch plans branch on (heads and key widths, query
runs below and above the batched-scan threshold, contexts below and above
the one-workgroup select limit, candidate pools, per-sequence positions,
both cache scale formats, bfloat16 and float32 outputs) drawn from one
seeded generator, each case checked against the oracle (bit-exact top-k,
attention within 2e-3 x RMS beyond the output rounding)."""

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
N_CASES = 96


def _case(rng):
    """One random configuration (plain ints, so the case prints compactly)."""
    Hi = int(rng.choice([1, 2, 4, 5, 8, 16]))
    Di = int(rng.choice([32, 64, 128]))
    if Hi * Di > 1024:
        Hi = 1024 // Di
    m = int(rng.choice([1, 3, 4]))
    B = int(rng.integers(1, 4))
    T = int(rng.choice([1, 2, 5, 16, 23]))
    n_vis = int(rng.choice([0, 7, 300, 2047, 2049, 6000, 8192, 9000]))
    pos0 = max(0, (n_vis + 1) * m - 1 - T // 2)
    k = int(rng.choice([1, 16, 100, 512, 1200]))
    ragged = bool(rng.integers(0, 2))
    cand_C = int(rng.choice([0, 0, 64, 900, 4096, 5000])) if T <= 2 else 0
    fmt = str(rng.choice(["e8m0", "e4m3"]))
    d, H = (int(rng.choice([128, 256, 512])), int(rng.choice([8, 20, 64])))
    out_f32 = bool(rng.integers(0, 2))
    return dict(Hi=Hi, Di=Di, m=m, B=B, T=T, pos0=pos0, k=k, ragged=ragged, cand_C=cand_C,
                fmt=fmt, d=d, H=H, out_f32=out_f32)


@pytest.mark.parametrize("case_id", range(N_CASES))
def test_random_case(case_id):
    rng = np.random.default_rng(1000 + case_id)
    c = _case(rng)
    print("case", case_id, c, flush=True)
    B, T, Hi, Di, m, k, d, H = c["B"], c["T"], c["Hi"], c["Di"], c["m"], c["k"], c["d"], c["H"]
    g = synth.generator(DEV, case_id, "fuzz")
    pos_max = c["pos0"]
    if c["ragged"]:
        pos = [int(x) for x in rng.integers(0, pos_max + 1, B)]
        pos[0] = pos_max
    else:
        pos = [pos_max] * B
    L = pos_max + T                      # tokens the caches must hold
    blk_cap = L // m + 2
    # indexer
    q_idx = torch.randint(-8, 8, (B, T, Hi, Di), generator=g, device=DEV, dtype=torch.int8)
    w = torch.randint(0, 4, (B, T, Hi), generator=g, device=DEV, dtype=torch.int8)
    keys = torch.randint(-8, 8, (B, blk_cap, Di), generator=g, device=DEV, dtype=torch.int8)
    cand = None
    if c["cand_C"]:
        C = c["cand_C"]
        cand = torch.stack([torch.sort(torch.randperm(max(blk_cap, C), generator=g,
                                                      device=DEV)[:C])[0]
                            for _ in range(B * T)]).reshape(B, T, C).to(torch.int32)
        cand = torch.where(cand >= blk_cap, torch.full_like(cand, -1), cand)
    idx = torch.full((B, T, k), -7, device=DEV, dtype=torch.int32)
    sc = torch.full((B, T, k), -7, device=DEV, dtype=torch.int32)
    pt = torch.tensor(pos, dtype=torch.int64, device=DEV)
    p_arg = pt if c["ragged"] else pos_max
    csa.index_topk(q_idx, w, keys, m, p_arg, k, idx, sc, cand=cand,
                   pos_max=pos_max if c["ragged"] else None)
    # cache, window ring, attention over the selected entries
    grp = 16 if c["fmt"] == "e4m3" else 32
    kv = torch.randn(B, L, d, generator=g, device=DEV)
    gate = torch.randn(B, L, generator=g, device=DEV)
    codes = torch.empty(B, blk_cap, d // 2, device=DEV, dtype=torch.uint8)
    scales = torch.empty(B, blk_cap, d // grp, device=DEV, dtype=torch.uint8)
    csa.compress_quantize(kv, gate, 0, m, codes, scales, fmt=c["fmt"])
    W, Wcap = 128, 128 + T
    win = torch.zeros(B, Wcap, d, device=DEV, dtype=torch.bfloat16)
    for b in range(B):
        last = pos[b] + T - 1
        p = torch.arange(max(0, last - Wcap + 1), last + 1, device=DEV)
        win[b, p % Wcap] = kv[b, p].to(torch.bfloat16)
    q = (torch.randn(B, T, H, d, generator=g, device=DEV) / math.sqrt(d)).to(torch.bfloat16)
    out = torch.empty(B, T, H, d, device=DEV,
                      dtype=torch.float32 if c["out_f32"] else torch.bfloat16)
    csa.sparse_attn(q, codes, scales, idx, win, W, p_arg, 1.0, out,
                    pos_max=pos_max if c["ragged"] else None, fmt=c["fmt"])
    torch.cuda.synchronize()

    qn, wn, kn = q_idx.cpu().numpy(), w.cpu().numpy(), keys.cpu().numpy()
    idn, scn = idx.cpu().numpy(), sc.cpu().numpy()
    cn = cand.cpu().numpy() if cand is not None else None
    codn, scln, winn, qb, on = (codes.cpu().numpy(), scales.cpu().numpy(), bf16_bits(win),
                                bf16_bits(q), to_np(out))
    for b in range(B):
        for ti in range(T):
            t = pos[b] + ti
            ri, rs = O.index_topk(qn[b, ti], wn[b, ti], kn[b], m, t, k,
                                  cand=None if cn is None else cn[b, ti])
            assert np.array_equal(idn[b, ti], ri), (b, ti)
            assert np.array_equal(scn[b, ti], rs), (b, ti)
            o, _ = O.sparse_attn(qb[b, ti], codn[b], scln[b], ri, winn[b], Wcap, W, t, 1.0,
                                 fmt=c["fmt"])
            ex, _ = attn_excess_error(on[b, ti][None], o[None], not c["out_f32"])
            assert ex <= REL_TOL, (b, ti, ex)
