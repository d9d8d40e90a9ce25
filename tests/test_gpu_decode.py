"""GPU parity of the decode path with ragged sequences: the token-by-token
cache append against the oracle's cache state, and the indexer and attention
calls with per-sequence positions against the oracle at each query's own
position (bit-exact for cache bytes and top-k sets, 2e-3 x RMS beyond the
output rounding for attention)."""

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


def gen(seed, *parts):
    return synth.generator(DEV, seed, *parts)


def say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- append ----

def _append_case(d, m, starts, ends, Wcap, seed):
    """Sequence b holds tokens 0 .. starts[b]-1 from a one-shot compression
    (ring and staging rows filled by the caller), then appends its tokens
    starts[b] .. ends[b]-1 one step at a time; sequences that are done sit
    at position -1. The final caches must equal the oracle's state."""
    B = len(starts)
    Lmax = max(ends)
    g = gen(seed, "append", d, m)
    kv = torch.randn(B, Lmax, d, generator=g, device=DEV)
    gate = torch.randn(B, Lmax, generator=g, device=DEV)
    cap = Lmax // m + 2
    codes = torch.full((B, cap, d // 2), 0xAB, device=DEV, dtype=torch.uint8)
    scales = torch.full((B, cap, d // 32), 0xCD, device=DEV, dtype=torch.uint8)
    win = torch.zeros(B, Wcap, d, device=DEV, dtype=torch.bfloat16)
    stage = torch.full((B, m, d), float("nan"), device=DEV)
    stage_gate = torch.full((B, m), float("nan"), device=DEV)
    for b in range(B):
        P = starts[b]
        if P:
            csa.compress_quantize(kv[b:b + 1, :P].contiguous(), gate[b:b + 1, :P].contiguous(), 0,
                                  m, codes[b:b + 1], scales[b:b + 1])
            for p in range(max(0, P - Wcap), P):
                win[b, p % Wcap] = kv[b, p].to(torch.bfloat16)
            r = P % m
            stage[b, :r] = kv[b, P - r:P]
            stage_gate[b, :r] = gate[b, P - r:P]
    steps = max(e - s for s, e in zip(starts, ends))
    pos = torch.empty(B, dtype=torch.int64, device=DEV)
    host_pos = np.zeros(B, np.int64)
    for s in range(steps):
        for b in range(B):
            host_pos[b] = starts[b] + s if starts[b] + s < ends[b] else -1
        pos.copy_(torch.from_numpy(host_pos))
        idx = torch.from_numpy(np.clip(host_pos, 0, None)).to(DEV)
        csa.decode_append(kv[torch.arange(B, device=DEV), idx].contiguous(),
                          gate[torch.arange(B, device=DEV), idx].contiguous(), pos, m, stage,
                          stage_gate, codes, scales, win)
    torch.cuda.synchronize()
    kvn, gn = kv.cpu().numpy(), gate.cpu().numpy()
    cn, sn, wn = codes.cpu().numpy(), scales.cpu().numpy(), bf16_bits(win)
    for b in range(B):
        rc, rs, ring = O.cache_after_appends(kvn[b], gn[b], m, ends[b], Wcap)
        nb = ends[b] // m
        assert np.array_equal(cn[b, :nb], rc), (d, m, b)
        assert np.array_equal(sn[b, :nb], rs), (d, m, b)
        # the block being filled has no entry yet (the trailing partial
        # block of a one-shot compression may have one, written before)
        if ends[b] % m and starts[b] <= nb * m:
            assert (cn[b, nb:] == 0xAB).all() and (sn[b, nb:] == 0xCD).all(), (d, m, b)
        for slot, row in ring.items():
            assert np.array_equal(wn[b, slot], row), (d, m, b, slot)


@pytest.mark.parametrize("d,m", [(512, 4), (128, 1), (64, 3), (256, 128)])
def test_decode_append(d, m):
    say("decode append", d, m)
    if m == 128:
        _append_case(d, m, [0, 200, 640], [520, 700, 900], 128, seed=70)
    else:
        _append_case(d, m, [0, 10, 33], [37, 64, 101], 16, seed=71)


def test_decode_append_block_cap_and_skip():
    """Blocks past blk_cap are not written; a sequence at -1 is untouched."""
    say("decode append edges")
    B, d, m, Wcap = 2, 128, 4, 8
    cap = 3
    g = gen(72, "append-edges")
    kv = torch.randn(B, d, generator=g, device=DEV)
    gate = torch.randn(B, generator=g, device=DEV)
    codes = torch.full((B, cap, d // 2), 0x11, device=DEV, dtype=torch.uint8)
    scales = torch.full((B, cap, d // 32), 0x22, device=DEV, dtype=torch.uint8)
    win = torch.zeros(B, Wcap, d, device=DEV, dtype=torch.bfloat16)
    stage = torch.zeros(B, m, d, device=DEV)
    stage_gate = torch.zeros(B, m, device=DEV)
    pos = torch.tensor([4 * cap + 3, -1], dtype=torch.int64, device=DEV)  # completes block cap
    csa.decode_append(kv, gate, pos, m, stage, stage_gate, codes, scales, win)
    torch.cuda.synchronize()
    assert (codes == 0x11).all() and (scales == 0x22).all()
    assert torch.equal(win[0, (4 * cap + 3) % Wcap], kv[0].to(torch.bfloat16))
    assert (win[1] == 0).all() and (stage[1] == 0).all()
    assert torch.equal(stage[0, 3], kv[0])


# ---------------------------------------------------------- ragged index ----

def _ragged_index_case(T, Hi, Di, m, pos, pos_max, k, blk_cap, seed, cand_C=0, phases=False):
    B = len(pos)
    g = gen(seed, "ragged-idx", B, T)
    q = torch.randint(-8, 8, (B, T, Hi, Di), generator=g, device=DEV, dtype=torch.int8)
    w = torch.randint(0, 4, (B, T, Hi), generator=g, device=DEV, dtype=torch.int8)
    keys = torch.randint(-8, 8, (B, blk_cap, Di), generator=g, device=DEV, dtype=torch.int8)
    cand = None
    if cand_C:  # distinct ascending block ids, some not visible to the shorter sequences
        cand = torch.stack([torch.sort(torch.randperm(blk_cap, generator=g, device=DEV)[:cand_C])[0]
                            for _ in range(B * T)]).reshape(B, T, cand_C).to(torch.int32)
    oi = torch.full((B, T, k), -7, device=DEV, dtype=torch.int32)
    os_ = torch.full((B, T, k), -7, device=DEV, dtype=torch.int32)
    pt = torch.tensor(pos, dtype=torch.int64, device=DEV)
    if phases:
        csa.index_scan(q, w, keys, m, pt, k, oi, os_, cand=cand, pos_max=pos_max)
        csa.index_select(q, w, keys, m, pt, k, oi, os_, cand=cand, pos_max=pos_max)
    else:
        csa.index_topk(q, w, keys, m, pt, k, oi, os_, cand=cand, pos_max=pos_max)
    torch.cuda.synchronize()
    qn, wn, kn = q.cpu().numpy(), w.cpu().numpy(), keys.cpu().numpy()
    oin, osn = oi.cpu().numpy(), os_.cpu().numpy()
    cn = cand.cpu().numpy() if cand is not None else None
    for b in range(B):
        base = min(max(pos[b], 0), pos_max)
        for ti in range(T):
            ri, rs = O.index_topk(qn[b, ti], wn[b, ti], kn[b], m, base + ti, k,
                                  cand=None if cn is None else cn[b, ti])
            assert np.array_equal(oin[b, ti], ri), (b, ti, base)
            assert np.array_equal(osn[b, ti], rs), (b, ti, base)


def test_index_ragged_decode():
    say("index ragged decode")
    # very different lengths in one batch, one past pos_max and one negative (clamped)
    _ragged_index_case(1, 8, 64, 4, [4 * 20000 - 1, 4 * 1234, 77, 4 * 3000 + 2, 90000, -5],
                       4 * 20000 - 1, 512, 20003, seed=73)
    _ragged_index_case(2, 8, 64, 4, [4 * 9000, 5, 4 * 2048 - 2], 4 * 9000, 256, 9003, seed=74,
                       cand_C=3000)
    _ragged_index_case(1, 8, 64, 4, [4 * 30000 - 1, 4 * 7000 + 1, 4 * 29000], 4 * 30000 - 1, 1024,
                       30000, seed=81, phases=True)


def test_index_ragged_prefill():
    """Runs of T >= 16 queries per sequence (batched scan) at different positions."""
    say("index ragged prefill")
    _ragged_index_case(20, 8, 64, 4, [3000, 0, 4 * 1500 + 1], 6100, 40, 1600, seed=75)
    _ragged_index_case(33, 4, 32, 4, [100, 7000], 7000, 64, 1800, seed=76)
    # over 8,192 entries (no score slab): one sequence at the start, one past
    # the slab limit, one in the middle, with ragged tiles
    _ragged_index_case(17, 8, 64, 4, [30, 4 * 11000 + 3, 4 * 5000], 4 * 11000 + 3, 300, 11050,
                       seed=77, phases=True)


# ------------------------------------------------------ ragged attention ----

def _attn_world(B, L, d, m, Wcap, seed, H, T):
    g = gen(seed, "ragged-attn", B, L, d, m)
    kv = torch.randn(B, L, d, generator=g, device=DEV)
    gate = torch.randn(B, L, generator=g, device=DEV)
    cap = O.n_blocks(L, m)
    codes = torch.empty(B, cap, d // 2, device=DEV, dtype=torch.uint8)
    scales = torch.empty(B, cap, d // 32, device=DEV, dtype=torch.uint8)
    csa.compress_quantize(kv, gate, 0, m, codes, scales)
    q = (torch.randn(B, T, H, d, generator=g, device=DEV) / math.sqrt(d)).to(torch.bfloat16)
    return kv, codes, scales, q, cap


def _ring_at(kv, pos, T, Wcap):
    """bf16 ring of each sequence holding its tokens up to pos[b] + T - 1."""
    B, L, d = kv.shape
    win = torch.zeros(B, Wcap, d, device=DEV, dtype=torch.bfloat16)
    for b in range(B):
        last = pos[b] + T - 1
        p = torch.arange(max(0, last - Wcap + 1), last + 1, device=DEV)
        win[b, p % Wcap] = kv[b, p].to(torch.bfloat16)
    return win


@pytest.mark.parametrize("T", [1, 3])
def test_sparse_attn_ragged(T):
    say("sparse attn ragged", T)
    B, L, d, m, H, W, Wcap, k = 4, 24000, 512, 4, 64, 128, 160, 256
    pos = [L - T, 5000, 37, 12345]
    kv, codes, scales, q, cap = _attn_world(B, L, d, m, Wcap, 77, H, T)
    win = _ring_at(kv, pos, T, Wcap)
    g = gen(78, "ragged-idx-sel")
    idx = torch.full((B, T, k), -1, device=DEV, dtype=torch.int32)
    for b in range(B):
        for ti in range(T):
            nv = (pos[b] + ti + 1) // m
            n = min(k, nv)
            idx[b, ti, :n] = torch.randperm(nv, generator=g, device=DEV)[:n].to(torch.int32)
    out = torch.empty(B, T, H, d, device=DEV, dtype=torch.bfloat16)
    lse = torch.empty(B, T, H, device=DEV, dtype=torch.float32)
    pt = torch.tensor(pos, dtype=torch.int64, device=DEV)
    csa.sparse_attn(q, codes, scales, idx, win, W, pt, 1.0, out, lse, pos_max=L - T)
    # sequence b of a uniform call at pos[b] gives the same bits (same batch,
    # same split plan)
    same = torch.empty_like(out)
    torch.cuda.synchronize()
    qb, cn, sn, wn = bf16_bits(q), codes.cpu().numpy(), scales.cpu().numpy(), bf16_bits(win)
    on, ln, idn = to_np(out), lse.cpu().numpy(), idx.cpu().numpy()
    for b in range(B):
        csa.sparse_attn(q, codes, scales, idx, win, W, pos[b], 1.0, same)
        torch.cuda.synchronize()
        assert torch.equal(same[b], out[b]), b
        for ti in range(T):
            o, ls = O.sparse_attn(qb[b, ti], cn[b], sn[b], idn[b, ti], wn[b], Wcap, W,
                                  pos[b] + ti, 1.0)
            ex, _ = attn_excess_error(on[b, ti][None], o[None], True)
            assert ex <= REL_TOL, (b, ti, ex)
            assert np.abs(ln[b, ti] - ls).max() <= 1e-4 * max(1.0, np.abs(ls).max()), (b, ti)


def test_hca_dense_ragged():
    say("hca dense ragged")
    B, L, d, m, H, W, Wcap, T = 3, 200000, 512, 128, 64, 128, 128, 1
    pos = [L - 1, 70000, 300]
    kv, codes, scales, q, cap = _attn_world(B, L, d, m, Wcap, 79, H, T)
    win = _ring_at(kv, pos, T, Wcap)
    out = torch.empty(B, T, H, d, device=DEV, dtype=torch.float32)
    pt = torch.tensor(pos, dtype=torch.int64, device=DEV)
    csa.hca_dense_attn(q, codes, scales, m, win, W, pt, 1.0, out, pos_max=L - 1)
    torch.cuda.synchronize()
    qb, cn, sn, wn, on = bf16_bits(q), codes.cpu().numpy(), scales.cpu().numpy(), bf16_bits(win), to_np(out)
    for b in range(B):
        o, _ = O.hca_dense_attn(qb[b, 0], cn[b], sn[b], m, wn[b], Wcap, W, pos[b], 1.0)
        ex, _ = attn_excess_error(on[b, 0][None], o[None], False)
        assert ex <= REL_TOL, (b, ex)


# --------------------------------------------------------- decode loop ----

def test_ragged_decode_loop():
    """A few decode steps of three sequences at different lengths: append
    the new token, index at the new position, attend; each step's top-k and
    output against the oracle on the caches as the oracle builds them."""
    say("ragged decode loop")
    B, d, m, H, Hi, Di, W, Wcap, k = 3, 512, 4, 16, 8, 64, 128, 128, 64
    starts = [6001, 2050, 130]
    steps = 6
    Lmax = max(starts) + steps
    g = gen(80, "loop")
    kv = torch.randn(B, Lmax, d, generator=g, device=DEV)
    gate = torch.randn(B, Lmax, generator=g, device=DEV)
    keys = torch.randint(-8, 8, (B, Lmax // m + 1, Di), generator=g, device=DEV, dtype=torch.int8)
    cap = keys.shape[1]
    codes = torch.zeros(B, cap, d // 2, device=DEV, dtype=torch.uint8)
    scales = torch.zeros(B, cap, d // 32, device=DEV, dtype=torch.uint8)
    win = torch.zeros(B, Wcap, d, device=DEV, dtype=torch.bfloat16)
    stage = torch.zeros(B, m, d, device=DEV)
    stage_gate = torch.zeros(B, m, device=DEV)
    for b in range(B):
        P = starts[b]
        csa.compress_quantize(kv[b:b + 1, :P].contiguous(), gate[b:b + 1, :P].contiguous(), 0, m,
                              codes[b:b + 1], scales[b:b + 1])
        p = torch.arange(max(0, P - Wcap), P, device=DEV)
        win[b, p % Wcap] = kv[b, p].to(torch.bfloat16)
        r = P % m
        stage[b, :r] = kv[b, P - r:P]
        stage_gate[b, :r] = gate[b, P - r:P]
    kvn, gn, kn = kv.cpu().numpy(), gate.cpu().numpy(), keys.cpu().numpy()
    ws, ws_a = csa.Workspace(DEV), csa.Workspace(DEV)
    pos_max = Lmax - 1
    for s in range(steps):
        host = [starts[b] + s for b in range(B)]
        pos = torch.tensor(host, dtype=torch.int64, device=DEV)
        ar = torch.arange(B, device=DEV)
        csa.decode_append(kv[ar, pos].contiguous(), gate[ar, pos].contiguous(), pos, m, stage,
                          stage_gate, codes, scales, win)
        q_idx = torch.randint(-8, 8, (B, 1, Hi, Di), generator=g, device=DEV, dtype=torch.int8)
        w = torch.randint(0, 4, (B, 1, Hi), generator=g, device=DEV, dtype=torch.int8)
        q = (torch.randn(B, 1, H, d, generator=g, device=DEV) / math.sqrt(d)).to(torch.bfloat16)
        idx = torch.empty(B, 1, k, device=DEV, dtype=torch.int32)
        out = torch.empty(B, 1, H, d, device=DEV, dtype=torch.bfloat16)
        csa.index_topk(q_idx, w, keys, m, pos, k, idx, workspace=ws, pos_max=pos_max)
        csa.sparse_attn(q, codes, scales, idx, win, W, pos, 1.0, out, workspace=ws_a,
                        pos_max=pos_max)
        torch.cuda.synchronize()
        qin, wi, qb, idn, on = (q_idx.cpu().numpy(), w.cpu().numpy(), bf16_bits(q),
                                idx.cpu().numpy(), to_np(out))
        for b in range(B):
            t = host[b]
            rc, rs, ring = O.cache_after_appends(kvn[b], gn[b], m, t + 1, Wcap)
            ri, _ = O.index_topk(qin[b, 0], wi[b, 0], kn[b], m, t, k)
            assert np.array_equal(idn[b, 0], ri), (s, b)
            ring_rows = np.zeros((Wcap, d), np.uint16)
            for slot, row in ring.items():
                ring_rows[slot] = row
            o, _ = O.sparse_attn(qb[b, 0], rc, rs, ri, ring_rows, Wcap, W, t, 1.0)
            ex, _ = attn_excess_error(on[b, 0][None], o[None], True)
            assert ex <= REL_TOL, (s, b, ex)
