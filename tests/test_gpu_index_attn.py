"""csa_index_attn (indexer top-k + sparse attention in one call, the top-k
resolved inside the attention kernel for decode) against the separate calls
csa_index_topk + csa_sparse_attn and against the oracle: out_idx bit-exact,
outputs within the attention bound of the separate calls (their split
plans may differ) and of the oracle. Covers both
in-kernel selections (per-tile candidate lists for long contexts, whole
score rows for <= 8192 candidates; lists that miss part of the threshold
bin, read from the score rows), a Reindex pool, per-sequence positions,
tie storms (the global-walk path), clustered top-k (the compaction path),
other head counts and widths, batch invariance of the split plan, and the
scan-only entry csa_index_attn_scan."""

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


def _world(seed, B, L, d, H, m, Hi, Di, T=1, Wcap=256, random_cache=False):
    """Cache, window ring, queries and indexer inputs for B sequences of L
    tokens; random_cache draws valid FP4 bytes directly (no latents)."""
    g = synth.generator(DEV, seed, "index_attn", B, L, d)
    cap = -(-L // m)
    if random_cache:
        codes = torch.randint(0, 256, (B, cap, d // 2), generator=g, device=DEV,
                              dtype=torch.int32).to(torch.uint8)
        scales = torch.randint(120, 131, (B, cap, d // 32), generator=g, device=DEV,
                               dtype=torch.int32).to(torch.uint8)
        win = (torch.randn(B, Wcap, d, generator=g, device=DEV)).to(torch.bfloat16)
    else:
        kv = torch.randn(B, L, d, generator=g, device=DEV)
        gate = torch.randn(B, L, generator=g, device=DEV)
        codes = torch.empty(B, cap, d // 2, device=DEV, dtype=torch.uint8)
        scales = torch.empty(B, cap, d // 32, device=DEV, dtype=torch.uint8)
        csa.compress_quantize(kv, gate, 0, m, codes, scales)
        win = torch.zeros(B, Wcap, d, device=DEV, dtype=torch.bfloat16)
        t0 = max(0, L - Wcap)
        win[:, torch.arange(t0, L, device=DEV) % Wcap] = kv[:, t0:L].to(torch.bfloat16)
        del kv
    q = (torch.randn(B, T, H, d, generator=g, device=DEV) / math.sqrt(d)).to(torch.bfloat16)
    q_idx = torch.randint(-8, 8, (B, T, Hi, Di), generator=g, device=DEV, dtype=torch.int8)
    w = torch.randint(0, 4, (B, T, Hi), generator=g, device=DEV, dtype=torch.int8)
    keys = torch.randint(-8, 8, (B, cap, Di), generator=g, device=DEV, dtype=torch.int8)
    return dict(codes=codes, scales=scales, win=win, q=q, q_idx=q_idx, w=w, keys=keys)


def _separate(x, m, pos0, k, W, out_dtype, cand=None, pos_max=None):
    B, T = x["q"].shape[:2]
    idx = torch.empty(B, T, k, device=DEV, dtype=torch.int32)
    sc = torch.empty(B, T, k, device=DEV, dtype=torch.int32)
    csa.index_topk(x["q_idx"], x["w"], x["keys"], m, pos0, k, idx, out_score=sc, cand=cand,
                   workspace=csa.Workspace(DEV), pos_max=pos_max)
    out = torch.empty(*x["q"].shape, device=DEV, dtype=out_dtype)
    lse = torch.empty(*x["q"].shape[:3], device=DEV, dtype=torch.float32)
    csa.sparse_attn(x["q"], x["codes"], x["scales"], idx, x["win"], W, pos0, 1.0, out, lse=lse,
                    workspace=csa.Workspace(DEV), pos_max=pos_max)
    return idx, sc, out, lse


def _fused(x, m, pos0, k, W, out_dtype, cand=None, pos_max=None, ws=None):
    B, T = x["q"].shape[:2]
    idx = torch.full((B, T, k), -7, device=DEV, dtype=torch.int32)
    sc = torch.full((B, T, k), -7, device=DEV, dtype=torch.int32)
    out = torch.full(x["q"].shape, 9.0, device=DEV, dtype=out_dtype)
    lse = torch.full(x["q"].shape[:3], 9.0, device=DEV, dtype=torch.float32)
    csa.index_attn(x["q_idx"], x["w"], x["keys"], m, pos0, k, x["q"], x["codes"], x["scales"],
                   x["win"], W, 1.0, idx, out, out_score=sc, lse=lse, cand=cand,
                   workspace=ws if ws is not None else csa.Workspace(DEV), pos_max=pos_max)
    return idx, sc, out, lse


def _compare(x, m, pos0, k, W, out_dtype, cand=None, pos_max=None, oracle_seqs=(0,),
             ws=None):
    ri, rs, ro, rl = _separate(x, m, pos0, k, W, out_dtype, cand, pos_max)
    fi, fs, fo, fl = _fused(x, m, pos0, k, W, out_dtype, cand, pos_max, ws)
    torch.cuda.synchronize()
    assert torch.equal(fi, ri), "top-k differs from csa_index_topk"
    assert torch.equal(fs, rs), "scores differ from csa_index_topk"
    # the fused call may split a query's slots differently (its plan also
    # weighs the indexer bytes; the fp16 probabilities are then taken against
    # other running maxima), so the two need not agree bit for bit: both are
    # held to the oracle below
    # the oracle, on a few sequences
    B, T = x["q"].shape[:2]
    kn, qin, wn = x["keys"].cpu().numpy(), x["q_idx"].cpu().numpy(), x["w"].cpu().numpy()
    cn, sn = x["codes"].cpu().numpy(), x["scales"].cpu().numpy()
    qb, wb = bf16_bits(x["q"]), bf16_bits(x["win"])
    cnd = cand.cpu().numpy() if cand is not None else None
    pn = pos0.cpu().numpy() if isinstance(pos0, torch.Tensor) else None
    for b in oracle_seqs:
        for ti in range(T):
            t = (int(pn[b]) if pn is not None else pos0) + ti
            ref_i, _ = O.index_topk(qin[b, ti], wn[b, ti], kn[b], m, t, k,
                                    cand=None if cnd is None else cnd[b, ti])
            assert np.array_equal(fi[b, ti].cpu().numpy(), ref_i), (b, ti)
            o, lref = O.sparse_attn(qb[b, ti], cn[b], sn[b], ref_i, wb[b], wb.shape[1], W, t, 1.0)
            ex_f, _ = attn_excess_error(to_np(fo[b, ti])[None], o[None],
                                        out_dtype == torch.bfloat16)
            ex_s, _ = attn_excess_error(to_np(ro[b, ti])[None], o[None],
                                        out_dtype == torch.bfloat16)
            say(f"   seq {b} query {ti}: excess / rms fused {ex_f:.3e} separate {ex_s:.3e}")
            assert ex_f <= REL_TOL and ex_s <= REL_TOL, (b, ti, ex_f, ex_s)
            assert np.abs(fl[b, ti].cpu().numpy() - lref).max() <= 1e-4 * max(1.0, np.abs(lref).max())
    return fi, fo


@pytest.mark.parametrize("L,k", [(4 * 60000, 1024), (4 * 6000, 512)])
def test_index_attn_matches_separate_calls(L, k):
    """Long context (per-tile candidate lists) and a context of <= 8192
    entries (whole score rows)."""
    say("index_attn", L, k)
    x = _world(1, 4, L, 512, 64, 4, 8, 64)
    for od in (torch.bfloat16, torch.float32):
        _compare(x, 4, L - 1, k, 128, od, oracle_seqs=(0, 1, 2, 3))


def test_index_attn_reindex_pool():
    """A Reindex layer: top-512 of a 4096-entry pool of the Full layer."""
    say("index_attn reindex")
    B, L = 3, 4 * 40000
    x = _world(2, B, L, 512, 64, 4, 8, 64)
    pool = torch.empty(B, 1, 4096, device=DEV, dtype=torch.int32)
    csa.index_topk(x["q_idx"], x["w"], x["keys"], 4, L - 1, 4096, pool, workspace=csa.Workspace(DEV))
    g = synth.generator(DEV, 3, "reidx")
    x2 = dict(x, q_idx=torch.randint(-8, 8, x["q_idx"].shape, generator=g, device=DEV,
                                     dtype=torch.int8),
              w=torch.randint(0, 4, x["w"].shape, generator=g, device=DEV, dtype=torch.int8))
    _compare(x2, 4, L - 1, 512, 128, torch.bfloat16, cand=pool, oracle_seqs=(1,))
    # a pool length that is not a multiple of 4: every row after the first
    # starts off a 16-byte boundary (its ids are then loaded one by one)
    odd = pool[:, :, :4093].contiguous()
    _compare(x2, 4, L - 1, 512, 128, torch.bfloat16, cand=odd, oracle_seqs=(2,))


def test_index_attn_ragged_positions():
    say("index_attn ragged")
    B, L = 4, 4 * 30000
    x = _world(4, B, L, 512, 64, 4, 8, 64, Wcap=512)
    pos = torch.tensor([L - 1, L - 70, 9000, 37], device=DEV, dtype=torch.int64)
    # ring slots hold the latest window of each sequence's own position
    _compare(x, 4, pos, 512, 128, torch.bfloat16, pos_max=L - 1, oracle_seqs=(1, 3))


def test_index_attn_tie_storm_and_clusters():
    """All indexer scores tied (w = 0: every query ties at 0, the candidate
    lists hold every visible entry, the global walk resolves them), and a
    top-k clustered in one tile (more candidates there than the first load
    round stages)."""
    say("index_attn ties / clusters")
    B, L = 2, 4 * 50000
    x = _world(5, B, L, 512, 64, 4, 8, 64)
    xt = dict(x, w=torch.zeros_like(x["w"]))
    _compare(xt, 4, L - 1, 1024, 128, torch.bfloat16, oracle_seqs=(0,))
    keys = x["keys"].clone()
    # entries of tile 5 (entries 10240..12287) score high for every query
    keys[:, 10240:12288] = 7
    qi = x["q_idx"].abs().to(torch.int8)
    xc = dict(x, keys=keys, q_idx=qi)
    _compare(xc, 4, L - 1, 1024, 128, torch.bfloat16, oracle_seqs=(1,))


@pytest.mark.parametrize("Hi,Di", [(4, 32), (16, 64), (8, 128), (3, 64)])
def test_index_attn_recomputed_scores(Hi, Di):
    """A top-k packed into one 2048-entry unit (every key of the unit scores
    high) overflows even the unit's wide list, so the selection walks the
    whole score row, recomputing each score from the keys and the indexer
    query (the list scan writes no score slab): exact against the separate
    calls and the oracle for other indexer shapes."""
    say("index_attn recomputed scores", Hi, Di)
    B, L = 2, 4 * 30000
    x = _world(11, B, L, 256, 20, 4, Hi, Di)
    keys = x["keys"].clone()
    keys[:, 4096:6144] = 7
    qi = x["q_idx"].abs().to(torch.int8)
    _compare(dict(x, keys=keys, q_idx=qi), 4, L - 1, 512, 128, torch.bfloat16, oracle_seqs=(0, 1))


@pytest.mark.parametrize("k", [512, 1024])
def test_index_attn_dense_topk_spills(k):
    """A top-k dense in a short context (12,000 entries in 24 units of 512):
    most units hold more entries at or above the threshold bin than their
    32-entry lists, so the selection reads those units' score rows."""
    say("index_attn dense top-k", k)
    L = 4 * 12000
    x = _world(10, 2, L, 512, 64, 4, 8, 64)
    _compare(x, 4, L - 1, k, 128, torch.bfloat16, oracle_seqs=(0, 1))
    pos = torch.tensor([L - 1, 4 * 9000 + 3], device=DEV, dtype=torch.int64)
    _compare(x, 4, pos, k, 128, torch.float32, pos_max=L - 1, oracle_seqs=(1,))


@pytest.mark.parametrize("d,H", [(128, 8), (256, 20), (512, 40)])
def test_index_attn_shapes(d, H):
    say("index_attn shapes", d, H)
    x = _world(6, 2, 4 * 20000, d, H, 4, 4, 32)
    _compare(x, 4, 4 * 20000 - 1, 256, 64, torch.float32, oracle_seqs=(1,))


def test_index_attn_small_k_and_early_positions():
    say("index_attn small k / early")
    x = _world(7, 3, 4 * 3000, 512, 64, 4, 8, 64)
    _compare(x, 4, 4 * 3000 - 1, 16, 128, torch.bfloat16, oracle_seqs=(2,))
    # a query before its first block completes, and one with fewer than k blocks
    pos = torch.tensor([2, 40, 4 * 3000 - 1], device=DEV, dtype=torch.int64)
    _compare(x, 4, pos, 64, 128, torch.float32, pos_max=4 * 3000 - 1, oracle_seqs=(0, 1))


def test_index_attn_whole_tile_units_small_and_large_k():
    """Whole-tile scan units (4 x 256 tiles: 1,024 scan workgroups, 2,048 entries
    each): every unit adds into the query's histogram only its bins at or above
    its own k-th largest score, which cuts deepest for a small k; a k above a
    unit's size adds every bin."""
    say("index_attn whole-tile units, k 64 / 3000")
    L = 4 * 524288
    x = _world(8, 4, L, 128, 16, 4, 8, 64, random_cache=True)
    for k in (64, 3000):
        _compare(x, 4, L - 1, k, 128, torch.bfloat16, oracle_seqs=(3,))


def test_index_attn_workspace_reuse():
    """One Workspace over repeated calls and a change of B*T: every call
    leaves the head zero, so results repeat exactly."""
    say("index_attn workspace reuse")
    x = _world(8, 4, 4 * 30000, 512, 64, 4, 8, 64)
    ws = csa.Workspace(DEV)
    a = _fused(x, 4, 4 * 30000 - 1, 1024, 128, torch.bfloat16, ws=ws)
    b = _fused(x, 4, 4 * 30000 - 1, 1024, 128, torch.bfloat16, ws=ws)
    x1 = {k_: v[:1].contiguous() for k_, v in x.items()}
    c = _fused(x1, 4, 4 * 30000 - 1, 1024, 128, torch.bfloat16, ws=ws)
    d_ = _fused(x, 4, 4 * 30000 - 1, 1024, 128, torch.bfloat16, ws=ws)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    for u, v in zip(a, d_):
        assert torch.equal(u, v)
    assert torch.equal(c[0][0], a[0][0]) and torch.equal(c[2][0], a[2][0])


def test_index_attn_scan_only():
    """csa_index_attn_scan launches the scan alone and writes no output; after
    a workspace clear the full call gives what it gives on a fresh workspace."""
    say("index_attn scan only")
    L = 4 * 40000
    x = _world(9, 2, L, 512, 64, 4, 8, 64)
    ref = _fused(x, 4, L - 1, 1024, 128, torch.bfloat16)
    ws = csa.Workspace(DEV)
    B = 2
    idx = torch.full((B, 1, 1024), -7, device=DEV, dtype=torch.int32)
    out = torch.full(x["q"].shape, 9.0, device=DEV, dtype=torch.bfloat16)
    for _ in range(2):
        csa.index_attn(x["q_idx"], x["w"], x["keys"], 4, L - 1, 1024, x["q"], x["codes"],
                       x["scales"], x["win"], 128, 1.0, idx, out, workspace=ws, scan_only=True)
    torch.cuda.synchronize()
    assert (idx == -7).all() and (out == 9.0).all()
    assert ws.buf.any(), "the scan wrote nothing into the workspace"
    csa.workspace_clear(ws.buf)
    got = _fused(x, 4, L - 1, 1024, 128, torch.bfloat16, ws=ws)
    torch.cuda.synchronize()
    for u, v in zip(ref, got):
        assert torch.equal(u, v)


def test_batch_invariance_decode_and_hca():
    """A decode_32k-shaped sequence (top-512 + 128-token window of 8192
    entries) gives bit-identical outputs alone and inside a batch of 64, via
    the separate calls and via csa_index_attn; an HCA sequence at 1M tokens
    (8192 entries of 128 tokens + window) alone and inside a batch of 16."""
    say("batch invariance")
    B, L, k, W = 64, 32768, 512, 128
    x = _world(9, B, L, 512, 64, 4, 8, 64, random_cache=True)
    sel = (0, 17, 63)
    ri, _, ro, _ = _separate(x, 4, L - 1, k, W, torch.bfloat16)
    fi, _, fo, _ = _fused(x, 4, L - 1, k, W, torch.bfloat16)
    for b in sel:
        xb = {k_: v[b:b + 1].contiguous() for k_, v in x.items()}
        i1, _, o1, _ = _separate(xb, 4, L - 1, k, W, torch.bfloat16)
        j1, _, p1, _ = _fused(xb, 4, L - 1, k, W, torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(i1[0], ri[b]) and torch.equal(o1[0], ro[b]), b
        assert torch.equal(j1[0], fi[b]) and torch.equal(p1[0], fo[b]), b
    del x
    B, L, m = 16, 1 << 20, 128
    x = _world(10, B, L, 512, 64, m, 8, 64, random_cache=True)
    out = torch.empty(B, 1, 64, 512, device=DEV, dtype=torch.bfloat16)
    csa.hca_dense_attn(x["q"], x["codes"], x["scales"], m, x["win"], W, L - 1, 1.0, out,
                       workspace=csa.Workspace(DEV))
    for b in (0, 9):
        o1 = torch.empty(1, 1, 64, 512, device=DEV, dtype=torch.bfloat16)
        csa.hca_dense_attn(x["q"][b:b + 1].contiguous(), x["codes"][b:b + 1].contiguous(),
                           x["scales"][b:b + 1].contiguous(), m, x["win"][b:b + 1].contiguous(),
                           W, L - 1, 1.0, o1, workspace=csa.Workspace(DEV))
        torch.cuda.synchronize()
        assert torch.equal(o1[0], out[b]), b
