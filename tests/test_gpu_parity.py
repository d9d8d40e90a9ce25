"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs. Cache bytes and top-k index sets must be bit-identical;
attention outputs must stay within 2e-3 x RMS(reference) beyond the final
output rounding."""

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


# ------------------------------------------------------------ dequantise ----

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_dequantize_exact(dtype):
    say("dequantize", dtype)
    B, cap, d = 2, 64, 512
    g = gen(1, "deq")
    codes = torch.randint(0, 256, (B, cap, d // 2), generator=g, device=DEV, dtype=torch.uint8)
    if dtype == torch.float16:
        sc = torch.randint(104, 141, (B, cap, d // 32), generator=g, device=DEV)
    else:
        pool = torch.tensor([1, 2, 60, 100, 103, 120, 126, 127, 128, 140, 142, 200, 251, 252],
                            device=DEV)
        sc = pool[torch.randint(0, len(pool), (B, cap, d // 32), generator=g, device=DEV)]
    scales = sc.to(torch.uint8).contiguous()
    out = torch.empty(B, 40, d, device=DEV, dtype=dtype)
    csa.dequantize(codes, scales, 7, 40, out)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    for b in range(B):
        ref = O.dequantize_rows(c[b, 7:47], s[b, 7:47])
        got = out[b].cpu().double().numpy()
        assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:5]


def test_dequantize_scale_byte_zero():
    """E8M0 byte 0 (2^-127): values are bfloat16 subnormals."""
    say("dequantize scale 0")
    codes = torch.arange(256, device=DEV, dtype=torch.int32).to(torch.uint8).reshape(1, 1, 256)
    scales = torch.zeros(1, 1, 16, device=DEV, dtype=torch.uint8)
    out = torch.empty(1, 1, 512, device=DEV, dtype=torch.float32)
    csa.dequantize(codes, scales, 0, 1, out)
    ref = O.dequantize_rows(codes[0].cpu().numpy(), scales[0].cpu().numpy())
    assert np.array_equal(out[0].cpu().double().numpy(), ref)


# -------------------------------------------------------------- compress ----

def _compress_case(B, L, d, m, tok0, seed, scale=1.0, chunks=None):
    g = gen(seed, "cmp", B, L, d, m)
    kv = torch.randn(B, L, d, generator=g, device=DEV) * scale
    gate = torch.randn(B, L, generator=g, device=DEV)
    cap = O.n_blocks(tok0 + L, m) + 3
    codes = torch.full((B, cap, d // 2), 0xAB, device=DEV, dtype=torch.uint8)
    scales = torch.full((B, cap, d // 32), 0xCD, device=DEV, dtype=torch.uint8)
    chunks = chunks or [L]
    t = 0
    for n in chunks:
        csa.compress_quantize(kv[:, t:t + n].contiguous(), gate[:, t:t + n].contiguous(),
                              tok0 + t, m, codes, scales)
        t += n
    torch.cuda.synchronize()
    kvn, gn = kv.cpu().numpy(), gate.cpu().numpy()
    cn, sn = codes.cpu().numpy(), scales.cpu().numpy()
    b0 = tok0 // m
    for b in range(B):
        rc, rs = O.compress_quantize(kvn[b], gn[b], m)
        nb = rc.shape[0]
        flag = O.near_decision_mask(kvn[b], gn[b], m)
        assert not flag.any()
        assert np.array_equal(cn[b, b0:b0 + nb], rc), (b, np.argwhere(cn[b, b0:b0 + nb] != rc)[:4])
        assert np.array_equal(sn[b, b0:b0 + nb], rs)
        # untouched outside the written range
        assert (cn[b, :b0] == 0xAB).all() and (cn[b, b0 + nb:] == 0xAB).all()
        assert (sn[b, b0 + nb:] == 0xCD).all()


@pytest.mark.parametrize("d", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("m", [1, 3, 4, 128])
def test_compress_shapes(d, m):
    say("compress", d, m)
    _compress_case(2, 517, d, m, 0, seed=3)


def test_compress_offset_and_chunks():
    say("compress chunks")
    _compress_case(1, 4096 + 6, 512, 4, 8, seed=4, chunks=[1024, 2048, 1030])
    _compress_case(3, 300, 128, 4, 400, seed=5, scale=1e-30)
    _compress_case(1, 256, 512, 128, 0, seed=6, scale=3e4)


def test_compress_tiny_workload():
    """The tiny causal workload (1 x 1024 tokens, d=128, m=4) from synth."""
    say("compress tiny_causal")
    wl = synth.WORKLOADS["tiny_causal"]
    kv = synth.latent_range(wl, 0, 0, wl.L, DEV)[None].contiguous()
    gate = synth.latent_range(wl, 0, 0, wl.L, DEV, gate=True)[None].contiguous()
    codes = torch.empty(1, wl.n_blocks, wl.d // 2, device=DEV, dtype=torch.uint8)
    scales = torch.empty(1, wl.n_blocks, wl.d // 32, device=DEV, dtype=torch.uint8)
    csa.compress_quantize(kv, gate, 0, wl.m, codes, scales)
    rc, rs = O.compress_quantize(kv[0].cpu().numpy(), gate[0].cpu().numpy(), wl.m)
    assert np.array_equal(codes[0].cpu().numpy(), rc)
    assert np.array_equal(scales[0].cpu().numpy(), rs)


# --------------------------------------------------------------- indexer ----

def _index_case(B, T, Hi, Di, m, pos0, k, blk_cap, seed, cand_C=0, wzero=False, keyrange=8,
                phases=False, sample=None, hot_tiles=()):
    g = gen(seed, "idx", B, T, Hi, Di)
    q = torch.randint(-8, 8, (B, T, Hi, Di), generator=g, device=DEV, dtype=torch.int8)
    w = torch.randint(0, 4, (B, T, Hi), generator=g, device=DEV, dtype=torch.int8)
    if wzero:
        w.zero_()
    keys = torch.randint(-keyrange, keyrange, (B, blk_cap, Di), generator=g, device=DEV,
                         dtype=torch.int8)
    for tl in hot_tiles:  # 2048-entry tiles of wide-range keys: the top-k clusters there
        keys[:, tl * 2048:(tl + 1) * 2048] = torch.randint(
            -100, 100, (B, min(2048, blk_cap - tl * 2048), Di), generator=g, device=DEV,
            dtype=torch.int8)
    cand = None
    if cand_C:
        nv = min(blk_cap, (pos0 + T) // m)
        pool = torch.stack([torch.randperm(nv + 50, generator=g, device=DEV)[:cand_C]
                            for _ in range(B * T)]).reshape(B, T, cand_C)
        pool = torch.where(pool >= nv + 40, torch.full_like(pool, -1), pool)
        cand = torch.sort(torch.where(pool < 0, torch.full_like(pool, 1 << 30), pool), dim=2)[0]
        cand = torch.where(cand == (1 << 30), torch.full_like(cand, -1), cand).to(torch.int32)
        cand = cand.contiguous()
    oi = torch.full((B, T, k), -7, device=DEV, dtype=torch.int32)
    os_ = torch.full((B, T, k), -7, device=DEV, dtype=torch.int32)
    if phases:
        csa.index_scan(q, w, keys, m, pos0, k, oi, os_, cand=cand)
        csa.index_select(q, w, keys, m, pos0, k, oi, os_, cand=cand)
    else:
        csa.index_topk(q, w, keys, m, pos0, k, oi, os_, cand=cand)
    torch.cuda.synchronize()
    qn, wn, kn = q.cpu().numpy(), w.cpu().numpy(), keys.cpu().numpy()
    oin, osn = oi.cpu().numpy(), os_.cpu().numpy()
    cn = cand.cpu().numpy() if cand is not None else None
    pairs = [(b, ti) for b in range(B) for ti in range(T)]
    if sample is not None:  # the first and last queries and a seeded sample of the rest
        rs = np.random.default_rng(seed)
        pick = set(rs.choice(len(pairs), size=min(sample, len(pairs)), replace=False).tolist())
        pick |= {0, len(pairs) - 1}
        pairs = [pairs[i] for i in sorted(pick)]
    for b, ti in pairs:
        if True:
            ref_i, ref_s = O.index_topk(qn[b, ti], wn[b, ti], kn[b], m, pos0 + ti, k,
                                        cand=None if cn is None else cn[b, ti])
            assert np.array_equal(oin[b, ti], ref_i), (b, ti, oin[b, ti][:8], ref_i[:8])
            assert np.array_equal(osn[b, ti], ref_s), (b, ti)
    return oi


@pytest.mark.parametrize("Hi,Di", [(1, 32), (3, 64), (4, 32), (8, 64), (16, 64), (8, 128)])
def test_index_decode_shapes(Hi, Di):
    say("index decode", Hi, Di)
    _index_case(3, 2, Hi, Di, 4, 4 * 5000 - 2, 64, 5100, seed=7)


def test_index_many_queries_compact():
    """A 1024-query run over more than 8,192 visible entries: batched scan, per-tile
    select, and the final pass with its compact LDS budget (launches of >= 1024
    queries); sampled queries against the oracle."""
    say("index 1024 queries, compact final pass")
    _index_case(1, 1024, 8, 64, 4, 4 * 9000, 512, 9000 + 260, seed=12, sample=40)


def test_index_many_queries_ties():
    """The same launch with every score tied (all weights zero) and with keys of
    one value: more candidates than the compact budget holds, so the final pass
    walks the per-tile lists in global memory."""
    say("index 1024 queries, ties")
    _index_case(1, 1024, 8, 64, 4, 4 * 9000, 512, 9000 + 260, seed=13, wzero=True, sample=12)
    _index_case(1, 1024, 4, 64, 4, 4 * 9000, 300, 9000 + 260, seed=14, keyrange=1, sample=12)


def test_index_decode_edges():
    say("index decode edges")
    _index_case(2, 1, 8, 64, 4, 2, 16, 64, seed=8)             # no visible block yet
    _index_case(2, 1, 8, 64, 4, 40, 64, 64, seed=9)            # k > visible
    _index_case(2, 3, 8, 64, 4, 4 * 3000, 100, 3000, seed=10, wzero=True)  # all ties
    _index_case(2, 1, 8, 64, 4, 4 * 9000, 300, 9000, seed=11, keyrange=1)  # massive ties
    _index_case(1, 1, 8, 64, 1, 2047, 2048, 4096, seed=12)     # k == visible exactly
    _index_case(2, 1, 8, 64, 4, 4 * 20000 - 1, 6000, 20000, seed=22)  # k > LDS capacity
    _index_case(2, 2, 8, 64, 4, 4 * 20000, 1000, 20000, seed=13, phases=True)


def test_index_large_k_few_queries():
    """A Full layer's candidate pool: few queries with k >= 2048 over up to
    1,048,576 entries (the final pass's stage then holds few candidates per
    list), ties, and k above the visible entries."""
    say("index large k")
    _index_case(3, 1, 8, 64, 4, 4 * 200000 - 1, 4096, 200000, seed=97)
    _index_case(2, 2, 8, 64, 4, 4 * 150000, 2048, 150010, seed=98, keyrange=1)
    _index_case(2, 1, 4, 32, 4, 4 * 9000, 10000, 9100, seed=99)
    _index_case(2, 1, 8, 64, 4, 4 * 1048575, 4096, 1048576, seed=100, sample=2)


def test_index_clustered_large_k():
    """Few queries whose top-k clusters in a few tiles: those lists overflow
    the final pass's stage, the rest are short or empty, so the candidates are
    gathered per thread across empty lists (and past 8,192 candidates through
    LDS or the global walk)."""
    say("index clustered large k")
    _index_case(2, 1, 8, 64, 4, 4 * 50000 - 1, 2000, 50000, seed=101, hot_tiles=(3, 17))
    _index_case(2, 1, 8, 64, 4, 4 * 50000 - 1, 3500, 50000, seed=102, hot_tiles=(0, 1, 24))
    _index_case(3, 1, 8, 64, 4, 4 * 120000 - 1, 7000, 120000, seed=103, hot_tiles=(5, 40, 58))


def test_index_candidates():
    say("index candidates")
    _index_case(4, 1, 8, 64, 4, 4 * 10000 - 1, 128, 10000, seed=14, cand_C=4096)
    _index_case(2, 2, 8, 64, 4, 4 * 3000 - 1, 512, 3000, seed=15, cand_C=600)
    _index_case(2, 1, 8, 64, 4, 4 * 3000 - 1, 64, 3000, seed=16, cand_C=300, wzero=True)
    # pools of at most 4096 entries take the one-workgroup select: both phases,
    # massive ties, k above the pool, 32- and 128-dim keys, a pool of one tile
    _index_case(2, 2, 8, 64, 4, 4 * 3000 - 1, 128, 3000, seed=30, cand_C=600, phases=True)
    _index_case(2, 1, 8, 64, 4, 4 * 3000 - 1, 200, 3000, seed=31, cand_C=1000, keyrange=1)
    _index_case(2, 1, 8, 64, 4, 4 * 3000 - 1, 512, 3000, seed=32, cand_C=300)
    _index_case(3, 1, 4, 32, 4, 4 * 5000 - 1, 256, 5000, seed=33, cand_C=4096)
    _index_case(2, 1, 4, 128, 4, 4 * 5000 - 1, 100, 5000, seed=34, cand_C=2049)
    _index_case(1, 1, 8, 64, 4, 4 * 5000 - 1, 16, 5000, seed=35, cand_C=13)


def test_index_many_queries():
    """Split scan with many short query runs (1920 queries, 1000 blocks
    each), with several ragged tiles per query, and with enough work that a
    scan workgroup takes two or four 2048-entry tiles (ragged last group)."""
    say("index many queries")
    _index_case(128, 15, 8, 64, 4, 4 * 1000 - 15, 96, 1007, seed=40)
    _index_case(30, 10, 8, 64, 4, 4 * 13000 - 10, 96, 13007, seed=41, phases=True)
    _index_case(128, 2, 8, 64, 4, 4 * 3000 - 2, 96, 3007, seed=42)     # 2 tiles per workgroup
    _index_case(64, 2, 8, 64, 4, 4 * 9500 - 2, 96, 9507, seed=43)      # 4 per workgroup, ragged
    _index_case(128, 2, 4, 128, 4, 4 * 3000 - 2, 64, 3007, seed=44)    # 128-dim keys, 2 per group
    _index_case(64, 2, 8, 64, 4, 4 * 9500 - 2, 96, 9507, seed=45, cand_C=4500)  # pool, 3 tiles


def _pool_case(B, T, Hi, Di, m, pos0, k, n_keep, blk_cap, seed, wzero=False, keyrange=8,
               reindex_k=0):
    """Full-mode top-k plus the blockwise pool against the oracle's top-k and
    block pool, element by element; with reindex_k, a Reindex top-k over the
    produced pool (partial groups leave -1 inside it) against the oracle."""
    g = gen(seed, "pool", B, T, Hi, Di)
    q = torch.randint(-8, 8, (B, T, Hi, Di), generator=g, device=DEV, dtype=torch.int8)
    w = torch.randint(0, 4, (B, T, Hi), generator=g, device=DEV, dtype=torch.int8)
    if wzero:
        w.zero_()
    keys = torch.randint(-keyrange, keyrange, (B, blk_cap, Di), generator=g, device=DEV,
                         dtype=torch.int8)
    oi = torch.full((B, T, k), -7, device=DEV, dtype=torch.int32)
    os_ = torch.full((B, T, k), -7, device=DEV, dtype=torch.int32)
    op = torch.full((B, T, 8 * n_keep), -7, device=DEV, dtype=torch.int32)
    csa.index_topk_pool(q, w, keys, m, pos0, k, oi, n_keep, op, out_score=os_)
    plain = torch.full((B, T, k), -7, device=DEV, dtype=torch.int32)
    csa.index_topk(q, w, keys, m, pos0, k, plain)
    ri = None
    if reindex_k:
        ri = torch.full((B, T, reindex_k), -7, device=DEV, dtype=torch.int32)
        csa.index_topk(q, w, keys, m, pos0, reindex_k, ri, cand=op)
    torch.cuda.synchronize()
    assert torch.equal(oi, plain)
    qn, wn, kn = q.cpu().numpy(), w.cpu().numpy(), keys.cpu().numpy()
    oin, osn, opn = oi.cpu().numpy(), os_.cpu().numpy(), op.cpu().numpy()
    rin = ri.cpu().numpy() if ri is not None else None
    for b in range(B):
        for ti in range(T):
            t = pos0 + ti
            ref_i, ref_s = O.index_topk(qn[b, ti], wn[b, ti], kn[b], m, t, k)
            assert np.array_equal(oin[b, ti], ref_i), (b, ti)
            assert np.array_equal(osn[b, ti], ref_s), (b, ti)
            ref_p = O.block_pool(qn[b, ti], wn[b, ti], kn[b], m, t, 8, n_keep)
            assert np.array_equal(opn[b, ti], ref_p), (b, ti, opn[b, ti][:16], ref_p[:16])
            if rin is not None:
                ref_r, _ = O.index_topk(qn[b, ti], wn[b, ti], kn[b], m, t, reindex_k,
                                        cand=ref_p)
                assert np.array_equal(rin[b, ti], ref_r), (b, ti)


@pytest.mark.parametrize("Hi,Di", [(8, 64), (4, 32), (16, 64), (8, 128)])
def test_index_block_pool_shapes(Hi, Di):
    """Decode queries: a 20,000-entry context (10 tiles, ragged) keeping 256
    groups, then a Reindex top-k over the pool."""
    say("index block pool", Hi, Di)
    _pool_case(4, 1, Hi, Di, 4, 4 * 20000 - 1, 512, 256, 20003, seed=60, reindex_k=256)


def test_index_block_pool_edges():
    say("index block pool edges")
    _pool_case(2, 1, 8, 64, 4, 2, 16, 8, 64, seed=61)                 # nothing visible
    _pool_case(2, 1, 8, 64, 4, 4 * 101 - 1, 32, 64, 400, seed=62)     # 13 groups < n_keep, partial
    _pool_case(2, 3, 8, 64, 4, 4 * 3000, 100, 40, 3000, seed=63, wzero=True)   # all ties
    _pool_case(2, 1, 8, 64, 4, 4 * 9000, 300, 500, 9000, seed=64, keyrange=1)  # massive ties
    _pool_case(1, 20, 8, 64, 4, 4 * 5000 - 20, 64, 100, 5007, seed=65,          # query run
               reindex_k=64)
    _pool_case(1, 1, 8, 64, 1, 2047, 2048, 256, 4096, seed=66)        # n_keep == visible groups
    # the long-context keep size (2,000 groups of a 32,768-entry context)
    _pool_case(2, 1, 8, 64, 4, 4 * 32768 - 1, 512, 2000, 32768, seed=67, reindex_k=512)


@pytest.mark.parametrize("Hi,Di", [(4, 32), (8, 64), (16, 64), (2, 128), (5, 64)])
def test_index_prefill_shapes(Hi, Di):
    say("index prefill", Hi, Di)
    _index_case(2, 100, Hi, Di, 4, 3000, 40, 2000, seed=17)


def test_index_prefill_edges():
    say("index prefill edges")
    _index_case(1, 64, 8, 64, 4, 0, 16, 64, seed=18)             # starts at position 0
    _index_case(1, 40, 8, 64, 4, 400, 32, 200, seed=19, wzero=True)
    _index_case(1, 33, 8, 64, 4, 800, 64, 1000, seed=20, keyrange=1)
    _index_case(1, 17, 8, 64, 1, 1000, 600, 1100, seed=21)


@pytest.mark.parametrize("Hi,Di", [(4, 32), (8, 64), (16, 64), (2, 128), (5, 64), (16, 32),
                                   (8, 128)])
def test_index_prefill_rescan_shapes(Hi, Di):
    """Query runs over more than 8,192 visible entries keep no score slab: the
    batched scan runs twice (histograms, then each query's candidates per wave
    quarter, joined per tile). 37 queries (a ragged last query group) over
    10,037 entries (a ragged last tile), every query against the oracle."""
    say("index prefill rescan", Hi, Di)
    _index_case(2, 37, Hi, Di, 4, 4 * 10000 + 3, 200, 10040, seed=90)


def test_index_prefill_rescan_edges():
    say("index prefill rescan edges")
    # scan and select as separate calls; k above a tile; k = 1
    _index_case(1, 20, 8, 64, 4, 4 * 9000, 2500, 9100, seed=91, phases=True)
    _index_case(1, 16, 8, 64, 4, 4 * 9000, 1, 9100, seed=92)
    # every score tied; keys of one value (every entry a candidate of its tile)
    _index_case(1, 18, 8, 64, 4, 4 * 8500, 700, 8600, seed=93, wzero=True)
    _index_case(1, 24, 4, 32, 4, 4 * 8500, 300, 8600, seed=94, keyrange=1)
    # a run whose first queries see fewer than 8,192 entries and its last more
    _index_case(1, 400, 8, 64, 1, 8000, 64, 8500, seed=95, sample=60)
    # more than 2,048 quarter lists (over 1,048,576 entries): the quarters are
    # joined per tile before the final pass
    _index_case(1, 16, 8, 64, 4, 4 * 1050000, 64, 1050040, seed=96, sample=4)


def test_index_tiny_workload():
    """All 1024 queries of the tiny causal workload (Hi=4, Di=32, k=16)."""
    say("index tiny_causal")
    wl = synth.WORKLOADS["tiny_causal"]
    q, w = synth.indexer_queries(wl, DEV)
    keys = synth.indexer_keys(wl, DEV)
    oi = torch.empty(1, wl.T, wl.k, device=DEV, dtype=torch.int32)
    csa.index_topk(q, w, keys, wl.m, 0, wl.k, oi)
    qn, wn, kn, oin = q.cpu().numpy(), w.cpu().numpy(), keys.cpu().numpy(), oi.cpu().numpy()
    for t in range(wl.T):
        ref, _ = O.index_topk(qn[0, t], wn[0, t], kn[0], wl.m, t, wl.k)
        assert np.array_equal(oin[0, t], ref), t


# ------------------------------------------------------------- attention ----

def _attn_world(B, L, d, m, Wcap, seed, H, T, W=128):
    g = gen(seed, "attn", B, L, d, m)
    kv = torch.randn(B, L, d, generator=g, device=DEV)
    gate = torch.randn(B, L, generator=g, device=DEV)
    cap = O.n_blocks(L, m)
    codes = torch.empty(B, cap, d // 2, device=DEV, dtype=torch.uint8)
    scales = torch.empty(B, cap, d // 32, device=DEV, dtype=torch.uint8)
    csa.compress_quantize(kv, gate, 0, m, codes, scales)
    win = torch.zeros(B, Wcap, d, device=DEV, dtype=torch.bfloat16)
    t0 = max(0, L - Wcap)
    pos = torch.arange(t0, L, device=DEV)
    win[:, pos % Wcap] = kv[:, t0:L].to(torch.bfloat16)
    q = (torch.randn(B, T, H, d, generator=g, device=DEV) / math.sqrt(d)).to(torch.bfloat16)
    return dict(codes=codes, scales=scales, win=win, q=q, cap=cap)


def _check_attn(wd, idx, pos0, W, out, lse, dense_m=None, scale=1.0):
    torch.cuda.synchronize()
    B, T, H, d = wd["q"].shape
    cn, sn = wd["codes"].cpu().numpy(), wd["scales"].cpu().numpy()
    wn = bf16_bits(wd["win"])
    qn = bf16_bits(wd["q"])
    on = to_np(out)
    ln = lse.cpu().numpy() if lse is not None else None
    idn = idx.cpu().numpy() if idx is not None else None
    refs, lrefs = [], []
    for b in range(B):
        for ti in range(T):
            t = pos0 + ti
            if dense_m is None:
                o, l = O.sparse_attn(qn[b, ti], cn[b], sn[b], idn[b, ti], wn[b], wn.shape[1], W, t,
                                     scale)
            else:
                o, l = O.hca_dense_attn(qn[b, ti], cn[b], sn[b], dense_m, wn[b], wn.shape[1], W, t,
                                        scale)
            refs.append(o)
            lrefs.append(l)
    ref = np.stack(refs).reshape(B, T, H, d)
    lref = np.stack(lrefs).reshape(B, T, H)
    ex, rms = attn_excess_error(on, ref, out.dtype == torch.bfloat16)
    say(f"   excess error / rms = {ex:.3e} (rms {rms:.3e})")
    assert ex <= REL_TOL, ex
    if ln is not None:
        assert np.abs(ln - lref).max() <= 1e-4 * max(1.0, np.abs(lref).max())
    return ex


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_sparse_attn_tiny_workload(out_dtype):
    """All 1024 queries of the tiny causal workload with the oracle's own top-k."""
    say("attn tiny_causal", out_dtype)
    wl = synth.WORKLOADS["tiny_causal"]
    kv = synth.latent_range(wl, 0, 0, wl.L, DEV)[None].contiguous()
    gate = synth.latent_range(wl, 0, 0, wl.L, DEV, gate=True)[None].contiguous()
    codes = torch.empty(1, wl.n_blocks, wl.d // 2, device=DEV, dtype=torch.uint8)
    scales = torch.empty(1, wl.n_blocks, wl.d // 32, device=DEV, dtype=torch.uint8)
    csa.compress_quantize(kv, gate, 0, wl.m, codes, scales)
    win = synth.window_ring(wl, wl.L - 1, DEV)
    q = synth.queries(wl, DEV)
    qi, w = synth.indexer_queries(wl, DEV)
    keys = synth.indexer_keys(wl, DEV)
    qin, wn, kn = qi.cpu().numpy(), w.cpu().numpy(), keys.cpu().numpy()
    idx = np.stack([O.index_topk(qin[0, t], wn[0, t], kn[0], wl.m, t, wl.k)[0]
                    for t in range(wl.T)])[None]
    idx_t = torch.from_numpy(idx).to(DEV).contiguous()
    out = torch.empty(1, wl.T, wl.H, wl.d, device=DEV, dtype=out_dtype)
    lse = torch.empty(1, wl.T, wl.H, device=DEV, dtype=torch.float32)
    csa.sparse_attn(q, codes, scales, idx_t, win, wl.W, 0, 1.0, out, lse)
    wd = dict(codes=codes, scales=scales, win=win, q=q)
    _check_attn(wd, idx_t, 0, wl.W, out, lse)


@pytest.mark.parametrize("d,H", [(512, 64), (128, 8), (256, 20)])
def test_sparse_attn_decode(d, H):
    say("attn decode", d, H)
    B, L, m, k, W = 3, 4 * 1500, 4, 512, 128
    wd = _attn_world(B, L, d, m, 128, seed=22, H=H, T=1)
    g = gen(23, "idx")
    nv = L // m
    idx = torch.stack([torch.randperm(nv, generator=g, device=DEV)[:k] for _ in range(B)])
    idx[:, 5] = -1
    idx[1, 7:20] = -1
    idx = idx.reshape(B, 1, k).to(torch.int32).contiguous()
    for od in (torch.bfloat16, torch.float32):
        out = torch.empty(B, 1, H, d, device=DEV, dtype=od)
        lse = torch.empty(B, 1, H, device=DEV, dtype=torch.float32)
        csa.sparse_attn(wd["q"], wd["codes"], wd["scales"], idx, wd["win"], W, L - 1, 1.0, out, lse)
        _check_attn(wd, idx, L - 1, W, out, lse)


def test_sparse_attn_decode_sharp_softmax():
    """Decode queries split 10 ways under a sharp softmax (scale 24): the
    splits' maxima differ by tens of log2 units, so most splits' merge
    weights 2^(m_s - M) are tiny or underflow, and the running-max rescale
    fires within passes; float32 and bfloat16 outputs and lse against the
    oracle."""
    say("attn decode sharp softmax")
    B, L, d, m, H, k, W = 2, 4 * 1500, 512, 4, 64, 512, 128
    wd = _attn_world(B, L, d, m, 128, seed=48, H=H, T=1)
    g = gen(49, "idx")
    idx = torch.stack([torch.randperm(L // m, generator=g, device=DEV)[:k] for _ in range(B)])
    idx = idx.reshape(B, 1, k).to(torch.int32).contiguous()
    for od in (torch.float32, torch.bfloat16):
        out = torch.empty(B, 1, H, d, device=DEV, dtype=od)
        lse = torch.empty(B, 1, H, device=DEV, dtype=torch.float32)
        csa.sparse_attn(wd["q"], wd["codes"], wd["scales"], idx, wd["win"], W, L - 1, 24.0,
                        out, lse)
        _check_attn(wd, idx, L - 1, W, out, lse, scale=24.0)


def test_sparse_attn_prefill_block():
    """64 consecutive queries, 512 entries each (one workgroup per query)."""
    say("attn prefill block")
    B, L, d, m, H, T, k, W = 1, 4096, 512, 4, 64, 64, 512, 128
    wd = _attn_world(B, L, d, m, 2048, seed=24, H=H, T=T)
    pos0 = L - T
    g = gen(25, "idx")
    idx = torch.stack([torch.randperm((pos0 + i + 1) // m, generator=g, device=DEV)[:k]
                       for i in range(T)]).reshape(1, T, k).to(torch.int32).contiguous()
    out = torch.empty(B, T, H, d, device=DEV, dtype=torch.bfloat16)
    lse = torch.empty(B, T, H, device=DEV, dtype=torch.float32)
    csa.sparse_attn(wd["q"], wd["codes"], wd["scales"], idx, wd["win"], W, pos0, 1.0, out, lse)
    _check_attn(wd, idx, pos0, W, out, lse)


def test_sparse_attn_edges():
    say("attn edges")
    B, L, d, m, H = 2, 512, 128, 4, 16
    wd = _attn_world(B, L, d, m, 256, seed=26, H=H, T=1)
    # only -1 slots: window alone; early position: window clipped at 0
    idx = torch.full((B, 1, 40), -1, device=DEV, dtype=torch.int32)
    out = torch.empty(B, 1, H, d, device=DEV, dtype=torch.float32)
    csa.sparse_attn(wd["q"], wd["codes"], wd["scales"], idx, wd["win"], 128, L - 1, 1.0, out)
    _check_attn(wd, idx, L - 1, 128, out, None)
    wd2 = _attn_world(B, 20, d, m, 256, seed=27, H=H, T=1)
    idx2 = torch.tensor([[[0, 3, -1, 4]]] * B, device=DEV, dtype=torch.int32)
    csa.sparse_attn(wd2["q"], wd2["codes"], wd2["scales"], idx2, wd2["win"], 128, 19, 0.5, out)
    _check_attn(wd2, idx2, 19, 128, out, None, scale=0.5)
    # k = 0
    idx0 = torch.empty(B, 1, 0, device=DEV, dtype=torch.int32)
    csa.sparse_attn(wd["q"], wd["codes"], wd["scales"], idx0, wd["win"], 7, L - 1, 1.0, out)
    _check_attn(wd, idx0, L - 1, 7, out, None)


@pytest.mark.parametrize("T", [1, 20])
def test_hca_dense(T):
    say("hca dense", T)
    B, L, d, m, H, W = 2, 128 * 300, 512, 128, 64, 128
    wd = _attn_world(B, L, d, m, 256, seed=28, H=H, T=T)
    pos0 = L - T
    out = torch.empty(B, T, H, d, device=DEV, dtype=torch.bfloat16)
    lse = torch.empty(B, T, H, device=DEV, dtype=torch.float32)
    csa.hca_dense_attn(wd["q"], wd["codes"], wd["scales"], m, wd["win"], W, pos0, 1.0, out, lse)
    _check_attn(wd, None, pos0, W, out, lse, dense_m=m)


# ------------------------------------------------------------ properties ----

def test_determinism_and_batch_invariance():
    """A sequence's outputs are bit-identical across runs and whether it is
    decoded alone or inside a larger batch (a batch this small does not
    change how the slots of a query are split over workgroups)."""
    say("determinism / batch invariance")
    B, L, d, m, H, k, W = 6, 4 * 3000, 512, 4, 64, 256, 128
    wd = _attn_world(B, L, d, m, 128, seed=29, H=H, T=1)
    g = gen(30, "bi")
    qi = torch.randint(-8, 8, (B, 1, 8, 64), generator=g, device=DEV, dtype=torch.int8)
    w = torch.randint(0, 4, (B, 1, 8), generator=g, device=DEV, dtype=torch.int8)
    keys = torch.randint(-8, 8, (B, wd["cap"], 64), generator=g, device=DEV, dtype=torch.int8)

    def run(sl):
        oi = torch.empty(len(range(*sl.indices(B))), 1, k, device=DEV, dtype=torch.int32)
        csa.index_topk(qi[sl].contiguous(), w[sl].contiguous(), keys[sl].contiguous(), m, L - 1,
                       k, oi)
        out = torch.empty(oi.shape[0], 1, H, d, device=DEV, dtype=torch.bfloat16)
        csa.sparse_attn(wd["q"][sl].contiguous(), wd["codes"][sl].contiguous(),
                        wd["scales"][sl].contiguous(), oi, wd["win"][sl].contiguous(), W, L - 1,
                        1.0, out)
        torch.cuda.synchronize()
        return oi.cpu(), out.cpu()

    i_all, o_all = run(slice(0, B))
    i_again, o_again = run(slice(0, B))
    assert torch.equal(i_all, i_again) and torch.equal(o_all.view(torch.int16), o_again.view(torch.int16))
    for b in (0, 3, 5):
        i1, o1 = run(slice(b, b + 1))
        assert torch.equal(i1[0], i_all[b])
        assert torch.equal(o1[0].view(torch.int16), o_all[b].view(torch.int16))


# ------------------------------------------- output rounding, row range ----

def test_bf16_output_is_rne_of_f32():
    """The bfloat16 output is the round-to-nearest-even of the float32 output
    of the same inputs, bit for bit (the bound on attention error applies to
    the error beyond that final rounding): split decode queries (merge path),
    whole-query workgroups and the dense call."""
    say("bf16 == RNE(f32)")
    B, L, d, m, H, W = 3, 4 * 1500, 512, 4, 64, 128
    for T in (1, 20):
        wd = _attn_world(B, L, d, m, 256, seed=40 + T, H=H, T=T)
        g = gen(41, "rne", T)
        pos0 = L - T
        k = 384
        idx = torch.stack([torch.randperm((pos0 + 1) // m, generator=g, device=DEV)[:k]
                           for _ in range(B * T)]).reshape(B, T, k).to(torch.int32).contiguous()
        for dense in (False, True):
            o32 = torch.empty(B, T, H, d, device=DEV, dtype=torch.float32)
            o16 = torch.empty(B, T, H, d, device=DEV, dtype=torch.bfloat16)
            for o in (o32, o16):
                if dense:
                    csa.hca_dense_attn(wd["q"], wd["codes"], wd["scales"], m, wd["win"], W, pos0,
                                       1.0, o)
                else:
                    csa.sparse_attn(wd["q"], wd["codes"], wd["scales"], idx, wd["win"], W, pos0,
                                    1.0, o)
            torch.cuda.synchronize()
            assert torch.isfinite(o32).all()
            rne = o32.to(torch.bfloat16)   # torch's float32 -> bfloat16 is round-to-nearest-even
            assert torch.equal(o16.view(torch.int16), rne.view(torch.int16)), (T, dense)


def test_rows_outside_float16_range():
    """A selected E8M0 entry with a scale byte above 140, or a window value of
    2^16 or more, makes that query's output and lse NaN in every head and
    leaves the other queries untouched; scale bytes below 104 stay within
    the error bound (their values are below 2^-21)."""
    say("rows outside float16 range")
    B, L, d, m, H, W, k = 3, 4 * 1000, 512, 4, 64, 128, 64
    wd = _attn_world(B, L, d, m, 256, seed=45, H=H, T=1)
    g = gen(46, "range")
    idx = torch.stack([torch.randperm(L // m, generator=g, device=DEV)[:k]
                       for _ in range(B)]).reshape(B, 1, k).to(torch.int32).contiguous()
    codes, scales, win = wd["codes"].clone(), wd["scales"].clone(), wd["win"].clone()
    # sequence 0: one selected entry's first group at scale byte 141 (codes of
    # magnitude 6 there overflow float16)
    e0 = int(idx[0, 0, 5])
    scales[0, e0, 0] = 141
    codes[0, e0, 0] = 0x77
    # sequence 1: one selected entry entirely at scale byte 100 (tiny values)
    e1 = int(idx[1, 0, 9])
    scales[1, e1, :] = 100
    # sequence 2: untouched. Then the same with a huge window value in sequence 2.
    wd1 = dict(wd, codes=codes, scales=scales)
    for od in (torch.float32, torch.bfloat16):
        out = torch.empty(B, 1, H, d, device=DEV, dtype=od)
        lse = torch.empty(B, 1, H, device=DEV, dtype=torch.float32)
        csa.sparse_attn(wd["q"], codes, scales, idx, wd["win"], W, L - 1, 1.0, out, lse)
        torch.cuda.synchronize()
        assert torch.isnan(out[0].float()).all() and torch.isnan(lse[0]).all()
        assert torch.isfinite(out[1:].float()).all() and torch.isfinite(lse[1:]).all()
        # sequences 1 and 2 against the oracle (exact dequantisation of every byte)
        sub = dict(q=wd["q"][1:], codes=codes[1:], scales=scales[1:], win=wd["win"][1:])
        _check_attn(sub, idx[1:], L - 1, W, out[1:], lse[1:])
    # window value of 2^16 in sequence 2 (its ring slot of position L - 3)
    win[2, (L - 3) % win.shape[1], 17] = 65536.0
    out = torch.empty(B, 1, H, d, device=DEV, dtype=torch.float32)
    lse = torch.empty(B, 1, H, device=DEV, dtype=torch.float32)
    csa.sparse_attn(wd["q"], wd["codes"], wd["scales"], idx, win, W, L - 1, 1.0, out, lse)
    torch.cuda.synchronize()
    assert torch.isnan(out[2]).all() and torch.isnan(lse[2]).all()
    assert torch.isfinite(out[:2]).all()
    # whole-query workgroups (20 queries per sequence) take the same rule
    wd20 = _attn_world(1, L, d, m, 256, seed=47, H=H, T=20)
    sc20 = wd20["scales"].clone()
    sc20[0, 3, 1] = 200
    out = torch.empty(1, 20, H, d, device=DEV, dtype=torch.float32)
    csa.hca_dense_attn(wd20["q"], wd20["codes"], sc20, m, wd20["win"], W, L - 20, 1.0, out)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()   # entry 3 is visible to every one of the 20 queries
