"""Parity at the full workload sizes, in the launch configuration the
benchmark uses, against the CPU oracle on sampled outputs.

* decode_32k: 64 sequences x 32,768 tokens; every query checked.
* decode_1m: 8 sequences x 1,048,576 tokens; every query checked.
* prefill_128k: one 131,072-token sequence in 16 chunks of 8192 queries;
  all cache bytes checked, and the top-k and output of the first and last 256
  queries of every chunk plus 4096 seeded-random positions (about 12,000 of
  the 131,072 queries), run through the oracle on a pool of host workers.
* hca_reindex_1m: 16 sequences x 1,048,576 tokens; HCA layer (m=128, dense)
  and three CSA2 layers sharing one m=4 cache: a Full layer (top-4096 pool
  then its own top-512) and two Reindex layers rescoring the pool; every
  query of every layer checked.
Cache bytes of the 1M-token caches are checked on sampled blocks (three
8192-token chunks per sequence), recomputed by the oracle from the same
seeded latents.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import compressed_sparse_attention_compress_amd as csa
import oracle.csa_oracle as O
from oracle.pool import HostArrays, query_job
import synth
from parity_util import REL_TOL, attn_excess_error, bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def build_cache(wl, seed, layer, m, L, check_chunks=()):
    cap = -(-L // m)
    codes = torch.empty(wl.B, cap, wl.d // 2, device=DEV, dtype=torch.uint8)
    scales = torch.empty(wl.B, cap, wl.d // 32, device=DEV, dtype=torch.uint8)
    for b in range(wl.B):
        for c in range(-(-L // synth.CHUNK)):
            kv = synth.latent_chunk(wl, b, c, DEV, seed, layer)[None]
            g = synth.gate_chunk(wl, b, c, DEV, seed, layer)[None]
            csa.compress_quantize(kv, g, c * synth.CHUNK, m, codes[b:b + 1], scales[b:b + 1])
    torch.cuda.synchronize()
    for b, c in check_chunks:
        kv = synth.latent_chunk(wl, b, c, DEV, seed, layer).cpu().numpy()
        g = synth.gate_chunk(wl, b, c, DEV, seed, layer).cpu().numpy()
        rc, rs = O.compress_quantize(kv, g, m)
        b0 = c * synth.CHUNK // m
        assert np.array_equal(codes[b, b0:b0 + len(rc)].cpu().numpy(), rc), (b, c)
        assert np.array_equal(scales[b, b0:b0 + len(rs)].cpu().numpy(), rs), (b, c)
    return codes, scales


def check_topk(q_idx, w, keys, m, pos0, k, idx, cand=None, rows=None):
    qn, wn, kn, on = q_idx.cpu().numpy(), w.cpu().numpy(), keys.cpu().numpy(), idx.cpu().numpy()
    cn = cand.cpu().numpy() if cand is not None else None
    B, T = on.shape[:2]
    rows = rows if rows is not None else [(b, t) for b in range(B) for t in range(T)]
    for b, t in rows:
        ref, _ = O.index_topk(qn[b, t], wn[b, t], kn[b], m, pos0 + t, k,
                              cand=None if cn is None else cn[b, t])
        assert np.array_equal(on[b, t], ref), (b, t)


def check_attn(q, codes, scales, idx, win, W, pos0, out, rows=None, dense_m=None):
    qn, wn = bf16_bits(q), bf16_bits(win)
    on = out.float().cpu().numpy()
    idn = idx.cpu().numpy() if idx is not None else None
    B, T = q.shape[:2]
    rows = rows if rows is not None else [(b, t) for b in range(B) for t in range(T)]
    got, ref = [], []
    cache = {}
    for b, t in rows:
        if b not in cache:
            cache = {b: (codes[b].cpu().numpy(), scales[b].cpu().numpy())}
        cn, sn = cache[b]
        if dense_m is None:
            o, _ = O.sparse_attn(qn[b, t], cn, sn, idn[b, t], wn[b], wn.shape[1], W, pos0 + t, 1.0)
        else:
            o, _ = O.hca_dense_attn(qn[b, t], cn, sn, dense_m, wn[b], wn.shape[1], W, pos0 + t, 1.0)
        got.append(on[b, t])
        ref.append(o)
    ex, rms = attn_excess_error(np.stack(got), np.stack(ref), out.dtype == torch.bfloat16)
    say(f"   attention excess error / rms = {ex:.3e}")
    assert ex <= REL_TOL, ex


@pytest.mark.parametrize("name", ["decode_32k", "decode_1m"])
def test_decode_workload(name):
    wl = synth.WORKLOADS[name]
    say("workload", name)
    nch = wl.L // synth.CHUNK
    checks = [(b, c) for b in (0, wl.B - 1) for c in (0, nch // 2, nch - 1)]
    codes, scales = build_cache(wl, 0, "main", wl.m, wl.L, checks)
    keys = synth.indexer_keys(wl, DEV)
    q_idx, w = synth.indexer_queries(wl, DEV)
    q = synth.queries(wl, DEV)
    win = synth.window_ring(wl, wl.L - 1, DEV)
    idx = torch.empty(wl.B, 1, wl.k, device=DEV, dtype=torch.int32)
    out = torch.empty(wl.B, 1, wl.H, wl.d, device=DEV, dtype=torch.bfloat16)
    csa.index_topk(q_idx, w, keys, wl.m, wl.L - 1, wl.k, idx)
    csa.sparse_attn(q, codes, scales, idx, win, wl.W, wl.L - 1, 1.0, out)
    torch.cuda.synchronize()
    check_topk(q_idx, w, keys, wl.m, wl.L - 1, wl.k, idx)
    check_attn(q, codes, scales, idx, win, wl.W, wl.L - 1, out)


def test_prefill_workload(oracle_pool):
    wl = synth.WORKLOADS["prefill_128k"]
    say("workload prefill_128k")
    cap = wl.n_blocks
    codes = torch.empty(1, cap, wl.d // 2, device=DEV, dtype=torch.uint8)
    scales = torch.empty(1, cap, wl.d // 32, device=DEV, dtype=torch.uint8)
    keys = synth.indexer_keys(wl, DEV)
    win = torch.zeros(1, wl.Wcap, wl.d, device=DEV, dtype=torch.bfloat16)
    T = wl.chunk
    nch = wl.L // T
    rand = np.random.default_rng(0).choice(wl.L, 4096, replace=False)
    jobs, got = [], []
    with HostArrays() as host:
        for c in range(nch):
            t0 = c * T
            kv = synth.latent_chunk(wl, 0, c, DEV)[None].contiguous()
            gate = synth.gate_chunk(wl, 0, c, DEV)[None].contiguous()
            csa.compress_quantize(kv, gate, t0, wl.m, codes, scales)
            pos = torch.arange(t0, t0 + T, device=DEV) % wl.Wcap
            win[0, pos] = kv[0].to(torch.bfloat16)
            q_idx, w = synth.indexer_queries(wl, DEV, layer=f"chunk{c}")
            q = synth.queries(wl, DEV, layer=f"chunk{c}")
            idx = torch.empty(1, T, wl.k, device=DEV, dtype=torch.int32)
            out = torch.empty(1, T, wl.H, wl.d, device=DEV, dtype=torch.bfloat16)
            csa.index_topk(q_idx, w, keys, wl.m, t0, wl.k, idx)
            csa.sparse_attn(q, codes, scales, idx, win, wl.W, t0, 1.0, out)
            torch.cuda.synchronize()
            rc, rs = O.compress_quantize(kv[0].cpu().numpy(), gate[0].cpu().numpy(), wl.m)
            assert np.array_equal(codes[0, t0 // 4:(t0 + T) // 4].cpu().numpy(), rc), c
            assert np.array_equal(scales[0, t0 // 4:(t0 + T) // 4].cpu().numpy(), rs), c
            # first and last 256 queries of the chunk, and the chunk's share
            # of 4096 seeded-random positions over the whole sequence
            ts = sorted(set(range(256)) | set(range(T - 256, T)) |
                        {int(t) - t0 for t in rand if t0 <= t < t0 + T})
            sel = torch.tensor(ts, device=DEV)
            wref = host.put(f"win{c}", bf16_bits(win[0]))
            qi, wn = q_idx[0, sel].cpu().numpy(), w[0, sel].cpu().numpy()
            qb = bf16_bits(q[0, sel])
            for r, ti in enumerate(ts):
                jobs.append(dict(b=0, q_idx=qi[r], w=wn[r], q=qb[r], win=wref, m=wl.m,
                                 t=t0 + ti, k=wl.k, Wcap=wl.Wcap, W=wl.W, fmt="e8m0"))
            got.append((c, ts, idx[0, sel].cpu().numpy(), out[0, sel].float().cpu().numpy()))
            say(f"  chunk {c}: cache bytes exact; {len(ts)} queries sampled")
        shared = dict(keys=host.put("keys", keys.cpu().numpy()),
                      codes=host.put("codes", codes.cpu().numpy()),
                      scales=host.put("scales", scales.cpu().numpy()))
        say(f"  oracle on {len(jobs)} queries over {oracle_pool.n} workers")
        res = oracle_pool.map(query_job, [dict(j, **shared) for j in jobs])
    n = 0
    for c, ts, gi, go in got:
        ref = res[n:n + len(ts)]
        n += len(ts)
        for r, ti in enumerate(ts):
            assert np.array_equal(gi[r], ref[r][0][0]), (c, ti)
        ex, _ = attn_excess_error(go, np.stack([o for (_, o), _ in ref]), True)
        say(f"  chunk {c}: top-k exact on {len(ts)} queries; attention excess / rms = {ex:.3e}")
        assert ex <= REL_TOL, (c, ex)


def test_hca_reindex_workload():
    wl = synth.WORKLOADS["hca_reindex_1m"]
    say("workload hca_reindex_1m")
    nch = wl.L // synth.CHUNK
    t = wl.L - 1
    # HCA layer: its own latent, m = 128, dense over all 8192 entries + window
    h_codes, h_scales = build_cache(wl, 0, "hca", wl.m_hca, wl.L, [(0, 0), (wl.B - 1, nch - 1)])
    h_win = synth.window_ring(wl, t, DEV, layer="hca")
    h_q = synth.queries(wl, DEV, layer="hca")
    h_out = torch.empty(wl.B, 1, wl.H, wl.d, device=DEV, dtype=torch.bfloat16)
    csa.hca_dense_attn(h_q, h_codes, h_scales, wl.m_hca, h_win, wl.W, t, 1.0, h_out)
    torch.cuda.synchronize()
    check_attn(h_q, h_codes, h_scales, None, h_win, wl.W, t, h_out, dense_m=wl.m_hca)
    del h_codes, h_scales
    # three CSA2 layers sharing one m = 4 cache and its indexer keys
    codes, scales = build_cache(wl, 0, "main", wl.m, wl.L, [(0, nch // 3), (wl.B - 1, 7)])
    keys = synth.indexer_keys(wl, DEV)
    win = synth.window_ring(wl, t, DEV)
    pool = torch.empty(wl.B, 1, wl.pool, device=DEV, dtype=torch.int32)
    for li, layer in enumerate(["full", "reindex1", "reindex2"]):
        q_idx, w = synth.indexer_queries(wl, DEV, layer=layer)
        q = synth.queries(wl, DEV, layer=layer)
        if li == 0:
            csa.index_topk(q_idx, w, keys, wl.m, t, wl.pool, pool)
            torch.cuda.synchronize()
            check_topk(q_idx, w, keys, wl.m, t, wl.pool, pool)
        idx = torch.empty(wl.B, 1, wl.k, device=DEV, dtype=torch.int32)
        csa.index_topk(q_idx, w, keys, wl.m, t, wl.k, idx, cand=pool)
        out = torch.empty(wl.B, 1, wl.H, wl.d, device=DEV, dtype=torch.bfloat16)
        csa.sparse_attn(q, codes, scales, idx, win, wl.W, t, 1.0, out)
        torch.cuda.synchronize()
        say(f"  layer {layer}")
        check_topk(q_idx, w, keys, wl.m, t, wl.k, idx, cand=pool)
        if li == 0:
            # the Full layer's own top-k equals its top-k over the whole range
            full = torch.empty_like(idx)
            csa.index_topk(q_idx, w, keys, wl.m, t, wl.k, full)
            assert torch.equal(full, idx)
        check_attn(q, codes, scales, idx, win, wl.W, t, out)
