"""Pins of the CPU oracle against facts that do not come from the oracle.

Each pin_* function raises AssertionError when the oracle disagrees with a
closed form, a hand-derived golden value, brute force on a tiny input, a
second independent implementation, or a library routine. They take the
oracle module so that test_oracle_mutations.py can run them on an oracle with
a planted mistake and check that at least one of them fails.
"""

from __future__ import annotations

import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_float(s: str) -> float:
    return float.fromhex(s) if "0x" in s else float(s)


def load_mxfp4_groups():
    groups = []
    with open(os.path.join(GOLDEN, "mxfp4_groups.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "group":
                groups.append({"name": tok[1], "scale": int(tok[2]), "vals": [], "codes": []})
            else:
                groups[-1]["vals"].append(_parse_float(tok[0]))
                groups[-1]["codes"].append(int(tok[1], 16))
    for g in groups:
        pad = 32 - len(g["vals"])
        g["vals"] += [0.0] * pad
        g["codes"] += [0] * pad
    return groups


def load_indexer_golden():
    q, w, keys, scores, selects = None, None, [], None, []
    with open(os.path.join(GOLDEN, "indexer_small.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "q":
                q = [[int(v) for v in part.split()] for part in " ".join(tok[1:]).split(";")]
            elif tok[0] == "w":
                w = [int(v) for v in tok[1:]]
            elif tok[0] == "key":
                keys.append([int(v) for v in tok[1:]])
            elif tok[0] == "scores":
                scores = [int(v) for v in tok[1:]]
            elif tok[0] == "select":
                lhs, rhs = " ".join(tok[1:]).split(":")
                m, t, k = (int(v) for v in lhs.split())
                selects.append((m, t, k, [int(v) for v in rhs.split()]))
    return (np.array(q, np.int8), np.array(w, np.int8), np.array(keys, np.int8),
            np.array(scores), selects)


def load_pool_golden():
    pools = []
    with open(os.path.join(GOLDEN, "indexer_small.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line.startswith("pool"):
                lhs, rhs = line[4:].split(":")
                m, t, G, n = (int(v) for v in lhs.split())
                pools.append((m, t, G, n, [int(v) for v in rhs.split()]))
    return pools


# ---------------------------------------------------------------- MXFP4 ----

def pin_golden_groups(O):
    """Hand-derived codes and scale bytes (golden/mxfp4_groups.txt)."""
    groups = load_mxfp4_groups()
    p = np.array([g["vals"] for g in groups], dtype=np.float64)
    codes, scales = O.quantize_rows(p)
    for i, g in enumerate(groups):
        assert int(scales[i, 0]) == g["scale"], (g["name"], int(scales[i, 0]), g["scale"])
        got = []
        for c in range(32):
            byte = int(codes[i, c // 2])
            got.append(byte & 0xF if c % 2 == 0 else byte >> 4)
        assert got == g["codes"], (g["name"], got, g["codes"])


def pin_two_quantizers_agree(O):
    """Midpoint-compare rounding == nearest-grid search, on every finite
    bfloat16 magnitude and on the float64 neighbours of every midpoint."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16           # finite, >= 0
    a = bits.view(np.float32).astype(np.float64)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 8.0])
    extra = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 10)])
    a = np.concatenate([a, extra])
    c1 = O.e2m1_magnitude_code(a)
    c2 = O.e2m1_magnitude_code_nearest(a)
    assert np.array_equal(c1, c2), int(np.flatnonzero(c1 != c2)[0])


def pin_tie_rule(O):
    """Exact midpoints go to the even code; just above/below go to the
    nearer value (IEEE round-half-even applied to the E2M1 grid)."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    lo_code = [0, 1, 2, 3, 4, 5, 6]
    for mid, lo in zip(mids, lo_code):
        even = lo if lo % 2 == 0 else lo + 1
        assert int(O.e2m1_magnitude_code(np.array([mid]))[0]) == even, mid
        assert int(O.e2m1_magnitude_code(np.array([np.nextafter(mid, 0)]))[0]) == lo, mid
        assert int(O.e2m1_magnitude_code(np.array([np.nextafter(mid, 9)]))[0]) == lo + 1, mid
    assert int(O.e2m1_magnitude_code(np.array([1e300]))[0]) == 7


def pin_scale_rule(O):
    """For amax > 0 (and no clamping) amax / 2**e lies in [4, 8): the largest
    element codes to 4 or 6; a power-of-two amax gives exactly 4."""
    rng = np.random.default_rng(1)
    p = rng.standard_normal((200, 64)) * np.exp(rng.uniform(-20, 20, (200, 1)))
    codes, scales = O.quantize_rows(p)
    e = scales.astype(np.int64) - 127
    amax = np.abs(p.reshape(200, 2, 32)).max(axis=2)
    r = amax / np.ldexp(1.0, e)
    assert np.all((r >= 4) & (r < 8)), r.min()
    deq = O.dequantize_rows(codes, scales).reshape(200, 2, 32)
    top = np.abs(deq).max(axis=2) / np.ldexp(1.0, e)
    assert set(np.unique(top)) <= {4.0, 6.0}
    pw = np.ldexp(1.0, rng.integers(-60, 60, 50)).astype(np.float64)
    q = np.zeros((50, 32))
    q[:, 3] = -pw
    q[:, 7] = pw * 0.3
    c2, s2 = O.quantize_rows(q)
    assert np.array_equal(O.dequantize_rows(c2, s2)[:, 3], -pw)
    assert np.all(s2[:, 0].astype(np.int64) - 127 == np.log2(pw).astype(np.int64) - 2)


def pin_grid_membership(O):
    """Every dequantised value is a signed E2M1 magnitude times 2**(s-127)."""
    rng = np.random.default_rng(2)
    p = rng.standard_normal((64, 128)) * rng.lognormal(0, 2, (1, 128))
    codes, scales = O.quantize_rows(p)
    v = O.dequantize_rows(codes, scales).reshape(64, 4, 32)
    y = np.abs(v) / np.ldexp(1.0, scales.astype(np.int64) - 127)[:, :, None]
    assert set(np.unique(y)) <= {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    # and dequantisation is within half a grid step of the input (no saturation
    # below 6 * 2**e, which holds here since amax / 2**e < 8 and codes <= 6)
    err = np.abs(v - p.reshape(64, 4, 32)) / np.ldexp(1.0, scales.astype(np.int64) - 127)[:, :, None]
    assert err.max() <= 2.0 + 1e-12


def pin_idempotent(O):
    """quantize(dequantize(c, s)) == (c, s)."""
    rng = np.random.default_rng(3)
    p = rng.standard_normal((100, 64)) * rng.lognormal(0, 3, (100, 1))
    p[5, :32] = 0.0
    p[6, 3] = -0.0
    c, s = O.quantize_rows(p)
    c2, s2 = O.quantize_rows(O.dequantize_rows(c, s))
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


def pin_nibble_order(O):
    """Channel 2i is the low nibble of byte i, channel 2i+1 the high one."""
    p = np.zeros((1, 32))
    p[0, 0] = 6.0      # amax 6 -> e = 0; code 7
    p[0, 1] = 1.0      # code 2
    p[0, 2] = -0.5     # code 9
    codes, scales = O.quantize_rows(p)
    assert int(codes[0, 0]) == 0x27 and int(codes[0, 1]) == 0x09, (codes[0, :2], scales)


# -------------------------------------------------------------- pooling ----

def pin_block_count_and_bytes(O):
    """ceil(L/m) entries of d/2 + d/32 bytes; per-token bytes 17 d / (32 m)."""
    rng = np.random.default_rng(4)
    for d in (32, 128):
        for m in (1, 3, 4, 128):
            for L in (1, 2, 3, 4, 5, 127, 128, 129, 300):
                kv = rng.standard_normal((L, d)).astype(np.float32)
                g = rng.standard_normal(L).astype(np.float32)
                c, s = O.compress_quantize(kv, g, m)
                assert c.shape == (math.ceil(L / m), d // 2), (d, m, L, c.shape)
                assert s.shape == (math.ceil(L / m), d // 32)
                assert O.n_blocks(L, m) == math.ceil(L / m)
                assert c.nbytes + s.nbytes == math.ceil(L / m) * 17 * d // 32
    assert O.entry_bytes(512) == 272 and O.entry_bytes(128) == 68
    assert O.entry_bytes(512) / 4 == 68.0 and O.entry_bytes(512) / 128 == 2.125
    assert O.entry_bytes(128) / 4 == 17.0


def pin_pool_special_cases(O):
    """m = 1 returns the token; equal logits give the mean; a logit larger
    than the rest by 1000 selects its token exactly; a partial last block
    pools only the tokens present; general case == scipy softmax weights."""
    from scipy.special import softmax
    rng = np.random.default_rng(5)
    kv = rng.standard_normal((10, 64)).astype(np.float32)
    g = rng.standard_normal(10).astype(np.float32)
    assert np.array_equal(O.pool_blocks(kv, g, 1), kv.astype(np.float64))
    p = O.pool_blocks(kv[:8], np.zeros(8, np.float32), 4)
    mean = np.array([[math.fsum(kv[4 * b + j, c] for j in range(4)) / 4 for c in range(64)]
                     for b in range(2)])
    assert np.allclose(p, mean, rtol=0, atol=1e-15)
    g2 = np.zeros(8, np.float32)
    g2[2] = 1000.0
    g2[4] = 1000.0
    p2 = O.pool_blocks(kv[:8], g2, 4)
    assert np.array_equal(p2[0], kv[2].astype(np.float64))
    assert np.array_equal(p2[1], kv[4].astype(np.float64))
    p3 = O.pool_blocks(kv, g, 4)            # 10 tokens: blocks of 4, 4, 2
    assert p3.shape == (3, 64)
    w = softmax(g[8:10].astype(np.float64))
    assert np.allclose(p3[2], w @ kv[8:10].astype(np.float64), rtol=1e-14, atol=1e-15)
    w0 = softmax(g[0:4].astype(np.float64))
    assert np.allclose(p3[0], w0 @ kv[0:4].astype(np.float64), rtol=1e-14, atol=1e-15)
    # gate is per token: permuting tokens together with their logits is a no-op
    perm = np.array([2, 0, 3, 1])
    pp = O.pool_blocks(kv[:4][perm], g[:4][perm], 4)
    assert np.allclose(pp[0], p3[0], rtol=1e-14, atol=1e-15)


# -------------------------------------------------------------- indexer ----

def pin_indexer_golden(O):
    q, w, keys, scores, selects = load_indexer_golden()
    assert np.array_equal(O.index_scores(q, w, keys), scores)
    for m, t, k, want in selects:
        idx, _ = O.index_topk(q, w, keys, m, t, k)
        want = want + [-1] * (k - len(want))
        assert list(idx) == want, (m, t, k, list(idx), want)


def pin_indexer_brute_force(O):
    """Pure-Python loops on a tiny random input."""
    rng = np.random.default_rng(6)
    Hi, Di, N = 3, 5, 40
    q = rng.integers(-8, 8, (Hi, Di)).astype(np.int8)
    w = rng.integers(0, 4, Hi).astype(np.int8)
    keys = rng.integers(-8, 8, (N, Di)).astype(np.int8)
    s = O.index_scores(q, w, keys)
    for b in range(N):
        tot = 0
        for h in range(Hi):
            dot = sum(int(q[h, c]) * int(keys[b, c]) for c in range(Di))
            tot += int(w[h]) * max(0, dot)
        assert int(s[b]) == tot


def pin_indexer_identities(O):
    """relu(x) - relu(-x) = x: s(q) - s(-q) = sum_h w_h q_h . k (linear);
    a one-hot query with one unit weight scores relu(keys[:, c])."""
    rng = np.random.default_rng(7)
    q = rng.integers(-8, 8, (4, 16)).astype(np.int8)
    w = rng.integers(0, 4, 4).astype(np.int8)
    keys = rng.integers(-8, 8, (100, 16)).astype(np.int8)
    lin = keys.astype(np.int64) @ (q.astype(np.int64).T @ w.astype(np.int64))
    assert np.array_equal(O.index_scores(q, w, keys) - O.index_scores(-q, w, keys), lin)
    oh = np.zeros((4, 16), np.int8)
    oh[0, 5] = 1
    w1 = np.array([1, 0, 0, 0], np.int8)
    assert np.array_equal(O.index_scores(oh, w1, keys), np.maximum(keys[:, 5].astype(np.int64), 0))


def pin_topk_against_stable_sort(O):
    """Top-k == first k of a stable descending sort (lower index first on
    ties), returned ascending; zero weights give blocks 0..k-1; k >= visible
    returns every visible block."""
    rng = np.random.default_rng(8)
    q = rng.integers(-8, 8, (2, 8)).astype(np.int8)
    w = rng.integers(0, 4, 2).astype(np.int8)
    keys = rng.integers(-2, 2, (500, 8)).astype(np.int8)       # many ties
    for m, t, k in ((4, 1999, 37), (4, 1000, 100), (1, 499, 250), (4, 10, 5), (8, 100, 12)):
        nv = (t + 1) // m
        s = O.index_scores(q, w, keys[:nv])
        order = np.argsort(-s, kind="stable")[:k]
        want = np.full(k, -1)
        want[:min(k, nv)] = np.sort(order)
        idx, sc = O.index_topk(q, w, keys, m, t, k)
        assert np.array_equal(idx, want), (m, t, k)
        valid = idx >= 0
        assert np.array_equal(sc[valid], s[idx[valid]])
    idx, _ = O.index_topk(q, np.zeros(2, np.int8), keys, 4, 1999, 20)
    assert list(idx) == list(range(20))
    idx, _ = O.index_topk(q, w, keys, 4, 99, 30)
    assert list(idx) == list(range(25)) + [-1] * 5


def pin_reindex_consistency(O):
    """Top-k within the query's own top-C pool equals its top-k overall;
    a pool holding invisible or -1 entries ignores them."""
    rng = np.random.default_rng(9)
    q = rng.integers(-8, 8, (4, 16)).astype(np.int8)
    w = rng.integers(0, 4, 4).astype(np.int8)
    keys = rng.integers(-8, 8, (3000, 16)).astype(np.int8)
    t = 4 * 3000 - 1
    full, _ = O.index_topk(q, w, keys, 4, t, 64)
    pool, _ = O.index_topk(q, w, keys, 4, t, 512)
    re, _ = O.index_topk(q, w, keys, 4, t, 64, cand=pool)
    assert np.array_equal(full, re)
    q2 = rng.integers(-8, 8, (4, 16)).astype(np.int8)
    re2, _ = O.index_topk(q2, w, keys, 4, t, 64, cand=pool)
    s2 = O.index_scores(q2, w, keys[pool])
    order = np.argsort(-s2, kind="stable")[:64]
    assert np.array_equal(re2, np.sort(pool[order]))
    cand = np.array([5, -1, 2999, 7, 1000], np.int64)
    idx, _ = O.index_topk(q, w, keys, 4, 4 * 1000 - 1, 10, cand=cand)   # 2999 not visible
    assert set(idx[idx >= 0]) == {5, 7} and sorted(idx[idx >= 0]) == list(idx[:2])


def pin_block_pool_golden(O):
    q, w, keys, _, _ = load_indexer_golden()
    for m, t, G, n, want in load_pool_golden():
        got = O.block_pool(q, w, keys, m, t, G, n)
        assert list(got) == want, (m, t, G, n, list(got), want)


def pin_block_pool_brute_force(O):
    """Pure-Python grouping and ordering on tiny random inputs (many ties),
    and two special cases: groups of one entry give the plain top-k; keeping
    every group pools every visible entry."""
    rng = np.random.default_rng(10)
    q = rng.integers(-8, 8, (3, 6)).astype(np.int8)
    w = rng.integers(0, 4, 3).astype(np.int8)
    keys = rng.integers(-2, 3, (90, 6)).astype(np.int8)
    for m, t, G, n in ((1, 89, 8, 4), (4, 200, 8, 3), (1, 60, 5, 7), (2, 150, 4, 30), (1, 2, 8, 2)):
        nv = min((t + 1) // m, len(keys))
        sc = []
        for b in range(nv):
            tot = 0
            for h in range(3):
                dot = sum(int(q[h, c]) * int(keys[b, c]) for c in range(6))
                tot += int(w[h]) * max(0, dot)
            sc.append(tot)
        groups = {}
        for b in range(nv):
            groups.setdefault(b // G, []).append(b)
        ranked = sorted(groups, key=lambda gi: (-max(sc[b] for b in groups[gi]), gi))[:n]
        want = []
        for gi in sorted(ranked):
            want += [gi * G + r if gi * G + r < nv else -1 for r in range(G)]
        want += [-1] * (G * n - len(want))
        assert list(O.block_pool(q, w, keys, m, t, G, n)) == want, (m, t, G, n)
    t = 4 * 90 - 1
    top, _ = O.index_topk(q, w, keys, 4, t, 17)
    assert np.array_equal(O.block_pool(q, w, keys, 4, t, 1, 17), top)
    every = O.block_pool(q, w, keys, 4, t, 8, 12)
    assert sorted(e for e in every if e >= 0) == list(range(90))


def pin_block_pool_contains_topk(O):
    """Every group holding an entry scored at least s_k (the k-th best score)
    has a maximum >= s_k, and every other group a maximum < s_k; when there
    are at most n such groups, a pool of n groups therefore holds every entry
    scored >= s_k, so a Reindex top-k over it equals the Full top-k."""
    rng = np.random.default_rng(11)
    q = rng.integers(-8, 8, (4, 32)).astype(np.int8)
    w = np.array([1, 2, 3, 1], np.int8)
    keys = rng.integers(-8, 8, (4000, 32)).astype(np.int8)
    t, k, G, n = 4 * 4000 - 1, 64, 8, 64
    s = O.index_scores(q, w, keys)
    s_k = np.sort(s)[::-1][k - 1]
    hot = np.flatnonzero(s >= s_k)
    assert len(set(hot // G)) <= n
    full, _ = O.index_topk(q, w, keys, 4, t, k)
    pool = O.block_pool(q, w, keys, 4, t, G, n)
    assert set(hot) <= set(pool) and set(full) <= set(pool)
    re, _ = O.index_topk(q, w, keys, 4, t, k, cand=pool)
    assert np.array_equal(re, full)


# ------------------------------------------------------------ attention ----

def _sdpa(q, rows, scale):
    qt = torch.from_numpy(q)[None]
    kt = torch.from_numpy(rows)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)
    lse = torch.logsumexp(scale * (qt @ kt.transpose(1, 2)), dim=-1)
    return o[0].numpy(), lse[0].numpy()


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def pin_attend_vs_sdpa(O):
    rng = np.random.default_rng(10)
    q = rng.standard_normal((8, 64))
    rows = rng.standard_normal((50, 64))
    for scale in (1.0, 0.125, 3.0):
        o, lse = O.attend(q, rows, scale)
        o2, lse2 = _sdpa(q, rows, scale)
        assert np.allclose(o, o2, rtol=1e-12, atol=1e-13)
        assert np.allclose(lse, lse2, rtol=1e-12, atol=1e-13)
    o, _ = O.attend(q, rows, 0.0)
    assert np.allclose(o, rows.mean(axis=0)[None].repeat(8, 0), rtol=1e-13, atol=1e-14)
    v = rng.standard_normal(64)
    o, _ = O.attend(q, np.tile(v, (7, 1)), 1.0)
    assert np.allclose(o, v[None].repeat(8, 0), rtol=1e-13, atol=1e-14)


def _small_cache(O, rng, L=256, d=64, m=4, Wcap=64):
    kv = rng.standard_normal((L, d)).astype(np.float32)
    g = rng.standard_normal(L).astype(np.float32)
    codes, scales = O.compress_quantize(kv, g, m)
    win = np.zeros((Wcap, d), np.uint16)
    for p in range(L - Wcap, L):
        win[p % Wcap] = _bf16_bits(kv[p])
    return kv, codes, scales, win


def pin_full_coverage_is_dense(O):
    """With k covering every visible block, sparse attention is dense softmax
    attention over [every visible dequantised entry ; the window tokens]."""
    rng = np.random.default_rng(11)
    L, d, m, W, Wcap = 256, 64, 4, 16, 64
    kv, codes, scales, win = _small_cache(O, rng, L, d, m, Wcap)
    qb = _bf16_bits(rng.standard_normal((4, d)) / 8)
    qi = rng.integers(-8, 8, (2, 8)).astype(np.int8)
    wi = rng.integers(0, 4, 2).astype(np.int8)
    keys = rng.integers(-8, 8, (L // m, 8)).astype(np.int8)
    for t in (L - 1, L - 3, L - 30):
        nv = (t + 1) // m
        idx, _ = O.index_topk(qi, wi, keys, m, t, 10 ** 4)
        o, lse = O.sparse_attn(qb, codes, scales, idx, win, Wcap, W, t, 0.7)
        ent = O.dequantize_rows(codes[:nv], scales[:nv])
        wr = np.stack([O.bf16_to_f64(win[p % Wcap]) for p in range(t - W + 1, t + 1)])
        o2, lse2 = _sdpa(O.bf16_to_f64(qb), np.concatenate([ent, wr]), 0.7)
        assert np.allclose(o, o2, rtol=1e-12, atol=1e-13), t
        assert np.allclose(lse, lse2, rtol=1e-12, atol=1e-13), t
        # window rows are exactly the bf16 roundings of the latest tokens
        exact = torch.from_numpy(kv[t - W + 1:t + 1]).to(torch.bfloat16).double().numpy()
        assert np.array_equal(wr, exact)


def pin_hca_is_full_csa(O):
    rng = np.random.default_rng(12)
    L, d, m, W, Wcap = 512, 64, 128, 8, 64
    kv, codes, scales, win = _small_cache(O, rng, L, d, m, Wcap)
    qb = _bf16_bits(rng.standard_normal((3, d)) / 8)
    for t in (511, 500, 383, 127):
        nv = (t + 1) // m
        o, lse = O.hca_dense_attn(qb, codes, scales, m, win, Wcap, W, t, 1.0)
        o2, lse2 = O.sparse_attn(qb, codes, scales, np.arange(nv), win, Wcap, W, t, 1.0)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
        rows = O.gather_rows(codes, scales, np.arange(nv), win, Wcap, t, W)
        assert rows.shape[0] == nv + W


def pin_attention_invariants(O):
    """Output does not depend on the order of idx nor on -1 slots; the early
    window is clipped at position 0; the ring slot is p % Wcap."""
    rng = np.random.default_rng(13)
    L, d, m, W, Wcap = 256, 64, 4, 16, 64
    kv, codes, scales, win = _small_cache(O, rng, L, d, m, Wcap)
    qb = _bf16_bits(rng.standard_normal((4, d)) / 8)
    idx = np.array([3, 50, 7, 60, -1, 11], np.int64)
    o1, _ = O.sparse_attn(qb, codes, scales, idx, win, Wcap, W, 255, 1.0)
    o2, _ = O.sparse_attn(qb, codes, scales, idx[[5, 2, 1, 4, 0, 3]], win, Wcap, W, 255, 1.0)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-14)
    assert list(O.window_positions(5, 128)) == list(range(6))
    assert list(O.window_positions(200, 128)) == list(range(73, 201))
    rows = O.gather_rows(codes, scales, np.array([-1]), win, Wcap, 255, W)
    exact = torch.from_numpy(kv[240:256]).to(torch.bfloat16).double().numpy()
    assert np.array_equal(rows, exact)


# ------------------------------------------------------- E4M3-per-16 ----

def _e4m3_torch(byte):
    return torch.tensor(np.asarray(byte, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def pin_e4m3_values(O):
    """Hand-derived values, then every finite non-negative byte against
    torch's float8_e4m3fn decoding."""
    v = lambda b: float(O.e4m3_value(b))
    assert v(0x00) == 0.0 and v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9
    assert v(0x08) == 2.0 ** -6 and v(0x38) == 1.0 and v(0x3C) == 1.5 and v(0x7E) == 448.0
    b = np.arange(0x7F)
    assert np.array_equal(O.e4m3_value(b), _e4m3_torch(b))
    assert np.all(np.diff(O.e4m3_value(b)) > 0)


def pin_e4m3_scale_rule(O):
    """The scale byte is the E4M3 rounding of amax / 6: against torch's
    float -> float8_e4m3fn conversion (round to nearest even) away from ties,
    at constructed exact ties (to the even byte), and at the ends."""
    rng = np.random.default_rng(22)
    amax = np.abs(rng.standard_normal(20000)) * np.exp2(rng.integers(-12, 12, 20000))
    amax = amax[(amax / 6 < 440) & (amax / 6 > 2.0 ** -8)]
    ref = torch.from_numpy(amax / 6).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_scale_byte(amax)
    vals = O.e4m3_value(np.arange(0x7F))
    mids = 3.0 * (vals[:-1] + vals[1:])            # 6 x every midpoint
    near = np.isin(amax, mids)
    assert np.array_equal(got[~near], ref[~near])
    i = np.arange(0x7E)
    assert np.array_equal(O.e4m3_scale_byte(mids), np.where(i % 2 == 1, i + 1, i))
    assert np.array_equal(O.e4m3_scale_byte(np.nextafter(mids, np.inf)), i + 1)
    assert np.array_equal(O.e4m3_scale_byte(np.nextafter(mids, 0)), i)
    assert int(O.e4m3_scale_byte(0.0)) == 0 and int(O.e4m3_scale_byte(6 * 448.0)) == 0x7E
    assert int(O.e4m3_scale_byte(1e30)) == 0x7E


def pin_e4m3_quantize_brute_force(O):
    """Each element is the nearest signed E2M1 multiple of its group's scale
    (ties to the even code, saturating at 6 s; a zero scale gives zero codes):
    brute force over the 8 magnitudes, with exact ties planted."""
    rng = np.random.default_rng(23)
    nb, d = 40, 64
    p = rng.standard_normal((nb, d)) * np.exp2(rng.integers(-8, 8, (nb, 1)))
    p[0, :16] = 0.0
    codes, sb = O.quantize_rows_e4m3(p)
    s = O.e4m3_value(sb)
    assert sb.shape == (nb, d // 16) and sb[0, 0] == 0
    # plant exact midpoints: in row 1 group 0, element c = s * midpoint
    s10 = s[1, 0]
    q = p.copy()
    for c, mid in enumerate(O.E2M1_MIDPOINTS):
        q[1, 1 + c] = s10 * mid
    q[1, 0] = np.abs(p[1, :16]).max() * np.sign(p[1, 0] or 1.0)  # keep the group max
    codes2, sb2 = O.quantize_rows_e4m3(q)
    grid = np.array(O.E2M1_MAGNITUDES)
    for pp, cc, ss in ((p, codes, sb), (q, codes2, sb2)):
        nib = np.empty((nb, d), np.int64)
        nib[:, 0::2], nib[:, 1::2] = cc & 15, cc >> 4
        sc = np.repeat(O.e4m3_value(ss), 16, axis=1)
        for r in range(nb):
            for c in range(d):
                a, sv = abs(pp[r, c]), sc[r, c]
                if sv == 0:
                    want = 0
                else:
                    dist = [abs(min(a, 6 * sv) - g * sv) for g in grid]
                    best = min(dist)
                    cand = [k for k in range(8) if dist[k] == best]
                    even = [k for k in cand if k % 2 == 0]
                    want = (even or cand)[0]
                assert nib[r, c] & 7 == want, (r, c)
                assert (nib[r, c] >> 3) == int(np.signbit(pp[r, c])), (r, c)
    # the planted ties went to the even code
    assert [int(x) for x in (codes2[1, 0] >> 4, codes2[1, 1] & 15)] == [0, 2]


def pin_e4m3_dequantize(O):
    """Dequantised values are the codes times the E4M3 scale, and quantising
    them again with the same scales reproduces the codes (the grid is a
    fixed point); the group maximum is within half a grid step of its value."""
    rng = np.random.default_rng(24)
    p = rng.standard_normal((30, 128))
    codes, sb = O.quantize_rows_e4m3(p)
    x = O.dequantize_rows_e4m3(codes, sb)
    ref_scale = np.repeat(_e4m3_torch(sb), 16, axis=1)
    grid = np.array(O.E2M1_MAGNITUDES)
    nib = np.empty(p.shape, np.int64)
    nib[:, 0::2], nib[:, 1::2] = codes & 15, codes >> 4
    assert np.array_equal(x, np.where(nib & 8, -1, 1) * grid[nib & 7] * ref_scale)
    c2 = (O.e2m1_magnitude_code_scaled(np.abs(x).reshape(30, 8, 16),
                                       O.e4m3_value(sb)[:, :, None]).reshape(30, 128))
    assert np.array_equal(c2, nib & 7)
    g = np.abs(p).reshape(30, 8, 16)
    gm = g.max(axis=2)
    xm = np.abs(x).reshape(30, 8, 16)[np.arange(30)[:, None], np.arange(8)[None], g.argmax(axis=2)]
    assert np.all(np.abs(gm - xm) <= O.e4m3_value(sb) * 1.0 + 1e-300)
    # attention reads the E4M3 rows when asked to
    win = np.zeros((4, 128), np.uint16)
    rows = O.gather_rows(codes, sb, np.array([5, -1, 2]), win, 4, 3, 2, fmt="e4m3")
    assert np.array_equal(rows[:2], x[[5, 2]]) and rows.shape == (4, 128)


# --------------------------------------------------------- decode append ----

def pin_bf16_rounding(O):
    """Hand-derived roundings (ties to even), then agreement with torch's
    float32 -> bfloat16 conversion over every exponent range."""
    f = lambda v: int(O.f32_to_bf16_bits(np.float32(v)))
    assert f(1.0) == 0x3F80 and f(-1.5) == 0xBFC0 and f(0.0) == 0 and f(-0.0) == 0x8000
    assert f(1 + 2.0 ** -8) == 0x3F80                   # tie, 0x3F80 is even
    assert f(1 + 3 * 2.0 ** -8) == 0x3F82               # tie, rounds up to the even 0x3F82
    assert f(1 + 2.0 ** -8 + 2.0 ** -20) == 0x3F81      # just above the tie
    assert f(1 + 2.0 ** -7 - 2.0 ** -20) == 0x3F81      # just below 0x3F81 + half
    # subnormals: 2^-133 is the smallest bfloat16 step; halfway cases go to even
    assert f(2.0 ** -133) == 0x0001 and f(2.0 ** -134) == 0x0000 and f(3 * 2.0 ** -134) == 0x0002
    rng = np.random.default_rng(20)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-60, 60, 200000))).astype(np.float32)
    bits = rng.integers(0, 1 << 16, 20000, dtype=np.uint32)  # every low half, exact ties included
    y = ((np.uint32(0x3F12) << 16) | bits).view(np.float32)
    for v in (x, y, -y):
        assert np.array_equal(O.f32_to_bf16_bits(v), _bf16_bits(v))


def pin_cache_after_appends_brute_force(O):
    """Token-by-token simulation (ring slot p % Wcap; a staging area of m
    rows; a block pooled and quantised when its m-th token arrives) against
    the closed description, for block sizes 1, 3 and 4 and lengths that end
    on and inside a block, shorter and longer than the ring."""
    rng = np.random.default_rng(21)
    d, Wcap = 32, 8
    for m in (1, 3, 4):
        L = 29
        kv = rng.standard_normal((L, d)).astype(np.float32)
        g = rng.standard_normal(L).astype(np.float32)
        ring, stage_x, stage_g, entries = {}, [None] * m, [None] * m, []
        for n_tok in range(1, L + 1):
            p = n_tok - 1
            ring[p % Wcap] = _bf16_bits(kv[p])
            stage_x[p % m], stage_g[p % m] = kv[p], g[p]
            if (p + 1) % m == 0:
                c, sc = O.quantize_rows(O.pool_blocks(np.stack(stage_x), np.array(stage_g), m))
                entries.append((c[0], sc[0]))
            codes, scales, r = O.cache_after_appends(kv, g, m, n_tok, Wcap)
            assert codes.shape[0] == len(entries) == n_tok // m, (m, n_tok)
            for i, (c, sc) in enumerate(entries):
                assert np.array_equal(codes[i], c) and np.array_equal(scales[i], sc), (m, n_tok, i)
            assert sorted(r) == sorted(ring) if n_tok >= Wcap else sorted(r) == list(range(n_tok))
            for slot, row in r.items():
                assert np.array_equal(row, ring[slot]), (m, n_tok, slot)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
