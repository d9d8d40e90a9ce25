"""The oracle's worker pool returns what direct oracle calls return."""

from __future__ import annotations

import numpy as np

import oracle.csa_oracle as O
from oracle.pool import HostArrays, layers_job, query_job


def _bf16(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _case(rng, B=2, L=2048, m=4, d=64, Hi=4, Di=32, H=4, W=16, Wcap=32):
    nv = L // m
    keys = rng.integers(-127, 128, (B, nv, Di), dtype=np.int8)
    cs = [O.compress_quantize(rng.standard_normal((L, d)), rng.standard_normal(L), m)
          for _ in range(B)]
    codes, scales = np.stack([c for c, _ in cs]), np.stack([s for _, s in cs])
    win = _bf16(rng.standard_normal((B, Wcap, d)))
    return dict(B=B, L=L, m=m, d=d, Hi=Hi, Di=Di, H=H, W=W, Wcap=Wcap, keys=keys, codes=codes,
                scales=scales, win=win)


def test_query_jobs_match_direct_calls(oracle_pool):
    rng = np.random.default_rng(3)
    c = _case(rng)
    jobs = []
    with HostArrays() as host:
        shared = {n: host.put(n, c[n]) for n in ("keys", "codes", "scales", "win")}
        for j in range(6):
            b, t = j % c["B"], int(rng.integers(100, c["L"]))
            jobs.append(dict(shared, b=b, t=t, m=c["m"], k=24, Wcap=c["Wcap"], W=c["W"],
                             fmt="e8m0",
                             q_idx=rng.integers(-127, 128, (c["Hi"], c["Di"]), dtype=np.int8),
                             w=rng.integers(-127, 128, c["Hi"], dtype=np.int8),
                             q=_bf16(rng.standard_normal((c["H"], c["d"])))))
        res = oracle_pool.map(query_job, jobs)
    for job, ((ri, ro), secs) in zip(jobs, res):
        b, t = job["b"], job["t"]
        ref_i, _ = O.index_topk(job["q_idx"], job["w"], c["keys"][b], c["m"], t, 24)
        ref_o, _ = O.sparse_attn(job["q"], c["codes"][b], c["scales"][b], ref_i, c["win"][b],
                                 c["Wcap"], c["W"], t, 1.0)
        assert np.array_equal(ri, ref_i)
        assert np.array_equal(ro, ref_o)
        assert secs >= 0


def test_layers_job_matches_direct_calls(oracle_pool):
    rng = np.random.default_rng(4)
    c = _case(rng, B=1)
    m_hca, t, k, pool_n = 16, c["L"] - 1, 16, 64
    hc, hs = O.compress_quantize(rng.standard_normal((c["L"], c["d"])),
                                 rng.standard_normal(c["L"]), m_hca)
    h_win = _bf16(rng.standard_normal((c["Wcap"], c["d"])))
    hq = _bf16(rng.standard_normal((c["H"], c["d"])))
    qs = {layer: (rng.integers(-127, 128, (c["Hi"], c["Di"]), dtype=np.int8),
                  rng.integers(-127, 128, c["Hi"], dtype=np.int8),
                  _bf16(rng.standard_normal((c["H"], c["d"]))))
          for layer in ("full", "reindex1")}
    rq = [_bf16(rng.standard_normal((c["H"], c["d"])))]
    job = dict(b=0, t=t, m=c["m"], k=k, m_hca=m_hca, pool=pool_n, n_groups=0, Wcap=c["Wcap"],
               W=c["W"], fmt="e8m0", keys=c["keys"], codes=c["codes"], scales=c["scales"],
               h_codes=hc[None], h_scales=hs[None], hq=hq, h_win=h_win, win=c["win"][0], qs=qs,
               rq=rq)
    (ho, pool, outs, reuse), _ = oracle_pool.map(layers_job, [job])[0]
    ref_h, _ = O.hca_dense_attn(hq, hc, hs, m_hca, h_win, c["Wcap"], c["W"], t, 1.0)
    assert np.array_equal(ho, ref_h)
    ref_pool, _ = O.index_topk(qs["full"][0], qs["full"][1], c["keys"][0], c["m"], t, pool_n)
    assert np.array_equal(pool, ref_pool)
    for layer, (qi, wi, qb) in qs.items():
        ri, _ = O.index_topk(qi, wi, c["keys"][0], c["m"], t, k, cand=ref_pool)
        assert np.array_equal(outs[layer][0], ri)
    ro, _ = O.sparse_attn(rq[0], c["codes"][0], c["scales"][0], outs["full"][0], c["win"][0],
                          c["Wcap"], c["W"], t, 1.0)
    assert np.array_equal(reuse[0], ro)


def test_timed_pass_reports_a_rate(oracle_pool):
    rng = np.random.default_rng(5)
    c = _case(rng, B=1, L=512)
    job = dict(b=0, t=400, m=c["m"], k=8, Wcap=c["Wcap"], W=c["W"], fmt="e8m0",
               keys=c["keys"], codes=c["codes"], scales=c["scales"], win=c["win"][0],
               q_idx=rng.integers(-127, 128, (c["Hi"], c["Di"]), dtype=np.int8),
               w=rng.integers(-127, 128, c["Hi"], dtype=np.int8),
               q=_bf16(rng.standard_normal((c["H"], c["d"]))))
    first, rate, n_timed, wall, per_job = oracle_pool.timed(query_job, [job], 0.2)
    assert len(first) == 1 and rate > 0 and n_timed % oracle_pool.n == 0 and wall > 0
