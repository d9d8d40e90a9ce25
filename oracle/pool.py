"""Runs the CPU oracle over a pool of single-thread worker processes.

TEST INFRASTRUCTURE ONLY, like the oracle itself: the test-suite and the CPU
baseline leg of the benchmark use it to check and time many queries at once.
It adds no arithmetic of its own: each job calls the oracle's functions on one
query (or one sequence through several layers) exactly as a single-threaded
caller would.

The workers are forked, so start the pool before anything in the process has
touched the GPU: they then hold no GPU state. Large inputs go to the workers as
memory-mapped files (HostArrays), so a job carries only names, scalars and the
query's own small arrays.
"""

from __future__ import annotations

import math
import os
import tempfile
import time

import numpy as np

from . import csa_oracle as O

_OPENED: dict = {}
_LIMITS = None


def pool_size(cap: int = 16) -> int:
    """Host CPUs this process may run on, capped at `cap`."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _init_worker():
    from threadpoolctl import threadpool_limits
    global _LIMITS
    _LIMITS = threadpool_limits(limits=1)  # one BLAS thread per worker, for its lifetime


class OraclePool:
    """A fork-started multiprocessing pool of single-thread oracle workers."""

    def __init__(self, n: int | None = None):
        import multiprocessing as mp
        self.n = n or pool_size()
        self.pool = mp.get_context("fork").Pool(self.n, initializer=_init_worker)

    def map(self, fn, jobs):
        return self.pool.map(fn, jobs, chunksize=1)

    def timed(self, fn, jobs, min_seconds):
        """Every job once (those results are returned), then the jobs
        round-robin for about min_seconds of wall time. Returns (results,
        jobs per wall second of the second pass, jobs in it, its wall time,
        mean seconds per job inside a worker in the first pass)."""
        t0 = time.perf_counter()
        first = self.map(fn, jobs)
        wall_first = time.perf_counter() - t0
        per_job = sum(s for _, s in first) / len(first)
        # sized by the slower of the workers' own time and the first pass's
        # wall clock per job slot (which includes moving the jobs over)
        per_slot = max(per_job, wall_first / math.ceil(len(jobs) / self.n))
        n_timed = max(self.n, math.ceil(min_seconds * self.n / max(per_slot, 1e-6)))
        n_timed = -(-n_timed // self.n) * self.n
        t0 = time.perf_counter()
        self.map(fn, [jobs[i % len(jobs)] for i in range(n_timed)])
        wall = time.perf_counter() - t0
        return [r for r, _ in first], n_timed / wall, n_timed, wall, per_job

    def close(self):
        self.pool.terminate()
        self.pool.join()


class HostArrays:
    """Arrays written once to memory-mapped .npy files that the workers open
    by path; put() returns the reference a job passes instead of the array."""

    def __init__(self):
        base = "/dev/shm" if os.path.isdir("/dev/shm") else None
        self.dir = tempfile.mkdtemp(prefix="csa_oracle_", dir=base)
        self.paths = []

    def put(self, name, arr):
        arr = np.ascontiguousarray(arr)
        path = os.path.join(self.dir, name + ".npy")
        mm = np.lib.format.open_memmap(path, mode="w+", dtype=arr.dtype, shape=arr.shape)
        mm[...] = arr
        mm.flush()
        del mm
        self.paths.append(path)
        return ("file", path)

    def close(self):
        for p in self.paths:
            os.unlink(p)
        os.rmdir(self.dir)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _arg(ref):
    if isinstance(ref, tuple) and len(ref) == 2 and ref[0] == "file":
        if ref[1] not in _OPENED:
            _OPENED[ref[1]] = np.load(ref[1], mmap_mode="r")
        return _OPENED[ref[1]]
    return ref


def _row(win, b):
    """A window ring [Wcap][d], or row b of a batch of them [B][Wcap][d]."""
    return win[b] if win.ndim == 3 else win


def query_job(job):
    """One query: the oracle's top-k over the b-th sequence's keys at position
    t, then its attention over those entries and the window. Returns
    ((top-k, output), seconds)."""
    a = {k: _arg(v) for k, v in job.items()}
    b, win = a["b"], _row(a["win"], a["b"])
    t0 = time.perf_counter()
    ri, _ = O.index_topk(a["q_idx"], a["w"], a["keys"][b], a["m"], a["t"], a["k"])
    ro, _ = O.sparse_attn(a["q"], a["codes"][b], a["scales"][b], ri, win, a["Wcap"], a["W"],
                          a["t"], 1.0, fmt=a["fmt"])
    return (ri, ro), time.perf_counter() - t0


def layers_job(job):
    """One sequence through a multi-layer decode step: the HCA layer (dense),
    the Full layer's candidate pool (its top-`pool` entries, or a blockwise
    pool of n_groups 8-entry groups), each CSA layer's top-k (Reindex layers
    over the pool) and attention, and Reuse layers attending the Full layer's
    top-k. Returns ((hca output, pool, {layer: (top-k, output)}, [reuse
    outputs]), seconds)."""
    a = {k: _arg(v) for k, v in job.items()}
    b, t, m, k, fmt = a["b"], a["t"], a["m"], a["k"], a["fmt"]
    keys, cn, sn = a["keys"][b], a["codes"][b], a["scales"][b]
    win, h_win = _row(a["win"], b), _row(a["h_win"], b)
    qs = a["qs"]
    t0 = time.perf_counter()
    ho, _ = O.hca_dense_attn(a["hq"], a["h_codes"][b], a["h_scales"][b], a["m_hca"], h_win,
                             a["Wcap"], a["W"], t, 1.0, fmt=fmt)
    if a["n_groups"]:
        pool = O.block_pool(qs["full"][0], qs["full"][1], keys, m, t, 8, a["n_groups"])
    else:
        pool, _ = O.index_topk(qs["full"][0], qs["full"][1], keys, m, t, a["pool"])
    outs = {}
    for layer, (qi, wi, qb) in qs.items():
        cand = None if (a["n_groups"] and layer == "full") else pool
        ri, _ = O.index_topk(qi, wi, keys, m, t, k, cand=cand)
        ro, _ = O.sparse_attn(qb, cn, sn, ri, win, a["Wcap"], a["W"], t, 1.0, fmt=fmt)
        outs[layer] = (ri, ro)
    reuse = [O.sparse_attn(rq, cn, sn, outs["full"][0], win, a["Wcap"], a["W"], t, 1.0,
                           fmt=fmt)[0] for rq in a["rq"]]
    return (ho, pool, outs, reuse), time.perf_counter() - t0
