"""Benchmark of the compressed sparse attention hot path on one MI355X.

Default workload, decode_1m: 8 sequences at 1,048,576 tokens, d=512, m=4
(262,144 MXFP4 entries each), 64 heads, 8x64 int8 indexer, top-1024 plus the
128-token window. One step = csa_index_topk + csa_sparse_attn for one new
query per sequence, on inputs resident in HBM. Several independent input
sets are rotated so that the 134 MB of indexer keys per step is read from
HBM rather than from the 256 MB Infinity Cache. Steps are enqueued eagerly,
each library call with its arguments marshalled once beforehand (--python-launch
times the Python wrappers instead; --graph captures one HIP graph per input set
and replays those, measured slower than eager launches on this path).

Other workloads (--workload), each printing its own line:
  decode_32k      64 sequences at 32,768 tokens, top-512 (same step).
  prefill_128k    one 131,072-token sequence in 16 chunks of 8192 queries:
                  one compress launch over the prompt, then per chunk index +
                  attention; one step = the compress and all 16 chunks.
  hca_reindex_1m  16 sequences at 1M tokens, one decode query each through
                  four layers: HCA (m=128, dense), a CSA Full layer (top-4096
                  pool, then its own top-512) and two Reindex layers scoring
                  the pool.

Prints one JSON line (see the "roofline" and "cpu_baseline" objects).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
# scale format of the FP4 caches (--fmt): E8M0 per 32 channels or E4M3 per 16
FMT = "e8m0"
SCALE_GROUP = {"e8m0": 32, "e4m3": 16}
CACHE_NAME = {"e8m0": "MXFP4 e2m1 + e8m0/32", "e4m3": "FP4 e2m1 + e4m3/16"}

METRIC = "CSA decode queries/sec + achieved HBM GB/s (% peak) at 1M ctx, 1 MI355X"
CSRC = os.path.join(ROOT, "compressed_sparse_attention_compress_amd", "csrc")
KERNEL_SOURCE = {"k_idx_scan": "indexer.hip", "k_idx_bscan": "indexer.hip",
                 "k_attn": "attn.hip", "k_compress_quantize": "compress.hip"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# input construction (untimed)
# --------------------------------------------------------------------------

def build_cache(csa, synth, wl, dev, seed, layer, m, L):
    """Compress L tokens of every sequence into an m-token MXFP4 cache: one
    launch per 8192-token chunk covering all B sequences (the cache write
    path, untimed here)."""
    import torch
    cap = -(-L // m)
    codes = torch.empty(wl.B, cap, wl.d // 2, device=dev, dtype=torch.uint8)
    scales = torch.empty(wl.B, cap, wl.d // SCALE_GROUP[FMT], device=dev, dtype=torch.uint8)
    for c in range(-(-L // synth.CHUNK)):
        kv = torch.stack([synth.latent_chunk(wl, b, c, dev, seed, layer) for b in range(wl.B)])
        g = torch.stack([synth.gate_chunk(wl, b, c, dev, seed, layer) for b in range(wl.B)])
        csa.compress_quantize(kv, g, c * synth.CHUNK, m, codes, scales, fmt=FMT)
        del kv, g
    return codes, scales


def decode_set(csa, synth, wl, dev, seed):
    import torch
    codes, scales = build_cache(csa, synth, wl, dev, seed, "main", wl.m, wl.L)
    keys = synth.indexer_keys(wl, dev, seed)
    q_idx, w = synth.indexer_queries(wl, dev, seed)
    q = synth.queries(wl, dev, seed)
    win = synth.window_ring(wl, wl.L - 1, dev, seed)
    idx = torch.empty(wl.B, 1, wl.k, device=dev, dtype=torch.int32)
    out = torch.empty(wl.B, 1, wl.H, wl.d, device=dev, dtype=torch.bfloat16)
    return dict(codes=codes, scales=scales, keys=keys, q_idx=q_idx, w=w, q=q, win=win, idx=idx,
                out=out, ws=csa.Workspace(dev), ws_attn=csa.Workspace(dev),
                ws_fused=csa.Workspace(dev))


# --------------------------------------------------------------------------
# algorithmic work
# --------------------------------------------------------------------------

def entry_bytes(wl):
    return wl.d // 2 + wl.d // SCALE_GROUP[FMT]


def decode_bytes_per_query(wl):
    """Bytes one decode query must move through one CSA layer: its keys, its
    indexer query and weights, the top-k list (written, read back), the
    selected entries, the window, q and out."""
    nv = wl.L // wl.m
    keys = nv * wl.Di
    qw = wl.Hi * wl.Di + wl.Hi
    idx = 2 * 4 * wl.k
    entries = wl.k * entry_bytes(wl)
    window = wl.W * wl.d * 2
    q_out = 2 * wl.H * wl.d * 2
    return dict(keys=keys, qw=qw, idx=idx, entries=entries, window=window, q_out=q_out,
                total=keys + qw + idx + entries + window + q_out)


def scan_bytes_per_query(wl):
    """Bytes the indexer scan kernel must move per query: its keys plus its
    indexer query and weights."""
    return (wl.L // wl.m) * wl.Di + wl.Hi * wl.Di + wl.Hi


def attn_flops(H, d, n_slots):
    """q.k and p.v multiply-adds (2 flops each) over n_slots slots, H heads."""
    return 4 * H * d * n_slots


# --------------------------------------------------------------------------
# timing helpers
# --------------------------------------------------------------------------

def capture_graphs(fns):
    """One HIP graph per callable (each already run eagerly once, so every
    workspace exists before capture)."""
    import torch
    graphs = []
    for f in fns:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f()
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def time_steps(runs, steps, warmup):
    """Warm up, then time exactly `steps` calls of runs[i % len(runs)]
    bracketed by device synchronisations. Returns seconds."""
    import torch
    for i in range(warmup):
        runs[i % len(runs)]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        runs[i % len(runs)]()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def back_to_back_ms(fn, n_sets, reps, workspaces):
    """Average device time (ms) of fn(i) launched `reps` times back to back
    (i rotating over the input sets) between two events on the current
    stream, so that the event overhead is spread over all launches. fn is a
    scan phase, which adds into the workspaces' histograms: they are zeroed
    afterwards."""
    import torch
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn(0)
    a.record(stream)
    for r in range(reps):
        fn(r % n_sets)
    b.record(stream)
    torch.cuda.synchronize()
    for ws in workspaces:
        ws.buf.zero_()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def marshalled(args, csa, fn, n_sets):
    """fn(i) for every input set with its library launches marshalled once
    (csa.prepare), unless --python-launch: a short kernel timed back to back
    or between two events then starts as soon as the stream reaches it,
    instead of after the Python wrapper's own work."""
    if args.python_launch:
        return fn
    calls = [csa.prepare(lambda i=i: fn(i)) for i in range(n_sets)]
    return lambda i: calls[i]()


def split_event_ms(first, second, n_sets, reps):
    """Average device time (ms) of first(i) measured with events on the
    current stream, second(i) following it untimed; i rotates over sets."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for r in range(reps):
        ev[r][0].record(stream)
        first(r % n_sets)
        ev[r][1].record(stream)
        if second is not None:
            second(r % n_sets)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps


def source_hash(kernel) -> str:
    path = os.path.join(CSRC, KERNEL_SOURCE[kernel])
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or
    None when they are missing or were taken on a different kernel source
    (or on the E8M0 cache when the E4M3 one is run)."""
    if FMT != "e8m0":
        workload += "_" + FMT
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration(nbytes: int, reps: int):
    """A plain device copy of known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters (each launch reads and writes nbytes)."""
    import torch
    src = torch.ones(nbytes // 4, device="cuda:0", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": reps}), flush=True)


def bf16_excess(got, ref):
    """max(|got - ref| - half a bfloat16 ulp of the larger, 0) / rms(ref)."""
    import numpy as np
    rms = float(np.sqrt(np.mean(ref ** 2)))
    half_ulp = np.ldexp(1.0, (np.floor(np.log2(np.maximum(
        np.maximum(np.abs(got), np.abs(ref)), 1e-30))) - 8).astype(int))
    return float(np.maximum(0, np.abs(got - ref) - half_ulp).max()) / rms


def host_bits(t):
    import numpy as np
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def timing_name(args):
    if args.graph:
        return "hip graph replay"
    return "eager launches (Python wrappers)" if args.python_launch else "eager launches"


def timed_runs(args, csa, steps):
    """The callables the timed loop issues, one per input set: HIP graph
    replays (--graph), the Python wrappers themselves (--python-launch), or by
    default the same library calls with their arguments marshalled once
    (csa.prepare), as a serving loop that reuses its buffers would issue them."""
    if args.graph:
        return [g.replay for g in capture_graphs(steps)]
    if args.python_launch:
        return steps
    return [csa.prepare(f) for f in steps]


# --------------------------------------------------------------------------
# cpu_baseline: the oracle over a pool of single-thread worker processes
# --------------------------------------------------------------------------

# oracle.pool.OraclePool, forked in main() before torch, the HIP library or
# the GPU are touched (so its workers hold no GPU state); None: no baseline
ORACLE_POOL = None


def pool_run(fn, jobs, min_seconds):
    return ORACLE_POOL.timed(fn, jobs, min_seconds)


def pool_record(rate, unit, n_timed, wall, per_job, sample):
    from oracle.pool import cpu_model
    n = ORACLE_POOL.n
    return dict(value=rate, unit=unit, cores=n, kind="oracle",
                sample=f"{sample}; {n_timed} jobs over {n} worker processes of one thread each "
                       f"(numpy fp64/int64), {per_job:.3f} s per job",
                cpu_model=cpu_model(), seconds=round(wall, 3))


# --------------------------------------------------------------------------
# decode (decode_1m, decode_32k)
# --------------------------------------------------------------------------

def cpu_baseline_decode(s, wl, n_queries, min_seconds):
    """The oracle on the first n_queries queries of input set s (index + top-k
    + attention each) over the worker pool; the first pass is checked against
    the device results."""
    import numpy as np
    from oracle.pool import HostArrays, query_job
    h = HostArrays()
    try:
        shared = dict(keys=h.put("keys", s["keys"][:n_queries].cpu().numpy()),
                      codes=h.put("codes", s["codes"][:n_queries].cpu().numpy()),
                      scales=h.put("scales", s["scales"][:n_queries].cpu().numpy()))
        q_idx, w = s["q_idx"].cpu().numpy(), s["w"].cpu().numpy()
        qb, win = host_bits(s["q"]), h.put("win", host_bits(s["win"])[:n_queries])
        jobs = [dict(shared, b=b, q_idx=q_idx[b, 0], w=w[b, 0], q=qb[b, 0], win=win, m=wl.m,
                     t=wl.L - 1, k=wl.k, Wcap=wl.Wcap, W=wl.W, fmt=FMT)
                for b in range(n_queries)]
        first, rate, n_timed, wall, per_job = pool_run(query_job, jobs, min_seconds)
    finally:
        h.close()
    gpu_idx = s["idx"].cpu().numpy()
    gpu_out = s["out"].cpu().float().numpy()
    idx_ok = all(bool(np.array_equal(ri, gpu_idx[b, 0])) for b, (ri, _) in enumerate(first))
    worst = max(bf16_excess(gpu_out[b, 0], ro) for b, (_, ro) in enumerate(first))
    nv = wl.L // wl.m
    return pool_record(rate, "queries/s", n_timed, wall, per_job,
                       f"{n_queries} of the {wl.B} decode queries of one step (full {nv:,}-entry "
                       f"index scan + top-{wl.k} + attention each)"), \
        dict(topk_exact=idx_ok, attn_excess_over_rms=worst)


def run_decode(args, csa, synth, wl, dev):
    import torch
    t_setup = time.time()
    sets = [decode_set(csa, synth, wl, dev, seed) for seed in range(args.sets)]
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s: {args.sets} input sets of {wl.name}")
    pos = wl.L - 1

    # the step's first kernel alone: the key scan of csa_index_attn (with the
    # per-unit short lists), or of csa_index_topk under --separate
    def scan(i):
        s = sets[i]
        if args.separate:
            csa.index_scan(s["q_idx"], s["w"], s["keys"], wl.m, pos, wl.k, s["idx"],
                           workspace=s["ws"])
        else:
            csa.index_attn(s["q_idx"], s["w"], s["keys"], wl.m, pos, wl.k, s["q"], s["codes"],
                           s["scales"], s["win"], wl.W, 1.0, s["idx"], s["out"],
                           workspace=s["ws_fused"], fmt=FMT, scan_only=True)

    def step_fn(i):
        def f():
            s = sets[i]
            if args.separate:
                csa.index_topk(s["q_idx"], s["w"], s["keys"], wl.m, pos, wl.k, s["idx"],
                               workspace=s["ws"])
                csa.sparse_attn(s["q"], s["codes"], s["scales"], s["idx"], s["win"], wl.W, pos,
                                1.0, s["out"], workspace=s["ws_attn"], fmt=FMT)
            else:
                csa.index_attn(s["q_idx"], s["w"], s["keys"], wl.m, pos, wl.k, s["q"], s["codes"],
                               s["scales"], s["win"], wl.W, 1.0, s["idx"], s["out"],
                               workspace=s["ws_fused"], fmt=FMT)
        return f

    eager = [step_fn(i) for i in range(len(sets))]
    for f in eager:
        f()
    torch.cuda.synchronize()
    runs = timed_runs(args, csa, eager)
    secs = time_steps(runs, args.steps, args.warmup)
    ms_per_step = secs * 1e3 / args.steps
    value = wl.B * args.steps / secs
    log(f"step {ms_per_step * 1e3:.1f} us, {value:.0f} queries/s ({timing_name(args)})")

    # dominant kernel: the indexer scan, timed with events on its launch stream
    # over back-to-back launches
    scan_ms = back_to_back_ms(marshalled(args, csa, scan, len(sets)), len(sets), args.steps,
                              [s["ws" if args.separate else "ws_fused"] for s in sets])
    scan_bytes = scan_bytes_per_query(wl) * wl.B
    achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
    per_q = decode_bytes_per_query(wl)
    step_gbs = per_q["total"] * wl.B / (ms_per_step * 1e-3) / 1e9
    log(f"scan {scan_ms * 1e3:.1f} us -> {achieved:.0f} GB/s")

    cpu = parity = None
    if not args.no_cpu_baseline:
        eager[0]()
        torch.cuda.synchronize()
        cpu, parity = cpu_baseline_decode(sets[0], wl, min(args.cpu_queries, wl.B),
                                          args.cpu_seconds)
        log(f"cpu baseline {cpu['value']:.3f} queries/s over {cpu['cores']} workers, "
            f"{cpu['seconds']} s; parity {parity}")

    return {
        "metric": METRIC if wl.name == "decode_1m" else
        f"CSA decode queries/sec + achieved HBM GB/s (% peak) at {wl.L // 1024}K ctx, 1 MI355X",
        "value": round(value, 1),
        "unit": "queries/s",
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.B, "context": wl.L, "d": wl.d, "m": wl.m,
            "heads": wl.H, "indexer": f"{wl.Hi}x{wl.Di} int8", "top_k": wl.k, "window": wl.W,
            "cache": CACHE_NAME[FMT], "input_sets_rotated": args.sets,
            "timing": timing_name(args),
            "step": "csa_index_topk + csa_sparse_attn" if args.separate else "csa_index_attn",
        },
        "step_hbm": {"algorithmic_bytes_per_query": per_q["total"],
                     "GB/s": round(step_gbs, 1), "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "roofline": {
            "kernel": "k_idx_scan (indexer key scan)" if args.separate else
                      "k_idx_scan (indexer key scan with per-unit short lists, the first kernel "
                      "of csa_index_attn)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("k_idx_scan", wl.name),
            "avg_launch_us": round(scan_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": scan_bytes,
        },
        "cpu_baseline": cpu,
        "parity": parity,
    }


# --------------------------------------------------------------------------
# ragged decode (decode_ragged_1m)
# --------------------------------------------------------------------------

def ragged_set(csa, synth, wl, dev, seed):
    """decode_set plus, per sequence, its position, its new token (latent and
    gate) and the staging rows of its block being filled."""
    import torch
    s = decode_set(csa, synth, wl, dev, seed)
    pos = wl.positions()
    s["pos_list"] = pos
    s["pos"] = torch.tensor(pos, dtype=torch.int64, device=dev)
    # the ring before the step holds tokens up to t - 1; the step appends t
    s["win"] = synth.window_ring(wl, [t - 1 for t in pos], dev, seed)
    s["kv_new"] = torch.stack([synth.latent_range(wl, b, t, t + 1, dev, seed)[0]
                               for b, t in enumerate(pos)]).contiguous()
    s["gate_new"] = torch.stack([synth.latent_range(wl, b, t, t + 1, dev, seed, gate=True)[0]
                                 for b, t in enumerate(pos)]).contiguous()
    s["dev"], s["seed"] = dev, seed
    s["stage"] = torch.zeros(wl.B, wl.m, wl.d, device=dev)
    s["stage_gate"] = torch.zeros(wl.B, wl.m, device=dev)
    for b, t in enumerate(pos):
        r = t % wl.m
        if r:
            s["stage"][b, :r] = synth.latent_range(wl, b, t - r, t, dev, seed)
            s["stage_gate"][b, :r] = synth.latent_range(wl, b, t - r, t, dev, seed, gate=True)
    return s


def cpu_baseline_ragged(s, wl, n_queries, min_seconds):
    """The oracle on the first n_queries sequences of a ragged step (index +
    top-k + attention at each sequence's own position) over the worker pool;
    the first pass is checked against the device results, and the entries the
    step's append completed against the oracle's compression of those blocks'
    tokens."""
    import numpy as np

    import oracle.csa_oracle as O
    import synth
    pos = s["pos_list"]
    ok = True
    for b, t in enumerate(pos):  # appended entries
        if (t + 1) % wl.m == 0:
            j0 = t + 1 - wl.m
            kv = synth.latent_range(wl, b, j0, t + 1, s["dev"], s["seed"]).cpu().numpy()
            g = synth.latent_range(wl, b, j0, t + 1, s["dev"], s["seed"], gate=True).cpu().numpy()
            quant = O.compress_quantize_e4m3 if FMT == "e4m3" else O.compress_quantize
            rc, rs = quant(kv, g, wl.m)
            blk = t // wl.m
            ok &= bool(np.array_equal(s["codes"][b, blk].cpu().numpy(), rc[0]))
            ok &= bool(np.array_equal(s["scales"][b, blk].cpu().numpy(), rs[0]))
    from oracle.pool import HostArrays, query_job
    h = HostArrays()
    try:
        shared = dict(keys=h.put("keys", s["keys"][:n_queries].cpu().numpy()),
                      codes=h.put("codes", s["codes"][:n_queries].cpu().numpy()),
                      scales=h.put("scales", s["scales"][:n_queries].cpu().numpy()))
        q_idx, w = s["q_idx"].cpu().numpy(), s["w"].cpu().numpy()
        qb, win = host_bits(s["q"]), h.put("win", host_bits(s["win"])[:n_queries])
        jobs = [dict(shared, b=b, q_idx=q_idx[b, 0], w=w[b, 0], q=qb[b, 0], win=win, m=wl.m,
                     t=pos[b], k=wl.k, Wcap=wl.Wcap, W=wl.W, fmt=FMT)
                for b in range(n_queries)]
        first, rate, n_timed, wall, per_job = pool_run(query_job, jobs, min_seconds)
    finally:
        h.close()
    gpu_idx = s["idx"].cpu().numpy()
    gpu_out = s["out"].cpu().float().numpy()
    ok &= all(bool(np.array_equal(ri, gpu_idx[b, 0])) for b, (ri, _) in enumerate(first))
    worst = max(bf16_excess(gpu_out[b, 0], ro) for b, (_, ro) in enumerate(first))
    lo, hi = min(pos[:n_queries]) // wl.m, max(pos[:n_queries]) // wl.m
    return pool_record(rate, "queries/s", n_timed, wall, per_job,
                       f"{n_queries} of the {wl.B} decode queries of one ragged step (index "
                       f"scans of {lo:,}-{hi:,} entries + top-{wl.k} + attention each)"), \
        dict(exact=ok, attn_excess_over_rms=worst)


def run_decode_ragged(args, csa, synth, wl, dev):
    """One step = append each sequence's new token, then index + attend at
    each sequence's own position (one launch each for the whole batch)."""
    import torch
    t_setup = time.time()
    sets = [ragged_set(csa, synth, wl, dev, seed) for seed in range(args.sets)]
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s: {args.sets} input sets of {wl.name}")
    pos_max = wl.L - 1

    def append(i):
        s = sets[i]
        csa.decode_append(s["kv_new"], s["gate_new"], s["pos"], wl.m, s["stage"],
                          s["stage_gate"], s["codes"], s["scales"], s["win"], fmt=FMT)

    def scan(i):
        s = sets[i]
        if args.separate:
            csa.index_scan(s["q_idx"], s["w"], s["keys"], wl.m, s["pos"], wl.k, s["idx"],
                           workspace=s["ws"], pos_max=pos_max)
        else:
            csa.index_attn(s["q_idx"], s["w"], s["keys"], wl.m, s["pos"], wl.k, s["q"],
                           s["codes"], s["scales"], s["win"], wl.W, 1.0, s["idx"], s["out"],
                           workspace=s["ws_fused"], pos_max=pos_max, fmt=FMT, scan_only=True)

    def step_fn(i):
        def f():
            s = sets[i]
            append(i)
            if args.separate:
                csa.index_topk(s["q_idx"], s["w"], s["keys"], wl.m, s["pos"], wl.k, s["idx"],
                               workspace=s["ws"], pos_max=pos_max)
                csa.sparse_attn(s["q"], s["codes"], s["scales"], s["idx"], s["win"], wl.W,
                                s["pos"], 1.0, s["out"], workspace=s["ws_attn"],
                                pos_max=pos_max, fmt=FMT)
            else:
                csa.index_attn(s["q_idx"], s["w"], s["keys"], wl.m, s["pos"], wl.k, s["q"],
                               s["codes"], s["scales"], s["win"], wl.W, 1.0, s["idx"], s["out"],
                               workspace=s["ws_fused"], pos_max=pos_max, fmt=FMT)
        return f

    eager = [step_fn(i) for i in range(len(sets))]
    for f in eager:
        f()
    torch.cuda.synchronize()
    runs = timed_runs(args, csa, eager)
    secs = time_steps(runs, args.steps, args.warmup)
    ms_per_step = secs * 1e3 / args.steps
    value = wl.B * args.steps / secs
    log(f"ragged step {ms_per_step * 1e3:.1f} us, {value:.0f} queries/s ({timing_name(args)})")

    # dominant kernel: the ragged indexer scan, timed with events on its stream
    scan_ms = back_to_back_ms(marshalled(args, csa, scan, len(sets)), len(sets), args.steps,
                              [s["ws" if args.separate else "ws_fused"] for s in sets])
    t_append = split_event_ms(marshalled(args, csa, append, len(sets)), None, len(sets),
                              args.steps)
    pos = wl.positions()
    scan_bytes = sum((t + 1) // wl.m * wl.Di + wl.Hi * wl.Di + wl.Hi for t in pos)
    log(f"append {t_append * 1e3:.1f} us; scan {scan_ms * 1e3:.1f} us")

    cpu = parity = None
    if not args.no_cpu_baseline:
        eager[0]()
        torch.cuda.synchronize()
        cpu, parity = cpu_baseline_ragged(sets[0], wl, min(args.cpu_queries, wl.B),
                                          args.cpu_seconds)
        log(f"cpu baseline {cpu['value']:.3f} queries/s over {cpu['cores']} workers, "
            f"{cpu['seconds']} s; parity {parity}")
    achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
    return {
        "metric": "CSA ragged decode queries/sec (append + index + attention) at 590K-1M ctx, "
                  "1 MI355X",
        "value": round(value, 1),
        "unit": "queries/s",
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.B, "positions": pos, "d": wl.d, "m": wl.m,
            "heads": wl.H, "indexer": f"{wl.Hi}x{wl.Di} int8", "top_k": wl.k, "window": wl.W,
            "cache": CACHE_NAME[FMT], "input_sets_rotated": args.sets,
            "timing": timing_name(args),
            "step": "csa_index_topk + csa_sparse_attn" if args.separate else "csa_index_attn",
        },
        "append_us": round(t_append * 1e3, 2),
        "roofline": {
            "kernel": "k_idx_scan (ragged indexer key scan" +
                      (")" if args.separate else " with per-unit short lists, the first kernel "
                       "of csa_index_attn)"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("k_idx_scan", wl.name),
            "avg_launch_us": round(scan_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": scan_bytes,
        },
        "cpu_baseline": cpu,
        "parity": parity,
    }


# --------------------------------------------------------------------------
# prefill (prefill_128k)
# --------------------------------------------------------------------------

def prefill_work(wl):
    """Per chunk: attention flops and indexer int8 ops of its queries."""
    att, ind = [], []
    T = wl.chunk
    for c in range(wl.L // T):
        a = i = 0
        for t in range(c * T, (c + 1) * T):
            nv = (t + 1) // wl.m
            a += attn_flops(wl.H, wl.d, min(wl.k, nv) + min(wl.W, t + 1))
            i += 2 * nv * wl.Hi * wl.Di
        att.append(a)
        ind.append(i)
    return att, ind


def cpu_baseline_prefill(wl, x, keys, codes, scales, c, n_queries, min_seconds):
    """The oracle on the last n_queries queries of chunk c (index + top-k +
    attention each) over the worker pool; the first pass is checked against
    the device results."""
    import numpy as np
    T = wl.chunk
    from oracle.pool import HostArrays, query_job
    h = HostArrays()
    try:
        shared = dict(keys=h.put("keys", keys[:1].cpu().numpy()),
                      codes=h.put("codes", codes[:1].cpu().numpy()),
                      scales=h.put("scales", scales[:1].cpu().numpy()))
        qi, wn = x["q_idx"][0].cpu().numpy(), x["w"][0].cpu().numpy()
        qb, win = host_bits(x["q"])[0], h.put("win", host_bits(x["win"])[0])
        tis = list(range(T - n_queries, T))
        jobs = [dict(shared, b=0, q_idx=qi[ti], w=wn[ti], q=qb[ti], win=win, m=wl.m,
                     t=c * T + ti, k=wl.k, Wcap=wl.Wcap, W=wl.W, fmt=FMT) for ti in tis]
        first, rate, n_timed, wall, per_job = pool_run(query_job, jobs, min_seconds)
    finally:
        h.close()
    gi = x["idx"][0].cpu().numpy()
    go = x["out"][0].cpu().float().numpy()
    ok = all(bool(np.array_equal(ri, gi[ti])) for ti, (ri, _) in zip(tis, first))
    worst = max(bf16_excess(go[ti], ro) for ti, (_, ro) in zip(tis, first))
    return pool_record(rate, "queries/s", n_timed, wall, per_job,
                       f"last {n_queries} queries of the last {T}-query chunk (index over "
                       f"{(c + 1) * T // wl.m:,} blocks + top-{wl.k} + attention each)"), \
        dict(topk_exact=ok, attn_excess_over_rms=worst)


def run_prefill(args, csa, synth, wl, dev):
    import torch
    T = wl.chunk
    nch = wl.L // T
    t_setup = time.time()
    codes = torch.empty(1, wl.n_blocks, wl.d // 2, device=dev, dtype=torch.uint8)
    scales = torch.empty(1, wl.n_blocks, wl.d // SCALE_GROUP[FMT], device=dev, dtype=torch.uint8)
    keys = synth.indexer_keys(wl, dev)
    # the prompt's latents and gate logits, [1][L][d] and [1][L]
    kv = torch.cat([synth.latent_chunk(wl, 0, c, dev) for c in range(nch)])[None].contiguous()
    gate = torch.cat([synth.gate_chunk(wl, 0, c, dev) for c in range(nch)])[None].contiguous()
    ch = []
    for c in range(nch):
        q_idx, w = synth.indexer_queries(wl, dev, layer=f"chunk{c}")
        ch.append(dict(
            q_idx=q_idx, w=w, q=synth.queries(wl, dev, layer=f"chunk{c}"),
            win=synth.window_ring(wl, (c + 1) * T - 1, dev),
            idx=torch.empty(1, T, wl.k, device=dev, dtype=torch.int32),
            out=torch.empty(1, T, wl.H, wl.d, device=dev, dtype=torch.bfloat16)))
    ws = csa.Workspace(dev)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s: {nch} chunks of {T} queries")

    def compress():
        csa.compress_quantize(kv, gate, 0, wl.m, codes, scales, fmt=FMT)

    def index(c):
        x = ch[c]
        csa.index_topk(x["q_idx"], x["w"], keys, wl.m, c * T, wl.k, x["idx"], workspace=ws)

    def attend(c):
        x = ch[c]
        csa.sparse_attn(x["q"], codes, scales, x["idx"], x["win"], wl.W, c * T, 1.0, x["out"],
                        fmt=FMT)

    def step():
        compress()
        for c in range(nch):
            index(c)
            attend(c)

    step()
    torch.cuda.synchronize()
    runs = timed_runs(args, csa, [step])
    secs = time_steps(runs, args.steps, args.warmup)
    ms_per_step = secs * 1e3 / args.steps
    value = wl.L * args.steps / secs
    log(f"prefill step {ms_per_step:.2f} ms, {value:.0f} tokens/s ({timing_name(args)})")

    # per-kernel device times (eager, events), one pass over the chunks
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nch)]
    reps = 10
    e_cmp = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e_cmp[0].record(stream)
    for _ in range(reps):
        compress()
    e_cmp[1].record(stream)
    for c in range(nch):
        ev[c][0].record(stream)
        index(c)
        ev[c][1].record(stream)
        attend(c)
        ev[c][2].record(stream)
    torch.cuda.synchronize()
    t_cmp = e_cmp[0].elapsed_time(e_cmp[1]) / reps
    t_idx = sum(ev[c][0].elapsed_time(ev[c][1]) for c in range(nch))
    t_att = sum(ev[c][1].elapsed_time(ev[c][2]) for c in range(nch))
    att, ind = prefill_work(wl)
    att_tf = sum(att) / (t_att * 1e-3) / 1e12
    ind_tops = sum(ind) / (t_idx * 1e-3) / 1e12
    cmp_bytes = wl.L * (wl.d * 4 + 4) + (wl.L // wl.m) * entry_bytes(wl)
    cmp_gbs = cmp_bytes / (t_cmp * 1e-3) / 1e9
    log(f"attention {t_att:.2f} ms -> {att_tf:.0f} TFLOP/s; indexer {t_idx:.2f} ms -> "
        f"{ind_tops:.0f} TOP/s; compress {t_cmp:.3f} ms -> {cmp_gbs:.0f} GB/s")

    cpu = parity = None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline_prefill(wl, ch[-1], keys, codes, scales, nch - 1,
                                           args.cpu_queries, args.cpu_seconds)
        log(f"cpu baseline {cpu['value']:.3f} queries/s over {cpu['cores']} workers, "
            f"{cpu['seconds']} s; parity {parity}")

    return {
        "metric": "CSA prefill tokens/sec at 128K ctx (16 chunks of 8192) + MFMA utilisation, "
                  "1 MI355X",
        "value": round(value, 1),
        "unit": "tokens/s",
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp16+int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "context": wl.L, "chunk": T, "d": wl.d, "m": wl.m,
                   "cache": CACHE_NAME[FMT],
                   "heads": wl.H, "indexer": f"{wl.Hi}x{wl.Di} int8", "top_k": wl.k,
                   "window": wl.W, "timing": timing_name(args)},
        "kernels_ms_per_step": {"compress": round(t_cmp, 4), "index_topk": round(t_idx, 4),
                                "attention": round(t_att, 4)},
        "indexer": {"bound": "mfma", "achieved": round(ind_tops, 1), "peak": INT8_PEAK_TOPS,
                    "unit": "TOP/s", "frac": round(ind_tops / INT8_PEAK_TOPS, 4),
                    "int8_ops_per_step": sum(ind)},
        "compress": {"kernel": "k_compress_quantize (the prompt's 131,072 tokens, one launch)",
                     "bound": "hbm", "achieved": round(cmp_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(cmp_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("k_compress_quantize", wl.name),
                     "avg_launch_us": round(t_cmp * 1e3, 2),
                     "algorithmic_bytes_per_launch": cmp_bytes},
        "roofline": {
            "kernel": "k_attn (sparse attention, one workgroup per query)",
            "bound": "mfma",
            "achieved": round(att_tf, 1),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(att_tf / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("k_attn", wl.name),
            "avg_launch_us": round(t_att * 1e3 / nch, 2),
            "algorithmic_flops_per_launch": round(sum(att) / nch),
        },
        "cpu_baseline": cpu,
        "parity": parity,
    }


# --------------------------------------------------------------------------
# four-layer decode (hca_reindex_1m)
# --------------------------------------------------------------------------

LAYERS = ("full", "reindex1", "reindex2")


def layers_set(csa, synth, wl, dev, seed, pool_len, n_reuse):
    import torch
    t = wl.L - 1
    s = {}
    s["h_codes"], s["h_scales"] = build_cache(csa, synth, wl, dev, seed, "hca", wl.m_hca, wl.L)
    s["h_win"] = synth.window_ring(wl, t, dev, seed, layer="hca")
    s["h_q"] = synth.queries(wl, dev, seed, layer="hca")
    s["h_out"] = torch.empty(wl.B, 1, wl.H, wl.d, device=dev, dtype=torch.bfloat16)
    s["codes"], s["scales"] = build_cache(csa, synth, wl, dev, seed, "main", wl.m, wl.L)
    s["keys"] = synth.indexer_keys(wl, dev, seed)
    s["win"] = synth.window_ring(wl, t, dev, seed)
    s["pool"] = torch.empty(wl.B, 1, pool_len, device=dev, dtype=torch.int32)
    for layer in LAYERS:
        q_idx, w = synth.indexer_queries(wl, dev, seed, layer=layer)
        s[layer] = dict(q_idx=q_idx, w=w, q=synth.queries(wl, dev, seed, layer=layer),
                        idx=torch.empty(wl.B, 1, wl.k, device=dev, dtype=torch.int32),
                        out=torch.empty(wl.B, 1, wl.H, wl.d, device=dev, dtype=torch.bfloat16))
    # Reuse layers: their own queries, the Full layer's top-k ([PODCAST] cue 12)
    s["reuse"] = [dict(q=synth.queries(wl, dev, seed, layer=f"reuse{j}"),
                       out=torch.empty(wl.B, 1, wl.H, wl.d, device=dev, dtype=torch.bfloat16))
                  for j in range(n_reuse)]
    s["ws"] = csa.Workspace(dev)
    s["ws_attn"] = csa.Workspace(dev)
    s["ws_fused"] = csa.Workspace(dev)
    return s


def cpu_baseline_layers(s, wl, n_queries, n_groups, min_seconds):
    """The oracle on the first n_queries sequences through all layers over the
    worker pool; the first pass is checked against the device results.
    n_groups > 0: the Full layer keeps a blockwise pool of n_groups 8-entry
    groups and attends its own top-k; else its pool is its top-`pool`
    entries, rescored to top-k."""
    import numpy as np
    t = wl.L - 1
    from oracle.pool import HostArrays, layers_job
    h = HostArrays()
    try:
        shared = {name: h.put(name, s[name][:n_queries].cpu().numpy())
                  for name in ("keys", "codes", "scales", "h_codes", "h_scales")}
        shared["win"] = h.put("win", host_bits(s["win"])[:n_queries])
        shared["h_win"] = h.put("h_win", host_bits(s["h_win"])[:n_queries])
        jobs = []
        for b in range(n_queries):
            qs = {layer: (s[layer]["q_idx"][b, 0].cpu().numpy(),
                          s[layer]["w"][b, 0].cpu().numpy(), host_bits(s[layer]["q"])[b, 0])
                  for layer in LAYERS}
            jobs.append(dict(shared, b=b, t=t, m=wl.m, k=wl.k, m_hca=wl.m_hca, pool=wl.pool,
                             n_groups=n_groups, Wcap=wl.Wcap, W=wl.W, fmt=FMT,
                             hq=host_bits(s["h_q"])[b, 0], qs=qs,
                             rq=[host_bits(r["q"])[b, 0] for r in s["reuse"]]))
        first, rate, n_timed, wall, per_job = pool_run(layers_job, jobs, min_seconds)
    finally:
        h.close()
    ok, worst = True, 0.0
    for b, (ho, pool, outs, reuse_o) in enumerate(first):
        ok &= bool(np.array_equal(pool, s["pool"][b, 0].cpu().numpy()))
        worst = max(worst, bf16_excess(s["h_out"][b, 0].cpu().float().numpy(), ho))
        for layer in LAYERS:
            ri, ro = outs[layer]
            ok &= bool(np.array_equal(ri, s[layer]["idx"][b, 0].cpu().numpy()))
            worst = max(worst, bf16_excess(s[layer]["out"][b, 0].cpu().float().numpy(), ro))
        for r, ro in zip(s["reuse"], reuse_o):
            worst = max(worst, bf16_excess(r["out"][b, 0].cpu().float().numpy(), ro))
    pool_txt = (f"top-{wl.k} + blockwise pool of {n_groups} 8-entry groups over "
                f"{wl.L // wl.m:,} blocks, two top-{wl.k} rescorings of the pool"
                if n_groups else
                f"top-{wl.pool} pool over {wl.L // wl.m:,} blocks, three top-{wl.k} "
                "rescorings of the pool")
    reuse_txt = (f", {len(s['reuse'])} Reuse layers attending the Full layer's top-{wl.k}"
                 if s["reuse"] else "")
    return pool_record(rate, "queries/s", n_timed, wall, per_job,
                       f"{n_queries} of the {wl.B} sequences through all layers (HCA dense "
                       f"over {wl.L // wl.m_hca:,} entries, {pool_txt} + attention{reuse_txt})"), \
        dict(topk_exact=ok, attn_excess_over_rms=worst)


def run_layers(args, csa, synth, wl, dev):
    import torch
    t = wl.L - 1
    t_setup = time.time()
    n_sets = min(args.sets, 2)
    # blockwise pool: as many 8-entry groups as make the flat pool's length,
    # unless --pool-groups says otherwise
    n_groups = (args.pool_groups or wl.pool // 8) if args.pool_kind == "blocks" else 0
    pool_len = 8 * n_groups if n_groups else wl.pool
    n_reuse = args.reuse_layers
    sets = [layers_set(csa, synth, wl, dev, seed, pool_len, n_reuse) for seed in range(n_sets)]
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s: {n_sets} input sets of {wl.name}")

    def hca(i):
        s = sets[i]
        csa.hca_dense_attn(s["h_q"], s["h_codes"], s["h_scales"], wl.m_hca, s["h_win"], wl.W, t,
                           1.0, s["h_out"], workspace=s["ws_attn"], fmt=FMT)

    def pool(i, fn="index_topk"):
        s = sets[i]
        x = s["full"]
        if n_groups:  # the Full layer's own top-k and the group pool, one key scan
            fn = {"index_topk": "index_topk_pool", "index_scan": "index_pool_scan",
                  "index_select": "index_pool_select"}[fn]
            getattr(csa, fn)(x["q_idx"], x["w"], s["keys"], wl.m, t, wl.k, x["idx"], n_groups,
                             s["pool"], workspace=s["ws"])
        else:
            getattr(csa, fn)(x["q_idx"], x["w"], s["keys"], wl.m, t, wl.pool, s["pool"],
                             workspace=s["ws"])

    def csa_layer(i, layer):
        s = sets[i]
        x = s[layer]
        if n_groups and layer == "full":  # its top-k came with the pool
            csa.sparse_attn(x["q"], s["codes"], s["scales"], x["idx"], s["win"], wl.W, t, 1.0,
                            x["out"], workspace=s["ws_attn"], fmt=FMT)
        elif not args.separate_layers:  # top-k over the pool resolved in the attention kernel
            csa.index_attn(x["q_idx"], x["w"], s["keys"], wl.m, t, wl.k, x["q"], s["codes"],
                           s["scales"], s["win"], wl.W, 1.0, x["idx"], x["out"], cand=s["pool"],
                           workspace=s["ws_fused"], fmt=FMT)
        else:
            csa.index_topk(x["q_idx"], x["w"], s["keys"], wl.m, t, wl.k, x["idx"],
                           cand=s["pool"], workspace=s["ws"])
            csa.sparse_attn(x["q"], s["codes"], s["scales"], x["idx"], s["win"], wl.W, t, 1.0,
                            x["out"], workspace=s["ws_attn"], fmt=FMT)

    def reuse_layer(i, j):
        s = sets[i]
        r = s["reuse"][j]
        csa.sparse_attn(r["q"], s["codes"], s["scales"], s["full"]["idx"], s["win"], wl.W, t,
                        1.0, r["out"], workspace=s["ws_attn"], fmt=FMT)

    def step_fn(i):
        def f():
            hca(i)
            pool(i)
            for layer in LAYERS:
                csa_layer(i, layer)
            for j in range(n_reuse):
                reuse_layer(i, j)
        return f

    eager = [step_fn(i) for i in range(n_sets)]
    for f in eager:
        f()
    torch.cuda.synchronize()
    runs = timed_runs(args, csa, eager)
    secs = time_steps(runs, args.steps, args.warmup)
    ms_per_step = secs * 1e3 / args.steps
    value = wl.B * args.steps / secs
    log(f"{4 + n_reuse}-layer step {ms_per_step * 1e3:.1f} us, {value:.0f} queries/s "
        f"({timing_name(args)})")

    # per-layer device times (eager, events)
    reps = max(4, min(args.steps, 20))
    def m(fn):
        return marshalled(args, csa, fn, n_sets)
    t_hca = split_event_ms(m(hca), None, n_sets, reps)
    t_pool = split_event_ms(m(pool), None, n_sets, reps)
    t_full = split_event_ms(m(lambda i: csa_layer(i, "full")), None, n_sets, reps)
    t_re = split_event_ms(m(lambda i: csa_layer(i, "reindex1")), None, n_sets, reps)
    t_reuse = split_event_ms(m(lambda i: reuse_layer(i, 0)), None, n_sets, reps) if n_reuse else 0.0
    scan_ms = back_to_back_ms(m(lambda i: pool(i, "index_scan")), n_sets, reps,
                              [s["ws"] for s in sets])
    nv = wl.L // wl.m
    scan_bytes = scan_bytes_per_query(wl) * wl.B
    achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
    n_hca = wl.L // wl.m_hca
    hca_flops = attn_flops(wl.H, wl.d, n_hca + wl.W) * wl.B
    hca_tf = hca_flops / (t_hca * 1e-3) / 1e12
    # algorithmic bytes per query. HCA: entries + window + q/out. Full: keys,
    # indexer query, pool list (written, read back), top-k list, entries,
    # window, q/out. Reindex: pool keys + pool ids, indexer query, top-k list,
    # entries, window, q/out. (The block pool's Full layer reads no pool back;
    # the flat-pool figure is kept for both as the bound is set by the keys.)
    eb = entry_bytes(wl)
    qo = 2 * wl.H * wl.d * 2
    win_b = wl.W * wl.d * 2
    qw = wl.Hi * wl.Di + wl.Hi
    hca_b = n_hca * eb + win_b + qo
    full_b = nv * wl.Di + qw + 2 * 4 * pool_len + 2 * 4 * wl.k + wl.k * eb + win_b + qo
    re_b = pool_len * (wl.Di + 4) + qw + 2 * 4 * wl.k + wl.k * eb + win_b + qo
    reuse_b = 4 * wl.k + wl.k * eb + win_b + qo  # top-k list read, entries, window, q/out
    per_q = hca_b + full_b + 2 * re_b + n_reuse * reuse_b
    step_gbs = per_q * wl.B / (ms_per_step * 1e-3) / 1e9
    log(f"hca {t_hca * 1e3:.1f} us ({hca_tf:.0f} TFLOP/s); pool {t_pool * 1e3:.1f} us "
        f"(scan {scan_ms * 1e3:.1f} us, {achieved:.0f} GB/s); full "
        f"{'attn' if n_groups else 'top-512+attn'} {t_full * 1e3:.1f} us; reindex "
        f"{t_re * 1e3:.1f} us" + (f"; reuse {t_reuse * 1e3:.1f} us" if n_reuse else ""))

    cpu = parity = None
    if not args.no_cpu_baseline:
        eager[0]()
        torch.cuda.synchronize()
        cpu, parity = cpu_baseline_layers(sets[0], wl, min(args.cpu_queries, wl.B), n_groups,
                                          args.cpu_seconds)
        log(f"cpu baseline {cpu['value']:.3f} queries/s over {cpu['cores']} workers, "
            f"{cpu['seconds']} s; parity {parity}")

    return {
        "metric": ("CSA2 four-layer decode queries/sec (HCA + Full + 2 Reindex) at 1M ctx, "
                   "1 MI355X" if not n_reuse else
                   f"CSA2 {4 + n_reuse}-layer decode queries/sec (HCA + Full + 2 Reindex + "
                   f"{n_reuse} Reuse) at 1M ctx, 1 MI355X"),
        "value": round(value, 1),
        "unit": "queries/s",
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "context": wl.L, "d": wl.d, "m": wl.m,
                   "cache": CACHE_NAME[FMT],
                   "m_hca": wl.m_hca, "heads": wl.H, "indexer": f"{wl.Hi}x{wl.Di} int8",
                   "pool": pool_len, "pool_kind": args.pool_kind, "reuse_layers": n_reuse,
                   **({"pool_groups": n_groups} if n_groups else {}),
                   "top_k": wl.k, "window": wl.W,
                   "input_sets_rotated": n_sets, "timing": timing_name(args),
                   "csa_layer_step": "csa_index_attn over the pool" if not args.separate_layers else
                   "csa_index_topk + csa_sparse_attn"},
        "layers_us": {"hca": round(t_hca * 1e3, 2), "full_pool_topk": round(t_pool * 1e3, 2),
                      ("full_attn" if n_groups else "full_topk_attn"): round(t_full * 1e3, 2),
                      "reindex_topk_attn": round(t_re * 1e3, 2),
                      **({"reuse_attn": round(t_reuse * 1e3, 2)} if n_reuse else {})},
        "step_hbm": {"algorithmic_bytes_per_query": per_q, "GB/s": round(step_gbs, 1),
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "hca": {"bound": "mfma", "achieved": round(hca_tf, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(hca_tf / BF16_PEAK_TFLOPS, 4),
                "flops_per_launch": hca_flops},
        "roofline": {
            "kernel": "k_idx_scan (Full layer key scan)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("k_idx_scan",
                                        wl.name + ("_blockpool" if n_groups else "")),
            "avg_launch_us": round(scan_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": scan_bytes,
        },
        "cpu_baseline": cpu,
        "parity": parity,
    }


# --------------------------------------------------------------------------
# main
# --------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_1m",
                    choices=["decode_1m", "decode_32k", "prefill_128k", "hca_reindex_1m",
                             "decode_ragged_1m"])
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--pool-kind", default="entries", choices=["entries", "blocks"],
                    help="hca_reindex_1m: the Full layer's pool is its top-`pool` entries "
                         "(entries) or a blockwise pool of 8-entry groups (blocks)")
    ap.add_argument("--reuse-layers", type=int, default=0,
                    help="hca_reindex_1m: add Reuse layers that attend the Full layer's top-k")
    ap.add_argument("--pool-groups", type=int, default=0,
                    help="groups kept by the blockwise pool (default: pool / 8)")
    ap.add_argument("--fmt", default="e8m0", choices=["e8m0", "e4m3"],
                    help="FP4 cache scales: E8M0 per 32 channels (MXFP4) or E4M3 per 16")
    ap.add_argument("--cpu-queries", type=int, default=16,
                    help="queries (sequences for hca_reindex_1m) in the cpu_baseline sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time the cpu_baseline sample is repeated for over its workers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--python-launch", action="store_true",
                    help="time the Python wrappers instead of pre-marshalled calls")
    ap.add_argument("--separate", action="store_true",
                    help="decode: time csa_index_topk + csa_sparse_attn as two calls instead of "
                         "the one-call csa_index_attn")
    ap.add_argument("--separate-layers", action="store_true",
                    help="hca_reindex_1m: run each CSA layer as csa_index_topk + csa_sparse_attn "
                         "over the pool instead of one csa_index_attn call")
    ap.add_argument("--graph", action="store_true",
                    help="time HIP graph replays instead of eager launches")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()
    global FMT
    FMT = args.fmt
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): a batch shards by "
              "sequence with no exchange between GPUs, and no run on several GPUs is made.",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        ap.error("--steps must be at least 1")
    global ORACLE_POOL
    if not args.no_cpu_baseline:
        from oracle.pool import OraclePool
        ORACLE_POOL = OraclePool()

    import torch

    import compressed_sparse_attention_compress_amd as csa
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    try:
        if args.workload == "prefill_128k":
            rec = run_prefill(args, csa, synth, wl, dev)
        elif args.workload == "hca_reindex_1m":
            rec = run_layers(args, csa, synth, wl, dev)
        elif args.workload == "decode_ragged_1m":
            rec = run_decode_ragged(args, csa, synth, wl, dev)
        else:
            rec = run_decode(args, csa, synth, wl, dev)
    finally:
        if ORACLE_POOL is not None:
            ORACLE_POOL.close()
    head = {"metric": rec.pop("metric"), "value": rec.pop("value"), "unit": rec.pop("unit"),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup}
    print(json.dumps({**head, **rec}), flush=True)


if __name__ == "__main__":
    main()
