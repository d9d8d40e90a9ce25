"""Benchmark of the compressed sparse attention hot path on one MI355X.

Default: the long-context decode workload (8 sequences at 1,048,576 tokens,
d=512, m=4 -> 262,144 MXFP4 entries each, 64 heads, 8x64 int8 indexer,
top-1024 + 128-token window). One step = csa_index_topk + csa_sparse_attn for
one new query per sequence, on inputs resident in HBM. Several independent
input sets are rotated so that the 134 MB of indexer keys per step is read
from HBM rather than from the 256 MB Infinity Cache.

Prints one JSON line (see the "roofline" and "cpu_baseline" objects).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
METRIC = "CSA decode queries/sec + achieved HBM GB/s (% peak) at 1M ctx, 1 MI355X"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# input construction (untimed)
# --------------------------------------------------------------------------

def build_cache(csa, synth, wl, dev, seed, layer, m, L):
    """Compress L tokens of every sequence into an m-token MXFP4 cache, one
    8192-token chunk at a time (the cache write path, untimed here)."""
    import torch
    cap = -(-L // m)
    codes = torch.empty(wl.B, cap, wl.d // 2, device=dev, dtype=torch.uint8)
    scales = torch.empty(wl.B, cap, wl.d // 32, device=dev, dtype=torch.uint8)
    for b in range(wl.B):
        for c in range(-(-L // synth.CHUNK)):
            kv = synth.latent_chunk(wl, b, c, dev, seed, layer)[None]
            g = synth.gate_chunk(wl, b, c, dev, seed, layer)[None]
            csa.compress_quantize(kv, g, c * synth.CHUNK, m, codes[b:b + 1], scales[b:b + 1])
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
                out=out, ws=csa.Workspace(dev))


# --------------------------------------------------------------------------
# algorithmic work
# --------------------------------------------------------------------------

def decode_bytes_per_query(wl):
    """Bytes the decode step must move per query."""
    nv = wl.L // wl.m
    ent = wl.d // 2 + wl.d // 32
    keys = nv * wl.Di
    qw = wl.Hi * wl.Di + wl.Hi
    idx = 2 * 4 * wl.k                    # idx written by the indexer, read by attention
    entries = wl.k * ent
    window = wl.W * wl.d * 2
    q_out = 2 * wl.H * wl.d * 2
    return dict(keys=keys, qw=qw, idx=idx, entries=entries, window=window, q_out=q_out,
                total=keys + qw + idx + entries + window + q_out)


def scan_bytes_per_query(wl):
    """Bytes the indexer scan kernel must move per query: its keys plus its
    indexer query and weights."""
    return (wl.L // wl.m) * wl.Di + wl.Hi * wl.Di + wl.Hi


# --------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample
# --------------------------------------------------------------------------

def cpu_baseline_decode(sets, wl, n_queries, check=True):
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle.csa_oracle as O
    s = sets[0]
    keys = s["keys"].cpu().numpy()
    q_idx, w = s["q_idx"].cpu().numpy(), s["w"].cpu().numpy()
    qb = s["q"].cpu().view(torch.int16).numpy().view(np.uint16)
    win = s["win"].cpu().view(torch.int16).numpy().view(np.uint16)
    gpu_idx = s["idx"].cpu().numpy()
    gpu_out = s["out"].cpu().float().numpy()
    t_total = 0.0
    worst = 0.0
    idx_ok = True
    with threadpool_limits(limits=1):
        for b in range(n_queries):
            codes = s["codes"][b].cpu().numpy()
            scales = s["scales"][b].cpu().numpy()
            t0 = time.perf_counter()
            ri, _ = O.index_topk(q_idx[b, 0], w[b, 0], keys[b], wl.m, wl.L - 1, wl.k)
            ro, _ = O.sparse_attn(qb[b, 0], codes, scales, ri, win[b], wl.Wcap, wl.W, wl.L - 1,
                                  1.0)
            t_total += time.perf_counter() - t0
            if check:
                idx_ok &= bool(np.array_equal(ri, gpu_idx[b, 0]))
                rms = float(np.sqrt(np.mean(ro ** 2)))
                err = np.abs(gpu_out[b, 0] - ro)
                half_ulp = np.ldexp(1.0, (np.floor(np.log2(np.maximum(
                    np.maximum(np.abs(gpu_out[b, 0]), np.abs(ro)), 1e-30))) - 8).astype(int))
                worst = max(worst, float(np.maximum(0, err - half_ulp).max()) / rms)
    return dict(value=n_queries / t_total, unit="queries/s", cores=1, kind="oracle",
                sample=f"{n_queries} of the {wl.B} decode queries of one step (full 262,144-entry "
                       f"index scan + top-{wl.k} + attention each), numpy fp64/int64, 1 thread",
                seconds=round(t_total, 3)), dict(topk_exact=idx_ok, attn_excess_over_rms=worst)


# --------------------------------------------------------------------------
# main
# --------------------------------------------------------------------------

SCAN_SOURCE = os.path.join(ROOT, "compressed_sparse_attention_compress_amd", "csrc", "indexer.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_idx_scan_decode_1m_traffic.json")


def scan_source_hash() -> str:
    import hashlib
    return hashlib.sha256(open(SCAN_SOURCE, "rb").read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per scan launch from the committed rocprofv3 counter runs, or
    None when they are missing or were taken on a different kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != scan_source_hash():
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_1m", choices=["decode_1m", "decode_32k"])
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--cpu-queries", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU layout "
              "is described in DESIGN.md and not run.", file=sys.stderr)
        sys.exit(2)

    import torch

    import compressed_sparse_attention_compress_amd as csa
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    t_setup = time.time()
    sets = [decode_set(csa, synth, wl, dev, seed) for seed in range(args.sets)]
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s: {args.sets} input sets of {wl.name}")

    def step(s):
        csa.index_topk(s["q_idx"], s["w"], s["keys"], wl.m, wl.L - 1, wl.k, s["idx"],
                       workspace=s["ws"])
        csa.sparse_attn(s["q"], s["codes"], s["scales"], s["idx"], s["win"], wl.W, wl.L - 1, 1.0,
                        s["out"])

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = wl.B * args.steps / (t1 - t0)
    log(f"step {ms_per_step * 1e3:.1f} us, {value:.0f} queries/s")

    # dominant kernel: the indexer scan, timed with events on the launch stream
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    ev_step = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for i in range(args.steps):
        s = sets[i % len(sets)]
        ev_step[i][0].record(stream)
        ev[i][0].record(stream)
        csa.index_scan(s["q_idx"], s["w"], s["keys"], wl.m, wl.L - 1, wl.k, s["idx"],
                       workspace=s["ws"])
        ev[i][1].record(stream)
        csa.index_select(s["q_idx"], s["w"], s["keys"], wl.m, wl.L - 1, wl.k, s["idx"],
                         workspace=s["ws"])
        csa.sparse_attn(s["q"], s["codes"], s["scales"], s["idx"], s["win"], wl.W, wl.L - 1, 1.0,
                        s["out"])
        ev_step[i][1].record(stream)
    torch.cuda.synchronize()
    scan_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    step_ev_ms = sum(a.elapsed_time(b) for a, b in ev_step) / len(ev_step)
    scan_bytes = scan_bytes_per_query(wl) * wl.B
    achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
    per_q = decode_bytes_per_query(wl)
    step_gbs = per_q["total"] * wl.B / (ms_per_step * 1e-3) / 1e9
    log(f"scan {scan_ms * 1e3:.1f} us -> {achieved:.0f} GB/s; step (events) {step_ev_ms * 1e3:.1f} us")

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        step(sets[0])
        torch.cuda.synchronize()
        cpu, parity = cpu_baseline_decode(sets, wl, min(args.cpu_queries, wl.B))
        log(f"cpu baseline {cpu['value']:.3f} queries/s over {cpu['seconds']} s; parity {parity}")

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.B, "context": wl.L, "d": wl.d, "m": wl.m,
            "heads": wl.H, "indexer": f"{wl.Hi}x{wl.Di} int8", "top_k": wl.k, "window": wl.W,
            "cache": "MXFP4 e2m1 + e8m0/32", "input_sets_rotated": args.sets,
        },
        "step_hbm": {"algorithmic_bytes_per_query": per_q["total"],
                     "GB/s": round(step_gbs, 1), "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "roofline": {
            "kernel": "k_idx_scan (indexer key scan)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "avg_launch_us": round(scan_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": scan_bytes,
        },
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
