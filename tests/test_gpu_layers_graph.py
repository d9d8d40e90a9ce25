"""The multi-layer CSA2 decode step at its full size (16 sequences at
1,048,576 tokens: an HCA layer, a Full layer whose top-4096 pool two Reindex
layers rescore, and a Reuse layer attending the Full layer's top-k; podcast
cues 12 and 14), with the CSA layers as single csa_index_attn calls, captured
in one HIP graph. Every replay, with other eager work on the same workspaces
between replays, must reproduce the eager results bit for bit; the eager
results of every sequence of every layer are checked against the oracle
(run on the pool of host workers)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import compressed_sparse_attention_compress_amd as csa
import synth
from oracle.pool import HostArrays, layers_job
from parity_util import REL_TOL, attn_excess_error, bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"
LAYERS = ("full", "reindex1", "reindex2")


def say(*a):
    print(*a, flush=True)


def _cache(wl, layer, m):
    """The layer's FP4 cache of all sequences, one compress launch per
    8192-token chunk over the whole batch."""
    cap = -(-wl.L // m)
    codes = torch.empty(wl.B, cap, wl.d // 2, device=DEV, dtype=torch.uint8)
    scales = torch.empty(wl.B, cap, wl.d // 32, device=DEV, dtype=torch.uint8)
    for c in range(wl.L // synth.CHUNK):
        kv = torch.stack([synth.latent_chunk(wl, b, c, DEV, 0, layer) for b in range(wl.B)])
        g = torch.stack([synth.gate_chunk(wl, b, c, DEV, 0, layer) for b in range(wl.B)])
        csa.compress_quantize(kv, g, c * synth.CHUNK, m, codes, scales)
    return codes, scales


def test_captured_four_layer_step_with_reuse(oracle_pool):
    wl = synth.WORKLOADS["hca_reindex_1m"]
    t = wl.L - 1
    say("setup", wl.name)
    h_codes, h_scales = _cache(wl, "hca", wl.m_hca)
    codes, scales = _cache(wl, "main", wl.m)
    keys = synth.indexer_keys(wl, DEV)
    h_win = synth.window_ring(wl, t, DEV, layer="hca")
    win = synth.window_ring(wl, t, DEV)
    h_q = synth.queries(wl, DEV, layer="hca")
    layer_in = {}
    for layer in LAYERS:
        q_idx, w = synth.indexer_queries(wl, DEV, layer=layer)
        layer_in[layer] = (q_idx, w, synth.queries(wl, DEV, layer=layer))
    rq = synth.queries(wl, DEV, layer="reuse0")
    out = {name: torch.empty(wl.B, 1, wl.H, wl.d, device=DEV, dtype=torch.bfloat16)
           for name in ("hca",) + LAYERS + ("reuse",)}
    idx = {layer: torch.empty(wl.B, 1, wl.k, device=DEV, dtype=torch.int32) for layer in LAYERS}
    pool = torch.empty(wl.B, 1, wl.pool, device=DEV, dtype=torch.int32)
    ws, ws_a, ws_f = csa.Workspace(DEV), csa.Workspace(DEV), csa.Workspace(DEV)

    def step():
        csa.hca_dense_attn(h_q, h_codes, h_scales, wl.m_hca, h_win, wl.W, t, 1.0, out["hca"],
                           workspace=ws_a)
        q_idx, w, _ = layer_in["full"]
        csa.index_topk(q_idx, w, keys, wl.m, t, wl.pool, pool, workspace=ws)
        for layer in LAYERS:
            q_idx, w, q = layer_in[layer]
            csa.index_attn(q_idx, w, keys, wl.m, t, wl.k, q, codes, scales, win, wl.W, 1.0,
                           idx[layer], out[layer], cand=pool, workspace=ws_f)
        csa.sparse_attn(rq, codes, scales, idx["full"], win, wl.W, t, 1.0, out["reuse"],
                        workspace=ws_a)

    bufs = [pool] + [idx[layer] for layer in LAYERS] + list(out.values())
    names = ["pool"] + [f"idx_{layer}" for layer in LAYERS] + [f"out_{n}" for n in out]
    step()
    torch.cuda.synchronize()
    ref = [b.clone() for b in bufs]
    say("capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    o_idx = torch.empty_like(idx["full"])
    o_out = torch.empty_like(out["full"])
    bufs_ws = (ws.buf, ws_a.buf, ws_f.buf)
    for r in range(3):
        for b in bufs:
            b.fill_(-3)
        graph.replay()
        torch.cuda.synchronize()
        for name, b, e in zip(names, bufs, ref):
            assert torch.equal(b, e), (r, name)
        # other work on the same workspaces between replays, in the layouts
        # the graph uses (a workspace that grew would leave the graph pointing
        # at freed memory): another pool, at an earlier position, rescored
        q_idx, w, q = layer_in["reindex1"]
        csa.index_topk(q_idx, w, keys, wl.m, t - 77, wl.pool, pool, workspace=ws)
        csa.index_attn(q_idx, w, keys, wl.m, t - 77, wl.k, q, codes, scales, win, wl.W, 1.0,
                       o_idx, o_out, cand=pool, workspace=ws_f)
        torch.cuda.synchronize()
        assert (ws.buf, ws_a.buf, ws_f.buf) == bufs_ws  # no workspace was replaced
        say(f"  replay {r} identical")

    # every sequence of every layer of the eager step against the oracle
    say("oracle over", wl.B, "sequences")
    ref = dict(zip(names, ref))
    with HostArrays() as host:
        shared = dict(keys=host.put("keys", keys.cpu().numpy()),
                      codes=host.put("codes", codes.cpu().numpy()),
                      scales=host.put("scales", scales.cpu().numpy()),
                      h_codes=host.put("h_codes", h_codes.cpu().numpy()),
                      h_scales=host.put("h_scales", h_scales.cpu().numpy()),
                      win=host.put("win", bf16_bits(win)),
                      h_win=host.put("h_win", bf16_bits(h_win)))
        qs_host = {layer: (layer_in[layer][0].cpu().numpy(), layer_in[layer][1].cpu().numpy(),
                           bf16_bits(layer_in[layer][2])) for layer in LAYERS}
        hq, rqb = bf16_bits(h_q), bf16_bits(rq)
        jobs = [dict(shared, b=b, t=t, m=wl.m, k=wl.k, m_hca=wl.m_hca, pool=wl.pool, n_groups=0,
                     Wcap=wl.Wcap, W=wl.W, fmt="e8m0", hq=hq[b, 0],
                     qs={layer: (v[0][b, 0], v[1][b, 0], v[2][b, 0])
                         for layer, v in qs_host.items()},
                     rq=[rqb[b, 0]]) for b in range(wl.B)]
        res = oracle_pool.map(layers_job, jobs)
    got = {name: ref[name].float().cpu().numpy() if name.startswith("out") else
           ref[name].cpu().numpy() for name in names}
    refs = {name: [] for name in ("hca",) + LAYERS + ("reuse",)}
    for b, ((ho, rpool, outs, reuse), _) in enumerate(res):
        assert np.array_equal(got["pool"][b, 0], rpool), ("pool", b)
        for layer in LAYERS:
            assert np.array_equal(got[f"idx_{layer}"][b, 0], outs[layer][0]), (layer, b)
            refs[layer].append(outs[layer][1])
        refs["hca"].append(ho)
        refs["reuse"].append(reuse[0])
    for name, rows in refs.items():
        ex, _ = attn_excess_error(got[f"out_{name}"][:, 0], np.stack(rows), True)
        say(f"  {name}: every sequence, excess / rms = {ex:.3e}")
        assert ex <= REL_TOL, (name, ex)
