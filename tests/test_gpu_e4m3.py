"""GPU parity of the FP4 cache with one E4M3 scale per 16 channels (the scale
layout the podcast's cue 16 names): compression, dequantisation, decode
append and attention against the oracle's E4M3 functions (bit-exact bytes,
2e-3 x RMS beyond the output rounding for attention)."""

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
FMT = "e4m3"


def gen(seed, *parts):
    return synth.generator(DEV, seed, *parts)


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_dequantize_e4m3(dtype):
    """Every code with every finite scale byte, exactly."""
    say("dequantize e4m3", dtype)
    B, cap, d = 2, 80, 256
    g = gen(90, "deq16")
    codes = torch.randint(0, 256, (B, cap, d // 2), generator=g, device=DEV, dtype=torch.uint8)
    scales = torch.randint(0, 0x7F, (B, cap, d // 16), generator=g, device=DEV).to(torch.uint8)
    # every finite scale byte appears in the dequantised rows
    scales[0, 3:11] = torch.arange(128, device=DEV).clamp(max=0x7E).reshape(8, 16).to(torch.uint8)
    out = torch.empty(B, 60, d, device=DEV, dtype=dtype)
    csa.dequantize(codes, scales, 3, 60, out, fmt=FMT)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    for b in range(B):
        ref = O.dequantize_rows_e4m3(c[b, 3:63], s[b, 3:63])
        got = out[b].cpu().double().numpy()
        assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:5]


def _compress_case(B, L, d, m, tok0, seed, scale=1.0, chunks=None):
    g = gen(seed, "cmp16", B, L, d, m)
    kv = torch.randn(B, L, d, generator=g, device=DEV) * scale
    gate = torch.randn(B, L, generator=g, device=DEV)
    cap = O.n_blocks(tok0 + L, m) + 3
    codes = torch.full((B, cap, d // 2), 0xAB, device=DEV, dtype=torch.uint8)
    scales = torch.full((B, cap, d // 16), 0xCD, device=DEV, dtype=torch.uint8)
    t = 0
    for n in chunks or [L]:
        csa.compress_quantize(kv[:, t:t + n].contiguous(), gate[:, t:t + n].contiguous(),
                              tok0 + t, m, codes, scales, fmt=FMT)
        t += n
    torch.cuda.synchronize()
    kvn, gn = kv.cpu().numpy(), gate.cpu().numpy()
    cn, sn = codes.cpu().numpy(), scales.cpu().numpy()
    b0 = tok0 // m
    for b in range(B):
        rc, rs = O.compress_quantize_e4m3(kvn[b], gn[b], m)
        nb = rc.shape[0]
        assert np.array_equal(cn[b, b0:b0 + nb], rc), (b, np.argwhere(cn[b, b0:b0 + nb] != rc)[:4])
        assert np.array_equal(sn[b, b0:b0 + nb], rs), (b, np.argwhere(sn[b, b0:b0 + nb] != rs)[:4])
        assert (cn[b, :b0] == 0xAB).all() and (cn[b, b0 + nb:] == 0xAB).all()
        assert (sn[b, b0 + nb:] == 0xCD).all()
    return sn


@pytest.mark.parametrize("d", [32, 128, 512])
@pytest.mark.parametrize("m", [1, 4, 128])
def test_compress_e4m3(d, m):
    say("compress e4m3", d, m)
    _compress_case(2, 517, d, m, 0, seed=91)


def test_compress_e4m3_scale_range():
    """Subnormal scales, saturation at 448 and all-zero scales."""
    say("compress e4m3 range")
    sn = _compress_case(1, 400, 128, 4, 8, seed=92, scale=3e-3)
    assert (sn[0, 2:102] < 8).any()                   # some scales are subnormal
    sn = _compress_case(1, 400, 128, 1, 0, seed=93, scale=2e3)
    assert (sn[0, :400] == 0x7E).any()                # some groups saturate
    sn = _compress_case(2, 64, 64, 4, 0, seed=94, scale=1e-30, chunks=[24, 40])
    assert (sn[:, :16] == 0).all()


def test_decode_append_e4m3():
    say("decode append e4m3")
    B, d, m, Wcap = 3, 128, 4, 16
    starts, ends = [0, 10, 33], [37, 64, 101]
    Lmax = max(ends)
    g = gen(95, "append16")
    kv = torch.randn(B, Lmax, d, generator=g, device=DEV)
    gate = torch.randn(B, Lmax, generator=g, device=DEV)
    cap = Lmax // m + 2
    codes = torch.zeros(B, cap, d // 2, device=DEV, dtype=torch.uint8)
    scales = torch.zeros(B, cap, d // 16, device=DEV, dtype=torch.uint8)
    win = torch.zeros(B, Wcap, d, device=DEV, dtype=torch.bfloat16)
    stage = torch.zeros(B, m, d, device=DEV)
    stage_gate = torch.zeros(B, m, device=DEV)
    for b in range(B):
        P = starts[b]
        if P:
            csa.compress_quantize(kv[b:b + 1, :P].contiguous(), gate[b:b + 1, :P].contiguous(), 0,
                                  m, codes[b:b + 1], scales[b:b + 1], fmt=FMT)
            r = P % m
            stage[b, :r] = kv[b, P - r:P]
            stage_gate[b, :r] = gate[b, P - r:P]
    ar = torch.arange(B, device=DEV)
    for s in range(max(e - st for st, e in zip(starts, ends))):
        host = [st + s if st + s < e else -1 for st, e in zip(starts, ends)]
        pos = torch.tensor(host, dtype=torch.int64, device=DEV)
        idx = pos.clamp(min=0)
        csa.decode_append(kv[ar, idx].contiguous(), gate[ar, idx].contiguous(), pos, m, stage,
                          stage_gate, codes, scales, win, fmt=FMT)
    torch.cuda.synchronize()
    kvn, gn = kv.cpu().numpy(), gate.cpu().numpy()
    for b in range(B):
        nb = ends[b] // m
        rc, rs = O.compress_quantize_e4m3(kvn[b, :nb * m], gn[b, :nb * m], m)
        assert np.array_equal(codes[b, :nb].cpu().numpy(), rc), b
        assert np.array_equal(scales[b, :nb].cpu().numpy(), rs), b


def _world(B, L, d, m, Wcap, seed, H, T):
    g = gen(seed, "attn16", B, L, d, m)
    kv = torch.randn(B, L, d, generator=g, device=DEV)
    gate = torch.randn(B, L, generator=g, device=DEV)
    cap = O.n_blocks(L, m)
    codes = torch.empty(B, cap, d // 2, device=DEV, dtype=torch.uint8)
    scales = torch.empty(B, cap, d // 16, device=DEV, dtype=torch.uint8)
    csa.compress_quantize(kv, gate, 0, m, codes, scales, fmt=FMT)
    win = torch.zeros(B, Wcap, d, device=DEV, dtype=torch.bfloat16)
    t0 = max(0, L - Wcap)
    win[:, torch.arange(t0, L, device=DEV) % Wcap] = kv[:, t0:L].to(torch.bfloat16)
    q = (torch.randn(B, T, H, d, generator=g, device=DEV) / math.sqrt(d)).to(torch.bfloat16)
    return dict(codes=codes, scales=scales, win=win, q=q)


def _check(wd, idx, pos0, W, out, lse, dense_m=None):
    torch.cuda.synchronize()
    B, T, H, d = wd["q"].shape
    cn, sn, wn, qn = (wd["codes"].cpu().numpy(), wd["scales"].cpu().numpy(), bf16_bits(wd["win"]),
                      bf16_bits(wd["q"]))
    idn = idx.cpu().numpy() if idx is not None else None
    refs, lrefs = [], []
    for b in range(B):
        for ti in range(T):
            t = pos0 + ti
            if dense_m is None:
                o, l = O.sparse_attn(qn[b, ti], cn[b], sn[b], idn[b, ti], wn[b], wn.shape[1], W, t,
                                     1.0, fmt=FMT)
            else:
                o, l = O.hca_dense_attn(qn[b, ti], cn[b], sn[b], dense_m, wn[b], wn.shape[1], W, t,
                                        1.0, fmt=FMT)
            refs.append(o)
            lrefs.append(l)
    ref = np.stack(refs).reshape(B, T, H, d)
    ex, rms = attn_excess_error(to_np(out), ref, out.dtype == torch.bfloat16)
    say(f"   excess error / rms = {ex:.3e}")
    assert ex <= REL_TOL, ex
    if lse is not None:
        lref = np.stack(lrefs).reshape(B, T, H)
        assert np.abs(lse.cpu().numpy() - lref).max() <= 1e-4 * max(1.0, np.abs(lref).max())


@pytest.mark.parametrize("d,H", [(512, 64), (128, 8)])
def test_sparse_attn_e4m3(d, H):
    say("attn e4m3", d, H)
    B, L, m, k, W = 3, 4 * 1500, 4, 512, 128
    wd = _world(B, L, d, m, 128, seed=96, H=H, T=1)
    g = gen(97, "idx16")
    idx = torch.stack([torch.randperm(L // m, generator=g, device=DEV)[:k] for _ in range(B)])
    idx[1, 7:20] = -1
    idx = idx.reshape(B, 1, k).to(torch.int32).contiguous()
    for od in (torch.bfloat16, torch.float32):
        out = torch.empty(B, 1, H, d, device=DEV, dtype=od)
        lse = torch.empty(B, 1, H, device=DEV, dtype=torch.float32)
        csa.sparse_attn(wd["q"], wd["codes"], wd["scales"], idx, wd["win"], W, L - 1, 1.0, out,
                        lse, fmt=FMT)
        _check(wd, idx, L - 1, W, out, lse)


def test_sparse_attn_e4m3_prefill_block():
    say("attn e4m3 prefill")
    B, L, d, m, H, T, k, W = 1, 4096, 512, 4, 64, 32, 512, 128
    wd = _world(B, L, d, m, 2048, seed=98, H=H, T=T)
    pos0 = L - T
    g = gen(99, "idx16p")
    idx = torch.stack([torch.randperm((pos0 + i + 1) // m, generator=g, device=DEV)[:k]
                       for i in range(T)]).reshape(1, T, k).to(torch.int32).contiguous()
    out = torch.empty(B, T, H, d, device=DEV, dtype=torch.bfloat16)
    csa.sparse_attn(wd["q"], wd["codes"], wd["scales"], idx, wd["win"], W, pos0, 1.0, out,
                    fmt=FMT)
    _check(wd, idx, pos0, W, out, None)


def test_hca_dense_e4m3():
    say("hca e4m3")
    B, L, d, m, H, W = 2, 128 * 300, 512, 128, 64, 128
    wd = _world(B, L, d, m, 256, seed=100, H=H, T=1)
    out = torch.empty(B, 1, H, d, device=DEV, dtype=torch.float32)
    csa.hca_dense_attn(wd["q"], wd["codes"], wd["scales"], m, wd["win"], W, L - 1, 1.0, out,
                       fmt=FMT)
    _check(wd, None, L - 1, W, out, None, dense_m=m)
