"""Comparison helpers for GPU-vs-oracle parity tests."""

from __future__ import annotations

import numpy as np
import torch

# max-abs-error bound on attention outputs, relative to the RMS of the
# reference output over the compared tensor
REL_TOL = 2e-3


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bfloat16 ulp at |x| (8 significant bits): 2**(floor(log2|x|) - 8)."""
    ax = np.abs(x).astype(np.float64)
    e = np.floor(np.log2(np.maximum(ax, 1e-300)))
    e = np.maximum(e, -126.0)
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def attn_excess_error(o_gpu: np.ndarray, o_ref: np.ndarray, out_is_bf16: bool):
    """Largest error beyond the final output rounding, divided by RMS(o_ref).
    For bfloat16 outputs half a bfloat16 ulp of the larger magnitude is the
    rounding allowance; float32 outputs get none."""
    o_gpu = o_gpu.astype(np.float64)
    err = np.abs(o_gpu - o_ref)
    if out_is_bf16:
        err = np.maximum(0.0, err - bf16_half_ulp(np.maximum(np.abs(o_gpu), np.abs(o_ref))))
    rms = float(np.sqrt(np.mean(o_ref ** 2)))
    return float(err.max()) / rms, rms


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy()
    return t.numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
