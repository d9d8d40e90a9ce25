"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the attention method: it only draws
random tensors (torch generators, on the host or on the device) with the
shapes and distributions of the workloads, and lays them out the way the
library expects. Every tensor comes from its own generator, seeded by a hash
of (seed, tensor name, indices), and large latent streams are drawn in fixed
CHUNK-token pieces so any token range can be redrawn on its own.

Distributions (one reading for what the workload descriptions leave open):
latents N(0,1) float32 (the tiny workload multiplies each channel by a
LogNormal(0, 0.5) factor), gate logits N(0,1), queries bfloat16 N(0, 1/d),
indexer queries and keys int8 uniform in [-8, 7], indexer head weights int8
uniform in [0, 3]. The window ring holds the bfloat16 rounding of the
latents it covers (torch's float32 -> bfloat16 conversion).
"""

from __future__ import annotations

import dataclasses
import hashlib
import math

import torch

CHUNK = 8192


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int            # sequences
    L: int            # context tokens per sequence (queries sit at L-T .. L-1)
    d: int            # latent width
    m: int            # tokens per compressed block
    H: int            # query heads sharing the latent
    Hi: int           # indexer heads
    Di: int           # indexer head dim
    k: int            # top-k blocks
    W: int = 128      # sliding window
    T: int = 1        # queries per sequence per call
    Wcap: int = 128   # window ring slots
    chan_lognormal: float = 0.0   # sigma of the per-channel LogNormal factor (0 = off)
    m_hca: int = 128  # block size of the dense heavily-compressed cache
    pool: int = 0     # candidate pool size for reindex layers (0 = none)
    chunk: int = 0    # prefill chunk length (0 = not chunked)
    len_step: int = 0  # ragged batches: sequence b decodes at position L - 1 - b * len_step

    def positions(self) -> list:
        """Decode position of each sequence (all L - 1 unless ragged)."""
        return [self.L - 1 - b * self.len_step for b in range(self.B)]

    @property
    def n_blocks(self) -> int:
        return -(-self.L // self.m)


WORKLOADS = {
    "tiny_causal": Workload("tiny_causal", B=1, L=1024, d=128, m=4, H=8, Hi=4, Di=32,
                            k=16, T=1024, Wcap=2048, chan_lognormal=0.5),
    "decode_32k": Workload("decode_32k", B=64, L=32768, d=512, m=4, H=64, Hi=8, Di=64,
                           k=512),
    "decode_1m": Workload("decode_1m", B=8, L=1 << 20, d=512, m=4, H=64, Hi=8, Di=64,
                          k=1024),
    "prefill_128k": Workload("prefill_128k", B=1, L=131072, d=512, m=4, H=64, Hi=8, Di=64,
                             k=512, T=8192, Wcap=16384, chunk=8192),
    "decode_ragged_1m": Workload("decode_ragged_1m", B=8, L=1 << 20, d=512, m=4, H=64, Hi=8,
                                 Di=64, k=1024, len_step=65_543),
    "hca_reindex_1m": Workload("hca_reindex_1m", B=16, L=1 << 20, d=512, m=4, H=64, Hi=8,
                               Di=64, k=512, pool=4096, m_hca=128),
}


def seed_of(seed: int, *parts) -> int:
    h = hashlib.sha256(repr((seed,) + tuple(parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def generator(device, seed: int, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(seed, *parts))
    return g


def channel_scale(wl: Workload, device, seed: int = 0, layer: str = "main"):
    if wl.chan_lognormal == 0.0:
        return None
    g = generator(device, seed, layer, "chan")
    z = torch.randn(wl.d, generator=g, device=device, dtype=torch.float32)
    return torch.exp(wl.chan_lognormal * z)


def latent_chunk(wl: Workload, b: int, c: int, device, seed: int = 0, layer: str = "main"):
    """float32 [rows][d] latents of tokens [c*CHUNK, min((c+1)*CHUNK, L))."""
    rows = min(CHUNK, wl.L - c * CHUNK)
    g = generator(device, seed, layer, "kv", b, c)
    x = torch.randn(rows, wl.d, generator=g, device=device, dtype=torch.float32)
    s = channel_scale(wl, device, seed, layer)
    return x if s is None else x * s


def gate_chunk(wl: Workload, b: int, c: int, device, seed: int = 0, layer: str = "main"):
    rows = min(CHUNK, wl.L - c * CHUNK)
    g = generator(device, seed, layer, "gate", b, c)
    return torch.randn(rows, generator=g, device=device, dtype=torch.float32)


def latent_range(wl: Workload, b: int, t0: int, t1: int, device, seed: int = 0,
                 layer: str = "main", gate: bool = False):
    """Latents (or gate logits) of tokens [t0, t1) of sequence b."""
    parts = []
    for c in range(t0 // CHUNK, (t1 - 1) // CHUNK + 1 if t1 > t0 else t0 // CHUNK):
        f = gate_chunk if gate else latent_chunk
        x = f(wl, b, c, device, seed, layer)
        lo = max(t0, c * CHUNK) - c * CHUNK
        hi = min(t1, (c + 1) * CHUNK) - c * CHUNK
        parts.append(x[lo:hi])
    if not parts:
        shape = (0,) if gate else (0, wl.d)
        return torch.empty(shape, device=device, dtype=torch.float32)
    return torch.cat(parts, 0)


def window_ring(wl: Workload, t_last, device, seed: int = 0, layer: str = "main",
                span: int | None = None):
    """bfloat16 ring [B][Wcap][d] holding tokens max(0, t_last-span+1) .. t_last
    in slot p % Wcap (span defaults to Wcap); t_last is one position for every
    sequence or a list of per-sequence positions."""
    span = wl.Wcap if span is None else span
    ring = torch.zeros(wl.B, wl.Wcap, wl.d, device=device, dtype=torch.bfloat16)
    for b in range(wl.B):
        tl = t_last[b] if isinstance(t_last, (list, tuple)) else t_last
        t0 = max(0, tl - span + 1)
        pos = torch.arange(t0, tl + 1, device=device) % wl.Wcap
        ring[b, pos] = latent_range(wl, b, t0, tl + 1, device, seed, layer).to(torch.bfloat16)
    return ring


def queries(wl: Workload, device, seed: int = 0, layer: str = "main", T: int | None = None):
    """bfloat16 [B][T][H][d], N(0, 1/d)."""
    T = wl.T if T is None else T
    g = generator(device, seed, layer, "q")
    x = torch.randn(wl.B, T, wl.H, wl.d, generator=g, device=device, dtype=torch.float32)
    return (x * (1.0 / math.sqrt(wl.d))).to(torch.bfloat16)


def indexer_queries(wl: Workload, device, seed: int = 0, layer: str = "main",
                    T: int | None = None):
    """(q_idx int8 [B][T][Hi][Di] in [-8, 7], w int8 [B][T][Hi] in [0, 3])."""
    T = wl.T if T is None else T
    g = generator(device, seed, layer, "qidx")
    q = torch.randint(-8, 8, (wl.B, T, wl.Hi, wl.Di), generator=g, device=device,
                      dtype=torch.int8)
    g = generator(device, seed, layer, "w")
    w = torch.randint(0, 4, (wl.B, T, wl.Hi), generator=g, device=device, dtype=torch.int8)
    return q, w


def indexer_keys(wl: Workload, device, seed: int = 0, layer: str = "main",
                 blk_cap: int | None = None):
    """int8 [B][blk_cap][Di] in [-8, 7] (one key per compressed block)."""
    cap = wl.n_blocks if blk_cap is None else blk_cap
    out = torch.empty(wl.B, cap, wl.Di, device=device, dtype=torch.int8)
    for b in range(wl.B):
        g = generator(device, seed, layer, "keys", b)
        out[b] = torch.randint(-8, 8, (cap, wl.Di), generator=g, device=device,
                               dtype=torch.int8)
    return out


def as_numpy(t: torch.Tensor):
    """Host numpy copy; bfloat16 comes back as its uint16 bit patterns."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
