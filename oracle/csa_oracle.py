"""Plain CPU oracle for compressed sparse attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test-suite, the package smoke check and the CPU
baseline leg of the benchmark use it. It shares no code with the HIP library
and imports nothing from it.

Everything is computed with numpy on the host, floating point in float64 and
integers in int64, one obvious step at a time. Sources (web pages, cited by
title and section):

* [NOTES4] "Frontier Architecture Decoding Notes (4): DeepSeek V4 -- Extreme
  Compression and Efficient Training", section 1 "Attention: CSA + HCA
  Hybrid": CSA compresses the KV into 4-token blocks and keeps a top-k of
  blocks; HCA compresses up to 128x and is attended densely; the most recent
  128 tokens are attended uncompressed.
* [RASCHKA] "Recent Developments in LLM Architectures: KV Sharing, mHC, and
  Compressed Attention", section "Data": the KV is shortened along the
  sequence by summarising groups of tokens; CSA is the milder, sparse form,
  HCA the heavier, dense form.
* [PODCAST] podcast transcript "DeepSeek-V4.1-Flash: Pushing the Limits of KV
  Cache Compression": cue 8 (shared latent entry, sequence compression,
  FP4), cue 12 (Full / Reindex / Reuse layer modes), cue 14 (the first Full
  layer scores every causally visible position; Reindex layers search only
  a shared candidate pool), cue 16 (MXFP4 E2M1 main cache, dequantised just
  before attention).
* [OCP-MX] the public OCP Microscaling Formats (MX) v1.0 specification, for
  the MXFP4 element grid (E2M1), the shared E8M0 scale and its derivation
  from the block's largest magnitude.

Where the pages leave a step open the reading taken here is stated at the
function that implements it (see the READINGS list at the bottom).

Parity status: every function below is pinned by the CPU tests
(tests/test_oracle_pins.py) against closed forms, brute force, a second
independent implementation or a library routine; none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

# MXFP4 element grid: the eight non-negative E2M1 magnitudes, indexed by the
# 3-bit magnitude code (exponent bits, then the mantissa bit) [OCP-MX].
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E2M1_EMAX = 2          # exponent of the largest E2M1 power of two (4 = 2**2)
E8M0_BIAS = 127
GROUP = 32             # elements sharing one E8M0 scale (reading A1)


# --------------------------------------------------------------------------
# Shapes and closed forms
# --------------------------------------------------------------------------

def n_blocks(n_tokens: int, m: int) -> int:
    """Number of compressed entries for n_tokens tokens: one per m-token block,
    the last one possibly partial ([NOTES4] s.1, [RASCHKA] Data)."""
    return -(-n_tokens // m)


def n_visible(t: int, m: int) -> int:
    """Blocks visible to the query at position t: block b covers tokens
    [b*m, (b+1)*m) and is visible once complete, i.e. (b+1)*m - 1 <= t
    ([PODCAST] cue 14, 'causally visible')."""
    return (t + 1) // m


def entry_bytes(d: int) -> int:
    """Bytes of one MXFP4 entry of d channels: d/2 code bytes + d/32 scales."""
    return d // 2 + d // GROUP


# --------------------------------------------------------------------------
# a1: block pooling
# --------------------------------------------------------------------------

def pool_blocks(kv: np.ndarray, gate: np.ndarray, m: int) -> np.ndarray:
    """Softmax-gated pooling of each m-token block (reading A5).

    kv: [n][d] float32 latents, gate: [n] float32 logits. Returns [nb][d]
    float64 where, for the tokens J of block b,
        w_j = exp(g_j - max_J g) / sum_J exp(g_i - max_J g)
        p   = sum_{j in J} w_j * x_j   (summed in token order)
    A final partial block pools over the tokens it has (reading A7).
    """
    kv = np.asarray(kv)
    gate = np.asarray(gate)
    n, d = kv.shape
    nb = n_blocks(n, m)
    out = np.empty((nb, d), dtype=np.float64)
    n_full = n // m
    spans = []
    if n_full:
        spans.append((0, n_full, m))
    if n_full * m < n:
        spans.append((n_full, n_full + 1, n - n_full * m))
    for b0, b1, size in spans:
        x = kv[b0 * m: b0 * m + (b1 - b0) * size].astype(np.float64)
        g = gate[b0 * m: b0 * m + (b1 - b0) * size].astype(np.float64)
        x = x.reshape(b1 - b0, size, d)
        g = g.reshape(b1 - b0, size)
        e = np.exp(g - g.max(axis=1, keepdims=True))
        s = e[:, 0].copy()
        for j in range(1, size):
            s = s + e[:, j]
        w = e / s[:, None]
        p = w[:, 0, None] * x[:, 0]
        for j in range(1, size):
            p = p + w[:, j, None] * x[:, j]
        out[b0:b1] = p
    return out


# --------------------------------------------------------------------------
# a2: MXFP4 quantisation
# --------------------------------------------------------------------------

def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared exponent of a 32-element group [OCP-MX]: floor(log2 amax) minus
    the E2M1 emax (2), clamped to the E8M0 range [-127, 127]; amax == 0 gives
    -127. floor(log2) is read exactly off the float64 exponent (frexp)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)            # amax = f * 2**ex, f in [0.5, 1)
    e = (ex.astype(np.int64) - 1) - E2M1_EMAX
    e = np.clip(e, -E8M0_BIAS, E8M0_BIAS)
    return np.where(amax == 0.0, -E8M0_BIAS, e)


def e2m1_magnitude_code(a: np.ndarray) -> np.ndarray:
    """Magnitude code (0..7) of |y| = a: round to the nearest E2M1 value,
    halfway cases to the even code, values beyond 6 saturate to 6 (readings
    A3). Written as comparisons against the midpoints of the grid."""
    a = np.asarray(a, dtype=np.float64)
    return ((a > 0.25).astype(np.int64) + (a >= 0.75) + (a > 1.25)
            + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0))


def e2m1_magnitude_code_nearest(a: np.ndarray) -> np.ndarray:
    """Second, independent rounding: search the grid for the nearest value
    (after saturating to 6), breaking exact ties toward the even code index.
    Used only to pin e2m1_magnitude_code."""
    a = np.minimum(np.asarray(a, dtype=np.float64), 6.0)
    grid = np.array(E2M1_MAGNITUDES)
    dist = np.abs(a[..., None] - grid)
    best = dist.min(axis=-1, keepdims=True)
    ties = dist == best
    # among tied candidates keep an even index when there is one
    even = ties & (np.arange(8) % 2 == 0)
    choose = np.where(even.any(axis=-1, keepdims=True), even, ties)
    return np.argmax(choose, axis=-1).astype(np.int64)


def quantize_rows(p: np.ndarray):
    """MXFP4-quantise rows of float64 values p[nb][d] (d % 32 == 0).

    Returns (codes uint8 [nb][d/2], scales uint8 [nb][d/32]). Per group G of
    32 channels: e = scale_exponent(max |p|), y = p / 2**e (exact), code =
    sign bit (bit 3, kept also when the magnitude rounds to 0) | magnitude
    code. Byte c//2 holds channel c in its low nibble when c is even and in
    its high nibble when c is odd (reading A4). Scale byte = e + 127.
    """
    p = np.asarray(p, dtype=np.float64)
    nb, d = p.shape
    g = p.reshape(nb, d // GROUP, GROUP)
    e = scale_exponent(np.abs(g).max(axis=2))
    y = np.ldexp(g, -e[:, :, None])
    mag = e2m1_magnitude_code(np.abs(y))
    code = (np.signbit(y).astype(np.int64) << 3) | mag
    code = code.reshape(nb, d)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + E8M0_BIAS).astype(np.uint8)


def dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse map: value = (-1)**s * E2M1[mag] * 2**(scale - 127), float64
    [nb][d] ([PODCAST] cue 16: entries are dequantised before attention)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    nb, half = codes.shape
    d = 2 * half
    nib = np.empty((nb, d), dtype=np.int64)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    mag = np.array(E2M1_MAGNITUDES)[nib & 7]
    val = np.where(nib & 8, -mag, mag)
    e = scales.astype(np.int64) - E8M0_BIAS
    return np.ldexp(val.reshape(nb, d // GROUP, GROUP), e[:, :, None]).reshape(nb, d)


# --------------------------------------------------------------------------
# f3: the E4M3-per-16 scale variant ([PODCAST] cue 16)
# --------------------------------------------------------------------------

GROUP16 = 16           # elements sharing one E4M3 scale (reading A25)
E4M3_MAX_BYTE = 0x7E   # 448, the largest finite OCP E4M3 value
E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def e4m3_value(byte) -> np.ndarray:
    """Value of a non-negative OCP FP8 E4M3 byte (0 .. 0x7E): exponent field
    bits 6..3 with bias 7, mantissa bits 2..0; exponent field 0 encodes the
    subnormals m * 2**-9. Returns float64 (exact)."""
    b = np.asarray(byte, dtype=np.int64)
    e = (b >> 3) & 0xF
    mnt = b & 7
    return np.where(e == 0, np.ldexp(mnt.astype(np.float64), -9),
                    np.ldexp((8 + mnt).astype(np.float64), e - 10))


def e4m3_scale_byte(amax) -> np.ndarray:
    """Scale byte of a 16-element group: the E4M3 value nearest to amax / 6
    (6 = the largest E2M1 magnitude), halfway cases to the even byte, values
    past 448 saturating to 448 (reading A25). Decided without dividing: amax
    is compared with 6 v (the candidates) and with 3 (v_lo + v_hi) (their
    midpoint times 6), products that are exact in float64."""
    amax = np.asarray(amax, dtype=np.float64)
    vals = e4m3_value(np.arange(E4M3_MAX_BYTE + 1))          # ascending
    i = np.searchsorted(6.0 * vals, amax, side="right") - 1  # 6 v_i <= amax
    i = np.clip(i, 0, E4M3_MAX_BYTE)
    j = np.minimum(i + 1, E4M3_MAX_BYTE)
    mid6 = 3.0 * (vals[i] + vals[j])
    up = (i < E4M3_MAX_BYTE) & ((amax > mid6) | ((amax == mid6) & (i % 2 == 1)))
    return (i + up).astype(np.uint8)


def e2m1_magnitude_code_scaled(a: np.ndarray, s: np.ndarray) -> np.ndarray:
    """e2m1_magnitude_code(a / s) decided without dividing: a is compared
    with s times each midpoint of the E2M1 grid (exact products, as s has at
    most 4 significant bits); s == 0 gives code 0."""
    a = np.asarray(a, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    # a tie at midpoint k goes to the even code: down (a > m) between codes
    # 2j and 2j + 1, up (a >= m) between codes 2j + 1 and 2j + 2
    mag = np.zeros(np.broadcast(a, s).shape, dtype=np.int64)
    for k, mid in enumerate(E2M1_MIDPOINTS):
        mag += (a > s * mid) if k % 2 == 0 else (a >= s * mid)
    return np.where(s == 0.0, 0, mag)


def quantize_rows_e4m3(p: np.ndarray):
    """FP4 with one E4M3 scale per 16 channels (no global scale; readings A25,
    A4 for nibble order and signed zero). Returns (codes uint8 [nb][d/2],
    scales uint8 [nb][d/16])."""
    p = np.asarray(p, dtype=np.float64)
    nb, d = p.shape
    g = p.reshape(nb, d // GROUP16, GROUP16)
    sb = e4m3_scale_byte(np.abs(g).max(axis=2))
    mag = e2m1_magnitude_code_scaled(np.abs(g), e4m3_value(sb)[:, :, None])
    code = ((np.signbit(g).astype(np.int64) << 3) | mag).reshape(nb, d)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sb


def dequantize_rows_e4m3(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """value = (-1)**s * E2M1[mag] * e4m3_value(scale), float64 [nb][d]."""
    codes = np.asarray(codes, dtype=np.uint8)
    nb, half = codes.shape
    d = 2 * half
    nib = np.empty((nb, d), dtype=np.int64)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    mag = np.array(E2M1_MAGNITUDES)[nib & 7]
    val = np.where(nib & 8, -mag, mag).reshape(nb, d // GROUP16, GROUP16)
    return (val * e4m3_value(scales)[:, :, None]).reshape(nb, d)


def compress_quantize_e4m3(kv: np.ndarray, gate: np.ndarray, m: int):
    """a1 + the E4M3-per-16 quantisation for one sequence."""
    return quantize_rows_e4m3(pool_blocks(kv, gate, m))


def compress_quantize(kv: np.ndarray, gate: np.ndarray, m: int):
    """a1 + a2 for one sequence whose first token starts block 0."""
    return quantize_rows(pool_blocks(kv, gate, m))


def near_decision_mask(kv: np.ndarray, gate: np.ndarray, m: int,
                       rel: float = 1e-12) -> np.ndarray:
    """Flags pooled elements whose code could depend on rounding order.

    Any two float64 evaluations of the pooling differ by far less than
    rel * max_j |x_j| (per channel, over the block's tokens). An element is
    flagged when its pooled value lies within that distance of a rounding
    midpoint, of zero (sign of a zero code), or when its group's amax lies
    within it of a power of two (the shared exponent could move). Returns a
    bool [nb][d] mask; for the seeded inputs used here it is all False.
    """
    kv = np.asarray(kv)
    n, d = kv.shape
    nb = n_blocks(n, m)
    p = pool_blocks(kv, gate, m)
    xmax = np.zeros((nb, d))
    for b in range(0, nb):
        blk = np.abs(kv[b * m: min((b + 1) * m, n)].astype(np.float64))
        xmax[b] = blk.max(axis=0)
    tol = rel * xmax + 1e-300
    g = p.reshape(nb, d // GROUP, GROUP)
    tg = tol.reshape(nb, d // GROUP, GROUP)
    amax = np.abs(g).max(axis=2)
    e = scale_exponent(amax)
    step = np.ldexp(1.0, e)[:, :, None]
    a = np.abs(g)
    flag = a <= tg                                           # sign of zero
    for mid in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
        flag |= np.abs(a - mid * step) <= tg
    tmax = tg.max(axis=2)
    pw = np.ldexp(1.0, np.frexp(amax)[1] - 1)                # 2**floor(log2)
    gflag = (np.abs(amax - pw) <= tmax) | (np.abs(amax - 2 * pw) <= tmax)
    flag |= gflag[:, :, None]
    return flag.reshape(nb, d)


# --------------------------------------------------------------------------
# a3 + a4 (+ a8): indexer scores and top-k
# --------------------------------------------------------------------------

def index_scores(q_idx: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Exact integer score of every key row (reading A9):
        s(b) = sum_h w[h] * max(0, sum_c q_idx[h, c] * keys[b, c]).
    q_idx: [Hi][Di] int8, w: [Hi] int8, keys: [N][Di] int8 -> int64 [N]."""
    q = np.asarray(q_idx, dtype=np.int64)
    k = np.asarray(keys, dtype=np.int64)
    dots = k @ q.T                                   # [N][Hi]
    return np.maximum(dots, 0) @ np.asarray(w, dtype=np.int64)


def select_topk(blocks: np.ndarray, scores: np.ndarray, k: int):
    """Top-k of the given blocks under the order (score descending, block
    index ascending) -- the lower index wins ties (reading A10). Returns
    (idx int32 [k], score int32 [k]): the kept blocks in ascending block
    order, then -1 padding (reading A11)."""
    blocks = np.asarray(blocks, dtype=np.int64)
    scores = np.asarray(scores, dtype=np.int64)
    order = np.lexsort((blocks, -scores))          # last key is primary
    keep = order[:min(k, blocks.size)]
    keep = keep[np.argsort(blocks[keep])]
    idx = np.full(k, -1, dtype=np.int32)
    sc = np.full(k, -1, dtype=np.int32)
    idx[:keep.size] = blocks[keep]
    sc[:keep.size] = scores[keep]
    return idx, sc


def index_topk(q_idx, w, keys, m: int, t: int, k: int, cand=None):
    """Indexer + top-k for the query at position t ([PODCAST] cues 12, 14).

    Full mode (cand is None): every causally visible block b < n_visible(t).
    Reindex mode: only the blocks listed in cand (-1 entries and blocks not
    yet visible are ignored) -- the shared candidate pool of cue 14.
    """
    nv = min(n_visible(t, m), len(keys))
    if cand is None:
        blocks = np.arange(nv, dtype=np.int64)
    else:
        c = np.asarray(cand, dtype=np.int64)
        blocks = c[(c >= 0) & (c < nv)]
    s = index_scores(q_idx, w, np.asarray(keys)[blocks]) if blocks.size else np.zeros(0, np.int64)
    return select_topk(blocks, s, k)


def block_pool(q_idx, w, keys, m: int, t: int, group: int, n_keep: int):
    """Blockwise candidate pool of a Full-mode layer ([PODCAST] cue 14: take
    the highest score of each block of positions, keep the best blocks and
    pool their positions for the Reindex layers).

    The causally visible entries 0 .. nv-1 are cut into groups of `group`
    consecutive entries (the last one may be partial); a group's score is the
    largest score of its visible entries (reading A22). The n_keep best groups
    under (score descending, group index ascending) are kept (reading A23).
    Returns int32 [group * n_keep]: kept group i (ascending group order)
    fills slots i*group .. i*group + group - 1 with its entries, -1 where an
    entry is not visible yet; slots of unused groups are -1.
    """
    nv = min(n_visible(t, m), len(keys))
    pool = np.full(group * n_keep, -1, dtype=np.int32)
    if nv == 0:
        return pool
    s = index_scores(q_idx, w, np.asarray(keys)[:nv])
    ng = -(-nv // group)
    padded = np.full(ng * group, -1, dtype=np.int64)   # scores are >= 0
    padded[:nv] = s
    gscore = padded.reshape(ng, group).max(axis=1)
    kept, _ = select_topk(np.arange(ng), gscore, n_keep)
    for i, gi in enumerate(kept):
        if gi < 0:
            break
        for r in range(group):
            e = int(gi) * group + r
            pool[i * group + r] = e if e < nv else -1
    return pool


# --------------------------------------------------------------------------
# a5 + a6 + a7: attention
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def attend(q: np.ndarray, rows: np.ndarray, softmax_scale: float):
    """Softmax attention of H query heads over one shared set of latent rows
    (K = V = the row, reading A15): logits l = scale * rows @ q_h,
    o_h = softmax(l) @ rows. q: [H][d] float64, rows: [n][d] float64.
    Returns (o [H][d], lse [H]) in float64."""
    logits = softmax_scale * (q @ rows.T)            # [H][n]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    lsum = e.sum(axis=1, keepdims=True)
    o = (e @ rows) / lsum
    return o, (mx + np.log(lsum))[:, 0]


def window_positions(t: int, W: int) -> np.ndarray:
    """Uncompressed window of the query at t: positions max(0, t-W+1) .. t
    ([NOTES4] s.1, the most recent W = 128 tokens; reading A12)."""
    return np.arange(max(0, t - W + 1), t + 1)


def gather_rows(codes, scales, blocks, win, Wcap: int, t: int, W: int,
                fmt: str = "e8m0") -> np.ndarray:
    """Rows attended by the query at t: the dequantised entries of `blocks`
    followed by the bf16 window tokens (ring slot p % Wcap), all under one
    softmax (readings A12, A17). fmt "e4m3" reads E4M3-per-16 scales."""
    blocks = np.asarray(blocks, dtype=np.int64)
    blocks = blocks[blocks >= 0]
    deq = dequantize_rows_e4m3 if fmt == "e4m3" else dequantize_rows
    ent = deq(np.asarray(codes)[blocks], np.asarray(scales)[blocks])
    pos = window_positions(t, W)
    wr = bf16_to_f64(np.asarray(win)[pos % Wcap])
    return np.concatenate([ent, wr], axis=0)


def sparse_attn(q_bf16, codes, scales, idx, win, Wcap: int, W: int, t: int,
                softmax_scale: float, fmt: str = "e8m0"):
    """Compressed sparse attention of one query: the selected entries plus
    the window ([NOTES4] s.1; [PODCAST] cues 12 and 16). q_bf16: [H][d]
    uint16. Returns (o [H][d], lse [H]) float64."""
    rows = gather_rows(codes, scales, idx, win, Wcap, t, W, fmt)
    return attend(bf16_to_f64(q_bf16), rows, softmax_scale)


def hca_dense_attn(q_bf16, codes, scales, m: int, win, Wcap: int, W: int, t: int,
                   softmax_scale: float, fmt: str = "e8m0"):
    """Heavily compressed attention: every visible entry of an m-token cache
    (m up to 128) plus the window, no indexer ([NOTES4] s.1; [RASCHKA] Data)."""
    nv = min(n_visible(t, m), len(codes))
    return sparse_attn(q_bf16, codes, scales, np.arange(nv), win, Wcap, W, t,
                       softmax_scale, fmt)


# --------------------------------------------------------------------------
# f2: the cache of a decoding sequence
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to
    the even pattern (reading A17; finite inputs). The 16 dropped bits are
    compared with half of the last kept bit's weight."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    hi = u >> 16
    lo = u & 0xFFFF
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    return (hi + up.astype(np.uint64)).astype(np.uint16)


def cache_after_appends(kv: np.ndarray, gate: np.ndarray, m: int, n_tok: int, Wcap: int):
    """State of one sequence's caches once its tokens 0 .. n_tok-1 have been
    appended ([NOTES4] s.1: finished blocks go to the compressed cache, the
    newest tokens stay uncompressed; reading A24).

    Returns (codes, scales, ring):
      codes, scales  the n_tok // m complete blocks, exactly as a one-shot
                     compression of tokens 0 .. (n_tok // m) * m - 1;
      ring           {slot: bf16 bits [d]} for the tokens p = max(0, n_tok -
                     Wcap) .. n_tok - 1, each in slot p % Wcap.
    A block still being filled has no entry (no query can see it, A8)."""
    nb = n_tok // m
    kv = np.asarray(kv, dtype=np.float32)
    gate = np.asarray(gate, dtype=np.float32)
    codes, scales = compress_quantize(kv[:nb * m], gate[:nb * m], m)
    ring = {int(p % Wcap): f32_to_bf16_bits(kv[p]) for p in range(max(0, n_tok - Wcap), n_tok)}
    return codes, scales, ring


READINGS = {
    "A1": "MXFP4 uses one E8M0 scale per 32 elements (OCP MX), not the E4M3-per-16 variant of [PODCAST] cue 16",
    "A2": "scale exponent = floor(log2 amax) - 2, clamped to [-127, 127]; amax 0 -> byte 0",
    "A3": "elements round to nearest, ties to the even code, saturating at 6",
    "A4": "a zero keeps its sign bit; even channel in the low nibble",
    "A5": "one scalar gate logit per token; softmax over the block's tokens; weighted sum of token vectors",
    "A7": "ceil(L/m) entries; a partial last block pools the tokens present",
    "A8": "block b is visible at t iff (b+1)*m - 1 <= t",
    "A9": "s = sum_h w_h * relu(q_h . k_b), exact integers",
    "A10": "ties at equal score go to the lower block index",
    "A11": "k_eff = min(k, candidates); -1 padding",
    "A12": "window = positions max(0, t-W+1)..t, no de-duplication against entries, one softmax",
    "A15": "K = V = the latent row",
    "A17": "window rows are bf16",
    "A22": "blockwise pool: groups of `group` consecutive compressed entries (8 per [PODCAST] cue 14); group score = max over its visible entries",
    "A23": "blockwise pool keeps n_keep groups (about 2000 per cue 14), ties to the lower group; the pool lists their visible entries ascending, -1 elsewhere",
    "A25": "E4M3 variant: one OCP E4M3 scale per 16 elements, no global scale; scale = the E4M3 value nearest amax/6 (ties to the even byte, saturating at 448); elements to the nearest E2M1 multiple of the scale (ties to even, saturating at 6); a zero scale gives zero codes",
    "A24": "decode append: a block's entry is written once its m-th token arrives, from the block's m float32 tokens; each token also enters the bf16 ring at slot p % Wcap; sequences of a batch may sit at different positions",
}
