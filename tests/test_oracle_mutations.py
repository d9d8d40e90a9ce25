"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them."""

import numpy as np
import pytest

import oracle.csa_oracle as O
import oracle_pins as P


def _fails(monkeypatch, **patches):
    for name, fn in patches.items():
        monkeypatch.setattr(O, name, fn)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(O)
        except AssertionError:
            failed.append(pin.__name__)
        except Exception:  # a crash also counts as caught
            failed.append(pin.__name__)
    return failed


orig_scale = O.scale_exponent
orig_mag = O.e2m1_magnitude_code
orig_quant = O.quantize_rows
orig_deq = O.dequantize_rows
orig_pool = O.pool_blocks
orig_scores = O.index_scores
orig_select = O.select_topk
orig_attend = O.attend
orig_win = O.window_positions
orig_nvis = O.n_visible
orig_gather = O.gather_rows
orig_bf16 = O.f32_to_bf16_bits
orig_sbyte = O.e4m3_scale_byte
orig_quant16 = O.quantize_rows_e4m3
orig_append = O.cache_after_appends


def m_scale_off_by_one(a):
    return orig_scale(a) + 1


def m_no_clamp(a):
    a = np.asarray(a, dtype=np.float64)
    _, ex = np.frexp(a)
    return np.where(a == 0, -127, ex.astype(np.int64) - 3)


def m_ties_up(a):
    a = np.asarray(a, dtype=np.float64)
    return ((a >= 0.25).astype(np.int64) + (a >= 0.75) + (a >= 1.25) + (a >= 1.75)
            + (a >= 2.5) + (a >= 3.5) + (a >= 5.0))


def m_nibbles_swapped(p):
    c, s = orig_quant(p)
    return ((c >> 4) | (c << 4)).astype(np.uint8), s


def m_drop_negative_zero(p):
    c, s = orig_quant(p)
    lo, hi = c & 0xF, c >> 4
    lo = np.where(lo == 8, 0, lo)
    hi = np.where(hi == 8, 0, hi)
    return (lo | (hi << 4)).astype(np.uint8), s


def m_deq_bias(c, s):
    return orig_deq(c, s) * 2.0


def m_pool_mean(kv, g, m):
    return orig_pool(kv, np.zeros_like(g), m)


def m_pool_drop_last(kv, g, m):
    kv = np.array(kv, copy=True)
    n = len(kv)
    for b in range(0, n, m):
        if min(b + m, n) - b > 1:
            kv[min(b + m, n) - 1] = kv[b]
    return orig_pool(kv, g, m)


def m_no_relu(q, w, keys):
    return (np.asarray(keys, np.int64) @ np.asarray(q, np.int64).T) @ np.asarray(w, np.int64)


def m_relu_after_sum(q, w, keys):
    d = np.asarray(keys, np.int64) @ np.asarray(q, np.int64).T
    return np.maximum(d @ np.asarray(w, np.int64), 0)


def m_ties_high(blocks, scores, k):
    blocks = np.asarray(blocks, np.int64)
    return orig_select(blocks[::-1], np.asarray(scores)[::-1], k) if blocks.size else orig_select(blocks, scores, k)


def m_ties_high2(blocks, scores, k):
    blocks = np.asarray(blocks, np.int64)
    scores = np.asarray(scores, np.int64)
    order = np.lexsort((-blocks, -scores))
    keep = np.sort(blocks[order[:min(k, blocks.size)]])
    idx = np.full(k, -1, np.int32)
    idx[:keep.size] = keep
    sc = np.full(k, -1, np.int32)
    return idx, sc


def m_score_order(blocks, scores, k):
    blocks = np.asarray(blocks, np.int64)
    scores = np.asarray(scores, np.int64)
    order = np.lexsort((blocks, -scores))[:min(k, blocks.size)]
    idx = np.full(k, -1, np.int32)
    idx[:order.size] = blocks[order]
    sc = np.full(k, -1, np.int32)
    sc[:order.size] = scores[order]
    return idx, sc


def m_visible_early(t, m):
    return (t + 2) // m


def m_window_off_by_one(t, W):
    return np.arange(max(0, t - W), t + 1)


def m_window_excludes_self(t, W):
    return np.arange(max(0, t - W + 1), t)


def m_attend_no_scale(q, rows, s):
    return orig_attend(q, rows, 1.0)


def m_attend_softmax_heads(q, rows, s):
    logits = s * (q @ rows.T)
    e = np.exp(logits - logits.max(axis=0, keepdims=True))
    e = e / e.sum(axis=0, keepdims=True)
    return e @ rows, np.zeros(q.shape[0])


def m_gather_no_window(codes, scales, blocks, win, Wcap, t, W):
    rows = orig_gather(codes, scales, blocks, win, Wcap, t, W)
    nwin = len(orig_win(t, W))
    return rows[:-nwin] if rows.shape[0] > nwin else rows


def _pool_variant(q, w, keys, m, t, group, n_keep, reduce="max", tie_low=True, visible=True,
                  shift=0):
    """block_pool with one planted deviation (group score reduction, tie
    order, visibility, or groups shifted by `shift` entries)."""
    nv = min(O.n_visible(t, m), len(keys)) if visible else len(keys)
    pool = np.full(group * n_keep, -1, np.int32)
    if nv == 0:
        return pool
    s = O.index_scores(q, w, np.asarray(keys)[:nv])
    first = [0] + list(range(shift, nv, group)) if shift else list(range(0, nv, group))
    first = sorted(set(first))
    bounds = first + [nv]
    gs = []
    for a, z in zip(bounds[:-1], bounds[1:]):
        seg = s[a:z]
        gs.append(seg.max() if reduce == "max" else (seg.min() if reduce == "min" else seg[0]))
    order = sorted(range(len(gs)), key=lambda i: (-gs[i], i if tie_low else -i))[:n_keep]
    slot = 0
    for i in sorted(order):
        for e in range(bounds[i], bounds[i] + group):
            pool[slot] = e if e < bounds[i + 1] else -1
            slot += 1
    return pool


def m_bf16_truncate(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def m_bf16_ties_up(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x8000) >> 16).astype(np.uint16)


def m_append_ring_shift(kv, gate, m, n_tok, Wcap):
    c, s, r = orig_append(kv, gate, m, n_tok, Wcap)
    return c, s, {(k + 1) % Wcap: v for k, v in r.items()}


def m_append_partial_block(kv, gate, m, n_tok, Wcap):
    _, _, r = orig_append(kv, gate, m, n_tok, Wcap)
    c, s = O.compress_quantize(np.asarray(kv)[:n_tok], np.asarray(gate)[:n_tok], m)
    return c, s, r


def m_append_ring_short(kv, gate, m, n_tok, Wcap):
    c, s, r = orig_append(kv, gate, m, n_tok, Wcap)
    first = max(0, n_tok - Wcap)
    r.pop(first % Wcap, None)
    return c, s, r


def m_e4m3_scale_truncated(amax):
    vals = O.e4m3_value(np.arange(0x7F))
    i = np.searchsorted(6.0 * vals, np.asarray(amax, np.float64), side="right") - 1
    return np.clip(i, 0, 0x7E).astype(np.uint8)


def m_e4m3_ties_odd(amax):
    b = orig_sbyte(amax).astype(np.int64)
    vals = O.e4m3_value(np.arange(0x7F))
    mid6 = 3.0 * (vals[np.maximum(b - 1, 0)] + vals[b])
    tie = (np.asarray(amax) == mid6) & (b > 0)
    return np.where(tie, b - 1, b).astype(np.uint8)


def m_e4m3_over_four(amax):
    return orig_sbyte(np.asarray(amax, np.float64) * 1.5)


def m_e4m3_group32(p):
    p = np.asarray(p, np.float64)
    nb, d = p.shape
    g = p.reshape(nb, d // 32, 32)
    sb = np.repeat(orig_sbyte(np.abs(g).max(axis=2)), 2, axis=1)
    mag = O.e2m1_magnitude_code_scaled(np.abs(p.reshape(nb, d // 16, 16)),
                                       O.e4m3_value(sb)[:, :, None])
    code = ((np.signbit(p).astype(np.int64) << 3) | mag.reshape(nb, d))
    return (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8), sb


MUTANTS = {
    "scale exponent off by one": {"scale_exponent": m_scale_off_by_one},
    "scale exponent not clamped": {"scale_exponent": m_no_clamp},
    "ties rounded up": {"e2m1_magnitude_code": m_ties_up},
    "nibbles swapped": {"quantize_rows": m_nibbles_swapped},
    "negative zero dropped": {"quantize_rows": m_drop_negative_zero},
    "dequant scale doubled": {"dequantize_rows": m_deq_bias},
    "pooling ignores gates": {"pool_blocks": m_pool_mean},
    "pooling drops last token": {"pool_blocks": m_pool_drop_last},
    "indexer without relu": {"index_scores": m_no_relu},
    "relu after head sum": {"index_scores": m_relu_after_sum},
    "ties to higher index": {"select_topk": m_ties_high2},
    "output in score order": {"select_topk": m_score_order},
    "block visible one token early": {"n_visible": m_visible_early},
    "window one too long": {"window_positions": m_window_off_by_one},
    "window excludes the query token": {"window_positions": m_window_excludes_self},
    "softmax scale ignored": {"attend": m_attend_no_scale},
    "softmax over heads": {"attend": m_attend_softmax_heads},
    "window dropped": {"gather_rows": m_gather_no_window},
    "pool group score is the minimum": {"block_pool": lambda *a: _pool_variant(*a, reduce="min")},
    "pool group score is the first entry": {"block_pool": lambda *a: _pool_variant(*a, reduce="first")},
    "pool ties to the higher group": {"block_pool": lambda *a: _pool_variant(*a, tie_low=False)},
    "pool ignores visibility": {"block_pool": lambda *a: _pool_variant(*a, visible=False)},
    "pool groups shifted": {"block_pool": lambda *a: _pool_variant(*a, shift=1)},
    "bf16 by truncation": {"f32_to_bf16_bits": m_bf16_truncate},
    "bf16 ties rounded up": {"f32_to_bf16_bits": m_bf16_ties_up},
    "append ring slot off by one": {"cache_after_appends": m_append_ring_shift},
    "append writes the partial block": {"cache_after_appends": m_append_partial_block},
    "append ring drops its oldest token": {"cache_after_appends": m_append_ring_short},
    "e4m3 scale truncated": {"e4m3_scale_byte": m_e4m3_scale_truncated},
    "e4m3 scale ties to odd": {"e4m3_scale_byte": m_e4m3_ties_odd},
    "e4m3 scale from amax / 4": {"e4m3_scale_byte": m_e4m3_over_four},
    "e4m3 scale shared by 32": {"quantize_rows_e4m3": m_e4m3_group32},
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    failed = _fails(monkeypatch, **MUTANTS[name])
    assert failed, f"no pin caught the planted mistake: {name}"
