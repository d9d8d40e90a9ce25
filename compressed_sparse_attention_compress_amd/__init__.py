"""Python binding of libcsa (compressed sparse attention for MI355X / gfx950).

Argument marshalling only: every function checks dtypes, devices, shapes and
contiguity of torch tensors, then calls the C symbol of the same name in
libcsa.so on torch's current HIP stream. No computation happens here, and
there is no fallback: if libcsa.so is missing or a call fails, an exception
is raised.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "CSAError", "lib", "cache_bytes", "compress_quantize", "dequantize", "index_topk",
    "index_scan", "index_select", "index_topk_workspace", "index_topk_pool",
    "index_topk_pool_workspace", "index_pool_scan", "index_pool_select", "decode_append",
    "workspace_clear",
    "sparse_attn",
    "hca_dense_attn", "attn_workspace", "Workspace", "BF16", "F32", "F16", "EXPORTED",
    "prepare", "sparse_attn_noalloc", "NOALLOC_SCRATCH_MAX", "index_attn", "index_attn_workspace",
]

BF16, F32, F16 = 0, 1, 2
# scale formats of the FP4 cache: E8M0 per 32 channels, E4M3 per 16 channels
SCALE_FMT = {"e8m0": 0, "e4m3": 1}
SCALE_GROUP = {"e8m0": 32, "e4m3": 16}
_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa.so")

# every symbol declared in include/csa.h
EXPORTED = [
    "csa_status_string", "csa_version", "csa_cache_bytes", "csa_compress_quantize",
    "csa_dequantize", "csa_index_topk_workspace", "csa_index_topk", "csa_index_scan",
    "csa_index_select", "csa_index_topk_pool_workspace", "csa_index_topk_pool",
    "csa_index_pool_scan", "csa_index_pool_select", "csa_decode_append",
    "csa_index_topk_ragged", "csa_index_scan_ragged", "csa_index_select_ragged",
    "csa_sparse_attn_ragged", "hca_dense_attn_ragged",
    "csa_workspace_clear", "csa_attn_workspace", "csa_sparse_attn", "hca_dense_attn",
    "csa_sparse_attn_noalloc", "csa_index_attn_workspace", "csa_index_attn", "csa_index_attn_scan",
]
# bytes of the static device scratch of csa_sparse_attn_noalloc (CSA_NOALLOC_SCRATCH_MAX)
NOALLOC_SCRATCH_MAX = 64 << 20


class CSAError(RuntimeError):
    pass


_lib = None
# While prepare() runs: the recorded calls, each (name, C function, marshalled
# arguments, index-workspace head requirement or None), and every tensor whose
# address was marshalled (kept alive by the recording).
_RECORD = None
_KEEP = None
_PENDING_HEAD = None  # head requirement of the index call being marshalled
_QUERIES = ("csa_status_string", "csa_version", "csa_cache_bytes")


class _RecordingLib:
    """The library seen through prepare(): size queries pass through, every
    other call is stored with its marshalled arguments instead of issued."""

    def __init__(self, L):
        self._L = L

    def __getattr__(self, name):
        fn = getattr(self._L, name)
        if name.endswith("_workspace") or name in _QUERIES:
            return fn

        def record(*args):
            global _PENDING_HEAD
            _RECORD.append((name, fn, args, _PENDING_HEAD))
            _PENDING_HEAD = None
            return 0
        return record


def _ensure_head(buf, key, stream=None):
    """An index workspace's head (per-query histograms) must be zero for the
    layout of `key` (B*T) when a call starts; every successful call leaves it
    so. A buffer last used under another key is zero-filled first (with the
    library's fill kernel on `stream`, or torch's on the current stream)."""
    if key is None or getattr(buf, "_csa_key", None) == key:
        return
    if stream is None:
        buf.zero_()
    else:
        _check(_lib.csa_workspace_clear(ctypes.c_void_p(buf.data_ptr()), buf.numel() // 4 * 4,
                                        stream), "csa_workspace_clear")
    buf._csa_key = key


def prepare(fn):
    """Run fn() once with every library launch it makes marshalled and stored
    instead of issued (workspaces are sized and allocated now). Returns a
    callable that issues exactly those launches again, on the streams that
    were current when they were recorded, with the same buffers: the argument
    marshalling of a serving loop done once.

    The callable keeps every tensor whose address was recorded alive
    (temporary workspaces included), so a replay never writes into freed
    memory. Before each recorded index call it checks that the workspace's
    head is laid out for that call's B*T; if another call has used the buffer
    under a different B*T since, the buffer is zero-filled on the recorded
    stream first."""
    global _RECORD, _KEEP, _PENDING_HEAD
    _RECORD, _KEEP, _PENDING_HEAD = [], [], None
    try:
        fn()
    finally:
        calls, keep, _RECORD, _KEEP, _PENDING_HEAD = _RECORD, _KEEP, None, None, None

    def run():
        for name, f, args, head in calls:
            if head is not None:
                _ensure_head(*head)
            st = f(*args)
            if st:
                _check(st, name)
    run.kept_tensors = keep
    return run


def lib():
    """The loaded libcsa.so (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CSAError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        sig = {
            "csa_status_string": (ctypes.c_char_p, [I]),
            "csa_version": (I, []),
            "csa_cache_bytes": (I64, [I64, I, I, I]),
            "csa_compress_quantize": (I, [P, I64, P, I, I64, I64, I, I, P, P, I64, I, P]),
            "csa_dequantize": (I, [P, P, I64, I, I64, I64, I, P, I, I, P]),
            "csa_index_topk_workspace": (I64, [I, I, I64, I, I]),
            "csa_index_topk": (I, [P, P, P, I64, I, I, I, I, I, I64, P, I, I, P, P, P, I64, P]),
            "csa_index_scan": (I, [P, P, P, I64, I, I, I, I, I, I64, P, I, I, P, P, P, I64, P]),
            "csa_index_select": (I, [P, P, P, I64, I, I, I, I, I, I64, P, I, I, P, P, P, I64, P]),
            "csa_index_topk_pool_workspace": (I64, [I, I, I64]),
            "csa_index_topk_pool": (I, [P, P, P, I64, I, I, I, I, I, I64, I, P, P, I, I, P, P,
                                        I64, P]),
            "csa_index_pool_scan": (I, [P, P, P, I64, I, I, I, I, I, I64, I, P, P, I, I, P, P,
                                        I64, P]),
            "csa_index_pool_select": (I, [P, P, P, I64, I, I, I, I, I, I64, I, P, P, I, I, P, P,
                                          I64, P]),
            "csa_decode_append": (I, [P, I64, P, P, I, I, I, P, P, P, P, I64, P, I, I, P]),
            "csa_index_topk_ragged": (I, [P, P, P, I64, I, I, I, I, I, P, I64, P, I, I, P, P, P,
                                          I64, P]),
            "csa_index_scan_ragged": (I, [P, P, P, I64, I, I, I, I, I, P, I64, P, I, I, P, P, P,
                                          I64, P]),
            "csa_index_select_ragged": (I, [P, P, P, I64, I, I, I, I, I, P, I64, P, I, I, P, P,
                                            P, I64, P]),
            "csa_sparse_attn_ragged": (I, [P, P, P, I64, P, I, P, I, I, I, I, I, I, P, I64, F, P,
                                           I, P, P, I64, I, P]),
            "hca_dense_attn_ragged": (I, [P, P, P, I64, I, P, I, I, I, I, I, I, P, I64, F, P, I,
                                          P, P, I64, I, P]),
            "csa_workspace_clear": (I, [P, I64, P]),
            "csa_attn_workspace": (I64, [I, I, I, I, I64]),
            "csa_sparse_attn": (I, [P, P, P, I64, P, I, P, I, I, I, I, I, I, I64, F, P, I, P,
                                    P, I64, I, P]),
            "hca_dense_attn": (I, [P, P, P, I64, I, P, I, I, I, I, I, I, I64, F, P, I, P, P,
                                   I64, I, P]),
            "csa_sparse_attn_noalloc": (I, [P, P, P, I64, P, I, P, I, I, I, I, I, I, I64, F, P, I,
                                            P, I, P]),
            "csa_index_attn_workspace": (I64, [I, I, I64, I, I, I, I]),
            "csa_index_attn": (I, [P, P, P, I64, I, I, I, I, I, I64, P, P, I, I, P, P, P, P, I, I,
                                   I, I, F, P, P, P, I, P, P, I64, I, P]),
            "csa_index_attn_scan": (I, [P, P, P, I64, I, I, I, I, I, I64, P, P, I, I, P, P, P, P,
                                        I, I, I, I, F, P, P, P, I, P, P, I64, I, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib if _RECORD is None else _RecordingLib(_lib)


def _check(status: int, what: str):
    if status != 0:
        msg = lib().csa_status_string(status).decode()
        raise CSAError(f"{what}: {msg} ({status})")


def _ptr(t):
    if t is None:
        return None
    if _KEEP is not None:
        _KEEP.append(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name, ndim=None):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")


def _fmt_code(fmt):
    if fmt not in SCALE_FMT:
        raise ValueError(f"unknown scale format {fmt!r} (e8m0 or e4m3)")
    return SCALE_FMT[fmt]


def _check_scales(scales, codes, fmt, what):
    if scales.shape[:2] != codes.shape[:2] or scales.shape[2] * SCALE_GROUP[fmt] != codes.shape[2] * 2:
        raise ValueError(f"{what}: scales must be [B][blk_cap][d/{SCALE_GROUP[fmt]}] for {fmt}")


def cache_bytes(n_tokens: int, d: int, m: int, fmt: str = "e8m0") -> int:
    return lib().csa_cache_bytes(n_tokens, d, m, _fmt_code(fmt))


class Workspace:
    """Zero-initialised device workspace that grows on demand."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None
        self.key = None

    def get(self, nbytes: int, key=None):
        """A buffer of at least nbytes. `key` names the layout of the
        workspace head (B*T for the indexer); the buffer is zero-filled
        again whenever it changes (the key is kept on the buffer itself, so
        replays of prepare() see what eager calls did to it)."""
        if nbytes <= 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(nbytes + 256, dtype=torch.uint8, device=self.device or "cuda")
            self.buf._csa_key = key
        _ensure_head(self.buf, key)
        self.key = key
        return self.buf


_DEFAULT_WS = {}


def _default_ws(device):
    """Per-device index workspace used when the caller passes none (calls on
    one device must then be ordered, e.g. issued on one stream)."""
    key = str(device)
    if key not in _DEFAULT_WS:
        _DEFAULT_WS[key] = Workspace(device)
    return _DEFAULT_WS[key]


def compress_quantize(kv, gate, tok0: int, m: int, codes, scales, fmt: str = "e8m0"):
    """kv float32 [B][n_tok][kv_ld] (d = codes.shape[2]*2 columns used),
    gate float32 [B][n_tok], codes uint8 [B][blk_cap][d/2], scales uint8
    [B][blk_cap][d/32] (fmt "e8m0") or [B][blk_cap][d/16] (fmt "e4m3")."""
    _need(kv, torch.float32, "kv", 3)
    _need(gate, torch.float32, "gate", 2)
    _need(codes, torch.uint8, "codes", 3)
    _need(scales, torch.uint8, "scales", 3)
    B, n_tok, ld = kv.shape
    d = codes.shape[2] * 2
    if gate.shape != (B, n_tok) or codes.shape[0] != B:
        raise ValueError("compress_quantize: inconsistent shapes")
    _check_scales(scales, codes, fmt, "compress_quantize")
    _check(lib().csa_compress_quantize(_ptr(kv), ld, _ptr(gate), B, tok0, n_tok, d, m,
                                       _ptr(codes), _ptr(scales), codes.shape[1], _fmt_code(fmt),
                                       _stream()), "csa_compress_quantize")


def decode_append(kv, gate, pos, m: int, stage, stage_gate, codes, scales, win,
                  fmt: str = "e8m0"):
    """One new token per sequence at its own position; see csa_decode_append.
    kv float32 [B][kv_ld] (d = codes.shape[2]*2 columns used), gate float32
    [B], pos int64 [B] (device; < 0 skips a sequence), stage float32
    [B][m][d], stage_gate float32 [B][m], win bfloat16 [B][Wcap][d]."""
    _need(kv, torch.float32, "kv", 2)
    _need(gate, torch.float32, "gate", 1)
    _need(pos, torch.int64, "pos", 1)
    _need(stage, torch.float32, "stage", 3)
    _need(stage_gate, torch.float32, "stage_gate", 2)
    _need(codes, torch.uint8, "codes", 3)
    _need(scales, torch.uint8, "scales", 3)
    _need(win, torch.bfloat16, "win", 3)
    B, ld = kv.shape
    d = codes.shape[2] * 2
    if (gate.shape != (B,) or pos.shape != (B,) or stage.shape != (B, m, d)
            or stage_gate.shape != (B, m) or codes.shape[0] != B
            or win.shape[0] != B or win.shape[2] != d):
        raise ValueError("decode_append: inconsistent shapes")
    _check_scales(scales, codes, fmt, "decode_append")
    _check(lib().csa_decode_append(_ptr(kv), ld, _ptr(gate), _ptr(pos), B, d, m, _ptr(stage),
                                   _ptr(stage_gate), _ptr(codes), _ptr(scales), codes.shape[1],
                                   _ptr(win), win.shape[1], _fmt_code(fmt), _stream()),
           "csa_decode_append")


def dequantize(codes, scales, blk0: int, n_blk: int, out, fmt: str = "e8m0"):
    _need(codes, torch.uint8, "codes", 3)
    _need(scales, torch.uint8, "scales", 3)
    _check_scales(scales, codes, fmt, "dequantize")
    B, cap, half = codes.shape
    dt = {torch.bfloat16: BF16, torch.float32: F32, torch.float16: F16}[out.dtype]
    _need(out, out.dtype, "out", 3)
    if out.shape != (B, n_blk, 2 * half):
        raise ValueError("dequantize: out must be [B][n_blk][d]")
    _check(lib().csa_dequantize(_ptr(codes), _ptr(scales), cap, B, blk0, n_blk, 2 * half,
                                _ptr(out), dt, _fmt_code(fmt), _stream()), "csa_dequantize")


def _note_head(workspace, ws, key):
    """While recording: the next recorded call needs the head of ws (a buffer
    of a Workspace) laid out for `key`. Raw tensors passed as workspaces are
    the caller's to clear, as in eager calls."""
    global _PENDING_HEAD
    if _RECORD is not None and ws is not None and isinstance(workspace, Workspace):
        _PENDING_HEAD = (ws, key, _stream())


def index_topk_workspace(B, T, n_max, k, cand_given=False) -> int:
    return lib().csa_index_topk_workspace(B, T, n_max, k, int(bool(cand_given)))


def _positions(pos0, pos_max, B, device, what):
    """(host pos0 or pos_max, device positions or None): pos0 is an int, or an
    int64 [B] tensor of per-sequence positions bounded by pos_max."""
    if not isinstance(pos0, torch.Tensor):
        return int(pos0), None
    if pos_max is None:
        raise ValueError(f"{what}: per-sequence positions need pos_max")
    _need(pos0, torch.int64, "pos", 1)
    if pos0.shape != (B,) or pos0.device != device:
        raise ValueError(f"{what}: pos must be an int64 [B] tensor on the data's device")
    return int(pos_max), pos0


def _index_call(fn_name, q_idx, w, keys, m, pos0, k, out_idx, out_score=None, cand=None,
                workspace=None, pos_max=None):
    _need(q_idx, torch.int8, "q_idx", 4)
    _need(w, torch.int8, "w", 3)
    _need(keys, torch.int8, "keys", 3)
    _need(out_idx, torch.int32, "out_idx", 3)
    _need(out_score, torch.int32, "out_score", 3)
    _need(cand, torch.int32, "cand", 3)
    B, T, Hi, Di = q_idx.shape
    pos0, pos = _positions(pos0, pos_max, B, q_idx.device, "index_topk")
    if w.shape != (B, T, Hi) or keys.shape[0] != B or keys.shape[2] != Di:
        raise ValueError("index_topk: inconsistent shapes")
    if out_idx.shape != (B, T, k) or (out_score is not None and out_score.shape != (B, T, k)):
        raise ValueError("index_topk: out_idx / out_score must be [B][T][k]")
    C = 0
    if cand is not None:
        if cand.shape[:2] != (B, T):
            raise ValueError("index_topk: cand must be [B][T][C]")
        C = cand.shape[2]
    blk_cap = keys.shape[1]
    n_max = C if cand is not None else min(blk_cap, (pos0 + T) // m)
    need = index_topk_workspace(B, T, n_max, k, cand is not None)
    if workspace is None:
        workspace = _default_ws(q_idx.device)
    ws = workspace.get(need, key=B * T) if isinstance(workspace, Workspace) else workspace
    ws_bytes = 0 if ws is None else ws.numel()
    _note_head(workspace, ws, B * T)
    if pos is not None:
        fn_name += "_ragged"
        _check(getattr(lib(), fn_name)(_ptr(q_idx), _ptr(w), _ptr(keys), blk_cap, B, T, Hi, Di,
                                       m, _ptr(pos), pos0, _ptr(cand), C, k, _ptr(out_idx),
                                       _ptr(out_score), _ptr(ws), ws_bytes, _stream()), fn_name)
        return
    _check(getattr(lib(), fn_name)(_ptr(q_idx), _ptr(w), _ptr(keys), blk_cap, B, T, Hi, Di, m,
                                   pos0, _ptr(cand), C, k, _ptr(out_idx), _ptr(out_score),
                                   _ptr(ws), ws_bytes, _stream()), fn_name)


def index_topk(*args, **kw):
    """Indexer scores + top-k; see csa_index_topk in include/csa.h. pos0 may
    be an int64 [B] tensor of per-sequence positions (then pass pos_max; see
    csa_index_topk_ragged)."""
    _index_call("csa_index_topk", *args, **kw)


def index_scan(*args, **kw):
    _index_call("csa_index_scan", *args, **kw)


def index_select(*args, **kw):
    _index_call("csa_index_select", *args, **kw)


def index_topk_pool_workspace(B, T, n_max) -> int:
    return lib().csa_index_topk_pool_workspace(B, T, n_max)


def index_topk_pool(*args, **kw):
    """Full-mode top-k plus the blockwise candidate pool; see
    csa_index_topk_pool in include/csa.h. out_pool: int32 [B][T][group*n_keep]."""
    _pool_call("csa_index_topk_pool", *args, **kw)


def index_pool_scan(*args, **kw):
    _pool_call("csa_index_pool_scan", *args, **kw)


def index_pool_select(*args, **kw):
    _pool_call("csa_index_pool_select", *args, **kw)


def _pool_call(fn_name, q_idx, w, keys, m, pos0, k, out_idx, n_keep, out_pool, out_score=None,
               group=8, workspace=None):
    _need(q_idx, torch.int8, "q_idx", 4)
    _need(w, torch.int8, "w", 3)
    _need(keys, torch.int8, "keys", 3)
    _need(out_idx, torch.int32, "out_idx", 3)
    _need(out_score, torch.int32, "out_score", 3)
    _need(out_pool, torch.int32, "out_pool", 3)
    B, T, Hi, Di = q_idx.shape
    if w.shape != (B, T, Hi) or keys.shape[0] != B or keys.shape[2] != Di:
        raise ValueError("index_topk_pool: inconsistent shapes")
    if out_idx.shape != (B, T, k) or (out_score is not None and out_score.shape != (B, T, k)):
        raise ValueError("index_topk_pool: out_idx / out_score must be [B][T][k]")
    if out_pool.shape != (B, T, group * n_keep):
        raise ValueError("index_topk_pool: out_pool must be [B][T][group * n_keep]")
    blk_cap = keys.shape[1]
    n_max = min(blk_cap, (pos0 + T) // m)
    need = index_topk_pool_workspace(B, T, n_max)
    if workspace is None:
        workspace = _default_ws(q_idx.device)
    ws = workspace.get(need, key=B * T) if isinstance(workspace, Workspace) else workspace
    ws_bytes = 0 if ws is None else ws.numel()
    _note_head(workspace, ws, B * T)
    _check(getattr(lib(), fn_name)(_ptr(q_idx), _ptr(w), _ptr(keys), blk_cap, B, T, Hi, Di, m,
                                   pos0, k, _ptr(out_idx), _ptr(out_score), group, n_keep,
                                   _ptr(out_pool), _ptr(ws), ws_bytes, _stream()), fn_name)


def workspace_clear(ws):
    _need(ws, torch.uint8, "ws")
    _check(lib().csa_workspace_clear(_ptr(ws), ws.numel() // 4 * 4, _stream()),
           "csa_workspace_clear")


def attn_workspace(B, T, H, d, n_slots) -> int:
    return lib().csa_attn_workspace(B, T, H, d, n_slots)


def _attn_common(q, codes, scales, win, out, lse, fmt):
    _need(q, torch.bfloat16, "q", 4)
    _need(codes, torch.uint8, "codes", 3)
    _need(scales, torch.uint8, "scales", 3)
    _need(win, torch.bfloat16, "win", 3)
    _need(lse, torch.float32, "lse", 3)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    _need(out, out.dtype, "out", 4)
    B, T, H, d = q.shape
    if out.shape != q.shape or win.shape[0] != B or win.shape[2] != d:
        raise ValueError("attention: inconsistent shapes")
    if codes.shape[0] != B or codes.shape[2] * 2 != d:
        raise ValueError("attention: cache shape mismatch")
    _check_scales(scales, codes, fmt, "attention")
    if lse is not None and lse.shape != (B, T, H):
        raise ValueError("lse must be [B][T][H]")
    return B, T, H, d, (BF16 if out.dtype == torch.bfloat16 else F32)


def sparse_attn(q, codes, scales, idx, win, W, pos0, softmax_scale, out, lse=None,
                workspace=None, pos_max=None, fmt: str = "e8m0"):
    """Attention over the idx-selected entries plus the window; see
    csa_sparse_attn (csa_sparse_attn_ragged when pos0 is an int64 [B] tensor
    of per-sequence positions, bounded by pos_max)."""
    B, T, H, d, dt = _attn_common(q, codes, scales, win, out, lse, fmt)
    pos0, pos = _positions(pos0, pos_max, B, q.device, "sparse_attn")
    _need(idx, torch.int32, "idx", 3)
    k = idx.shape[2]
    if idx.shape[:2] != (B, T):
        raise ValueError("idx must be [B][T][k]")
    need = attn_workspace(B, T, H, d, k + W)
    ws = workspace.get(need) if isinstance(workspace, Workspace) else workspace
    if need > 0 and ws is None:
        ws = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if ws is None else ws.numel()
    if pos is not None:
        _check(lib().csa_sparse_attn_ragged(_ptr(q), _ptr(codes), _ptr(scales), codes.shape[1],
                                            _ptr(idx), k, _ptr(win), win.shape[1], W, B, T, H, d,
                                            _ptr(pos), pos0, float(softmax_scale), _ptr(out), dt,
                                            _ptr(lse), _ptr(ws), ws_bytes, _fmt_code(fmt),
                                            _stream()), "csa_sparse_attn_ragged")
        return
    _check(lib().csa_sparse_attn(_ptr(q), _ptr(codes), _ptr(scales), codes.shape[1], _ptr(idx), k,
                                 _ptr(win), win.shape[1], W, B, T, H, d, pos0,
                                 float(softmax_scale), _ptr(out), dt, _ptr(lse), _ptr(ws),
                                 ws_bytes, _fmt_code(fmt), _stream()), "csa_sparse_attn")


def hca_dense_attn(q, codes, scales, m, win, W, pos0, softmax_scale, out, lse=None,
                   workspace=None, pos_max=None, fmt: str = "e8m0"):
    """Attention over every visible entry of an m-token cache plus the window
    (hca_dense_attn_ragged when pos0 is an int64 [B] tensor, bounded by
    pos_max)."""
    B, T, H, d, dt = _attn_common(q, codes, scales, win, out, lse, fmt)
    pos0, pos = _positions(pos0, pos_max, B, q.device, "hca_dense_attn")
    n_slots = min(codes.shape[1], (pos0 + T) // m) + W
    need = attn_workspace(B, T, H, d, n_slots)
    ws = workspace.get(need) if isinstance(workspace, Workspace) else workspace
    if need > 0 and ws is None:
        ws = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if ws is None else ws.numel()
    if pos is not None:
        _check(lib().hca_dense_attn_ragged(_ptr(q), _ptr(codes), _ptr(scales), codes.shape[1], m,
                                           _ptr(win), win.shape[1], W, B, T, H, d, _ptr(pos),
                                           pos0, float(softmax_scale), _ptr(out), dt, _ptr(lse),
                                           _ptr(ws), ws_bytes, _fmt_code(fmt), _stream()),
               "hca_dense_attn_ragged")
        return
    _check(lib().hca_dense_attn(_ptr(q), _ptr(codes), _ptr(scales), codes.shape[1], m, _ptr(win),
                                win.shape[1], W, B, T, H, d, pos0, float(softmax_scale),
                                _ptr(out), dt, _ptr(lse), _ptr(ws), ws_bytes, _fmt_code(fmt),
                                _stream()), "hca_dense_attn")


def sparse_attn_noalloc(q, codes, scales, idx, win, W, pos0, softmax_scale, out, lse=None,
                        fmt: str = "e8m0"):
    """sparse_attn without a workspace: the split partials live in the
    library's static device scratch (csa_sparse_attn_noalloc). Allocates
    nothing; calls on one GPU must not overlap in time."""
    B, T, H, d, dt = _attn_common(q, codes, scales, win, out, lse, fmt)
    _need(idx, torch.int32, "idx", 3)
    if idx.shape[:2] != (B, T):
        raise ValueError("idx must be [B][T][k]")
    _check(lib().csa_sparse_attn_noalloc(_ptr(q), _ptr(codes), _ptr(scales), codes.shape[1],
                                         _ptr(idx), idx.shape[2], _ptr(win), win.shape[1], W, B, T,
                                         H, d, int(pos0), float(softmax_scale), _ptr(out), dt,
                                         _ptr(lse), _fmt_code(fmt), _stream()),
           "csa_sparse_attn_noalloc")


def index_attn_workspace(B, T, n_max, k, H, d, W) -> int:
    return lib().csa_index_attn_workspace(B, T, n_max, k, H, d, W)


def index_attn(q_idx, w, keys, m, pos0, k, q, codes, scales, win, W, softmax_scale, out_idx, out,
               out_score=None, lse=None, cand=None, workspace=None, pos_max=None,
               fmt: str = "e8m0", scan_only: bool = False):
    """Indexer top-k + sparse attention of one layer in one call; see
    csa_index_attn in include/csa.h. Same arguments as index_topk followed
    by those of sparse_attn (keys and the FP4 cache share blk_cap). pos0 may
    be an int64 [B] tensor of per-sequence positions bounded by pos_max.
    workspace: a Workspace (kept per B*T as for index_topk) or a raw uint8
    tensor the caller keeps cleared. scan_only: launch only the key scan
    (csa_index_attn_scan), after which the workspace must be cleared."""
    _need(q_idx, torch.int8, "q_idx", 4)
    _need(w, torch.int8, "w", 3)
    _need(keys, torch.int8, "keys", 3)
    _need(out_idx, torch.int32, "out_idx", 3)
    _need(out_score, torch.int32, "out_score", 3)
    _need(cand, torch.int32, "cand", 3)
    B, T, Hi, Di = q_idx.shape
    Bq, Tq, H, d, dt = _attn_common(q, codes, scales, win, out, lse, fmt)
    if (Bq, Tq) != (B, T):
        raise ValueError("index_attn: q and q_idx disagree on [B][T]")
    pos0, pos = _positions(pos0, pos_max, B, q_idx.device, "index_attn")
    if w.shape != (B, T, Hi) or keys.shape[0] != B or keys.shape[2] != Di:
        raise ValueError("index_attn: inconsistent indexer shapes")
    if keys.shape[1] != codes.shape[1]:
        raise ValueError("index_attn: keys and codes must share blk_cap")
    if out_idx.shape != (B, T, k) or (out_score is not None and out_score.shape != (B, T, k)):
        raise ValueError("index_attn: out_idx / out_score must be [B][T][k]")
    C = 0
    if cand is not None:
        if cand.shape[:2] != (B, T):
            raise ValueError("index_attn: cand must be [B][T][C]")
        C = cand.shape[2]
    blk_cap = keys.shape[1]
    n_max = C if cand is not None else min(blk_cap, (pos0 + T) // m)
    need = index_attn_workspace(B, T, n_max, k, H, d, W)
    if workspace is None:
        workspace = _default_ws(q_idx.device)
    ws = workspace.get(need, key=B * T) if isinstance(workspace, Workspace) else workspace
    ws_bytes = 0 if ws is None else ws.numel()
    _note_head(workspace, ws, B * T)
    name = "csa_index_attn_scan" if scan_only else "csa_index_attn"
    _check(getattr(lib(), name)(_ptr(q_idx), _ptr(w), _ptr(keys), blk_cap, B, T, Hi, Di, m, pos0,
                                _ptr(pos), _ptr(cand), C, k, _ptr(q), _ptr(codes), _ptr(scales),
                                _ptr(win), win.shape[1], W, H, d, float(softmax_scale),
                                _ptr(out_idx), _ptr(out_score), _ptr(out), dt, _ptr(lse),
                                _ptr(ws), ws_bytes, _fmt_code(fmt), _stream()), name)
