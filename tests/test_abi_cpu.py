"""The C-ABI library loads and exports every symbol the header declares; host
only argument checks return their status codes (no GPU needed: these calls
return before any HIP call)."""

import ctypes
import math
import os
import re

import pytest

import compressed_sparse_attention_compress_amd as csa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(csa.LIB_PATH):
        from compressed_sparse_attention_compress_amd import _build
        _build.build()
    return csa.lib()


def header_functions():
    src = open(os.path.join(ROOT, "include", "csa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b((?:csa|hca)_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) >= 12
    assert sorted(csa.EXPORTED) == names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    for s in range(-8, 1):
        assert L.csa_status_string(s).startswith(b"CSA")
    assert L.csa_version() >= 100


def test_cache_bytes_closed_form(L):
    for d in (32, 128, 512):
        for m in (1, 4, 128):
            for n in (0, 1, 4, 5, 1 << 20, 3 * (1 << 20) + 1):
                assert L.csa_cache_bytes(n, d, m, 0) == math.ceil(n / m) * (d // 2 + d // 32)
                assert L.csa_cache_bytes(n, d, m, 1) == math.ceil(n / m) * (d // 2 + d // 16)
    assert L.csa_cache_bytes((1 << 20) * 8, 512, 4, 0) == 8 * 262144 * 272
    assert L.csa_cache_bytes((1 << 20) * 8, 512, 4, 1) == 8 * 262144 * 288
    assert L.csa_cache_bytes(-1, 512, 4, 0) == -1
    assert L.csa_cache_bytes(8, 100, 4, 0) == -1
    assert L.csa_cache_bytes(8, 512, 4, 2) == -1


def test_argument_errors_before_launch(L):
    P = ctypes.c_void_p
    fake = P(256)
    # compress: m out of range, d unsupported, tok0 not block aligned, NULL
    cq = lambda kv, tok0, d, m, cap, fmt=0: L.csa_compress_quantize(kv, 512, fake, 1, tok0, 8, d,
                                                                    m, fake, fake, cap, fmt, None)
    assert cq(fake, 0, 512, 0, 4) == -2
    assert cq(fake, 0, 100, 4, 4) == -2
    assert cq(fake, 2, 512, 4, 4) == -3
    assert cq(None, 0, 512, 4, 4) == -1
    assert cq(fake, 0, 512, 4, 1) == -3
    assert cq(P(258), 0, 512, 4, 4) == -7
    assert cq(fake, 0, 512, 4, 4, fmt=5) == -5          # unknown scale format
    # indexer: bad Hi / Di / k, missing workspace
    args = lambda Hi, Di, k, ws: (fake, fake, fake, 100, 1, 1, Hi, Di, 4, 399, None, 0, k,
                                  fake, None, ws, 1 << 20, None)
    assert L.csa_index_topk(*args(0, 64, 8, fake)) == -2
    assert L.csa_index_topk(*args(8, 48, 8, fake)) == -2
    assert L.csa_index_topk(*args(8, 64, 0, fake)) == -2
    assert L.csa_index_topk(*args(8, 64, 8, None)) == -4
    assert L.csa_index_topk(fake, fake, fake, 100, 1, 1, 8, 64, 4, 399, None, 0, 8, fake, None,
                            fake, 16, None) == -4
    # blockwise pool: group other than 8, n_keep < 1, missing pool output
    pool = lambda group, n_keep, out: (fake, fake, fake, 100, 1, 1, 8, 64, 4, 399, 8, fake, None,
                                       group, n_keep, out, fake, 1 << 20, None)
    assert L.csa_index_topk_pool(*pool(4, 16, fake)) == -2
    assert L.csa_index_topk_pool(*pool(8, 0, fake)) == -2
    assert L.csa_index_topk_pool(*pool(8, 16, None)) == -1
    # ragged indexer: positions missing or misaligned
    rag = lambda pos: (fake, fake, fake, 100, 1, 1, 8, 64, 4, pos, 399, None, 0, 8, fake, None,
                       fake, 1 << 20, None)
    assert L.csa_index_topk_ragged(*rag(None)) == -1
    assert L.csa_index_topk_ragged(*rag(P(260))) == -7
    # decode append: bad m, bad d, missing positions, misaligned stage
    app = lambda d, m, pos, stage: (fake, 512, fake, pos, 2, d, m, stage, fake, fake, fake, 10,
                                    fake, 128, 0, None)
    assert L.csa_decode_append(*app(512, 0, fake, fake)) == -2
    assert L.csa_decode_append(*app(96, 4, fake, fake)) == -2
    assert L.csa_decode_append(*app(512, 4, None, fake)) == -1
    assert L.csa_decode_append(*app(512, 4, fake, P(264))) == -7
    # attention: bad d, H, window ring too small, dtype
    a = lambda d, H, W, Wcap, T, dt, fmt=0: (fake, fake, fake, 100, fake, 8, fake, Wcap, W, 1, T,
                                             H, d, 399, ctypes.c_float(1.0), fake, dt, None, fake,
                                             1 << 30, fmt, None)
    assert L.csa_sparse_attn(*a(96, 8, 128, 128, 1, 0)) == -2
    assert L.csa_sparse_attn(*a(512, 65, 128, 128, 1, 0)) == -2
    assert L.csa_sparse_attn(*a(512, 64, 128, 128, 2, 0)) == -3
    assert L.csa_sparse_attn(*a(512, 64, 0, 128, 1, 0)) == -2
    assert L.csa_sparse_attn(*a(512, 64, 128, 128, 1, 7)) == -5
    assert L.csa_sparse_attn(*a(512, 64, 128, 128, 1, 0, fmt=3)) == -5
    # positions must fit 31 bits (the window ring slot is a 32-bit remainder)
    far = list(a(512, 64, 128, 128, 1, 0))
    far[13] = (1 << 31) - 1
    assert L.csa_sparse_attn(*far) == -3
    # ragged attention: positions missing
    ra = (fake, fake, fake, 100, fake, 8, fake, 128, 128, 1, 1, 64, 512, None, 399,
          ctypes.c_float(1.0), fake, 0, None, fake, 1 << 30, 0, None)
    assert L.csa_sparse_attn_ragged(*ra) == -1
    rh = (fake, fake, fake, 100, 4, fake, 128, 128, 1, 1, 64, 512, None, 399,
          ctypes.c_float(1.0), fake, 0, None, fake, 1 << 30, 0, None)
    assert L.hca_dense_attn_ragged(*rh) == -1


def test_workspace_sizes(L):
    # every plan keeps a score and a candidate slot per visible entry
    assert L.csa_index_topk_workspace(8, 1, 262144, 1024, 0) > 8 * 262144 * 12
    assert L.csa_index_topk_workspace(1, 8192, 32768, 512, 0) > 8192 * 32768 * 12
    assert L.csa_index_topk_workspace(16, 1, 4096, 512, 1) > 0
    # the pool adds a group score and a group candidate slot per 8 entries
    for BT, n in ((8, 262144), (1, 100), (64, 4096)):
        plain = L.csa_index_topk_workspace(BT, 1, n, 512, 0)
        assert L.csa_index_topk_pool_workspace(BT, 1, n) >= plain + BT * (n // 8) * 12
    assert L.csa_index_topk_pool_workspace(-1, 1, 8) == -1
    assert L.csa_attn_workspace(1, 8192, 64, 512, 640) == 0
    assert L.csa_attn_workspace(8, 1, 64, 512, 1152) >= 8 * 9 * 64 * 512 * 4


def test_noalloc_scratch_limit(L):
    """csa_sparse_attn_noalloc refuses, before any HIP call, a plan whose
    split partials exceed the static scratch; host argument errors come
    first, as in csa_sparse_attn."""
    P = ctypes.c_void_p
    fake = P(256)
    na = lambda B, T, H, d, k, W, Wcap: (fake, fake, fake, 1 << 20, fake, k, fake, Wcap, W, B, T,
                                         H, d, 399 + T, ctypes.c_float(1.0), fake, 0, None, 0,
                                         None)
    assert L.csa_sparse_attn_noalloc(*na(1, 1, 64, 96, 8, 128, 128)) == -2
    assert L.csa_sparse_attn_noalloc(*na(1, 1, 65, 512, 8, 128, 128)) == -2
    assert L.csa_sparse_attn_noalloc(*na(0, 1, 64, 512, 8, 128, 128)) == 0
    limit = csa.NOALLOC_SCRATCH_MAX
    over = None
    for B in (1, 2, 7, 64, 255, 1024, 4096, 65535):
        for k in (16, 1024, 8192, 65536):
            if L.csa_attn_workspace(B, 1, 64, 512, k + 128) > limit:
                over = (B, k)
                break
        if over:
            break
    if over is not None:
        B, k = over
        assert L.csa_sparse_attn_noalloc(*na(B, 1, 64, 512, k, 128, 128)) == -8
    else:
        # no decode plan at these shapes needs more than the static scratch
        assert L.csa_attn_workspace(255, 1, 64, 512, 1024 + 128) <= limit


def test_prepare_keeps_marshalled_tensors_alive():
    """prepare() holds every tensor whose address it marshalled, so a replay
    never reaches freed memory (checked with a CPU tensor: no GPU call)."""
    import gc
    import weakref

    import torch
    t = torch.zeros(16)
    ref = weakref.ref(t)
    run = csa.prepare(lambda: csa._ptr(t))
    del t
    gc.collect()
    assert ref() is not None and any(k is ref() for k in run.kept_tensors)
    del run
    gc.collect()
    assert ref() is None


def test_index_attn_argument_errors(L):
    """csa_index_attn checks the indexer and the attention arguments, then
    the workspace, before launching anything."""
    P = ctypes.c_void_p
    fake = P(256)

    def call(k=64, Di=64, d=512, H=64, W=128, ws=fake, ws_bytes=1 << 30, pos=None, out_dtype=0):
        return L.csa_index_attn(fake, fake, fake, 1 << 16, 2, 1, 8, Di, 4, 4 * 1000, pos, None, 0,
                                k, fake, fake, fake, fake, 256, W, H, d, ctypes.c_float(1.0),
                                fake, None, fake, out_dtype, None, ws, ws_bytes, 0, None)
    assert call(k=0) == -2
    assert call(Di=48) == -2
    assert call(d=96) == -2
    assert call(H=65) == -2
    assert call(out_dtype=9) == -5
    assert call(pos=P(260)) == -7
    assert call(ws=None) == -4
    assert call(ws_bytes=1024) == -4
    need = L.csa_index_attn_workspace(2, 1, 1000, 64, 64, 512, 128)
    assert need > L.csa_index_topk_workspace(2, 1, 1000, 64, 0)
    assert L.csa_index_attn_workspace(2, 1, 1000, 0, 64, 512, 128) == -1


def test_index_attn_workspace_covers_pool_plan(L):
    """A call with a candidate pool takes the plain split plan (10 splits of 64
    slots for 512 + 128 slots), not the byte-capped one, so the workspace size
    (which does not know whether a pool is given) covers its partials: 16
    queries x 10 splits x 64 heads x 512 channels x 4 B, on top of the index
    part."""
    B, n_pool, k, H, d, W = 16, 4096, 512, 64, 512, 128
    partials = B * 10 * H * d * 4
    ws = L.csa_index_attn_workspace(B, 1, n_pool, k, H, d, W)
    assert ws >= partials + B * 10 * H * 8
    assert ws >= L.csa_attn_workspace(B, 1, H, d, k + W)
    # the capped plan of a long context without a pool is covered as well
    assert L.csa_index_attn_workspace(8, 1, 262144, 1024, H, d, W) >= 8 * 18 * H * d * 4
