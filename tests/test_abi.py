"""C-ABI boundary checks that need no GPU (CPU only).

The library must load, export every function include/w4a16.h declares, and
reject invalid arguments with the documented status and message before any
HIP call (so these calls are safe on a host without a GPU).
"""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import mixed_precision_w4a16_repack_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

OK, INVALID, UNSUPPORTED, SIZE = 0, -1, -2, -3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4.LIB_PATH):
        from mixed_precision_w4a16_repack_amd import build

        build.build()
    return w4.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a(?:16|8)_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_signatures():
    assert set(_declared_functions()) == set(w4.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(w4.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(raw, name), name


def test_abi_version(lib):
    assert w4.abi_version() == 1


def test_packed_size_values(lib):
    # codes N*K/2, scales N*Kg*2 at align256, zeros N*Kg at align256
    assert w4.packed_size(16, 128, 128, w4.UINT4B8) == 1280
    assert w4.packed_size(16, 128, -1, w4.UINT4) == 1536
    assert w4.packed_size(4096, 4096, 128, w4.UINT4B8) == 4096 * 2048 + 4096 * 32 * 2
    assert w4.packed_size(6144, 4096, 32, w4.UINT4) == 6144 * 2048 + 6144 * 128 * 3
    # G = K behaves like G = -1
    assert w4.packed_size(4096, 14336, 14336, w4.UINT4) == w4.packed_size(4096, 14336, -1, w4.UINT4)


@pytest.mark.parametrize("N,K,G,qtype", [(16, 40, -1, 0), (48, 96, 32, 1), (32, 2880, 64, 0), (4096, 1216, 64, 1),
                                          (256, 200, -1, 1), (4096, 14344, -1, 0), (24, 128, 128, 0),
                                          (8, 40, -1, 1), (1224, 2880, 64, 1)])
def test_packed_size_padded_k_matches_oracle(N, K, G, qtype):
    import oracle

    assert w4.packed_size(N, K, G, qtype) == oracle.device_size(N, K, G, qtype)


@pytest.mark.parametrize(
    "N,K,G,qtype,status,needle",
    [
        (4100, 4096, 128, 0, UNSUPPORTED, "N=4100 must be divisible by 8"),
        (4096, 4100, 128, 0, UNSUPPORTED, "K=4100 must be divisible by 8"),
        (4096, 4000, 128, 0, UNSUPPORTED, "K=4000 must be divisible by group_size=128"),
        (4096, 4096, 96, 0, UNSUPPORTED, "group_size=96 not supported"),
        (4096, 4096, 16, 0, UNSUPPORTED, "group_size=16 not supported"),
        (4096, 384, 256, 0, UNSUPPORTED, "K=384 must be divisible by group_size=256"),
        (4096, 4096, 128, 3, INVALID, "qtype=3"),
        (0, 4096, 128, 0, INVALID, "must be positive"),
        (4096, -128, 128, 0, INVALID, "must be positive"),
    ],
)
def test_packed_size_rejects(lib, N, K, G, qtype, status, needle):
    out = ctypes.c_size_t(0)
    st = lib.w4a16_packed_size(N, K, G, qtype, ctypes.byref(out))
    assert st == status
    assert needle in w4.last_error()


def test_null_out_pointer(lib):
    assert lib.w4a16_packed_size(16, 128, 128, 0, None) == INVALID
    assert "out_bytes is NULL" in w4.last_error()


def _gemm(lib, **kw):
    args = dict(A=ctypes.c_void_p(4096), M=4, lda=4096, packed=ctypes.c_void_p(4096), N=4096, K=4096, G=128,
                qtype=0, dtype=0, bias=None, C=ctypes.c_void_p(4096), ldc=4096, path=0, smax=0, ws=None, wsb=0)
    args.update(kw)
    return lib.w4a16_gemm(args["A"], args["M"], args["lda"], args["packed"], args["N"], args["K"], args["G"],
                          args["qtype"], args["dtype"], args["bias"], args["C"], args["ldc"], args["path"],
                          args["smax"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize(
    "kw,status,needle",
    [
        (dict(dtype=2), INVALID, "dtype=2"),
        (dict(path=5), INVALID, "path=5"),
        (dict(M=-1), INVALID, "M=-1"),
        (dict(A=None), INVALID, "must not be NULL"),
        (dict(C=None), INVALID, "must not be NULL"),
        (dict(lda=4000), INVALID, "lda=4000 must be >= K=4096"),
        (dict(ldc=100), INVALID, "ldc=100 must be >= N=4096"),
        (dict(lda=4100), UNSUPPORTED, "lda % 8 == 0"),
        (dict(A=ctypes.c_void_p(4104)), UNSUPPORTED, "16-byte aligned"),
        (dict(packed=ctypes.c_void_p(4100)), INVALID, "256-byte aligned"),
        (dict(K=4004, lda=4004), UNSUPPORTED, "K=4004 must be divisible by 8"),
        (dict(bias=ctypes.c_void_p(4097)), INVALID, "2-byte aligned"),
        # the tiled path addresses one workgroup's tile with 32-bit offsets
        (dict(M=256, lda=1 << 23), UNSUPPORTED, "too large for the tiled path"),
        # a narrow weight (64 n-tiles) splits K on the skinny path and needs a workspace
        (dict(M=1, N=1024, ldc=1024), SIZE, "workspace of 0 bytes is smaller"),
        (dict(M=1, N=1024, ldc=1024, ws=ctypes.c_void_p(4096), wsb=16), SIZE, "workspace of 16 bytes is smaller"),
    ],
)
def test_gemm_rejects_before_any_hip_call(lib, kw, status, needle):
    assert _gemm(lib, **kw) == status
    assert needle in w4.last_error()


def _gemm_noalloc(lib, **kw):
    args = dict(A=ctypes.c_void_p(4096), M=4, lda=4096, packed=ctypes.c_void_p(4096), N=4096, K=4096, G=128,
                qtype=0, dtype=0, bias=None, C=ctypes.c_void_p(4096), ldc=4096, path=0, smax=0)
    args.update(kw)
    return lib.w4a16_gemm_noalloc(args["A"], args["M"], args["lda"], args["packed"], args["N"], args["K"],
                                  args["G"], args["qtype"], args["dtype"], args["bias"], args["C"], args["ldc"],
                                  args["path"], args["smax"], None)


@pytest.mark.parametrize(
    "kw,status,needle",
    [
        (dict(dtype=2), INVALID, "dtype=2"),
        (dict(lda=4000), INVALID, "lda=4000 must be >= K=4096"),
        (dict(A=ctypes.c_void_p(4104)), UNSUPPORTED, "16-byte aligned"),
        (dict(K=4100, lda=4104), UNSUPPORTED, "must be divisible by"),
        # 128 n-tiles with K = 131072 split over 256 chunks: 33.5 MB of partial sums
        (dict(M=1, N=2048, ldc=2048, K=131072, lda=131072), SIZE, "more than the 8454144 bytes of the static scratch"),
    ],
)
def test_gemm_noalloc_rejects_before_any_hip_call(lib, kw, status, needle):
    assert _gemm_noalloc(lib, **kw) == status
    assert needle in w4.last_error()


def test_gemm_noalloc_m_zero_is_a_noop(lib):
    assert _gemm_noalloc(lib, M=0) == OK
    assert w4.last_error() == ""


def test_gemm_noalloc_scratch_limit_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define W4A16_NOALLOC_MAX_WORKSPACE_BYTES \(\(size_t\)\(64 \* 1024\) \+ \(\(size_t\)8 << 20\)\)", text)
    assert m, "the documented scratch size changed"
    # the largest workspace of the decode shapes fits
    for (M, N, K) in [(16, 4096, 14336), (16, 14336, 4096), (16, 4096, 4096), (16, 1024, 14336)]:
        assert w4.workspace_size(M, N, K, 128, w4.PATH_AUTO) <= 64 * 1024 + (8 << 20)


def test_gemm_m_zero_is_a_noop(lib):
    # Pointers are never dereferenced for M == 0.
    assert _gemm(lib, M=0) == OK
    assert w4.last_error() == ""


def test_repack_rejects(lib):
    p = ctypes.c_void_p(4096)
    assert lib.w4a16_repack(None, p, None, 16, 128, 128, 0, p, 1 << 20, None) == INVALID
    assert "weight_packed is NULL" in w4.last_error()
    assert lib.w4a16_repack(p, p, None, 16, 128, 128, 0, p, 1000, None) == SIZE
    assert "packed_bytes=1000" in w4.last_error()
    assert lib.w4a16_repack(p, p, None, 16, 128, 128, 0, ctypes.c_void_p(4160), 1 << 20, None) == INVALID
    assert "256-byte aligned" in w4.last_error()


@pytest.mark.parametrize("dims,needle", [
    ((2, 1, 0, 0), "weight_output_dim=2"),
    ((0, -1, 0, 0), "weight_packed_dim=-1"),
    ((0, 1, 3, 0), "scale_output_dim=3"),
    ((0, 1, 0, 2), "zero_output_dim=2"),
])
def test_repack_layout_rejects_bad_dims(lib, dims, needle):
    p = ctypes.c_void_p(4096)
    od, pd, sd, zd = dims
    assert lib.w4a16_repack_layout(p, od, pd, p, sd, None, zd, 16, 128, 128, 0, p, 1 << 20, None) == INVALID
    assert needle in w4.last_error()


def test_repack_layout_rejects_like_repack(lib):
    p = ctypes.c_void_p(4096)
    for od in (0, 1):
        for pd in (0, 1):
            assert lib.w4a16_repack_layout(None, od, pd, p, 1, None, 1, 16, 128, 128, 0, p, 1 << 20, None) == INVALID
            assert "weight_packed is NULL" in w4.last_error()
            assert lib.w4a16_repack_layout(p, od, pd, p, 1, None, 1, 16, 128, 128, 0, p, 1000, None) == SIZE
            assert lib.w4a16_repack_layout(p, od, pd, p, 1, None, 1, 20, 128, 128, 0, p, 1 << 20, None) == UNSUPPORTED


def test_select_path(lib):
    assert w4.select_path(1) == w4.PATH_SKINNY
    assert w4.select_path(16) == w4.PATH_SKINNY
    assert w4.select_path(17) == w4.PATH_MFMA
    assert w4.select_path(32, skinny_max_m=32) == w4.PATH_SKINNY
    assert w4.select_path(1, path=w4.PATH_MFMA) == w4.PATH_MFMA
    assert w4.select_path(4096, path=w4.PATH_SKINNY) == w4.PATH_SKINNY
    with pytest.raises(RuntimeError, match="path=9"):
        w4.select_path(1, path=9)


def test_workspace_size(lib):
    assert w4.workspace_size(2048, 4096, 4096, 128) == 0  # 128 x 256 tiles fill the CUs: no split
    # medium M: K split over the tiles' workgroups, partial tiles in the workspace
    assert w4.workspace_size(256, 4096, 4096, 128) > w4.workspace_counter_bytes()
    assert w4.workspace_size(256, 4096, 4104, -1) == 0  # a K tail takes the unsplit 64-column tiles
    assert w4.workspace_size(17, 4096, 4096, 128) > 0  # the first M past the skinny path splits K too
    assert w4.workspace_size(96, 512, 1024, 128) == 0  # too few tiles to fill half the CUs: unsplit
    assert w4.workspace_size(16, 4096, 4096, 128) == 0  # wide weights: K is not split
    # long K, one n-tile per workgroup: all of K in one workgroup up to 4 rows
    assert w4.workspace_size(4, 4096, 14336, 128) == 0
    assert w4.workspace_size(1, 4096, 16384, -1) == 0
    assert w4.workspace_size(5, 4096, 14336, 128) > w4.workspace_counter_bytes()  # 5 rows: K chunks
    assert w4.workspace_size(1, 4096, 14336, 64) > w4.workspace_counter_bytes()  # 2 fold blocks per 128 k
    assert w4.workspace_size(16, 4096, 14336, 128) >= w4.workspace_size(1, 4096, 14336, 64)
    ws = w4.workspace_size(16, 1024, 4096, 128)  # narrow weights split K
    assert ws > w4.workspace_counter_bytes()
    # sized for 16 rows, so every M <= 16 fits the same workspace
    assert w4.workspace_size(1, 1024, 4096, 128) == ws
    assert w4.workspace_size(300, 1024, 4096, 128, path=w4.PATH_SKINNY) == ws


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(w4, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        w4.load_library(str(tmp_path / "libw4a16.so"))


def _dequant(lib, **kw):
    args = dict(packed=ctypes.c_void_p(4096), N=4096, K=4096, G=128, qtype=0, dtype=1, dense=ctypes.c_void_p(8192),
                ldw=4096)
    args.update(kw)
    return lib.w4a16_dequant(args["packed"], args["N"], args["K"], args["G"], args["qtype"], args["dtype"],
                             args["dense"], args["ldw"], None)


@pytest.mark.parametrize(
    "kw,status,needle",
    [
        (dict(dtype=2), INVALID, "dtype=2"),
        (dict(K=4004, ldw=4004), UNSUPPORTED, "K=4004 must be divisible by 8"),
        (dict(packed=None), INVALID, "must not be NULL"),
        (dict(dense=None), INVALID, "must not be NULL"),
        (dict(packed=ctypes.c_void_p(4100)), INVALID, "256-byte aligned"),
        (dict(ldw=4000), INVALID, "ldw=4000 must be >= K=4096"),
        (dict(ldw=4100), UNSUPPORTED, "ldw % 8 == 0"),
        (dict(dense=ctypes.c_void_p(8200)), UNSUPPORTED, "16-byte aligned"),
    ],
)
def test_dequant_rejects_before_any_hip_call(lib, kw, status, needle):
    assert _dequant(lib, **kw) == status
    assert needle in w4.last_error()


def _gemm_dense(lib, **kw):
    args = dict(A=ctypes.c_void_p(4096), M=2048, lda=4096, W=ctypes.c_void_p(8192), N=4096, K=4096, ldw=4096,
                dtype=1, bias=None, C=ctypes.c_void_p(16384), ldc=4096, ws=None, wsb=0)
    args.update(kw)
    return lib.w4a16_gemm_dense(args["A"], args["M"], args["lda"], args["W"], args["N"], args["K"], args["ldw"],
                                args["dtype"], args["bias"], args["C"], args["ldc"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize(
    "kw,status,needle",
    [
        (dict(dtype=3), INVALID, "dtype=3"),
        (dict(M=-2), INVALID, "M=-2"),
        (dict(N=0), INVALID, "must be positive"),
        (dict(A=None), INVALID, "must not be NULL"),
        (dict(W=None), INVALID, "must not be NULL"),
        (dict(C=None), INVALID, "must not be NULL"),
        (dict(lda=100), INVALID, "lda=100 must be >= K=4096"),
        (dict(ldw=100), INVALID, "ldw=100 must be >= K=4096"),
        (dict(ldc=100), INVALID, "ldc=100 must be >= N=4096"),
        (dict(bias=ctypes.c_void_p(4097)), INVALID, "2-byte aligned"),
    ],
)
def test_gemm_dense_rejects_before_any_hip_call(lib, kw, status, needle):
    assert _gemm_dense(lib, **kw) == status
    assert needle in w4.last_error()


def test_gemm_dense_m_zero_is_a_noop(lib):
    assert _gemm_dense(lib, M=0) == OK
    assert w4.last_error() == ""


# ---------------------------------------------------------------- W4A8


def _quant(lib, **kw):
    a = dict(A=ctypes.c_void_p(4096), M=4, K=4096, lda=4096, dtype=0, qa=ctypes.c_void_p(8192), ldq=4096,
             xs=ctypes.c_void_p(16384))
    a.update(kw)
    return lib.w4a8_quantize(a["A"], a["M"], a["K"], a["lda"], a["dtype"], a["qa"], a["ldq"], a["xs"], None)


@pytest.mark.parametrize(
    "kw,status,needle",
    [
        (dict(dtype=2), INVALID, "dtype=2"),
        (dict(K=12, lda=12, ldq=16), UNSUPPORTED, "K=12 must be divisible by 8"),
        (dict(lda=4000), INVALID, "lda=4000 must be >= K=4096"),
        (dict(ldq=4000), INVALID, "ldq=4000 must be >= K=4096"),
        (dict(A=None), INVALID, "must not be NULL"),
        (dict(A=ctypes.c_void_p(4104)), UNSUPPORTED, "16-byte aligned"),
        (dict(qa=ctypes.c_void_p(8196)), UNSUPPORTED, "8-byte aligned"),
        (dict(M=-1), INVALID, "M=-1"),
    ],
)
def test_quantize_a8_rejects_before_any_hip_call(lib, kw, status, needle):
    assert _quant(lib, **kw) == status
    assert needle in w4.last_error()


def test_quantize_a8_m_zero_is_a_noop(lib):
    assert _quant(lib, M=0, A=None, qa=None, xs=None) == OK


def _w4a8(lib, **kw):
    a = dict(qa=ctypes.c_void_p(4096), xs=ctypes.c_void_p(8192), M=4096, ldq=4096, packed=ctypes.c_void_p(1 << 20),
             N=4096, K=4096, G=128, dtype=1, bias=None, C=ctypes.c_void_p(16384), ldc=4096, ws=None, wsb=0)
    a.update(kw)
    return lib.w4a8_gemm(a["qa"], a["xs"], a["M"], a["ldq"], a["packed"], a["N"], a["K"], a["G"], a["dtype"],
                         a["bias"], a["C"], a["ldc"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize(
    "kw,status,needle",
    [
        (dict(G=96), UNSUPPORTED, "group_size=96 not supported"),
        (dict(dtype=3), INVALID, "dtype=3"),
        (dict(ldq=100), INVALID, "ldq=100 must be >= K=4096"),
        (dict(ldc=100), INVALID, "ldc=100 must be >= N=4096"),
        (dict(qa=None), INVALID, "must not be NULL"),
        (dict(packed=ctypes.c_void_p(4100)), INVALID, "256-byte aligned"),
        (dict(qa=ctypes.c_void_p(4100)), UNSUPPORTED, "8-byte aligned"),
        # one row over 4096 x 4096 splits K and needs the partials workspace
        (dict(M=1), SIZE, "workspace of 0 bytes is smaller"),
    ],
)
def test_w4a8_gemm_rejects_before_any_hip_call(lib, kw, status, needle):
    assert _w4a8(lib, **kw) == status
    assert needle in w4.last_error()


def test_w4a8_gemm_m_zero_is_a_noop(lib):
    assert _w4a8(lib, M=0, qa=None, xs=None, C=None) == OK


def test_w4a8_workspace_size():
    assert w4.w4a8_workspace_size(1, 4096, 4096, 128) > 0
    assert w4.w4a8_workspace_size(4096, 4096, 4096, 128) == 0
    assert w4.w4a8_workspace_size(0, 4096, 4096, 128) == 0
    # 256 x 4096 x 14336: the tiled kernel splits K into 8 chunks of 14
    # k-tiles (32 tiles, about one workgroup per CU), more than the register
    # kernel's 4; the size covers the larger.
    assert w4.w4a8_workspace_size(256, 4096, 14336, 128) == 8 * 256 * 4096 * 4
