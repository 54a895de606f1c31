"""CPU oracle for the W4A16 linear layer -- TEST INFRASTRUCTURE, NOT THE PRODUCT.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library and its Python binding
never import it, and it imports nothing from them.

The arithmetic lives in ``w4a16_oracle.c`` (plain C, fp64, OpenMP over output
rows); this file compiles it with gcc and marshals numpy/torch arrays. See the
C file's header for the passages each function follows. The readers of the
other checkpoint orientations (``unpack_int4``, ``weight_codes_nk``,
``scales_nk``, ``zeros_nk``) are index work only and are plain numpy here.

Parity: every function here is pinned by ``tests/test_oracle.py`` against hand
words derived from the stated bit positions, the little-endian byte view,
exact rational brute force on tiny cases, closed forms and invariants.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a16_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

UINT4B8 = 0
UINT4 = 1

# Parity tolerances of the product path (relative max error), from the
# project's statement of the target: fp16 2e-3, bf16 1e-2.
TOLERANCE = {"f16": 2e-3, "bf16": 1e-2}

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP). Returns the library path."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _open(path: str):
    lib = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.w4o_unpack_codes.argtypes = [p, i64, i64, p]
    lib.w4o_pack_codes.argtypes = [p, i64, i64, p]
    lib.w4o_unpack_zeros.argtypes = [p, i64, i64, p]
    lib.w4o_pack_zeros.argtypes = [p, i64, i64, p]
    lib.w4o_dequant.argtypes = [p, p, p, i32, i64, i64, i64, p]
    lib.w4o_gemm.argtypes = [p, i64, i64, p, p, p, i32, i64, i64, i64, p, p, i32]
    lib.w4o_gemm.restype = i32
    lib.w4o_device_size.argtypes = [i64, i64, i64, i32]
    lib.w4o_device_size.restype = i64
    lib.w4o_encode_device.argtypes = [p, p, p, i32, i64, i64, i64, p]
    lib.w4o_max_threads.restype = i32
    lib.w4o_quant_rows_a8.argtypes = [p, i64, i64, p, p]
    lib.w4o_gemm_w4a8.argtypes = [p, p, i64, i64, p, p, i64, i64, p, p]
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = _open(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def _use_library(path: str):
    """Route this module's calls to another build of the oracle source (the
    mutation tests use it to check that the pins catch planted mistakes)."""
    global _lib
    saved = _load()
    _lib = _open(path)
    try:
        yield
    finally:
        _lib = saved


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _words(x) -> np.ndarray:
    """Any int32/uint32 array (numpy or CPU torch) as contiguous uint32 bits."""
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    x = np.ascontiguousarray(x)
    if x.dtype not in (np.int32, np.uint32):
        raise TypeError(f"packed words must be int32/uint32, got {x.dtype}")
    return x.view(np.uint32)


def _f64(x) -> np.ndarray:
    """fp16/bf16/fp32/fp64 values widened exactly to fp64."""
    if isinstance(x, torch.Tensor):
        return np.ascontiguousarray(x.detach().cpu().to(torch.float64).numpy())
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def max_threads() -> int:
    return int(_load().w4o_max_threads())


def unpack_codes(words, K: int | None = None) -> np.ndarray:
    """[N, K/8] packed words -> [N, K] uint8 codes."""
    w = _words(words)
    N, K8 = w.shape
    K = K8 * 8 if K is None else K
    out = np.empty((N, K), dtype=np.uint8)
    _load().w4o_unpack_codes(_ptr(w), N, K, _ptr(out))
    return out


def pack_codes(codes) -> np.ndarray:
    """[N, K] codes (values 0..15) -> [N, K/8] int32 words."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    N, K = c.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    out = np.empty((N, K // 8), dtype=np.uint32)
    _load().w4o_pack_codes(_ptr(c), N, K, _ptr(out))
    return out.view(np.int32)


def unpack_zeros(zp_words, N: int) -> np.ndarray:
    """[N/8, Kg] packed zero-point words -> [N, Kg] uint8 zeros."""
    w = _words(zp_words)
    if w.shape[0] * 8 != N:
        raise ValueError("zero-point words must be [N/8, Kg]")
    Kg = w.shape[1]
    out = np.empty((N, Kg), dtype=np.uint8)
    _load().w4o_unpack_zeros(_ptr(w), N, Kg, _ptr(out))
    return out


def pack_zeros(zeros) -> np.ndarray:
    """[N, Kg] zeros (0..15) -> [N/8, Kg] int32 words."""
    z = np.ascontiguousarray(np.asarray(zeros, dtype=np.uint8))
    N, Kg = z.shape
    if N % 8:
        raise ValueError("N must be a multiple of 8")
    out = np.empty((N // 8, Kg), dtype=np.uint32)
    _load().w4o_pack_zeros(_ptr(z), N, Kg, _ptr(out))
    return out.view(np.int32)


def unpack_int4(words, dim: int) -> np.ndarray:
    """Eight 4-bit values per int32 word along tensor dimension ``dim``.

    The step the MI300 Triton W4A16 page's ``process_weights_after_loading``
    takes first on any checkpoint (``unpack_quantized_values_into_int32`` with
    ``packed_dim``): dimension ``dim`` grows eightfold, word ``j`` of it giving
    entries ``8j .. 8j+7``, entry ``8j + i`` from bits ``[4i, 4i+4)`` (the nibble
    order the compressed-tensors layout states for its words). Plain numpy, no
    C; shared by no product code.
    """
    w = _words(words)
    if w.ndim != 2 or dim not in (0, 1):
        raise ValueError("words must be 2-D and dim 0 or 1")
    w = np.moveaxis(w, dim, -1)
    shifts = np.arange(8, dtype=np.uint32) * 4
    v = (w[..., None] >> shifts) & np.uint32(0xF)
    v = v.reshape(w.shape[0], w.shape[1] * 8)
    return np.ascontiguousarray(np.moveaxis(v, -1, dim).astype(np.uint8))


def weight_codes_nk(weight, output_dim: int, packed_dim: int) -> np.ndarray:
    """A packed weight in any orientation the pages name -> codes [N, K].

    The MI300 Triton W4A16 page (``process_weights_after_loading``) unpacks
    the weight along its ``packed_dim`` and then transposes it when its
    ``output_dim`` (the dimension over the N output features) is not 0: AWQ
    weights arrive as (K, N) with ``output_dim=1``, compressed-tensors ones as
    (N, K) with ``output_dim=0``.
    """
    if output_dim not in (0, 1) or packed_dim not in (0, 1):
        raise ValueError("output_dim and packed_dim must be 0 or 1")
    codes = unpack_int4(weight, packed_dim)
    return np.ascontiguousarray(codes.T) if output_dim != 0 else codes


def scales_nk(scale, output_dim: int) -> torch.Tensor:
    """Scales [N, Kg] (output_dim 0) or [Kg, N] (output_dim 1) -> [N, Kg],
    the page's ``permute_param_layout_(w_s, input_dim=1, output_dim=0)``."""
    if output_dim not in (0, 1):
        raise ValueError("output_dim must be 0 or 1")
    if not isinstance(scale, torch.Tensor):
        raise TypeError("scale must be a torch tensor")
    s = scale.detach().cpu()
    return (s.t() if output_dim != 0 else s).contiguous()


def zeros_nk(zero_point, output_dim: int) -> np.ndarray:
    """Zero points, eight per int32 word along N, -> zeros [N, Kg].

    The MI300 kernel section of the same page: with ``output_dim=1`` the
    tensor is already [K/G, N/8] (AutoGPTQ), with ``output_dim=0`` it is
    [N/8, K/G] (compressed-tensors); either way the words are permuted to
    [N/8, K/G] and unpacked along that first dimension.
    """
    if output_dim not in (0, 1):
        raise ValueError("output_dim must be 0 or 1")
    zw = _words(zero_point)
    if output_dim != 0:
        zw = np.ascontiguousarray(zw.T)
    return unpack_int4(zw, 0)


def dequant(words, scales, zp_words, qtype: int, G: int) -> np.ndarray:
    """Dense fp64 W[N, K] = (q - z) * s."""
    w = _words(words)
    N, K8 = w.shape
    K = K8 * 8
    s = _f64(scales)
    zp = None if zp_words is None else _words(zp_words)
    out = np.empty((N, K), dtype=np.float64)
    _load().w4o_dequant(_ptr(w), _ptr(s), _ptr(zp), qtype, N, K, G, _ptr(out))
    return out


def gemm(A, words, scales, zp_words, qtype: int, G: int, bias=None, rows=None, nthreads: int = 0):
    """fp64 C = A[rows] @ dequant(W)^T (+ bias). Returns (C, threads_used).

    ``rows`` selects a subset of A's rows (the result has one row per entry);
    None means all rows.
    """
    a = _f64(A)
    if rows is not None:
        a = np.ascontiguousarray(a[np.asarray(rows)])
    M, K = a.shape
    w = _words(words)
    N = w.shape[0]
    if w.shape[1] * 8 != K:
        raise ValueError(f"A has K={K} but words imply K={w.shape[1] * 8}")
    s = _f64(scales)
    zp = None if zp_words is None else _words(zp_words)
    b = None if bias is None else _f64(bias)
    C = np.empty((M, N), dtype=np.float64)
    used = _load().w4o_gemm(_ptr(a), M, K, _ptr(w), _ptr(s), _ptr(zp), qtype, N, K, G, _ptr(b), _ptr(C), nthreads)
    if used < 0:
        raise MemoryError("oracle could not allocate a row buffer")
    return C, int(used)


def quant_rows_a8(A):
    """Per-token symmetric int8 quantisation of A [M, K] (fp16/bf16/fp32
    values) -> (q int8 [M, K], xs float32 [M]); see the C file for the rule."""
    a = _f64(A)
    M, K = a.shape
    q = np.empty((M, K), dtype=np.int8)
    xs = np.empty((M,), dtype=np.float32)
    _load().w4o_quant_rows_a8(_ptr(a), M, K, _ptr(q), _ptr(xs))
    return q, xs


def gemm_w4a8(q, xs, words, scales, G: int, bias=None) -> np.ndarray:
    """fp64 C[M, N] = xs[m] * sum_g s[n,g] * sum_{k in g} q[m,k] * (code[n,k] - 8) (+ bias)."""
    qq = np.ascontiguousarray(np.asarray(q, dtype=np.int8))
    x = np.ascontiguousarray(np.asarray(xs, dtype=np.float32))
    w = _words(words)
    s = _f64(scales)
    M, K = qq.shape
    N = w.shape[0]
    if w.shape[1] * 8 != K or x.shape != (M,) or s.shape[0] != N:
        raise ValueError("shape mismatch")
    b = None if bias is None else _f64(bias)
    C = np.empty((M, N), dtype=np.float64)
    _load().w4o_gemm_w4a8(_ptr(qq), _ptr(x), M, K, _ptr(w), _ptr(s), N, G, _ptr(b), _ptr(C))
    return C


def device_size(N: int, K: int, G: int, qtype: int) -> int:
    return int(_load().w4o_device_size(N, K, G, qtype))


def encode_device(codes, scales, zeros, qtype: int, G: int) -> np.ndarray:
    """The device-layout bytes for codes [N,K], act-dtype scales [N,Kg] and zeros [N,Kg] (or None)."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    N, K = c.shape
    if not isinstance(scales, torch.Tensor) or scales.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("scales must be an fp16/bf16 torch tensor")
    bits = np.ascontiguousarray(scales.detach().cpu().contiguous().view(torch.int16).numpy()).view(np.uint16)
    z = None if zeros is None else np.ascontiguousarray(np.asarray(zeros, dtype=np.uint8))
    out = np.empty(device_size(N, K, G, qtype), dtype=np.uint8)
    _load().w4o_encode_device(_ptr(c), _ptr(bits), _ptr(z), qtype, N, K, G, _ptr(out))
    return out


def rel_err(C_test, C_ref) -> float:
    """max|C_test - C_ref| / max|C_ref| in fp64 (C_test upcast exactly).

    When max|C_ref| is 0 the result is max|C_test| (so only an exact 0 passes).
    """
    t = _f64(C_test)
    r = _f64(C_ref)
    if t.shape != r.shape:
        raise ValueError(f"shape mismatch {t.shape} vs {r.shape}")
    if t.size == 0:
        return 0.0
    num = float(np.max(np.abs(t - r)))
    den = float(np.max(np.abs(r)))
    return num / den if den > 0 else num
