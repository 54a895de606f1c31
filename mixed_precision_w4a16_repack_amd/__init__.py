"""Python binding of libw4a16.so: the fused W4A16 linear layer on MI355X.

Argument marshalling only. Every step of the path (repack, dequantisation,
products, reductions, bias, rounding) runs in the HIP kernels of the C
library; this module passes torch tensors' device pointers and the current
stream, allocates outputs with torch, and raises ``RuntimeError`` with the
library's message on any non-zero status. It never falls back to another
implementation: without the built library every call raises.

Names follow the C ABI (include/w4a16.h): ``packed_size``, ``repack``,
``unpack``, ``workspace_size``, ``select_path``, ``gemm``, and the dense
prefill variant ``dequant`` and ``gemm_dense``.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

UINT4B8 = 0
UINT4 = 1
F16 = 0
BF16 = 1
PATH_AUTO = 0
PATH_SKINNY = 1
PATH_MFMA = 2

_DTYPE_CODE = {torch.float16: F16, torch.bfloat16: BF16}

# C ABI function signatures: name -> (restype, argtypes)
_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
SIGNATURES = {
    "w4a16_abi_version": (_I32, []),
    "w4a16_last_error": (ctypes.c_char_p, []),
    "w4a16_packed_size": (ctypes.c_int, [_I64, _I64, _I32, _I32, ctypes.POINTER(_SZ)]),
    "w4a16_repack": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I32, _I32, _P, _SZ, _P]),
    "w4a16_repack_layout": (ctypes.c_int, [_P, _I32, _I32, _P, _I32, _P, _I32, _I64, _I64, _I32, _I32, _P, _SZ, _P]),
    "w4a16_unpack": (ctypes.c_int, [_P, _I64, _I64, _I32, _I32, _P, _P, _P, _P]),
    "w4a16_workspace_size": (ctypes.c_int, [_I64, _I64, _I64, _I32, _I32, _I32, ctypes.POINTER(_SZ)]),
    "w4a16_workspace_counter_bytes": (_SZ, []),
    "w4a16_select_path": (_I32, [_I64, _I32, _I32]),
    "w4a16_gemm": (
        ctypes.c_int,
        [_P, _I64, _I64, _P, _I64, _I64, _I32, _I32, _I32, _P, _P, _I64, _I32, _I32, _P, _SZ, _P],
    ),
    "w4a16_gemm_noalloc": (
        ctypes.c_int,
        [_P, _I64, _I64, _P, _I64, _I64, _I32, _I32, _I32, _P, _P, _I64, _I32, _I32, _P],
    ),
    "w4a16_dequant": (ctypes.c_int, [_P, _I64, _I64, _I32, _I32, _I32, _P, _I64, _P]),
    "w4a8_quantize": (ctypes.c_int, [_P, _I64, _I64, _I64, _I32, _P, _I64, _P, _P]),
    "w4a8_workspace_size": (ctypes.c_int, [_I64, _I64, _I64, _I32, ctypes.POINTER(_SZ)]),
    "w4a8_gemm": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, _I64, _I32, _I32, _P, _P, _I64, _P, _SZ, _P]),
    "w4a16_gemm_dense": (
        ctypes.c_int,
        [_P, _I64, _I64, _P, _I64, _I64, _I64, _I32, _P, _P, _I64, _P, _SZ, _P],
    ),
}

_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH):
    """Load libw4a16.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build it with `python -m mixed_precision_w4a16_repack_amd.build` "
                    "(there is no fallback implementation)"
                )
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def abi_version() -> int:
    return int(load_library().w4a16_abi_version())


def last_error() -> str:
    return load_library().w4a16_last_error().decode()


def _check(status: int):
    if status != 0:
        raise RuntimeError(f"w4a16 status {status}: {last_error()}")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(name: str, t: torch.Tensor | None, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def packed_size(N: int, K: int, group_size: int, qtype: int) -> int:
    out = _SZ(0)
    _check(load_library().w4a16_packed_size(N, K, group_size, qtype, ctypes.byref(out)))
    return int(out.value)


def repack(weight_packed: torch.Tensor, weight_scale: torch.Tensor, weight_zero_point: torch.Tensor | None,
           group_size: int, qtype: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Checkpoint tensors (GPU) -> packed uint8 buffer (GPU)."""
    _need_cuda("weight_packed", weight_packed, torch.int32)
    _need_cuda("weight_scale", weight_scale, (torch.float16, torch.bfloat16))
    _need_cuda("weight_zero_point", weight_zero_point, torch.int32)
    N, K8 = weight_packed.shape
    K = K8 * 8
    for name, t in (("weight_packed", weight_packed), ("weight_scale", weight_scale),
                    ("weight_zero_point", weight_zero_point)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    nbytes = packed_size(N, K, group_size, qtype)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=weight_packed.device)
    _check(load_library().w4a16_repack(
        _ptr(weight_packed), _ptr(weight_scale), _ptr(weight_zero_point), N, K, group_size, qtype,
        _ptr(out), out.numel() * out.element_size(), _stream(weight_packed)))
    return out


def repack_layout(weight: torch.Tensor, weight_output_dim: int, weight_packed_dim: int, weight_scale: torch.Tensor,
                  scale_output_dim: int, weight_zero_point: torch.Tensor | None, zero_output_dim: int,
                  group_size: int, qtype: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Checkpoint tensors in any orientation w4a16_repack_layout accepts -> packed buffer.

    N and K follow from the weight's shape and dims (the packed dimension holds
    a word per eight entries); the scale and zero-point shapes are checked
    against them before the call.
    """
    _need_cuda("weight", weight, torch.int32)
    _need_cuda("weight_scale", weight_scale, (torch.float16, torch.bfloat16))
    _need_cuda("weight_zero_point", weight_zero_point, torch.int32)
    for name, d in (("weight_output_dim", weight_output_dim), ("weight_packed_dim", weight_packed_dim),
                    ("scale_output_dim", scale_output_dim), ("zero_output_dim", zero_output_dim)):
        if d not in (0, 1):
            raise ValueError(f"{name} must be 0 or 1")
    if weight.dim() != 2:
        raise ValueError("weight must be 2-D")
    dims = list(weight.shape)
    dims[weight_packed_dim] *= 8
    N, K = dims[weight_output_dim], dims[1 - weight_output_dim]
    Kg = 1 if group_size == -1 else (K // group_size if group_size > 0 else 0)
    want_s = (N, Kg) if scale_output_dim == 0 else (Kg, N)
    if tuple(weight_scale.shape) != want_s:
        raise ValueError(f"weight_scale must be {list(want_s)}, got {list(weight_scale.shape)}")
    if weight_zero_point is not None:
        want_z = (N // 8, Kg) if zero_output_dim == 0 else (Kg, N // 8)
        if tuple(weight_zero_point.shape) != want_z:
            raise ValueError(f"weight_zero_point must be {list(want_z)}, got {list(weight_zero_point.shape)}")
    for name, t in (("weight", weight), ("weight_scale", weight_scale), ("weight_zero_point", weight_zero_point)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    nbytes = packed_size(N, K, group_size, qtype)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=weight.device)
    _check(load_library().w4a16_repack_layout(
        _ptr(weight), weight_output_dim, weight_packed_dim, _ptr(weight_scale), scale_output_dim,
        _ptr(weight_zero_point), zero_output_dim, N, K, group_size, qtype,
        _ptr(out), out.numel() * out.element_size(), _stream(weight)))
    return out


def unpack(packed: torch.Tensor, N: int, K: int, group_size: int, qtype: int):
    """Packed buffer -> (codes [N,K] uint8, scale bits [N,Kg] int16, zeros [N,Kg] uint8 or None)."""
    _need_cuda("packed", packed)
    Kg = 1 if group_size == -1 else K // group_size
    dev = packed.device
    codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sbits = torch.empty((N, Kg), dtype=torch.int16, device=dev)
    zeros = torch.empty((N, Kg), dtype=torch.uint8, device=dev) if qtype == UINT4 else None
    _check(load_library().w4a16_unpack(_ptr(packed), N, K, group_size, qtype, _ptr(codes), _ptr(sbits),
                                       _ptr(zeros), _stream(packed)))
    return codes, sbits, zeros


def workspace_size(M: int, N: int, K: int, group_size: int, path: int = PATH_AUTO, skinny_max_m: int = 0) -> int:
    out = _SZ(0)
    _check(load_library().w4a16_workspace_size(M, N, K, group_size, path, skinny_max_m, ctypes.byref(out)))
    return int(out.value)


def workspace_counter_bytes() -> int:
    return int(load_library().w4a16_workspace_counter_bytes())


def select_path(M: int, path: int = PATH_AUTO, skinny_max_m: int = 0) -> int:
    r = int(load_library().w4a16_select_path(M, path, skinny_max_m))
    if r < 0:
        raise RuntimeError(f"w4a16 status {r}: {last_error()}")
    return r


class Workspace:
    """A zero-initialised device workspace that grows on demand.

    The library returns the counter region to zero after every call, so one
    workspace serves every shape; calls that share it must be stream-ordered.
    """

    def __init__(self, device):
        self.device = torch.device(device)
        self.buf: torch.Tensor | None = None

    def get(self, nbytes: int) -> torch.Tensor | None:
        if nbytes == 0:
            return self.buf
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf


_workspaces: dict = {}


def _default_workspace(device, kind: str = "w4a16") -> Workspace:
    """The default workspace of one kind of call on a device and stream.
    w4a16_gemm and w4a8_gemm get separate ones: w4a16_gemm needs the counter
    region at the start of its workspace to be zero, and w4a8_gemm writes its
    partial results from the start of its own."""
    key = (kind, torch.device(device).index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None:
        ws = _workspaces[key] = Workspace(device)
    return ws


def gemm(A: torch.Tensor, packed: torch.Tensor, N: int, K: int, group_size: int, qtype: int,
         bias: torch.Tensor | None = None, out: torch.Tensor | None = None, path: int = PATH_AUTO,
         skinny_max_m: int = 0, workspace: Workspace | None = None) -> torch.Tensor:
    """C[M, N] = A[M, K] @ dequant(W)^T (+ bias), on the current stream."""
    _need_cuda("A", A, (torch.float16, torch.bfloat16))
    _need_cuda("packed", packed)
    _need_cuda("bias", bias, A.dtype)
    if A.dim() != 2 or A.shape[1] != K or A.stride(1) != 1:
        raise ValueError(f"A must be [M, K={K}] with unit column stride, got {tuple(A.shape)} {A.stride()}")
    M = A.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    _need_cuda("out", out, A.dtype)
    if out.dim() != 2 or tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise ValueError(f"out must be [M={M}, N={N}] with unit column stride")
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != N or not bias.is_contiguous()):
        raise ValueError(f"bias must be a contiguous [N={N}] tensor")
    ws_bytes = workspace_size(M, N, K, group_size, path, skinny_max_m) if M > 0 else 0
    ws = (workspace or _default_workspace(A.device)).get(ws_bytes)
    _check(load_library().w4a16_gemm(
        _ptr(A), M, A.stride(0), _ptr(packed), N, K, group_size, qtype, _DTYPE_CODE[A.dtype], _ptr(bias),
        _ptr(out), out.stride(0), path, skinny_max_m, _ptr(ws) if ws_bytes else None,
        ws.numel() if (ws is not None and ws_bytes) else 0, _stream(A)))
    return out


def gemm_noalloc(A: torch.Tensor, packed: torch.Tensor, N: int, K: int, group_size: int, qtype: int,
                 bias: torch.Tensor | None = None, out: torch.Tensor | None = None, path: int = PATH_AUTO,
                 skinny_max_m: int = 0) -> torch.Tensor:
    """``gemm`` through w4a16_gemm_noalloc: the split-K workspace is the
    library's static device scratch (no workspace argument). With ``out``
    given, the call allocates nothing, here or in the library."""
    _need_cuda("A", A, (torch.float16, torch.bfloat16))
    _need_cuda("packed", packed)
    _need_cuda("bias", bias, A.dtype)
    if A.dim() != 2 or A.shape[1] != K or A.stride(1) != 1:
        raise ValueError(f"A must be [M, K={K}] with unit column stride, got {tuple(A.shape)} {A.stride()}")
    M = A.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    _need_cuda("out", out, A.dtype)
    if out.dim() != 2 or tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise ValueError(f"out must be [M={M}, N={N}] with unit column stride")
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != N or not bias.is_contiguous()):
        raise ValueError(f"bias must be a contiguous [N={N}] tensor")
    _check(load_library().w4a16_gemm_noalloc(
        _ptr(A), M, A.stride(0), _ptr(packed), N, K, group_size, qtype, _DTYPE_CODE[A.dtype], _ptr(bias),
        _ptr(out), out.stride(0), path, skinny_max_m, _stream(A)))
    return out


def dequant(packed: torch.Tensor, N: int, K: int, group_size: int, qtype: int, dtype: torch.dtype,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """Packed buffer -> dense [N, K] weight RN((q - z) * s) in ``dtype`` (fp16 or bf16)."""
    _need_cuda("packed", packed)
    if dtype not in _DTYPE_CODE:
        raise ValueError(f"dtype {dtype} is not fp16 or bf16")
    if out is None:
        out = torch.empty((N, K), dtype=dtype, device=packed.device)
    _need_cuda("out", out, dtype)
    if out.dim() != 2 or tuple(out.shape) != (N, K) or out.stride(1) != 1:
        raise ValueError(f"out must be [N={N}, K={K}] with unit column stride")
    _check(load_library().w4a16_dequant(_ptr(packed), N, K, group_size, qtype, _DTYPE_CODE[dtype], _ptr(out),
                                        out.stride(0), _stream(packed)))
    return out


def quantize_a8(A: torch.Tensor, out: tuple[torch.Tensor, torch.Tensor] | None = None):
    """Per-token symmetric int8 quantisation: A [M, K] -> (qa [M, K] int8, xs [M] fp32).

    Each run of 8 codes of qa is stored in the order 0, 4, 1, 5, 2, 6, 3, 7
    (the packed weight's code order, which ``gemm_w4a8`` expects)."""
    _need_cuda("A", A, (torch.float16, torch.bfloat16))
    if A.dim() != 2 or A.stride(1) != 1:
        raise ValueError("A must be 2-D with unit column stride")
    M, K = A.shape
    if out is None:
        qa = torch.empty((M, K), dtype=torch.int8, device=A.device)
        xs = torch.empty((M,), dtype=torch.float32, device=A.device)
    else:
        qa, xs = out
        _need_cuda("qa", qa, torch.int8)
        _need_cuda("xs", xs, torch.float32)
        if qa.dim() != 2 or tuple(qa.shape) != (M, K) or qa.stride(1) != 1 or xs.shape != (M,):
            raise ValueError("out must be (qa [M, K] with unit column stride, xs [M])")
    _check(load_library().w4a8_quantize(_ptr(A), M, K, A.stride(0), _DTYPE_CODE[A.dtype], _ptr(qa), qa.stride(0),
                                        _ptr(xs), _stream(A)))
    return qa, xs


def w4a8_workspace_size(M: int, N: int, K: int, group_size: int) -> int:
    out = _SZ(0)
    _check(load_library().w4a8_workspace_size(M, N, K, group_size, ctypes.byref(out)))
    return int(out.value)


def gemm_w4a8(qa: torch.Tensor, xs: torch.Tensor, packed: torch.Tensor, N: int, K: int, group_size: int,
              dtype: torch.dtype, bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
              workspace: Workspace | None = None) -> torch.Tensor:
    """C[M, N] from int8 activations (quantize_a8) and a symmetric (uint4b8) packed weight."""
    _need_cuda("qa", qa, torch.int8)
    _need_cuda("xs", xs, torch.float32)
    _need_cuda("packed", packed)
    if dtype not in _DTYPE_CODE:
        raise ValueError(f"dtype {dtype} is not fp16 or bf16")
    _need_cuda("bias", bias, dtype)
    if qa.dim() != 2 or qa.shape[1] != K or qa.stride(1) != 1:
        raise ValueError(f"qa must be [M, K={K}] with unit column stride")
    M = qa.shape[0]
    if xs.shape != (M,) or not xs.is_contiguous():
        raise ValueError(f"xs must be a contiguous [M={M}] tensor")
    if out is None:
        out = torch.empty((M, N), dtype=dtype, device=qa.device)
    _need_cuda("out", out, dtype)
    if out.dim() != 2 or tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise ValueError(f"out must be [M={M}, N={N}] with unit column stride")
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != N or not bias.is_contiguous()):
        raise ValueError(f"bias must be a contiguous [N={N}] tensor")
    ws_bytes = w4a8_workspace_size(M, N, K, group_size) if M > 0 else 0
    ws = (workspace or _default_workspace(qa.device, "w4a8")).get(ws_bytes)
    _check(load_library().w4a8_gemm(
        _ptr(qa), _ptr(xs), M, qa.stride(0), _ptr(packed), N, K, group_size, _DTYPE_CODE[dtype], _ptr(bias),
        _ptr(out), out.stride(0), _ptr(ws) if ws_bytes else None, ws.numel() if (ws is not None and ws_bytes) else 0,
        _stream(qa)))
    return out


def gemm_dense(A: torch.Tensor, W: torch.Tensor, bias: torch.Tensor | None = None,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """C[M, N] = A[M, K] @ W[N, K]^T (+ bias) for a dense weight (e.g. from ``dequant``), via hipBLASLt."""
    _need_cuda("A", A, (torch.float16, torch.bfloat16))
    _need_cuda("W", W, A.dtype)
    _need_cuda("bias", bias, A.dtype)
    if A.dim() != 2 or A.stride(1) != 1 or W.dim() != 2 or W.stride(1) != 1 or W.shape[1] != A.shape[1]:
        raise ValueError(f"A [M, K] and W [N, K] need unit column strides and equal K, got {tuple(A.shape)}, {tuple(W.shape)}")
    M, K = A.shape
    N = W.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    _need_cuda("out", out, A.dtype)
    if out.dim() != 2 or tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise ValueError(f"out must be [M={M}, N={N}] with unit column stride")
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != N or not bias.is_contiguous()):
        raise ValueError(f"bias must be a contiguous [N={N}] tensor")
    _need_cuda("workspace", workspace)
    _check(load_library().w4a16_gemm_dense(
        _ptr(A), M, A.stride(0), _ptr(W), N, K, W.stride(0), _DTYPE_CODE[A.dtype], _ptr(bias), _ptr(out),
        out.stride(0), _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(A)))
    return out
