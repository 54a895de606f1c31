"""Seeded synthetic inputs for the W4A16 linear layer, in checkpoint layout.

This module is shared by the tests, the benchmark and the smoke check. It
holds no step of the method: it only draws random bits and numbers and rounds
them to the activation dtype. Unpacking, dequantisation and the product live
in ``oracle/`` (the CPU reference) and in the HIP library, and neither imports
the other.

Checkpoint layout drawn here (compressed-tensors ``wNa16``, as the MI300 Triton
W4A16 page's module docstring lists it):

* ``weight_packed``     ``[N, K/8]`` int32, eight 4-bit codes per word
* ``weight_scale``      ``[N, Kg]`` in the activation dtype, ``Kg = K / G``
* ``weight_zero_point`` ``[N/8, Kg]`` int32, eight 4-bit zeros per word
  (asymmetric ``uint4`` only)

Codes and zeros are "uniform in [0, 15]" and independent. A 32-bit word whose
eight nibbles are independent and uniform over 0..15 is a word uniform over
all 2**32 values, so the packed words are drawn directly as uniform 32-bit
integers: no packing arithmetic is needed to build an input.

Draw order for one case (fixed, so a case is a pure function of its key):
  1. weight words, 2. scales ~ U[0.005, 0.02] in fp64 then rounded to the act
  dtype, 3. zero-point words (uint4 only), 4. activations ~ N(0, sigma) in
  fp64 then rounded, 5. bias ~ N(0, 1) then rounded (only when asked for).
Rounding to fp16/bf16 uses torch's conversion of the fp64 array.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

UINT4B8 = 0  # symmetric, implicit zero 8
UINT4 = 1  # asymmetric, explicit zero points

ACT_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}
DTYPE_CODES = {"f16": 0, "bf16": 1}


def effective_group(K: int, G: int) -> int:
    """G = -1 means one group spanning all of K (per-channel scales)."""
    return K if G == -1 else G


@dataclasses.dataclass
class Case:
    M: int
    N: int
    K: int
    G: int  # as given; -1 allowed
    qtype: int
    dtype: str  # "f16" | "bf16"
    weight_packed: np.ndarray  # int32 [N, K/8]
    weight_scale: torch.Tensor  # act [N, Kg] (CPU)
    weight_zero_point: np.ndarray | None  # int32 [N/8, Kg] or None
    A: torch.Tensor  # act [M, K] (CPU)
    bias: torch.Tensor | None  # act [N] or None

    @property
    def Kg(self) -> int:
        return self.K // effective_group(self.K, self.G)

    @property
    def torch_dtype(self) -> torch.dtype:
        return ACT_DTYPES[self.dtype]


def _to_act(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(ACT_DTYPES[dtype])


def case_seed(cfg_id: int, M: int, N: int, K: int, G: int, qtype: int, dtype: str, extra: int = 0):
    # SeedSequence entropy must be non-negative; G = -1 is stored as 0.
    return [cfg_id, M, N, K, max(G, 0), qtype, DTYPE_CODES[dtype], extra]


def make_case(
    cfg_id: int,
    M: int,
    N: int,
    K: int,
    G: int,
    qtype: int,
    dtype: str,
    *,
    sigma: float = 1.0,
    mean: float = 0.0,
    with_zero_point: bool | None = None,
    with_bias: bool = False,
    extra: int = 0,
) -> Case:
    """Draw one case. ``with_zero_point`` defaults to ``qtype == UINT4``.
    ``mean`` shifts the activations, A ~ N(mean, sigma) (0 everywhere except
    the tests of sums over long K of non-zero-mean activations)."""
    if with_zero_point is None:
        with_zero_point = qtype == UINT4
    Ge = effective_group(K, G)
    if K % 8 or Ge <= 0 or K % Ge:
        raise ValueError(f"cannot draw K={K}, G={G}")
    Kg = K // Ge
    rng = np.random.default_rng(case_seed(cfg_id, M, N, K, G, qtype, dtype, extra))
    words = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    scales = _to_act(rng.uniform(0.005, 0.02, size=(N, Kg)), dtype)
    zp = None
    if with_zero_point:
        if N % 8:
            raise ValueError(f"zero points need N % 8 == 0, got N={N}")
        zp = rng.integers(0, 2**32, size=(N // 8, Kg), dtype=np.uint64).astype(np.uint32).view(np.int32)
    A = _to_act(rng.normal(mean, sigma, size=(M, K)), dtype)
    bias = _to_act(rng.normal(0.0, 1.0, size=(N,)), dtype) if with_bias else None
    return Case(M, N, K, G, qtype, dtype, words.view(np.int32), scales, zp, A, bias)


@dataclasses.dataclass
class LayoutWeights:
    """A checkpoint drawn directly in one of the other orientations: the
    weight words ``[N, K/8]``, ``[N/8, K]``, ``[K, N/8]`` or ``[K/8, N]`` by
    (output_dim, packed_dim), scales ``[N, Kg]`` or ``[Kg, N]``, zero-point words
    ``[N/8, Kg]`` or ``[Kg, N/8]``."""

    N: int
    K: int
    G: int
    qtype: int
    dtype: str
    weight_output_dim: int
    weight_packed_dim: int
    scale_output_dim: int
    zero_output_dim: int
    weight: np.ndarray  # int32
    weight_scale: torch.Tensor  # act dtype (CPU)
    weight_zero_point: np.ndarray | None  # int32


def make_layout_weights(cfg_id: int, N: int, K: int, G: int, qtype: int, dtype: str, weight_output_dim: int,
                        weight_packed_dim: int, scale_output_dim: int, zero_output_dim: int,
                        with_zero_point: bool | None = None) -> LayoutWeights:
    """Draw a weight, scales and zero points in the given orientation: uniform
    32-bit words (eight independent uniform nibbles each), scales as in
    ``make_case``. Same draw order as ``make_case``, without activations."""
    if with_zero_point is None:
        with_zero_point = qtype == UINT4
    Ge = effective_group(K, G)
    if K % 8 or N % 8 or Ge <= 0 or K % Ge:
        raise ValueError(f"cannot draw N={N}, K={K}, G={G}")
    Kg = K // Ge
    wdims = [N, K] if weight_output_dim == 0 else [K, N]
    wdims[weight_packed_dim] //= 8
    rng = np.random.default_rng(case_seed(cfg_id, 0, N, K, G, qtype, dtype,
                                          1000 + 8 * weight_output_dim + 4 * weight_packed_dim
                                          + 2 * scale_output_dim + zero_output_dim))
    words = rng.integers(0, 2**32, size=tuple(wdims), dtype=np.uint64).astype(np.uint32).view(np.int32)
    sdims = (N, Kg) if scale_output_dim == 0 else (Kg, N)
    scales = _to_act(rng.uniform(0.005, 0.02, size=sdims), dtype)
    zp = None
    if with_zero_point:
        zdims = (N // 8, Kg) if zero_output_dim == 0 else (Kg, N // 8)
        zp = rng.integers(0, 2**32, size=zdims, dtype=np.uint64).astype(np.uint32).view(np.int32)
    return LayoutWeights(N, K, G, qtype, dtype, weight_output_dim, weight_packed_dim, scale_output_dim,
                         zero_output_dim, words, scales, zp)


def centred_codes(seed: int, centre: np.ndarray, sd: float = 2.5) -> np.ndarray:
    """Integer codes in [0, 15] drawn around a per-element centre: round a
    N(centre, sd) draw to the nearest integer and clip it to the code range.
    ``centre`` has the shape of the codes (e.g. [N, K], the zero of each
    weight). Returns uint8 codes; packing them is left to the caller."""
    rng = np.random.default_rng([seed, 4242])
    x = rng.normal(0.0, sd, size=centre.shape) + centre
    return np.clip(np.rint(x), 0, 15).astype(np.uint8)


def random_activations(cfg_id: int, M: int, K: int, dtype: str, sigma: float = 1.0, extra: int = 0) -> torch.Tensor:
    """Activations alone, for benchmarks that rotate several activation buffers."""
    rng = np.random.default_rng([cfg_id, M, K, DTYPE_CODES[dtype], 7919, extra])
    return _to_act(rng.normal(0.0, sigma, size=(M, K)), dtype)


# The workloads of the benchmark and the parity tests: (name, cfg_id, dtype, G,
# qtype, sigma, list of (M, N, K)).
WORKLOADS = {
    "tiny": dict(cfg_id=1, dtype="f16", G=128, qtype=UINT4B8, sigma=1.0, shapes=[(1, 256, 512)]),
    "decode_sym": dict(
        cfg_id=2,
        dtype="f16",
        G=128,
        qtype=UINT4B8,
        sigma=1.0,
        shapes=[(M, N, K) for (N, K) in [(4096, 4096), (14336, 4096), (4096, 14336)] for M in (1, 4, 8, 16)],
    ),
    "decode_asym": dict(
        cfg_id=3, dtype="bf16", G=32, qtype=UINT4, sigma=1.0, shapes=[(M, 6144, 4096) for M in (1, 8)]
    ),
    "crossover": dict(
        cfg_id=4, dtype="f16", G=64, qtype=UINT4B8, sigma=0.5, shapes=[(M, 14336, 4096) for M in (32, 64, 128, 256)]
    ),
    # prefill: G in {-1, 256} x {uint4b8, uint4}; listed per (G, qtype) below
    "prefill": dict(
        cfg_id=5,
        dtype="bf16",
        sigma=1.0,
        variants=[(-1, UINT4B8), (256, UINT4B8), (-1, UINT4), (256, UINT4)],
        shapes=[(M, N, K) for M in (2048, 8192) for (N, K) in [(14336, 4096), (4096, 14336)]],
    ),
}
