"""Helpers shared by the GPU parity tests: move a seeded case to the GPU,
repack it through the C ABI, run the GEMM, and compute the oracle reference
(on all rows, or on a sampled subset for large M)."""

from __future__ import annotations

import numpy as np
import torch

import mixed_precision_w4a16_repack_amd as w4
import oracle
import w4a16_inputs as wi

DEV = "cuda:0"


def to_dev(case: wi.Case):
    wq = torch.from_numpy(case.weight_packed).to(DEV)
    ws = case.weight_scale.to(DEV)
    zp = None if case.weight_zero_point is None else torch.from_numpy(case.weight_zero_point).to(DEV)
    A = case.A.to(DEV)
    bias = None if case.bias is None else case.bias.to(DEV)
    return wq, ws, zp, A, bias


def repack(case: wi.Case):
    wq, ws, zp, _, _ = to_dev(case)
    return w4.repack(wq, ws, zp, case.G, case.qtype)


def sample_rows(M: int, seed: int = 0, full_below: int = 64) -> np.ndarray:
    """All rows for small M; else rows 0..15, the last 16 and 32 seeded rows."""
    if M <= full_below:
        return np.arange(M)
    rng = np.random.default_rng([M, seed])
    rows = set(range(16)) | set(range(M - 16, M)) | set(rng.choice(M, size=32, replace=False).tolist())
    return np.array(sorted(rows))


def oracle_ref(case: wi.Case, rows=None, qtype=None):
    C, _ = oracle.gemm(case.A, case.weight_packed, case.weight_scale, case.weight_zero_point,
                       case.qtype if qtype is None else qtype, case.G, case.bias, rows=rows)
    return C


def expected_codes_scales_zeros(case: wi.Case):
    codes = oracle.unpack_codes(case.weight_packed)
    zeros = None
    if case.qtype == wi.UINT4:
        zeros = (oracle.unpack_zeros(case.weight_zero_point, case.N) if case.weight_zero_point is not None
                 else np.zeros((case.N, case.Kg), dtype=np.uint8))
    return codes, case.weight_scale, zeros


def rel_err_rows(C_gpu: torch.Tensor, C_ref: np.ndarray, rows) -> float:
    return oracle.rel_err(C_gpu.cpu()[torch.as_tensor(rows)], C_ref)


def pair_order_codes(q: np.ndarray) -> np.ndarray:
    """Row-major int8 codes [..., K] in the stored order of w4a8_quantize:
    each run of 8 columns as 0, 4, 1, 5, 2, 6, 3, 7 (K % 8 == 0)."""
    shape = q.shape
    r = q.reshape(shape[:-1] + (shape[-1] // 8, 8))
    return r[..., [0, 4, 1, 5, 2, 6, 3, 7]].reshape(shape)
