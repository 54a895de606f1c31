"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

* repack / unpack: bit-exact against the oracle's layout encoder and unpack;
* dequantisation: identity activations make C equal RN_act((q - z) * s)
  bit for bit on both kernels;
* GEMM: max|C - C_ref| / max|C_ref| within 2e-3 (fp16) / 1e-2 (bf16) on every
  workload shape at full size (all rows for M <= 64, sampled rows above), on
  the forced skinny and MFMA kernels and on the dispatcher;
* edge cases: M = 0, ragged M and N tails, strided A and C, bias, minimal and
  very large K, G = -1 vs G = K, uint4 without zero points, determinism and
  workspace reuse.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import mixed_precision_w4a16_repack_amd as w4
import oracle
import w4a16_inputs as wi
from tests.gpu_cases import (DEV, expected_codes_scales_zeros, oracle_ref, pair_order_codes, rel_err_rows, repack,
                             sample_rows, to_dev)

pytestmark = pytest.mark.gpu

UINT4B8, UINT4 = wi.UINT4B8, wi.UINT4
SKINNY, MFMA, AUTO = w4.PATH_SKINNY, w4.PATH_MFMA, w4.PATH_AUTO


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    w4.load_library()
    yield
    torch.cuda.synchronize()


def _case(cfg, M, N, K, G, qtype, dtype, **kw):
    return wi.make_case(cfg, M, N, K, G, qtype, dtype, **kw)


# ------------------------------------------------------------------ repack


REPACK_SHAPES = [
    # (N, K, G, qtype, with_zero_point)
    (16, 128, 128, UINT4B8, False),
    (16, 128, -1, UINT4, True),
    (48, 384, 32, UINT4, True),
    (32, 256, 64, UINT4, False),  # uint4 without zero points: zeros are 0
    (256, 512, 128, UINT4B8, False),
    (4096, 4096, 128, UINT4B8, False),
    (6144, 4096, 32, UINT4, True),
    (14336, 4096, 64, UINT4B8, False),
    (4096, 14336, 256, UINT4, True),
    (14336, 4096, -1, UINT4, True),
]


@pytest.mark.parametrize("N,K,G,qtype,zp", REPACK_SHAPES, ids=[f"{s[0]}x{s[1]}g{s[2]}q{s[3]}z{int(s[4])}" for s in REPACK_SHAPES])
def test_repack_bit_exact(N, K, G, qtype, zp):
    case = _case(11, 1, N, K, G, qtype, "bf16" if qtype == UINT4 else "f16", with_zero_point=zp)
    packed = repack(case)
    codes, scales, zeros = expected_codes_scales_zeros(case)
    expect = oracle.encode_device(codes, scales, zeros, qtype, G)
    got = packed.cpu().numpy()
    assert got.shape == expect.shape
    mism = np.flatnonzero(got != expect)
    assert mism.size == 0, f"{mism.size} bytes differ, first at {mism[:8]}"
    # and the inverse
    c2, s2, z2 = w4.unpack(packed, N, K, G, qtype)
    np.testing.assert_array_equal(c2.cpu().numpy(), codes)
    np.testing.assert_array_equal(s2.cpu().numpy(), scales.view(torch.int16).numpy())
    if qtype == UINT4:
        np.testing.assert_array_equal(z2.cpu().numpy(), zeros)


def test_repack_is_deterministic_and_ignores_prior_contents():
    case = _case(12, 1, 64, 512, 64, UINT4, "f16")
    wq, ws, zp, _, _ = to_dev(case)
    a = w4.repack(wq, ws, zp, 64, UINT4)
    b = torch.full_like(a, 0xA5)
    w4.repack(wq, ws, zp, 64, UINT4, out=b)
    assert torch.equal(a, b)


def test_repack_symmetric_ignores_zero_points():
    case = _case(13, 1, 64, 256, 32, UINT4, "f16")
    wq, ws, zp, _, _ = to_dev(case)
    assert torch.equal(w4.repack(wq, ws, zp, 32, UINT4B8), w4.repack(wq, ws, None, 32, UINT4B8))


# ------------------------------------------- repack from other orientations


LAYOUTS = [
    # (N, K, G, qtype, weight_output_dim, weight_packed_dim, scale_output_dim, zero_output_dim, zero points)
    (16, 128, 128, UINT4B8, 1, 1, 1, 1, False),  # AWQ orientation, one tile
    (48, 384, 32, UINT4, 1, 1, 1, 1, True),  # AWQ weight, AutoGPTQ zeros, several tiles
    (48, 384, 64, UINT4, 1, 0, 1, 1, True),  # AutoGPTQ weight
    (32, 256, -1, UINT4, 0, 0, 0, 0, True),  # packed along N, N first
    (64, 512, 128, UINT4, 0, 1, 1, 0, True),  # compressed-tensors weight, (K/G, N) scales
    (80, 640, 128, UINT4, 1, 1, 0, 1, False),  # uint4 without zero points
    (4096, 4096, 128, UINT4, 1, 1, 1, 1, True),
    (14336, 4096, 128, UINT4B8, 1, 0, 1, 1, False),
    (4096, 14336, 32, UINT4, 0, 0, 0, 1, True),
    (6144, 4096, -1, UINT4, 1, 1, 1, 1, True),
]


def _layout_dev(L):
    w = torch.from_numpy(L.weight).to(DEV)
    s = L.weight_scale.to(DEV)
    z = None if L.weight_zero_point is None else torch.from_numpy(L.weight_zero_point).to(DEV)
    return w, s, z


def _layout_expect(L):
    codes = oracle.weight_codes_nk(L.weight, L.weight_output_dim, L.weight_packed_dim)
    scales = oracle.scales_nk(L.weight_scale, L.scale_output_dim)
    zeros = None
    if L.qtype == UINT4:
        Kg = scales.shape[1]
        zeros = (oracle.zeros_nk(L.weight_zero_point, L.zero_output_dim) if L.weight_zero_point is not None
                 else np.zeros((L.N, Kg), dtype=np.uint8))
    return codes, scales, zeros


@pytest.mark.parametrize("N,K,G,qtype,od,pd,sd,zd,zp", LAYOUTS,
                         ids=[f"{c[0]}x{c[1]}g{c[2]}q{c[3]}w{c[4]}{c[5]}s{c[6]}z{c[7]}{int(c[8])}" for c in LAYOUTS])
def test_repack_layout_bit_exact(N, K, G, qtype, od, pd, sd, zd, zp):
    L = wi.make_layout_weights(14, N, K, G, qtype, "bf16" if qtype == UINT4 else "f16", od, pd, sd, zd,
                               with_zero_point=zp)
    w, s, z = _layout_dev(L)
    packed = w4.repack_layout(w, od, pd, s, sd, z, zd, G, qtype)
    codes, scales, zeros = _layout_expect(L)
    expect = oracle.encode_device(codes, scales, zeros, qtype, G)
    got = packed.cpu().numpy()
    assert got.shape == expect.shape
    mism = np.flatnonzero(got != expect)
    assert mism.size == 0, f"{mism.size} bytes differ, first at {mism[:8]}"


def test_repack_layout_canonical_is_repack():
    case = _case(15, 1, 96, 768, 64, UINT4, "bf16")
    wq, ws, zp, _, _ = to_dev(case)
    a = w4.repack(wq, ws, zp, 64, UINT4)
    b = w4.repack_layout(wq, 0, 1, ws, 0, zp, 0, 64, UINT4)
    assert torch.equal(a, b)
    # Every orientation of the same checkpoint gives the same buffer.
    N, K = 96, 768
    wt = wq.t().contiguous()  # (K/8, N): output_dim 1, packed_dim 0
    st = ws.t().contiguous()
    zt = zp.t().contiguous()
    assert torch.equal(w4.repack_layout(wt, 1, 0, st, 1, zt, 1, 64, UINT4), a)
    assert a.numel() == w4.packed_size(N, K, 64, UINT4)


@pytest.mark.parametrize("path", [w4.PATH_SKINNY, w4.PATH_MFMA])
def test_gemm_from_awq_orientation(path):
    # End to end: an AWQ-oriented checkpoint, repacked, multiplied; the
    # oracle multiplies the same codes re-packed into its own input layout.
    N, K, G, M = 256, 1024, 128, 16 if path == w4.PATH_SKINNY else 200
    L = wi.make_layout_weights(16, N, K, G, UINT4, "bf16", 1, 1, 1, 1)
    w, s, z = _layout_dev(L)
    packed = w4.repack_layout(w, 1, 1, s, 1, z, 1, G, UINT4)
    codes, scales, zeros = _layout_expect(L)
    A = wi.random_activations(16, M, K, "bf16")
    C = w4.gemm(A.to(DEV), packed, N, K, G, UINT4, path=path)
    ref, _ = oracle.gemm(A, oracle.pack_codes(codes), scales, oracle.pack_zeros(zeros), UINT4, G)
    assert oracle.rel_err(C.cpu(), ref) <= oracle.TOLERANCE["bf16"]


def test_repack_layout_binding_rejects_shapes():
    L = wi.make_layout_weights(17, 32, 256, 32, UINT4, "f16", 1, 1, 1, 1)  # Kg = 8, N/8 = 4
    w, s, z = _layout_dev(L)
    with pytest.raises(ValueError, match="weight_scale must be"):
        w4.repack_layout(w, 1, 1, s.t().contiguous(), 1, z, 1, 32, UINT4)
    with pytest.raises(ValueError, match="weight_zero_point must be"):
        w4.repack_layout(w, 1, 1, s, 1, z.t().contiguous(), 1, 32, UINT4)


# ------------------------------------------- K not a multiple of 128


KTAIL_REPACK = [
    # (N, K, G, qtype, zero points): the packed layout pads K to a multiple of 128
    (16, 40, -1, UINT4B8, False),
    (48, 96, 32, UINT4, True),
    (32, 2880, 64, UINT4, True),
    (64, 1216, 64, UINT4B8, False),
    (256, 200, -1, UINT4, True),
    (4096, 2880, 32, UINT4, True),
]


@pytest.mark.parametrize("N,K,G,qtype,zp", KTAIL_REPACK, ids=[f"{c[0]}x{c[1]}g{c[2]}q{c[3]}" for c in KTAIL_REPACK])
def test_repack_k_tail_bit_exact(N, K, G, qtype, zp):
    case = _case(41, 1, N, K, G, qtype, "bf16", with_zero_point=zp)
    packed = repack(case)
    codes, scales, zeros = expected_codes_scales_zeros(case)
    expect = oracle.encode_device(codes, scales, zeros, qtype, G)
    got = packed.cpu().numpy()
    assert got.shape == expect.shape
    mism = np.flatnonzero(got != expect)
    assert mism.size == 0, f"{mism.size} bytes differ, first at {mism[:8]}"
    c2, s2, z2 = w4.unpack(packed, N, K, G, qtype)
    np.testing.assert_array_equal(c2.cpu().numpy(), codes)
    np.testing.assert_array_equal(s2.cpu().numpy(), scales.view(torch.int16).numpy())
    if qtype == UINT4:
        np.testing.assert_array_equal(z2.cpu().numpy(), zeros)


@pytest.mark.parametrize("od,pd", [(1, 1), (1, 0), (0, 0)])
def test_repack_layout_k_tail_bit_exact(od, pd):
    N, K, G = 48, 160, 32
    L = wi.make_layout_weights(42, N, K, G, UINT4, "f16", od, pd, 1, 1)
    w, s_, z = _layout_dev(L)
    packed = w4.repack_layout(w, od, pd, s_, 1, z, 1, G, UINT4)
    codes, scales, zeros = _layout_expect(L)
    np.testing.assert_array_equal(packed.cpu().numpy(), oracle.encode_device(codes, scales, zeros, UINT4, G))


def _nan_padded(A: torch.Tensor, pad: int = 64) -> torch.Tensor:
    """A as a view with lda = K + pad whose padding columns hold NaN: any
    read of a column past K would reach C."""
    M, K = A.shape
    big = torch.full((M, K + pad), float("nan"), dtype=A.dtype, device=A.device)
    big[:, :K] = A
    return big[:, :K]


KTAIL_GEMM = [
    # (M, N, K, G, qtype, dtype, path): every kernel family with K % 128 != 0
    (1, 256, 2880, 64, UINT4, "bf16", SKINNY),  # few n-tiles: split-K skinny kernel
    (4, 4096, 1216, 64, UINT4B8, "f16", SKINNY),  # one n-tile per workgroup (resident)
    (1, 4096, 40, -1, UINT4, "f16", SKINNY),  # a single, mostly padded k-tile
    (8, 14336, 2880, -1, UINT4B8, "bf16", SKINNY),  # several n-tiles per workgroup (registers)
    (16, 4096, 14400, 64, UINT4, "f16", SKINNY),  # K > 4096: K chunks meet in the workspace
    (3, 1024, 2880, 32, UINT4, "bf16", SKINNY),
    (200, 2880, 2880, 64, UINT4, "f16", MFMA),  # staged kernel (G < 128)
    (64, 4096, 1216, -1, UINT4B8, "bf16", MFMA),
    (2048, 4096, 2880, -1, UINT4B8, "bf16", MFMA),  # ring kernel (one group per row)
    (2048, 4096, 2880, -1, UINT4, "f16", MFMA),
    (1990, 2880, 1216, 32, UINT4, "bf16", MFMA),
    (96, 256, 96, 32, UINT4, "f16", MFMA),
]


@pytest.mark.parametrize("M,N,K,G,qtype,dtype,path", KTAIL_GEMM,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}g{c[3]}q{c[4]}{c[5]}p{c[6]}" for c in KTAIL_GEMM])
def test_gemm_k_tail(M, N, K, G, qtype, dtype, path):
    case = _case(43, M, N, K, G, qtype, dtype, with_bias=True)
    wq, ws, zp, A, bias = to_dev(case)
    packed = w4.repack(wq, ws, zp, G, qtype)
    C = w4.gemm(_nan_padded(A), packed, N, K, G, qtype, bias=bias, path=path)
    torch.cuda.synchronize()
    assert not torch.isnan(C).any(), "a column past K reached C"
    rows = sample_rows(M)
    err = rel_err_rows(C, oracle_ref(case, rows=rows), rows)
    assert err <= oracle.TOLERANCE[dtype], f"rel err {err:.3e}"
    # The same with lda == K (nothing past K exists to read).
    C2 = w4.gemm(A, packed, N, K, G, qtype, bias=bias, path=path)
    assert torch.equal(C, C2)


@pytest.mark.parametrize("path", [SKINNY, MFMA])
def test_identity_k_tail(path):
    # A = I (M = K = 96): C = RN((q - z) * s) bit for bit, through the padded layout.
    N, K, G = 256, 96, 32
    for qtype, dtype in [(UINT4, "bf16"), (UINT4B8, "f16")]:
        case = _case(44, K, N, K, G, qtype, dtype)
        wq, ws, zp, _, _ = to_dev(case)
        packed = w4.repack(wq, ws, zp, G, qtype)
        eye = torch.eye(K, dtype=case.torch_dtype, device=DEV)
        if path == SKINNY:
            C = torch.cat([w4.gemm(eye[i:i + 16], packed, N, K, G, qtype, path=SKINNY) for i in range(0, K, 16)])
        else:
            C = w4.gemm(eye, packed, N, K, G, qtype, path=MFMA)
        W = oracle.dequant(case.weight_packed, case.weight_scale, case.weight_zero_point, qtype, G)
        assert torch.equal(C.cpu(), torch.from_numpy(W.T.copy()).to(case.torch_dtype))


def test_dense_variant_k_tail():
    N, K, G, M = 2880, 2880, 64, 512
    case = _case(45, M, N, K, G, UINT4, "bf16", with_bias=True)
    wq, ws, zp, A, bias = to_dev(case)
    packed = w4.repack(wq, ws, zp, G, UINT4)
    dense = w4.dequant(packed, N, K, G, UINT4, torch.bfloat16)
    W = oracle.dequant(case.weight_packed, case.weight_scale, case.weight_zero_point, UINT4, G)
    assert torch.equal(dense.cpu(), torch.from_numpy(W).to(torch.bfloat16))
    C = w4.gemm_dense(A, dense, bias=bias)
    rows = sample_rows(M)
    assert rel_err_rows(C, oracle_ref(case, rows=rows), rows) <= oracle.TOLERANCE["bf16"]


# ------------------------------------------- N not a multiple of 16


NTAIL_REPACK = [
    # (N, K, G, qtype, zero points): the packed layout pads N to a multiple of 16
    (24, 128, 128, UINT4B8, False),
    (8, 40, -1, UINT4, True),
    (1224, 2880, 64, UINT4, True),
    (4104, 4096, 128, UINT4B8, False),
]


@pytest.mark.parametrize("N,K,G,qtype,zp", NTAIL_REPACK, ids=[f"{c[0]}x{c[1]}g{c[2]}q{c[3]}" for c in NTAIL_REPACK])
def test_repack_n_tail_bit_exact(N, K, G, qtype, zp):
    case = _case(46, 1, N, K, G, qtype, "f16", with_zero_point=zp)
    packed = repack(case)
    codes, scales, zeros = expected_codes_scales_zeros(case)
    expect = oracle.encode_device(codes, scales, zeros, qtype, G)
    got = packed.cpu().numpy()
    assert got.shape == expect.shape
    mism = np.flatnonzero(got != expect)
    assert mism.size == 0, f"{mism.size} bytes differ, first at {mism[:8]}"
    c2, s2, z2 = w4.unpack(packed, N, K, G, qtype)
    np.testing.assert_array_equal(c2.cpu().numpy(), codes)
    np.testing.assert_array_equal(s2.cpu().numpy(), scales.view(torch.int16).numpy())
    if qtype == UINT4:
        np.testing.assert_array_equal(z2.cpu().numpy(), zeros)


def test_repack_layout_n_tail_bit_exact():
    N, K, G = 40, 160, 32  # AWQ words (K, N/8 = 5), AutoGPTQ zero points (K/G, 5)
    L = wi.make_layout_weights(47, N, K, G, UINT4, "bf16", 1, 1, 1, 1)
    w, s_, z = _layout_dev(L)
    packed = w4.repack_layout(w, 1, 1, s_, 1, z, 1, G, UINT4)
    codes, scales, zeros = _layout_expect(L)
    np.testing.assert_array_equal(packed.cpu().numpy(), oracle.encode_device(codes, scales, zeros, UINT4, G))


NTAIL_GEMM = [
    # (M, N, K, G, qtype, dtype, path): every kernel family with N % 16 != 0
    (1, 24, 512, 128, UINT4B8, "f16", SKINNY),  # split kernel, one n-tile
    (8, 4104, 4096, 128, UINT4, "bf16", SKINNY),  # wide N: still the split kernel (N tail)
    (4, 4104, 4096, -1, UINT4B8, "f16", SKINNY),
    (16, 1224, 2880, 64, UINT4, "bf16", SKINNY),  # N and K tails together
    (2048, 4104, 4096, -1, UINT4B8, "bf16", MFMA),  # ring kernel, one group per row
    (2048, 14344, 4096, 256, UINT4, "bf16", MFMA),  # ring kernel, groups of 256
    (200, 1224, 1216, 64, UINT4, "f16", MFMA),  # staged kernel with both tails
    (64, 4104, 4096, 32, UINT4B8, "f16", MFMA),  # staged kernel
]


@pytest.mark.parametrize("M,N,K,G,qtype,dtype,path", NTAIL_GEMM,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}g{c[3]}q{c[4]}{c[5]}p{c[6]}" for c in NTAIL_GEMM])
def test_gemm_n_tail(M, N, K, G, qtype, dtype, path):
    case = _case(48, M, N, K, G, qtype, dtype, with_bias=True)
    wq, ws, zp, A, bias = to_dev(case)
    packed = w4.repack(wq, ws, zp, G, qtype)
    # C as a view of a wider buffer whose extra columns hold a sentinel: no
    # store may land past column N.
    sentinel = 1234.0
    big = torch.full((M, N + 24), sentinel, dtype=case.torch_dtype, device=DEV)
    C = w4.gemm(_nan_padded(A) if K % 128 else A, packed, N, K, G, qtype, bias=bias, out=big[:, :N], path=path)
    torch.cuda.synchronize()
    assert torch.all(big[:, N:] == sentinel), "a store landed past column N"
    rows = sample_rows(M)
    err = rel_err_rows(C, oracle_ref(case, rows=rows), rows)
    assert err <= oracle.TOLERANCE[dtype], f"rel err {err:.3e}"


def test_identity_n_tail():
    N, K, G = 24, 128, 32
    for path in (SKINNY, MFMA):
        case = _case(49, K, N, K, G, UINT4, "bf16")
        wq, ws, zp, _, _ = to_dev(case)
        packed = w4.repack(wq, ws, zp, G, UINT4)
        eye = torch.eye(K, dtype=torch.bfloat16, device=DEV)
        if path == SKINNY:
            C = torch.cat([w4.gemm(eye[i:i + 16], packed, N, K, G, UINT4, path=SKINNY) for i in range(0, K, 16)])
        else:
            C = w4.gemm(eye, packed, N, K, G, UINT4, path=MFMA)
        W = oracle.dequant(case.weight_packed, case.weight_scale, case.weight_zero_point, UINT4, G)
        assert torch.equal(C.cpu(), torch.from_numpy(W.T.copy()).to(torch.bfloat16))


def test_dense_variant_n_tail():
    N, K, G, M = 1224, 2880, 64, 300
    case = _case(50, M, N, K, G, UINT4B8, "f16", with_bias=True)
    wq, ws, _, A, bias = to_dev(case)
    packed = w4.repack(wq, ws, None, G, UINT4B8)
    big = torch.full((N + 8, K), 7.0, dtype=torch.float16, device=DEV)
    dense = w4.dequant(packed, N, K, G, UINT4B8, torch.float16, out=big[:N])
    assert torch.all(big[N:] == 7.0)
    W = oracle.dequant(case.weight_packed, case.weight_scale, None, UINT4B8, G)
    assert torch.equal(dense.cpu(), torch.from_numpy(W).to(torch.float16))
    C = w4.gemm_dense(A, dense, bias=bias)
    rows = sample_rows(M)
    assert rel_err_rows(C, oracle_ref(case, rows=rows), rows) <= oracle.TOLERANCE["f16"]


# ------------------------------------------------------------------ dequant


IDENTITY = [
    # (N, K, G, qtype, dtype, path, one_rounding)
    (48, 128, 32, UINT4, "f16", SKINNY, True),
    (64, 256, 128, UINT4B8, "bf16", SKINNY, True),
    (32, 256, -1, UINT4, "bf16", SKINNY, True),
    (48, 128, 32, UINT4, "bf16", MFMA, True),
    (272, 256, 64, UINT4B8, "f16", MFMA, True),
    (64, 256, -1, UINT4, "f16", MFMA, True),
    # 128 x 256 ring tiles (at least one workgroup per CU): groups folded at
    # K-step ends, each group's scale applied to its own partial sum
    (32768, 256, 128, UINT4, "bf16", MFMA, True),
    (32768, 256, 256, UINT4B8, "f16", MFMA, True),
    (32768, 1024, -1, UINT4B8, "f16", MFMA, True),     # 128 x 512 tiles, one group per row
    # 128 x 512 tiles with groups: the accumulators are rescaled by
    # s_g / s_{g+1} at each group end, an fp32 rounding per group end, so a
    # product that lies exactly on a rounding tie of the act dtype may round
    # either way
    (32768, 512, 256, UINT4, "f16", MFMA, False),      # two K steps per group
]


@pytest.mark.parametrize("N,K,G,qtype,dtype,path,one_rounding", IDENTITY)
def test_identity_activations_give_rounded_weights(N, K, G, qtype, dtype, path, one_rounding):
    # A = I_K: C[m, n] = (q - z) * s rounded once to the act dtype, whether a
    # kernel scales before or after the products (the product is exact in
    # fp32), or, with rescaled accumulators, the rounding of a value within a
    # relative 1e-5 of it.
    case = _case(14, 1, N, K, G, qtype, dtype)
    packed = repack(case)
    A = torch.eye(K, dtype=case.torch_dtype, device=DEV)
    C = w4.gemm(A, packed, N, K, G, qtype, path=path)
    W = oracle.dequant(case.weight_packed, case.weight_scale, case.weight_zero_point, qtype, G)
    x = torch.from_numpy(W.T.copy())
    got = C.cpu().view(torch.int16)
    expect = x.to(case.torch_dtype).view(torch.int16)
    if one_rounding:
        bad = (got != expect).sum().item()
    else:
        near = [(x * (1.0 + d)).to(case.torch_dtype).view(torch.int16) for d in (1e-5, -1e-5)]
        bad = ((got != expect) & (got != near[0]) & (got != near[1])).sum().item()
    assert bad == 0, f"{bad} of {got.numel()} values differ from RN((q - z) * s)"


# ------------------------------------------------------------------ GEMM parity


def _workload_cases():
    out = []
    for name in ("tiny", "decode_sym", "decode_asym", "crossover"):
        wl = wi.WORKLOADS[name]
        for (M, N, K) in wl["shapes"]:
            paths = [AUTO] if name != "crossover" else [SKINNY, MFMA]
            for p in paths:
                out.append((name, wl["cfg_id"], M, N, K, wl["G"], wl["qtype"], wl["dtype"], wl["sigma"], p))
    wl = wi.WORKLOADS["prefill"]
    for (G, qt) in wl["variants"]:
        for (M, N, K) in wl["shapes"]:
            out.append(("prefill", wl["cfg_id"], M, N, K, G, qt, wl["dtype"], wl["sigma"], AUTO))
    return out


WORKLOAD_CASES = _workload_cases()


@pytest.mark.parametrize(
    "name,cfg,M,N,K,G,qtype,dtype,sigma,path", WORKLOAD_CASES,
    ids=[f"{c[0]}-M{c[2]}-N{c[3]}-K{c[4]}-G{c[5]}-q{c[6]}-p{c[9]}" for c in WORKLOAD_CASES],
)
def test_workload_parity(name, cfg, M, N, K, G, qtype, dtype, sigma, path):
    case = _case(cfg, M, N, K, G, qtype, dtype, sigma=sigma)
    print(f"[case] {name} M={M} N={N} K={K} G={G} qtype={qtype} {dtype} path={path}", flush=True)
    packed = repack(case)
    A = case.A.to(DEV)
    C = w4.gemm(A, packed, N, K, G, qtype, path=path)
    torch.cuda.synchronize()
    rows = sample_rows(M)
    ref = oracle_ref(case, rows=rows)
    err = rel_err_rows(C, ref, rows)
    tol = oracle.TOLERANCE[dtype]
    assert err <= tol, f"rel err {err:.3e} > {tol}"
    if path == AUTO:
        forced = SKINNY if M <= 16 else MFMA
        C2 = w4.gemm(A, packed, N, K, G, qtype, path=forced)
        assert torch.equal(C.view(torch.int16), C2.view(torch.int16)), "dispatcher picked another kernel"


# ------------------------------------------------------------------ edges


@pytest.mark.parametrize("path", [SKINNY, MFMA])
@pytest.mark.parametrize("qtype,dtype", [(UINT4B8, "f16"), (UINT4, "bf16")])
def test_bias_strides_and_ragged_tails(path, qtype, dtype):
    # N = 400 is not a multiple of any tile width; M ragged for both kernels.
    M = 11 if path == SKINNY else 300
    N, K, G = 400, 640, 64
    case = _case(15, M, N, K, G, qtype, dtype, with_bias=True)
    packed = repack(case)
    A_big = torch.zeros((M, K + 64), dtype=case.torch_dtype, device=DEV)
    A_big[:, :K] = case.A.to(DEV)
    A = A_big[:, :K]  # lda = K + 64
    C_big = torch.full((M, N + 48), 7.0, dtype=case.torch_dtype, device=DEV)
    C = C_big[:, :N]  # ldc = N + 48
    w4.gemm(A, packed, N, K, G, qtype, bias=case.bias.to(DEV), out=C, path=path)
    ref = oracle_ref(case)
    assert oracle.rel_err(C.cpu(), ref) <= oracle.TOLERANCE[dtype]
    assert torch.all(C_big[:, N:] == 7.0), "wrote outside [M, N]"


@pytest.mark.parametrize("path", [SKINNY, MFMA])
def test_zero_weights_give_bias_exactly(path):
    # All codes equal to the zero point: C = bias exactly (one rounding of bias).
    M, N, K, G = 24, 64, 256, 32
    rng = np.random.default_rng(16)
    z = rng.integers(0, 16, size=(N, K // G))
    words = oracle.pack_codes(np.repeat(z, G, axis=1))
    zp = oracle.pack_zeros(z)
    scales = torch.from_numpy(rng.uniform(0.005, 0.02, size=(N, K // G))).to(torch.float16)
    bias = torch.from_numpy(rng.normal(0, 1, size=(N,))).to(torch.float16)
    A = torch.from_numpy(rng.normal(0, 1, size=(M, K))).to(torch.float16)
    packed = w4.repack(torch.from_numpy(words).to(DEV), scales.to(DEV), torch.from_numpy(zp).to(DEV), G, UINT4)
    C = w4.gemm(A.to(DEV), packed, N, K, G, UINT4, bias=bias.to(DEV), path=path)
    assert torch.equal(C.cpu(), bias.expand(M, N))
    C0 = w4.gemm(A.to(DEV), packed, N, K, G, UINT4, path=path)
    assert torch.all(C0 == 0)


@pytest.mark.parametrize("path", [SKINNY, MFMA])
def test_every_small_m(path):
    N, K, G = 256, 1024, 128
    case = _case(17, 16, N, K, G, UINT4B8, "f16")
    packed = repack(case)
    ref = oracle_ref(case)
    A = case.A.to(DEV)
    for M in range(1, 17):
        C = w4.gemm(A[:M], packed, N, K, G, UINT4B8, path=path)
        err = oracle.rel_err(C.cpu(), ref[:M])
        assert err <= oracle.TOLERANCE["f16"], f"M={M}: {err}"


def test_forced_skinny_slices_large_m():
    N, K, G = 512, 512, 64
    case = _case(18, 40, N, K, G, UINT4, "bf16")
    packed = repack(case)
    C = w4.gemm(case.A.to(DEV), packed, N, K, G, UINT4, path=SKINNY)
    assert oracle.rel_err(C.cpu(), oracle_ref(case)) <= oracle.TOLERANCE["bf16"]


@pytest.mark.parametrize("path", [SKINNY, MFMA])
def test_group_minus_one_equals_group_k(path):
    N, K = 128, 512
    case = _case(19, 8 if path == SKINNY else 64, N, K, -1, UINT4, "f16")
    wq, ws, zp, A, _ = to_dev(case)
    p1 = w4.repack(wq, ws, zp, -1, UINT4)
    p2 = w4.repack(wq, ws, zp, K, UINT4)
    assert torch.equal(p1, p2)
    C1 = w4.gemm(A, p1, N, K, -1, UINT4, path=path)
    C2 = w4.gemm(A, p2, N, K, K, UINT4, path=path)
    assert torch.equal(C1, C2)
    assert oracle.rel_err(C1.cpu(), oracle_ref(case)) <= oracle.TOLERANCE["f16"]


@pytest.mark.parametrize("path", [SKINNY, MFMA])
def test_uint4_without_zero_points(path):
    N, K, G = 64, 256, 64
    case = _case(20, 4 if path == SKINNY else 40, N, K, G, UINT4, "bf16", with_zero_point=False)
    packed = repack(case)
    C = w4.gemm(case.A.to(DEV), packed, N, K, G, UINT4, path=path)
    assert oracle.rel_err(C.cpu(), oracle_ref(case)) <= oracle.TOLERANCE["bf16"]


def test_m_zero_is_a_noop():
    case = _case(21, 1, 64, 256, 64, UINT4B8, "f16")
    packed = repack(case)
    A = torch.empty((0, 256), dtype=torch.float16, device=DEV)
    C = w4.gemm(A, packed, 64, 256, 64, UINT4B8)
    assert C.shape == (0, 64)


@pytest.mark.parametrize(
    "M,N,K", [(16, 4096, 4096), (1, 14336, 4096), (7, 4096, 14336), (256, 4096, 14336), (1, 1024, 14336), (16, 512, 4096)]
)
def test_deterministic_and_workspace_returns_to_zero(M, N, K):
    # Split-K partials meet through the workspace; repeated calls must give
    # identical bits and leave every arrival counter at zero.
    case = _case(22, M, N, K, 128, UINT4B8, "f16")
    packed = repack(case)
    A = case.A.to(DEV)
    ws = w4.Workspace(DEV)
    C1 = w4.gemm(A, packed, N, K, 128, UINT4B8, workspace=ws)
    for _ in range(20):
        C2 = w4.gemm(A, packed, N, K, 128, UINT4B8, workspace=ws)
        assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    torch.cuda.synchronize()
    if ws.buf is not None:
        nctr = w4.workspace_counter_bytes()
        assert torch.all(ws.buf[:nctr] == 0)
    if M <= 16:
        rows = sample_rows(M)
        assert rel_err_rows(C1, oracle_ref(case, rows=rows), rows) <= oracle.TOLERANCE["f16"]


@pytest.mark.parametrize("K", [128, 384, 16384, 20480])
def test_skinny_k_extremes(K):
    # One tile (K = 128), a ragged last wave chunk (K = 384), the largest K
    # with one chunk per wave (16384) and beyond it, where waves loop (20480).
    N, G = 64, 128
    case = _case(23, 5, N, K, G, UINT4, "bf16")
    packed = repack(case)
    C = w4.gemm(case.A.to(DEV), packed, N, K, G, UINT4, path=SKINNY)
    assert oracle.rel_err(C.cpu(), oracle_ref(case)) <= oracle.TOLERANCE["bf16"]


# 128 x 256 tiles (at least 256 workgroups): the three-stage ring for one
# group per row or groups of 128 k or more (a last round at most half full
# runs as 64-row halves), the staged kernel with scale-first dequantisation
# for groups of 32 or 64 k. Each case names the edge it reaches.
RING = [
    # (M, N, K, G, qtype, dtype, bias)
    (2048, 4096, 128, -1, UINT4B8, "bf16", False),  # one K step: only the loop tail runs
    (2000, 4112, 1024, 256, UINT4, "f16", True),    # ragged M and N (257 n-tiles), 8 steps: tail of 2
    (4096, 4096, 512, 128, UINT4B8, "f16", False),  # a group per step, tail of 1
    (2048, 8192, 1536, 256, UINT4, "bf16", True),   # 2 steps per group, 12 steps: no tail
    (1930, 8192, 896, -1, UINT4, "f16", False),     # 7 steps: tail of 1, ragged M
    (2048, 14336, 512, 256, UINT4B8, "bf16", True), # 896 tiles: the last 128 as 64-row halves
    (1390, 14336, 256, -1, UINT4B8, "f16", False),  # halves over m-tiles 9-10, ragged M
    (1930, 14336, 256, 128, UINT4B8, "f16", True),  # a half tile lies wholly past M
    (2048, 4096, 1024, 64, UINT4, "bf16", True),    # G = 64: staged tiles, scale first
    (1000, 8192, 512, 32, UINT4B8, "f16", False),   # G = 32: staged tiles, scale first, ragged M
    # Two tail steps after the loop (steps % 3 == 2) in the grouped mode:
    # the tail requests no loads and waits for every one (the last step's
    # successor scale is zero).
    (2048, 4096, 640, 128, UINT4, "f16", True),     # 5 steps, a group per step, zero points
    (2048, 4096, 1024, 256, UINT4B8, "bf16", False),# 8 steps, two steps per group
    (2048, 4096, 4096, 256, UINT4, "f16", True),    # 32 steps, the K of the 14336 x 4096 prefill weight
    # 128 x 512 tiles (one group per row, whole rounds of 256 tiles, at
    # least 1024 tiles, or a last round at least three quarters full): two
    # LDS stages, tiles ordered per XCD.
    (4096, 4096, 1024, -1, UINT4B8, "bf16", False), # 256 tiles, 8 steps
    (4096, 4000, 896, -1, UINT4, "f16", True),      # ragged N (250 n-tiles), 7 steps: odd tail step
    (4000, 4096, 1000, -1, UINT4B8, "f16", False),  # ragged M, K tail
    (8192, 4096, 256, -1, UINT4, "bf16", True),     # 512 tiles: two rounds
    (8192, 14336, 128, -1, UINT4B8, "bf16", False), # 1792 tiles, a single K step
    (4470, 15872, 128, -1, UINT4B8, "f16", True),   # 1085 tiles: not a multiple of 8 (no XCD grouping)
    (1990, 14336, 256, -1, UINT4B8, "f16", False),  # 448 tiles: a last round three quarters full, ragged M
    # 128 x 512 tiles with groups of 128 k or more (accumulators rescaled at
    # each group end); with zero points also for a last round at least three
    # quarters full.
    (4096, 4096, 1024, 256, UINT4, "bf16", True),   # 4 groups of 2 steps, zero points
    (8192, 14336, 512, 128, UINT4, "f16", False),   # 1792 tiles, a group per step
    (4000, 4008, 768, 256, UINT4B8, "bf16", True),  # ragged M and N, 3 groups
    (4096, 4096, 384, 128, UINT4B8, "f16", False),  # 3 steps: odd tail step ends the last group
    (2048, 14336, 512, 256, UINT4, "bf16", True),   # zero points: 448 tiles, a last round three quarters full
    (1930, 14336, 256, 128, UINT4, "f16", True),    # the same with ragged M
]


@pytest.mark.parametrize("M,N,K,G,qtype,dtype,bias", RING,
                         ids=[f"M{c[0]}-N{c[1]}-K{c[2]}-G{c[3]}-q{c[4]}-{c[5]}" for c in RING])
def test_ring_tiles(M, N, K, G, qtype, dtype, bias):
    print(f"[case] ring M={M} N={N} K={K} G={G} qtype={qtype} {dtype} bias={bias}", flush=True)
    case = _case(25, M, N, K, G, qtype, dtype, with_bias=bias)
    packed = repack(case)
    _, _, _, A, b = to_dev(case)
    C = w4.gemm(A, packed, N, K, G, qtype, bias=b, path=MFMA)
    torch.cuda.synchronize()
    rows = sample_rows(M)
    err = rel_err_rows(C, oracle_ref(case, rows=rows), rows)
    assert err <= oracle.TOLERANCE[dtype], f"rel err {err:.3e}"


# The 128 x 256 tiles store four adjacent outputs of a row with one 8-byte
# store when C's row stride keeps them aligned, the 128 x 512 tiles whole
# 16-byte row chunks staged through LDS when the stride is a multiple of 8;
# an odd stride takes the element-wise stores. Sentinels past column N must
# survive.
ODD_LDC = [
    # (M, N, K, G, qtype, dtype): kernel reached
    (2048, 4096, 256, -1, UINT4B8, "bf16"),  # ring, one group per row
    (2048, 4096, 512, 256, UINT4, "f16"),    # ring, groups of 256
    (4096, 4096, 256, -1, UINT4, "f16"),     # 128 x 512 tiles
    (4096, 4008, 256, -1, UINT4B8, "bf16"),  # 128 x 512 tiles, N not a multiple of 16
    (4096, 4096, 512, 256, UINT4, "f16"),    # 128 x 512 tiles, groups of 256
]


@pytest.mark.parametrize("M,N,K,G,qtype,dtype", ODD_LDC,
                         ids=[f"M{c[0]}-N{c[1]}-K{c[2]}-G{c[3]}-q{c[4]}-{c[5]}" for c in ODD_LDC])
@pytest.mark.parametrize("pad", [3, 4])
def test_tiled_output_strides(M, N, K, G, qtype, dtype, pad):
    print(f"[case] tiled stride M={M} N={N} K={K} G={G} qtype={qtype} {dtype} pad={pad}", flush=True)
    case = _case(29, M, N, K, G, qtype, dtype, with_bias=True)
    packed = repack(case)
    _, _, _, A, b = to_dev(case)
    big = torch.full((M, N + pad), 1234.0, dtype=case.torch_dtype, device=DEV)
    C = w4.gemm(A, packed, N, K, G, qtype, bias=b, out=big[:, :N], path=MFMA)
    torch.cuda.synchronize()
    assert torch.all(big[:, N:] == 1234.0), "a store landed past column N"
    rows = sample_rows(M)
    err = rel_err_rows(C, oracle_ref(case, rows=rows), rows)
    assert err <= oracle.TOLERANCE[dtype], f"rel err {err:.3e}"
    C2 = w4.gemm(A, packed, N, K, G, qtype, bias=b, path=MFMA)
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16)), "strided and contiguous outputs differ"


# Groups on the 128 x 512 tiles: the accumulators are carried in units of
# the current group's scale and rescaled at each group end, and a group whose
# scale is zero is masked out of the products. Scales spanning three decades
# (ratios up to 1000 between neighbouring groups) and zero scales (a single
# group of some columns, a whole column, the first and the last group) must
# still match the oracle.
@pytest.mark.parametrize("qtype,dtype,G", [(UINT4, "bf16", 256), (UINT4B8, "f16", 128)])
@pytest.mark.parametrize("pattern", ["decades", "zeros"])
def test_grouped_wide_scales(qtype, dtype, G, pattern):
    M, N, K = 4096, 4096, 2048
    print(f"[case] grouped wide scales {pattern} qtype={qtype} {dtype} G={G}", flush=True)
    case = _case(31, M, N, K, G, qtype, dtype, with_bias=True)
    sc = case.weight_scale.clone().float()
    Kg = sc.shape[1]
    if pattern == "decades":
        rng = np.random.default_rng(7)
        sc = sc * torch.from_numpy(10.0 ** -rng.uniform(0, 3, size=sc.shape)).float()
    else:
        sc[::7, 1] = 0.0           # one group of every 7th column
        sc[5, :] = 0.0             # a whole column
        sc[100:116, 0] = 0.0       # the first group of an n-tile
        sc[2000:2048, Kg - 1] = 0.0  # the last group of three n-tiles
    case.weight_scale = sc.to(case.weight_scale.dtype)
    packed = repack(case)
    _, _, _, A, b = to_dev(case)
    C = w4.gemm(A, packed, N, K, G, qtype, bias=b, path=MFMA)
    torch.cuda.synchronize()
    rows = sample_rows(M)
    ref = oracle_ref(case, rows=rows)
    err = rel_err_rows(C, ref, rows)
    assert err <= oracle.TOLERANCE[dtype], f"rel err {err:.3e}"
    if pattern == "zeros":
        # A column whose scales are all zero is the bias alone (one rounding).
        got = C[torch.from_numpy(rows).to(DEV), 5].cpu().float()
        assert torch.equal(got, b[5].cpu().float().expand_as(got))


# Medium M (17 up to a few hundred rows, fewer 128 x 256 tiles than CUs):
# BM x 256 tiles (BM = 32, 64 or 128) with K split over workgroups, partial
# tiles through the workspace and summed in split order by a second kernel;
# scale-first dequantisation for every group size. Each case names what it
# reaches.
MEDIUM = [
    # (M, N, K, G, qtype, dtype)
    (32, 14336, 4096, 64, UINT4B8, "f16"),   # the crossover shapes: 32-row tiles, 4 splits (6 stages)
    (64, 14336, 4096, 64, UINT4B8, "f16"),   # 64-row tiles (4 stages)
    (128, 14336, 4096, 64, UINT4B8, "f16"),  # 128-row tiles (3 stages)
    (256, 14336, 4096, 64, UINT4B8, "f16"),  # two m-tiles, 2 splits
    (17, 4096, 4096, 32, UINT4, "bf16"),     # the first M past the skinny path, 4 groups per K step (5 stages)
    (48, 4096, 14336, 64, UINT4, "f16"),     # long K: 8 splits of 14 steps
    (100, 4104, 2048, 128, UINT4, "f16"),    # ragged M and N
    (129, 4096, 4096, 32, UINT4, "bf16"),    # a second m-tile of one row
    (200, 4104, 2048, 128, UINT4, "f16"),    # ragged M and N
    (200, 8192, 4096, -1, UINT4B8, "bf16"),  # one group per row, ragged second m-tile
    (160, 4096, 14336, 64, UINT4, "f16"),    # long K: 8 splits of 14 steps
    (256, 1024, 8192, 256, UINT4B8, "bf16"), # 8 tiles, 16 splits
    (192, 14336, 1664, 64, UINT4B8, "f16"),  # 13 steps in splits of 7 and 6 (odd tails)
    (384, 14336, 1024, 64, UINT4, "bf16"),   # 168 tiles: no split
    (512, 14336, 640, 32, UINT4B8, "f16"),   # 224 tiles, 5 steps (a ring of 3 stages: a tail of 2)
]


@pytest.mark.parametrize("M,N,K,G,qtype,dtype", MEDIUM,
                         ids=[f"M{c[0]}-N{c[1]}-K{c[2]}-G{c[3]}-q{c[4]}-{c[5]}" for c in MEDIUM])
def test_medium_m_split_k_tiles(M, N, K, G, qtype, dtype):
    print(f"[case] medium M={M} N={N} K={K} G={G} qtype={qtype} {dtype}", flush=True)
    case = _case(33, M, N, K, G, qtype, dtype, with_bias=True)
    packed = repack(case)
    _, _, _, A, b = to_dev(case)
    C = w4.gemm(A, packed, N, K, G, qtype, bias=b, path=MFMA)
    torch.cuda.synchronize()
    rows = sample_rows(M)
    err = rel_err_rows(C, oracle_ref(case, rows=rows), rows)
    assert err <= oracle.TOLERANCE[dtype], f"rel err {err:.3e}"
    # A second call on the same workspace (its counters were left at zero)
    # gives the same bits.
    C2 = w4.gemm(A, packed, N, K, G, qtype, bias=b, path=MFMA)
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16))


# Long sums of non-zero-mean activations. The offset-corrected kernels feed
# the MFMA exact operand values with a constant offset (b = c0 + c1*q) and
# take the offset back out with row sums S = sum A; with A ~ N(mu, 1) the
# partial sums grow like mu*K, which is the one input property that fp32
# rounding of those sums is sensitive to. Codes "centred" on the zero
# (q = clip(round(N(z, 2.5)))) make C itself small, the hardest case for the
# relative error. K = 14336 is the deepest decode/prefill shape.
SHIFTED = [
    # (M, N, K, G, qtype, dtype, mean, codes, path): the kernel each reaches
    (2048, 4096, 14336, -1, UINT4B8, "f16", 1.0, "uniform", MFMA),   # ring, one group per row
    (2048, 4096, 14336, -1, UINT4B8, "f16", 3.0, "centred", MFMA),
    (2048, 4096, 14336, 256, UINT4B8, "f16", 1.0, "uniform", MFMA),  # ring, folded groups
    (2048, 4096, 14336, 256, UINT4B8, "f16", 3.0, "centred", MFMA),
    (2048, 4096, 14336, 256, UINT4, "f16", 3.0, "centred", MFMA),    # ring, zero points, codes around each zero
    (2048, 4096, 14272, -1, UINT4B8, "f16", 3.0, "centred", MFMA),   # ring with a K tail
    (4096, 4096, 14336, -1, UINT4B8, "f16", 3.0, "centred", MFMA),   # 128 x 512 tiles
    (4096, 4096, 14336, -1, UINT4, "bf16", 3.0, "centred", MFMA),
    (4096, 4096, 14336, 256, UINT4B8, "f16", 3.0, "centred", MFMA),  # 128 x 512 tiles, rescaled groups
    (4096, 4096, 14336, 128, UINT4, "bf16", 3.0, "centred", MFMA),
    (64, 4096, 14336, -1, UINT4B8, "f16", 1.0, "uniform", MFMA),     # staged tiles, one group per row
    (64, 4096, 14336, -1, UINT4B8, "f16", 3.0, "centred", MFMA),
    (64, 4096, 14272, -1, UINT4, "f16", 3.0, "centred", MFMA),       # staged tiles with a K tail
    (128, 14336, 4096, 64, UINT4B8, "f16", 3.0, "centred", MFMA),    # staged tiles, scale first (G = 64)
    (2048, 4096, 14336, -1, UINT4, "bf16", 3.0, "centred", MFMA),
    (2048, 4096, 14336, 256, UINT4B8, "bf16", 3.0, "centred", MFMA),
    (16, 4096, 14336, -1, UINT4B8, "f16", 3.0, "centred", SKINNY),   # skinny fold blocks, K split in chunks
    (16, 14336, 4096, 128, UINT4, "f16", 3.0, "centred", SKINNY),
    (8, 1024, 14336, 256, UINT4B8, "f16", 3.0, "centred", SKINNY),   # split-K kernel
    (4, 4096, 14336, 128, UINT4B8, "f16", 3.0, "centred", SKINNY),   # long K in one workgroup, S over 4 k-tiles
    (1, 4096, 16384, -1, UINT4, "f16", 3.0, "centred", SKINNY),
    (8, 4096, 4096, 128, UINT4B8, "f16", 3.0, "centred", SKINNY),    # S over 2 k-tiles
]


def _centred_case(cfg, M, N, K, G, qtype, dtype, mean):
    """A case whose codes are drawn around their zero (8, or each group's
    zero point), packed by the oracle's packer."""
    case = _case(cfg, M, N, K, G, qtype, dtype, mean=mean)
    Ge = wi.effective_group(K, G)
    if qtype == UINT4:
        z = oracle.unpack_zeros(case.weight_zero_point, N).astype(np.float64)
        centre = np.repeat(z, Ge, axis=1)
    else:
        centre = np.full((N, K), 8.0)
    codes = wi.centred_codes(cfg * 7919 + K, centre)
    case.weight_packed = oracle.pack_codes(codes)
    return case


@pytest.mark.parametrize("M,N,K,G,qtype,dtype,mean,codes,path", SHIFTED,
                         ids=[f"M{c[0]}-N{c[1]}-K{c[2]}-G{c[3]}-q{c[4]}-{c[5]}-mu{c[6]:g}-{c[7]}" for c in SHIFTED])
def test_shifted_activations_long_k(M, N, K, G, qtype, dtype, mean, codes, path):
    print(f"[case] shifted M={M} N={N} K={K} G={G} qtype={qtype} {dtype} mean={mean} {codes} path={path}",
          flush=True)
    case = (_centred_case(27, M, N, K, G, qtype, dtype, mean) if codes == "centred"
            else _case(27, M, N, K, G, qtype, dtype, mean=mean))
    packed = repack(case)
    C = w4.gemm(case.A.to(DEV), packed, N, K, G, qtype, path=path)
    torch.cuda.synchronize()
    rows = sample_rows(M)
    err = rel_err_rows(C, oracle_ref(case, rows=rows), rows)
    print(f"[result] rel err {err:.3e}", flush=True)
    assert err <= oracle.TOLERANCE[dtype], f"rel err {err:.3e} > {oracle.TOLERANCE[dtype]}"


# Full-K skinny kernels (N >= 3072): activations in registers or staged in
# LDS, all weight tiles of a wave in registers, or a streamed ring. Each case
# names the variant and edge it reaches.
FULL_K = [
    # (N, K, M, G, qtype, dtype, bias)
    (4096, 128, 16, 128, UINT4B8, "f16", True),   # one k-tile, one wave, LDS activations
    (4096, 384, 3, 64, UINT4, "bf16", False),     # two waves (2 and 1 k-tiles), LDS activations (up to 8 rows)
    (4096, 640, 9, 32, UINT4, "f16", True),       # three waves (2, 2 and 1 k-tiles), a scale per word
    (4112, 1024, 5, 128, UINT4B8, "bf16", False), # 257 n-tiles: 2 per workgroup, the last has 1
    (14416, 512, 2, 64, UINT4, "f16", True),      # 901 n-tiles: 4 per workgroup, ragged last ones
    (14336, 4096, 2, 64, UINT4, "f16", False),    # 4 n-tiles per workgroup with zeros, 2 fold blocks
    (4096, 4224, 16, 128, UINT4B8, "f16", False), # 33 k-tiles: K split in chunks of 20 and 13
    (3072, 14336, 3, 128, UINT4, "bf16", True),   # K split in 4 chunks, 3 n-tiles per workgroup
    (4096, 16384, 12, -1, UINT4B8, "f16", False), # K split in 4 chunks, one group per row
    (14336, 4096, 7, 32, UINT4, "bf16", True),    # streamed: 4 n-tiles per workgroup, a scale per word
    (6144, 4096, 16, 32, UINT4, "bf16", True),    # 2 n-tiles per workgroup, a scale per word
    # One n-tile per workgroup, one fold block per k-tile: up to 8 rows share
    # each S MFMA over a wave's 2 k-tiles; waves take every nwaves-th k-tile.
    (4096, 640, 3, 128, UINT4, "f16", True),      # 5 k-tiles over 3 waves (2, 2 and 1): a partial pair
    (4096, 128, 2, -1, UINT4B8, "bf16", False),   # one k-tile: the S operand repeats it for the pair
    (4096, 1280, 7, 256, UINT4, "bf16", True),    # 10 k-tiles over 5 waves, up to 8 rows
    (4096, 4096, 6, 128, UINT4B8, "f16", False),
    (4096, 4096, 1, 128, UINT4, "bf16", True),
    (4096, 4096, 4, -1, UINT4, "f16", False),
    # Long K, one n-tile per workgroup, up to 4 rows: all of K in one
    # workgroup, 8 k-tiles per wave (up to 16 waves), S over 4 k-tiles,
    # activation rows in LDS.
    (4096, 14336, 1, 128, UINT4B8, "f16", False),
    (4096, 14336, 4, 128, UINT4, "bf16", True),
    (3072, 13952, 3, 128, UINT4B8, "f16", True),  # 109 k-tiles: 14 waves of 8 or 7
    (4096, 16384, 2, -1, UINT4, "f16", False),    # one group per row, 16 waves of 8
    (4096, 4224, 4, 128, UINT4, "f16", True),     # 33 k-tiles: 5 waves of 7 or 6
    (3200, 8192, 1, -1, UINT4B8, "bf16", True),   # 64 k-tiles: 8 waves of 8
    (4096, 8320, 3, 128, UINT4, "bf16", False),   # 65 k-tiles: 9 waves of 8 or 7
    # Long K with K split over workgroups (partials through the workspace).
    (4096, 14336, 2, 64, UINT4, "f16", True),     # two fold blocks per 128 k
    (4096, 14336, 5, 128, UINT4B8, "bf16", False),  # 5 rows
    (4096, 16512, 1, 128, UINT4B8, "f16", False),  # 129 k-tiles: the streamed variant
]


@pytest.mark.parametrize("N,K,M,G,qtype,dtype,bias", FULL_K,
                         ids=[f"N{c[0]}-K{c[1]}-M{c[2]}-G{c[3]}-q{c[4]}-{c[5]}" for c in FULL_K])
def test_full_k_variants(N, K, M, G, qtype, dtype, bias):
    print(f"[case] full-K N={N} K={K} M={M} G={G} qtype={qtype} {dtype} bias={bias}", flush=True)
    case = _case(24, M, N, K, G, qtype, dtype, with_bias=bias)
    packed = repack(case)
    _, _, _, A, b = to_dev(case)
    C = w4.gemm(A, packed, N, K, G, qtype, bias=b, path=SKINNY)
    assert oracle.rel_err(C.cpu(), oracle_ref(case)) <= oracle.TOLERANCE[dtype]


@pytest.mark.parametrize("N,dtype,qtype,G", [(4096, "f16", UINT4B8, 128), (4096, "bf16", UINT4, 32),
                                             (14336, "f16", UINT4, 64)])
def test_identity_through_full_k(N, dtype, qtype, G):
    # A = I_128 over 16-row slices of the full-K skinny kernels (one n-tile per
    # workgroup with LDS activations; four with register activations):
    # bit-exact RN_act((q - z) * s), as in the identity test above.
    K = 128
    print(f"[case] identity full-K N={N} {dtype} G={G}", flush=True)
    case = _case(25, 1, N, K, G, qtype, dtype)
    packed = repack(case)
    A = torch.eye(K, dtype=case.torch_dtype, device=DEV)
    C = w4.gemm(A, packed, N, K, G, qtype, path=SKINNY)
    W = oracle.dequant(case.weight_packed, case.weight_scale, case.weight_zero_point, qtype, G)
    expect = torch.from_numpy(W.T.copy()).to(case.torch_dtype)
    bad = (C.cpu().view(torch.int16) != expect.view(torch.int16)).sum().item()
    assert bad == 0, f"{bad} of {C.numel()} values differ from RN((q - z) * s)"


@pytest.mark.parametrize("rows,dtype,qtype,G", [(4, "f16", UINT4B8, 128), (1, "bf16", UINT4, -1),
                                                 (8, "bf16", UINT4B8, 256), (3, "f16", UINT4, 128)])
def test_identity_small_m_slices(rows, dtype, qtype, G):
    # A = I_512 in slices of `rows` rows through the one-n-tile skinny kernel,
    # where up to 4 (8) rows share each S MFMA over 4 (2) k-tiles and lane
    # groups fold different k-tiles: still bit-exact RN_act((q - z) * s).
    N, K = 4096, 512
    print(f"[case] identity small-M slices rows={rows} {dtype} qtype={qtype} G={G}", flush=True)
    case = _case(26, 1, N, K, G, qtype, dtype)
    packed = repack(case)
    eye = torch.eye(K, dtype=case.torch_dtype, device=DEV)
    C = torch.cat([w4.gemm(eye[i:i + rows], packed, N, K, G, qtype, path=SKINNY) for i in range(0, K, rows)])
    W = oracle.dequant(case.weight_packed, case.weight_scale, case.weight_zero_point, qtype, G)
    expect = torch.from_numpy(W.T.copy()).to(case.torch_dtype)
    bad = (C.cpu().view(torch.int16) != expect.view(torch.int16)).sum().item()
    assert bad == 0, f"{bad} of {C.numel()} values differ from RN((q - z) * s)"


# ------------------------------------------------------------------ dense prefill variant
# (dequantise once into a dense weight, then a library GEMM on it)


DEQUANT = [
    # (N, K, G, qtype, dtype, pad): pad = extra columns of the dense rows (ldw = K + pad)
    (16, 128, 128, UINT4B8, "f16", 0),
    (48, 256, 32, UINT4, "bf16", 8),
    (272, 512, 64, UINT4B8, "bf16", 0),
    (4096, 1024, -1, UINT4, "f16", 64),
    (14336, 4096, 256, UINT4B8, "bf16", 0),
    (6144, 4096, 32, UINT4, "bf16", 0),
]


@pytest.mark.parametrize("N,K,G,qtype,dtype,pad", DEQUANT,
                         ids=[f"{c[0]}x{c[1]}g{c[2]}q{c[3]}-{c[4]}-pad{c[5]}" for c in DEQUANT])
def test_dequant_bit_exact(N, K, G, qtype, dtype, pad):
    # Every dense value must be RN_act((q - z) * s) bit for bit (q - z is a
    # small integer, so the product is exact before its one rounding).
    print(f"[case] dequant N={N} K={K} G={G} qtype={qtype} {dtype} pad={pad}", flush=True)
    case = _case(26, 1, N, K, G, qtype, dtype)
    packed = repack(case)
    big = torch.full((N, K + pad), 3.0, dtype=case.torch_dtype, device=DEV)
    w4.dequant(packed, N, K, G, qtype, case.torch_dtype, out=big[:, :K])
    W = oracle.dequant(case.weight_packed, case.weight_scale, case.weight_zero_point, qtype, G)
    expect = torch.from_numpy(W).to(case.torch_dtype)
    got = big[:, :K].cpu()
    bad = (got.view(torch.int16) != expect.view(torch.int16)).sum().item()
    assert bad == 0, f"{bad} of {got.numel()} values differ from RN((q - z) * s)"
    if pad:
        assert torch.all(big[:, K:] == 3.0), "wrote outside [N, K]"


DENSE_GEMM = [
    # (M, N, K, G, qtype, dtype, bias)
    (300, 400, 640, 64, UINT4, "f16", True),
    (2048, 14336, 4096, 256, UINT4B8, "bf16", False),
    (2048, 4096, 14336, -1, UINT4, "bf16", True),
]


@pytest.mark.parametrize("M,N,K,G,qtype,dtype,bias", DENSE_GEMM,
                         ids=[f"M{c[0]}-N{c[1]}-K{c[2]}-G{c[3]}-q{c[4]}-{c[5]}" for c in DENSE_GEMM])
def test_dense_prefill_parity(M, N, K, G, qtype, dtype, bias):
    print(f"[case] dense M={M} N={N} K={K} G={G} qtype={qtype} {dtype} bias={bias}", flush=True)
    case = _case(27, M, N, K, G, qtype, dtype, with_bias=bias)
    packed = repack(case)
    _, _, _, A, b = to_dev(case)
    Wd = w4.dequant(packed, N, K, G, qtype, case.torch_dtype)
    C = w4.gemm_dense(A, Wd, bias=b)
    torch.cuda.synchronize()
    rows = sample_rows(M)
    err = rel_err_rows(C, oracle_ref(case, rows=rows), rows)
    assert err <= oracle.TOLERANCE[dtype], f"rel err {err:.3e}"


def test_dense_gemm_strides():
    # A, W and C with row strides beyond their widths; C's padding untouched.
    M, N, K, G = 64, 256, 512, 128
    case = _case(28, M, N, K, G, UINT4B8, "bf16", with_bias=True)
    packed = repack(case)
    _, _, _, A, b = to_dev(case)
    A_big = torch.zeros((M, K + 32), dtype=torch.bfloat16, device=DEV)
    A_big[:, :K] = A
    W_big = torch.zeros((N, K + 16), dtype=torch.bfloat16, device=DEV)
    w4.dequant(packed, N, K, G, UINT4B8, torch.bfloat16, out=W_big[:, :K])
    C_big = torch.full((M, N + 24), 7.0, dtype=torch.bfloat16, device=DEV)
    w4.gemm_dense(A_big[:, :K], W_big[:, :K], bias=b, out=C_big[:, :N])
    assert oracle.rel_err(C_big[:, :N].cpu(), oracle_ref(case)) <= oracle.TOLERANCE["bf16"]
    assert torch.all(C_big[:, N:] == 7.0), "wrote outside [M, N]"


# ------------------------------------------------------------------ operands beyond 2 GiB
# The kernels address buffers with 32-bit offsets from per-launch or
# per-workgroup bases. These cases put A, or the packed weight, past 2^31
# bytes. Inputs are drawn on the GPU (seeded); the oracle checks sampled rows
# and column blocks at both ends of the weight.


def test_activations_beyond_2gib():
    M, N, K, G = 65600, 256, 16384, 128  # A is 2.15 GB; 513 tiles, the last as halves
    print(f"[case] A beyond 2 GiB M={M} N={N} K={K}", flush=True)
    case = _case(29, 1, N, K, G, UINT4B8, "bf16")  # the weight (its 1-row A is unused)
    packed = repack(case)
    gen = torch.Generator(device=DEV).manual_seed(29)
    A = torch.randn((M, K), device=DEV, generator=gen).to(torch.bfloat16)
    assert A.numel() * 2 > 2**31
    C = w4.gemm(A, packed, N, K, G, UINT4B8, path=MFMA)
    torch.cuda.synchronize()
    rows = torch.as_tensor(sample_rows(M), device=DEV)
    ref, _ = oracle.gemm(A[rows].cpu(), case.weight_packed, case.weight_scale, None, UINT4B8, G)
    assert oracle.rel_err(C[rows].cpu(), ref) <= oracle.TOLERANCE["bf16"]


@pytest.mark.parametrize("M,path", [(256, MFMA), (16, SKINNY)])
def test_weights_beyond_2gib(M, path):
    N, K, G = 65552, 65536, 128  # 2.15 GB of codes; 4097 n-tiles
    print(f"[case] weight beyond 2 GiB M={M} N={N} K={K} path={path}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(30)
    wq = torch.randint(-2**31, 2**31, (N, K // 8), dtype=torch.int32, device=DEV, generator=gen)
    ws = torch.empty((N, K // G), dtype=torch.bfloat16, device=DEV).uniform_(0.005, 0.02, generator=gen)
    packed = w4.repack(wq, ws, None, G, UINT4B8)
    assert N * K // 2 > 2**31
    A = torch.randn((M, K), device=DEV, generator=gen).to(torch.bfloat16)
    C = w4.gemm(A, packed, N, K, G, UINT4B8, path=path, workspace=w4.Workspace(DEV))
    torch.cuda.synchronize()
    rows = torch.as_tensor(sample_rows(M))
    A_rows = A.cpu()[rows]
    for n0 in (0, N - 48):  # the last n-tiles sit past 2 GiB in the packed buffer
        ref, _ = oracle.gemm(A_rows, wq[n0:n0 + 48].cpu().numpy(), ws[n0:n0 + 48].cpu(), None, UINT4B8, G)
        err = oracle.rel_err(C[:, n0:n0 + 48].cpu()[rows], ref)
        assert err <= oracle.TOLERANCE["bf16"], f"columns {n0}..: rel err {err:.3e}"


# ------------------------------------------------------------------ W4A8


A8_QUANT = [(1, 4096, "f16", 0), (16, 14336, "bf16", 0), (37, 2880, "bf16", 64), (300, 1216, "f16", 8),
            (3, 20480, "bf16", 16)]  # the last: more than 8 chunks per thread, two reads of the row


@pytest.mark.parametrize("M,K,dtype,pad", A8_QUANT, ids=[f"{c[0]}x{c[1]}{c[2]}p{c[3]}" for c in A8_QUANT])
def test_quantize_a8_bit_exact(M, K, dtype, pad):
    A = wi.random_activations(51, M, K, dtype, sigma=2.0)
    A[min(3, M - 1)] = 0  # a row of zeros: scale 0, codes 0
    if M > 5:
        A[5, 7] = 1000.0  # one large value sets the row's scale
    big = torch.zeros((M, K + pad), dtype=A.dtype, device=DEV)
    big[:, :K] = A.to(DEV)
    qa, xs = w4.quantize_a8(big[:, :K])
    q_ref, xs_ref = oracle.quant_rows_a8(A)
    np.testing.assert_array_equal(xs.cpu().numpy(), xs_ref)
    np.testing.assert_array_equal(qa.cpu().numpy(), pair_order_codes(q_ref))


W4A8_GEMM = [
    # (M, N, K, G, dtype)
    (1, 4096, 4096, 128, "f16"),
    (8, 14336, 4096, -1, "bf16"),
    (16, 4096, 14336, 32, "f16"),
    (3, 1224, 2880, 64, "bf16"),  # N and K tails
    (100, 4096, 4096, 256, "bf16"),
    (2048, 4096, 4096, 128, "f16"),
    (2048, 14336, 4096, -1, "bf16"),
    (600, 2880, 1216, 32, "f16"),
    # 128 x 256 ring tiles (at least one per CU): groups of 64, 128, 256 k
    # and one group, with ragged M and a ragged last column block.
    (2000, 4104, 4096, 64, "bf16"),
    (1100, 14336, 2048, 128, "bf16"),
    (2048, 4096, 14336, 256, "f16"),
    (1999, 4232, 2944, -1, "f16"),
    # Tail steps after the 4-step loop with folded groups: 11 steps (three
    # tail steps, the third reads the stage the loop's last step loaded) and
    # 10 steps (two).
    (2048, 4096, 1408, 64, "bf16"),
    (2048, 4096, 1408, 128, "f16"),
    (2048, 4096, 1280, 256, "bf16"),
    # Fewer ring tiles than CUs: K in chunks (fp32 partials, second kernel).
    (300, 14336, 2048, 128, "f16"),
    (384, 4096, 14336, 256, "bf16"),
    (200, 14336, 4096, -1, "bf16"),
    # The largest prefill shapes of the bench, sampled rows.
    (8192, 14336, 4096, -1, "bf16"),
    (8192, 4096, 14336, 256, "bf16"),
]


@pytest.mark.parametrize("M,N,K,G,dtype", W4A8_GEMM, ids=[f"{c[0]}x{c[1]}x{c[2]}g{c[3]}{c[4]}" for c in W4A8_GEMM])
def test_w4a8_gemm_parity(M, N, K, G, dtype):
    case = _case(52, M, N, K, G, UINT4B8, dtype, with_bias=True)
    wq, ws, _, A, bias = to_dev(case)
    packed = w4.repack(wq, ws, None, G, UINT4B8)
    qa, xs = w4.quantize_a8(A)
    C = w4.gemm_w4a8(qa, xs, packed, N, K, G, case.torch_dtype, bias=bias)
    torch.cuda.synchronize()
    rows = sample_rows(M)
    q_ref, xs_ref = oracle.quant_rows_a8(case.A[torch.as_tensor(rows)])
    np.testing.assert_array_equal(qa.cpu().numpy()[rows], pair_order_codes(q_ref))
    ref = oracle.gemm_w4a8(q_ref, xs_ref, case.weight_packed, case.weight_scale, G, case.bias)
    err = rel_err_rows(C, ref, rows)
    assert err <= oracle.TOLERANCE[dtype], f"rel err {err:.3e}"


def test_w4a8_zero_row_gives_bias_and_no_store_past_n():
    M, N, K, G = 4, 1224, 1216, 64
    case = _case(53, M, N, K, G, UINT4B8, "bf16", with_bias=True)
    wq, ws, _, A, bias = to_dev(case)
    A[2] = 0
    packed = w4.repack(wq, ws, None, G, UINT4B8)
    qa, xs = w4.quantize_a8(A)
    big = torch.full((M, N + 16), 77.0, dtype=torch.bfloat16, device=DEV)
    C = w4.gemm_w4a8(qa, xs, packed, N, K, G, torch.bfloat16, bias=bias, out=big[:, :N])
    torch.cuda.synchronize()
    assert torch.all(big[:, N:] == 77.0)
    assert torch.equal(C[2].cpu(), case.bias)


@pytest.mark.parametrize("M,N,K,G", [(2048, 4096, 4096, 128), (1100, 8200, 2048, 256), (2000, 4096, 4096, -1),
                                     (2048, 4096, 2048, 64), (640, 14336, 4096, 128)])
def test_w4a8_ring_equals_register_kernel(M, N, K, G):
    """The tiled ring kernel (16-byte aligned codes, ldq % 16 == 0) and the
    register kernel (ldq % 16 == 8) form the same exact integer group sums
    and fold them identically, so their results agree bit for bit."""
    case = _case(54, M, N, K, G, UINT4B8, "bf16", with_bias=True)
    wq, ws, _, A, bias = to_dev(case)
    packed = w4.repack(wq, ws, None, G, UINT4B8)
    qa, xs = w4.quantize_a8(A)
    padded = torch.zeros((M, K + 8), dtype=torch.int8, device=DEV)
    padded[:, :K] = qa
    C_ring = w4.gemm_w4a8(qa, xs, packed, N, K, G, torch.bfloat16, bias=bias)
    C_reg = w4.gemm_w4a8(padded[:, :K], xs, packed, N, K, G, torch.bfloat16, bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(C_ring, C_reg)


def test_w4a8_then_w4a16_with_default_workspaces():
    """A W4A8 call that splits K writes partial results into its workspace;
    a following W4A16 split-K call on the binding's default workspace must
    still find its arrival counters at zero (the two kinds of call get
    separate default workspaces)."""
    M, N, K, G = 300, 14336, 2048, 128
    case = _case(56, M, N, K, G, UINT4B8, "f16")
    wq, ws, _, A, _ = to_dev(case)
    packed = w4.repack(wq, ws, None, G, UINT4B8)
    assert w4.w4a8_workspace_size(M, N, K, G) > 0
    qa, xs = w4.quantize_a8(A)
    w4.gemm_w4a8(qa, xs, packed, N, K, G, torch.float16)
    case2 = _case(57, 16, 4096, 14336, 128, UINT4B8, "f16")
    assert w4.workspace_size(16, 4096, 14336, 128) > 0
    C = w4.gemm(case2.A.to(DEV), repack(case2), 4096, 14336, 128, UINT4B8)
    torch.cuda.synchronize()
    assert oracle.rel_err(C.cpu(), oracle_ref(case2)) <= oracle.TOLERANCE["f16"]


def test_w4a8_unaligned_output_and_no_bias():
    """C rows that are not 16-byte multiples (ldc % 8 != 0) take the register
    kernel; bias None on the tiled kernel. Same exact sums, same results."""
    M, N, K, G = 2048, 4096, 4096, 64
    case = _case(55, M, N, K, G, UINT4B8, "f16", with_bias=False)
    wq, ws, _, A, _ = to_dev(case)
    packed = w4.repack(wq, ws, None, G, UINT4B8)
    qa, xs = w4.quantize_a8(A)
    C_ring = w4.gemm_w4a8(qa, xs, packed, N, K, G, torch.float16)
    big = torch.full((M, N + 4), 5.0, dtype=torch.float16, device=DEV)
    C_reg = w4.gemm_w4a8(qa, xs, packed, N, K, G, torch.float16, out=big[:, :N])
    torch.cuda.synchronize()
    assert torch.equal(C_ring, C_reg)
    assert torch.all(big[:, N:] == 5.0)
    rows = sample_rows(M)
    q_ref, xs_ref = oracle.quant_rows_a8(case.A[torch.as_tensor(rows)])
    ref = oracle.gemm_w4a8(q_ref, xs_ref, case.weight_packed, case.weight_scale, G, None)
    assert rel_err_rows(C_ring, ref, rows) <= oracle.TOLERANCE["f16"]
