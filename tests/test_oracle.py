"""Pins of the CPU oracle against facts other than itself (CPU only).

Each pin ties an oracle function to something the pages or mathematics fix:
hand words derived from the stated bit positions, the little-endian byte view
of the packed tensor, closed forms of special inputs, a library matmul, exact
rational arithmetic on tiny inputs, and invariants (permutation, K split,
identity activations). ``tests/test_oracle_mutants.py`` plants mistakes in the
oracle source and checks that these pins catch them.
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import w4a16_inputs as wi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
UINT4B8, UINT4 = wi.UINT4B8, wi.UINT4


def _load_gptq_words():
    words, codes = [], []
    with open(os.path.join(GOLDEN, "gptq_words.txt")) as f:
        for ln in f:
            ln = ln.split("#")[0].split()
            if not ln:
                continue
            words.append(int(ln[0], 16))
            codes.append([int(c) for c in ln[1:9]])
    return np.array(words, dtype=np.uint32), np.array(codes, dtype=np.uint8)


def _load_zero_words():
    words, zeros = [], {}
    with open(os.path.join(GOLDEN, "zero_point_words.txt")) as f:
        for ln in f:
            ln = ln.split("#")[0].split()
            if not ln:
                continue
            if ln[0] == "words":
                words.append([int(x, 16) for x in ln[1:]])
            elif ln[0] == "zero":
                zeros[int(ln[1])] = [int(x) for x in ln[2:]]
    z = np.array([zeros[n] for n in range(len(zeros))], dtype=np.uint8)
    return np.array(words, dtype=np.uint32), z


def _act(x, dtype=torch.float16):
    return torch.as_tensor(np.asarray(x, dtype=np.float64)).to(dtype)


# ---------------------------------------------------------------- bit layout


def test_gptq_hand_words(oracle_mod):
    words, codes = _load_gptq_words()
    got = oracle_mod.unpack_codes(words.reshape(-1, 1))
    np.testing.assert_array_equal(got, codes)
    back = oracle_mod.pack_codes(codes).view(np.uint32).reshape(-1)
    np.testing.assert_array_equal(back, words)


def test_gptq_signed_words(oracle_mod):
    # The checkpoint stores int32; a word whose top nibble is >= 8 is negative.
    w = np.array([[-1, np.iinfo(np.int32).min, 0x7FFFFFFF]], dtype=np.int32)
    c = oracle_mod.unpack_codes(w)
    assert list(c[0, 0:8]) == [15] * 8
    assert list(c[0, 8:16]) == [0] * 7 + [8]
    assert list(c[0, 16:24]) == [15] * 7 + [7]
    np.testing.assert_array_equal(oracle_mod.pack_codes(c), w)


def test_gptq_single_nibbles(oracle_mod):
    # Every value at every position, alone in its word: 8 x 16 words.
    words = np.array([[v << (4 * i)] for i in range(8) for v in range(16)], dtype=np.uint64).astype(np.uint32)
    c = oracle_mod.unpack_codes(words)
    for idx, (i, v) in enumerate((i, v) for i in range(8) for v in range(16)):
        expect = [0] * 8
        expect[i] = v
        assert list(c[idx]) == expect


def test_gptq_little_endian_byte_view(oracle_mod):
    # The mixed_precision package page (zentorch W4A16 section): [N, K/8] int32
    # is the same memory as [N, K/2] bytes, little-endian. So byte j of a row
    # holds codes 2j (low nibble) and 2j+1 (high nibble).
    rng = np.random.default_rng(11)
    N, K = 7, 96
    words = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    b = words.view(np.uint8).reshape(N, K // 2)
    expect = np.empty((N, K), dtype=np.uint8)
    expect[:, 0::2] = b & 0xF
    expect[:, 1::2] = b >> 4
    np.testing.assert_array_equal(oracle_mod.unpack_codes(words), expect)


def test_gptq_round_trip(oracle_mod):
    rng = np.random.default_rng(12)
    words = rng.integers(0, 2**32, size=(1000, 1000), dtype=np.uint64).astype(np.uint32)
    words[0, :4] = [0, 0xFFFFFFFF, 0x80000000, 0x7FFFFFFF]
    np.testing.assert_array_equal(oracle_mod.pack_codes(oracle_mod.unpack_codes(words)).view(np.uint32), words)
    codes = rng.integers(0, 16, size=(33, 256), dtype=np.uint8)
    np.testing.assert_array_equal(oracle_mod.unpack_codes(oracle_mod.pack_codes(codes)), codes)


def test_zero_point_hand_words(oracle_mod):
    words, zeros = _load_zero_words()
    np.testing.assert_array_equal(oracle_mod.unpack_zeros(words, 16), zeros)
    np.testing.assert_array_equal(oracle_mod.pack_zeros(zeros).view(np.uint32), words)


def test_zero_point_byte_view(oracle_mod):
    # Byte j of word (b, g) holds rows 8b+2j (low nibble) and 8b+2j+1 (high).
    rng = np.random.default_rng(13)
    N, Kg = 40, 6
    words = rng.integers(0, 2**32, size=(N // 8, Kg), dtype=np.uint64).astype(np.uint32)
    by = words.view(np.uint8).reshape(N // 8, Kg, 4)
    expect = np.empty((N, Kg), dtype=np.uint8)
    for b in range(N // 8):
        for j in range(4):
            expect[8 * b + 2 * j] = by[b, :, j] & 0xF
            expect[8 * b + 2 * j + 1] = by[b, :, j] >> 4
    np.testing.assert_array_equal(oracle_mod.unpack_zeros(words, N), expect)
    np.testing.assert_array_equal(oracle_mod.pack_zeros(expect).view(np.uint32), words)


# ------------------------------------------------- checkpoint orientations


def _load_layout_blocks():
    blocks, cur = [], None
    with open(os.path.join(GOLDEN, "layout_words.txt")) as f:
        for ln in f:
            ln = ln.split("#")[0].split()
            if not ln:
                continue
            if ln[0] in ("weight", "zero"):
                od, pd, r, c = (int(x) for x in ln[1:5])
                cur = dict(kind=ln[0], od=od, pd=pd, words=np.zeros((r, c), dtype=np.uint32), expect=[])
            elif ln[0] == "word":
                cur["words"][int(ln[1]), int(ln[2])] = int(ln[3], 16)
            elif ln[0] == "expect":
                cur["expect"].append(tuple(int(x) for x in ln[1:4]))
            elif ln[0] == "end":
                blocks.append(cur)
    return blocks


def _nk_shape(b):
    r, c = b["words"].shape
    n_dim = b["od"]  # the tensor dimension over N
    dims = [r, c]
    dims[b["pd"]] *= 8
    return (dims[n_dim], dims[1 - n_dim])


@pytest.mark.parametrize("idx", range(6))
def test_layout_hand_words(oracle_mod, idx):
    b = _load_layout_blocks()[idx]
    if b["kind"] == "weight":
        got = oracle_mod.weight_codes_nk(b["words"], b["od"], b["pd"])
    else:
        assert b["pd"] == b["od"]  # zero points are packed along N
        got = oracle_mod.zeros_nk(b["words"], b["od"])
    expect = np.zeros(_nk_shape(b), dtype=np.uint8)
    for n, k, v in b["expect"]:
        expect[n, k] = v
    assert got.shape == expect.shape
    np.testing.assert_array_equal(got, expect)


def test_layout_blocks_cover_every_orientation():
    seen = {(b["kind"], b["od"], b["pd"]) for b in _load_layout_blocks()}
    assert seen == {("weight", 0, 0), ("weight", 0, 1), ("weight", 1, 0), ("weight", 1, 1),
                    ("zero", 0, 0), ("zero", 1, 1)}


def test_layout_canonical_matches_c_unpack(oracle_mod):
    # Two independent readers of the compressed-tensors words (numpy here, C
    # for the GEMM oracle) agree, and the transposed (K/8, N) tensor with
    # output_dim=1, packed_dim=0 holds the same codes.
    rng = np.random.default_rng(21)
    words = rng.integers(0, 2**32, size=(24, 40), dtype=np.uint64).astype(np.uint32)
    ref = oracle_mod.unpack_codes(words)
    np.testing.assert_array_equal(oracle_mod.weight_codes_nk(words, 0, 1), ref)
    np.testing.assert_array_equal(oracle_mod.weight_codes_nk(np.ascontiguousarray(words.T), 1, 0), ref)
    # (N/8, K) and its transpose (K, N/8) with the packed dimension along N.
    wn = rng.integers(0, 2**32, size=(5, 72), dtype=np.uint64).astype(np.uint32)
    a = oracle_mod.weight_codes_nk(wn, 0, 0)
    np.testing.assert_array_equal(oracle_mod.weight_codes_nk(np.ascontiguousarray(wn.T), 1, 1), a)
    # Packed along N, column k of the codes is the C zero-point reader applied
    # to column k of the words (the same "eight rows per word" rule).
    np.testing.assert_array_equal(a, oracle_mod.unpack_zeros(wn, 40))


def test_layout_zero_points_match_c_unpack(oracle_mod):
    rng = np.random.default_rng(22)
    zw = rng.integers(0, 2**32, size=(6, 9), dtype=np.uint64).astype(np.uint32)
    ref = oracle_mod.unpack_zeros(zw, 48)
    np.testing.assert_array_equal(oracle_mod.zeros_nk(zw, 0), ref)
    np.testing.assert_array_equal(oracle_mod.zeros_nk(np.ascontiguousarray(zw.T), 1), ref)


def test_layout_scales_orientation(oracle_mod):
    t = torch.tensor([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]], dtype=torch.bfloat16)  # [Kg=2, N=3]
    got = oracle_mod.scales_nk(t, 1)
    assert got.dtype == torch.bfloat16 and got.is_contiguous()
    assert got.tolist() == [[1.0, 4.0], [2.0, 5.0], [3.0, 6.0]]
    assert torch.equal(oracle_mod.scales_nk(t, 0), t)


def test_layout_rejects_bad_dims(oracle_mod):
    w = np.zeros((2, 2), dtype=np.uint32)
    for od, pd in ((2, 0), (0, 2), (-1, 1)):
        with pytest.raises(ValueError):
            oracle_mod.weight_codes_nk(w, od, pd)
    with pytest.raises(ValueError):
        oracle_mod.zeros_nk(w, 2)


# ---------------------------------------------------------------- dequant


def _rand_scales(rng, N, Kg, dtype=torch.float16):
    return _act(rng.uniform(0.005, 0.02, size=(N, Kg)), dtype)


@pytest.mark.parametrize("G", [32, 64, 128, -1])
def test_dequant_symmetric_closed_form(oracle_mod, G):
    # uint4b8: w = (q - 8) * s. Codes 8 + c give c * s, with s repeated over
    # the G consecutive k of each group.
    rng = np.random.default_rng(20)
    N, K = 16, 256
    Ge = K if G == -1 else G
    c = rng.integers(-8, 8, size=(N, K))
    s = _rand_scales(rng, N, K // Ge)
    W = oracle_mod.dequant(oracle_mod.pack_codes(c + 8), s, None, UINT4B8, G)
    expect = c * np.repeat(s.double().numpy(), Ge, axis=1)
    np.testing.assert_array_equal(W, expect)
    # all codes 8 -> exactly 0 for any scale
    W0 = oracle_mod.dequant(oracle_mod.pack_codes(np.full((N, K), 8)), s, None, UINT4B8, G)
    assert np.all(W0 == 0)


@pytest.mark.parametrize("G", [32, 128, -1])
def test_dequant_asymmetric_closed_form(oracle_mod, G):
    rng = np.random.default_rng(21)
    N, K = 24, 256
    Ge = K if G == -1 else G
    Kg = K // Ge
    z = rng.integers(0, 16, size=(N, Kg))
    zfull = np.repeat(z, Ge, axis=1)
    s = _rand_scales(rng, N, Kg, torch.bfloat16)
    zp = oracle_mod.pack_zeros(z)
    # codes equal to the zero -> exactly 0
    W0 = oracle_mod.dequant(oracle_mod.pack_codes(zfull), s, zp, UINT4, G)
    assert np.all(W0 == 0)
    # q = z + d with d in [-z, 15 - z] -> d * s
    q = rng.integers(0, 16, size=(N, K))
    W = oracle_mod.dequant(oracle_mod.pack_codes(q), s, zp, UINT4, G)
    np.testing.assert_array_equal(W, (q - zfull) * np.repeat(s.double().numpy(), Ge, axis=1))
    # uint4 without zero points subtracts nothing
    Wn = oracle_mod.dequant(oracle_mod.pack_codes(q), s, None, UINT4, G)
    np.testing.assert_array_equal(Wn, q * np.repeat(s.double().numpy(), Ge, axis=1))


def test_dequant_symmetric_ignores_zero_points(oracle_mod):
    c = wi.make_case(9, 1, 32, 256, 64, UINT4, "f16")
    a = oracle_mod.dequant(c.weight_packed, c.weight_scale, c.weight_zero_point, UINT4B8, 64)
    b = oracle_mod.dequant(c.weight_packed, c.weight_scale, None, UINT4B8, 64)
    np.testing.assert_array_equal(a, b)


def test_dequant_group_minus_one_is_K(oracle_mod):
    c = wi.make_case(9, 1, 16, 384, -1, UINT4, "bf16")
    a = oracle_mod.dequant(c.weight_packed, c.weight_scale, c.weight_zero_point, UINT4, -1)
    b = oracle_mod.dequant(c.weight_packed, c.weight_scale, c.weight_zero_point, UINT4, 384)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- GEMM


def _bound(A64, W64, bias=None):
    """A rigorous bound on fp64 rounding of a K-term dot product (+ bias)."""
    K = A64.shape[1]
    mag = np.abs(A64) @ np.abs(W64).T
    if bias is not None:
        mag = mag + np.abs(bias)[None, :]
    return (K + 2) * 2.0**-52 * mag + 1e-300


@pytest.mark.parametrize(
    "M,N,K,G,qtype,dtype,bias",
    [
        (3, 48, 256, 32, UINT4, "bf16", True),
        (5, 32, 384, 128, UINT4B8, "f16", False),
        (1, 16, 128, -1, UINT4B8, "f16", True),
        (8, 40, 512, 64, UINT4, "f16", False),
    ],
)
def test_gemm_matches_library_matmul(oracle_mod, M, N, K, G, qtype, dtype, bias):
    c = wi.make_case(8, M, N, K, G, qtype, dtype, with_bias=bias)
    C, _ = oracle_mod.gemm(c.A, c.weight_packed, c.weight_scale, c.weight_zero_point, qtype, G, c.bias)
    W = oracle_mod.dequant(c.weight_packed, c.weight_scale, c.weight_zero_point, qtype, G)
    A64 = c.A.double().numpy()
    b64 = None if c.bias is None else c.bias.double().numpy()
    ref = np.matmul(A64, W.T) + (0 if b64 is None else b64[None, :])
    assert np.all(np.abs(C - ref) <= _bound(A64, W, b64))


def _fraction_gemm(A, codes, zeros, scales, G, bias):
    """Exact rational C for tiny inputs: every fp16/bf16 value is dyadic."""
    M, K = len(A), len(A[0])
    N = len(codes)
    Ge = K if G == -1 else G
    C = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // Ge
                acc += Fraction(A[m][k]) * (codes[n][k] - zeros[n][g]) * Fraction(scales[n][g])
            if bias is not None:
                acc += Fraction(bias[n])
            row.append(acc)
        C.append(row)
    return C


@pytest.mark.parametrize(
    "M,N,K,G,qtype,with_bias",
    [
        (1, 8, 128, 32, UINT4B8, False),
        (2, 16, 128, 128, UINT4, True),
        (3, 8, 256, -1, UINT4, False),
        (2, 16, 256, 32, UINT4B8, True),
    ],
)
def test_gemm_exact_rational(oracle_mod, M, N, K, G, qtype, with_bias):
    rng = np.random.default_rng([M, N, K, G + 2, qtype])
    Ge = K if G == -1 else G
    Kg = K // Ge
    codes = rng.integers(0, 16, size=(N, K))
    z = rng.integers(0, 16, size=(N, Kg)) if qtype == UINT4 else np.full((N, Kg), 8)
    s = _rand_scales(rng, N, Kg)
    A = _act(rng.normal(0, 1, size=(M, K)))
    bias = _act(rng.normal(0, 1, size=(N,))) if with_bias else None
    zp = oracle_mod.pack_zeros(z) if qtype == UINT4 else None
    C, _ = oracle_mod.gemm(A, oracle_mod.pack_codes(codes), s, zp, qtype, G, bias)
    exact = _fraction_gemm(
        A.double().tolist(), codes.tolist(), z.tolist(), s.double().tolist(), G,
        None if bias is None else bias.double().tolist(),
    )
    W = (codes - np.repeat(z, Ge, axis=1)) * np.repeat(s.double().numpy(), Ge, axis=1)
    bnd = _bound(A.double().numpy(), W, None if bias is None else bias.double().numpy())
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(C[m, n]) - exact[m][n]) <= Fraction(bnd[m, n])


@pytest.mark.parametrize("qtype", [UINT4B8, UINT4])
def test_gemm_zero_weights_give_bias(oracle_mod, qtype):
    rng = np.random.default_rng(30)
    M, N, K, G = 4, 32, 256, 64
    z = rng.integers(0, 16, size=(N, K // G)) if qtype == UINT4 else np.full((N, K // G), 8)
    codes = np.repeat(z, G, axis=1)
    zp = oracle_mod.pack_zeros(z) if qtype == UINT4 else None
    s = _rand_scales(rng, N, K // G)
    A = _act(rng.normal(0, 1, size=(M, K)))
    bias = _act(rng.normal(0, 1, size=(N,)))
    C, _ = oracle_mod.gemm(A, oracle_mod.pack_codes(codes), s, zp, qtype, G)
    assert np.all(C == 0)
    Cb, _ = oracle_mod.gemm(A, oracle_mod.pack_codes(codes), s, zp, qtype, G, bias)
    np.testing.assert_array_equal(Cb, np.broadcast_to(bias.double().numpy(), (M, N)))


@pytest.mark.parametrize("cval", [-8, -3, 1, 7])
def test_gemm_uniform_codes_unit_scales(oracle_mod, cval):
    # codes 8 + c, scales 1: C[m, n] = c * sum_k A[m, k]. The fp16 values of A
    # span fewer than 40 binary orders, so every partial sum is exact in fp64
    # and the equality is exact.
    rng = np.random.default_rng(31)
    M, N, K, G = 3, 16, 512, 128
    codes = np.full((N, K), 8 + cval)
    s = torch.ones((N, K // G), dtype=torch.float16)
    A = _act(rng.normal(0, 1, size=(M, K)))
    C, _ = oracle_mod.gemm(A, oracle_mod.pack_codes(codes), s, None, UINT4B8, G)
    rowsum = A.double().numpy().sum(axis=1)
    np.testing.assert_array_equal(C, np.broadcast_to((cval * rowsum)[:, None], (M, N)))


def test_gemm_unit_codes_group_scales(oracle_mod):
    # codes z + 1: C[m, n] = sum_g s[n, g] * (sum of A[m, k] over group g).
    rng = np.random.default_rng(32)
    M, N, K, G = 2, 24, 256, 32
    Kg = K // G
    z = rng.integers(0, 15, size=(N, Kg))
    codes = np.repeat(z + 1, G, axis=1)
    s = _rand_scales(rng, N, Kg, torch.bfloat16)
    A = _act(rng.normal(0, 1, size=(M, K)), torch.bfloat16)
    C, _ = oracle_mod.gemm(A, oracle_mod.pack_codes(codes), s, oracle_mod.pack_zeros(z), UINT4, G)
    gsum = A.double().numpy().reshape(M, Kg, G).sum(axis=2)  # exact
    ref = gsum @ s.double().numpy().T
    bnd = (Kg + 2) * 2.0**-52 * (np.abs(gsum) @ np.abs(s.double().numpy()).T)
    assert np.all(np.abs(C - ref) <= bnd + 1e-300)


def test_gemm_identity_activations(oracle_mod):
    # A = I: C[m, n] = W[n, m] exactly; a transposed operand fails this.
    c = wi.make_case(33, 1, 48, 128, 32, UINT4, "f16")
    A = torch.eye(128, dtype=torch.float16)
    C, _ = oracle_mod.gemm(A, c.weight_packed, c.weight_scale, c.weight_zero_point, UINT4, 32)
    codes = oracle_mod.unpack_codes(c.weight_packed)
    z = np.repeat(oracle_mod.unpack_zeros(c.weight_zero_point, 48), 32, axis=1)
    W = (codes.astype(np.int64) - z) * np.repeat(c.weight_scale.double().numpy(), 32, axis=1)
    np.testing.assert_array_equal(C, W.T)


def test_gemm_row_permutation(oracle_mod):
    c = wi.make_case(34, 3, 64, 256, 64, UINT4B8, "f16")
    C, _ = oracle_mod.gemm(c.A, c.weight_packed, c.weight_scale, None, UINT4B8, 64)
    perm = np.random.default_rng(34).permutation(64)
    Cp, _ = oracle_mod.gemm(c.A, c.weight_packed[perm], c.weight_scale[torch.as_tensor(perm)], None, UINT4B8, 64)
    np.testing.assert_array_equal(Cp, C[:, perm])


def test_gemm_k_split_linearity(oracle_mod):
    c = wi.make_case(35, 4, 32, 512, 64, UINT4, "bf16")
    K1 = 192  # group aligned
    C, _ = oracle_mod.gemm(c.A, c.weight_packed, c.weight_scale, c.weight_zero_point, UINT4, 64)
    C1, _ = oracle_mod.gemm(
        c.A[:, :K1], c.weight_packed[:, : K1 // 8], c.weight_scale[:, : K1 // 64],
        c.weight_zero_point[:, : K1 // 64], UINT4, 64,
    )
    C2, _ = oracle_mod.gemm(
        c.A[:, K1:], c.weight_packed[:, K1 // 8 :], c.weight_scale[:, K1 // 64 :],
        c.weight_zero_point[:, K1 // 64 :], UINT4, 64,
    )
    W = oracle_mod.dequant(c.weight_packed, c.weight_scale, c.weight_zero_point, UINT4, 64)
    assert np.all(np.abs(C - (C1 + C2)) <= 2 * _bound(c.A.double().numpy(), W))


def test_gemm_rows_subset_and_threads(oracle_mod):
    c = wi.make_case(36, 9, 32, 256, 128, UINT4B8, "f16", with_bias=True)
    C, used = oracle_mod.gemm(c.A, c.weight_packed, c.weight_scale, None, UINT4B8, 128, c.bias)
    assert used >= 1
    rows = [8, 0, 3]
    Cs, _ = oracle_mod.gemm(c.A, c.weight_packed, c.weight_scale, None, UINT4B8, 128, c.bias, rows=rows)
    np.testing.assert_array_equal(Cs, C[rows])
    C1, used1 = oracle_mod.gemm(c.A, c.weight_packed, c.weight_scale, None, UINT4B8, 128, c.bias, nthreads=1)
    assert used1 == 1
    np.testing.assert_array_equal(C1, C)


def test_rel_err_definition(oracle_mod):
    ref = np.array([[1.0, -4.0], [2.0, 0.5]])
    test = torch.tensor([[1.0, -4.0], [2.0, 0.25]], dtype=torch.float16)
    assert oracle_mod.rel_err(test, ref) == pytest.approx(0.25 / 4.0)
    assert oracle_mod.rel_err(np.zeros((2, 2)), np.zeros((2, 2))) == 0.0
    assert oracle_mod.rel_err(np.full((1, 1), 1e-3), np.zeros((1, 1))) == 1e-3


# ---------------------------------------------------------------- device layout


def test_device_size_hand_values(oracle_mod):
    # N=16, K=128, one group: codes 1024 B; scales 16*2 = 32 B at 1024; end 1056 -> 1280.
    assert oracle_mod.device_size(16, 128, 128, UINT4B8) == 1280
    # uint4 adds 16 zero bytes at align256(1056) = 1280 -> end 1296 -> 1536.
    assert oracle_mod.device_size(16, 128, -1, UINT4) == 1536
    # N=4096, K=4096, G=128: 8 MiB codes + 256 KiB scales.
    assert oracle_mod.device_size(4096, 4096, 128, UINT4B8) == 4096 * 2048 + 4096 * 32 * 2
    # K not a multiple of 128 pads K to Kp and the groups to Kp / G.
    # N=16, K=96, G=32: Kp=128, 4 stored groups: codes 1024; scales 16*4*2 = 128
    # -> 1152; zeros at 1280, 64 bytes -> 1344 -> 1536 (uint4b8: 1152 -> 1280).
    assert oracle_mod.device_size(16, 96, 32, UINT4) == 1536
    assert oracle_mod.device_size(16, 96, 32, UINT4B8) == 1280
    # N=16, K=40, one group: Kp=128: codes 1024, scales 32 -> 1056 -> 1280.
    assert oracle_mod.device_size(16, 40, -1, UINT4B8) == 1280
    # N=32, K=2880, G=64: Kp=2944, 46 stored groups (45 real): codes 47104
    # (256-aligned), scales 32*46*2 = 2944 -> 50048 -> 50176.
    assert oracle_mod.device_size(32, 2880, 64, UINT4B8) == 50176
    # N not a multiple of 16 pads N to Np. N=24, K=128, one group: Np=32:
    # codes 2048; scales 64 -> 2112 -> 2304.
    assert oracle_mod.device_size(24, 128, 128, UINT4B8) == 2304
    # N=8, K=40, uint4: Np=16, Kp=128: codes 1024, scales 32 -> 1056; zeros at
    # 1280, 16 bytes -> 1296 -> 1536.
    assert oracle_mod.device_size(8, 40, -1, UINT4) == 1536


def test_device_encoder_hand_words(oracle_mod):
    # Codes c(n, k) = k % 16 on rows 0..15 and (k + 5) % 16 on rows 16..31
    # (N = 32, K = 256: two n-tiles by two k-tiles). Words derived by hand
    # from the layout rule: tile (nt, kt) at (nt*2 + kt)*1024; word 4l + s
    # holds row 16nt + l%16, k = 128kt + 32s + 8(l//16) + i, code i at bit
    # 4*(i//2) + 16*(i%2).
    N, K = 32, 256
    k = np.arange(K)
    codes = np.empty((N, K), dtype=np.uint8)
    codes[:16] = k % 16
    codes[16:] = (k + 5) % 16
    s = torch.full((N, 2), 0.5, dtype=torch.float16)
    out = oracle_mod.encode_device(codes, s, None, UINT4B8, 128)
    w = out[: N * K // 2].view(np.uint32)
    # tile (0,0), l=0, s=0: k 0..7 -> codes 0..7 -> pairs (0,1)(2,3)(4,5)(6,7)
    # low halves 0,2,4,6 at bits 0,4,8,12; high halves 1,3,5,7 at 16,20,24,28.
    assert w[0] == 0x75316420
    # tile (0,0), l=16 (row 0, k-subblock 1), s=0: k 8..15 -> codes 8..15
    assert w[4 * 16 + 0] == 0xFDB9ECA8
    # tile (0,0), l=0, s=1: k 32..39 -> codes 0..7 again (k % 16)
    assert w[1] == 0x75316420
    # tile (0,1), l=5 (row 5), s=3: k = 128 + 96 + 0..7 = 224..231 -> codes 0..7
    assert w[256 * 1 + 4 * 5 + 3] == 0x75316420
    # tile (1,0), l=0 (row 16), s=0: codes (k+5)%16 for k 0..7 = 5..12
    # lows 5,7,9,11 -> 0xB975 ; highs 6,8,10,12 -> 0xCA86
    assert w[256 * 2] == 0xCA86B975
    # tile (1,1), l=63 (row 31, sub 3), s=2: k = 128+64+24 = 216..223,
    # (k+5)%16 = 13,14,15,0,1,2,3,4 -> lows 13,15,1,3 ; highs 14,0,2,4
    assert w[256 * 3 + 4 * 63 + 2] == 0x420E31FD
    # scales: region at N*K/2 = 4096 (already 256-aligned), 32*2 elements,
    # (nt, g, r) at 4096 + ((nt*2+g)*16+r)*2; fp16 0.5 is 0x3800. The region
    # ends at 4224, so the buffer is 4352 bytes.
    sb = out[4096 : 4096 + 64 * 2].view(np.uint16)
    assert np.all(sb == 0x3800)
    assert len(out) == 4352


def test_device_encoder_padded_k_hand_words(oracle_mod):
    # N = 16, K = 40 (one group): Kp = 128, one tile; codes c(n, k) = k % 16.
    # Word 4l + s holds row l%16 at k = 32s + 8(l//16) + i; k >= 40 holds 0.
    N, K = 16, 40
    codes = np.tile((np.arange(K) % 16).astype(np.uint8), (N, 1))
    out = oracle_mod.encode_device(codes, torch.full((N, 1), 0.5, dtype=torch.float16), None, UINT4B8, -1)
    assert len(out) == 1280
    w = out[:1024].view(np.uint32)
    assert w[4 * 0 + 0] == 0x75316420  # l=0,  s=0: k 0..7   -> codes 0..7
    assert w[4 * 16 + 0] == 0xFDB9ECA8  # l=16, s=0: k 8..15  -> codes 8..15
    assert w[4 * 48 + 0] == 0xFDB9ECA8  # l=48, s=0: k 24..31 -> codes 8..15
    assert w[4 * 0 + 1] == 0x75316420  # l=0,  s=1: k 32..39 -> codes 0..7
    assert w[4 * 16 + 1] == 0  # l=16, s=1: k 40..47, past K
    assert w[4 * 5 + 2] == 0 and w[4 * 63 + 3] == 0  # k >= 64
    # 1 KB of codes, then the 16 scales (fp16 0.5 = 0x3800) at 1024.
    assert np.all(out[1024:1056].view(np.uint16) == 0x3800)
    assert np.all(out[1056:] == 0)


def test_device_encoder_padded_n_hand_words(oracle_mod):
    # N = 8, K = 128: one tile whose rows 8..15 are padding; c(n, k) = k % 16.
    N, K = 8, 128
    codes = np.tile((np.arange(K) % 16).astype(np.uint8), (N, 1))
    out = oracle_mod.encode_device(codes, torch.full((N, 1), 0.5, dtype=torch.float16), None, UINT4B8, -1)
    assert len(out) == 1280
    w = out[:1024].view(np.uint32)
    assert w[4 * 0 + 0] == 0x75316420  # l=0 (row 0), s=0: k 0..7
    assert w[4 * 23 + 0] == 0xFDB9ECA8  # l=23 (row 7, k-subblock 1), s=0: k 8..15
    assert w[4 * 8 + 0] == 0 and w[4 * 31 + 3] == 0 and w[4 * 63 + 2] == 0  # rows 8, 15, 15
    # scales (nt=0, g=0, r): rows 0..7 hold 0.5 (0x3800), rows 8..15 hold 0
    sreg = out[1024:1056].view(np.uint16)
    assert np.all(sreg[:8] == 0x3800) and np.all(sreg[8:] == 0)


def test_device_encoder_padded_n_inverse(oracle_mod):
    # N = 24 (Np = 32), K = 160 (Kp = 256), G = 32 (Kg 5, Kgp 8), uint4.
    c = wi.make_case(39, 1, 24, 160, 32, UINT4, "bf16")
    codes = oracle_mod.unpack_codes(c.weight_packed)
    zeros = oracle_mod.unpack_zeros(c.weight_zero_point, 24)
    out = oracle_mod.encode_device(codes, c.weight_scale, zeros, UINT4, 32)
    N, Np, K, Kp, Kg, Kgp, KT = 24, 32, 160, 256, 5, 8, 2
    words = out[: Np * Kp // 2].view(np.uint32)
    for n in range(Np):
        for k in range(0, Kp, 8):
            nt, r, kt = n // 16, n % 16, k // 128
            s_, sub = (k % 128) // 32, (k % 32) // 8
            word = int(words[(nt * KT + kt) * 256 + 4 * (16 * sub + r) + s_])
            for i in range(8):
                want = codes[n, k + i] if (n < N and k + i < K) else 0
                assert (word >> (4 * (i // 2) + 16 * (i % 2))) & 0xF == want
    S0 = Np * Kp // 2
    sbits = c.weight_scale.view(torch.int16).numpy().view(np.uint16)
    sreg = out[S0 : S0 + Np * Kgp * 2].view(np.uint16)
    Z0 = S0 + ((Np * Kgp * 2 + 255) // 256) * 256
    for n in range(Np):
        for g in range(Kgp):
            idx = ((n // 16) * Kgp + g) * 16 + n % 16
            real = n < N and g < Kg
            assert sreg[idx] == (sbits[n, g] if real else 0)
            assert out[Z0 + idx] == (zeros[n, g] if real else 0)
    assert len(out) == oracle_mod.device_size(N, K, 32, UINT4)


def test_device_encoder_padded_groups_hand_values(oracle_mod):
    # N = 16, K = 96, G = 32: Kg = 3 real groups, 4 stored; scale of group g
    # is g + 1 (fp16 0x3C00, 0x4000, 0x4200), zero of (n, g) is (n + g) % 16.
    N, K, G = 16, 96, 32
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = torch.tensor([[1.0, 2.0, 3.0]] * N, dtype=torch.float16)
    zeros = np.array([[(n + g) % 16 for g in range(3)] for n in range(N)], dtype=np.uint8)
    out = oracle_mod.encode_device(codes, scales, zeros, UINT4, G)
    assert len(out) == 1536
    sreg = out[1024:1024 + 4 * 16 * 2].view(np.uint16).reshape(4, 16)  # (g, r) of n-tile 0
    assert np.all(sreg[0] == 0x3C00) and np.all(sreg[1] == 0x4000) and np.all(sreg[2] == 0x4200)
    assert np.all(sreg[3] == 0)
    zreg = out[1280:1280 + 64].reshape(4, 16)
    for g in range(3):
        assert list(zreg[g]) == [(r + g) % 16 for r in range(16)]
    assert np.all(zreg[3] == 0)
    assert np.all(out[:1024] == 0) and np.all(out[1344:] == 0)


def test_device_encoder_padded_inverse(oracle_mod):
    # K = 160, G = 32: Kp = 256 (two k-tiles), Kg = 5, Kgp = 8; read every
    # code, scale and zero back by the layout rule, and check the padding.
    c = wi.make_case(38, 1, 32, 160, 32, UINT4, "f16")
    codes = oracle_mod.unpack_codes(c.weight_packed)
    zeros = oracle_mod.unpack_zeros(c.weight_zero_point, 32)
    out = oracle_mod.encode_device(codes, c.weight_scale, zeros, UINT4, 32)
    N, K, Kp, Kg, Kgp, KT = 32, 160, 256, 5, 8, 2
    words = out[: N * Kp // 2].view(np.uint32)
    for n in range(N):
        for k in range(0, Kp, 8):
            nt, r, kt = n // 16, n % 16, k // 128
            s_, sub = (k % 128) // 32, (k % 32) // 8
            word = int(words[(nt * KT + kt) * 256 + 4 * (16 * sub + r) + s_])
            for i in range(8):
                want = codes[n, k + i] if k + i < K else 0
                assert (word >> (4 * (i // 2) + 16 * (i % 2))) & 0xF == want
    S0 = N * Kp // 2
    sbits = c.weight_scale.view(torch.int16).numpy().view(np.uint16)
    sreg = out[S0 : S0 + N * Kgp * 2].view(np.uint16)
    Z0 = S0 + ((N * Kgp * 2 + 255) // 256) * 256
    for n in range(N):
        for g in range(Kgp):
            idx = ((n // 16) * Kgp + g) * 16 + n % 16
            assert sreg[idx] == (sbits[n, g] if g < Kg else 0)
            assert out[Z0 + idx] == (zeros[n, g] if g < Kg else 0)
    assert len(out) == oracle_mod.device_size(N, K, 32, UINT4)


def test_device_encoder_inverse(oracle_mod):
    # Read every code, scale and zero back from the bytes by the layout rule.
    c = wi.make_case(37, 1, 48, 384, 32, UINT4, "bf16")
    codes = oracle_mod.unpack_codes(c.weight_packed)
    zeros = oracle_mod.unpack_zeros(c.weight_zero_point, 48)
    out = oracle_mod.encode_device(codes, c.weight_scale, zeros, UINT4, 32)
    N, K, Kg, KT = 48, 384, 12, 3
    words = out[: N * K // 2].view(np.uint32)
    for n in range(N):
        for k in range(0, K, 8):
            nt, r, kt = n // 16, n % 16, k // 128
            s_, sub = (k % 128) // 32, (k % 32) // 8
            word = int(words[(nt * KT + kt) * 256 + 4 * (16 * sub + r) + s_])
            for i in range(8):
                assert (word >> (4 * (i // 2) + 16 * (i % 2))) & 0xF == codes[n, k + i]
    S0 = N * K // 2
    sbits = c.weight_scale.view(torch.int16).numpy().view(np.uint16)
    sreg = out[S0 : S0 + N * Kg * 2].view(np.uint16)
    Z0 = S0 + ((N * Kg * 2 + 255) // 256) * 256
    for n in range(N):
        for g in range(Kg):
            assert sreg[((n // 16) * Kg + g) * 16 + n % 16] == sbits[n, g]
            assert out[Z0 + ((n // 16) * Kg + g) * 16 + n % 16] == zeros[n, g]


# ---------------------------------------------------------------- W4A8


def test_quant_a8_hand_values(oracle_mod):
    # Row 0: max |x| = 127, so the scale is exactly 1 and q = rint(x) (half to
    # even: 2.5 -> 2); fp16 0.4 is 0.39990234375 -> 0, fp16 -0.6 -> -1.
    # Row 1: max |x| = 254, scale 2: 3/2 = 1.5 -> 2, 5/2 = 2.5 -> 2, 1/2 -> 0.
    # Row 2: all zero: scale 0, codes 0.
    A = torch.tensor([[127.0, -63.0, 1.0, 0.4, -0.6, 2.5, 0.0, 0.0],
                      [3.0, 5.0, -254.0, 1.0, 0.0, 0.0, 0.0, 0.0],
                      [0.0] * 8], dtype=torch.float16)
    q, xs = oracle_mod.quant_rows_a8(A)
    assert q.tolist() == [[127, -63, 1, 0, -1, 2, 0, 0], [2, 2, -127, 0, 0, 0, 0, 0], [0] * 8]
    assert xs.tolist() == [1.0, 2.0, 0.0]


def test_quant_a8_properties(oracle_mod):
    rng = np.random.default_rng(31)
    A = torch.from_numpy(rng.normal(0, 3, size=(40, 96))).to(torch.bfloat16)
    q, xs = oracle_mod.quant_rows_a8(A)
    a = A.to(torch.float32).numpy()
    amax = np.abs(a).max(axis=1)
    assert np.array_equal(xs, (amax / np.float32(127)).astype(np.float32))
    assert np.abs(q.astype(int)).max() <= 127
    assert np.all(np.abs(q.astype(int)).max(axis=1) == 127)  # the largest value maps to +-127
    # |q*s - x| <= s/2 (plus the rounding of the division)
    err = np.abs(q * xs[:, None].astype(np.float64) - a)
    assert np.all(err <= xs[:, None] * (0.5 + 2e-5))  # x / s rounds with relative error 2^-24 on |q| <= 127


@pytest.mark.parametrize("G,with_bias", [(32, True), (-1, False), (64, True)])
def test_gemm_w4a8_exact_rational(oracle_mod, G, with_bias):
    rng = np.random.default_rng([32, G + 2])
    M, N, K = 2, 8, 64
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    xs = rng.uniform(0.001, 0.05, size=M).astype(np.float32)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    Ge = K if G == -1 else G
    scales = torch.from_numpy(rng.uniform(0.005, 0.02, size=(N, K // Ge))).to(torch.float16)
    bias = torch.from_numpy(rng.normal(0, 1, size=N)).to(torch.float16) if with_bias else None
    C = oracle_mod.gemm_w4a8(q, xs, oracle_mod.pack_codes(codes), scales, G, bias)
    sf = scales.to(torch.float64).numpy()
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for g in range(K // Ge):
                isum = sum(int(q[m, k]) * (int(codes[n, k]) - 8) for k in range(g * Ge, (g + 1) * Ge))
                acc += Fraction(float(sf[n, g])) * isum
            acc *= Fraction(float(xs[m]))
            if bias is not None:
                acc += Fraction(float(bias[n]))
            assert abs(Fraction(C[m, n]) - acc) <= abs(acc) * Fraction(1, 2**50) + Fraction(1, 2**80)


def test_gemm_w4a8_zero_weights_give_bias(oracle_mod):
    M, N, K = 3, 16, 128
    q = np.full((M, K), 100, dtype=np.int8)
    codes = np.full((N, K), 8, dtype=np.uint8)
    bias = torch.arange(N, dtype=torch.float16)
    C = oracle_mod.gemm_w4a8(q, np.ones(M, np.float32), oracle_mod.pack_codes(codes),
                             torch.ones((N, 1), dtype=torch.float16), -1, bias)
    assert np.array_equal(C, np.tile(np.arange(N, dtype=np.float64), (M, 1)))


def test_gemm_w4a8_matches_dequantised_product(oracle_mod):
    # xs * (q @ W^T) with W the dequantised symmetric weights, by the library matmul.
    rng = np.random.default_rng(33)
    M, N, K, G = 5, 24, 256, 128
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    xs = rng.uniform(0.001, 0.05, size=M).astype(np.float32)
    words = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    scales = torch.from_numpy(rng.uniform(0.005, 0.02, size=(N, K // G))).to(torch.bfloat16)
    W = oracle_mod.dequant(words, scales, None, UINT4B8, G)
    ref = (q.astype(np.float64) @ W.T) * xs[:, None].astype(np.float64)
    C = oracle_mod.gemm_w4a8(q, xs, words, scales, G)
    assert np.max(np.abs(C - ref)) <= 1e-12 * np.max(np.abs(ref))
