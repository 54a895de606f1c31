"""GPU tests of w4a16_gemm_noalloc, the entry point that allocates nothing
(its split-K workspace is the library's static device scratch).

Two calls in a row, the second with a smaller input, each compared bit for
bit with w4a16_gemm on a caller workspace (same kernels, fixed summation
order) and with the oracle within the W4A16 tolerance; the tiled path (no
workspace); and replays of a captured graph against the eager result.
"""

from __future__ import annotations

import pytest
import torch

import mixed_precision_w4a16_repack_amd as w4
import oracle
import w4a16_inputs as wi
from tests.gpu_cases import DEV, oracle_ref, rel_err_rows, repack, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    w4.load_library()
    yield
    torch.cuda.synchronize()


def _run_pair(case, path):
    packed = repack(case)
    A = case.A.to(DEV)
    bias = None if case.bias is None else case.bias.to(DEV)
    out = torch.full((case.M, case.N), 3.0, dtype=case.torch_dtype, device=DEV)
    C_static = w4.gemm_noalloc(A, packed, case.N, case.K, case.G, case.qtype, bias=bias, out=out, path=path)
    C_ws = w4.gemm(A, packed, case.N, case.K, case.G, case.qtype, bias=bias, path=path)
    torch.cuda.synchronize()
    return C_static, C_ws


# (M, N, K, G, qtype, dtype): the first splits K over workgroups of the
# register kernel (1 MiB of partial sums), the second, smaller one runs the
# split-K kernel of narrow weights; both use the scratch.
SEQUENCE = [(16, 4096, 14336, 128, wi.UINT4B8, "f16"), (5, 1024, 4096, 64, wi.UINT4, "bf16")]


def test_two_calls_in_a_row_match_the_workspace_entry_point():
    for i, (M, N, K, G, qt, dt) in enumerate(SEQUENCE):
        print(f"[case] noalloc call {i}: M={M} N={N} K={K} G={G} qtype={qt} {dt}", flush=True)
        assert w4.workspace_size(M, N, K, G, w4.PATH_AUTO) > 0, "the case must use the split-K workspace"
        case = wi.make_case(61, M, N, K, G, qt, dt, with_bias=True)
        C_static, C_ws = _run_pair(case, w4.PATH_AUTO)
        assert torch.equal(C_static.view(torch.int16), C_ws.view(torch.int16))
        rows = sample_rows(M)
        err = rel_err_rows(C_static, oracle_ref(case, rows=rows), rows)
        assert err <= oracle.TOLERANCE[dt], f"rel err {err:.3e}"


# The medium-M tiles split K over workgroups with their partial tiles in the
# scratch (the first exactly fills its 8 MiB): two calls in a row, the second
# smaller, the same split as with a caller workspace.
SPLIT_K_SEQUENCE = [(64, 4096, 4096, 64, wi.UINT4B8, "f16"), (32, 4096, 4096, 32, wi.UINT4, "bf16")]


def test_split_k_tiles_two_calls_in_a_row():
    for i, (M, N, K, G, qt, dt) in enumerate(SPLIT_K_SEQUENCE):
        print(f"[case] noalloc split-K tiles call {i}: M={M} N={N} K={K} G={G} qtype={qt} {dt}", flush=True)
        assert 0 < w4.workspace_size(M, N, K, G, w4.PATH_AUTO) <= 64 * 1024 + (8 << 20)
        case = wi.make_case(64, M, N, K, G, qt, dt, with_bias=True)
        C_static, C_ws = _run_pair(case, w4.PATH_AUTO)
        assert torch.equal(C_static.view(torch.int16), C_ws.view(torch.int16))
        rows = sample_rows(M)
        err = rel_err_rows(C_static, oracle_ref(case, rows=rows), rows)
        assert err <= oracle.TOLERANCE[dt], f"rel err {err:.3e}"


def test_tiled_path_needs_no_scratch():
    case = wi.make_case(62, 96, 512, 1024, 128, wi.UINT4B8, "f16", with_bias=True)
    C_static, C_ws = _run_pair(case, w4.PATH_MFMA)
    assert torch.equal(C_static.view(torch.int16), C_ws.view(torch.int16))


def test_graph_replays_match_eager():
    M, N, K, G = 8, 4096, 14336, 128
    case = wi.make_case(63, M, N, K, G, wi.UINT4B8, "f16")
    packed = repack(case)
    A = case.A.to(DEV)
    eager = w4.gemm_noalloc(A, packed, N, K, G, wi.UINT4B8)
    out = torch.empty_like(eager)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        w4.gemm_noalloc(A, packed, N, K, G, wi.UINT4B8, out=out)
    for rep in range(3):
        out.fill_(0.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep} differs"
        # eager work on the same scratch between replays
        w4.gemm_noalloc(A, packed, N, K, G, wi.UINT4B8, out=torch.empty_like(eager))
        torch.cuda.synchronize()
