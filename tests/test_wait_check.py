"""CPU tests of the build check on hand-counted memory waits (wait_check).

The check reads gfx950 assembly; here it runs on small hand-written
listings whose counts are known (a matching pipeline, a dropped load, an
extra load on one branch, loads reordered across the last direct-to-LDS
load, a prologue that issues more stages than it waits for) and on the
assembly of the committed kernel sources. The same holds for the MFMA
operand check (an inline-asm VALU result read by an MFMA too soon).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil

import pytest

from mixed_precision_w4a16_repack_amd import build as lib_build
from mixed_precision_w4a16_repack_amd import wait_check

WAIT = "\t;;#ASMSTART\n\ts_waitcnt vmcnt({n})\n\t;;#ASMEND\n"
BARRIER = "\t;;#ASMSTART\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier\n\t;;#ASMEND\n"
LDS = "\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds\n"
REG = "\tbuffer_load_dwordx4 v[2:5], v1, s[4:7], 0 offen\n"


def listing(name: str, body: str) -> str:
    return f"{name}:\n{body}\ts_endpgm\n.Lfunc_end0:\n"


RING = "_Z16mfma_ring_kernelv"
LDSK = "_Z15mfma_lds_kernelv"
A8 = "_Z16w4a8_ring_kernelv"


def ring_loop(step_loads: str, n: int, extra_branch: str = "") -> str:
    prologue = LDS * 2 * n + WAIT.format(n=n) + BARRIER
    loop = (".LBB0_1:\n" + step_loads + extra_branch + WAIT.format(n=n) + BARRIER +
            "\ts_cbranch_scc1 .LBB0_1\n")
    return prologue + loop


def problems(name: str, body: str):
    n, probs = wait_check.check_asm(listing(name, body))
    assert n == 1
    return probs


def test_matching_ring_pipeline_passes():
    assert problems(RING, ring_loop(LDS * 3 + REG * 2, 5)) == []


def test_dropped_load_is_found():
    # five loads counted, four emitted (a dead register load dropped)
    probs = problems(RING, ring_loop(LDS * 3 + REG, 5))
    assert probs and "vmcnt(5) but 4" in probs[0]


def test_extra_load_on_one_branch_is_found():
    branch = ("\ts_cbranch_execz .LBB0_3\n" + REG + ".LBB0_3:\n")
    probs = problems(RING, ring_loop(LDS * 3 + REG * 2, 5, extra_branch=branch))
    assert any("but 6" in p for p in probs)


def test_prologue_needs_only_at_least_n():
    body = LDS * 4 + WAIT.format(n=2) + BARRIER
    assert problems(RING, body) == []
    body = LDS * 1 + WAIT.format(n=2) + BARRIER
    assert problems(RING, body) != []


def test_lds_rule_counts_after_the_last_direct_load():
    ok = LDS * 4 + REG * 2 + WAIT.format(n=2) + BARRIER
    assert problems(LDSK, ok) == []
    # a register load scheduled between the direct loads: one fewer after the last
    mixed = LDS * 3 + REG + LDS + REG + WAIT.format(n=2) + BARRIER
    probs = problems(LDSK, mixed)
    assert probs and "vmcnt(2) but 1" in probs[0]


def test_w4a8_rule_spans_two_steps():
    step = LDS * 2 + REG
    body = (LDS * 9 + WAIT.format(n=6) + BARRIER + ".LBB0_1:\n" + step + WAIT.format(n=6) + BARRIER +
            step + WAIT.format(n=6) + BARRIER + "\ts_cbranch_scc1 .LBB0_1\n")
    assert problems(A8, body) == []
    short = LDS * 2
    body = (LDS * 9 + WAIT.format(n=6) + BARRIER + ".LBB0_1:\n" + step + WAIT.format(n=6) + BARRIER +
            short + WAIT.format(n=6) + BARRIER + "\ts_cbranch_scc1 .LBB0_1\n")
    assert any("but 5" in p for p in problems(A8, body))


def test_kernel_without_hand_wait_is_reported():
    assert problems(RING, LDS + BARRIER) != []


def test_other_kernels_are_ignored():
    n, probs = wait_check.check_asm(listing("_Z12skinny_kernelv", LDS + WAIT.format(n=3) + BARRIER))
    assert n == 0 and probs == []


# MFMA operand hazard: an inline-asm VALU result read by an MFMA needs 2
# wait states first.
ASM_AND_OR = "\t;;#ASMSTART\n\tv_and_or_b32 v58, v37, v63, v65\n\t;;#ASMEND\n"
MFMA = "\tv_mfma_f32_16x16x32_f16 v[50:53], v[14:17], v[58:61], v[50:53]\n"


def hazards(body: str):
    return wait_check.mfma_operand_hazards(listing("_Z18skinny_reg_kernelv", body))


def test_asm_result_read_one_wait_state_later_is_found():
    probs = hazards(ASM_AND_OR + "\ts_nop 0\n" + MFMA)
    assert probs and "after 1 wait states" in probs[0]


def test_asm_result_read_at_once_is_found():
    assert hazards(ASM_AND_OR + MFMA)


def test_two_wait_states_or_other_registers_pass():
    assert hazards(ASM_AND_OR + "\ts_nop 1\n" + MFMA) == []
    assert hazards(ASM_AND_OR + "\tv_add_u32_e32 v1, 4, v0\n\tv_add_u32_e32 v2, 4, v0\n" + MFMA) == []
    other = ASM_AND_OR.replace("v58", "v70")
    assert hazards(other + MFMA) == []


def test_compiler_emitted_valu_is_left_to_the_compiler():
    assert hazards("\tv_and_or_b32 v58, v37, v63, v65\n" + MFMA) == []


def test_accumulator_operand_is_checked_too():
    acc = ASM_AND_OR.replace("v58", "v51")
    assert hazards(acc + MFMA)


ASM_SHIFT = "\t;;#ASMSTART\n\tv_lshlrev_b64 v[50:51], 2, v[114:115]\n\t;;#ASMEND\n"


def test_asm_write_of_a_register_an_mfma_just_read_is_found():
    probs = hazards(MFMA + ASM_SHIFT)
    assert probs and "writes a register an MFMA read 0 wait states before" in probs[0]
    assert hazards(MFMA + "\ts_nop 7\n" * 2 + ASM_SHIFT) == []
    assert hazards(MFMA + ASM_SHIFT.replace("v[50:51]", "v[80:81]")) == []


needs_hipcc = pytest.mark.skipif(not os.path.exists(lib_build.HIPCC) and shutil.which("hipcc") is None,
                                 reason="needs hipcc")


@pytest.fixture(scope="module")
def committed_assembly():
    """gfx950 assembly of every committed source with MFMA kernels, compiled
    once for the tests below (in parallel)."""
    os.makedirs(lib_build.BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(lib_build.ASSEMBLED)) as ex:
        return dict(zip(lib_build.ASSEMBLED, ex.map(lib_build._assembly, lib_build.ASSEMBLED)))


@needs_hipcc
def test_committed_kernels_pass(committed_assembly):
    lib_build.check_waits([committed_assembly[s] for s in lib_build.STAGED])


@needs_hipcc
def test_committed_kernels_have_no_mfma_operand_hazard(committed_assembly):
    lib_build.check_mfma_operands(list(committed_assembly.values()))
