"""The MFMAs are issued through inline asm, so the compiler inserts no wait
states for them; check the generated gfx950 code for the MFMA hazards instead.
CPU-only: it compiles the kernels to assembly, it runs nothing."""
import os
import re
import shutil

import pytest

from speculative_decode_mla_amd import build
from tests import asm_hazards

KERNELS = os.path.join(build.HERE, "csrc", "mla_verify_kernels.hip")
FUNCTIONS = ["_ZN4mlav18mla_verify_partialILb0EEEvPKiS2_iiiiiNS_11PartialArgsE",  # per-request splits
             "_ZN4mlav18mla_verify_partialILb1EEEvPKiS2_iiiiiNS_11PartialArgsE",  # range plan
             "_ZN4mlav21mla_verify_partial_2sEPKiS1_iiiiiNS_11PartialArgsE",
             "_ZN4mlav21mla_verify_partial_4sEPKiS1_iiiiiNS_11PartialArgsE"]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "kernels.s"
    build.device_asm(KERNELS, str(out))
    return out.read_text()


@pytest.mark.parametrize("fn", FUNCTIONS)
def test_no_mfma_hazards(asm, fn):
    insns, labels = asm_hazards.parse_function(asm, fn)
    assert sum(asm_hazards.is_mfma(x) for x in insns) >= 68  # the whole main loop was parsed
    problems = asm_hazards.check(insns, labels)
    assert not problems, "\n".join(problems[:20])


@pytest.mark.parametrize("fn", FUNCTIONS)
def test_no_scratch(asm, fn):
    """No kernel-1 form spills to scratch (a spill, or a register array the compiler could not keep in
    registers, would be private memory traffic inside the step loop)."""
    seg = asm[asm.index(fn + ":"):]
    m = re.search(r"; ScratchSize: (\d+)", seg)
    assert m is not None and int(m.group(1)) == 0, m.group(0) if m else "no ScratchSize line"


@pytest.mark.parametrize("fn", FUNCTIONS)
def test_untracked_loads_awaited_before_use(asm, fn):
    insns, _ = asm_hazards.parse_function(asm, fn)
    loads = [x for x in insns if x.inline_asm and x.op.startswith("global_load_dword")]
    assert len(loads) >= 2  # the prologue's slot indices were found
    problems = asm_hazards.check_untracked_loads(insns)
    assert not problems, "\n".join(problems[:20])


def test_untracked_load_checker_flags_early_use():
    def run(text):
        src = "f:\n" + "\n".join("\t" + l for l in text) + "\n.Lfunc_end0:\n"
        insns, _ = asm_hazards.parse_function(src, "f")
        return asm_hazards.check_untracked_loads(insns)

    ld = [";;#ASMSTART", "global_load_dwordx4 v[4:7], v[0:1], off", ";;#ASMEND"]
    other = "global_load_dword v8, v[2:3], off"
    assert not run(ld + [other, "s_waitcnt vmcnt(1)", "v_mov_b32 v9, v5", "s_endpgm"])
    assert run(ld + [other, "s_waitcnt vmcnt(2)", "v_mov_b32 v9, v5", "s_waitcnt vmcnt(0)", "s_endpgm"])
    assert run(ld + ["v_mov_b32 v9, v6", "s_waitcnt vmcnt(0)", "s_endpgm"])     # read before the wait
    assert run(ld + ["v_mov_b32 v7, 0", "s_waitcnt vmcnt(0)", "s_endpgm"])      # overwritten before the wait
    assert run(ld + ["s_cbranch_scc1 .LBB0_1", ".LBB0_1:", "s_waitcnt vmcnt(0)", "s_endpgm"])
    assert run(ld + ["s_endpgm"])                                                # never awaited
    assert not run(["global_load_dwordx4 v[4:7], v[0:1], off", "v_mov_b32 v9, v5"])  # compiler-issued: not checked


def test_checker_flags_planted_hazards():
    """The checker itself: each rule fires on a minimal sequence and stays quiet when padded."""
    def run(text):
        src = "f:\n" + "\n".join("\t" + l for l in text) + "\n.Lfunc_end0:\n"
        insns, labels = asm_hazards.parse_function(src, "f")
        return asm_hazards.check(insns, labels)

    mf = "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]"
    assert run(["v_mov_b32 v17, 0", mf, "s_nop 7", "s_nop 7", "s_nop 7"])      # VALU -> A operand
    assert not run(["v_mov_b32 v17, 0", "s_nop 3", mf, "s_nop 7", "s_nop 7", "s_nop 7"])
    assert run([mf, "s_nop 7", "v_add_f32 v30, v3, v4"])                         # result read too early
    assert not run([mf, "s_nop 7", "s_nop 7", "s_nop 7", "v_add_f32 v30, v3, v4"])
    assert run([mf, "v_mfma_f32_32x32x16_bf16 v[32:47], v[0:3], v[20:23], v[32:47]", "s_nop 7", "s_nop 7", "s_nop 7"])
    assert not run([mf, mf, "s_nop 7", "s_nop 7", "s_nop 7"])                   # accumulate chain is fine
    assert run(["v_exp_f32 v40, v41", "v_cvt_pk_bf16_f32 v42, v40, v43"])       # trans result read at once
    assert not run(["v_exp_f32 v40, v41", "s_nop 0", "v_cvt_pk_bf16_f32 v42, v40, v43"])
    # across a branch: the write sits before the label, the MFMA after it
    assert run(["v_mov_b32 v20, 0", "s_cbranch_scc1 .LBB0_1", "s_nop 0", ".LBB0_1:", mf,
                "s_nop 7", "s_nop 7", "s_nop 7"])
