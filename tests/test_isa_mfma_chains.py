"""The built library's gfx950 code has no dependent MFMA chain that mixes instructions.

When an MFMA takes the result of an earlier MFMA as its accumulator in the same registers, the
compiler may issue it with no wait between them, whatever the two instructions are; chains of one
instruction are exact, and chains that mixed 16x16x32 and 16x16x16 products gave wrong values.
The kernels keep one instruction per chain (each MFMA family has its own accumulator type); this
test reads the library's machine code and checks the rule where it matters, after compilation.
"""
import os
import shutil

import pytest

from linear_rnn_amd import wkv
from tests import isa_lint

pytestmark = pytest.mark.skipif(not shutil.which(os.path.join(isa_lint.LLVM, "llvm-objdump")),
                                reason="ROCm LLVM tools not installed")


def _parse(body):
    return isa_lint.functions("0000000000000000 <f>:\n" + "".join("\t" + l.strip() + "\n"
                                                                      for l in body.strip().splitlines()))["f"]


def test_lint_flags_a_mixed_accumulator_chain():
    insts = _parse("""
        v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0
        v_mov_b32 v20, v21
        v_mfma_f32_16x16x16_f16 v[0:3], v[12:13], v[14:15], v[0:3]
    """)
    found = isa_lint.mixed_accumulator_chains(insts)
    assert [(r, w) for _, r, w, _ in found] == [("v_mfma_f32_16x16x16_f16", "v_mfma_f32_16x16x32_f16")]
    assert found[0][3] == 1  # one instruction between them
    # bf16 Gram result as the accumulator of an f16 product: also mixed
    insts = _parse("""
        v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], 0
        v_mfma_f32_16x16x16_f16 a[0:3], v[12:13], v[14:15], a[0:3]
    """)
    assert len(isa_lint.mixed_accumulator_chains(insts)) == 1


def test_lint_accepts_one_instruction_chains_and_rewritten_registers():
    same = _parse("""
        v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0
        v_mfma_f32_16x16x32_f16 v[0:3], v[12:15], v[16:19], v[0:3]
    """)
    assert isa_lint.mixed_accumulator_chains(same) == []
    # the accumulator rewritten by the vector unit in between: no MFMA-to-MFMA dependency
    via_valu = _parse("""
        v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0
        v_add_f32_e32 v0, v0, v20
        v_add_f32_e32 v1, v1, v20
        v_add_f32_e32 v2, v2, v20
        v_add_f32_e32 v3, v3, v20
        v_mfma_f32_16x16x16_f16 v[0:3], v[12:13], v[14:15], v[0:3]
    """)
    assert isa_lint.mixed_accumulator_chains(via_valu) == []
    # the result read as an A/B operand (the compiler waits for that) is not an accumulator chain
    as_operand = _parse("""
        v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0
        v_cvt_pk_f16_f32 v12, v0, v1
        v_cvt_pk_f16_f32 v13, v2, v3
        v_mfma_f32_16x16x16_f16 v[20:23], v[12:13], v[14:15], 0
    """)
    assert isa_lint.mixed_accumulator_chains(as_operand) == []


def test_lint_sees_a_chain_carried_around_a_loop():
    # the accumulator of the first product at the loop's top was last written by the other
    # instruction at the loop's bottom, on the previous iteration
    insts = _parse("""
        v_mfma_f32_16x16x16_f16 v[0:3], v[12:13], v[14:15], v[0:3]
        v_mov_b32 v30, v31
        v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], v[0:3]
        s_cbranch_scc1 65530
    """)
    found = isa_lint.mixed_accumulator_chains(insts)
    assert ("v_mfma_f32_16x16x16_f16", "v_mfma_f32_16x16x32_f16") in [(r, w) for _, r, w, _ in found]


def test_built_library_has_no_mixed_mfma_chain(tmp_path):
    path = wkv.LIB_PATH
    assert os.path.exists(path), "build the library first"
    texts = isa_lint.disassemble(path, str(tmp_path))
    with_mfma, bad = [], []
    for t in texts:
        for name, insts in isa_lint.functions(t).items():
            n = sum(1 for mn, _ in insts if mn.startswith("v_mfma"))
            if n:
                with_mfma.append(name)
                bad += [(name, f) for f in isa_lint.mixed_accumulator_chains(insts)]
    # the chunked kernels are there and use MFMA (so the check is not vacuous)
    for k in ("wkv7_fused_kernel", "wkv7_prep_kernel", "wkv7_scan_kernel"):
        assert any(k in n for n in with_mfma), k
    assert bad == []
