"""The matrix-core attention kernel's inline-asm MFMAs respect the MFMA
dependency rules in the code the compiler actually emits.

The output accumulators are updated by inline-asm MFMAs the compiler's hazard
recognizer does not see, so this test compiles the kernel to gfx950 assembly
with the library's own options and checks every path with
tree_verify_mla_amd.isa_check (result registers untouched for 11 wait states
except by the next accumulation; no VALU write of an operand within 2 wait
states before an MFMA).  The checker itself is exercised on a planted
violation.
"""
import shutil

import pytest

from tree_verify_mla_amd import build, isa_check

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not build.Path("/opt/rocm/bin/hipcc").exists(),
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "verify_attn_bf16.s"
    build.device_asm("verify_attn_bf16.hip", out)
    return out.read_text()


@pytest.mark.parametrize("instance", ["attn_bf16_kernelILb1", "attn_bf16_kernelILb0"])
def test_attention_kernel_has_no_mfma_hazards(kernel_asm, instance):
    problems, n = isa_check.check(kernel_asm, instance)
    assert n >= 68, "expected the score and value MFMAs of the block loop"
    assert not problems, "\n".join(problems[:10])


PLANTED = """
k:
	v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]
	v_mfma_f32_32x32x16_bf16 v[0:15], v[24:27], v[28:31], v[0:15]
	s_nop 3
	v_mov_b32_e32 v40, v3
	v_add_f32_e32 v20, v41, v42
	v_mfma_f32_32x32x16_bf16 a[0:15], v[16:19], v[20:23], a[0:15]
	s_endpgm
.Lfunc_end0:
"""


def test_checker_flags_planted_violations():
    problems, n = isa_check.check(PLANTED, "k")
    assert n == 3
    # v3 read 4 wait states after the second MFMA; v20 written right before the third
    assert any("v_mov_b32_e32 v40, v3" in p for p in problems)
    assert any("v_add_f32_e32 v20" in p for p in problems)
    # back-to-back accumulation into the same registers is allowed
    assert not any("v_mfma_f32_32x32x16_bf16 v[0:15], v[24:27]" in p.split(" touches")[0] for p in problems)
