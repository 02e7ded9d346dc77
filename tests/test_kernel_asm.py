"""The built code of the four-wave kernels (dense 256x256 and 128x256
blocks, grouped), checked on the CPU (not gpu).

The checks live in invariant_bi_gemm_amd.asm_check, which every build also
runs; the tests here run each one on its own, and show that they catch the
mistakes they are for on hand-made assembly.
"""
import os
import shutil

import pytest

from invariant_bi_gemm_amd import asm_check, build

KERNELS = asm_check.KERNELS


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = build.hipcc()
    if not (os.path.isabs(hipcc) and os.path.exists(hipcc)) and shutil.which(hipcc) is None:
        pytest.skip("hipcc not available")
    return asm_check.assemble(str(tmp_path_factory.mktemp("asm") / "bigemm_kernels.s"))


@pytest.mark.parametrize("kernel", KERNELS)
def test_accumulation_registers_only_in_the_chains(asm, kernel):
    assert asm_check.accumulators_only_in_chains(asm, kernel) == []


@pytest.mark.parametrize("kernel", KERNELS)
def test_descriptor_reserves_the_accumulators(asm, kernel):
    assert asm_check.descriptor_reserves_accumulators(asm, kernel) == []


def test_no_kernel_spills_to_scratch(asm):
    assert asm_check.no_kernel_spills(asm) == []


@pytest.mark.parametrize("kernel", KERNELS)
def test_mfma_inputs_not_written_just_before(asm, kernel):
    assert asm_check.mfma_inputs_not_written_just_before(asm, kernel) == []


@pytest.mark.parametrize("kernel", KERNELS)
def test_results_read_after_the_wait_states(asm, kernel):
    assert asm_check.results_read_after_wait_states(asm, kernel) == []


def test_all_checks_together(asm):
    assert asm_check.problems(asm) == []


# hand-made assembly: one kernel whose body has the mistake each check is for
_K = "_ZN6bigemm12_GLOBAL__N_113bigemm_tiled4ILi4ELi0E"


def _fake(lines, nv=384, acc=128, scratch=0):
    body = "\n".join("\t" + l for l in lines)
    return ("%s_fake:\n%s\n.Lfunc_end0:\n.amdhsa_kernel %s_fake\n\t.amdhsa_next_free_vgpr %d\n"
            "\t.amdhsa_accum_offset %d\n\t.amdhsa_private_segment_fixed_size %d\n.end_amdhsa_kernel\n"
            % (_K, body, _K, nv, acc, scratch))


def _good_lines():
    mf = ["v_mfma_f32_16x16x32_bf16 a[%d:%d], v[0:3], v[4:7], a[%d:%d]" % (4 * t, 4 * t + 3, 4 * t, 4 * t + 3)
          for t in range(32)]
    return mf * 2 + ["s_nop 7", "s_nop 7", "s_nop 7"] + ["v_accvgpr_read_b32 v%d, a%d" % (8 + i, i) for i in range(128)]


def test_checks_pass_on_sound_fake():
    a = _fake(_good_lines())
    assert asm_check.accumulators_only_in_chains(a, _K) == []
    assert asm_check.results_read_after_wait_states(a, _K) == []
    assert asm_check.descriptor_reserves_accumulators(a, _K) == []
    assert asm_check.mfma_inputs_not_written_just_before(a, _K) == []


def test_checks_catch_planted_mistakes():
    spill = _good_lines()
    spill.insert(5, "v_accvgpr_write_b32 a3, v9")
    assert asm_check.accumulators_only_in_chains(_fake(spill), _K)
    early = _good_lines()
    early = [l for l in early if not l.startswith("s_nop")]
    assert asm_check.results_read_after_wait_states(_fake(early), _K)
    clobber = _good_lines()
    clobber.insert(3, "v_add_u32 v5, v1, v2")
    assert asm_check.mfma_inputs_not_written_just_before(_fake(clobber), _K)
    assert asm_check.descriptor_reserves_accumulators(_fake(_good_lines(), nv=300, acc=128), _K)
    assert asm_check.descriptor_reserves_accumulators(_fake(_good_lines(), scratch=16), _K)
    assert asm_check.no_kernel_spills(_fake(_good_lines(), scratch=16))
