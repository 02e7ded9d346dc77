"""The built code of the four-wave kernels (dense 256x256 and 128x256
blocks, grouped), checked on the CPU.

Its accumulators live in a0..a255, written only by inline-asm MFMAs and read
only by the epilogue; the compiler does not know they are live.  So the
compiled kernel must not touch an accumulation register anywhere else (a
compiler spill or copy into one would corrupt a result), must not spill to
scratch, must leave the MFMA inputs alone right before each MFMA (a vector
write there needs wait states the compiler does not insert for inline asm),
and must wait out the last MFMAs before reading their results.  The checks
read the assembly hipcc emits for gfx950 with the library's own flags.
"""
import os
import re
import shutil
import subprocess

import pytest

from invariant_bi_gemm_amd import build

SRC = os.path.join(build.CSRC, "bigemm_kernels.hip")
# the dense kernels (8 and 4 x tiles per wave) and the grouped one (plain and
# indexed rows; both block heights in one kernel), with the accumulator tiles
# each of their epilogues reads
KERNELS = {"_ZN6bigemm12_GLOBAL__N_113bigemm_tiled4ILi8E": [64],
           "_ZN6bigemm12_GLOBAL__N_113bigemm_tiled4ILi4E": [32],
           "_ZN6bigemm12_GLOBAL__N_121bigemm_tiled4_groupedILb0E": [64, 32],
           "_ZN6bigemm12_GLOBAL__N_121bigemm_tiled4_groupedILb1E": [64, 32]}
MFMA_AGPR = re.compile(r"v_mfma_f32_16x16x32_bf16 a\[\d+:\d+\], v\[\d+:\d+\], v\[\d+:\d+\], (a\[\d+:\d+\]|0)$")
AGPR = re.compile(r"\ba\d+\b|\ba\[\d+:\d+\]")


def vregs(op):
    m = re.match(r"v\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", op)
    return {int(m.group(1))} if m else set()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = build.hipcc()
    if not (os.path.isabs(hipcc) and os.path.exists(hipcc)) and shutil.which(hipcc) is None:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "bigemm_kernels.s")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    res = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", "-o", out, SRC],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return open(out).read()


def body(asm, name):
    m = re.search(r"^(%s\w*):" % name, asm, re.M)
    assert m, "kernel %s not in the assembly" % name
    end = asm.index(".Lfunc_end", m.end())
    lines = []
    for l in asm[m.end():end].splitlines():
        t = l.strip()
        if t and not t.startswith((";", "//", ".")) and not t.endswith(":"):
            lines.append(t)
    return m.group(1), lines


@pytest.mark.parametrize("kernel", KERNELS)
def test_accumulation_registers_only_in_the_chains(asm, kernel):
    _, ins = body(asm, kernel)
    bad = [t for t in ins if AGPR.search(t) and not MFMA_AGPR.match(t)
           and not re.match(r"v_accvgpr_read_b32 v\d+, a\d+$", t)]
    assert not bad, "compiler-placed accumulation-register use: %s" % bad[:5]
    assert sum(1 for t in ins if t.startswith("v_mfma")) >= 2 * sum(KERNELS[kernel])
    assert sum(1 for t in ins if t.startswith("v_accvgpr_read_b32")) == 4 * sum(KERNELS[kernel])


@pytest.mark.parametrize("kernel", KERNELS)
def test_descriptor_reserves_the_accumulators(asm, kernel):
    name, _ = body(asm, kernel)
    d = asm[asm.index(".amdhsa_kernel " + name):]
    d = d[:d.index(".end_amdhsa_kernel")]
    nv = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", d).group(1))
    acc = int(re.search(r"\.amdhsa_accum_offset (\d+)", d).group(1))
    assert nv - acc == 256 and nv <= 512, (nv, acc)
    assert int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", d).group(1)) == 0


def test_no_kernel_spills_to_scratch(asm):
    sizes = re.findall(r"\.amdhsa_kernel (\S+)\n(?:.*\n)*?\s*\.amdhsa_private_segment_fixed_size (\d+)", asm)
    assert sizes
    assert all(int(n) == 0 for _, n in sizes), [k for k, n in sizes if int(n)]


@pytest.mark.parametrize("kernel", KERNELS)
def test_mfma_inputs_not_written_just_before(asm, kernel):
    _, ins = body(asm, kernel)
    for i, t in enumerate(ins):
        if not t.startswith("v_mfma"):
            continue
        ops = [o.strip() for o in t.split(None, 1)[1].split(",")]
        src = vregs(ops[1]) | vregs(ops[2])
        for p in ins[max(0, i - 4):i]:
            if p.startswith("v_") and not p.startswith("v_mfma") and " " in p:
                dst = vregs(p.split(None, 1)[1].split(",")[0].strip())
                assert not dst & src, "vector write right before an MFMA reads it: %r then %r" % (p, t)


@pytest.mark.parametrize("kernel", KERNELS)
def test_results_read_after_the_wait_states(asm, kernel):
    """Each epilogue (a run of result reads with no MFMA inside it) starts at
    least 18 wait states after the MFMA before it, and reads every tile."""
    _, ins = body(asm, kernel)
    runs, last_mfma = [], None
    for i, t in enumerate(ins):
        if t.startswith("v_mfma"):
            last_mfma = i
        elif t.startswith("v_accvgpr_read_b32"):
            if not runs or runs[-1]["mfma"] != last_mfma:
                assert last_mfma is not None, "a result read before any MFMA"
                nops = sum(int(x.split()[1]) + 1 for x in ins[last_mfma + 1:i] if x.startswith("s_nop"))
                assert nops >= 18, "only %d wait states between the last MFMA and a first result read" % nops
                runs.append({"mfma": last_mfma, "reads": 0})
            runs[-1]["reads"] += 1
    assert sorted(r["reads"] for r in runs) == sorted(4 * n for n in KERNELS[kernel])
