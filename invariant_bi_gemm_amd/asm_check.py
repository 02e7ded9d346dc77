"""Checks on the built code of the four-wave kernels (dense 256x256,
192x256, 160x256 and 128x256 blocks, grouped), run on the CPU by every build.

Their accumulators live in a0..a255, written only by inline-asm MFMAs and
read only by the epilogue; the compiler does not know they are live.  So the
compiled kernel must not touch an accumulation register anywhere else (a
compiler spill or copy into one would corrupt a result), must not spill to
scratch, must leave the MFMA inputs alone right before each MFMA (a vector
write there needs wait states the compiler does not insert for inline asm),
and must wait out the last MFMAs before reading their results.  The checks
read the assembly hipcc emits for gfx950 with the library's own flags.
"""
from __future__ import annotations

import os
import re
import subprocess

from . import build

SRC = os.path.join(build.CSRC, "bigemm_kernels.hip")
# the dense kernels (8, 6, 5 and 4 x tiles per wave; the product instance and the
# comparison path's split-K instance) and the grouped one (plain and indexed
# rows, and the gated projection's SwiGLU epilogue; both block heights in one
# kernel), with the accumulator tiles each of their epilogues reads
KERNELS = {"_ZN6bigemm12_GLOBAL__N_113bigemm_tiled4ILi8ELi0E": [64],
           "_ZN6bigemm12_GLOBAL__N_113bigemm_tiled4ILi4ELi0E": [32],
           "_ZN6bigemm12_GLOBAL__N_113bigemm_tiled4ILi8ELi1E": [64],
           "_ZN6bigemm12_GLOBAL__N_113bigemm_tiled4ILi4ELi1E": [32],
           "_ZN6bigemm12_GLOBAL__N_113bigemm_tiled4ILi5ELi0E": [40],
           "_ZN6bigemm12_GLOBAL__N_113bigemm_tiled4ILi5ELi1E": [40],
           "_ZN6bigemm12_GLOBAL__N_113bigemm_tiled4ILi6ELi0E": [48],
           "_ZN6bigemm12_GLOBAL__N_113bigemm_tiled4ILi6ELi1E": [48],
           "_ZN6bigemm12_GLOBAL__N_121bigemm_tiled4_groupedILb0ELb0ELb0E": [64, 32],
           "_ZN6bigemm12_GLOBAL__N_121bigemm_tiled4_groupedILb1ELb0ELb0E": [64, 32],
           "_ZN6bigemm12_GLOBAL__N_121bigemm_tiled4_groupedILb1ELb1ELb0E": [64, 32],
           # the same with non-temporal W loads
           "_ZN6bigemm12_GLOBAL__N_121bigemm_tiled4_groupedILb0ELb0ELb1E": [64, 32],
           "_ZN6bigemm12_GLOBAL__N_121bigemm_tiled4_groupedILb1ELb0ELb1E": [64, 32],
           "_ZN6bigemm12_GLOBAL__N_121bigemm_tiled4_groupedILb1ELb1ELb1E": [64, 32]}
MFMA_AGPR = re.compile(r"v_mfma_f32_16x16x32_bf16 a\[\d+:\d+\], v\[\d+:\d+\], v\[\d+:\d+\], (a\[\d+:\d+\]|0)$")
AGPR = re.compile(r"\ba\d+\b|\ba\[\d+:\d+\]")


def assemble(out_path: str, src: str = SRC) -> str:
    """gfx950 device assembly of `src` with the library's flags."""
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    res = subprocess.run([build.hipcc(), *flags, "--cuda-device-only", "-S", "-o", out_path, src],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc -S failed:\n" + res.stderr[-3000:])
    with open(out_path) as f:
        return f.read()


def vregs(op):
    m = re.match(r"v\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", op)
    return {int(m.group(1))} if m else set()


def body(asm, name):
    """(mangled name, instruction lines) of the kernel whose name starts with `name`."""
    m = re.search(r"^(%s\w*):" % name, asm, re.M)
    if not m:
        raise ValueError("kernel %s not in the assembly" % name)
    end = asm.index(".Lfunc_end", m.end())
    lines = []
    for l in asm[m.end():end].splitlines():
        t = l.strip()
        if t and not t.startswith((";", "//", ".")) and not t.endswith(":"):
            lines.append(t)
    return m.group(1), lines


def accumulators_only_in_chains(asm, kernel):
    _, ins = body(asm, kernel)
    bad = [t for t in ins if AGPR.search(t) and not MFMA_AGPR.match(t)
           and not re.match(r"v_accvgpr_read_b32 v\d+, a\d+$", t)]
    out = []
    if bad:
        out.append("%s: compiler-placed accumulation-register use: %s" % (kernel, bad[:5]))
    if sum(1 for t in ins if t.startswith("v_mfma")) < 2 * sum(KERNELS[kernel]):
        out.append("%s: fewer MFMAs than accumulator tiles" % kernel)
    reads = sum(1 for t in ins if t.startswith("v_accvgpr_read_b32"))
    if reads != 4 * sum(KERNELS[kernel]):
        out.append("%s: %d result reads, expected %d" % (kernel, reads, 4 * sum(KERNELS[kernel])))
    return out


def descriptor_reserves_accumulators(asm, kernel):
    name, _ = body(asm, kernel)
    d = asm[asm.index(".amdhsa_kernel " + name):]
    d = d[:d.index(".end_amdhsa_kernel")]
    nv = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", d).group(1))
    acc = int(re.search(r"\.amdhsa_accum_offset (\d+)", d).group(1))
    scratch = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", d).group(1))
    out = []
    if not (nv - acc == 256 and nv <= 512):
        out.append("%s: descriptor reserves %d accumulation registers (next_free_vgpr %d, accum_offset %d)"
                   % (kernel, nv - acc, nv, acc))
    if scratch:
        out.append("%s: %d bytes of scratch" % (kernel, scratch))
    return out


def no_kernel_spills(asm):
    sizes = re.findall(r"\.amdhsa_kernel (\S+)\n(?:.*\n)*?\s*\.amdhsa_private_segment_fixed_size (\d+)", asm)
    if not sizes:
        return ["no kernel descriptors found"]
    return ["%s spills %s bytes to scratch" % (k, n) for k, n in sizes if int(n)]


def mfma_inputs_not_written_just_before(asm, kernel):
    _, ins = body(asm, kernel)
    out = []
    for i, t in enumerate(ins):
        if not t.startswith("v_mfma"):
            continue
        ops = [o.strip() for o in t.split(None, 1)[1].split(",")]
        src = vregs(ops[1]) | vregs(ops[2])
        for p in ins[max(0, i - 4):i]:
            if p.startswith("v_") and not p.startswith("v_mfma") and " " in p:
                dst = vregs(p.split(None, 1)[1].split(",")[0].strip())
                if dst & src:
                    out.append("%s: vector write right before an MFMA reads it: %r then %r" % (kernel, p, t))
    return out


def results_read_after_wait_states(asm, kernel):
    """Each epilogue (a run of result reads with no MFMA inside it) starts at
    least 18 wait states after the MFMA before it, and reads every tile."""
    _, ins = body(asm, kernel)
    runs, last_mfma = [], None
    out = []
    for i, t in enumerate(ins):
        if t.startswith("v_mfma"):
            last_mfma = i
        elif t.startswith("v_accvgpr_read_b32"):
            if not runs or runs[-1]["mfma"] != last_mfma:
                if last_mfma is None:
                    return ["%s: a result read before any MFMA" % kernel]
                nops = sum(int(x.split()[1]) + 1 for x in ins[last_mfma + 1:i] if x.startswith("s_nop"))
                if nops < 18:
                    out.append("%s: only %d wait states between the last MFMA and a first result read"
                               % (kernel, nops))
                runs.append({"mfma": last_mfma, "reads": 0})
            runs[-1]["reads"] += 1
    if sorted(r["reads"] for r in runs) != sorted(4 * n for n in KERNELS[kernel]):
        out.append("%s: epilogue reads %s, expected %s" % (
            kernel, sorted(r["reads"] for r in runs), sorted(4 * n for n in KERNELS[kernel])))
    return out


CHECKS = (accumulators_only_in_chains, descriptor_reserves_accumulators, mfma_inputs_not_written_just_before,
          results_read_after_wait_states)


def problems(asm: str):
    """Every failed check, as messages (empty: the built code is sound)."""
    out = no_kernel_spills(asm)
    for kernel in KERNELS:
        for check in CHECKS:
            out += check(asm, kernel)
    return out
