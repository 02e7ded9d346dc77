"""Build the gfx950 HIP library ``libbigemm.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbigemm.so")
SOURCES = ["bigemm_api.cpp", "bigemm_kernels.hip", "moe_api.cpp", "moe_kernels.hip", "norm_api.cpp",
           "norm_kernels.hip", "attn_api.cpp", "attn_kernels.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 instructions anywhere (the fold and epilogue use plain
    # fp32 adds), no FMA contraction, no fast-math reassociation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off",
    # keep MFMA accumulators in VGPRs: avoids AGPR round trips in the chains
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


# AddressSanitizer on the host code only (argument checks, handles, the pin
# table parser); the device code is built exactly as in the product library.
ASAN_HOST_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer -shared-libsan".split()


def asan_runtime() -> str:
    """The sanitizer runtime hipcc links the host code against (to preload
    into a Python process that loads the sanitized library)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the host AddressSanitizer runtime was not found")
    return path


def build(verbose: bool = False, asan: bool = False, out: str | None = None, check_asm: bool = True) -> str:
    """Compile every source into libbigemm.so (always recompiles), then check
    the built code of the four-wave kernels (asm_check).  asan: a copy with
    the host code under AddressSanitizer, at `out`, for the CPU ABI tests."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    target = out or LIB
    tmp = target + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *(ASAN_HOST_FLAGS if asan else []), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, target)
    if check_asm and not asan:
        from . import asm_check

        problems = asm_check.problems(asm_check.assemble(target + ".s"))
        os.remove(target + ".s")
        if problems:
            raise RuntimeError("the built four-wave kernels fail their code checks:\n  " + "\n  ".join(problems))
        if verbose:
            print("built-code checks of the four-wave kernels: ok")
    return target


if __name__ == "__main__":
    if __package__ in (None, ""):
        sys.path.insert(0, os.path.dirname(HERE))
        from invariant_bi_gemm_amd import build as _self

        print(_self.build(verbose=True))
    else:
        print(build(verbose=True))
