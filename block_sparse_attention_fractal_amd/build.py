"""Build libnabla.so (all HIP kernels + the C ABI) for gfx950, in-tree.

``python -m block_sparse_attention_fractal_amd.build`` compiles every
``csrc/*.hip`` with hipcc into ``block_sparse_attention_fractal_amd/libnabla.so``.

Flags:
  -ffp-contract=off   the estimator's fp32 rounding order is fixed; the only
                      fused multiply-adds are explicit ``__builtin_fmaf`` calls;
  -packed-fp32-ops    off: packed fp32 VALU forms are not emitted;
  -amdgpu-mfma-vgpr-form=1
                      MFMAs written as builtins take their accumulators in VGPRs
                      (the score products, which VALU code reads); accumulators
                      meant to stay in AGPRs use inline-asm MFMAs.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnabla.so")
ARCH = os.environ.get("NABLA_OFFLOAD_ARCH", "gfx950")

HIPFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPFLAGS, *extra, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + errs)
    if verbose and errs.strip():
        print(errs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
