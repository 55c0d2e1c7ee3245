"""Builds libgemm_epi.so (the HIP kernels and the C ABI) for gfx950, in-tree.

hipcc compiles the translation units csrc/gemm_epi.hip (the C ABI and the
fp16 kernels), csrc/gemm_epi_bf16.hip (the bfloat16 kernels) and
csrc/gemm_epi_f32e.hip, csrc/gemm_epi_bf16_f32e.hip (fp16 / bfloat16 A and B
with fp32 epilogue tensors) and csrc/gemm_epi_f16_bf16e.hip,
csrc/gemm_epi_bf16_f16e.hip (the other 16-bit type for the epilogue tensors)
in parallel for --offload-arch=gfx950 only, then links them into one shared
library.
Packed-fp32 VALU instructions are switched off (-packed-fp32-ops): the
epilogue is plain scalar fp32 arithmetic.
"""
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("gemm_epi.hip", "gemm_epi_bf16.hip", "gemm_epi_f32e.hip",
                                               "gemm_epi_bf16_f32e.hip", "gemm_epi_f16_bf16e.hip",
                                               "gemm_epi_bf16_f16e.hip")]
LIB = os.path.join(PKG, "libgemm_epi.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgemm_epi.so)")


def build(verbose: bool = False) -> str:
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
    objs = [LIB + f".{i}.o" for i in range(len(SRCS))]
    procs = []
    for src, obj in zip(SRCS, objs):
        cmd = [hipcc(), *flags, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
    failed = [cmd for cmd, proc in procs if proc.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    link = [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    for obj in objs:
        os.remove(obj)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
