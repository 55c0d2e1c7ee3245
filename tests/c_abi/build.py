"""Builds tests/c_abi/c_abi_check (test infrastructure): a plain C program
that calls libgemm_epi.so through include/gemm_epi.h and compares with the
CPU oracle (liboracle.so).  Host compiler only (gcc); the HIP runtime's C API
comes from /opt/rocm."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "c_abi_check.c")
EXE = os.path.join(HERE, "c_abi_check")
PKG = os.path.join(ROOT, "dense_gemm_elementwise_amd")
ORACLE = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out=EXE):
    return ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-o", out, SRC,
            "-L", PKG, "-lgemm_epi", "-L", ORACLE, "-loracle", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
            "-Wl,-rpath,$ORIGIN/../../dense_gemm_elementwise_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
            f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]


def build(verbose: bool = False) -> str:
    cmd = command()
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
