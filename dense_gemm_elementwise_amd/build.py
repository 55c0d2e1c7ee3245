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

Every kernel's register use is taken from the compiler's resource remarks
and written to libgemm_epi.resources.json beside the library; the build fails
if any kernel spills to scratch memory (a spill is a slow global-memory round
trip inside the main loop or the epilogue).
"""
import json
import os
import re
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("gemm_epi.hip", "gemm_epi_bf16.hip", "gemm_epi_f32e.hip",
                                               "gemm_epi_bf16_f32e.hip", "gemm_epi_f16_bf16e.hip",
                                               "gemm_epi_bf16_f16e.hip")]
LIB = os.path.join(PKG, "libgemm_epi.so")
RESOURCES = os.path.join(PKG, "libgemm_epi.resources.json")
ARCH = "gfx950"

_REMARK = re.compile(r"remark: +(Function Name|VGPRs|AGPRs|ScratchSize|Occupancy|VGPRs Spill|SGPRs Spill)"
                     r"(?: \[[^\]]*\])?: (\S+) \[-Rpass-analysis=kernel-resource-usage\]")


def parse_resources(text: str) -> list:
    """Kernel resource records from the compiler's kernel-resource-usage remarks."""
    out, cur = [], None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = {"kernel": val}
            out.append(cur)
        elif cur is not None:
            cur[key] = int(val)
    return out


def spilling(resources: list) -> list:
    return [r for r in resources
            if r.get("ScratchSize", 0) > 0 or r.get("VGPRs Spill", 0) > 0 or r.get("SGPRs Spill", 0) > 0]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgemm_epi.so)")


def build(verbose: bool = False) -> str:
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", "-Rpass-analysis=kernel-resource-usage"]
    objs = [LIB + f".{i}.o" for i in range(len(SRCS))]
    procs = []
    for src, obj in zip(SRCS, objs):
        cmd = [hipcc(), *flags, "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
    failed, resources = [], []
    for cmd, proc in procs:
        _, err = proc.communicate()
        resources += parse_resources(err)
        if proc.returncode != 0:
            # the compiler's diagnostics, without the resource remarks and their source context
            print("\n".join(ln for ln in err.splitlines() if "error" in ln or "warning:" in ln), flush=True)
            failed.append(cmd)
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    with open(RESOURCES, "w") as f:
        json.dump(resources, f, indent=0)
    bad = spilling(resources)
    if bad:
        raise RuntimeError("kernels spill registers to scratch memory:\n" +
                           "\n".join(f"{r['kernel']}: scratch {r.get('ScratchSize')} B/lane" for r in bad))
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
