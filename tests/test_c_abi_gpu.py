"""The C ABI from plain C on the GPU: tests/c_abi/c_abi_check (built by
__graft_entry__.build()) calls gemm_epi_run_typed for fp16 and bf16 tensors
and gemm_epi_run_mixed for the other element-type pairs (fp32 or the other
16-bit type for the epilogue tensors) on integer inputs, fast and general
kernels, and gemm_epi_run_ws_typed with the workspace gemm_epi_plan_ws
reports, which stages ragged operands for the fast kernel; it compares every
output bit for bit with the CPU oracle and checks that an argument error
comes back as a status code.  It runs as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "c_abi_check")


def test_c_program_against_the_oracle():
    assert os.path.exists(EXE), f"{EXE} is missing: run __graft_entry__.build() first"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("PASS kind=") == 16 and r.stdout.count(" staged\n") == 4
    assert "PASS: 0 failing case(s)" in r.stdout
