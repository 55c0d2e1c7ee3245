"""The unfused composition (gemm_epi_run_unfused: a GEMM launch writing the
fp32 accumulator, then an elementwise epilogue launch) against the fused
kernel and the oracle, on the GPU.

It computes the same accumulator and applies the same fp32 epilogue
arithmetic, so its outputs must equal the fused kernel's bit for bit, on
every kind, on the 16-byte vector paths and the element-wise ones; on
integer inputs they also equal the oracle's.  This is the three-kernel
composition the fusion replaces (Custom Epilogue Example, Overview), kept
to measure what fusing saves.
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_elementwise_amd as ge
from dense_gemm_elementwise_amd import workloads

from test_parity_gpu import KIND_SCALARS, alloc_out, assert_bit_exact, assert_close, assert_output, log, oracle_full, oracle_ref, to_dev

pytestmark = pytest.mark.gpu


def run_both(p, kind, alpha, beta, s3, offset=0):
    t = to_dev(p, offset)
    L, M, K = p["A"].shape
    N = p["B"].shape[2]
    outs = []
    for fused in (True, False):
        D = alloc_out(L, M, N, offset)
        Aux = alloc_out(L, M, N, offset) if kind in ge.HAS_AUX else None
        acc = alloc_out(L, M, N, offset, torch.float32) if kind in ge.HAS_ACC else None
        ws = None if fused else torch.full((L * M * N + offset,), float("nan"), dtype=torch.float32,
                                           device="cuda:0")[offset:]
        ge.run(t["A"], t["B"], t["C"], t["X"], kind=kind, alpha=alpha, beta=beta, s3=s3, D=D, Aux=Aux,
               row_bias=t["row_bias"], col_bias=t["col_bias"], acc_out=acc, unfused_workspace=ws)
        o = {"D": D.cpu().numpy()}
        if Aux is not None:
            o["Aux"] = Aux.cpu().numpy()
        if acc is not None:
            o["Acc"] = acc.cpu().numpy()
        outs.append(o)
    return outs


@pytest.mark.parametrize("kind", workloads.KINDS)
@pytest.mark.parametrize("shape,offset", [((2, 200, 136, 264), 0),    # vector paths
                                          ((2, 200, 136, 264), 1),    # misaligned: element-wise paths
                                          ((3, 77, 45, 61), 0),       # K, N not multiples of 8 (N % 4 != 0)
                                          ((1, 300, 520, 136), 0),
                                          ((1, 1960, 2000, 72), 0),   # the 4-wave tiles: 128 x 128,
                                          ((1, 2000, 3000, 72), 0),   # 128 x 256
                                          ((1, 3112, 3928, 40), 0),   # and 256 x 256
                                          ((1, 2100, 2100, 61), 0)])  # general kernel, 256 x 128 tiles
def test_unfused_equals_fused_and_oracle(kind, shape, offset):
    L, M, N, K = shape
    a, b, s = KIND_SCALARS[kind]
    log(f"[unfused] kind={kind} shape={shape} offset={offset}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=M + N * K)
    fused, unfused = run_both(p, kind, a, b, s, offset)
    ref = oracle_ref(p, kind, a, b, s, exact=True)
    for name in fused:
        assert np.array_equal(fused[name].view(np.uint8), unfused[name].view(np.uint8)), f"{kind} {name} fused != unfused"
        if name == "Acc":
            assert np.array_equal(unfused[name], ref[name]), f"{kind} acc_out"
        else:
            assert_output(unfused[name], ref, name, kind, True, f"unfused {kind} {name}")


@pytest.mark.parametrize("kind", ["LINCOMB_X_ACC", "RELU_SCALE_ACC", "BIAS_ROW_COL"])
def test_unfused_equals_fused_gaussian(kind):
    L, M, N, K = 1, 1024, 1024, 1024
    a, b, s = KIND_SCALARS[kind]
    log(f"[unfused] gaussian kind={kind}")
    p = workloads.make_problem(L, M, N, K, kind, init="normal", seed=29)
    fused, unfused = run_both(p, kind, a, b, s)
    ref = oracle_ref(p, kind, a, b, s, exact=False)
    for name in fused:
        assert np.array_equal(fused[name].view(np.uint8), unfused[name].view(np.uint8)), f"{kind} {name}"
        if name == "Acc":
            assert_close(unfused[name], ref["Acc64"], f"unfused gaussian {kind} acc_out")
        else:
            assert_output(unfused[name], ref, name, kind, False, f"unfused gaussian {kind} {name}")
