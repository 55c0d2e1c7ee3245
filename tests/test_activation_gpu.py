"""Activation epilogues on the GPU: D = act(alpha*acc + beta*C) for sigmoid,
tanh, GELU, SiLU, leaky ReLU and hardswish (the built-in activations of the
CUTLASS Python examples article's "Epilogue" section), against the CPU
oracle.

Bar: where alpha*acc + beta*C is exact in fp32 (integer inputs, power-of-two
scalars, or acc equal to one fp16 input), every output lies within one fp16
ulp of the oracle's unrounded value and at least 98% are bit-identical to its
correctly rounded fp16 (the kernels' fp32 activations are accurate to about
1e-6).  Gaussian inputs at full size: the tolerance of the other kinds at
sampled points, plus range properties of the whole output.
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_elementwise_amd as ge
from dense_gemm_elementwise_amd import workloads
from test_parity_gpu import (alloc_out, assert_close, assert_within_ulp, check_full, gpu_run, log, oracle_points,
                             sample_points, to_dev)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("act", workloads.ACTIVATIONS)
def test_page_workload_256(act):
    """The Epilogue example's own problem: m = n = k = 256, inputs built as in
    the Basic GEMM example (integers), alpha = 1, beta = 0."""
    w = workloads.WORKLOADS[f"{act.lower()}_256"]
    log(f"[activation] {w.name}: L={w.L} M={w.M} N={w.N} K={w.K}")
    p = workloads.make_inputs(w)
    check_full(p, w.kind, w.alpha, w.beta, w.s3, exact=True, what=w.name)


def fp16_sweep(lo=-12.0, hi=12.0):
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    v = v[np.isfinite(v) & (v >= lo) & (v <= hi)]
    return np.unique(v)


@pytest.mark.parametrize("act", workloads.ACTIVATIONS)
def test_every_fp16_input(act):
    """acc = t exactly for every fp16 t in [-12, 12] (A's first column holds t,
    B's first row is ones, the rest zeros), through the vector kernel: the
    activation approximations themselves, tails included."""
    t = fp16_sweep()
    M, N, K = t.size, 8, 8
    A = np.zeros((1, M, K), np.float16)
    A[0, :, 0] = t
    B = np.zeros((1, K, N), np.float16)
    B[0, 0, :] = 1.0
    C = np.zeros((1, M, N), np.float16)
    p = {"A": A, "B": B, "C": C, "X": None, "row_bias": None, "col_bias": None}
    s3 = 0.125 if act == "LEAKY_RELU" else 0.0
    log(f"[activation] sweep {act}: {M} inputs")
    check_full(p, act, 1.0, 0.0, s3, exact=True, what=f"sweep {act}")


def fp16_midpoints(lo, hi):
    """(v, h): every fp16 v in [lo, hi) whose upper neighbour is finite, and
    h, half the gap to it, so that v + h is the fp16 rounding midpoint."""
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    v = bits.view(np.float16).astype(np.float64)
    nxt = (bits + 1).view(np.float16).astype(np.float64)
    keep = (v >= lo) & (v < hi) & np.isfinite(nxt)
    return v[keep], (nxt[keep] - v[keep]) / 2


@pytest.mark.parametrize("act,lo", [("SILU", 17.0), ("GELU", 6.0)])
def test_saturated_midpoints_round_correctly(act, lo):
    """acc = an fp16 rounding midpoint m (A's first two columns hold v and
    half the gap to v's upper neighbour, B's first two rows are ones), for
    every midpoint from where the factor sigmoid(m) or Phi(m) rounds to 1 in
    fp32 up to 65504.  The exact output lies just below m, so its fp16
    rounding is v; the fp32 value m itself would round the tie to even.
    Every output equals the oracle's correctly rounded fp16."""
    v, h = fp16_midpoints(lo, 65504.0)
    M, N, K = v.size, 8, 8
    A = np.zeros((1, M, K), np.float16)
    A[0, :, 0] = v
    A[0, :, 1] = h
    B = np.zeros((1, K, N), np.float16)
    B[0, :2, :] = 1.0
    C = np.zeros((1, M, N), np.float16)
    p = {"A": A, "B": B, "C": C, "X": None, "row_bias": None, "col_bias": None}
    log(f"[activation] {act} at {M} fp16 midpoints")
    got = gpu_run(p, act, 1.0, 0.0, 0.0)
    ref = oracle.gemm_epi(p["A"], p["B"], p["C"], kind=act, alpha=1.0, beta=0.0)
    assert np.array_equal(ref["D"][0, :, 0].astype(np.float64), v), "the oracle rounds each midpoint down"
    bad = np.count_nonzero(got["D"].view(np.uint16) != ref["D"].view(np.uint16))
    assert bad == 0, f"{act}: {bad} of {got['D'].size} outputs differ from the correctly rounded fp16"


def test_gelu_8192_sampled_and_properties():
    w = workloads.WORKLOADS["gelu_8192"]
    log(f"[activation] {w.name}: L={w.L} M={w.M} N={w.N} K={w.K}")
    p = workloads.make_inputs(w)
    t = to_dev(p)
    D = alloc_out(w.L, w.M, w.N)
    ge.run(t["A"], t["B"], t["C"], kind=w.kind, alpha=w.alpha, beta=w.beta, D=D)
    # whole output: finite, and above GELU's minimum (-0.16997 at t = -0.7518)
    assert bool(torch.isfinite(D).all())
    assert float(D.min()) >= -0.1700, float(D.min())
    l, i, j = sample_points(w.L, w.M, w.N, 20000, seed=5)
    ref = oracle_points(p, w.kind, w.alpha, w.beta, w.s3, l, i, j)
    assert_close(D.cpu().numpy()[l, i, j], ref["D64"], "gelu_8192 D")
