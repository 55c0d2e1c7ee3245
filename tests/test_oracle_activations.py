"""Pins of the oracle's activation epilogues (SIGMOID, TANH, GELU, SILU,
LEAKY_RELU, HARDSWISH: D = act(alpha*acc + beta*C)), independent of the
oracle's own code.

The activations are the built-in list of the CUTLASS Python examples
article's "Epilogue" section; the pages give no formulas, so the standard
definitions are the reference (sigmoid 1/(1+e^-t), tanh, GELU t*Phi(t) in its
exact form, SiLU t*sigmoid(t), leaky ReLU with the slope in the third scalar,
hardswish t*min(max(t+3,0),6)/6 as in MobileNetV3).  What pins them:
  - library special cases: with K = 1, B = 1 and beta = 0 the accumulator is
    the fp16 input itself, so over a sweep of every fp16 value in [-12, 12]
    the oracle's unrounded D must match scipy.special.expit, numpy.tanh,
    t * scipy.special.ndtr(t) (Phi from the Cephes library, not erfc), and the
    closed forms; its fp16 D must be those values rounded by numpy;
  - identities: sigmoid(t) + sigmoid(-t) = 1, tanh(t) = 2 sigmoid(2t) - 1,
    gelu(t) - gelu(-t) = t, silu = t * sigmoid;
  - the linear combination reaches the activation unrounded: act applied to
    the LINCOMB kind's unrounded D of the same inputs;
  - the hand-worked cases in tests/golden/hand_worked.json.
"""
import numpy as np
import pytest
import scipy.special

import oracle
from dense_gemm_elementwise_amd import workloads

SLOPE = 0.125


def reference(kind, t):
    t = np.asarray(t, np.float64)
    if kind == "SIGMOID":
        return scipy.special.expit(t)
    if kind == "TANH":
        return np.tanh(t)
    if kind == "GELU":
        return t * scipy.special.ndtr(t)
    if kind == "SILU":
        return t * scipy.special.expit(t)
    if kind == "LEAKY_RELU":
        return np.where(t > 0, t, SLOPE * t)
    if kind == "HARDSWISH":
        return t * np.clip(t + 3.0, 0.0, 6.0) / 6.0
    raise ValueError(kind)


def fp16_sweep(lo=-12.0, hi=12.0):
    """Every finite fp16 value in [lo, hi]."""
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    v = v[np.isfinite(v)]
    v = v[(v >= lo) & (v <= hi)]
    return np.unique(v)


def apply(kind, t16, s3=SLOPE):
    """D of the oracle with acc = t exactly: A = t (M x 1), B = [[1]], beta = 0."""
    M = t16.size
    A = t16.reshape(1, M, 1)
    B = np.ones((1, 1, 1), np.float16)
    C = np.zeros((1, M, 1), np.float16)
    out = oracle.gemm_epi(A, B, C, kind=kind, alpha=1.0, beta=0.0, s3=s3, want64=True)
    return out["D"].reshape(M), out["D64"].reshape(M)


@pytest.mark.parametrize("kind", oracle.ACTIVATIONS)
def test_activation_matches_library_on_every_fp16_input(kind):
    t16 = fp16_sweep()
    d16, d64 = apply(kind, t16)
    ref = reference(kind, t16.astype(np.float64))
    tol = 1e-13 * np.abs(ref) + 1e-300
    if kind == "GELU":
        # ndtr is accurate to a few units in the last place; far in the left
        # tail gelu is below every fp16 subnormal anyway
        tol = 1e-12 * np.abs(ref) + 1e-30
    assert np.all(np.abs(d64 - ref) <= tol), np.max(np.abs(d64 - ref) / (np.abs(ref) + 1e-300))
    # one rounding, double -> fp16, to nearest (numpy rounds the same way)
    want = ref.astype(np.float16)
    assert np.array_equal(d16.astype(np.float64), want.astype(np.float64))


@pytest.mark.parametrize("kind", oracle.ACTIVATIONS)
def test_activation_of_the_linear_combination(kind):
    # act(alpha*acc + beta*C) with acc a real GEMM and C read: the activation
    # sees the unrounded combination, i.e. act(D64 of LINCOMB)
    p = workloads.make_problem(2, 24, 40, 64, "LINCOMB", init="normal", seed=41)
    lin = oracle.gemm_epi(p["A"], p["B"], p["C"], kind="LINCOMB", alpha=0.125, beta=0.5, want64=True)
    act = oracle.gemm_epi(p["A"], p["B"], p["C"], kind=kind, alpha=0.125, beta=0.5, s3=SLOPE, want64=True)
    ref = reference(kind, lin["D64"])
    assert np.all(np.abs(act["D64"] - ref) <= 1e-12 * np.abs(ref) + 1e-300)
    assert np.array_equal(act["D"].astype(np.float64), ref.astype(np.float16).astype(np.float64))
    assert "Aux" not in act or act["Aux"] is None


def test_activation_identities():
    t16 = fp16_sweep(-8.0, 8.0)
    t = t16.astype(np.float64)
    _, sig = apply("SIGMOID", t16)
    _, sig_neg = apply("SIGMOID", (-t).astype(np.float16))
    assert np.allclose(sig + sig_neg, 1.0, rtol=0, atol=1e-15)
    _, th = apply("TANH", t16)
    twice = (2 * t).astype(np.float16)   # exact: doubling an fp16 value in [-8, 8]
    _, sig2 = apply("SIGMOID", twice)
    assert np.allclose(th, 2 * sig2 - 1, rtol=0, atol=1e-15)
    _, g = apply("GELU", t16)
    _, g_neg = apply("GELU", (-t).astype(np.float16))
    assert np.allclose(g - g_neg, t, rtol=0, atol=1e-14)
    _, si = apply("SILU", t16)
    assert np.allclose(si, t * sig, rtol=1e-15, atol=0)


def test_activation_special_points():
    pts = np.array([0.0, 3.0, -3.0, 6.0, -6.0, 1.0], np.float16)
    _, sig = apply("SIGMOID", pts)
    _, th = apply("TANH", pts)
    _, g = apply("GELU", pts)
    _, si = apply("SILU", pts)
    _, hs = apply("HARDSWISH", pts)
    _, lr = apply("LEAKY_RELU", pts, s3=0.5)
    assert sig[0] == 0.5 and th[0] == 0.0 and g[0] == 0.0 and si[0] == 0.0 and hs[0] == 0.0
    # hardswish: identity from t = 3 up, zero from t = -3 down, 2/3 at 1
    assert hs[1] == 3.0 and hs[3] == 6.0 and hs[2] == 0.0 and hs[4] == 0.0
    assert abs(hs[5] - 2.0 / 3.0) < 1e-15
    # leaky ReLU: identity above zero, slope * t below
    assert lr[1] == 3.0 and lr[2] == -1.5 and lr[4] == -3.0
    # gelu(t) -> t for large t (from below, within one double ulp: 12 (1 - Phi(12))
    # is below 1e-31), -> 0 for very negative t
    _, g_far = apply("GELU", np.array([12.0, -12.0], np.float16))
    assert 12.0 - np.spacing(12.0) <= g_far[0] < 12.0 and abs(g_far[1]) < 1e-30


def test_leaky_relu_slope_is_the_third_scalar():
    t16 = np.array([-2.0, -0.5, 0.5, 2.0], np.float16)
    for slope in (0.0, 0.01, 0.5, 2.0):
        _, d = apply("LEAKY_RELU", t16, s3=slope)
        np.testing.assert_array_equal(d, np.where(t16 > 0, t16.astype(np.float64), np.float32(slope) * t16.astype(np.float64)))


def midpoints(dtype, lo, hi):
    """(v, h, m): every value v of the format in [lo, hi) with a finite upper
    neighbour, half the gap to that neighbour, and the rounding midpoint
    m = v + h between them (exact in double)."""
    bits = np.arange(0, 0x7F80 if dtype == "bf16" else 0x7C00, dtype=np.uint16)
    dec = oracle.bf16_decode if dtype == "bf16" else (lambda b: b.view(np.float16).astype(np.float64))
    v, nxt = dec(bits), dec(bits + 1)
    keep = (v >= lo) & (v < hi) & np.isfinite(nxt)
    h = (nxt[keep] - v[keep]) / 2
    return bits[keep], v[keep], h, v[keep] + h


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("kind,lo", [("SILU", 17.0), ("GELU", 6.0)])
def test_far_right_midpoints_round_down(kind, lo, dtype):
    """For m > 0, m - silu(m) = m / (1 + e^m) < m e^-m and m - gelu(m) =
    m (1 - Phi(m)) < e^(-m^2/2) / sqrt(2 pi) (Mills' ratio): from m = 17 and
    m = 6 on, both are positive and far below half the gap between
    neighbouring fp16 or bfloat16 values.  So at each rounding midpoint m of
    the format the exact output lies just below m and rounds to the lower
    neighbour, while m itself would round its tie to the even one.  acc = m
    exactly (A's two columns v and h, B's two rows ones)."""
    bits, v, h, m = midpoints(dtype, lo, 60000.0 if dtype == "f16" else 1e6)
    gap_below = m * np.exp(-m) if kind == "SILU" else np.exp(-m * m / 2)   # the bounds above
    assert np.all(gap_below < h / 4)
    M = m.size
    if dtype == "bf16":
        A = np.stack([bits, oracle.bf16_encode(h)], axis=1).reshape(1, M, 2)
        one = np.uint16(0x3F80)
        B = np.full((1, 2, 1), one, np.uint16)
        C = np.zeros((1, M, 1), np.uint16)
        out = oracle.gemm_epi(A, B, C, kind=kind, alpha=1.0, beta=0.0, want64=True, dtype="bf16")
    else:
        A = np.stack([v, h], axis=1).astype(np.float16).reshape(1, M, 2)
        B = np.ones((1, 2, 1), np.float16)
        C = np.zeros((1, M, 1), np.float16)
        out = oracle.gemm_epi(A, B, C, kind=kind, alpha=1.0, beta=0.0, want64=True)
    d64 = out["D64"].reshape(M)
    assert np.all((d64 < m) & (d64 > m - h)), "the unrounded output lies just below each midpoint"
    got = out["D"].reshape(M).view(np.uint16)
    assert np.array_equal(got, bits), f"{np.count_nonzero(got != bits)} of {M} midpoints not rounded down"
