"""Pins of the oracle's bfloat16 path (the Custom Epilogue Example's "Data
Type Support": BF16 among the input and output types), independent of the
oracle's own code.

bfloat16 is the upper half of an IEEE 754 binary32 (1 sign, 8 exponent, 7
fraction bits), so:
  - decoding every one of the 65,536 patterns must equal the binary32 whose
    upper half they are (numpy's float32 view of bits << 16);
  - encoding must round once to nearest, ties to even: for float32 inputs it
    must agree with torch's float32 -> bfloat16 conversion (round to nearest
    even); every midpoint between neighbours must go to the even one; a
    double just above a midpoint must round up even where a detour through
    float32 would land on the midpoint and round down;
  - the bf16 GEMM on integer inputs (exact sums) must equal torch's
    rounding of the exact result, and agree with the fp16 path wherever a
    value is representable in both formats.
"""
import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)


def upper_half_float(bits):
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def torch_bf16_bits(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def test_decode_every_pattern():
    got = oracle.bf16_decode(ALL)
    want = upper_half_float(ALL)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))  # -0 stays -0


def test_encode_round_trips_every_finite_pattern():
    v = oracle.bf16_decode(ALL)
    fin = np.isfinite(v)
    assert np.array_equal(oracle.bf16_encode(v[fin]), ALL[fin])
    assert np.all(np.isnan(oracle.bf16_decode(oracle.bf16_encode(v[np.isnan(v)]))))


def test_encode_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(100000) * 1e-38).astype(np.float32),     # subnormal range
        np.clip(rng.standard_normal(100000) * 1e38, -3.3e38, 3.3e38).astype(np.float32),  # near overflow
        rng.integers(-2 ** 24, 2 ** 24, 100000).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895313892515355e38, -3.3895313892515355e38], np.float32),
    ])
    assert np.array_equal(oracle.bf16_encode(x.astype(np.float64)), torch_bf16_bits(x))


def test_every_midpoint_rounds_to_even():
    v = oracle.bf16_decode(ALL[:0x7F80])          # +0 .. the largest finite positive
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2                           # exact in double
    got = oracle.bf16_encode(mid)
    even = np.where(ALL[:0x7F7F] % 2 == 0, ALL[:0x7F7F], ALL[1:0x7F80])
    assert np.array_equal(got, even)
    assert np.array_equal(oracle.bf16_encode(-mid), even | 0x8000)


def test_no_double_rounding_and_overflow():
    # 1 + 2^-8 is the midpoint between 1 and 1 + 2^-7: ties to even -> 1.0;
    # a hair above it must round up, although float32 would first round the
    # hair away and land on the midpoint
    assert oracle.bf16_encode(np.array([1 + 2.0 ** -8]))[0] == 0x3F80
    assert oracle.bf16_encode(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    assert torch_bf16_bits(np.array([1 + 2.0 ** -8 + 2.0 ** -40], np.float32))[0] == 0x3F80  # the detour's answer
    big = (2 - 2.0 ** -7) * 2.0 ** 127                # largest finite
    mid = (2 - 2.0 ** -8) * 2.0 ** 127                # midpoint to 2^128
    assert oracle.bf16_encode(np.array([big]))[0] == 0x7F7F
    assert oracle.bf16_encode(np.array([np.nextafter(mid, 0)]))[0] == 0x7F7F
    assert oracle.bf16_encode(np.array([mid, -mid]))[0] == 0x7F80
    assert oracle.bf16_encode(np.array([-mid]))[0] == 0xFF80
    # the smallest subnormal and half of it (a tie with zero -> zero)
    assert oracle.bf16_encode(np.array([2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -134]))[0] == 1
    assert list(oracle.bf16_encode(np.array([2.0 ** -134, 1.5 * 2.0 ** -134]))) == [0, 1]


def bf16_ints(shape, rng, lo=-3, hi=3):
    return torch_bf16_bits(rng.integers(lo, hi + 1, shape).astype(np.float32))


@pytest.mark.parametrize("kind", ["LINCOMB", "AUX_SCALE", "LINCOMB_X_ACC", "RELU_SQUARE", "RELU_SCALE_ACC"])
def test_bf16_gemm_on_integers_matches_torch(kind):
    """Integer inputs: every sum is exact, so the fp64 result rounded by torch
    (through float32, exact here) is the reference."""
    rng = np.random.default_rng(11)
    L, M, N, K = 2, 13, 17, 40
    A, B = bf16_ints((L, M, K), rng), bf16_ints((L, K, N), rng)
    C, X = bf16_ints((L, M, N), rng), bf16_ints((L, M, N), rng)
    alpha, beta, s3 = 2.0, 0.5, 0.25
    out = oracle.gemm_epi(A, B, C, X if kind == "LINCOMB_X_ACC" else None, kind=kind, alpha=alpha, beta=beta, s3=s3,
                          dtype="bf16")
    a, b = upper_half_float(A), upper_half_float(B)
    c, x = upper_half_float(C), upper_half_float(X)
    acc = np.einsum("lmk,lkn->lmn", a, b)       # exact: integers far below 2^53
    lin = alpha * acc + beta * c
    if kind == "LINCOMB":
        d, aux = lin, None
    elif kind == "AUX_SCALE":
        d, aux = s3 * lin, lin
    elif kind == "LINCOMB_X_ACC":
        d, aux = lin + s3 * x, acc
    elif kind == "RELU_SQUARE":
        d = np.maximum(lin, 0.0)
        aux = d * d
    else:  # RELU_SCALE_ACC
        aux = np.maximum(lin, 0.0)
        d = s3 * aux
    assert np.array_equal(out["D"], torch_bf16_bits(d.astype(np.float32)))   # all exact in float32
    if aux is not None:
        assert np.array_equal(out["Aux"], torch_bf16_bits(aux.astype(np.float32)))
    if kind == "RELU_SCALE_ACC":
        assert np.array_equal(out["Acc"], acc.astype(np.float32))


def test_bf16_and_fp16_paths_agree_where_both_are_exact():
    # small integers with small sums: every input and output is exact in
    # both formats, so the two element types must give the same values
    rng = np.random.default_rng(3)
    L, M, N, K = 1, 9, 11, 6
    a = rng.integers(-2, 3, (L, M, K)).astype(np.float32)
    b = rng.integers(-2, 3, (L, K, N)).astype(np.float32)
    c = rng.integers(-2, 3, (L, M, N)).astype(np.float32)
    f16 = oracle.gemm_epi(a.astype(np.float16), b.astype(np.float16), c.astype(np.float16), kind="AUX_SCALE",
                          alpha=1.0, beta=2.0, s3=0.5, want64=True)
    bf = oracle.gemm_epi(torch_bf16_bits(a), torch_bf16_bits(b), torch_bf16_bits(c), kind="AUX_SCALE", alpha=1.0,
                         beta=2.0, s3=0.5, want64=True, dtype="bf16")
    assert np.array_equal(f16["D64"], bf["D64"]) and np.array_equal(f16["Aux64"], bf["Aux64"])
    assert np.array_equal(f16["D"].astype(np.float64), oracle.bf16_decode(bf["D"]))
    assert np.array_equal(f16["Aux"].astype(np.float64), oracle.bf16_decode(bf["Aux"]))


def test_bf16_points_match_full():
    rng = np.random.default_rng(5)
    L, M, N, K = 2, 20, 24, 33
    p = {k: torch_bf16_bits(rng.standard_normal(s).astype(np.float32))
         for k, s in (("A", (L, M, K)), ("B", (L, K, N)), ("C", (L, M, N)))}
    full = oracle.gemm_epi(p["A"], p["B"], p["C"], kind="GELU", alpha=0.25, beta=1.0, dtype="bf16", want64=True)
    l, i, j = rng.integers(0, L, 300), rng.integers(0, M, 300), rng.integers(0, N, 300)
    pts = oracle.gemm_epi_points(p["A"], p["B"], p["C"], kind="GELU", alpha=0.25, beta=1.0, l=l, i=i, j=j,
                                 dtype="bf16")
    assert np.array_equal(pts["D"], full["D"][l, i, j])
    assert np.array_equal(pts["D64"], full["D64"][l, i, j])


def test_rejects_unknown_element_type():
    L = oracle.lib()
    h = np.zeros(16, np.uint16)
    sc = np.zeros(3, np.float32)
    P, S = h.ctypes.data, sc.ctypes.data
    assert L.oracle_gemm_epi_typed(1, 1, 1, 1, P, P, P, P, None, None, S, 0, P, P, None, None, None, None, 2) == 8
    assert L.oracle_gemm_epi_typed(1, 1, 1, 1, P, P, P, P, None, None, S, 0, P, P, None, None, None, None, 1) == 0
