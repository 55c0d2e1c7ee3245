"""Pins of the oracle's fp32-epilogue-tensor path (oracle.gemm_epi_f32e: fp16
or bf16 A and B, fp32 C, X, biases, D and Aux; the Custom Epilogue
Example's "Data Type Support" lists FP32 among the C and D types).

Each pin is fixed by something other than the oracle itself:
  * library special case: with integer A, B and power-of-two scalars every
    value before the last rounding is exact in float64, so the outputs equal
    NumPy's float64 -> float32 conversion of NumPy's float64 arithmetic;
  * closed forms at A = 0 and A = I;
  * the 16-bit path's own pins: with C exactly representable in fp16, the
    unrounded outputs equal those of oracle.gemm_epi bit for bit;
  * float32 overflow gives inf;
  * activations against NumPy / SciPy's float64 functions, within one float32
    ulp of the correctly rounded value.
"""
import numpy as np
import pytest
from scipy import special

import oracle

LINEAR = ["LINCOMB", "AUX_SCALE", "LINCOMB_X_ACC", "RELU", "SQUARE", "RELU_SQUARE", "RELU_AUX_STORE",
          "RELU_SCALE_ACC", "BIAS_ROW_COL"]


def ints(rng, shape, dtype):
    v = rng.integers(-2, 3, shape).astype(np.float32)
    if dtype == "f16":
        return v.astype(np.float16)
    return (v.view(np.uint32) >> 16).astype(np.uint16)  # integers are exact in bfloat16


def as64(a, dtype):
    if dtype == "f16":
        return np.asarray(a, np.float64)
    return (np.asarray(a, np.uint32) << 16).view(np.float32).astype(np.float64)


def numpy_reference(kind, acc, C, X, rb, cb, alpha, beta, s):
    """The kinds' formulas in NumPy float64 (exact here), then one cast."""
    lin = alpha * acc + beta * C
    relu = np.where(lin > 0, lin, 0.0)
    out = {
        "LINCOMB": {"D": lin},
        "AUX_SCALE": {"Aux": lin, "D": s * lin},
        "LINCOMB_X_ACC": {"Aux": acc, "D": lin + s * X},
        "RELU": {"D": relu},
        "SQUARE": {"D": lin, "Aux": lin * lin},
        "RELU_SQUARE": {"D": relu, "Aux": relu * relu},
        "RELU_AUX_STORE": {"Aux": lin, "D": relu},
        "RELU_SCALE_ACC": {"Aux": relu, "D": s * relu},
        "BIAS_ROW_COL": {"D": (alpha * acc + rb[None, None, :]) + cb[None, :, None]},
    }[kind]
    return {k: v.astype(np.float32) for k, v in out.items()}


@pytest.mark.parametrize("ab", ["f16", "bf16"])
@pytest.mark.parametrize("kind", LINEAR)
def test_exact_integer_products_equal_numpy(kind, ab):
    rng = np.random.default_rng(hash((kind, ab)) % 2**32)
    L, M, N, K = 2, 9, 11, 13
    A, B = ints(rng, (L, M, K), ab), ints(rng, (L, K, N), ab)
    # fp32 epilogue inputs with few significant bits, so alpha*acc + beta*C stays exact in float64
    C = (rng.integers(-2**20, 2**20, (L, M, N)) * 2.0 ** -7).astype(np.float32)
    X = (rng.integers(-2**20, 2**20, (L, M, N)) * 2.0 ** -9).astype(np.float32)
    rb = (rng.integers(-999, 999, N) * 0.25).astype(np.float32)
    cb = (rng.integers(-999, 999, M) * 0.5).astype(np.float32)
    alpha, beta, s = 2.0, 0.5, 0.25
    got = oracle.gemm_epi_f32e(A, B, C, X, kind=kind, alpha=alpha, beta=beta, s3=s, row_bias=rb, col_bias=cb,
                               ab_dtype=ab)
    acc = np.matmul(as64(A, ab), as64(B, ab))
    want = numpy_reference(kind, acc, C.astype(np.float64), X.astype(np.float64), rb.astype(np.float64),
                           cb.astype(np.float64), alpha, beta, s)
    for name, w in want.items():
        assert got[name].dtype == np.float32
        assert np.array_equal(got[name], w), f"{kind} {ab} {name}"
    if kind == "RELU_SCALE_ACC":
        assert np.array_equal(got["Acc"], acc.astype(np.float32))


def test_closed_forms():
    rng = np.random.default_rng(3)
    L, M, N, K = 1, 6, 5, 6
    C = rng.standard_normal((L, M, N)).astype(np.float32)
    X = rng.standard_normal((L, M, N)).astype(np.float32)
    Bm = rng.integers(-3, 4, (L, K, N)).astype(np.float16)
    zero = np.zeros((L, M, K), np.float16)
    r = oracle.gemm_epi_f32e(zero, Bm, C, X, kind="LINCOMB_X_ACC", alpha=2.0, beta=3.0, s3=5.0)
    assert np.all(r["Aux"] == 0)
    assert np.array_equal(r["D"], (3.0 * C.astype(np.float64) + 5.0 * X.astype(np.float64)).astype(np.float32))
    eye = np.eye(M, K, dtype=np.float16)[None]
    r = oracle.gemm_epi_f32e(eye, Bm, C, kind="LINCOMB", alpha=1.0, beta=0.0)
    assert np.array_equal(r["D"], Bm.astype(np.float32))


@pytest.mark.parametrize("kind", LINEAR + ["GELU"])
def test_agrees_with_the_16_bit_path(kind):
    """C, X and the biases exactly fp16-valued: the unrounded outputs equal the
    16-bit oracle's (the same definition), and the fp32 outputs are their
    float32 roundings."""
    rng = np.random.default_rng(11)
    L, M, N, K = 2, 7, 10, 33
    A = rng.standard_normal((L, M, K)).astype(np.float16)
    B = rng.standard_normal((L, K, N)).astype(np.float16)
    C = rng.standard_normal((L, M, N)).astype(np.float16)
    X = rng.standard_normal((L, M, N)).astype(np.float16)
    rb = rng.standard_normal(N).astype(np.float16)
    cb = rng.standard_normal(M).astype(np.float16)
    kw = dict(kind=kind, alpha=1.5, beta=-0.75, s3=0.5, want64=True)
    r16 = oracle.gemm_epi(A, B, C, X, row_bias=rb, col_bias=cb, **kw)
    r32 = oracle.gemm_epi_f32e(A, B, C.astype(np.float32), X.astype(np.float32), row_bias=rb.astype(np.float32),
                               col_bias=cb.astype(np.float32), **kw)
    for name in ("D", "Aux"):
        if name in r16:
            assert np.array_equal(r16[name + "64"], r32[name + "64"]), name
            assert np.array_equal(r32[name], r32[name + "64"].astype(np.float32)), name


def test_overflow_gives_inf():
    A = np.full((1, 2, 4), 256.0, np.float16)
    B = np.full((1, 4, 3), 256.0, np.float16)          # acc = 2^18
    C = np.zeros((1, 2, 3), np.float32)
    r = oracle.gemm_epi_f32e(A, B, C, kind="LINCOMB", alpha=2.0 ** 120, beta=0.0)   # 2^138 > FLT_MAX
    assert np.all(np.isposinf(r["D"]))
    r = oracle.gemm_epi_f32e(A, B, C, kind="LINCOMB", alpha=-(2.0 ** 100), beta=0.0)  # -2^118 is finite
    assert np.all(r["D"] == np.float32(-(2.0 ** 118)))


ACTS = {"SIGMOID": lambda t: special.expit(t), "TANH": np.tanh, "GELU": lambda t: 0.5 * t * special.erfc(-t / np.sqrt(2)),
        "SILU": lambda t: t * special.expit(t), "HARDSWISH": lambda t: t * np.clip(t + 3, 0, 6) / 6}


@pytest.mark.parametrize("act", sorted(ACTS))
def test_activations_within_one_float32_ulp(act):
    t = np.linspace(-20, 20, 4001)
    t16 = t.astype(np.float16)
    A = t16.reshape(1, -1, 1)
    B = np.ones((1, 1, 1), np.float16)
    C = np.zeros((1, t.size, 1), np.float32)
    got = oracle.gemm_epi_f32e(A, B, C, kind=act, alpha=1.0, beta=0.0)["D"].ravel().astype(np.float64)
    want = ACTS[act](t16.astype(np.float64))
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - want) <= ulp), act
