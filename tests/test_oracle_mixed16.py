"""Pins of the oracle with separate 16-bit element types for A, B and for the
epilogue tensors (oracle.gemm_epi(..., dtype=..., epi_dtype=...): fp16 A, B
with bfloat16 C, X, biases, D, Aux, and the reverse; the Custom Epilogue
Example's "Data Type Support" lists FP16 and BF16 among both the input and
the output types).

Fixed by something other than the oracle: with small integers every value
before the last rounding is exact, so the outputs are NumPy's float64 result
rounded once -- to fp16 by NumPy's own conversion, to bfloat16 by the
oracle's bfloat16 encoder (pinned on its own by test_oracle_bf16.py) -- and
where the exact result is itself a small integer no rounding happens at all.
"""
import numpy as np
import pytest

import oracle

KINDS = ["LINCOMB", "AUX_SCALE", "LINCOMB_X_ACC", "RELU", "SQUARE", "RELU_SQUARE", "RELU_AUX_STORE",
         "RELU_SCALE_ACC", "BIAS_ROW_COL"]


def to_type(v, dtype):
    """float64 integers -> that 16-bit type (exact for these magnitudes)."""
    if dtype == "f16":
        return v.astype(np.float16)
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def from_type(a, dtype):
    """uint16 bit patterns of that type -> float64."""
    if dtype == "f16":
        return np.asarray(a, np.uint16).view(np.float16).astype(np.float64)
    return (np.asarray(a, np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to(v, dtype):
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    return oracle.bf16_encode(v)


@pytest.mark.parametrize("ab,epi", [("f16", "bf16"), ("bf16", "f16")])
@pytest.mark.parametrize("kind", KINDS)
def test_small_integers(kind, ab, epi):
    rng = np.random.default_rng(hash((kind, ab)) % 2**32)
    L, M, N, K = 2, 7, 9, 5
    A = rng.integers(-2, 3, (L, M, K)).astype(np.float64)
    B = rng.integers(-2, 3, (L, K, N)).astype(np.float64)
    C = rng.integers(-3, 4, (L, M, N)).astype(np.float64)
    X = rng.integers(-3, 4, (L, M, N)).astype(np.float64)
    rb = rng.integers(-3, 4, N).astype(np.float64)
    cb = rng.integers(-3, 4, M).astype(np.float64)
    alpha, beta, s = 1.0, 2.0, 0.5
    got = oracle.gemm_epi(to_type(A, ab), to_type(B, ab), to_type(C, epi), to_type(X, epi), kind=kind, alpha=alpha,
                          beta=beta, s3=s, row_bias=to_type(rb, epi), col_bias=to_type(cb, epi), dtype=ab,
                          epi_dtype=epi)
    acc = np.matmul(A, B)
    lin = alpha * acc + beta * C
    relu = np.where(lin > 0, lin, 0.0)
    want = {"LINCOMB": {"D": lin}, "AUX_SCALE": {"Aux": lin, "D": s * lin}, "LINCOMB_X_ACC": {"Aux": acc, "D": lin + s * X},
            "RELU": {"D": relu}, "SQUARE": {"D": lin, "Aux": lin * lin}, "RELU_SQUARE": {"D": relu, "Aux": relu * relu},
            "RELU_AUX_STORE": {"Aux": lin, "D": relu}, "RELU_SCALE_ACC": {"Aux": relu, "D": s * relu},
            "BIAS_ROW_COL": {"D": (alpha * acc + rb[None, None, :]) + cb[None, :, None]}}[kind]
    for name, w in want.items():
        g = np.asarray(got[name]).view(np.uint16)
        assert np.array_equal(g, round_to(w, epi)), f"{kind} {ab}->{epi} {name}"
        small = np.abs(w) <= 256  # exactly representable in both types: no rounding
        assert np.array_equal(from_type(g, epi)[small], w[small]), f"{kind} {ab}->{epi} {name}"
    if kind == "RELU_SCALE_ACC":
        assert np.array_equal(got["Acc"], acc.astype(np.float32))


def test_same_types_are_the_typed_call():
    rng = np.random.default_rng(1)
    A = rng.standard_normal((1, 6, 40)).astype(np.float16)
    B = rng.standard_normal((1, 40, 5)).astype(np.float16)
    C = rng.standard_normal((1, 6, 5)).astype(np.float16)
    a = oracle.gemm_epi(A, B, C, kind="AUX_SCALE", alpha=1.5, beta=-2.0, s3=0.5, want64=True)
    b = oracle.gemm_epi(A, B, C, kind="AUX_SCALE", alpha=1.5, beta=-2.0, s3=0.5, want64=True, epi_dtype="f16")
    for k in a:
        assert np.array_equal(np.asarray(a[k]).view(np.uint8), np.asarray(b[k]).view(np.uint8)), k
