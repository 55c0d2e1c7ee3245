"""Pins for the tutorial's further epilogues in the oracle (CPU only):
relu_aux_store (CUTLASS Operator API tutorial "Custom epilogue fusions for
GEMMs", cell [6]; cell [8] is the same function with other scalars),
relu_scale_return_acc (cell [7], with the fp32 accumulator as a third
output) and the row / column broadcast bias (cell [9]).

Each is pinned to something other than the oracle itself: NumPy's float64
matmul on the pages' integer inputs (exact), relations to the other kinds
that follow from the definitions, and closed forms of the broadcasts.  The
exact-rational sweep over every kind lives in test_oracle_gemm.py.
"""
import numpy as np
import pytest

import oracle
from dense_gemm_elementwise_amd import workloads


def bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


def run(p, kind, alpha, beta, s3, want64=False):
    return oracle.gemm_epi(p["A"], p["B"], p["C"], p["X"], kind=kind, alpha=alpha, beta=beta, s3=s3,
                           row_bias=p["row_bias"], col_bias=p["col_bias"], want64=want64)


def exact_acc(p):
    return np.matmul(p["A"].astype(np.float64), p["B"].astype(np.float64))


@pytest.mark.parametrize("name", ["relu_aux_store_1024", "relu_scale_acc_1024", "bias_row_col_1024"])
def test_page_workloads_against_numpy(name):
    """On the tutorial's 1024^3 integer inputs every value below is exact in
    float64, so NumPy's float64 -> float16 cast is the single rounding."""
    w = workloads.WORKLOADS[name]
    p = workloads.make_inputs(w)
    out = run(p, w.kind, w.alpha, w.beta, w.s3, want64=True)
    acc = exact_acc(p)
    assert np.array_equal(out["Acc64"], acc)
    if w.kind == "RELU_AUX_STORE":
        f = w.alpha * acc + w.beta * p["C"].astype(np.float64)
        assert np.array_equal(out["Aux64"], f)
        assert np.array_equal(bits(out["Aux"]), f.astype(np.float16).view(np.uint16))
        assert np.array_equal(out["D"].astype(np.float64), np.maximum(f, 0.0).astype(np.float16).astype(np.float64))
    elif w.kind == "RELU_SCALE_ACC":
        f = np.maximum(w.alpha * acc + w.beta * p["C"].astype(np.float64), 0.0)
        assert np.array_equal(out["Aux64"], f)
        assert np.array_equal(out["D64"], w.s3 * f)
        assert np.array_equal(out["D"].astype(np.float64), (w.s3 * f).astype(np.float16).astype(np.float64))
        assert np.array_equal(out["Acc"], acc.astype(np.float32))  # |acc| < 2^24: exact in fp32
    else:
        d = (w.alpha * acc + p["row_bias"].astype(np.float64)[None, None, :]) \
            + p["col_bias"].astype(np.float64)[None, :, None]
        assert np.array_equal(out["D64"], d)
        assert np.array_equal(bits(out["D"]), d.astype(np.float16).view(np.uint16))


def test_relations_to_the_other_kinds():
    L, M, N, K = 2, 37, 45, 96
    p = workloads.make_problem(L, M, N, K, "LINCOMB", init="normal", seed=21)
    p["row_bias"], p["col_bias"] = None, None
    a, b = 1.25, -0.5
    lin = run(p, "LINCOMB", a, b, 0.0, want64=True)
    relu = run(p, "RELU", a, b, 0.0, want64=True)
    ras = run(p, "RELU_AUX_STORE", a, b, 0.0, want64=True)
    rsa = run(p, "RELU_SCALE_ACC", a, b, 0.5, want64=True)
    # relu_aux_store: F is LINCOMB's D, D is RELU's D, and D = relu(F) after rounding too
    assert np.array_equal(bits(ras["Aux"]), bits(lin["D"]))
    assert np.array_equal(bits(ras["D"]), bits(relu["D"]))
    fa = ras["Aux"].astype(np.float64)
    assert np.array_equal(ras["D"].astype(np.float64), np.where(fa > 0, fa, 0.0))
    # relu_scale_return_acc: F is RELU's D; D = F / 2 exactly for normal values
    assert np.array_equal(bits(rsa["Aux"]), bits(relu["D"]))
    fb = bits(rsa["Aux"]).astype(np.int32)
    normal = (((fb >> 10) & 31) >= 2) & (((fb >> 10) & 31) < 31)
    assert np.array_equal(bits(rsa["D"])[normal], (fb[normal] - 0x400).astype(np.uint16))
    # the accumulator output is the exact sum rounded once to fp32
    assert np.array_equal(rsa["Acc"], rsa["Acc64"].astype(np.float32))
    acc_only = run(p, "LINCOMB", 1.0, 0.0, 0.0, want64=True)
    assert np.array_equal(rsa["Acc64"], acc_only["D64"])


def test_bias_closed_forms():
    L, M, N, K = 3, 29, 41, 50
    p = workloads.make_problem(L, M, N, K, "BIAS_ROW_COL", init="normal", seed=22)
    assert p["C"] is None and p["row_bias"].shape == (N,) and p["col_bias"].shape == (M,)
    out = run(p, "BIAS_ROW_COL", 1.5, 0.0, 0.0, want64=True)
    # zero biases: alpha * acc, the LINCOMB of beta = 0
    q = dict(p)
    q["row_bias"] = np.zeros_like(p["row_bias"])
    q["col_bias"] = np.zeros_like(p["col_bias"])
    z = run(q, "BIAS_ROW_COL", 1.5, 0.0, 0.0, want64=True)
    lin = oracle.gemm_epi(p["A"], p["B"], np.zeros((L, M, N), np.float16), kind="LINCOMB", alpha=1.5, beta=0.0,
                          want64=True)
    assert np.array_equal(z["D64"], lin["D64"])
    # the row bias is the same for every row and batch entry, the column bias
    # the same for every column: D64 - z.D64 is row_bias[j] + col_bias[i]
    # up to the rounding of the two additions (bounded by 2 ulp of the result)
    diff = out["D64"] - z["D64"]
    want = p["row_bias"].astype(np.float64)[None, None, :] + p["col_bias"].astype(np.float64)[None, :, None]
    tol = 4 * np.finfo(np.float64).eps * (np.abs(out["D64"]) + np.abs(z["D64"]) + 1)
    assert np.all(np.abs(diff - want) <= tol)
    # swapping the biases' roles is not a symmetry: a transposed row/column
    # bias gives a different result on a non-square problem
    assert M != N


def test_bias_batches_share_the_biases():
    L, M, N, K = 3, 8, 12, 16
    p = workloads.make_problem(L, M, N, K, "BIAS_ROW_COL", init="small_int", seed=23)
    full = run(p, "BIAS_ROW_COL", 1.0, 0.0, 0.0, want64=True)
    for l in range(L):
        one = oracle.gemm_epi(p["A"][l:l + 1], p["B"][l:l + 1], kind="BIAS_ROW_COL", alpha=1.0,
                              row_bias=p["row_bias"], col_bias=p["col_bias"], want64=True)
        assert np.array_equal(one["D64"][0], full["D64"][l])


def test_bias_shape_checks():
    p = workloads.make_problem(1, 4, 6, 8, "BIAS_ROW_COL", init="small_int", seed=24)
    with pytest.raises(ValueError):
        oracle.gemm_epi(p["A"], p["B"], kind="BIAS_ROW_COL", row_bias=p["col_bias"], col_bias=p["row_bias"])
    with pytest.raises(ValueError):
        oracle.gemm_epi(p["A"], p["B"], kind="BIAS_ROW_COL", row_bias=p["row_bias"], col_bias=None)
