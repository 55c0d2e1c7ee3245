"""Pins for the oracle's fused GEMM + epilogue (CPU only).

The oracle computes the plain definition epi(A @ B, ...) of the pages:
my_epilogue, relu_aux_store, relu_scale_return_acc and the row/column
broadcast epilogue (CUTLASS Operator API tutorial "Custom epilogue fusions
for GEMMs", cells [2], [6], [7], [9]), the Alpha-Beta example's
epilogue_operation, ReLU and the multi-output pair (CUTLASS "Custom Epilogue
Example": "Basic Example", "Activation Functions", "Multiple Outputs") and
D = alpha*(A@B) + beta*C (CUTLASS Python examples article, "Basic GEMM" /
"Epilogue").  It is pinned here to things other than itself:
  - exact rational arithmetic (fractions.Fraction) on tiny problems, with an
    independent nearest-fp16 search, for every epilogue kind;
  - NumPy's float64 matmul, which is exact on small-integer inputs (the
    pages' own exactness argument: integer-valued inputs compare exactly);
  - closed forms (A = 0, A = I, B = I), the transpose identity, invariants
    between kinds, hand-worked cases in tests/golden/hand_worked.json;
  - the fp64 accumulation error bound on Gaussian inputs.
"""
import bisect
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dense_gemm_elementwise_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")

# ---------------------------------------------------------------------------
# Independent exact reference: Fraction arithmetic + nearest fp16 by search.
# ---------------------------------------------------------------------------
_POS_BITS = np.arange(0, 0x7C00, dtype=np.uint16)
_POS_VALS = [Fraction(float(v)) for v in _POS_BITS.view(np.float16).astype(np.float64)]
_MAX_HALF = Fraction(65504)
_OVERFLOW = Fraction(65520)


def exact_rne_bits(q: Fraction, negative_zero=False) -> int:
    """Nearest fp16 (ties to the even bit pattern) of an exact rational."""
    if q == 0:
        return 0x8000 if negative_zero else 0
    sign = 0x8000 if q < 0 else 0
    a = -q if q < 0 else q
    if a >= _OVERFLOW:
        return sign | 0x7C00
    if a >= _MAX_HALF:
        return sign | 0x7BFF
    idx = bisect.bisect_left(_POS_VALS, a)
    if _POS_VALS[idx] == a:
        return sign | int(_POS_BITS[idx])
    lo, hi = idx - 1, idx
    dl, dh = a - _POS_VALS[lo], _POS_VALS[hi] - a
    if dl < dh:
        pick = lo
    elif dh < dl:
        pick = hi
    else:
        pick = lo if (int(_POS_BITS[lo]) & 1) == 0 else hi
    return sign | int(_POS_BITS[pick])


def frac(x):
    return Fraction(float(x))


def exact_rne_f32(q: Fraction) -> float:
    """Nearest float32 (ties to even) of an exact rational, found with integer
    arithmetic (no intermediate double rounding)."""
    if q == 0:
        return 0.0
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                    # subnormals share the quantum 2^-149
    scaled = a / Fraction(2) ** (e - 23)  # in [2^23, 2^24) for normal values
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = float(Fraction(n) * Fraction(2) ** (e - 23))
    if v > float(np.finfo(np.float32).max):
        v = float("inf")
    return -v if neg else v


def exact_outputs(A, B, C, X, kind, alpha, beta, s3, row_bias=None, col_bias=None):
    """Exact rational outputs of the definition, per element: D, the second
    output (or None) and the accumulator."""
    L, M, K = A.shape
    N = B.shape[2]
    al, be, s = frac(np.float32(alpha)), frac(np.float32(beta)), frac(np.float32(s3))
    D = np.empty((L, M, N), dtype=object)
    Aux = np.empty((L, M, N), dtype=object)
    Acc = np.empty((L, M, N), dtype=object)
    for l in range(L):
        for i in range(M):
            for j in range(N):
                acc = sum((frac(A[l, i, k]) * frac(B[l, k, j]) for k in range(K)), Fraction(0))
                c = frac(C[l, i, j]) if C is not None else Fraction(0)
                t = al * acc + be * c
                if kind == "LINCOMB":
                    d, aux = t, None
                elif kind == "AUX_SCALE":
                    d, aux = s * t, t
                elif kind == "LINCOMB_X_ACC":
                    d, aux = t + s * frac(X[l, i, j]), acc
                elif kind == "RELU":
                    d, aux = (t if t > 0 else Fraction(0)), None
                elif kind == "SQUARE":
                    d, aux = t, t * t
                elif kind == "RELU_SQUARE":
                    r = t if t > 0 else Fraction(0)
                    d, aux = r, r * r
                elif kind == "RELU_AUX_STORE":
                    d, aux = (t if t > 0 else Fraction(0)), t
                elif kind == "RELU_SCALE_ACC":
                    r = t if t > 0 else Fraction(0)
                    d, aux = s * r, r
                elif kind == "BIAS_ROW_COL":
                    d, aux = al * acc + frac(row_bias[j]) + frac(col_bias[i]), None
                D[l, i, j] = d
                Aux[l, i, j] = aux
                Acc[l, i, j] = acc
    return D, Aux, Acc


def bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


def same_value_bits(got_bits, want_bits):
    """Bitwise equality, with +0 and -0 treated as equal."""
    g = np.asarray(got_bits, np.uint16)
    w = np.asarray(want_bits, np.uint16)
    zero = ((g & 0x7FFF) == 0) & ((w & 0x7FFF) == 0)
    return np.all((g == w) | zero)


def run_oracle(p, kind, alpha, beta, s3, want64=False):
    return oracle.gemm_epi(p["A"], p["B"], p["C"], p["X"], kind=kind, alpha=alpha, beta=beta, s3=s3,
                           row_bias=p.get("row_bias"), col_bias=p.get("col_bias"), want64=want64)


# ---------------------------------------------------------------------------
# Brute force in exact arithmetic
# ---------------------------------------------------------------------------
def test_exhaustive_2x2x2_over_minus1_0_1():
    """All 3^8 pairs (A, B) of 2x2 matrices over {-1, 0, 1}, batched along L,
    for every kind, against exact arithmetic."""
    vals = np.array([-1, 0, 1], np.float16)
    idx = np.indices((3,) * 8).reshape(8, -1).T  # 6561 x 8
    A = vals[idx[:, :4]].reshape(-1, 2, 2)
    B = vals[idx[:, 4:]].reshape(-1, 2, 2)
    Lb = A.shape[0]
    rng = np.random.default_rng(7)
    C = rng.integers(-3, 4, (Lb, 2, 2)).astype(np.float16)
    X = rng.integers(-3, 4, (Lb, 2, 2)).astype(np.float16)
    # exact products of small integers: the sums are small integers too
    acc = np.einsum("lik,lkj->lij", A.astype(np.int64), B.astype(np.int64))
    rb = rng.integers(-3, 4, 2).astype(np.float16)   # row bias, one per column
    cb = rng.integers(-3, 4, 2).astype(np.float16)   # column bias, one per row
    for kind, (alpha, beta, s3) in {"LINCOMB": (1.0, 2.0, 0.0), "AUX_SCALE": (1.0, 2.0, 0.5),
                                    "LINCOMB_X_ACC": (2.0, 1.0, 3.0), "RELU": (1.0, -1.0, 0.0),
                                    "SQUARE": (-1.0, 1.0, 0.0), "RELU_SQUARE": (3.0, 1.0, 0.0),
                                    "RELU_AUX_STORE": (3.0, 2.0, 0.0), "RELU_SCALE_ACC": (1.0, -2.0, 0.5),
                                    "BIAS_ROW_COL": (-1.0, 0.0, 0.0)}.items():
        bias = kind == "BIAS_ROW_COL"
        out = oracle.gemm_epi(A, B, None if bias else C, X if kind == "LINCOMB_X_ACC" else None, kind=kind,
                              alpha=alpha, beta=beta, s3=s3, row_bias=rb if bias else None,
                              col_bias=cb if bias else None)
        # exact rational epilogue per element, then the independent RNE search
        t = [Fraction(int(a)) * Fraction(alpha) + Fraction(beta) * frac(c)
             for a, c in zip(acc.ravel(), C.ravel())]
        if kind == "LINCOMB":
            d = t
            aux = None
        elif kind == "AUX_SCALE":
            d, aux = [Fraction(s3) * v for v in t], t
        elif kind == "LINCOMB_X_ACC":
            d = [v + Fraction(s3) * frac(x) for v, x in zip(t, X.ravel())]
            aux = [Fraction(int(a)) for a in acc.ravel()]
        elif kind == "RELU":
            d, aux = [max(v, Fraction(0)) for v in t], None
        elif kind == "SQUARE":
            d, aux = t, [v * v for v in t]
        elif kind == "RELU_SQUARE":
            r = [max(v, Fraction(0)) for v in t]
            d, aux = r, [v * v for v in r]
        elif kind == "RELU_AUX_STORE":
            d, aux = [max(v, Fraction(0)) for v in t], t
        elif kind == "RELU_SCALE_ACC":
            r = [max(v, Fraction(0)) for v in t]
            d, aux = [Fraction(s3) * v for v in r], r
        else:  # BIAS_ROW_COL: element (l, i, j) gets row_bias[j] + col_bias[i]
            ij = np.indices((Lb, 2, 2)).reshape(3, -1).T
            d = [Fraction(alpha) * Fraction(int(a)) + frac(rb[j]) + frac(cb[i])
                 for a, (_, i, j) in zip(acc.ravel(), ij)]
            aux = None
        want_d = np.array([exact_rne_bits(v) for v in d], np.uint16)
        assert same_value_bits(bits(out["D"]).ravel(), want_d), kind
        if aux is not None:
            want_a = np.array([exact_rne_bits(v) for v in aux], np.uint16)
            assert same_value_bits(bits(out["Aux"]).ravel(), want_a), kind
        if kind in workloads.HAS_ACC:
            assert np.array_equal(out["Acc"].ravel(), acc.ravel().astype(np.float32)), kind


@pytest.mark.parametrize("shape", [(1, 4, 4, 4), (2, 3, 5, 2), (3, 2, 3, 7), (1, 1, 1, 1), (1, 5, 1, 3)])
@pytest.mark.parametrize("kind", workloads.EXACT_KINDS)
def test_random_fp16_tiny_against_exact(shape, kind):
    """Gaussian fp16 inputs on tiny non-square shapes (a transposed operand or a
    wrong index cannot pass): the unrounded fp64 outputs lie within the fp64
    summation bound of the exact result, and the fp16 outputs equal the
    exact result's nearest fp16 unless the exact value sits within that
    bound of a rounding boundary."""
    L, M, N, K = shape
    p = workloads.make_problem(L, M, N, K, kind, init="normal", seed=sum(shape) * 31 + len(kind))
    check_tiny_against_exact(p, kind, 1.5, -0.75, 2.0)


def check_tiny_against_exact(p, kind, alpha, beta, s3):
    """The oracle on problem p against exact rational arithmetic, as described
    in test_random_fp16_tiny_against_exact."""
    L, M, N, K = p["A"].shape[0], p["A"].shape[1], p["B"].shape[2], p["A"].shape[2]
    out = run_oracle(p, kind, alpha, beta, s3, want64=True)
    exD, exAux, exAcc = exact_outputs(p["A"], p["B"], p["C"], p["X"], kind, alpha, beta, s3,
                                      p["row_bias"], p["col_bias"])
    A64 = p["A"].astype(np.float64)
    B64 = p["B"].astype(np.float64)
    absprod = np.einsum("lik,lkj->lij", np.abs(A64), np.abs(B64))
    gamma = K * 2.0 ** -53 / (1 - K * 2.0 ** -53)
    # bound on |fl(acc) - acc|, propagated through at most two more roundings and
    # a square, with generous constants (values are O(10))
    bound = 8 * (gamma * absprod + 2.0 ** -50 * (1 + absprod)) * (1 + np.abs(absprod)) ** 2
    for name, ex in (("D", exD), ("Aux", exAux)):
        if name == "Aux" and kind not in workloads.HAS_AUX:
            continue
        got64 = out[name + "64"]
        got = bits(out[name])
        for idx in np.ndindex(got.shape):
            e = ex[idx]
            assert abs(Fraction(float(got64[idx])) - e) <= Fraction(float(bound[idx])), (name, idx)
            want = exact_rne_bits(e)
            # skip the (vanishingly rare) case where the bound straddles a rounding boundary
            lo = exact_rne_bits(e - Fraction(float(bound[idx])))
            hi = exact_rne_bits(e + Fraction(float(bound[idx])))
            if lo == hi == want:
                assert same_value_bits([got[idx]], [want]), (name, idx)
    if kind in workloads.HAS_ACC:
        for idx in np.ndindex(out["Acc"].shape):
            e = exAcc[idx]
            b = Fraction(float(bound[idx]))
            assert abs(Fraction(float(out["Acc64"][idx])) - e) <= b
            want = exact_rne_f32(e)
            if exact_rne_f32(e - b) == exact_rne_f32(e + b) == want:
                assert float(out["Acc"][idx]) == want, idx


@pytest.mark.parametrize("chunk", range(10))
def test_random_tiny_sweep_against_exact(chunk):
    """1,200 seeded random cases (120 per chunk): shapes L in 1..2, M, N in
    1..5, K in 1..9, every exactly checkable kind, Gaussian fp16 inputs and
    scalars drawn from small dyadic and non-dyadic sets, each against exact
    rational arithmetic."""
    rng = np.random.default_rng(20261203 + chunk)
    kinds = list(workloads.EXACT_KINDS)
    scal = [0.0, 1.0, -1.0, 0.5, 2.0, -0.75, 1.5, 0.1, 3.0]
    for case in range(120):
        L, M, N, K = int(rng.integers(1, 3)), int(rng.integers(1, 6)), int(rng.integers(1, 6)), int(rng.integers(1, 10))
        kind = kinds[(chunk * 120 + case) % len(kinds)]
        p = workloads.make_problem(L, M, N, K, kind, init="normal", seed=int(rng.integers(0, 2**31)))
        alpha, beta, s3 = (float(rng.choice(scal)) for _ in range(3))
        check_tiny_against_exact(p, kind, alpha, beta, s3)


# ---------------------------------------------------------------------------
# Library special case: exact integer products agree with NumPy float64 matmul
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(1, 37, 29, 53), (2, 64, 48, 96), (1, 128, 128, 128), (3, 17, 70, 9)])
def test_integer_accumulator_equals_numpy_matmul(shape):
    L, M, N, K = shape
    p = workloads.make_problem(L, M, N, K, "LINCOMB", init="small_int", seed=L * M + N + K)
    out = run_oracle(p, "LINCOMB", 1.0, 0.0, 0.0, want64=True)
    ref = np.matmul(p["A"].astype(np.float64), p["B"].astype(np.float64))
    assert np.array_equal(out["D64"], ref)


def test_page_workload_aux_scale_128_accumulator_exact():
    """The 128^3 my_epilogue workload: Aux equals NumPy's exact float64
    alpha*(A@B) + beta*C and D equals Aux/2, both representable in fp16 (so
    the comparison is exact, as the pages' integer-input checks are)."""
    w = workloads.WORKLOADS["aux_scale_128"]
    p = workloads.make_inputs(w)
    out = run_oracle(p, w.kind, w.alpha, w.beta, w.s3, want64=True)
    acc = np.matmul(p["A"].astype(np.float64), p["B"].astype(np.float64))
    aux = w.alpha * acc + w.beta * p["C"].astype(np.float64)
    assert np.array_equal(out["Aux64"], aux)
    assert np.array_equal(out["D64"], aux * 0.5)
    assert np.all(np.abs(aux) <= 2048)  # every value is exactly representable
    assert np.array_equal(out["Aux"].astype(np.float64), aux)
    assert np.array_equal(out["D"].astype(np.float64), aux * 0.5)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind", workloads.EXACT_KINDS)
def test_zero_A_closed_forms(kind):
    L, M, N, K = 2, 19, 23, 11
    p = workloads.make_problem(L, M, N, K, kind, init="normal", seed=5)
    p["A"] = np.zeros_like(p["A"])
    alpha, beta, s3 = 1.25, -2.0, 0.5
    out = run_oracle(p, kind, alpha, beta, s3)
    bc = beta * p["C"].astype(np.float64) if p["C"] is not None else None  # exact: |beta| is a power of two
    if kind == "LINCOMB":
        d, aux = bc, None
    elif kind == "AUX_SCALE":
        d, aux = s3 * bc, bc
    elif kind == "LINCOMB_X_ACC":
        d, aux = bc + s3 * p["X"].astype(np.float64), np.zeros_like(bc)
    elif kind == "RELU":
        d, aux = np.maximum(bc, 0.0), None
    elif kind == "SQUARE":
        d, aux = bc, bc * bc
    elif kind == "RELU_SQUARE":
        d = np.maximum(bc, 0.0)
        aux = d * d
    elif kind == "RELU_AUX_STORE":
        d, aux = np.maximum(bc, 0.0), bc
    elif kind == "RELU_SCALE_ACC":
        aux = np.maximum(bc, 0.0)
        d = s3 * aux
    else:  # BIAS_ROW_COL: row bias of the column plus column bias of the row
        d = (p["row_bias"].astype(np.float64)[None, None, :] + p["col_bias"].astype(np.float64)[None, :, None]
             + np.zeros((L, M, N)))
        aux = None
    # each of these is exact in float64, so NumPy's float16 cast is the single rounding
    assert same_value_bits(bits(out["D"]), d.astype(np.float16).view(np.uint16))
    if aux is not None:
        assert same_value_bits(bits(out["Aux"]), aux.astype(np.float16).view(np.uint16))
    if kind in workloads.HAS_ACC:
        assert np.all(out["Acc"] == 0.0)


def test_identity_A_gives_B_and_identity_B_gives_A():
    L, M, N = 2, 24, 40
    p = workloads.make_problem(L, M, N, M, "LINCOMB", init="normal", seed=11)
    eye = np.broadcast_to(np.eye(M, dtype=np.float16), (L, M, M)).copy()
    out = oracle.gemm_epi(eye, p["B"], p["C"], kind="LINCOMB", alpha=1.0, beta=0.0)
    assert np.array_equal(bits(out["D"]), bits(p["B"]))
    K = 33
    q = workloads.make_problem(L, M, K, K, "LINCOMB", init="normal", seed=12)
    eyeK = np.broadcast_to(np.eye(K, dtype=np.float16), (L, K, K)).copy()
    out = oracle.gemm_epi(q["A"], eyeK, q["C"], kind="LINCOMB", alpha=1.0, beta=0.0)
    assert np.array_equal(bits(out["D"]), bits(q["A"]))


def test_transpose_identity():
    """(A B)^T = B^T A^T: with every product commuting exactly and the same
    k order, the transposed problem gives the transposed result bit for bit."""
    L, M, N, K = 2, 13, 21, 34
    p = workloads.make_problem(L, M, N, K, "LINCOMB", init="normal", seed=13)
    out = oracle.gemm_epi(p["A"], p["B"], p["C"], kind="LINCOMB", alpha=1.0, beta=1.0, want64=True)
    At = np.ascontiguousarray(p["A"].transpose(0, 2, 1))
    Bt = np.ascontiguousarray(p["B"].transpose(0, 2, 1))
    Ct = np.ascontiguousarray(p["C"].transpose(0, 2, 1))
    outT = oracle.gemm_epi(Bt, At, Ct, kind="LINCOMB", alpha=1.0, beta=1.0, want64=True)
    assert np.array_equal(outT["D64"].transpose(0, 2, 1), out["D64"])


def test_batches_are_independent():
    """A batched call equals one call per batch entry."""
    L, M, N, K = 3, 9, 14, 20
    p = workloads.make_problem(L, M, N, K, "LINCOMB_X_ACC", init="normal", seed=14)
    full = run_oracle(p, "LINCOMB_X_ACC", 2.0, 1.0, 3.0, want64=True)
    for l in range(L):
        one = oracle.gemm_epi(p["A"][l:l + 1], p["B"][l:l + 1], p["C"][l:l + 1], p["X"][l:l + 1],
                              kind="LINCOMB_X_ACC", alpha=2.0, beta=1.0, s3=3.0, want64=True)
        assert np.array_equal(one["D64"][0], full["D64"][l])
        assert np.array_equal(one["Aux64"][0], full["Aux64"][l])


# ---------------------------------------------------------------------------
# Invariants between kinds
# ---------------------------------------------------------------------------
def test_kind_invariants():
    L, M, N, K = 2, 31, 45, 64
    p = workloads.make_problem(L, M, N, K, "LINCOMB_X_ACC", init="normal", seed=15)
    a, b = 1.0, 2.0
    lin = run_oracle(p, "LINCOMB", a, b, 0.0, want64=True)
    aux = run_oracle(p, "AUX_SCALE", a, b, 0.5, want64=True)
    relu = run_oracle(p, "RELU", a, b, 0.0)
    sq = run_oracle(p, "SQUARE", a, b, 0.0, want64=True)
    rsq = run_oracle(p, "RELU_SQUARE", a, b, 0.0, want64=True)
    # AUX_SCALE's Aux is LINCOMB's D; halving a normal fp16 value (exponent >= 2)
    # subtracts one from its exponent field
    assert np.array_equal(bits(aux["Aux"]), bits(lin["D"]))
    ab = bits(aux["Aux"]).astype(np.int32)
    normal = ((ab >> 10) & 31) >= 2
    normal &= ((ab >> 10) & 31) < 31
    assert np.array_equal(bits(aux["D"])[normal], (ab[normal] - 0x400).astype(np.uint16))
    # RELU is LINCOMB clamped at +0
    lind = lin["D"].astype(np.float64)
    assert np.array_equal(relu["D"].astype(np.float64), np.where(lind > 0, lind, 0.0))
    # SQUARE's D is LINCOMB's D, E is the square of the unrounded D
    assert np.array_equal(bits(sq["D"]), bits(lin["D"]))
    assert np.array_equal(sq["Aux64"], sq["D64"] * sq["D64"])
    assert np.array_equal(bits(sq["Aux"]), sq["Aux64"].astype(np.float16).view(np.uint16))
    # RELU_SQUARE's D is RELU's D; E is 0 where D is 0
    assert np.array_equal(rsq["D"].astype(np.float64), relu["D"].astype(np.float64))
    assert np.all(rsq["Aux"][rsq["D64"] == 0] == 0)
    # X_ACC with X = 0 gives LINCOMB's D; its Y is LINCOMB with alpha 1, beta 0
    q = dict(p)
    q["X"] = np.zeros_like(p["X"])
    xz = run_oracle(q, "LINCOMB_X_ACC", a, b, 3.0)
    assert same_value_bits(bits(xz["D"]), bits(lin["D"]))
    acc_only = run_oracle(p, "LINCOMB", 1.0, 0.0, 0.0)
    xa = run_oracle(p, "LINCOMB_X_ACC", a, b, 3.0)
    assert same_value_bits(bits(xa["Aux"]), bits(acc_only["D"]))


# ---------------------------------------------------------------------------
# Hand-worked cases
# ---------------------------------------------------------------------------
def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_worked(case):
    def arr(x):
        return np.array([[float(v) for v in row] for row in x], np.float16)[None]

    def vec(x):
        return np.array([float(v) for v in x], np.float16)
    A, B = arr(case["A"]), arr(case["B"])
    C = arr(case["C"]) if "C" in case else None
    X = arr(case["X"]) if "X" in case else None
    rb = vec(case["row_bias"]) if "row_bias" in case else None
    cb = vec(case["col_bias"]) if "col_bias" in case else None
    out = oracle.gemm_epi(A, B, C, X, kind=case["kind"], alpha=case["alpha"], beta=case["beta"], s3=case["s3"],
                          row_bias=rb, col_bias=cb)
    assert np.array_equal(out["D"][0].astype(np.float64), arr(case["D"])[0].astype(np.float64))
    if "Aux" in case:
        assert np.array_equal(out["Aux"][0].astype(np.float64), arr(case["Aux"])[0].astype(np.float64))
    if "Acc" in case:
        assert np.array_equal(out["Acc"][0].astype(np.float64), arr(case["Acc"])[0].astype(np.float64))


# ---------------------------------------------------------------------------
# Gaussian inputs: fp64 accumulation error bound, and the sampled-point entry
# ---------------------------------------------------------------------------
def test_gaussian_accumulator_within_fp64_bound():
    L, M, N, K = 1, 48, 40, 2048
    p = workloads.make_problem(L, M, N, K, "LINCOMB", init="normal", seed=16)
    out = run_oracle(p, "LINCOMB", 1.0, 0.0, 0.0, want64=True)
    A64 = p["A"].astype(np.float64)
    B64 = p["B"].astype(np.float64)
    # exact reference: float64 products are exact (11 x 11 bits); sum them with
    # math.fsum, which is correctly rounded
    import math
    ref = np.array([[math.fsum(A64[0, i, :] * B64[0, :, j]) for j in range(N)] for i in range(M)])
    bound = K * 2.0 ** -53 * np.abs(A64[0]) @ np.abs(B64[0])
    assert np.all(np.abs(out["D64"][0] - ref) <= bound)


@pytest.mark.parametrize("kind", workloads.KINDS)
def test_points_equal_full(kind):
    L, M, N, K = 2, 33, 27, 70
    p = workloads.make_problem(L, M, N, K, kind, init="normal", seed=17)
    full = run_oracle(p, kind, 1.5, 0.5, 2.0, want64=True)
    rng = np.random.default_rng(3)
    n = 200
    l, i, j = rng.integers(0, L, n), rng.integers(0, M, n), rng.integers(0, N, n)
    pts = oracle.gemm_epi_points(p["A"], p["B"], p["C"], p["X"], kind=kind, alpha=1.5, beta=0.5, s3=2.0,
                                 row_bias=p["row_bias"], col_bias=p["col_bias"], l=l, i=i, j=j)
    assert np.array_equal(bits(pts["D"]), bits(full["D"][l, i, j]))
    assert np.array_equal(pts["D64"], full["D64"][l, i, j])
    assert np.array_equal(pts["Acc64"], full["Acc64"][l, i, j])
    if kind in workloads.HAS_AUX:
        assert np.array_equal(bits(pts["Aux"]), bits(full["Aux"][l, i, j]))
    if kind in workloads.HAS_ACC:
        assert np.array_equal(pts["Acc"], full["Acc"][l, i, j])


def test_rejects_invalid_arguments(oracle_lib):
    import ctypes
    h = np.zeros(16, np.uint16)
    sc = np.zeros(3, np.float32)
    f = oracle_lib.oracle_gemm_epi
    P = h.ctypes.data
    S = sc.ctypes.data
    assert f(0, 1, 1, 1, P, P, P, P, S, 0, P, P, None, None) == 1
    assert f(1, 1, 1, 1, None, P, P, P, S, 0, P, P, None, None) == 2
    assert f(1, 1, 1, 1, P, P, P, None, S, 2, P, P, None, None) == 2
    assert f(1, 1, 1, 1, P, P, P, P, S, 15, P, P, None, None) == 4
    assert f(1, 1, 1, 1, P, P, P, P, S, -1, P, P, None, None) == 4
    assert f(1, 1, 1, 1, P, P, P, P, S, 1, P, None, None, None) == 3
    assert f(1, 1, 1, 1, P, P, P, P, S, 0, None, None, None, None) == 3
    assert f(1, 1, 1, 1, P, P, P, None, S, 0, P, None, None, None) == 0
    # the entry point without bias inputs / accumulator output rejects the kinds that need them
    assert f(1, 1, 1, 1, P, P, P, P, S, 8, P, P, None, None) == 2
    assert f(1, 1, 1, 1, P, P, P, P, S, 7, P, P, None, None) == 3
    g = oracle_lib.oracle_gemm_epi_ext
    acc = np.zeros(4, np.float32)
    Q = acc.ctypes.data
    assert g(1, 1, 1, 1, P, P, None, None, P, P, S, 8, P, None, None, None, None, None) == 0  # no C
    assert g(1, 1, 1, 1, P, P, None, None, P, None, S, 8, P, None, None, None, None, None) == 2
    assert g(1, 1, 1, 1, P, P, None, None, P, P, S, 7, P, P, Q, None, None, None) == 2     # kind 7 reads C
    assert g(1, 1, 1, 1, P, P, P, None, None, None, S, 7, P, P, None, None, None, None) == 3
    assert g(1, 1, 1, 1, P, P, P, None, None, None, S, 7, P, P, Q, None, None, None) == 0
    assert g(1, 1, 1, 1, P, P, P, None, None, None, S, 6, P, None, None, None, None, None) == 3
    assert g(1, 1, 1, 1, P, P, P, P, P, P, S, 15, P, P, Q, None, None, None) == 4
    del ctypes
