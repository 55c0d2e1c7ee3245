"""fp32 epilogue tensors on the GPU (gemm_epi_run_mixed, reached through run()
with float16 / bfloat16 A, B and float32 C, X, biases, D, Aux), against the
oracle's fp32-epilogue path (oracle.gemm_epi_f32e).

Bar: with integer A, B and fp32 C, X, biases of few significant bits, every
value before an output's rounding is exact in fp32 on the GPU and in fp64 in
the oracle, and the one rounding (of a square or of nothing) is the same
nearest-even on both sides: bit-exact, for every kind but the activations.
The activations (fp32 formulas accurate to about 1e-6) within 8e-6 relative
plus 2^-126 absolute of the oracle's unrounded value, GELU's left tail within
the bound its fp32 exponential's argument sets (activation_rel_bound).
Gaussian inputs:
|gpu - ref| <= 5e-2 + 1e-2 |ref|.
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_elementwise_amd as ge
from dense_gemm_elementwise_amd import workloads
from test_parity_gpu import KIND_SCALARS, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def ab_tensor(a, ab, offset):
    if ab == "f16":
        t = torch.from_numpy(np.ascontiguousarray(a))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return place(t, offset)


def place(t, offset):
    if not offset:
        return t.to(DEV)
    buf = torch.empty(t.numel() + offset, dtype=t.dtype, device=DEV)
    d = buf[offset:].view(t.shape)
    d.copy_(t)
    return d


def out32(shape, offset):
    n = int(np.prod(shape))
    return torch.full((n + offset,), float("nan"), dtype=torch.float32, device=DEV)[offset:].view(shape)


def problem(L, M, N, K, kind, ab, seed, init):
    rng = np.random.default_rng(seed)
    if init == "small_int":
        v = lambda shape: rng.integers(-2, 3, shape).astype(np.float32)                           # noqa: E731
        e = lambda shape: (rng.integers(-2 ** 20, 2 ** 20, shape) * 2.0 ** -7).astype(np.float32)  # noqa: E731
    else:
        v = lambda shape: rng.standard_normal(shape).astype(np.float32)                            # noqa: E731
        e = v
    A, B = v((L, M, K)), v((L, K, N))
    if ab == "f16":
        A, B = A.astype(np.float16), B.astype(np.float16)
    else:  # round to nearest even in the top 16 bits
        A, B = [((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
                for x in (A, B)]
    p = {"A": A, "B": B, "C": e((L, M, N)), "X": e((L, M, N)) if kind == "LINCOMB_X_ACC" else None,
         "row_bias": None, "col_bias": None}
    if kind == "BIAS_ROW_COL":
        p["row_bias"], p["col_bias"] = e((N,)), e((M,))
    return p


def run_gpu(p, kind, ab, a, b, s, offset):
    L, M, K = p["A"].shape
    N = p["B"].shape[2]
    A, B = ab_tensor(p["A"], ab, offset), ab_tensor(p["B"], ab, offset)
    f = lambda x: None if x is None else place(torch.from_numpy(x), offset)  # noqa: E731
    D = out32((L, M, N), offset)
    Aux = out32((L, M, N), offset) if kind in ge.HAS_AUX else None
    acc = out32((L, M, N), offset) if kind in ge.HAS_ACC else None
    ge.run(A, B, f(p["C"]), f(p["X"]), kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux, row_bias=f(p["row_bias"]),
           col_bias=f(p["col_bias"]), acc_out=acc)
    out = {"D": D.cpu().numpy()}
    if Aux is not None:
        out["Aux"] = Aux.cpu().numpy()
    if acc is not None:
        out["Acc"] = acc.cpu().numpy()
    return out


def activation_rel_bound(kind, lin):
    """Relative error bound of the kernels' fp32 activations.  8e-6 covers
    the formulas themselves (hardware exp2 and reciprocal, a few roundings).
    GELU's e^{-z^2} (z^2 = lin^2 / 2) also carries the roundings of its
    exponent's argument: each fp32 rounding of z, z*z and the log2(e) scaling
    moves the argument by up to z^2 * 2^-24 and the result by as much
    relative, and the factor is formed as a square, so 8 z^2 2^-24 is added;
    that term exceeds 1e-5 only for results below 1e-20."""
    if kind != "GELU":
        return 8e-6
    return 8e-6 + 8.0 * (lin * lin / 2.0) * 2.0 ** -24


def check(p, kind, ab, a, b, s, exact, offset=0, what=""):
    got = run_gpu(p, kind, ab, a, b, s, offset)
    ref = oracle.gemm_epi_f32e(p["A"], p["B"], p["C"], p["X"], kind=kind, alpha=a, beta=b, s3=s,
                               row_bias=p["row_bias"], col_bias=p["col_bias"], want64=True, ab_dtype=ab)
    for name in ("D", "Aux"):
        if name not in ref:
            continue
        g = got[name].astype(np.float64)
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite output"
        if exact and kind not in ge.ACTIVATIONS:
            bad = np.count_nonzero((got[name] != ref[name]) & ~((got[name] == 0) & (ref[name] == 0)))
            assert bad == 0, f"{what} {name}: {bad} of {g.size} elements differ from the oracle"
        elif exact:
            r = ref[name + "64"]
            err = np.abs(g - r)
            lin_all = a * ref["Acc64"] + b * np.asarray(p["C"], np.float64)
            ok = err <= activation_rel_bound(kind, lin_all) * np.abs(r) + 2.0 ** -126
            if not np.all(ok):
                w = np.argmax(np.where(ok, 0.0, err / (np.abs(r) + 2.0 ** -126)))
                lin = lin_all.ravel()[w]
                raise AssertionError(f"{what} {name}: {np.count_nonzero(~ok)} outside; worst at lin={lin!r}: "
                                     f"gpu {g.ravel()[w]!r} oracle {r.ravel()[w]!r}")
        else:
            r = ref[name + "64"]
            err = np.abs(g - r)
            assert np.all(err <= 5e-2 + 1e-2 * np.abs(r)), f"{what} {name}: max err {err.max()}"
    if kind in ge.HAS_ACC:
        if exact:
            assert np.array_equal(got["Acc"], ref["Acc"]), f"{what} acc_out"
        else:
            assert np.all(np.abs(got["Acc"] - ref["Acc64"]) <= 5e-2 + 1e-2 * np.abs(ref["Acc64"])), f"{what} acc"


@pytest.mark.parametrize("ab", ["f16", "bf16"])
@pytest.mark.parametrize("kind", workloads.KINDS)
@pytest.mark.parametrize("shape,offset", [((2, 200, 136, 264), 0),    # vector kernel, ragged M
                                          ((2, 200, 136, 264), 1),    # misaligned: general kernel
                                          ((3, 77, 45, 61), 0),       # K, N not multiples of 8: general
                                          ((1, 3112, 3928, 40), 0),   # 256 x 256 tiles (mixed types: 128 x 256)
                                          ((2, 300, 520, 648), 0),    # 64 x 64 x 128 tile (K >= 256), ragged last stage
                                          ((1, 1280, 1280, 648), 0),  # the same with the 2-stage ring (400 tiles)
                                          ((1, 300, 520, 136), 0),    # 64 x 64 x 64 tile (K < 256), ragged last stage
                                          ((1, 1960, 2000, 72), 0),   # 128 x 128 tiles, ragged M, N
                                          ((1, 2100, 2100, 61), 0)])  # general kernel, 256 x 128 tiles
def test_every_kind_integer_inputs(kind, ab, shape, offset):
    L, M, N, K = shape
    a, b, s = KIND_SCALARS[kind]
    log(f"[f32e] kind={kind} ab={ab} shape={shape} offset={offset}")
    p = problem(L, M, N, K, kind, ab, seed=M * N + K, init="small_int")
    check(p, kind, ab, a, b, s, exact=True, offset=offset, what=f"f32e {kind} {ab} {shape} off{offset}")


@pytest.mark.parametrize("ab", ["f16", "bf16"])
@pytest.mark.parametrize("kind", ["LINCOMB_X_ACC", "RELU_SQUARE", "RELU_SCALE_ACC", "BIAS_ROW_COL", "GELU"])
def test_gaussian_inputs(kind, ab):
    L, M, N, K = 2, 520, 392, 768
    a, b, s = KIND_SCALARS[kind]
    log(f"[f32e] gaussian kind={kind} ab={ab}")
    p = problem(L, M, N, K, kind, ab, seed=29, init="normal")
    check(p, kind, ab, a, b, s, exact=False, what=f"f32e gaussian {kind} {ab}")


def test_same_accumulator_as_the_16_bit_call():
    """The 8192^3-class tile on both epilogue types: with C, X exactly fp16,
    the fp16 outputs of the 16-bit call are the fp16 roundings of the fp32
    call's outputs (the same fp32 epilogue values, rounded once more)."""
    L, M, N, K = 1, 1024, 1024, 1024
    rng = np.random.default_rng(5)
    A = rng.standard_normal((L, M, K)).astype(np.float16)
    B = rng.standard_normal((L, K, N)).astype(np.float16)
    C = rng.standard_normal((L, M, N)).astype(np.float16)
    X = rng.standard_normal((L, M, N)).astype(np.float16)
    t = {k: torch.from_numpy(v).to(DEV) for k, v in (("A", A), ("B", B), ("C", C), ("X", X))}
    D16, Y16 = torch.empty((L, M, N), dtype=torch.float16, device=DEV), torch.empty((L, M, N), dtype=torch.float16,
                                                                                     device=DEV)
    D32, Y32 = out32((L, M, N), 0), out32((L, M, N), 0)
    ge.run(t["A"], t["B"], t["C"], t["X"], kind="LINCOMB_X_ACC", alpha=2.0, beta=1.0, s3=3.0, D=D16, Aux=Y16)
    ge.run(t["A"], t["B"], t["C"].float(), t["X"].float(), kind="LINCOMB_X_ACC", alpha=2.0, beta=1.0, s3=3.0,
           D=D32, Aux=Y32)
    assert torch.equal(D32.half(), D16) and torch.equal(Y32.half(), Y16)


def test_x_acc_8192_every_element():
    """The Alpha-Beta example's size with fp32 epilogue tensors: Gaussian fp16
    A, B and fp32 C, X; every D and Y element against the full oracle (fp64,
    about 14 s on 16 cores) within the Gaussian tolerance, none non-finite."""
    L, M, N, K = 1, 8192, 8192, 8192
    log("[f32e] x_acc 8192^3, every element")
    p = problem(L, M, N, K, "LINCOMB_X_ACC", "f16", seed=2025, init="normal")
    check(p, "LINCOMB_X_ACC", "f16", 2.0, 1.0, 3.0, exact=False, what="f32e x_acc 8192")
