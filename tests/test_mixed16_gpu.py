"""Mixed 16-bit element types on the GPU (gemm_epi_run_mixed through run():
fp16 A, B with bfloat16 C, X, biases, D, Aux, and bfloat16 A, B with fp16
ones), against the oracle with the same pair of types.

Bar, as for one element type: on integer inputs every product and partial
sum is exact and the final store is the only rounding on both sides, so the
outputs are bit-identical (+0 and -0 equal); activations within one ulp of
the epilogue type and at least 98% bit-identical.  Gaussian inputs:
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
TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


def bits_of(v, dtype):
    """float32 values -> uint16 bit patterns of that type (nearest-even)."""
    v = np.asarray(v, np.float32)
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    u = v.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def decode(b, dtype):
    return oracle.f16_decode(b) if dtype == "f16" else oracle.bf16_decode(b)


def to_dev(b, dtype, offset):
    t = torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(TORCH[dtype])
    if not offset:
        return t.to(DEV)
    buf = torch.empty(t.numel() + offset, dtype=t.dtype, device=DEV)
    d = buf[offset:].view(t.shape)
    d.copy_(t)
    return d


def out16(shape, dtype, offset):
    n = int(np.prod(shape))
    return torch.full((n + offset,), float("nan"), dtype=TORCH[dtype], device=DEV)[offset:].view(shape)


def problem(L, M, N, K, kind, ab, epi, seed, init):
    rng = np.random.default_rng(seed)
    draw = (lambda shape: rng.integers(-2, 3, shape).astype(np.float32)) if init == "small_int" else \
        (lambda shape: rng.standard_normal(shape).astype(np.float32))
    p = {"A": bits_of(draw((L, M, K)), ab), "B": bits_of(draw((L, K, N)), ab), "C": bits_of(draw((L, M, N)), epi),
         "X": bits_of(draw((L, M, N)), epi) if kind == "LINCOMB_X_ACC" else None, "row_bias": None, "col_bias": None}
    if kind == "BIAS_ROW_COL":
        p["row_bias"], p["col_bias"] = bits_of(draw((N,)), epi), bits_of(draw((M,)), epi)
    return p


def check(p, kind, ab, epi, a, b, s, exact, offset=0, what=""):
    L, M, K = p["A"].shape
    N = p["B"].shape[2]
    f = lambda x: None if x is None else to_dev(x, epi, offset)  # noqa: E731
    D = out16((L, M, N), epi, offset)
    Aux = out16((L, M, N), epi, offset) if kind in ge.HAS_AUX else None
    acc = torch.full((L * M * N + offset,), float("nan"), dtype=torch.float32, device=DEV)[offset:].view(L, M, N) \
        if kind in ge.HAS_ACC else None
    ge.run(to_dev(p["A"], ab, offset), to_dev(p["B"], ab, offset), f(p["C"]), f(p["X"]), kind=kind, alpha=a, beta=b,
           s3=s, D=D, Aux=Aux, row_bias=f(p["row_bias"]), col_bias=f(p["col_bias"]), acc_out=acc)
    ref = oracle.gemm_epi(p["A"], p["B"], p["C"], p["X"], kind=kind, alpha=a, beta=b, s3=s, row_bias=p["row_bias"],
                          col_bias=p["col_bias"], want64=True, dtype=ab, epi_dtype=epi)
    for name, t in (("D", D), ("Aux", Aux)):
        if t is None:
            continue
        got = t.cpu().view(torch.int16).numpy().view(np.uint16)
        want = np.asarray(ref[name]).view(np.uint16)
        g = decode(got, epi)
        # non-finite only where the oracle's rounded output overflows too (E = D*D can pass fp16's 65504)
        assert np.all(np.isfinite(g) | ~np.isfinite(decode(want, epi))), f"{what} {name}: non-finite"
        if exact and kind not in ge.ACTIVATIONS:
            bad = np.count_nonzero((got != want) & (((got | want) & 0x7FFF) != 0))
            assert bad == 0, f"{what} {name}: {bad} of {got.size} differ"
        elif exact:
            r64 = ref[name + "64"]
            ulp = np.abs(decode(want ^ 1, epi) - decode(want, epi))  # one step of the epilogue type at the result
            assert np.all(np.abs(g - r64) <= np.maximum(ulp, 2.0 ** -133)), f"{what} {name}: more than 1 ulp off"
            assert np.mean(got == want) >= 0.98, f"{what} {name}: too few bit-identical"
        else:
            r64 = ref[name + "64"]
            assert np.all(np.abs(g - r64) <= 5e-2 + 1e-2 * np.abs(r64)), f"{what} {name}"
    if acc is not None:
        got = acc.cpu().numpy()
        if exact:
            assert np.array_equal(got, ref["Acc"]), f"{what} acc_out"
        else:
            assert np.all(np.abs(got - ref["Acc64"]) <= 5e-2 + 1e-2 * np.abs(ref["Acc64"])), f"{what} acc_out"


PAIRS = [("f16", "bf16"), ("bf16", "f16")]


@pytest.mark.parametrize("ab,epi", PAIRS)
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
def test_every_kind_integer_inputs(kind, ab, epi, shape, offset):
    L, M, N, K = shape
    a, b, s = KIND_SCALARS[kind]
    log(f"[mixed16] kind={kind} {ab}->{epi} shape={shape} offset={offset}")
    p = problem(L, M, N, K, kind, ab, epi, seed=M * N + K, init="small_int")
    check(p, kind, ab, epi, a, b, s, exact=True, offset=offset, what=f"mixed16 {kind} {ab}->{epi} {shape}")


@pytest.mark.parametrize("ab,epi", PAIRS)
@pytest.mark.parametrize("kind", ["LINCOMB_X_ACC", "RELU_SCALE_ACC", "GELU"])
def test_gaussian_inputs(kind, ab, epi):
    L, M, N, K = 2, 520, 392, 768
    a, b, s = KIND_SCALARS[kind]
    log(f"[mixed16] gaussian kind={kind} {ab}->{epi}")
    p = problem(L, M, N, K, kind, ab, epi, seed=31, init="normal")
    check(p, kind, ab, epi, a, b, s, exact=False, what=f"mixed16 gaussian {kind} {ab}->{epi}")
