"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Bar (per the method's exactness argument: integer-valued fp16 inputs make
every fp32 partial sum exact, so the only rounding is the final fp16 store):
  - integer-valued inputs: every output bit-identical to the oracle (+0 and
    -0 compare equal);
  - Gaussian inputs: |gpu - ref| <= 5e-2 + 1e-2 * |ref| for every compared
    element, ref = the oracle's unrounded fp64 value, and no non-finite
    output.
  - activation kinds (sigmoid, tanh, GELU, SiLU, leaky ReLU, hardswish) on
    integer-valued inputs with scalars that keep alpha*acc + beta*C exact in
    fp32: within one fp16 unit in the last place of the oracle's unrounded
    value, and at least 98% bit-identical to the oracle's fp16 (the fp32
    activations are accurate to about 1e-6, so they differ from the correctly
    rounded value only next to a rounding boundary).
Full-size problems that the oracle cannot finish in seconds are compared at
sampled points (the oracle's per-element entry) plus whole-output properties
that hold at any size.
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_elementwise_amd as ge
from dense_gemm_elementwise_amd import workloads

pytestmark = pytest.mark.gpu

ATOL, RTOL = 5e-2, 1e-2
DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)


def to_dev(p, offset=0):
    """Uploads host arrays; offset > 0 places each tensor `offset` elements into
    a larger buffer (misaligned pointers, the general kernel)."""
    out = {}
    for k, v in p.items():
        if v is None:
            out[k] = None
            continue
        if offset:
            buf = torch.empty(v.size + offset, dtype=torch.float16, device=DEV)
            t = buf[offset:].view(v.shape)
            t.copy_(torch.from_numpy(v))
        else:
            t = torch.from_numpy(v).to(DEV)
        out[k] = t
    return out


def alloc_out(L, M, N, offset=0, dtype=torch.float16):
    if offset:
        return torch.full((L * M * N + offset,), float("nan"), dtype=dtype, device=DEV)[offset:].view(L, M, N)
    return torch.full((L, M, N), float("nan"), dtype=dtype, device=DEV)


def gpu_run(p, kind, alpha, beta, s3, offset=0):
    t = to_dev(p, offset)
    L, M, K = p["A"].shape
    N = p["B"].shape[2]
    D = alloc_out(L, M, N, offset)
    Aux = alloc_out(L, M, N, offset) if kind in ge.HAS_AUX else None
    acc = alloc_out(L, M, N, offset, torch.float32) if kind in ge.HAS_ACC else None
    ge.run(t["A"], t["B"], t["C"], t["X"], kind=kind, alpha=alpha, beta=beta, s3=s3, D=D, Aux=Aux,
           row_bias=t.get("row_bias"), col_bias=t.get("col_bias"), acc_out=acc)
    out = {"D": D.cpu().numpy()}
    if Aux is not None:
        out["Aux"] = Aux.cpu().numpy()
    if acc is not None:
        out["Acc"] = acc.cpu().numpy()
    return out


def oracle_full(p, kind, alpha, beta, s3, want64):
    return oracle.gemm_epi(p["A"], p["B"], p["C"], p["X"], kind=kind, alpha=alpha, beta=beta, s3=s3,
                           row_bias=p.get("row_bias"), col_bias=p.get("col_bias"), want64=want64)


def oracle_points(p, kind, alpha, beta, s3, l, i, j):
    return oracle.gemm_epi_points(p["A"], p["B"], p["C"], p["X"], kind=kind, alpha=alpha, beta=beta, s3=s3,
                                  row_bias=p.get("row_bias"), col_bias=p.get("col_bias"), l=l, i=i, j=j)


def bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


def assert_bit_exact(got, want, what):
    g, w = bits(got), bits(want)
    zero = ((g & 0x7FFF) == 0) & ((w & 0x7FFF) == 0)
    bad = (g != w) & ~zero
    n = int(np.count_nonzero(bad))
    if n:
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(i), float(np.asarray(got)[tuple(i)]), float(np.asarray(want)[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {n} of {g.size} outputs differ from the oracle, e.g. {detail}")


def assert_close(got, ref64, what, overflow=None):
    """Within ATOL + RTOL |ref| of the oracle's unrounded value.  overflow, the
    format's overflow threshold (65520 for fp16), admits +-inf where the
    unrounded value is within the tolerance of it or beyond, with its sign;
    without it every output must be finite."""
    g = np.asarray(got, np.float64)
    lim = ATOL + RTOL * np.abs(ref64)
    if overflow is None:
        assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    else:
        inf = np.isinf(g)
        ok = inf & (np.sign(g) == np.sign(ref64)) & (np.abs(ref64) >= overflow - lim)
        assert np.all(~np.isnan(g)) and np.all(ok | ~inf), f"{what}: an infinity where the oracle's value is finite"
        g = np.where(inf, ref64, g)
    err = np.abs(g - ref64)
    bad = err > lim
    n = int(np.count_nonzero(bad))
    if n:
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{what}: {n} of {g.size} outside tolerance; worst at {i}: gpu {g[i]} ref {ref64[i]}")


def ulp16(x):
    """fp16 spacing at |x| (2^-24 in the subnormal range)."""
    ax = np.abs(np.asarray(x, np.float64))
    return 2.0 ** (np.floor(np.log2(np.maximum(ax, 2.0 ** -14))) - 10)


def assert_within_ulp(got, ref64, ref16, what, min_exact=0.98):
    """Activation outputs: within one fp16 ulp of the oracle's unrounded value,
    and mostly bit-identical to the oracle's correctly rounded fp16."""
    g = np.asarray(got, np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref64)
    lim = ulp16(ref64)
    bad = err > lim
    n = int(np.count_nonzero(bad))
    if n:
        i = np.unravel_index(np.argmax(err / lim), err.shape)
        raise AssertionError(f"{what}: {n} of {g.size} more than 1 ulp off; worst at {i}: gpu {g[i]} ref {ref64[i]}")
    same = float(np.mean(g == np.asarray(ref16, np.float64)))
    assert same >= min_exact, f"{what}: only {same:.4f} of the outputs equal the oracle's fp16"


def oracle_ref(p, kind, alpha, beta, s3, exact):
    return oracle_full(p, kind, alpha, beta, s3, want64=(not exact) or kind in ge.ACTIVATIONS)


def assert_output(got, ref, name, kind, exact, what):
    """The bar for one output: bit-exact (integer inputs), the activation ulp
    bound (integer inputs, activation kinds), or the tolerance (Gaussian)."""
    if exact and kind in ge.ACTIVATIONS:
        assert_within_ulp(got, ref[name + "64"], ref[name], what)
    elif exact:
        assert_bit_exact(got, ref[name], what)
    else:
        assert_close(got, ref[name + "64"], what)


def check_full(p, kind, alpha, beta, s3, exact, offset=0, what=""):
    got = gpu_run(p, kind, alpha, beta, s3, offset)
    ref = oracle_ref(p, kind, alpha, beta, s3, exact)
    for name in ("D", "Aux"):
        if name not in ref:
            continue
        assert_output(got[name], ref, name, kind, exact, f"{what} {name}")
    if kind in ge.HAS_ACC:
        if exact:  # integer inputs: every fp32 partial sum is exact
            n = int(np.count_nonzero(got["Acc"] != ref["Acc"]))
            assert n == 0, f"{what} acc_out: {n} values differ from the oracle"
        else:
            assert_close(got["Acc"], ref["Acc64"], f"{what} acc_out")
    return got


# ---------------------------------------------------------------------------
# The five workloads at their real sizes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["aux_scale_128", "aux_scale_1024", "lincomb_2400x3232x4096",
                                  "relu_aux_store_1024", "relu_scale_acc_1024"])
def test_integer_workloads_bit_exact(name):
    w = workloads.WORKLOADS[name]
    log(f"[parity] {name}: L={w.L} M={w.M} N={w.N} K={w.K} {w.kind}")
    p = workloads.make_inputs(w)
    check_full(p, w.kind, w.alpha, w.beta, w.s3, exact=True, what=name)


def test_bias_workload_1024():
    """The tutorial's broadcast epilogue on its own draws: integer A, B and
    Gaussian fp16 biases, so the tolerance applies."""
    w = workloads.WORKLOADS["bias_row_col_1024"]
    log(f"[parity] {w.name}: L={w.L} M={w.M} N={w.N} K={w.K} {w.kind}")
    p = workloads.make_inputs(w)
    check_full(p, w.kind, w.alpha, w.beta, w.s3, exact=False, what=w.name)


def sample_points(L, M, N, n, seed, tile=256):
    """Random points plus every element of a few rows and columns at tile
    edges (first/last row and column of tiles, the matrix edges)."""
    rng = np.random.default_rng(seed)
    l = [rng.integers(0, L, n)]
    i = [rng.integers(0, M, n)]
    j = [rng.integers(0, N, n)]
    rows = sorted({0, 1, tile - 1, tile, M // 2, M - 2, M - 1} & set(range(M)))
    cols = sorted({0, 31, 32, tile - 1, tile, N // 2, N - 1} & set(range(N)))
    for r in rows:
        cj = rng.choice(N, size=min(N, 512), replace=False)
        l.append(rng.integers(0, L, cj.size))
        i.append(np.full(cj.size, r))
        j.append(cj)
    for c in cols:
        ri = rng.choice(M, size=min(M, 512), replace=False)
        l.append(rng.integers(0, L, ri.size))
        i.append(ri)
        j.append(np.full(ri.size, c))
    return np.concatenate(l), np.concatenate(i), np.concatenate(j)


def test_x_acc_8192_sampled_and_properties():
    w = workloads.WORKLOADS["x_acc_8192"]
    log(f"[parity] {w.name}: L={w.L} M={w.M} N={w.N} K={w.K} {w.kind}")
    p = workloads.make_inputs(w)
    t = to_dev(p)
    D = alloc_out(w.L, w.M, w.N)
    Y = alloc_out(w.L, w.M, w.N)
    ge.run(t["A"], t["B"], t["C"], t["X"], kind=w.kind, alpha=w.alpha, beta=w.beta, s3=w.s3, D=D, Aux=Y)
    # whole-output properties: finite everywhere, and D agrees with the
    # epilogue applied to the stored Y = acc (Y is acc rounded once, so
    # |D - (alpha Y + beta C + x X)| <= alpha ulp(Y) + ulp(D)/2 + fp32 slack)
    assert bool(torch.isfinite(D).all()) and bool(torch.isfinite(Y).all())
    D64, Y64 = D.double(), Y.double()
    C64, X64 = t["C"].double(), t["X"].double()
    recon = w.alpha * Y64 + w.beta * C64 + w.s3 * X64
    lim = 2.0 ** -10 * w.alpha * Y64.abs() + 2.0 ** -10 * D64.abs() + 1e-4
    assert bool(((D64 - recon).abs() <= lim).all()), "D inconsistent with Y, C, X somewhere"
    del D64, Y64, C64, X64, recon, lim
    # sampled points against the oracle
    l, i, j = sample_points(w.L, w.M, w.N, 20000, seed=1)
    ref = oracle.gemm_epi_points(p["A"], p["B"], p["C"], p["X"], kind=w.kind, alpha=w.alpha, beta=w.beta,
                                 s3=w.s3, l=l, i=i, j=j)
    d = D.cpu().numpy()[l, i, j]
    y = Y.cpu().numpy()[l, i, j]
    assert_close(d, ref["D64"], "x_acc_8192 D")
    assert_close(y, ref["Aux64"], "x_acc_8192 Y")


def test_relu_square_batched_sampled_and_properties():
    w = workloads.WORKLOADS["relu_square_16x2048x2048x1024"]
    log(f"[parity] {w.name}: L={w.L} M={w.M} N={w.N} K={w.K} {w.kind}")
    p = workloads.make_inputs(w)
    t = to_dev(p)
    D = alloc_out(w.L, w.M, w.N)
    E = alloc_out(w.L, w.M, w.N)
    ge.run(t["A"], t["B"], t["C"], kind=w.kind, alpha=w.alpha, beta=w.beta, s3=w.s3, D=D, Aux=E)
    assert bool(torch.isfinite(D).all()) and bool(torch.isfinite(E).all())
    assert bool((D >= 0).all()), "ReLU output negative"
    D64, E64 = D.double(), E.double()
    assert bool(((E64 - D64 * D64).abs() <= 2.0 ** -8 * D64 * D64 + 1e-6).all()), "E != D*D somewhere"
    del D64, E64
    # two whole batch entries (first and last) against the full oracle
    Dh, Eh = D.cpu().numpy(), E.cpu().numpy()
    for l in (0, w.L - 1):
        sub = {k: (v[l:l + 1] if v is not None else None) for k, v in p.items()}
        ref = oracle.gemm_epi(sub["A"], sub["B"], sub["C"], None, kind=w.kind, alpha=w.alpha, beta=w.beta,
                              want64=True)
        assert_close(Dh[l:l + 1], ref["D64"], f"batch {l} D")
        assert_close(Eh[l:l + 1], ref["Aux64"], f"batch {l} E")
    # sampled points over every batch entry
    l, i, j = sample_points(w.L, w.M, w.N, 20000, seed=2)
    ref = oracle.gemm_epi_points(p["A"], p["B"], p["C"], None, kind=w.kind, alpha=w.alpha, beta=w.beta,
                                 l=l, i=i, j=j)
    assert_close(Dh[l, i, j], ref["D64"], "relu_square D")
    assert_close(Eh[l, i, j], ref["Aux64"], "relu_square E")


def test_relu_scale_acc_8192_sampled_and_properties():
    w = workloads.WORKLOADS["relu_scale_acc_8192"]
    log(f"[parity] {w.name}: L={w.L} M={w.M} N={w.N} K={w.K} {w.kind}")
    p = workloads.make_inputs(w)
    t = to_dev(p)
    D = alloc_out(w.L, w.M, w.N)
    F = alloc_out(w.L, w.M, w.N)
    acc = alloc_out(w.L, w.M, w.N, dtype=torch.float32)
    ge.run(t["A"], t["B"], t["C"], kind=w.kind, alpha=w.alpha, beta=w.beta, s3=w.s3, D=D, Aux=F, acc_out=acc)
    # whole-output properties: F >= 0, D = s * F exactly (s = 1/2 halves a normal
    # value), and F agrees with relu(alpha acc + beta C) built from the stored acc
    assert bool(torch.isfinite(D).all()) and bool(torch.isfinite(F).all()) and bool(torch.isfinite(acc).all())
    assert bool((F >= 0).all())
    normal = F.abs() >= 2.0 ** -13
    assert bool((D[normal].double() == 0.5 * F[normal].double()).all()), "D != F / 2 somewhere"
    recon = torch.relu(w.alpha * acc.double() + w.beta * t["C"].double())
    assert bool(((F.double() - recon).abs() <= 2.0 ** -10 * recon + 1e-6).all()), "F inconsistent with acc, C"
    del recon, normal
    l, i, j = sample_points(w.L, w.M, w.N, 20000, seed=3)
    ref = oracle_points(p, w.kind, w.alpha, w.beta, w.s3, l, i, j)
    assert_close(D.cpu().numpy()[l, i, j], ref["D64"], "relu_scale_acc D")
    assert_close(F.cpu().numpy()[l, i, j], ref["Aux64"], "relu_scale_acc F")
    assert_close(acc.cpu().numpy()[l, i, j], ref["Acc64"], "relu_scale_acc acc_out")


def test_bias_row_col_8192_sampled_and_properties():
    w = workloads.WORKLOADS["bias_row_col_8192"]
    log(f"[parity] {w.name}: L={w.L} M={w.M} N={w.N} K={w.K} {w.kind}")
    p = workloads.make_inputs(w)
    t = to_dev(p)
    D = alloc_out(w.L, w.M, w.N)
    ge.run(t["A"], t["B"], kind=w.kind, alpha=w.alpha, D=D, row_bias=t["row_bias"], col_bias=t["col_bias"])
    assert bool(torch.isfinite(D).all())
    l, i, j = sample_points(w.L, w.M, w.N, 20000, seed=4)
    ref = oracle_points(p, w.kind, w.alpha, w.beta, w.s3, l, i, j)
    assert_close(D.cpu().numpy()[l, i, j], ref["D64"], "bias_row_col D")


# ---------------------------------------------------------------------------
# Every kind, both kernels, ragged shapes
# ---------------------------------------------------------------------------
KIND_SCALARS = {"LINCOMB": (1.0, 2.0, 0.0), "AUX_SCALE": (1.0, 2.0, 0.5), "LINCOMB_X_ACC": (2.0, 1.0, 3.0),
                "RELU": (1.0, -1.0, 0.0), "SQUARE": (1.0, 1.0, 0.0), "RELU_SQUARE": (0.5, 1.0, 0.0),
                "RELU_AUX_STORE": (3.0, 2.0, 0.0), "RELU_SCALE_ACC": (1.0, 2.0, 0.5), "BIAS_ROW_COL": (1.5, 0.0, 0.0)}
# activations: alpha = 1/32 and beta = 1/2 keep alpha*acc + beta*C exact in fp32
# on integer inputs and put it where the activations are not flat
KIND_SCALARS.update({a: (2.0 ** -5, 0.5, 0.125 if a == "LEAKY_RELU" else 0.0) for a in workloads.ACTIVATIONS})


@pytest.mark.parametrize("kind,scalars", [("SQUARE", (1.0, 1.0, 0.0)), ("RELU_SQUARE", (1.0, 1.0, 0.0)),
                                          ("LINCOMB", (512.0, 1.0, 0.0)), ("AUX_SCALE", (1.0, 1.0, 512.0))])
@pytest.mark.parametrize("shape,offset", [((1, 256, 264, 4096), 0),   # fast path
                                          ((1, 256, 264, 4096), 1),   # general kernel
                                          ((1, 130, 77, 4093), 0)])   # general kernel, ragged
def test_fp16_overflow_to_inf(kind, scalars, shape, offset):
    """Outputs past fp16's range round to +-inf (no saturation), bit for bit
    with the oracle: on integer inputs every value is exact in fp32, so the
    same elements overflow on both sides.  With K = 4096 integer draws of
    standard deviation 2, acc has one of about 256: E = D*D passes 65520 where
    |D| >= 256, and 512*acc (or 512*Aux) where |acc| >= 128, with both signs."""
    L, M, N, K = shape
    a, b, s = scalars
    log(f"[parity] overflow kind={kind} shape={shape} offset={offset}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=M + N + K)
    got = check_full(p, kind, a, b, s, exact=True, offset=offset, what=f"overflow {kind} {shape} off{offset}")
    out = got["Aux" if kind in ("SQUARE", "RELU_SQUARE") else "D"].astype(np.float64)
    assert np.count_nonzero(out == np.inf) > 0, "some outputs overflow to +inf"
    if kind in ("LINCOMB", "AUX_SCALE"):
        assert np.count_nonzero(out == -np.inf) > 0, "and some to -inf"


@pytest.mark.parametrize("offset", [0, 1])
def test_fp16_overflow_gaussian(offset):
    """Gaussian inputs with a long K: E = D*D passes fp16's range on a good
    share of the elements.  Each output is +-inf where the oracle's value is
    within the tolerance of 65520 or beyond, and within the tolerance
    elsewhere (near the threshold either side of it may overflow)."""
    L, M, N, K = 1, 256, 264, 16384
    log(f"[parity] overflow gaussian offset={offset}")
    p = workloads.make_problem(L, M, N, K, "SQUARE", init="normal", seed=71)
    got = gpu_run(p, "SQUARE", 1.0, 1.0, 0.0, offset)
    ref = oracle_ref(p, "SQUARE", 1.0, 1.0, 0.0, exact=False)
    assert_close(got["D"], ref["D64"], "overflow gaussian D")
    assert_close(got["Aux"], ref["Aux64"], "overflow gaussian E", overflow=65520.0)
    assert np.count_nonzero(np.isinf(got["Aux"])) > 0, "some E overflow"


@pytest.mark.parametrize("kind", workloads.KINDS)
@pytest.mark.parametrize("shape,offset", [((2, 200, 136, 264), 0),    # fast path, ragged M
                                          ((2, 200, 136, 264), 1),    # misaligned -> general kernel
                                          ((3, 77, 45, 61), 0),       # K, N not multiples of 8 -> general
                                          ((1, 300, 520, 136), 0),    # fast path, several tiles
                                          ((1, 3112, 3928, 40), 0),   # 256 x 256 tiles (mixed types: 128 x 256)
                                          ((1, 1960, 2000, 72), 0),   # 128 x 128 tiles, ragged M, N
                                          ((1, 2100, 2100, 61), 0)])  # general kernel, 256 x 128 tiles
def test_every_kind_integer_inputs_bit_exact(kind, shape, offset):
    L, M, N, K = shape
    a, b, s = KIND_SCALARS[kind]
    log(f"[parity] kind={kind} shape={shape} offset={offset}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=M * N + K)
    check_full(p, kind, a, b, s, exact=True, offset=offset, what=f"{kind} {shape} off{offset}")


@pytest.mark.parametrize("kind", workloads.KINDS)
def test_every_kind_gaussian_inputs(kind):
    L, M, N, K = 3, 520, 392, 768
    a, b, s = KIND_SCALARS[kind]
    log(f"[parity] gaussian kind={kind}")
    p = workloads.make_problem(L, M, N, K, kind, init="normal", seed=17)
    check_full(p, kind, a, b, s, exact=False, what=f"gaussian {kind}")


TAIL_SHAPES = [
    (1, 1, 1, 1), (1, 1, 8, 8), (1, 8, 1, 8), (1, 7, 9, 5), (1, 15, 17, 63), (1, 63, 64, 65),
    (1, 64, 64, 64), (1, 65, 63, 127), (1, 127, 129, 129), (1, 129, 128, 255), (1, 255, 256, 257),
    (1, 257, 264, 1000), (2, 1000, 1000, 72), (1, 8, 1000, 1000), (1, 1000, 8, 16), (2, 33, 2056, 40),
    (1, 513, 1032, 8), (4, 64, 64, 1), (1, 256, 512, 1024), (1, 512, 256, 1024), (1, 520, 776, 88),
]


# shapes whose tile choice is 128 x 128 and 256 x 128 (the others are reached above)
TILE_SHAPES = [(1, 768, 2816, 72), (1, 2304, 2048, 40), (1, 2400, 1032, 24)]

# the 256 x 256 tile (k stages of 32 in a 4-slot ring, steps in groups of 4)
# with 1 to 9 k stages, full and ragged last ones, and ragged M and N: its
# prologue, the zero-fed ring past the last stage and the group remainders
BIG_TILE_SHAPES = [(1, 4000, 4000, 8), (1, 4000, 4000, 24), (1, 4000, 4000, 32), (1, 4000, 4000, 40),
                   (1, 4000, 4000, 72), (1, 4000, 4000, 104), (1, 4000, 4000, 136), (1, 4000, 4000, 200),
                   (1, 4000, 4000, 248), (1, 3000, 5000, 256), (1, 3000, 5000, 264)]

# the 64 x 64 tile with its 128-deep K step (K >= 256): 4 full stages, a
# ragged last stage of 8 and of 120, more stages than the ring holds, ragged
# M and N, batches; the last two have more tiles than compute units (2-stage
# ring)
DEEP_SMALL_SHAPES = [(1, 64, 64, 256), (1, 64, 64, 512), (1, 1000, 1000, 520), (1, 777, 1000, 1016), (2, 300, 520, 2056),
                     (3, 200, 136, 1160), (1, 1280, 1280, 648), (2, 1000, 600, 1032)]


# the 4-wave 128 x 256, 256 x 128 and 128 x 128 tiles: 1 to 32 k stages,
# ragged last stages, ragged M and N, batches
MID_TILE_SHAPES = [(1, 3000, 2000, 520), (1, 1500, 4000, 1000), (1, 2000, 3000, 264), (1, 1500, 4000, 8),
                   (1, 3000, 2000, 136), (2, 1100, 2600, 96), (1, 2000, 2000, 8), (1, 1800, 2040, 264),
                   (1, 1900, 2000, 1000), (1, 1960, 2000, 72), (2, 1100, 1304, 136), (1, 2047, 2040, 520)]


@pytest.mark.parametrize("shape", TAIL_SHAPES + TILE_SHAPES + BIG_TILE_SHAPES + DEEP_SMALL_SHAPES + MID_TILE_SHAPES)
def test_tails_bit_exact(shape):
    L, M, N, K = shape
    kind = "AUX_SCALE"
    log(f"[parity] tails shape={shape}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=L + M + N + K)
    check_full(p, kind, 1.0, 2.0, 0.5, exact=True, what=f"tails {shape}")


# Short K on every 4-wave tile (2 to 4 k steps), called many times: the last k
# step refills the B slot that slower waves read their last operands from, and
# only its barrier keeps the two apart.  Without it the damage was rare (one
# 16-column block of one wave, in some launches), so each shape repeats.
FOUR_WAVE_SHORT_K = [(1, 1960, 2000, 72), (1, 1960, 2000, 40), (1, 2000, 3000, 72), (1, 3000, 2000, 104),
                     (1, 3112, 3928, 72)]


@pytest.mark.parametrize("shape", FOUR_WAVE_SHORT_K)
def test_four_wave_tiles_repeated_short_k(shape):
    L, M, N, K = shape
    kind, a, b, s = "AUX_SCALE", 1.0, 2.0, 0.5
    log(f"[parity] 4-wave short K shape={shape}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=7 * K + M)
    want = oracle_full(p, kind, a, b, s, want64=False)
    t = to_dev(p)
    D = alloc_out(L, M, N)
    Aux = alloc_out(L, M, N)
    for rep in range(12):
        D.fill_(float("nan"))
        Aux.fill_(float("nan"))
        ge.run(t["A"], t["B"], t["C"], t["X"], kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux)
        assert_bit_exact(D.cpu().numpy(), want["D"], f"{shape} launch {rep} D")
        assert_bit_exact(Aux.cpu().numpy(), want["Aux"], f"{shape} launch {rep} Aux")


def test_every_tile_configuration_is_exercised():
    """The shapes above reach all compiled tile configurations of the fast path.
    The 64 x 64 x 128 tile has two LDS rings: 4 stages, or 2 when the grid
    has more tiles than the 256 compute units (the host's rule), so the ring
    is told apart by the workgroup count."""
    seen = set()
    P = 0x7F0000001000
    shapes = TAIL_SHAPES + TILE_SHAPES + DEEP_SMALL_SHAPES + [(2, 200, 136, 264), (1, 300, 520, 136)] + [
        (w.L, w.M, w.N, w.K) for w in workloads.WORKLOADS.values()]
    for (L, M, N, K) in shapes:
        rc, cfg = ge.gemm_epi_plan(L, M, N, K, P, P, P, P, 1, P, P)
        assert rc == 0
        if cfg["vec"]:
            ring = "2-stage" if cfg["bk"] == 128 and cfg["workgroups"] > 256 else ""
            seen.add((cfg["bm"], cfg["bn"], cfg["bk"], ring))
    assert seen == {(256, 256, 32, ""), (128, 256, 32, ""), (256, 128, 32, ""), (128, 128, 32, ""), (64, 64, 64, ""),
                    (64, 64, 128, ""), (64, 64, 128, "2-stage")}, seen


def test_identity_and_zero_closed_forms_on_gpu():
    """A = I gives D = B exactly; A = 0 gives D = RNE(beta C) (LINCOMB)."""
    L, M, N = 2, 192, 264
    p = workloads.make_problem(L, M, N, M, "LINCOMB", init="normal", seed=3)
    p["A"] = np.broadcast_to(np.eye(M, dtype=np.float16), (L, M, M)).copy()
    got = gpu_run(p, "LINCOMB", 1.0, 0.0, 0.0)
    assert np.array_equal(bits(got["D"]), bits(p["B"]))
    p["A"] = np.zeros_like(p["A"])
    got = gpu_run(p, "LINCOMB", 1.0, -0.5, 0.0)
    want = (-0.5 * p["C"].astype(np.float64)).astype(np.float16)
    assert_bit_exact(got["D"], want, "A = 0")


def test_runs_on_a_side_stream():
    L, M, N, K = 1, 384, 256, 512
    p = workloads.make_problem(L, M, N, K, "LINCOMB", init="small_int", seed=9)
    t = to_dev(p)
    D = alloc_out(L, M, N)
    s = torch.cuda.Stream(device=DEV)
    torch.cuda.synchronize()
    ge.run(t["A"], t["B"], t["C"], kind="LINCOMB", alpha=1.0, beta=2.0, D=D, stream=s, sync=True)
    ref = oracle.gemm_epi(p["A"], p["B"], p["C"], kind="LINCOMB", alpha=1.0, beta=2.0)
    assert_bit_exact(D.cpu().numpy(), ref["D"], "side stream")


def test_large_operand_uses_general_kernel_with_64bit_offsets():
    """One batch entry of A spans more than 2 GiB: the general kernel runs and
    64-bit offsets reach the far end of A."""
    L, M, N, K = 1, 16392, 24, 65536
    P = 0x7F0000001000
    rc, cfg = ge.gemm_epi_plan(L, M, N, K, P, P, P, None, 0, P, None)
    assert rc == 0 and cfg["vec"] == 0
    log(f"[parity] large operand L={L} M={M} N={N} K={K}")
    g = torch.Generator(device="cpu").manual_seed(5)
    A = torch.randint(-2, 3, (L, M, K), generator=g, dtype=torch.float16)
    B = torch.randint(-2, 3, (L, K, N), generator=g, dtype=torch.float16)
    C = torch.randint(-2, 3, (L, M, N), generator=g, dtype=torch.float16)
    tA, tB, tC = A.to(DEV), B.to(DEV), C.to(DEV)
    D = alloc_out(L, M, N)
    ge.run(tA, tB, tC, kind="LINCOMB", alpha=1.0, beta=1.0, D=D)
    rows = np.array([0, 1, 8191, 8192, 16383, 16384, M - 1])
    l, i, j = [], [], []
    for r in rows:
        l.append(np.zeros(N, np.int64))
        i.append(np.full(N, r))
        j.append(np.arange(N))
    l, i, j = np.concatenate(l), np.concatenate(i), np.concatenate(j)
    ref = oracle.gemm_epi_points(A.numpy(), B.numpy(), C.numpy(), kind="LINCOMB", alpha=1.0, beta=1.0,
                                 l=l, i=i, j=j)
    assert_bit_exact(D.cpu().numpy()[l, i, j], ref["D"], "large operand rows")


# ---------------------------------------------------------------------------
# Closed forms on the GPU output alone (no oracle): A = I makes acc = B
# exactly, A = 0 makes acc = +0, so each epilogue reduces to elementwise
# arithmetic on B and C that numpy rounds the same way (one rounding of an
# exact value: the small-integer inputs keep every intermediate exact).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind,alpha,beta,s3", [("LINCOMB", 1.0, 2.0, 0.0), ("AUX_SCALE", 3.0, 2.0, 0.5),
                                                ("RELU_SQUARE", 0.5, 1.0, 0.0), ("LINCOMB_X_ACC", 2.0, 1.0, 3.0)])
@pytest.mark.parametrize("a_form", ["identity", "zero"])
def test_closed_forms_on_gpu_output(kind, alpha, beta, s3, a_form):
    L, M, N = 2, 136, 264
    K = M
    log(f"[parity] closed form A={a_form} kind={kind}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=9)
    p["A"] = (np.broadcast_to(np.eye(M, dtype=np.float16), (L, M, M)) if a_form == "identity"
              else np.zeros((L, M, K), np.float16)).copy()
    got = gpu_run(p, kind, alpha, beta, s3)
    acc = p["B"].astype(np.float64) if a_form == "identity" else np.zeros((L, M, N))
    c = p["C"].astype(np.float64)
    lin = alpha * acc + beta * c
    if kind == "LINCOMB":
        want = {"D": lin}
    elif kind == "AUX_SCALE":
        want = {"Aux": lin, "D": s3 * lin}
    elif kind == "RELU_SQUARE":
        d = np.maximum(lin, 0.0)
        want = {"D": d, "Aux": d * d}
    else:
        want = {"Aux": acc, "D": lin + s3 * p["X"].astype(np.float64)}
    for name, w in want.items():
        assert_bit_exact(got[name], w.astype(np.float16), f"closed form A={a_form} {kind} {name}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prepared_call_matches_the_oracle(dtype):
    """ge.prepared: the same C-ABI call with its arguments converted once,
    repeated; every repetition bit-exact against the oracle."""
    L, M, N, K = 2, 200, 136, 264
    kind = "AUX_SCALE"
    a, b, s3 = KIND_SCALARS[kind]
    log(f"[prepared] {dtype}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=321, dtype=dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16

    def dev(v):
        return torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(tdt).to(DEV)
    A, B, C = dev(p["A"]), dev(p["B"]), dev(p["C"])
    D = torch.full((L, M, N), float("nan"), dtype=tdt, device=DEV)
    Aux = torch.full((L, M, N), float("nan"), dtype=tdt, device=DEV)
    stream = torch.cuda.current_stream()
    call = ge.prepared("gemm_epi_run_typed", L, M, N, K, A.data_ptr(), B.data_ptr(), C.data_ptr(), None, None,
                       None, (a, b, s3), kind, D.data_ptr(), Aux.data_ptr(), None, dtype, stream.cuda_stream)
    ref = oracle.gemm_epi(p["A"], p["B"], p["C"], None, kind=kind, alpha=a, beta=b, s3=s3, dtype=dtype)
    for _ in range(3):
        D.fill_(float("nan"))
        Aux.fill_(float("nan"))
        assert call() == 0
        torch.cuda.synchronize()
        assert_bit_exact(D.cpu().view(torch.int16).numpy().view(np.uint16), ref["D"], "prepared D")
        assert_bit_exact(Aux.cpu().view(torch.int16).numpy().view(np.uint16), ref["Aux"], "prepared Aux")
