"""bfloat16 tensors on the GPU (gemm_epi_run_typed with GEMM_EPI_BF16, reached
through run() with torch.bfloat16 tensors; the unfused and stream-K
compositions through gemm_epi_run_unfused_typed and gemm_epi_run_ws_typed),
against the oracle's bfloat16 path.

Bar: integer-valued inputs make every product and partial sum exact, so the
only rounding is the final bfloat16 store, on both sides: every output is
bit-identical to the oracle (+0 and -0 compare equal); activation kinds are
within one bfloat16 ulp and at least 98% bit-identical.  Gaussian inputs:
|gpu - ref| <= 5e-2 + 1e-2 |ref| against the oracle's unrounded value (a
bfloat16 output's own rounding is at most 2^-9 relative).
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_elementwise_amd as ge
from dense_gemm_elementwise_amd import workloads
from test_parity_gpu import KIND_SCALARS, assert_bit_exact, assert_close, log, sample_points

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev_bf16(p, offset=0):
    out = {}
    for k, v in p.items():
        if v is None:
            out[k] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16)
        if offset:
            buf = torch.empty(v.size + offset, dtype=torch.bfloat16, device=DEV)
            d = buf[offset:].view(v.shape)
            d.copy_(t.reshape(v.shape))
        else:
            d = t.to(DEV)
        out[k] = d
    return out


def alloc_bf16(L, M, N, offset=0, dtype=torch.bfloat16):
    if offset:
        return torch.full((L * M * N + offset,), float("nan"), dtype=dtype, device=DEV)[offset:].view(L, M, N)
    return torch.full((L, M, N), float("nan"), dtype=dtype, device=DEV)


def bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def gpu_run_bf16(p, kind, alpha, beta, s3, offset=0, **compose):
    """One call through run(); compose may name unfused_workspace or
    stream_k_workspace to run that composition instead of the fused call."""
    t = to_dev_bf16(p, offset)
    L, M, K = p["A"].shape
    N = p["B"].shape[2]
    D = alloc_bf16(L, M, N, offset)
    Aux = alloc_bf16(L, M, N, offset) if kind in ge.HAS_AUX else None
    acc = alloc_bf16(L, M, N, offset, torch.float32) if kind in ge.HAS_ACC else None
    ge.run(t["A"], t["B"], t["C"], t["X"], kind=kind, alpha=alpha, beta=beta, s3=s3, D=D, Aux=Aux,
           row_bias=t.get("row_bias"), col_bias=t.get("col_bias"), acc_out=acc, **compose)
    out = {"D": bits(D)}
    if Aux is not None:
        out["Aux"] = bits(Aux)
    if acc is not None:
        out["Acc"] = acc.cpu().numpy()
    return out


def ulp_bf16(x):
    ax = np.abs(np.asarray(x, np.float64))
    return 2.0 ** (np.floor(np.log2(np.maximum(ax, 2.0 ** -126))) - 7)


def check_bf16(p, kind, a, b, s, exact, offset=0, what="", **compose):
    got = gpu_run_bf16(p, kind, a, b, s, offset, **compose)
    compare_bf16(got, p, kind, a, b, s, exact, what)
    return got


def compare_bf16(got, p, kind, a, b, s, exact, what):
    ref = oracle.gemm_epi(p["A"], p["B"], p["C"], p["X"], kind=kind, alpha=a, beta=b, s3=s,
                          row_bias=p.get("row_bias"), col_bias=p.get("col_bias"), want64=True, dtype="bf16")
    for name in ("D", "Aux"):
        if name not in ref:
            continue
        g = oracle.bf16_decode(got[name])
        if exact and kind in ge.ACTIVATIONS:
            r64 = ref[name + "64"]
            assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
            assert np.all(np.abs(g - r64) <= ulp_bf16(r64)), f"{what} {name}: more than 1 ulp off"
            assert np.mean(got[name] == ref[name]) >= 0.98, f"{what} {name}: too few bit-identical"
        elif exact:
            assert_bit_exact(got[name], ref[name], f"{what} {name}")
        else:
            assert_close(g, ref[name + "64"], f"{what} {name}")
    if kind in ge.HAS_ACC:
        if exact:
            assert np.array_equal(got["Acc"], ref["Acc"]), f"{what} acc_out"
        else:
            assert_close(got["Acc"], ref["Acc64"], f"{what} acc_out")


def test_integer_workload_1024_bit_exact():
    w = workloads.WORKLOADS["aux_scale_bf16_1024"]
    log(f"[bf16] {w.name}: L={w.L} M={w.M} N={w.N} K={w.K} {w.kind}")
    check_bf16(workloads.make_inputs(w), w.kind, w.alpha, w.beta, w.s3, exact=True, what=w.name)


@pytest.mark.parametrize("kind", workloads.KINDS)
@pytest.mark.parametrize("shape,offset", [((2, 200, 136, 264), 0),    # fast path, ragged M
                                          ((2, 200, 136, 264), 1),    # misaligned -> general kernel
                                          ((3, 77, 45, 61), 0),       # K, N not multiples of 8 -> general
                                          ((1, 3112, 3928, 40), 0),   # 256 x 256 tiles (mixed types: 128 x 256)
                                          ((2, 300, 520, 648), 0),    # 64 x 64 x 128 tile (K >= 256), ragged last stage
                                          ((1, 1280, 1280, 648), 0),  # the same with the 2-stage ring (400 tiles)
                                          ((1, 300, 520, 136), 0),    # 64 x 64 x 64 tile (K < 256), ragged last stage
                                          ((1, 1960, 2000, 72), 0),   # 128 x 128 tiles, ragged M, N
                                          ((1, 2100, 2100, 61), 0)])  # general kernel, 256 x 128 tiles
def test_every_kind_integer_inputs(kind, shape, offset):
    L, M, N, K = shape
    a, b, s = KIND_SCALARS[kind]
    log(f"[bf16] kind={kind} shape={shape} offset={offset}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=M * N + K, dtype="bf16")
    check_bf16(p, kind, a, b, s, exact=True, offset=offset, what=f"bf16 {kind} {shape} off{offset}")


@pytest.mark.parametrize("kind", ["LINCOMB_X_ACC", "RELU_SCALE_ACC", "BIAS_ROW_COL", "GELU"])
def test_gaussian_inputs(kind):
    L, M, N, K = 2, 520, 392, 768
    a, b, s = KIND_SCALARS[kind]
    log(f"[bf16] gaussian kind={kind}")
    p = workloads.make_problem(L, M, N, K, kind, init="normal", seed=23, dtype="bf16")
    check_bf16(p, kind, a, b, s, exact=False, what=f"bf16 gaussian {kind}")


@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (1, 7, 9, 5), (1, 65, 63, 127), (1, 257, 264, 1000),
                                   (2, 33, 2056, 40), (1, 2304, 2048, 40)])
def test_tails_bit_exact(shape):
    L, M, N, K = shape
    log(f"[bf16] tails shape={shape}")
    p = workloads.make_problem(L, M, N, K, "AUX_SCALE", init="small_int", seed=L + M + N + K, dtype="bf16")
    check_bf16(p, "AUX_SCALE", 1.0, 2.0, 0.5, exact=True, what=f"bf16 tails {shape}")


@pytest.mark.parametrize("kind", ["AUX_SCALE", "SQUARE"])
def test_four_wave_128x128_repeated_short_k(kind):
    """The bf16 128 x 128 tile with 3 k steps, called many times (the last k
    step's barrier; see the fp16 test of every 4-wave tile)."""
    L, M, N, K = 1, 1960, 2000, 72
    a, b, s = KIND_SCALARS[kind]
    log(f"[bf16] 4-wave 128x128 short K kind={kind}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=M * N + K, dtype="bf16")
    want = oracle.gemm_epi(p["A"], p["B"], p["C"], p["X"], kind=kind, alpha=a, beta=b, s3=s, dtype="bf16")
    t = to_dev_bf16(p)
    D, Aux = alloc_bf16(L, M, N), alloc_bf16(L, M, N)
    for rep in range(12):
        D.fill_(float("nan"))
        Aux.fill_(float("nan"))
        ge.run(t["A"], t["B"], t["C"], t["X"], kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux)
        assert_bit_exact(bits(D), want["D"], f"bf16 {kind} launch {rep} D")
        assert_bit_exact(bits(Aux), want["Aux"], f"bf16 {kind} launch {rep} Aux")


def test_x_acc_bf16_8192_sampled_and_properties():
    w = workloads.WORKLOADS["x_acc_bf16_8192"]
    log(f"[bf16] {w.name}: L={w.L} M={w.M} N={w.N} K={w.K} {w.kind}")
    p = workloads.make_inputs(w)
    t = to_dev_bf16(p)
    D = alloc_bf16(w.L, w.M, w.N)
    Y = alloc_bf16(w.L, w.M, w.N)
    ge.run(t["A"], t["B"], t["C"], t["X"], kind=w.kind, alpha=w.alpha, beta=w.beta, s3=w.s3, D=D, Aux=Y)
    assert bool(torch.isfinite(D.float()).all()) and bool(torch.isfinite(Y.float()).all())
    # D agrees with the epilogue applied to the stored Y = acc (Y rounded once
    # to bfloat16: |D - (alpha Y + beta C + x X)| <= alpha ulp(Y) + ulp(D) + slack)
    D64, Y64 = D.double(), Y.double()
    recon = w.alpha * Y64 + w.beta * t["C"].double() + w.s3 * t["X"].double()
    lim = 2.0 ** -7 * w.alpha * Y64.abs() + 2.0 ** -7 * D64.abs() + 1e-3
    assert bool(((D64 - recon).abs() <= lim).all()), "D inconsistent with Y, C, X somewhere"
    del D64, Y64, recon, lim
    l, i, j = sample_points(w.L, w.M, w.N, 20000, seed=6)
    ref = oracle.gemm_epi_points(p["A"], p["B"], p["C"], p["X"], kind=w.kind, alpha=w.alpha, beta=w.beta, s3=w.s3,
                                 l=l, i=i, j=j, dtype="bf16")
    assert_close(oracle.bf16_decode(bits(D)[l, i, j]), ref["D64"], "x_acc_bf16_8192 D")
    assert_close(oracle.bf16_decode(bits(Y)[l, i, j]), ref["Aux64"], "x_acc_bf16_8192 Y")


# ---- the unfused and stream-K compositions on bfloat16 tensors ----------------

@pytest.mark.parametrize("kind", workloads.KINDS)
@pytest.mark.parametrize("shape,offset", [((2, 200, 136, 264), 0),    # vector paths
                                          ((2, 200, 136, 264), 1),    # misaligned: element-wise paths
                                          ((3, 77, 45, 61), 0),       # K, N not multiples of 8 (N % 4 != 0)
                                          ((1, 1960, 2000, 72), 0),   # the 4-wave tiles: 128 x 128,
                                          ((1, 2000, 3000, 72), 0),   # 128 x 256
                                          ((1, 3112, 3928, 40), 0),   # and 256 x 256
                                          ((1, 2100, 2100, 61), 0)])  # general kernel, 256 x 128 tiles
def test_unfused_bf16_equals_fused_and_oracle(kind, shape, offset):
    """gemm_epi_run_unfused_typed: the same accumulator and the same fp32
    epilogue arithmetic as the fused kernel, so the same bits; on integer
    inputs also the oracle's."""
    L, M, N, K = shape
    a, b, s = KIND_SCALARS[kind]
    log(f"[bf16 unfused] kind={kind} shape={shape} offset={offset}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=M + N * K, dtype="bf16")
    ws = torch.full((L * M * N + offset,), float("nan"), dtype=torch.float32, device=DEV)[offset:]
    unfused = check_bf16(p, kind, a, b, s, exact=True, offset=offset, what=f"bf16 unfused {kind} {shape}",
                         unfused_workspace=ws)
    fused = gpu_run_bf16(p, kind, a, b, s, offset)
    for name in fused:
        assert np.array_equal(np.asarray(fused[name]).view(np.uint8), np.asarray(unfused[name]).view(np.uint8)), \
            f"bf16 {kind} {name}: fused != unfused"


# few tiles and a long K, so that the planner splits K across workgroups
BF16_SPLIT = [((1, 200, 304, 12000), workloads.KINDS),
              ((1, 256, 256, 16384), ["AUX_SCALE", "LINCOMB_X_ACC", "RELU_SCALE_ACC", "BIAS_ROW_COL", "GELU"])]


@pytest.mark.parametrize("shape,kind", [(sh, k) for sh, kinds in BF16_SPLIT for k in kinds])
def test_stream_k_bf16_integer(shape, kind):
    """gemm_epi_run_ws_typed with a split: every partial sum is exact on
    integer inputs, so the outputs equal the oracle's (activations within one
    bfloat16 ulp), on two calls that share the workspace, whose counters
    must be back at zero after each."""
    from test_stream_k_gpu import counters_are_zero, plan, workspace
    L, M, N, K = shape
    a, b, s = KIND_SCALARS[kind]
    cfg = plan(shape, kind)
    log(f"[bf16 stream-k] kind={kind} shape={shape} workgroups={cfg['workgroups']}")
    ws = workspace(cfg)
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=L + M + 3 * N + K, dtype="bf16")
    for call in range(2):
        got = gpu_run_bf16(p, kind, a, b, s, stream_k_workspace=ws)
        compare_bf16(got, p, kind, a, b, s, True, f"bf16 stream-k call {call} {kind} {shape}")
        assert counters_are_zero(ws, cfg)


@pytest.mark.parametrize("act", workloads.ACTIVATIONS)
def test_every_bf16_input(act):
    """acc = t exactly for every bfloat16 t with 2^-60 <= |t| <= 120, and 0
    (A's first column holds t, B's first row is ones, the rest zeros): the
    activations over their whole range, including the left tails whose
    results are bfloat16 subnormals (sigmoid and SiLU below x = -87, GELU
    below x = -13.2)."""
    patterns = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_decode(patterns)
    keep = np.isfinite(v) & (np.abs(v) <= 120.0) & ((np.abs(v) >= 2.0 ** -60) | (v == 0))
    t = patterns[keep]
    M, N, K = t.size, 8, 8
    A = np.zeros((1, M, K), np.uint16)
    A[0, :, 0] = t
    B = np.zeros((1, K, N), np.uint16)
    B[0, 0, :] = 0x3F80  # 1.0
    C = np.zeros((1, M, N), np.uint16)
    p = {"A": A, "B": B, "C": C, "X": None, "row_bias": None, "col_bias": None}
    s3 = 0.125 if act == "LEAKY_RELU" else 0.0
    log(f"[bf16] sweep {act}: {M} inputs")
    check_bf16(p, act, 1.0, 0.0, s3, exact=True, what=f"bf16 sweep {act}")


@pytest.mark.parametrize("act,lo", [("SILU", 17.0), ("GELU", 6.0)])
def test_saturated_midpoints_round_correctly(act, lo):
    """acc = a bfloat16 rounding midpoint m (A's first two columns hold v and
    half the gap to v's upper neighbour, B's first two rows are ones), for
    every midpoint from where sigmoid(m) or Phi(m) rounds to 1 in fp32 up to
    10^6.  The exact output lies just below m and rounds to v, while the
    fp32 value m itself would round the tie to even.  Every output equals
    the oracle's correctly rounded bfloat16."""
    bits = np.arange(0, 0x7F80, dtype=np.uint16)
    v, nxt = oracle.bf16_decode(bits), oracle.bf16_decode(bits + 1)
    keep = (v >= lo) & (v < 1e6) & np.isfinite(nxt)
    M, N, K = int(keep.sum()), 8, 8
    A = np.zeros((1, M, K), np.uint16)
    A[0, :, 0] = bits[keep]
    A[0, :, 1] = oracle.bf16_encode((nxt[keep] - v[keep]) / 2)
    B = np.zeros((1, K, N), np.uint16)
    B[0, :2, :] = 0x3F80  # 1.0
    C = np.zeros((1, M, N), np.uint16)
    p = {"A": A, "B": B, "C": C, "X": None, "row_bias": None, "col_bias": None}
    log(f"[bf16] {act} at {M} midpoints")
    got = gpu_run_bf16(p, act, 1.0, 0.0, 0.0)
    ref = oracle.gemm_epi(p["A"], p["B"], p["C"], kind=act, alpha=1.0, beta=0.0, dtype="bf16")
    assert np.array_equal(ref["D"][0, :, 0], bits[keep]), "the oracle rounds each midpoint down"
    bad = np.count_nonzero(got["D"] != ref["D"])
    assert bad == 0, f"{act}: {bad} of {got['D'].size} outputs differ from the correctly rounded bfloat16"
