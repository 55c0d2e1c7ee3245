"""Operands staged through the workspace (gemm_epi_run_ws) on the GPU,
against the oracle.

A call whose tensors miss the fast kernel's layout rules (K or N not a
multiple of 8, or a pointer not 16-byte aligned: the 16-byte rule of the
Custom Epilogue Example's Constraints) runs the fast kernel on aligned,
zero-padded copies in the workspace and copies its padded outputs back, when
the workspace holds what gemm_epi_plan_ws reports.  Zero products leave every
sum unchanged, so the bars are the usual ones: bit-exact on integer inputs
(one ulp for the activation kinds), the tolerance on Gaussian inputs.  Every
case also checks that the copies back touch nothing outside the outputs and
that the stream-K counter block at the workspace's start stays zero.
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_elementwise_amd as ge
from dense_gemm_elementwise_amd import workloads

from test_parity_gpu import DEV, KIND_SCALARS, assert_close, assert_output, log, oracle_ref
from test_bf16_gpu import compare_bf16

pytestmark = pytest.mark.gpu

GUARD = 64            # spare elements before and after each output
SENTINEL = 0x5A5A     # their bits
COUNTER_BYTES = 16384  # the stream-K counter block at the workspace's start


def place(v, off, dtype):
    """v on the device, `off` elements into a buffer that ends where v ends."""
    buf = torch.empty(v.size + off, dtype=dtype, device=DEV)
    t = buf[off:].view(v.shape)
    if dtype == torch.bfloat16:
        t.copy_(torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).reshape(v.shape))
    else:
        t.copy_(torch.from_numpy(np.ascontiguousarray(v)))
    return t


def guarded(shape, off, dtype):
    """An output `off` elements past GUARD sentinel elements, GUARD more after it."""
    n = int(np.prod(shape))
    idt = torch.int32 if dtype == torch.float32 else torch.int16
    buf = torch.full((GUARD + off + n + GUARD,), SENTINEL, dtype=idt, device=DEV).view(dtype)
    return buf, buf[GUARD + off:GUARD + off + n].view(shape)


def check_guard(buf, off, n, what):
    raw = buf.view(torch.int32 if buf.dtype == torch.float32 else torch.int16).cpu().numpy()
    outside = np.concatenate([raw[:GUARD + off], raw[GUARD + off + n:]])
    assert np.all(outside == SENTINEL), f"{what}: a copy back wrote outside the output"


def run_staged(p, kind, offs, dtype, workspace_bytes=None, expect_staged=True):
    """One gemm_epi_run_ws call with A, B at element offsets offs[0], offs[1],
    the epilogue inputs at offs[2] and the outputs at offs[3]."""
    L, M, K = p["A"].shape
    N = p["B"].shape[2]
    a, b, s = KIND_SCALARS[kind]
    A, B = place(p["A"], offs[0], dtype), place(p["B"], offs[1], dtype)
    C = place(p["C"], offs[2], dtype) if p["C"] is not None else None
    X = place(p["X"], offs[2], dtype) if p["X"] is not None else None
    rb = place(p["row_bias"], offs[2], dtype) if p.get("row_bias") is not None else None
    cb = place(p["col_bias"], offs[2], dtype) if p.get("col_bias") is not None else None
    dbuf, D = guarded((L, M, N), offs[3], dtype)
    abuf, Aux = guarded((L, M, N), offs[3], dtype) if kind in ge.HAS_AUX else (None, None)
    cbuf, acc = guarded((L, M, N), offs[3], torch.float32) if kind in ge.HAS_ACC else (None, None)
    ptr = lambda t: t.data_ptr() if t is not None else None
    rc, cfg = ge.gemm_epi_plan_ws(L, M, N, K, ptr(A), ptr(B), ptr(C), ptr(X), ptr(rb), ptr(cb), kind, ptr(D),
                                  ptr(Aux), ptr(acc))
    assert rc == 0
    if expect_staged:  # the fast kernel runs, on operands staged in the workspace
        assert cfg["vec"] == 1 and cfg["workspace_bytes"] > COUNTER_BYTES, cfg
    nbytes = cfg["workspace_bytes"] if workspace_bytes is None else workspace_bytes
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    ge.run(A, B, C, X, kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux, row_bias=rb, col_bias=cb, acc_out=acc,
           workspace=ws)
    n = L * M * N
    check_guard(dbuf, offs[3], n, "D")
    if Aux is not None:
        check_guard(abuf, offs[3], n, "Aux")
    if acc is not None:
        check_guard(cbuf, offs[3], n, "acc_out")
    assert int(torch.count_nonzero(ws[:min(COUNTER_BYTES, ws.numel())])) == 0, "staging wrote the counter block"
    if dtype == torch.bfloat16:
        out = {"D": D.cpu().view(torch.int16).numpy().view(np.uint16)}
        if Aux is not None:
            out["Aux"] = Aux.cpu().view(torch.int16).numpy().view(np.uint16)
    else:
        out = {"D": D.cpu().numpy()}
        if Aux is not None:
            out["Aux"] = Aux.cpu().numpy()
    if acc is not None:
        out["Acc"] = acc.cpu().numpy()
    return out


def compare(got, p, kind, exact, dtype, what):
    a, b, s = KIND_SCALARS[kind]
    if dtype == torch.bfloat16:
        compare_bf16(got, p, kind, a, b, s, exact, what)
        return
    ref = oracle_ref(p, kind, a, b, s, exact)
    for name in ("D", "Aux"):
        if name in ref:
            assert_output(got[name], ref, name, kind, exact, f"{what} {name}")
    if kind in ge.HAS_ACC:
        if exact:
            assert np.array_equal(got["Acc"], ref["Acc"]), f"{what} acc_out"
        else:
            assert_close(got["Acc"], ref["Acc64"], f"{what} acc_out")


# (shape, element offsets of A, B, the epilogue inputs, the outputs)
STAGED_CASES = [((2, 300, 520, 61), (0, 0, 0, 0)),      # K % 8 != 0: A padded to K8, B read with its K rows
                ((1, 300, 517, 136), (0, 0, 0, 0)),     # N % 8 != 0: B and every M x N tensor padded
                ((3, 77, 45, 61), (0, 0, 0, 0)),        # both
                ((2, 200, 136, 264), (1, 1, 1, 1)),     # every pointer 2 bytes off
                ((1, 520, 776, 88), (0, 0, 3, 0)),      # only the epilogue inputs off
                ((1, 520, 776, 88), (0, 5, 0, 7))]      # only B and the outputs off


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("kind", workloads.KINDS)
@pytest.mark.parametrize("shape,offs", STAGED_CASES)
def test_staged_every_kind_integer_inputs(shape, offs, kind, dtype):
    L, M, N, K = shape
    dt = "bf16" if dtype == torch.bfloat16 else "f16"
    log(f"[staged] {dt} kind={kind} shape={shape} offsets={offs}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=M * N + K + sum(offs), dtype=dt)
    got = run_staged(p, kind, offs, dtype)
    compare(got, p, kind, True, dtype, f"staged {dt} {kind} {shape} {offs}")


@pytest.mark.parametrize("shape,offs,kind", [((1, 1960, 2001, 77), (0, 0, 0, 0), "AUX_SCALE"),
                                             ((1, 2400, 3231, 4095), (0, 0, 0, 0), "LINCOMB"),
                                             ((2, 1000, 1000, 1000), (1, 0, 0, 0), "RELU_SCALE_ACC"),
                                             ((1, 1024, 1030, 1024), (0, 0, 0, 0), "BIAS_ROW_COL")])
def test_staged_larger_shapes(shape, offs, kind):
    """The 4-wave tiles on staged operands: integer inputs bit-exact, then
    Gaussian inputs within the tolerance."""
    L, M, N, K = shape
    log(f"[staged] larger {kind} shape={shape} offsets={offs}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=M + N + K)
    compare(run_staged(p, kind, offs, torch.float16), p, kind, True, torch.float16, f"staged int {shape}")
    p = workloads.make_problem(L, M, N, K, kind, init="normal", seed=M + N + K + 1)
    compare(run_staged(p, kind, offs, torch.float16), p, kind, False, torch.float16, f"staged gaussian {shape}")


@pytest.mark.parametrize("shape,kind,dtype", [((1, 256, 256, 65535), "LINCOMB", torch.float16),
                                              ((2, 200, 136, 24001), "AUX_SCALE", torch.float16),
                                              ((1, 130, 300, 30001), "RELU_SCALE_ACC", torch.bfloat16)])
def test_staged_deep_k_is_split(shape, kind, dtype):
    """Few tiles and a long, ragged K: the staged operands go through the
    stream-K split (the plan reports a split's workgroup count)."""
    L, M, N, K = shape
    dt = "bf16" if dtype == torch.bfloat16 else "f16"
    log(f"[staged] deep K {dt} {kind} shape={shape}")
    P = 0x7F0000001000
    _, cfg = ge.gemm_epi_plan_ws(L, M, N, K, P, P, P, None, P, P, kind, P, P, P)
    assert cfg["bm"] == 128 and cfg["bn"] == 128 and cfg["workgroups"] <= 256, cfg  # the split tile
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=M + N + K, dtype=dt)
    got = run_staged(p, kind, (0, 0, 0, 0), dtype)
    compare(got, p, kind, True, dtype, f"staged deep K {shape}")


def test_small_workspace_runs_the_general_kernel():
    """With less workspace than the plan reports, the call still computes the
    same outputs, on the general kernel, and leaves the workspace alone."""
    L, M, N, K = 2, 300, 517, 61
    kind = "AUX_SCALE"
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=5)
    for nbytes in (0, COUNTER_BYTES + 1024):
        got = run_staged(p, kind, (0, 0, 0, 0), torch.float16, workspace_bytes=nbytes)
        compare(got, p, kind, True, torch.float16, f"small workspace {nbytes}")


def test_misaligned_workspace_runs_the_general_kernel():
    """A workspace that is not 16-byte aligned is not used for staging: the
    general kernel computes the same outputs and the workspace stays zero."""
    L, M, N, K = 2, 300, 517, 61
    kind, a, b, s = "AUX_SCALE", 1.0, 2.0, 0.5
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=6)
    P = 0x7F0000001000
    _, cfg = ge.gemm_epi_plan_ws(L, M, N, K, P, P, P, None, None, None, kind, P, P, None)
    buf = torch.zeros(cfg["workspace_bytes"] + 64, dtype=torch.uint8, device=DEV)
    ws = buf[8:8 + cfg["workspace_bytes"]]
    A, B, C = (torch.from_numpy(p[k]).to(DEV) for k in ("A", "B", "C"))
    D = torch.full((L, M, N), float("nan"), dtype=torch.float16, device=DEV)
    Aux = torch.full_like(D, float("nan"))
    ge.run(A, B, C, kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux, workspace=ws)
    compare({"D": D.cpu().numpy(), "Aux": Aux.cpu().numpy()}, p, kind, True, torch.float16, "misaligned workspace")
    assert int(torch.count_nonzero(buf)) == 0, "a misaligned workspace was written"


def test_staged_and_stream_k_calls_share_a_workspace():
    """Staging leaves the counter block alone, so one zero-filled workspace
    serves stream-K splits and staged calls in any order."""
    kind = "AUX_SCALE"
    a, b, s = KIND_SCALARS[kind]
    sk = workloads.make_problem(1, 256, 256, 16384, kind, init="small_int", seed=11)
    st = workloads.make_problem(1, 300, 517, 61, kind, init="small_int", seed=12)
    P = 0x7F0000001000
    _, cfg_sk = ge.gemm_epi_plan_ws(1, 256, 256, 16384, P, P, P, None, None, None, kind, P, P, None)
    _, cfg_st = ge.gemm_epi_plan_ws(1, 300, 517, 61, P, P, P, None, None, None, kind, P, P, None)
    assert cfg_sk["workspace_bytes"] > 0 and cfg_sk["workgroups"] <= 256  # a split
    ws = torch.zeros(max(cfg_sk["workspace_bytes"], cfg_st["workspace_bytes"]), dtype=torch.uint8, device=DEV)
    refs = {id(q): oracle_ref(q, kind, a, b, s, True) for q in (sk, st)}
    for rep, q in enumerate((st, sk, st, sk)):
        L, M, K = q["A"].shape
        N = q["B"].shape[2]
        A, B, C = (torch.from_numpy(q[k]).to(DEV) for k in ("A", "B", "C"))
        D = torch.full((L, M, N), float("nan"), dtype=torch.float16, device=DEV)
        Aux = torch.full((L, M, N), float("nan"), dtype=torch.float16, device=DEV)
        ge.run(A, B, C, None, kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux, workspace=ws)
        ref = refs[id(q)]
        assert_output(D.cpu().numpy(), ref, "D", kind, True, f"shared workspace call {rep} D")
        assert_output(Aux.cpu().numpy(), ref, "Aux", kind, True, f"shared workspace call {rep} Aux")
        assert int(torch.count_nonzero(ws[:COUNTER_BYTES])) == 0, f"call {rep} left a counter set"
