"""The fused call, and the workspace calls that stage ragged operands or
split the K range, under HIP graph capture.

A caller may record gemm_epi_run_ext / gemm_epi_run_typed into a HIP graph
(torch.cuda.graph captures the current stream): the entry points queue one
kernel launch and nothing else (no allocation, no memset, no
synchronisation), so the captured graph must replay to the same bits as
eager calls.  Each replay is checked, with eager work on the same buffers
between replays, so that a stale capture would show.
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_elementwise_amd as ge
from dense_gemm_elementwise_amd import workloads
from test_parity_gpu import assert_bit_exact, log, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("kind", ["AUX_SCALE", "LINCOMB_X_ACC", "GELU"])
def test_captured_call_replays_to_the_eager_result(kind):
    L, M, N, K = 2, 520, 392, 264
    a, b, s = {"AUX_SCALE": (1.0, 2.0, 0.5), "LINCOMB_X_ACC": (2.0, 1.0, 3.0), "GELU": (2.0 ** -5, 0.5, 0.0)}[kind]
    log(f"[graph] kind={kind}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=77)
    t = to_dev(p)
    D = torch.zeros((L, M, N), dtype=torch.float16, device=DEV)
    Aux = torch.zeros_like(D) if kind in ge.HAS_AUX else None
    ref = oracle.gemm_epi(p["A"], p["B"], p["C"], p["X"], kind=kind, alpha=a, beta=b, s3=s, want64=True)

    # eager result first (also warms up the library on this stream)
    ge.run(t["A"], t["B"], t["C"], t["X"], kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux)
    eager_d = D.clone()
    eager_aux = Aux.clone() if Aux is not None else None

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ge.run(t["A"], t["B"], t["C"], t["X"], kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux, sync=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work in between: clobber the outputs, perturb nothing else
        D.fill_(float("nan"))
        if Aux is not None:
            Aux.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(D.view(torch.int16), eager_d.view(torch.int16)), f"replay {rep}: D differs from eager"
        if Aux is not None:
            assert torch.equal(Aux.view(torch.int16), eager_aux.view(torch.int16)), f"replay {rep}: Aux differs"
    # and the eager result is the oracle's
    if kind in ge.ACTIVATIONS:
        g64 = eager_d.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(g64 - ref["D64"]) <= 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref["D64"]), 2.0 ** -14))) - 10))
    else:
        assert_bit_exact(eager_d.cpu().numpy(), ref["D"], f"graph {kind} D")
        if Aux is not None:
            assert_bit_exact(eager_aux.cpu().numpy(), ref["Aux"], f"graph {kind} Aux")


def test_captured_inputs_changed_between_replays():
    """The graph holds pointers, not values: new input values written into the
    same buffers between replays give the new product."""
    L, M, N, K = 1, 256, 256, 128
    log("[graph] inputs updated between replays")
    D = torch.zeros((L, M, N), dtype=torch.float16, device=DEV)
    p0 = workloads.make_problem(L, M, N, K, "LINCOMB", init="small_int", seed=1)
    t = to_dev(p0)
    ge.run(t["A"], t["B"], t["C"], kind="LINCOMB", alpha=1.0, beta=2.0, D=D)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ge.run(t["A"], t["B"], t["C"], kind="LINCOMB", alpha=1.0, beta=2.0, D=D, sync=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for seed in (2, 3, 4):
        p = workloads.make_problem(L, M, N, K, "LINCOMB", init="small_int", seed=seed)
        for k in ("A", "B", "C"):
            t[k].copy_(torch.from_numpy(p[k]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.gemm_epi(p["A"], p["B"], p["C"], kind="LINCOMB", alpha=1.0, beta=2.0)
        assert_bit_exact(D.cpu().numpy(), ref["D"], f"graph replay with seed {seed}")


def test_captured_staged_call_replays_with_new_inputs():
    """A workspace call that stages ragged operands (copies in, the fast
    kernel, copies back: kernels only) records into a graph too; each replay
    after new input values are written gives the new result."""
    L, M, N, K = 2, 300, 517, 61
    kind, a, b, s = "AUX_SCALE", 1.0, 2.0, 0.5
    log("[graph] staged call")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=31)
    t = to_dev(p)
    D = torch.zeros((L, M, N), dtype=torch.float16, device=DEV)
    Aux = torch.zeros_like(D)
    P = lambda x: x.data_ptr()
    rc, plan = ge.gemm_epi_plan_ws(L, M, N, K, P(t["A"]), P(t["B"]), P(t["C"]), None, None, None, kind, P(D), P(Aux),
                                   None)
    assert rc == 0 and plan["vec"] == 1 and plan["workspace_bytes"] > 16384  # staged for the fast kernel
    ws = torch.zeros(plan["workspace_bytes"], dtype=torch.uint8, device=DEV)
    ge.run(t["A"], t["B"], t["C"], kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux, workspace=ws)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ge.run(t["A"], t["B"], t["C"], kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux, workspace=ws, sync=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for seed in (32, 33, 34):
        q = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=seed)
        for k in ("A", "B", "C"):
            t[k].copy_(torch.from_numpy(q[k]))
        D.fill_(float("nan"))
        Aux.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.gemm_epi(q["A"], q["B"], q["C"], kind=kind, alpha=a, beta=b, s3=s)
        assert_bit_exact(D.cpu().numpy(), ref["D"], f"staged graph replay {seed} D")
        assert_bit_exact(Aux.cpu().numpy(), ref["Aux"], f"staged graph replay {seed} Aux")


def test_captured_split_call_replays_with_new_inputs():
    """A workspace call whose K range is split over workgroups (partial sums
    and per-tile counters in the workspace, the last contributor resetting
    its counter) records into a graph as kernels alone; every replay, with
    new input values written between replays, gives the new result."""
    L, M, N, K = 1, 512, 512, 8192
    kind, a, b, s = "AUX_SCALE", 1.0, 2.0, 0.5
    log("[graph] split call")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=41)
    t = to_dev(p)
    D = torch.zeros((L, M, N), dtype=torch.float16, device=DEV)
    Aux = torch.zeros_like(D)
    P = lambda x: x.data_ptr()
    rc, plan = ge.gemm_epi_plan_ws(L, M, N, K, P(t["A"]), P(t["B"]), P(t["C"]), None, None, None, kind, P(D), P(Aux),
                                   None)
    # aligned operands are never staged, so a workspace here means a split
    assert rc == 0 and plan["workspace_bytes"] > 0 and plan["bm"] == 128, plan
    ws = torch.zeros(plan["workspace_bytes"], dtype=torch.uint8, device=DEV)
    ge.run(t["A"], t["B"], t["C"], kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux, workspace=ws)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ge.run(t["A"], t["B"], t["C"], kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux, workspace=ws, sync=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for seed in (42, 43, 44):
        q = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=seed)
        for k in ("A", "B", "C"):
            t[k].copy_(torch.from_numpy(q[k]))
        D.fill_(float("nan"))
        Aux.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.gemm_epi(q["A"], q["B"], q["C"], kind=kind, alpha=a, beta=b, s3=s)
        assert_bit_exact(D.cpu().numpy(), ref["D"], f"split graph replay {seed} D")
        assert_bit_exact(Aux.cpu().numpy(), ref["Aux"], f"split graph replay {seed} Aux")
    # the counters are back at zero after the replays
    assert int(ws[:16384].view(torch.int32).abs().sum()) == 0
