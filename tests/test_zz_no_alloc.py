"""gemm_epi_run_ws_static (the stream-K call whose split keeps its counters
and partial sums in the library's per-device static array, for callers that
cannot allocate) against gemm_epi_run_ws_typed with a caller-allocated
workspace, through the C ABI on the GPU: two calls in a row, the second on
a smaller problem, each bit-exact on integer-valued inputs (every partial
sum is exact whatever the split) and checked against the oracle too.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import dense_gemm_elementwise_amd as ge
from dense_gemm_elementwise_amd import workloads

from test_parity_gpu import KIND_SCALARS, assert_output, log, oracle_ref, to_dev

pytestmark = pytest.mark.gpu

P = 0x7F0000001000


def _call(fn, p, kind, dtype, extra):
    t = to_dev(p)
    L, M, K = p["A"].shape
    N = p["B"].shape[2]
    dev = torch.device("cuda:0")
    D = torch.full((L, M, N), float("nan"), dtype=torch.float16, device=dev)
    Aux = torch.full_like(D, float("nan")) if kind in ge.HAS_AUX else None
    acc = torch.full((L, M, N), float("nan"), dtype=torch.float32, device=dev) if kind in ge.HAS_ACC else None

    def ptr(x):
        return x.data_ptr() if x is not None else None
    a, b, s = KIND_SCALARS[kind]
    stream = torch.cuda.current_stream(dev)
    rc = fn(L, M, N, K, ptr(t["A"]), ptr(t["B"]), ptr(t["C"]), ptr(t["X"]), ptr(t["row_bias"]), ptr(t["col_bias"]),
            (a, b, s), ge.KINDS[kind], ptr(D), ptr(Aux), ptr(acc), *extra(stream))
    assert rc == 0, ge.gemm_epi_status_string(rc)
    torch.cuda.synchronize()
    out = {"D": D.cpu().numpy()}
    if Aux is not None:
        out["Aux"] = Aux.cpu().numpy()
    if acc is not None:
        out["Acc"] = acc.cpu().numpy()
    return out


@pytest.mark.parametrize("kind", ["AUX_SCALE", "RELU_SCALE_ACC"])
def test_static_scratch_matches_workspace_call(kind):
    shapes = [(1, 512, 512, 8192), (1, 200, 304, 12000)]   # the second smaller (and ragged)
    for n, (L, M, N, K) in enumerate(shapes):
        rc, cfg = ge.gemm_epi_plan_ws(L, M, N, K, P, P, P, P, P, P, ge.KINDS[kind], P, P, P)
        assert rc == 0 and cfg["workspace_bytes"] > 0, ("this shape should be split", cfg)
        log(f"[no-alloc] call {n} kind={kind} shape={(L, M, N, K)} workgroups={cfg['workgroups']}")
        p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=7 + n)
        ws = torch.zeros(cfg["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
        want = _call(ge.gemm_epi_run_ws_typed, p, kind, "f16",
                     lambda st: (ws.data_ptr(), cfg["workspace_bytes"], ge.DTYPES["f16"], st.cuda_stream))
        got = _call(ge.gemm_epi_run_ws_static, p, kind, "f16", lambda st: (ge.DTYPES["f16"], st.cuda_stream))
        a, b, s = KIND_SCALARS[kind]
        ref = oracle_ref(p, kind, a, b, s, exact=True)
        for name in got:
            if name == "Acc":
                assert np.array_equal(got[name], want[name]), f"call {n} {name}"
                assert np.array_equal(got[name], ref["Acc"]), f"call {n} {name} vs oracle"
                continue
            assert np.array_equal(got[name].view(np.uint16), want[name].view(np.uint16)), f"call {n} {name}"
            assert_output(got[name], ref, name, kind, True, f"static scratch call {n} {name}")


def test_static_scratch_call_replays_from_a_graph():
    """The callers this entry point is for include code under HIP graph
    capture: recorded after a first eager call on the device (which looks up
    the array and clears its counters), the split call replays as kernels
    alone, and each replay, with new input values written between replays,
    gives the oracle's result."""
    L, M, N, K = 1, 512, 512, 8192
    kind = "AUX_SCALE"
    a, b, s = KIND_SCALARS[kind]
    rc, cfg = ge.gemm_epi_plan_ws(L, M, N, K, P, P, P, P, P, P, ge.KINDS[kind], P, P, P)
    assert rc == 0 and cfg["workspace_bytes"] > 0, ("this shape should be split", cfg)
    log(f"[no-alloc] graph capture kind={kind} shape={(L, M, N, K)}")
    dev = torch.device("cuda:0")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=51)
    t = to_dev(p)
    D = torch.zeros((L, M, N), dtype=torch.float16, device=dev)
    Aux = torch.zeros_like(D)

    def call(stream):
        rc = ge.gemm_epi_run_ws_static(L, M, N, K, t["A"].data_ptr(), t["B"].data_ptr(), t["C"].data_ptr(), None,
                                       None, None, (a, b, s), ge.KINDS[kind], D.data_ptr(), Aux.data_ptr(), None,
                                       ge.DTYPES["f16"], stream.cuda_stream)
        assert rc == 0, ge.gemm_epi_status_string(rc)

    call(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            call(side)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    for seed in (52, 53, 54):
        q = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=seed)
        for k in ("A", "B", "C"):
            t[k].copy_(torch.from_numpy(q[k]))
        D.fill_(float("nan"))
        Aux.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle_ref(q, kind, a, b, s, exact=True)
        assert_output(D.cpu().numpy(), ref, "D", kind, True, f"static scratch graph replay {seed} D")
        assert_output(Aux.cpu().numpy(), ref, "Aux", kind, True, f"static scratch graph replay {seed} Aux")


def _first_call_captured():
    """In a fresh process: the first call of the entry point on the device is
    made under graph capture, so its lookup of the array and the kernel that
    clears the counters are what capture sees.  Prints "ok" when every replay
    (new inputs before each) gives the oracle's result."""
    L, M, N, K = 1, 512, 512, 8192
    kind = "AUX_SCALE"
    a, b, s = KIND_SCALARS[kind]
    dev = torch.device("cuda:0")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=61)
    t = to_dev(p)
    D = torch.zeros((L, M, N), dtype=torch.float16, device=dev)
    Aux = torch.zeros_like(D)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            rc = ge.gemm_epi_run_ws_static(L, M, N, K, t["A"].data_ptr(), t["B"].data_ptr(), t["C"].data_ptr(),
                                           None, None, None, (a, b, s), ge.KINDS[kind], D.data_ptr(),
                                           Aux.data_ptr(), None, ge.DTYPES["f16"], side.cuda_stream)
    assert rc == 0, ge.gemm_epi_status_string(rc)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    for seed in (62, 63, 64):
        q = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=seed)
        for k in ("A", "B", "C"):
            t[k].copy_(torch.from_numpy(q[k]))
        D.fill_(float("nan"))
        Aux.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle_ref(q, kind, a, b, s, exact=True)
        assert_output(D.cpu().numpy(), ref, "D", kind, True, f"first call captured, replay {seed} D")
        assert_output(Aux.cpu().numpy(), ref, "Aux", kind, True, f"first call captured, replay {seed} Aux")
    print("ok", flush=True)


def test_static_scratch_first_call_under_capture():
    """A caller whose very first call runs under graph capture: run in a
    fresh process, since this one has made its first call already."""
    log("[no-alloc] first call under graph capture, in a fresh process")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([root, os.environ.get("PYTHONPATH", "")]))
    r = subprocess.run([sys.executable, "-u", os.path.abspath(__file__), "first-call-captured"], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.returncode, r.stdout[-2000:], r.stderr[-2000:])


if __name__ == "__main__" and sys.argv[1:] == ["first-call-captured"]:
    _first_call_captured()
