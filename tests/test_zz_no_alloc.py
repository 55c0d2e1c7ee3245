"""gemm_epi_run_ws_static (the stream-K call whose split keeps its counters
and partial sums in the library's per-device static array, for callers that
cannot allocate) against gemm_epi_run_ws_typed with a caller-allocated
workspace, through the C ABI on the GPU: two calls in a row, the second on
a smaller problem, each bit-exact on integer-valued inputs (every partial
sum is exact whatever the split) and checked against the oracle too.
"""
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
