"""gemm_epi_run_ws (stream-K: K ranges of tiles split across workgroups, the
partial sums added by the last contributor of each tile before the
epilogue) against the oracle, on the GPU.

On integer-valued inputs every partial sum is exact, so the results must be
bit-exact whatever the split; on Gaussian inputs they are within the
tolerance and identical from call to call (the partials of a tile are added
in k order, whichever workgroup finishes last).  Each call must leave the
workspace's counters at zero for the next one.
"""
import numpy as np
import pytest
import torch

import dense_gemm_elementwise_amd as ge
from dense_gemm_elementwise_amd import workloads

from test_parity_gpu import (KIND_SCALARS, alloc_out, assert_bit_exact, assert_close, assert_output, log, oracle_full,
                             oracle_ref, to_dev)

pytestmark = pytest.mark.gpu

P = 0x7F0000001000


def plan(shape, kind):
    L, M, N, K = shape
    rc, cfg = ge.gemm_epi_plan_ws(L, M, N, K, P, P, P, P, P, P, ge.KINDS[kind], P, P, P)
    assert rc == 0
    return cfg


def run_ws(p, kind, alpha, beta, s3, ws, times=1):
    t = to_dev(p)
    L, M, K = p["A"].shape
    N = p["B"].shape[2]
    outs = []
    for _ in range(times):
        D = alloc_out(L, M, N)
        Aux = alloc_out(L, M, N) if kind in ge.HAS_AUX else None
        acc = alloc_out(L, M, N, dtype=torch.float32) if kind in ge.HAS_ACC else None
        ge.run(t["A"], t["B"], t["C"], t["X"], kind=kind, alpha=alpha, beta=beta, s3=s3, D=D, Aux=Aux,
               row_bias=t["row_bias"], col_bias=t["col_bias"], acc_out=acc, stream_k_workspace=ws)
        o = {"D": D.cpu().numpy()}
        if Aux is not None:
            o["Aux"] = Aux.cpu().numpy()
        if acc is not None:
            o["Acc"] = acc.cpu().numpy()
        outs.append(o)
    return outs


def workspace(cfg):
    assert cfg["workspace_bytes"] > 0, "this shape should be split"
    return torch.zeros(cfg["workspace_bytes"], dtype=torch.uint8, device="cuda:0")


# the per-tile counters sit at the start of the workspace, in a block of fixed
# size whatever the plan (include/gemm_epi.h, gemm_epi_run_ws)
SK_COUNTER_BYTES = 16384


def counters_are_zero(ws, cfg):
    return bool((ws[:SK_COUNTER_BYTES] == 0).all())


# shapes with few tiles and a long K (the planner splits them): ragged M and N
# with a K tail, a batch, two square ones
SPLIT_SHAPES = [(1, 256, 256, 16384), (1, 200, 304, 12000), (2, 128, 384, 8192), (1, 512, 512, 8192)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
@pytest.mark.parametrize("kind", workloads.KINDS)
def test_stream_k_integer_bit_exact(shape, kind):
    L, M, N, K = shape
    a, b, s = KIND_SCALARS[kind]
    cfg = plan(shape, kind)
    log(f"[stream-k] kind={kind} shape={shape} workgroups={cfg['workgroups']} ws={cfg['workspace_bytes']}")
    ws = workspace(cfg)
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=L + M + 3 * N + K)
    ref = oracle_ref(p, kind, a, b, s, exact=True)
    outs = run_ws(p, kind, a, b, s, ws, times=2)   # the second call reuses the workspace
    assert counters_are_zero(ws, cfg)
    for n, got in enumerate(outs):
        for name in ("D", "Aux"):
            if name in ref:
                assert_output(got[name], ref, name, kind, True, f"stream-k call {n} {kind} {shape} {name}")
        if kind in ge.HAS_ACC:
            assert np.array_equal(got["Acc"], ref["Acc"]), f"stream-k call {n} acc_out"


@pytest.mark.parametrize("kind", ["LINCOMB_X_ACC", "RELU_SCALE_ACC", "BIAS_ROW_COL"])
def test_stream_k_gaussian_and_deterministic(kind):
    shape = (1, 256, 256, 16384)
    L, M, N, K = shape
    a, b, s = KIND_SCALARS[kind]
    cfg = plan(shape, kind)
    log(f"[stream-k] gaussian kind={kind}")
    ws = workspace(cfg)
    p = workloads.make_problem(L, M, N, K, kind, init="normal", seed=31)
    ref = oracle_full(p, kind, a, b, s, want64=True)
    outs = run_ws(p, kind, a, b, s, ws, times=3)
    for name in ("D", "Aux"):
        if name in ref:
            assert_close(outs[0][name], ref[name + "64"], f"stream-k gaussian {kind} {name}")
    if kind in ge.HAS_ACC:
        assert_close(outs[0]["Acc"], ref["Acc64"], f"stream-k gaussian {kind} acc_out")
    for o in outs[1:]:
        for name in outs[0]:
            assert np.array_equal(o[name].view(np.uint8), outs[0][name].view(np.uint8)), f"{kind} {name} changed"


def test_no_split_is_the_plain_call():
    """Where no split is planned (1024^3: enough tiles), gemm_epi_run_ws is
    gemm_epi_run_ext: same bits, workspace untouched (None accepted)."""
    w = workloads.WORKLOADS["aux_scale_1024"]
    cfg = plan((w.L, w.M, w.N, w.K), w.kind)
    assert cfg["workspace_bytes"] == 0
    log(f"[stream-k] {w.name} (no split)")
    p = workloads.make_inputs(w)
    t = to_dev(p)
    outs = []
    for ws in (None, torch.zeros(16, dtype=torch.uint8, device="cuda:0")):
        D, Aux = alloc_out(w.L, w.M, w.N), alloc_out(w.L, w.M, w.N)
        if ws is None:
            ge.run(t["A"], t["B"], t["C"], kind=w.kind, alpha=w.alpha, beta=w.beta, s3=w.s3, D=D, Aux=Aux)
        else:
            ge.run(t["A"], t["B"], t["C"], kind=w.kind, alpha=w.alpha, beta=w.beta, s3=w.s3, D=D, Aux=Aux,
                   stream_k_workspace=ws)
            assert bool((ws == 0).all())
        outs.append((D.cpu().numpy(), Aux.cpu().numpy()))
    assert np.array_equal(outs[0][0].view(np.uint16), outs[1][0].view(np.uint16))
    assert np.array_equal(outs[0][1].view(np.uint16), outs[1][1].view(np.uint16))


def test_deep_k_workload():
    """The deep-K workload (few output tiles, K = 65536) through the split,
    every output against the oracle."""
    w = workloads.WORKLOADS["lincomb_deep_k_256x256x65536"]
    cfg = plan((w.L, w.M, w.N, w.K), w.kind)
    log(f"[stream-k] {w.name}: workgroups={cfg['workgroups']}")
    ws = workspace(cfg)
    p = workloads.make_inputs(w)
    ref = oracle_full(p, w.kind, w.alpha, w.beta, w.s3, want64=True)
    got = run_ws(p, w.kind, w.alpha, w.beta, w.s3, ws)[0]
    assert_close(got["D"], ref["D64"], "deep-K D")


def test_one_workspace_serves_plans_with_different_workgroup_counts():
    """A workspace reused across shapes whose splits use different workgroup
    counts (so different partial-slot areas): each call must find its
    counters at zero and stay bit-exact against the oracle."""
    kind = "AUX_SCALE"
    a, b, s = KIND_SCALARS[kind]
    shapes = [(1, 512, 512, 8192), (1, 256, 256, 16384), (1, 512, 512, 8192)]
    cfgs = [plan(sh, kind) for sh in shapes]
    assert len({c["workgroups"] for c in cfgs}) > 1, cfgs
    ws = torch.zeros(max(c["workspace_bytes"] for c in cfgs), dtype=torch.uint8, device="cuda:0")
    for sh, cfg in zip(shapes, cfgs):
        L, M, N, K = sh
        log(f"[stream-k] shared workspace shape={sh} workgroups={cfg['workgroups']}")
        p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=M + K)
        ref = oracle_ref(p, kind, a, b, s, exact=True)
        got = run_ws(p, kind, a, b, s, ws)[0]
        assert counters_are_zero(ws, cfg)
        for name in got:
            assert_output(got[name], ref, name, kind, True, f"shared workspace {sh} {name}")
