"""Seeded random sweep over the shape space: batch 1-3, M, N, K from 1 to
700 (K up to 2100), every kind, fp16 and bf16 tensors, aligned and
misaligned pointers (fast and general kernels), the fused call, the
stream-K entry point and the staging of ragged or misaligned operands
through its workspace, and epilogue tensors of another type than A and B
(fp32 or the other 16-bit type).  Integer-valued inputs keep every sum exact, so each
case is bit-exact against the oracle (activation kinds: within one ulp and
mostly bit-identical, as in the other parity tests).
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_elementwise_amd as ge
from dense_gemm_elementwise_amd import workloads
from test_bf16_gpu import check_bf16
from test_parity_gpu import KIND_SCALARS, check_full, log

pytestmark = pytest.mark.gpu


def cases(n=48, seed=20251202):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        L = int(rng.integers(1, 4))
        M, N = (int(v) for v in rng.integers(1, 701, 2))
        K = int(rng.integers(1, 2101))
        if rng.random() < 0.5:   # half the cases on the 16-byte fast path
            N, K = max(8, N - N % 8), max(8, K - K % 8)
        kind = workloads.KINDS[int(rng.integers(0, len(workloads.KINDS)))]
        dtype = "bf16" if rng.random() < 0.3 else "f16"
        offset = 1 if (dtype == "f16" and rng.random() < 0.2) else 0
        out.append((c, L, M, N, K, kind, dtype, offset))
    return out


@pytest.mark.parametrize("case", cases(), ids=lambda c: f"c{c[0]}-{c[5]}-{c[6]}-{c[1]}x{c[2]}x{c[3]}x{c[4]}-off{c[7]}")
def test_random_case(case):
    c, L, M, N, K, kind, dtype, offset = case
    a, b, s = KIND_SCALARS[kind]
    log(f"[random] case {c}: L={L} M={M} N={N} K={K} {kind} {dtype} offset={offset}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=1000 + c, dtype=dtype)
    if dtype == "bf16":
        check_bf16(p, kind, a, b, s, exact=True, what=f"random case {c}")
    else:
        check_full(p, kind, a, b, s, exact=True, offset=offset, what=f"random case {c}")


@pytest.mark.parametrize("seed", range(6))
def test_random_stream_k_case(seed):
    """Few tiles and a long K, so that the planner splits: through run() with a
    stream-K workspace, against the oracle."""
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 3))
    M, N = int(rng.integers(1, 400)), 8 * int(rng.integers(1, 50))
    K = 8 * int(rng.integers(1000, 3000))
    kind = workloads.EXACT_KINDS[int(rng.integers(0, len(workloads.EXACT_KINDS)))]
    a, b, s = KIND_SCALARS[kind]
    rc, plan = ge.gemm_epi_plan_ws(L, M, N, K, 16, 16, 16, 16, 16, 16, kind, 16, 16, 16)
    assert rc == 0
    log(f"[random stream-k] seed {seed}: L={L} M={M} N={N} K={K} {kind} workspace={plan['workspace_bytes']}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=500 + seed)
    dev = "cuda:0"
    t = {k: (torch.from_numpy(v).to(dev) if v is not None else None) for k, v in p.items()}
    D = torch.full((L, M, N), float("nan"), dtype=torch.float16, device=dev)
    Aux = torch.full_like(D, float("nan")) if kind in ge.HAS_AUX else None
    acc = torch.full((L, M, N), float("nan"), dtype=torch.float32, device=dev) if kind in ge.HAS_ACC else None
    ws = torch.zeros(max(plan["workspace_bytes"], 16), dtype=torch.uint8, device=dev)
    ge.run(t["A"], t["B"], t["C"], t["X"], kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux, acc_out=acc,
           row_bias=t["row_bias"], col_bias=t["col_bias"], stream_k_workspace=ws)
    ref = oracle.gemm_epi(p["A"], p["B"], p["C"], p["X"], kind=kind, alpha=a, beta=b, s3=s,
                          row_bias=p["row_bias"], col_bias=p["col_bias"])
    from test_parity_gpu import assert_bit_exact
    assert_bit_exact(D.cpu().numpy(), ref["D"], f"random stream-k {seed} D")
    if Aux is not None:
        assert_bit_exact(Aux.cpu().numpy(), ref["Aux"], f"random stream-k {seed} Aux")
    if acc is not None:
        assert np.array_equal(acc.cpu().numpy(), ref["Acc"])


def mixed_cases(n=24, seed=20251203):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        L = int(rng.integers(1, 3))
        M, N = (int(v) for v in rng.integers(1, 601, 2))
        K = int(rng.integers(1, 1501))
        if rng.random() < 0.5:
            N, K = max(8, N - N % 8), max(8, K - K % 8)
        kind = workloads.KINDS[int(rng.integers(0, len(workloads.KINDS)))]
        ab = "bf16" if rng.random() < 0.5 else "f16"
        epi = "f32" if rng.random() < 0.5 else ("f16" if ab == "bf16" else "bf16")
        offset = 1 if rng.random() < 0.2 else 0
        out.append((c, L, M, N, K, kind, ab, epi, offset))
    return out


@pytest.mark.parametrize("case", mixed_cases(),
                         ids=lambda c: f"m{c[0]}-{c[5]}-{c[6]}to{c[7]}-{c[1]}x{c[2]}x{c[3]}x{c[4]}-off{c[8]}")
def test_random_mixed_types_case(case):
    """The same sweep for epilogue tensors of another type than A and B
    (gemm_epi_run_mixed): fp32, or the other 16-bit type."""
    c, L, M, N, K, kind, ab, epi, offset = case
    a, b, s = KIND_SCALARS[kind]
    log(f"[random mixed] case {c}: L={L} M={M} N={N} K={K} {kind} {ab}->{epi} offset={offset}")
    if epi == "f32":
        import test_f32e_gpu as f32e
        p = f32e.problem(L, M, N, K, kind, ab, seed=3000 + c, init="small_int")
        f32e.check(p, kind, ab, a, b, s, exact=True, offset=offset, what=f"random mixed case {c}")
    else:
        import test_mixed16_gpu as m16
        p = m16.problem(L, M, N, K, kind, ab, epi, seed=3000 + c, init="small_int")
        m16.check(p, kind, ab, epi, a, b, s, exact=True, offset=offset, what=f"random mixed case {c}")


def staged_cases(n=24, seed=20251203):
    """Shapes or pointers off the 16-byte rule: K or N not a multiple of 8, or
    tensors at odd element offsets."""
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        L = int(rng.integers(1, 4))
        M, N = (int(v) for v in rng.integers(1, 701, 2))
        K = int(rng.integers(1, 2101))
        offs = (0, 0, 0, 0)
        if rng.random() < 0.4 or (N % 8 == 0 and K % 8 == 0):  # tensors off their 16-byte boundary too
            offs = tuple(int(v) for v in rng.integers(0, 8, 4))
            if not any(offs):
                offs = (1, 0, 0, 0)
        kind = workloads.KINDS[int(rng.integers(0, len(workloads.KINDS)))]
        dtype = torch.bfloat16 if rng.random() < 0.3 else torch.float16
        out.append((c, L, M, N, K, kind, dtype, offs))
    return out


@pytest.mark.parametrize("case", staged_cases(),
                         ids=lambda c: f"s{c[0]}-{c[5]}-{str(c[6])[6:]}-{c[1]}x{c[2]}x{c[3]}x{c[4]}-{''.join(map(str, c[7]))}")
def test_random_staged_case(case):
    """The workspace call staging the operands for the fast kernel."""
    from test_staged_gpu import compare, run_staged
    c, L, M, N, K, kind, dtype, offs = case
    dt = "bf16" if dtype == torch.bfloat16 else "f16"
    log(f"[random staged] case {c}: L={L} M={M} N={N} K={K} {kind} {dt} offsets={offs}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=3000 + c, dtype=dt)
    got = run_staged(p, kind, offs, dtype)
    compare(got, p, kind, True, dtype, f"random staged case {c}")
