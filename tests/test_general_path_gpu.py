"""The general kernel's operand staging on the GPU: every byte offset of a
chunk and every K and N residue, against the oracle.

The general kernel (K or N not a multiple of 8, or a tensor not 16-byte
aligned) reads each 8-element operand chunk with one 16-byte buffer load
from the 4-byte aligned address at or below it and one 4-byte load, and cuts
the chunk out in registers; the elements past K or N are zeroed there.  These
cases place A and B at every element offset 0..7 of a 16-byte block (so the
chunk's byte offset within its window takes every even value), put each
tensor flush against the end of its allocation (the last window reaches past
the tensor), and sweep K and N over every residue mod 8.  Integer-valued
inputs make the result exact, so the outputs must equal the oracle's bit for
bit (Custom Epilogue Example, Constraints: the 16-byte alignment rule the
fast path needs, and which this path does without).
"""
import numpy as np
import pytest
import torch

import oracle
import dense_gemm_elementwise_amd as ge
from dense_gemm_elementwise_amd import workloads

from test_parity_gpu import DEV, KIND_SCALARS, assert_bit_exact, assert_within_ulp, log, oracle_full

pytestmark = pytest.mark.gpu


def place(v, off, dtype=torch.float16):
    """v on the device, `off` elements into a buffer that ends where v ends."""
    buf = torch.empty(v.size + off, dtype=dtype, device=DEV)
    t = buf[off:].view(v.shape)
    t.copy_(torch.from_numpy(v.view(np.int16)).view(dtype) if dtype == torch.bfloat16 else torch.from_numpy(v))
    return t


def run_placed(p, kind, offs, dtype=torch.float16):
    L, M, K = p["A"].shape
    N = p["B"].shape[2]
    a, b, s = KIND_SCALARS[kind]
    A = place(p["A"], offs[0], dtype)
    B = place(p["B"], offs[1], dtype)
    C = place(p["C"], offs[2], dtype) if p["C"] is not None else None
    X = place(p["X"], offs[2], dtype) if p["X"] is not None else None
    D = torch.empty(L * M * N + offs[3], dtype=dtype, device=DEV)[offs[3]:].view(L, M, N)
    Aux = torch.empty(L * M * N + offs[3], dtype=dtype, device=DEV)[offs[3]:].view(L, M, N) if kind in ge.HAS_AUX else None
    rb = place(p["row_bias"], offs[2], dtype) if p.get("row_bias") is not None else None
    cb = place(p["col_bias"], offs[2], dtype) if p.get("col_bias") is not None else None
    acc = (torch.empty(L * M * N + offs[3], dtype=torch.float32, device=DEV)[offs[3]:].view(L, M, N)
           if kind in ge.HAS_ACC else None)
    ge.run(A, B, C, X, kind=kind, alpha=a, beta=b, s3=s, D=D, Aux=Aux, row_bias=rb, col_bias=cb, acc_out=acc)
    out = {"D": D.cpu().view(torch.int16).numpy()}
    if Aux is not None:
        out["Aux"] = Aux.cpu().view(torch.int16).numpy()
    if acc is not None:
        out["Acc"] = acc.cpu().numpy()
    return out


@pytest.mark.parametrize("offa", range(8))
@pytest.mark.parametrize("offb", [0, 3, 5])
def test_operand_byte_offsets(offa, offb):
    L, M, N, K = 2, 70, 88, 136
    kind = "LINCOMB_X_ACC"
    log(f"[general] offsets A={offa} B={offb}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=100 + 8 * offa + offb)
    got = run_placed(p, kind, (offa, offb, 1, 2))
    ref = oracle_full(p, kind, *KIND_SCALARS[kind], want64=False)
    for name in got:
        assert_bit_exact(got[name].view(np.float16), ref[name], f"general offsets {offa},{offb} {name}")


@pytest.mark.parametrize("k", range(129, 137))
def test_k_residues(k):
    kind = "AUX_SCALE"
    log(f"[general] K={k}")
    p = workloads.make_problem(1, 72, 64, k, kind, init="small_int", seed=k)
    got = run_placed(p, kind, (0, 0, 0, 0))
    ref = oracle_full(p, kind, *KIND_SCALARS[kind], want64=False)
    for name in got:
        assert_bit_exact(got[name].view(np.float16), ref[name], f"general K={k} {name}")


@pytest.mark.parametrize("n", range(129, 137))
def test_n_residues(n):
    kind = "RELU_AUX_STORE"
    log(f"[general] N={n}")
    p = workloads.make_problem(2, 65, n, 200, kind, init="small_int", seed=n)
    got = run_placed(p, kind, (1, 1, 1, 1))
    ref = oracle_full(p, kind, *KIND_SCALARS[kind], want64=False)
    for name in got:
        assert_bit_exact(got[name].view(np.float16), ref[name], f"general N={n} {name}")


def test_bf16_offsets_and_residues():
    """The staging moves raw 16-bit elements: the same on bfloat16 tensors."""
    kind = "LINCOMB"
    a, b, s3 = KIND_SCALARS[kind]
    log("[general] bf16")
    p = workloads.make_problem(1, 100, 131, 77, kind, init="small_int", seed=7, dtype="bf16")
    got = run_placed(p, kind, (3, 6, 1, 5), torch.bfloat16)
    ref = oracle.gemm_epi(p["A"], p["B"], p["C"], p["X"], kind=kind, alpha=a, beta=b, s3=s3, dtype="bf16")
    assert_bit_exact(got["D"].view(np.uint16), ref["D"], "general bf16 D")


def general_cases(n=40, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        L = int(rng.integers(1, 3))
        M, N = (int(v) for v in rng.integers(1, 601, 2))
        K = int(rng.integers(1, 1201))
        kind = workloads.KINDS[int(rng.integers(0, len(workloads.KINDS)))]
        offs = tuple(int(v) for v in rng.integers(0, 8, 4))
        out.append((c, L, M, N, K, kind, offs))
    return out


@pytest.mark.parametrize("case", general_cases(), ids=lambda c: f"g{c[0]}-{c[5]}-{c[1]}x{c[2]}x{c[3]}x{c[4]}-{c[6]}")
def test_random_general_case(case):
    """Seeded random shapes, kinds and independent element offsets of A, B,
    the epilogue inputs (and biases) and the outputs; bit-exact against the oracle (the
    activation kinds within one ulp, as in the other parity tests)."""
    c, L, M, N, K, kind, offs = case
    log(f"[general random] case {c}: L={L} M={M} N={N} K={K} {kind} offsets={offs}")
    p = workloads.make_problem(L, M, N, K, kind, init="small_int", seed=2000 + c)
    got = run_placed(p, kind, offs)
    exact = kind not in ge.ACTIVATIONS
    ref = oracle_full(p, kind, *KIND_SCALARS[kind], want64=not exact)
    for name in got:
        if name == "Acc":  # integer inputs: every fp32 partial sum is exact
            assert np.array_equal(got[name], ref["Acc"]), f"general random {c} acc_out"
            continue
        g = got[name].view(np.float16)
        if exact:
            assert_bit_exact(g, ref[name], f"general random {c} {name}")
        else:
            assert_within_ulp(g, ref[name + "64"], ref[name], f"general random {c} {name}")
