"""Seeded synthetic workloads for the fused fp16 GEMM + epilogue.

This module only draws inputs: it holds none of the method's arithmetic (no
product, no epilogue, no rounding of results).  Both the HIP path and the CPU
oracle are fed from it, so a workload's inputs are bit-identical on both
sides.  All tensors are packed row-major host arrays of float16 (for a bfloat16
workload: uint16 arrays holding bfloat16 bit patterns, numpy having no such
type): A (L,M,K), B (L,K,N), C and X (L,M,N), row_bias (N,) and col_bias (M,).

The draws follow the constructions on the pages:
  - "randint_pm2": integers uniform in {-2..2}, drawn A, then B, then C from
    one generator seeded 2025 (CUTLASS Operator API tutorial "Custom epilogue
    fusions for GEMMs", cell [2]; the page draws on the GPU, here the CPU
    generator is used so the values can be reproduced anywhere);
  - "ceil_uniform_pm4": ceil(float16(uniform(-4, 4))) from NumPy's legacy
    RandomState(1234), A then B then C (CUTLASS Python examples article,
    "Basic GEMM", input construction; the cast happens before the ceil, as
    printed, so zeros come out as -0.0 and the values lie in {-4..4});
  - "normal": N(0, 1) drawn in float32 from a generator seeded 2025, then
    rounded to float16, in the order A, B, C, X (the pages do not show how the
    Alpha-Beta example fills its tensors).
A bfloat16 workload draws the same values with the same generator and
rounds them to bfloat16 instead (the integer recipes are exact in both).
For the bias kind (tutorial cell [9]) C is not drawn; the row bias (N,) and
the column bias (M,) follow A and B from the same generator: N(0, 1) rounded
to float16 as the page draws them (torch.randn in float16), or integers in
{-3..3} for the integer test recipe, so that those cases stay exact.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

ACTIVATIONS = ("SIGMOID", "TANH", "GELU", "SILU", "LEAKY_RELU", "HARDSWISH")
KINDS = ("LINCOMB", "AUX_SCALE", "LINCOMB_X_ACC", "RELU", "SQUARE", "RELU_SQUARE", "RELU_AUX_STORE",
         "RELU_SCALE_ACC", "BIAS_ROW_COL") + ACTIVATIONS
# kinds made of + - * and ReLU only: exact on integer inputs and rational
# arithmetic (the activations have their own bar and pins)
EXACT_KINDS = tuple(k for k in KINDS if k not in ACTIVATIONS)
HAS_AUX = ("AUX_SCALE", "LINCOMB_X_ACC", "SQUARE", "RELU_SQUARE", "RELU_AUX_STORE", "RELU_SCALE_ACC")
READS_X = ("LINCOMB_X_ACC",)
READS_C = tuple(k for k in KINDS if k != "BIAS_ROW_COL")
READS_BIAS = ("BIAS_ROW_COL",)
HAS_ACC = ("RELU_SCALE_ACC",)  # also writes the fp32 accumulator


@dataclass(frozen=True)
class Workload:
    name: str
    L: int
    M: int
    N: int
    K: int
    kind: str
    alpha: float
    beta: float
    s3: float
    init: str
    seed: int
    exact: bool  # integer-valued inputs: results must be bit-exact
    note: str = field(default="", compare=False)
    dtype: str = "f16"  # element type of the 16-bit tensors: "f16" or "bf16"

    @property
    def flops(self) -> int:
        """Algorithmic work of one call: 2*L*M*N*K."""
        return 2 * self.L * self.M * self.N * self.K

    @property
    def epilogue_bytes(self) -> int:
        """Epilogue traffic of one call: C / X / the biases read once, D, the second output and the
        fp32 accumulator (if the kind has them) written once."""
        return epilogue_bytes(self.kind, self.L, self.M, self.N)

    @property
    def hbm_bytes(self) -> int:
        """Compulsory HBM traffic: every operand read once, every output written once."""
        return 2 * (self.L * self.M * self.K + self.L * self.K * self.N) + self.epilogue_bytes


def epilogue_bytes(kind: str, L: int, M: int, N: int) -> int:
    halves_mn = ((kind in READS_C) + (kind in READS_X) + 1 + (kind in HAS_AUX) + 2 * (kind in HAS_ACC))
    bias = (M + N) if kind in READS_BIAS else 0
    return 2 * (halves_mn * L * M * N + bias)


# The workloads.  The first five, smallest first: the third is the pages' "run a bigger
# problem" case (not tile multiples), the fourth is the Alpha-Beta example's
# command line, the fifth is the batched multi-output case.
WORKLOADS: Dict[str, Workload] = {w.name: w for w in (
    Workload("aux_scale_128", 1, 128, 128, 128, "AUX_SCALE", 1.0, 2.0, 0.5, "randint_pm2", 2025, True),
    Workload("aux_scale_1024", 1, 1024, 1024, 1024, "AUX_SCALE", 1.0, 2.0, 0.5, "randint_pm2", 2025, True),
    Workload("lincomb_2400x3232x4096", 1, 2400, 3232, 4096, "LINCOMB", 1.0, 2.0, 0.0, "ceil_uniform_pm4", 1234, True),
    Workload("x_acc_8192", 1, 8192, 8192, 8192, "LINCOMB_X_ACC", 2.0, 1.0, 3.0, "normal", 2025, False),
    Workload("relu_square_16x2048x2048x1024", 16, 2048, 2048, 1024, "RELU_SQUARE", 1.0, 1.0, 0.0, "normal", 2025,
             False),
    # the tutorial's further epilogues, on its own shape and draws (cells [2], [6], [7], [9])
    Workload("relu_aux_store_1024", 1, 1024, 1024, 1024, "RELU_AUX_STORE", 3.0, 2.0, 0.0, "randint_pm2", 2025, True),
    Workload("relu_scale_acc_1024", 1, 1024, 1024, 1024, "RELU_SCALE_ACC", 1.0, 2.0, 0.5, "randint_pm2", 2025, True),
    Workload("bias_row_col_1024", 1, 1024, 1024, 1024, "BIAS_ROW_COL", 1.0, 0.0, 0.0, "randint_pm2", 2025, False),
    # the heaviest and the lightest of those epilogues at the headline size
    Workload("relu_scale_acc_8192", 1, 8192, 8192, 8192, "RELU_SCALE_ACC", 1.0, 2.0, 0.5, "normal", 2025, False),
    Workload("bias_row_col_8192", 1, 8192, 8192, 8192, "BIAS_ROW_COL", 1.0, 0.0, 0.0, "normal", 2025, False),
    # few output tiles and a deep K (not one of the pages' runs): the case a
    # stream-K split of K across workgroups is for
    Workload("lincomb_deep_k_256x256x65536", 1, 256, 256, 65536, "LINCOMB", 1.0, 2.0, 0.0, "normal", 2025, False),
    # the built-in activations on the Python examples article's Epilogue
    # example: m = n = k = 256, inputs built as in its Basic GEMM example,
    # plan.run's default alpha = 1, beta = 0 (leaky ReLU's slope: 1/8)
    *(Workload(f"{a.lower()}_256", 1, 256, 256, 256, a, 1.0, 0.0, 0.125 if a == "LEAKY_RELU" else 0.0,
               "ceil_uniform_pm4", 1234, False) for a in ACTIVATIONS),
    # GELU at the headline size; alpha = 1/64 puts alpha*acc + beta*C (acc has
    # standard deviation sqrt(K) = 90.5) where the activation is not flat
    Workload("gelu_8192", 1, 8192, 8192, 8192, "GELU", 1.0 / 64, 1.0, 0.0, "normal", 2025, False),
    # bfloat16 operands and outputs (the Custom Epilogue Example's "Data Type
    # Support"): the tutorial's 1024^3 case (integers, exact) and the headline
    Workload("aux_scale_bf16_1024", 1, 1024, 1024, 1024, "AUX_SCALE", 1.0, 2.0, 0.5, "randint_pm2", 2025, True,
             dtype="bf16"),
    Workload("x_acc_bf16_8192", 1, 8192, 8192, 8192, "LINCOMB_X_ACC", 2.0, 1.0, 3.0, "normal", 2025, False,
             dtype="bf16"),
)}

# The workload the headline throughput is quoted on.
HEADLINE = "x_acc_8192"
# The five configurations the throughput is reported on, in order: 128^3 and
# 1024^3 (tutorial cell [2]), the Python article's 2400 x 3232 x 4096, the
# headline, and the 16-batch multi-output case.
CONFIGS = ("aux_scale_128", "aux_scale_1024", "lincomb_2400x3232x4096", "x_acc_8192",
           "relu_square_16x2048x2048x1024")


def to_bf16_bits(t) -> np.ndarray:
    """A float32 (or exactly convertible) torch tensor rounded to bfloat16,
    to nearest with ties to even, as a uint16 numpy array of bit patterns."""
    return t.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float32 values (exact)."""
    return (np.ascontiguousarray(bits).astype(np.uint32) << 16).view(np.float32)


def draw(init: str, seed: int, L: int, M: int, N: int, K: int, with_x: bool, kind: str = "LINCOMB",
         dtype: str = "f16"):
    """Draws the inputs of one problem with the named recipe, in the order
    A, B, then C (and X) or, for the bias kind, the row and column biases.
    Returns a list of float16 numpy arrays in that order (uint16 bfloat16
    bit patterns when dtype is "bf16")."""
    if dtype == "bf16":
        # the same values, drawn in float32 from the same generator
        if init == "randint_pm2":
            g = torch.Generator().manual_seed(seed)
            shapes = [(L, M, K), (L, K, N)] + ([] if kind in READS_BIAS else [(L, M, N)] * (2 if with_x else 1))
            out = [to_bf16_bits(torch.randint(-2, 3, s, generator=g, dtype=torch.float32)) for s in shapes]
            if kind in READS_BIAS:
                out += [to_bf16_bits(torch.randn(s, generator=g, dtype=torch.float32)) for s in ((N,), (M,))]
            return out
        if init in ("normal", "small_int"):
            f = draw(init, seed, L, M, N, K, with_x, kind, dtype="f32")
            return [to_bf16_bits(torch.from_numpy(a)) for a in f]
        raise ValueError(f"recipe {init!r} has no bfloat16 form")
    bias = kind in READS_BIAS
    shapes = [(L, M, K), (L, K, N)]
    if not bias:
        shapes.append((L, M, N))
        if with_x:
            shapes.append((L, M, N))
    if init == "randint_pm2":
        g = torch.Generator().manual_seed(seed)
        out = [torch.randint(-2, 3, s, generator=g, dtype=torch.float16).numpy() for s in shapes]
        if bias:
            out += [torch.randn(s, generator=g, dtype=torch.float16).numpy() for s in ((N,), (M,))]
    elif init == "ceil_uniform_pm4":
        rs = np.random.RandomState(seed)
        out = [np.ceil(rs.uniform(-4, 4, size=s).astype(np.float16)) for s in shapes]
        if bias:
            out += [np.ceil(rs.uniform(-4, 4, size=s).astype(np.float16)) for s in ((N,), (M,))]
    elif init == "normal":
        g = torch.Generator().manual_seed(seed)
        cast = (lambda t: t.numpy()) if dtype == "f32" else (lambda t: t.to(torch.float16).numpy())
        out = [cast(torch.randn(s, generator=g, dtype=torch.float32)) for s in shapes]
        if bias:
            out += [cast(torch.randn(s, generator=g, dtype=torch.float32)) for s in ((N,), (M,))]
    elif init == "small_int":
        # integers uniform in {-3..3}; used by the tail and kind sweeps
        g = torch.Generator().manual_seed(seed)
        tdt = torch.float32 if dtype == "f32" else torch.float16
        out = [torch.randint(-3, 4, s, generator=g, dtype=tdt).numpy() for s in shapes]
        if bias:
            out += [torch.randint(-3, 4, s, generator=g, dtype=tdt).numpy() for s in ((N,), (M,))]
    else:
        raise ValueError(f"unknown init recipe {init!r}")
    return [np.ascontiguousarray(a) for a in out]


def _as_dict(arrs, kind):
    if kind in READS_BIAS:
        return {"A": arrs[0], "B": arrs[1], "C": None, "X": None, "row_bias": arrs[2], "col_bias": arrs[3]}
    return {"A": arrs[0], "B": arrs[1], "C": arrs[2], "X": arrs[3] if len(arrs) > 3 else None,
            "row_bias": None, "col_bias": None}


def make_inputs(w: Workload) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of a named workload: dict with A, B, C, X, row_bias, col_bias
    (None where the kind does not read them)."""
    return _as_dict(draw(w.init, w.seed, w.L, w.M, w.N, w.K, w.kind in READS_X, w.kind, w.dtype), w.kind)


def make_problem(L, M, N, K, kind, init="small_int", seed=0, dtype="f16"):
    """Inputs for an arbitrary shape (tests), as make_inputs returns them."""
    return _as_dict(draw(init, seed, L, M, N, K, kind in READS_X, kind, dtype), kind)
