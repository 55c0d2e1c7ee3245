"""Seeded synthetic workloads for the fused fp16 GEMM + epilogue.

This module only draws inputs: it holds none of the method's arithmetic (no
product, no epilogue, no rounding of results).  Both the HIP path and the CPU
oracle are fed from it, so a workload's inputs are bit-identical on both
sides.  All tensors are packed row-major host arrays of float16:
A (L,M,K), B (L,K,N), C and X (L,M,N).

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
"""
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

KINDS = ("LINCOMB", "AUX_SCALE", "LINCOMB_X_ACC", "RELU", "SQUARE", "RELU_SQUARE")
HAS_AUX = ("AUX_SCALE", "LINCOMB_X_ACC", "SQUARE", "RELU_SQUARE")
READS_X = ("LINCOMB_X_ACC",)


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

    @property
    def flops(self) -> int:
        """Algorithmic work of one call: 2*L*M*N*K."""
        return 2 * self.L * self.M * self.N * self.K

    @property
    def epilogue_bytes(self) -> int:
        """Epilogue traffic of one call: C (and X) read once, D (and the second output) written once."""
        n_in_mn = 1 + (1 if self.kind in READS_X else 0)
        n_out = 1 + (1 if self.kind in HAS_AUX else 0)
        return 2 * (n_in_mn + n_out) * self.L * self.M * self.N

    @property
    def hbm_bytes(self) -> int:
        """Compulsory HBM traffic: every operand read once, every output written once."""
        n_in_mn = 1 + (1 if self.kind in READS_X else 0)
        n_out = 1 + (1 if self.kind in HAS_AUX else 0)
        return 2 * (self.L * self.M * self.K + self.L * self.K * self.N + (n_in_mn + n_out) * self.L * self.M * self.N)


# The five workloads, smallest first.  The third is the pages' "run a bigger
# problem" case (not tile multiples), the fourth is the Alpha-Beta example's
# command line, the fifth is the batched multi-output case.
WORKLOADS: Dict[str, Workload] = {w.name: w for w in (
    Workload("aux_scale_128", 1, 128, 128, 128, "AUX_SCALE", 1.0, 2.0, 0.5, "randint_pm2", 2025, True),
    Workload("aux_scale_1024", 1, 1024, 1024, 1024, "AUX_SCALE", 1.0, 2.0, 0.5, "randint_pm2", 2025, True),
    Workload("lincomb_2400x3232x4096", 1, 2400, 3232, 4096, "LINCOMB", 1.0, 2.0, 0.0, "ceil_uniform_pm4", 1234, True),
    Workload("x_acc_8192", 1, 8192, 8192, 8192, "LINCOMB_X_ACC", 2.0, 1.0, 3.0, "normal", 2025, False),
    Workload("relu_square_16x2048x2048x1024", 16, 2048, 2048, 1024, "RELU_SQUARE", 1.0, 1.0, 0.0, "normal", 2025,
             False),
)}

# The workload the headline throughput is quoted on.
HEADLINE = "x_acc_8192"


def _shapes(L, M, N, K, with_x):
    shapes = [(L, M, K), (L, K, N), (L, M, N)]
    if with_x:
        shapes.append((L, M, N))
    return shapes


def draw(init: str, seed: int, L: int, M: int, N: int, K: int, with_x: bool):
    """Draws A, B, C (and X) as float16 numpy arrays with the named recipe."""
    shapes = _shapes(L, M, N, K, with_x)
    if init == "randint_pm2":
        g = torch.Generator().manual_seed(seed)
        out = [torch.randint(-2, 3, s, generator=g, dtype=torch.float16).numpy() for s in shapes]
    elif init == "ceil_uniform_pm4":
        rs = np.random.RandomState(seed)
        out = [np.ceil(rs.uniform(-4, 4, size=s).astype(np.float16)) for s in shapes]
    elif init == "normal":
        g = torch.Generator().manual_seed(seed)
        out = [torch.randn(s, generator=g, dtype=torch.float32).to(torch.float16).numpy() for s in shapes]
    elif init == "small_int":
        # integers uniform in {-3..3}; used by the tail and kind sweeps
        g = torch.Generator().manual_seed(seed)
        out = [torch.randint(-3, 4, s, generator=g, dtype=torch.float16).numpy() for s in shapes]
    else:
        raise ValueError(f"unknown init recipe {init!r}")
    return [np.ascontiguousarray(a) for a in out]


def make_inputs(w: Workload) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of a named workload: dict with A, B, C and X (None if unused)."""
    arrs = draw(w.init, w.seed, w.L, w.M, w.N, w.K, w.kind in READS_X)
    return {"A": arrs[0], "B": arrs[1], "C": arrs[2], "X": arrs[3] if len(arrs) > 3 else None}


def make_problem(L, M, N, K, kind, init="small_int", seed=0):
    """Inputs for an arbitrary shape (tests): dict with A, B, C and X (None if unused)."""
    arrs = draw(init, seed, L, M, N, K, kind in READS_X)
    return {"A": arrs[0], "B": arrs[1], "C": arrs[2], "X": arrs[3] if len(arrs) > 3 else None}
