"""Every output element of the full-size workloads against the oracle.

The 8192^3 products (the Alpha-Beta example's size) and the 16-batch case
are compared element by element with the full oracle (fp64, OpenMP over the
host's cores: about 14 s per 8192^3 product on 16 cores), not only at sampled
points: |gpu - ref| <= 5e-2 + 1e-2 |ref| for every D, Aux and acc_out
element, ref the oracle's unrounded value, and no non-finite output.
"""
import pytest

from dense_gemm_elementwise_amd import workloads
from test_bf16_gpu import check_bf16
from test_parity_gpu import check_full, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["x_acc_8192", "relu_square_16x2048x2048x1024", "relu_scale_acc_8192",
                                  "bias_row_col_8192", "gelu_8192", "x_acc_bf16_8192"])
def test_whole_output_against_the_oracle(name):
    w = workloads.WORKLOADS[name]
    log(f"[full] {w.name}: L={w.L} M={w.M} N={w.N} K={w.K} {w.kind} {w.dtype}")
    p = workloads.make_inputs(w)
    if w.dtype == "bf16":
        check_bf16(p, w.kind, w.alpha, w.beta, w.s3, exact=w.exact, what=f"full {w.name}")
    else:
        check_full(p, w.kind, w.alpha, w.beta, w.s3, exact=w.exact, what=f"full {w.name}")
