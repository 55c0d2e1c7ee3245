"""The C-ABI boundary without a GPU: the library loads, exports every function
include/gemm_epi.h declares, and rejects bad arguments with the documented
status codes before making any HIP call.  The status codes mirror the
argument errors of the CUTLASS Operator API tutorial "Custom epilogue
fusions for GEMMs" (cells [10]-[13]: an output or operand that is not
provided) and the early, readable errors of the CUTLASS Python examples
article ("Basic GEMM", error handling)."""
import ctypes
import os
import re

import pytest

import dense_gemm_elementwise_amd as ge
from dense_gemm_elementwise_amd import binding, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_epi.h")

# fake device addresses: never dereferenced by the checks under test
P16 = 0x7F0000001000  # 16-byte aligned
P2 = 0x7F0000001002   # 2-byte aligned only
P1 = 0x7F0000001001   # misaligned
SC = (1.0, 2.0, 0.5)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_epi_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == {"gemm_epi_run", "gemm_epi_run_ext", "gemm_epi_run_typed", "gemm_epi_run_ws",
                          "gemm_epi_run_unfused", "gemm_epi_run_ws_typed", "gemm_epi_run_unfused_typed",
                          "gemm_epi_run_mixed",
                          "gemm_epi_status_string", "gemm_epi_last_hip_error", "gemm_epi_plan", "gemm_epi_plan_ext",
                          "gemm_epi_plan_ws", "gemm_epi_run_ws_static"}
    raw = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(binding.EXPORTS) == set(names)


def test_enum_values_match_header():
    text = open(HEADER).read()
    for name, val in ge.KINDS.items():
        assert re.search(rf"GEMM_EPI_{name}\s*=\s*{val}\b", text), name
    for val, name in binding.STATUS.items():
        assert re.search(rf"{name}\s*=\s*{val}\b", text), name
    for name, val in binding.DTYPES.items():
        assert re.search(rf"GEMM_EPI_{name.upper()}\s*=\s*{val}\b", text), name


def test_status_strings():
    for code in range(9):
        s = ge.gemm_epi_status_string(code)
        assert isinstance(s, str) and s
    assert ge.gemm_epi_status_string(0) == "ok"
    assert ge.gemm_epi_status_string(99) == "unknown status"
    assert ge.gemm_epi_last_hip_error() == 0


def run(L=1, M=8, N=8, K=8, A=P16, B=P16, C=P16, X=P16, sc=SC, kind=0, D=P16, Aux=P16):
    return ge.gemm_epi_run(L, M, N, K, A, B, C, X, sc, kind, D, Aux, None)


@pytest.mark.parametrize("shape", [(0, 8, 8, 8), (1, 0, 8, 8), (1, 8, 0, 8), (1, 8, 8, 0), (-1, 8, 8, 8),
                                   (1, 2 ** 31, 8, 8), (1, 8, 8, 2 ** 31), (2 ** 40, 2 ** 20, 2 ** 20, 8)])
def test_bad_shapes(shape):
    L, M, N, K = shape
    assert run(L=L, M=M, N=N, K=K) == 1


def test_missing_inputs():
    assert run(A=None) == 2
    assert run(B=None) == 2
    assert run(C=None) == 2  # every kind but the bias kind reads C, also with beta = 0
    assert run(sc=None) == 2
    assert run(kind=2, X=None) == 2  # LINCOMB_X_ACC reads X


def test_missing_outputs():
    assert run(D=None) == 3
    for kind in ("AUX_SCALE", "LINCOMB_X_ACC", "SQUARE", "RELU_SQUARE", "RELU_AUX_STORE"):
        assert run(kind=ge.KINDS[kind], Aux=None) == 3, kind


@pytest.mark.parametrize("kind", [-1, 15, 100])
def test_unknown_kind(kind):
    assert run(kind=kind) == 4


def run_ext(L=1, M=8, N=8, K=8, A=P16, B=P16, C=P16, X=P16, rb=P16, cb=P16, sc=SC, kind=0, D=P16, Aux=P16,
            acc=P16):
    return ge.gemm_epi_run_ext(L, M, N, K, A, B, C, X, rb, cb, sc, kind, D, Aux, acc, None)


def plan_ext(L=1, M=256, N=256, K=256, A=P16, B=P16, C=P16, X=None, rb=None, cb=None, kind=0, D=P16, Aux=None,
             acc=None):
    return ge.gemm_epi_plan_ext(L, M, N, K, A, B, C, X, rb, cb, kind, D, Aux, acc)


def test_kinds_needing_ext_operands_are_rejected_by_the_plain_entry_point():
    # gemm_epi_run has no bias inputs and no accumulator output
    assert run(kind=ge.KINDS["BIAS_ROW_COL"]) == 2
    assert run(kind=ge.KINDS["RELU_SCALE_ACC"]) == 3
    assert ge.gemm_epi_plan(1, 8, 8, 8, P16, P16, P16, None, ge.KINDS["BIAS_ROW_COL"], P16, None)[0] == 2


def test_ext_operand_checks():
    bias, acc = ge.KINDS["BIAS_ROW_COL"], ge.KINDS["RELU_SCALE_ACC"]
    assert run_ext(kind=bias, rb=None) == 2
    assert run_ext(kind=bias, cb=None) == 2
    assert run_ext(kind=acc, acc=None) == 3
    assert run_ext(kind=acc, Aux=None) == 3
    assert run_ext(kind=acc, C=None) == 2          # RELU_SCALE_ACC reads C
    assert run_ext(kind=ge.KINDS["RELU_AUX_STORE"], Aux=None) == 3
    assert run_ext(kind=acc, acc=P2) == 5          # fp32 output not 4-byte aligned
    assert run_ext(kind=bias, rb=P1) == 5
    assert run_ext(kind=bias, cb=P1) == 5
    assert run_ext(kind=bias, sc=None) == 2
    # valid argument sets (checked by the host-only planner, nothing is launched)
    assert plan_ext(kind=bias, C=None, rb=P16, cb=P16)[0] == 0   # the bias kind does not read C
    assert plan_ext(kind=acc, Aux=P16, acc=P16)[0] == 0
    assert plan_ext(kind=ge.KINDS["RELU_AUX_STORE"], Aux=P16)[0] == 0


def test_typed_entry_point_checks():
    def typed(dtype, **kw):
        a = dict(A=P16, B=P16, C=P16, X=P16, rb=P16, cb=P16, D=P16, Aux=P16, acc=P16)
        a.update(kw)
        return ge.gemm_epi_run_typed(1, 8, 8, 8, a["A"], a["B"], a["C"], a["X"], a["rb"], a["cb"], SC, 0, a["D"],
                                     a["Aux"], a["acc"], dtype, None)
    assert typed(2) == 8 and typed(-1) == 8            # unknown element type
    assert typed("bf16", A=None) == 2                  # the argument checks come first
    assert typed("bf16", D=None) == 3
    assert typed("bf16", C=P1) == 5
    assert ge.gemm_epi_status_string(8) == "unknown element type"


def test_typed_composition_checks():
    """gemm_epi_run_ws_typed and gemm_epi_run_unfused_typed check the element
    type after the operands and before anything else (no launch here)."""
    def ws_typed(dtype, **kw):
        a = dict(A=P16, D=P16, ws=P16, ws_bytes=1 << 30)
        a.update(kw)
        return ge.gemm_epi_run_ws_typed(1, 256, 256, 65536, a["A"], P16, P16, None, None, None, SC, 0, a["D"],
                                        None, None, a["ws"], a["ws_bytes"], dtype, None)

    def unfused_typed(dtype, **kw):
        a = dict(A=P16, D=P16, ws=P16, ws_bytes=8 * 8 * 4)
        a.update(kw)
        return ge.gemm_epi_run_unfused_typed(1, 8, 8, 8, a["A"], P16, P16, None, None, None, SC, 0, a["D"], None,
                                             None, a["ws"], a["ws_bytes"], dtype, None)
    for f in (ws_typed, unfused_typed):
        assert f(2) == 8 and f(-1) == 8                # unknown element type
        assert f("bf16", A=None) == 2                  # the argument checks come first
        assert f("bf16", D=None) == 3
        assert f(7, A=P1) == 5
    # the workspace checks follow the element type's
    assert ws_typed("bf16", ws=None) == 7
    assert ws_typed("bf16", ws_bytes=16) == 7
    assert ws_typed("bf16", ws=P2) == 5
    assert unfused_typed("bf16", ws=None) == 7
    assert unfused_typed("bf16", ws_bytes=8 * 8 * 4 - 1) == 7


def test_mixed_entry_point_checks():
    """gemm_epi_run_mixed: A and B fp16 or bf16; epilogue tensors fp16, bf16
    or fp32; fp32 tensors 4-byte aligned (no launch here)."""
    def mixed(ab, epi, **kw):
        a = dict(A=P16, C=P16, D=P16, Aux=P16)
        a.update(kw)
        return ge.gemm_epi_run_mixed(1, 8, 8, 8, a["A"], P16, a["C"], P16, P16, P16, SC, 1, a["D"], a["Aux"], None,
                                     ab, epi, None)
    assert mixed("f32", "f32") == 8            # fp32 A and B are not a combination
    assert mixed(5, "f32") == 8 and mixed("f16", 7) == 8 and mixed("bf16", -1) == 8
    assert mixed("f16", "f32", A=None) == 2    # the argument checks come first
    assert mixed("bf16", "f32", Aux=None) == 3
    assert mixed("f16", "f32", C=P2) == 5      # fp32 C only 2-byte aligned
    assert mixed("bf16", "f32", D=P2) == 5
    assert mixed("f16", "f32", D=P1) == 5
    assert mixed("f16", "bf16", C=P1) == 5     # 16-bit C must be 2-byte aligned
    assert mixed("bf16", "f16", A=None) == 2


def test_unfused_workspace_checks():
    def unfused(kind=0, ws=P16, ws_bytes=8 * 8 * 4, acc=None, Aux=P16):
        return ge.gemm_epi_run_unfused(1, 8, 8, 8, P16, P16, P16, P16, P16, P16, SC, kind, P16, Aux, acc, ws,
                                       ws_bytes, None)
    assert unfused(ws=None) == 7
    assert unfused(ws_bytes=8 * 8 * 4 - 1) == 7
    assert unfused(ws=P2) == 5                      # fp32 workspace not 4-byte aligned
    assert unfused(kind=ge.KINDS["RELU_SCALE_ACC"], ws=None, acc=None) == 3   # needs acc_out
    assert unfused(kind=-3) == 4
    assert ge.gemm_epi_status_string(7).startswith("the workspace")


def test_stream_k_plan_and_workspace_checks():
    def plan_ws(L, M, N, K):
        return ge.gemm_epi_plan_ws(L, M, N, K, P16, P16, P16, None, None, None, 0, P16, None, None)
    # few tiles, long K: split over 128 x 128 tiles.  The workgroup count is
    # searched: a shorter K per workgroup against more partial sums per tile
    # (for 256 x 256 x 65536, 128 workgroups measured fastest of 16..256).  The
    # workspace holds a fixed 16 KiB counter block (one int32 per tile, at most
    # 4096 split tiles) and then two partial slots per workgroup.
    rc, cfg = plan_ws(1, 256, 256, 65536)
    assert rc == 0 and (cfg["bm"], cfg["bn"], cfg["workgroups"]) == (128, 128, 128)
    assert cfg["workspace_bytes"] == 16384 + 2 * 128 * 128 * 128 * 4
    rc, cfg = plan_ws(1, 256, 256, 16384)
    assert rc == 0 and (cfg["bm"], cfg["bn"], cfg["workgroups"]) == (128, 128, 64)
    assert cfg["workspace_bytes"] == 16384 + 2 * 64 * 128 * 128 * 4
    for shape in ((1, 200, 304, 12000), (2, 128, 384, 8192), (1, 512, 512, 8192)):
        rc, cfg = plan_ws(*shape)
        assert rc == 0 and cfg["workspace_bytes"] > 0, shape
    # enough tiles (or too short a K for the split's fixed cost): no split, no
    # workspace, the same plan as gemm_epi_plan
    # (1024 x 1024 x 8192 measured slower split at 256 workgroups: the
    # contributors' operand streams share little in L2)
    for shape in ((1, 8192, 8192, 8192), (1, 1024, 1024, 1024), (1, 128, 128, 128), (1, 1024, 1024, 8192)):
        rc, cfg = plan_ws(*shape)
        rc0, cfg0 = ge.gemm_epi_plan(*shape, P16, P16, P16, None, 0, P16, None)
        assert rc == rc0 == 0 and cfg["workspace_bytes"] == 0
        assert all(cfg[k] == cfg0[k] for k in cfg0), shape
    # a split call without (enough) workspace is refused before any launch
    need = 16384 + 2 * 64 * 128 * 128 * 4
    args = (1, 256, 256, 16384, P16, P16, P16, None, None, None, SC, 0, P16, None, None)
    assert ge.gemm_epi_run_ws(*args, None, need, None) == 7
    assert ge.gemm_epi_run_ws(*args, P16, need - 1, None) == 7
    assert ge.gemm_epi_run_ws(*args, 0x7F0000001008, need, None) == 5   # not 16-byte aligned


def test_ext_fast_path_conditions():
    bias, acc = ge.KINDS["BIAS_ROW_COL"], ge.KINDS["RELU_SCALE_ACC"]
    rc, cfg = plan_ext(kind=bias, C=None, rb=P16, cb=P2)
    assert rc == 0 and cfg["vec"] == 1             # the column bias is read one value at a time
    rc, cfg = plan_ext(kind=bias, C=None, rb=P2, cb=P16)
    assert rc == 0 and cfg["vec"] == 0             # the row bias is read in 16-byte vectors
    rc, cfg = plan_ext(kind=acc, Aux=P16, acc=P16)
    assert rc == 0 and cfg["vec"] == 1
    rc, cfg = plan_ext(kind=acc, Aux=P16, acc=0x7F0000001004)
    assert rc == 0 and cfg["vec"] == 0             # fp32 output stored in 16-byte vectors


def test_misaligned_pointers():
    for arg in ("A", "B", "C", "D"):
        assert run(**{arg: P1}) == 5, arg
    assert run(kind=2, X=P1) == 5
    assert run(kind=1, Aux=P1) == 5


def test_plan_fast_and_general_paths():
    rc, cfg = ge.gemm_epi_plan(1, 256, 256, 256, P16, P16, P16, None, 0, P16, None)
    assert rc == 0 and cfg["vec"] == 1 and cfg["threads"] in (256, 512) and cfg["bk"] in (32, 64, 128)
    # K or N not a multiple of 8, or a pointer not 16-byte aligned -> general kernel
    for args in ((1, 256, 256, 250), (1, 256, 250, 256)):
        rc, cfg = ge.gemm_epi_plan(*args, P16, P16, P16, None, 0, P16, None)
        assert rc == 0 and cfg["vec"] == 0
    rc, cfg = ge.gemm_epi_plan(1, 256, 256, 256, P2, P16, P16, None, 0, P16, None)
    assert rc == 0 and cfg["vec"] == 0
    # one batch entry of A at 2 GiB or more -> general kernel (32-bit buffer offsets)
    rc, cfg = ge.gemm_epi_plan(1, 2 ** 15, 8, 2 ** 15, P16, P16, P16, None, 0, P16, None)
    assert rc == 0 and cfg["vec"] == 0
    # errors are reported by plan as by run
    assert ge.gemm_epi_plan(1, 8, 8, 8, None, P16, P16, None, 0, P16, None)[0] == 2


def test_plan_tiles_for_the_workloads():
    want = {
        "aux_scale_128": (64, 64, 64, 4),
        "aux_scale_1024": (64, 64, 128, 256),
        "lincomb_2400x3232x4096": (128, 256, 32, 19 * 13),
        "x_acc_8192": (256, 256, 32, 1024),
        "relu_square_16x2048x2048x1024": (256, 256, 32, 1024),
        "relu_aux_store_1024": (64, 64, 128, 256),
        "relu_scale_acc_1024": (64, 64, 128, 256),
        "bias_row_col_1024": (64, 64, 128, 256),
        "relu_scale_acc_8192": (256, 256, 32, 1024),
        "bias_row_col_8192": (256, 256, 32, 1024),
        "lincomb_deep_k_256x256x65536": (64, 64, 128, 16),
        "gelu_8192": (256, 256, 32, 1024),
        "aux_scale_bf16_1024": (64, 64, 128, 256),     # the tile choice does not depend on the element type
        "x_acc_bf16_8192": (256, 256, 32, 1024),
    }
    want.update({f"{a.lower()}_256": (64, 64, 128, 16) for a in workloads.ACTIVATIONS})
    assert set(want) == set(workloads.WORKLOADS)
    for name, (bm, bn, bk, wgs) in want.items():
        w = workloads.WORKLOADS[name]
        rc, cfg = ge.gemm_epi_plan_ext(w.L, w.M, w.N, w.K, P16, P16, P16, P16, P16, P16, ge.KINDS[w.kind], P16, P16,
                                       P16)
        assert rc == 0, name
        assert (cfg["bm"], cfg["bn"], cfg["bk"], cfg["workgroups"]) == (bm, bn, bk, wgs), (name, cfg)
        assert cfg["vec"] == 1


def test_small_tile_k_step_follows_k():
    """The 64 x 64 tile steps K by 64 below K = 256 and by 128 from there on;
    the other tiles and the general kernel do not depend on K."""
    for K, bk in ((8, 64), (128, 64), (248, 64), (256, 128), (520, 128), (8192, 128)):
        rc, cfg = ge.gemm_epi_plan(1, 1024, 1024, K, P16, P16, P16, None, 0, P16, None)
        assert rc == 0 and (cfg["bm"], cfg["bn"], cfg["bk"], cfg["vec"]) == (64, 64, bk, 1), (K, cfg)
    for K in (256, 512, 4096):
        rc, cfg = ge.gemm_epi_plan(1, 8192, 8192, K, P16, P16, P16, None, 0, P16, None)
        assert rc == 0 and (cfg["bm"], cfg["bn"], cfg["bk"], cfg["threads"]) == (256, 256, 32, 256), (K, cfg)
        rc, cfg = ge.gemm_epi_plan(1, 1024, 1024, K + 2, P16, P16, P16, None, 0, P16, None)
        assert rc == 0 and cfg["vec"] == 0 and cfg["bk"] == 64, (K, cfg)


def test_python_wrapper_rejects_bad_tensors():
    import torch
    A = torch.zeros(1, 8, 8, dtype=torch.float16)
    with pytest.raises(ValueError):
        ge.run(A, A, A, kind="LINCOMB", D=A)  # CPU tensors
    with pytest.raises(TypeError):
        ge.run(A.float(), A, A, kind="LINCOMB", D=A)
    with pytest.raises(ValueError):
        ge.run(A[:, :, :4], A, A, kind="LINCOMB", D=A)


def test_workload_draws_follow_the_pages():
    """Input recipes: P1-style integers in {-2..2}; the Python article's
    ceil(float16(uniform(-4, 4))) (values in {-4..4}, zeros are -0.0)."""
    import numpy as np
    a = workloads.draw("randint_pm2", 2025, 1, 64, 64, 64, False)
    for x in a:
        assert set(np.unique(x).tolist()) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
    c = workloads.draw("ceil_uniform_pm4", 1234, 1, 128, 128, 128, False)
    for x in c:
        v = set(np.unique(x).tolist())
        assert v <= {-4.0, -3.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0, 4.0}
        z = x[x == 0]
        assert z.size > 0 and np.all(np.signbit(z))
    # the first draws equal NumPy's RandomState(1234) stream cast then ceiled
    rs = np.random.RandomState(1234)
    first = np.ceil(rs.uniform(-4, 4, size=(1, 128, 128)).astype(np.float16))
    assert np.array_equal(first.view(np.uint16), c[0].view(np.uint16))


def test_c_program_builds_against_the_header(tmp_path):
    """The C ABI compiles from plain C (gcc, C11, -Wall -Wextra) and links
    against libgemm_epi.so: tests/c_abi/c_abi_check.c."""
    import subprocess
    import sys
    sys.path.insert(0, ROOT)
    from tests.c_abi import build as c_abi_build
    out = str(tmp_path / "c_abi_check")
    r = subprocess.run(c_abi_build.command(out), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "warning" not in r.stderr, r.stderr


def test_status_errors_are_value_errors_with_the_status_string():
    """A nonzero status surfaces from the Python wrapper as a ValueError
    carrying the library's status string (the wrapper the boundary
    specifies; the tutorial's failing calls raise)."""
    assert issubclass(ge.GemmEpiError, ValueError)
    e = ge.GemmEpiError(7, ge.gemm_epi_status_string(7))
    assert isinstance(e, ValueError) and e.status == 7
    assert "GEMM_EPI_ERR_WORKSPACE" in str(e) and ge.gemm_epi_status_string(7) in str(e)


def test_prepared_call_checks_its_entry_point_and_arguments():
    """prepared() converts the arguments once; it accepts only the run entry
    points and their exact argument count (no call is made here)."""
    args = (1, 64, 64, 64, P16, P16, P16, None, None, None, (1.0, 0.5, 2.0), "AUX_SCALE", P16, P16, None, None)
    call = ge.prepared("gemm_epi_run_ext", *args)
    assert callable(call)
    typed = ge.prepared("gemm_epi_run_typed", *args[:-1], "bf16", None)
    assert callable(typed)
    with pytest.raises(ValueError):
        ge.prepared("gemm_epi_plan_ext", *args)
    with pytest.raises(ValueError):
        ge.prepared("no_such_entry", *args)
    with pytest.raises(ValueError):
        ge.prepared("gemm_epi_run_ext", *args[:-1])


def test_plan_ws_stages_operands_that_miss_the_layout_rules():
    """A shape or pointer off the fast path's 16-byte rule gets the fast kernel
    on staged copies: the plan reports that kernel's tile (vec 1) and the
    workspace of the zero-padded copies, each in 256-byte granules after the
    16 KiB stream-K counter block, which staging leaves alone."""
    r256 = lambda n: (n + 255) // 256 * 256

    def ws(L, M, N, K, kind, a=P16, b=P16, c=P16, d=P16, aux=None, acc=None, rb=None, cb=None):
        rc, cfg = ge.gemm_epi_plan_ws(L, M, N, K, a, b, c, None, rb, cb, kind, d, aux, acc)
        assert rc == 0
        return cfg

    sq = 4096 * 4096 * 2
    cfg = ws(1, 4096, 4096, 4095, "LINCOMB")  # K % 8 != 0: A alone (M x K8); B keeps its K rows
    assert (cfg["bm"], cfg["bn"], cfg["bk"], cfg["vec"]) == (256, 256, 32, 1)
    assert cfg["workspace_bytes"] == 16384 + sq
    cfg = ws(1, 4096, 4095, 4095, "LINCOMB")  # both: A (M x K8), B (K x N8), C and D (M x N8)
    assert cfg["workspace_bytes"] == 16384 + sq + r256(4095 * 4096 * 2) + 2 * sq
    cfg = ws(1, 4096, 4095, 4096, "LINCOMB")  # N % 8 != 0: B, C and D with rows of N8
    assert cfg["vec"] == 1 and cfg["workspace_bytes"] == 16384 + 3 * sq
    cfg = ws(1, 64, 64, 64, "LINCOMB", a=P16 + 2)  # only A misaligned
    assert cfg["vec"] == 1 and cfg["workspace_bytes"] == 16384 + 64 * 64 * 2
    cfg = ws(1, 64, 64, 64, "LINCOMB", c=P16 + 6, d=P16 + 2)  # only C and D
    assert cfg["workspace_bytes"] == 16384 + 2 * 64 * 64 * 2
    # N = 99 -> 104: B, C, D, Aux (F) and the fp32 accumulator
    cfg = ws(1, 100, 99, 64, "RELU_SCALE_ACC", aux=P16, acc=P16)
    assert cfg["workspace_bytes"] == 16384 + r256(64 * 104 * 2) + 3 * r256(100 * 104 * 2) + r256(100 * 104 * 4)
    # N = 60 -> 64: B, the row bias and D (no C); the column bias needs no copy
    cfg = ws(1, 64, 60, 64, "BIAS_ROW_COL", c=None, rb=P16, cb=P16 + 2)
    assert cfg["workspace_bytes"] == 16384 + 64 * 64 * 2 + 256 + 64 * 64 * 2
    # aligned shapes and pointers stage nothing
    assert ws(1, 1024, 1024, 1024, "LINCOMB")["workspace_bytes"] == 0
    # a staged A of 2 GiB or more breaks the fast path's 32-bit offsets: the general kernel, no workspace
    cfg = ws(1, 1 << 21, 1000, 1001, "LINCOMB")
    assert cfg["vec"] == 0 and cfg["workspace_bytes"] == 0


def test_plan_ws_splits_a_staged_deep_k_product():
    """A few tiles with a long, ragged K: the staged operands also get the
    stream-K split.  The workspace is the counter block, then the split's
    partial sums, then the staging regions."""
    rc, cfg = ge.gemm_epi_plan_ws(1, 256, 256, 65535, P16, P16, P16, None, None, None, "LINCOMB", P16, None, None)
    assert rc == 0 and (cfg["bm"], cfg["bn"], cfg["vec"]) == (128, 128, 1)
    groups = cfg["workgroups"]
    assert 1 < groups <= 256
    # A (256 x 65536) is the only staged tensor: N = 256 is a multiple of 8 and B keeps its K rows
    assert cfg["workspace_bytes"] == 16384 + 2 * groups * 128 * 128 * 4 + 256 * 65536 * 2
    # the same product with K a multiple of 8 splits the same way, with no staging
    rc, al = ge.gemm_epi_plan_ws(1, 256, 256, 65536, P16, P16, P16, None, None, None, "LINCOMB", P16, None, None)
    assert al["workgroups"] == groups and al["workspace_bytes"] == 16384 + 2 * groups * 128 * 128 * 4


def test_general_kernel_tile_follows_the_grid():
    """Off the 16-byte rule and without a workspace: the general kernel's
    128 x 128 tile on small grids, its 256 x 128 tile where the grid fills the
    chip several times (same cost model as the fast path)."""
    def plan(L, M, N, K):
        rc, cfg = ge.gemm_epi_plan(L, M, N, K, P16, P16, P16, None, "LINCOMB", P16, None)
        assert rc == 0 and cfg["vec"] == 0
        return (cfg["bm"], cfg["bn"], cfg["bk"], cfg["threads"])
    assert plan(1, 1001, 1001, 1001) == (128, 128, 64, 512)
    assert plan(1, 3000, 3000, 1001) == (128, 128, 64, 512)
    assert plan(1, 2100, 2100, 61) == (256, 128, 64, 512)
    assert plan(1, 4096, 4096, 4095) == (256, 128, 64, 512)
