"""Thin ctypes binding of libgemm_epi.so.

Only argument marshalling lives here: every step of the GEMM and its epilogue
runs in the HIP kernels behind gemm_epi_run.  The functions keep the C names
and argument order of include/gemm_epi.h; run() is the torch-tensor
convenience wrapper (PyTorch provides device memory and streams only).
There is no fallback: if the library is missing or cannot load, every call
raises.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgemm_epi.so")

KINDS = {
    "LINCOMB": 0,
    "AUX_SCALE": 1,
    "LINCOMB_X_ACC": 2,
    "RELU": 3,
    "SQUARE": 4,
    "RELU_SQUARE": 5,
    "RELU_AUX_STORE": 6,
    "RELU_SCALE_ACC": 7,
    "BIAS_ROW_COL": 8,
    "SIGMOID": 9,
    "TANH": 10,
    "GELU": 11,
    "SILU": 12,
    "LEAKY_RELU": 13,
    "HARDSWISH": 14,
}
ACTIVATIONS = ("SIGMOID", "TANH", "GELU", "SILU", "LEAKY_RELU", "HARDSWISH")
HAS_AUX = ("AUX_SCALE", "LINCOMB_X_ACC", "SQUARE", "RELU_SQUARE", "RELU_AUX_STORE", "RELU_SCALE_ACC")
READS_X = ("LINCOMB_X_ACC",)
READS_C = tuple(k for k in KINDS if k != "BIAS_ROW_COL")
READS_BIAS = ("BIAS_ROW_COL",)
HAS_ACC = ("RELU_SCALE_ACC",)

STATUS = {
    0: "GEMM_EPI_OK",
    1: "GEMM_EPI_ERR_SHAPE",
    2: "GEMM_EPI_ERR_NULL_INPUT",
    3: "GEMM_EPI_ERR_NULL_OUTPUT",
    4: "GEMM_EPI_ERR_KIND",
    5: "GEMM_EPI_ERR_ALIGN",
    6: "GEMM_EPI_ERR_HIP",
    7: "GEMM_EPI_ERR_WORKSPACE",
    8: "GEMM_EPI_ERR_DTYPE",
}
# element types of the 16-bit tensors (gemm_epi_run_typed)
DTYPES = {"f16": 0, "bf16": 1, "f32": 2}

# every function include/gemm_epi.h declares
EXPORTS = ("gemm_epi_run", "gemm_epi_run_ext", "gemm_epi_run_typed", "gemm_epi_run_mixed", "gemm_epi_run_ws",
           "gemm_epi_run_unfused", "gemm_epi_run_ws_typed", "gemm_epi_run_unfused_typed", "gemm_epi_status_string",
           "gemm_epi_last_hip_error", "gemm_epi_plan", "gemm_epi_plan_ext", "gemm_epi_plan_ws",
           "gemm_epi_run_ws_static")


class GemmEpiError(ValueError):
    """A nonzero status of the C ABI, with its status string."""
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded libgemm_epi.so.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; "
                           "g.build()' or python -m dense_gemm_elementwise_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    L.gemm_epi_run.restype = ctypes.c_int
    L.gemm_epi_run.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_float), ctypes.c_int,
                               vp, vp, vp]
    L.gemm_epi_run_ext.restype = ctypes.c_int
    L.gemm_epi_run_ext.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_float),
                                   ctypes.c_int, vp, vp, vp, vp]
    L.gemm_epi_run_typed.restype = ctypes.c_int
    L.gemm_epi_run_typed.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_float),
                                     ctypes.c_int, vp, vp, vp, ctypes.c_int, vp]
    L.gemm_epi_run_mixed.restype = ctypes.c_int
    L.gemm_epi_run_mixed.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_float),
                                     ctypes.c_int, vp, vp, vp, ctypes.c_int, ctypes.c_int, vp]
    L.gemm_epi_run_unfused.restype = ctypes.c_int
    L.gemm_epi_run_unfused.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_float),
                                       ctypes.c_int, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.gemm_epi_run_ws.restype = ctypes.c_int
    L.gemm_epi_run_ws.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_float),
                                  ctypes.c_int, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.gemm_epi_run_unfused_typed.restype = ctypes.c_int
    L.gemm_epi_run_unfused_typed.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                             ctypes.POINTER(ctypes.c_float), ctypes.c_int, vp, vp, vp, vp,
                                             ctypes.c_size_t, ctypes.c_int, vp]
    L.gemm_epi_run_ws_typed.restype = ctypes.c_int
    L.gemm_epi_run_ws_typed.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_float),
                                        ctypes.c_int, vp, vp, vp, vp, ctypes.c_size_t, ctypes.c_int, vp]
    L.gemm_epi_run_ws_static.restype = ctypes.c_int
    L.gemm_epi_run_ws_static.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_float),
                                         ctypes.c_int, vp, vp, vp, ctypes.c_int, vp]
    L.gemm_epi_plan_ws.restype = ctypes.c_int
    L.gemm_epi_plan_ws.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                                   ctypes.POINTER(i64)]
    L.gemm_epi_status_string.restype = ctypes.c_char_p
    L.gemm_epi_status_string.argtypes = [ctypes.c_int]
    L.gemm_epi_last_hip_error.restype = ctypes.c_int
    L.gemm_epi_last_hip_error.argtypes = []
    L.gemm_epi_plan.restype = ctypes.c_int
    L.gemm_epi_plan.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.POINTER(i64)]
    L.gemm_epi_plan_ext.restype = ctypes.c_int
    L.gemm_epi_plan_ext.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                                    ctypes.POINTER(i64)]
    _lib = L
    return L


def _dtype_id(dtype):
    return DTYPES[dtype] if isinstance(dtype, str) else int(dtype)


def _kind_id(kind):
    if isinstance(kind, str):
        return KINDS[kind]
    return int(kind)


def gemm_epi_status_string(status: int) -> str:
    return lib().gemm_epi_status_string(int(status)).decode()


def gemm_epi_last_hip_error() -> int:
    return lib().gemm_epi_last_hip_error()


def gemm_epi_run(L, M, N, K, A, B, C, X, scalars, epilogue_kind, D, Aux, stream) -> int:
    """Pointer-level call, same arguments as the C function.  A, B, C, X, D,
    Aux and stream are integers (device addresses / hipStream_t) or None;
    scalars is a sequence of 3 floats.  Returns the status code."""
    sc = (ctypes.c_float * 3)(*[float(v) for v in scalars]) if scalars is not None else None
    return lib().gemm_epi_run(int(L), int(M), int(N), int(K), A, B, C, X, sc, _kind_id(epilogue_kind), D, Aux,
                              stream)


def gemm_epi_run_ext(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux, acc_out,
                     stream) -> int:
    """Pointer-level call of gemm_epi_run_ext (adds the row / column bias
    inputs and the fp32 accumulator output).  Returns the status code."""
    sc = (ctypes.c_float * 3)(*[float(v) for v in scalars]) if scalars is not None else None
    return lib().gemm_epi_run_ext(int(L), int(M), int(N), int(K), A, B, C, X, row_bias, col_bias, sc,
                                  _kind_id(epilogue_kind), D, Aux, acc_out, stream)


def prepared(entry, *args):
    """A call of C-ABI entry point `entry` (a name from EXPORTS) that repeats
    with the same arguments, converted to ctypes once: for loops that issue
    the same call many times (timing, serving).  Arguments as for the
    pointer-level wrapper of that entry point: sizes, device addresses (int or
    None), the scalars as a sequence, the kind and element types as names or
    enum values, the stream as an address.  Returns a function of no
    arguments that makes the call and returns its status code."""
    if entry not in EXPORTS or not entry.startswith("gemm_epi_run"):
        raise ValueError(f"not a run entry point: {entry}")
    f = getattr(lib(), entry)
    if len(args) != len(f.argtypes):
        raise ValueError(f"{entry} takes {len(f.argtypes)} arguments, got {len(args)}")
    conv = []
    ints = 0  # the first int argument of a run entry point is the kind, any later ones element types
    for t, a in zip(f.argtypes, args):
        if a is None:
            conv.append(None)
        elif t is ctypes.POINTER(ctypes.c_float):
            conv.append((ctypes.c_float * len(a))(*[float(v) for v in a]))
        elif t is ctypes.c_int:
            conv.append(t(_kind_id(a) if ints == 0 else _dtype_id(a)))
            ints += 1
        else:
            conv.append(t(a))
    return lambda: f(*conv)


def gemm_epi_run_typed(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux, acc_out,
                       dtype, stream) -> int:
    """Pointer-level call of gemm_epi_run_typed: gemm_epi_run_ext with the
    element type of the 16-bit tensors ("f16" / "bf16" or the enum value)."""
    sc = (ctypes.c_float * 3)(*[float(v) for v in scalars]) if scalars is not None else None
    return lib().gemm_epi_run_typed(int(L), int(M), int(N), int(K), A, B, C, X, row_bias, col_bias, sc,
                                    _kind_id(epilogue_kind), D, Aux, acc_out, _dtype_id(dtype), stream)


def gemm_epi_run_mixed(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux, acc_out,
                       ab_dtype, epi_dtype, stream) -> int:
    """Pointer-level call of gemm_epi_run_mixed: the element type of A and B
    ("f16" / "bf16") and that of the epilogue tensors ("f32", or the same as
    A and B) given separately."""
    sc = (ctypes.c_float * 3)(*[float(v) for v in scalars]) if scalars is not None else None
    return lib().gemm_epi_run_mixed(int(L), int(M), int(N), int(K), A, B, C, X, row_bias, col_bias, sc,
                                    _kind_id(epilogue_kind), D, Aux, acc_out, _dtype_id(ab_dtype),
                                    _dtype_id(epi_dtype), stream)


def gemm_epi_run_unfused(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux, acc_out,
                         workspace, workspace_bytes, stream) -> int:
    """Pointer-level call of gemm_epi_run_unfused: the same operation in two
    launches (GEMM to an fp32 workspace, then the elementwise epilogue).
    Returns the status code."""
    sc = (ctypes.c_float * 3)(*[float(v) for v in scalars]) if scalars is not None else None
    return lib().gemm_epi_run_unfused(int(L), int(M), int(N), int(K), A, B, C, X, row_bias, col_bias, sc,
                                      _kind_id(epilogue_kind), D, Aux, acc_out, workspace, int(workspace_bytes),
                                      stream)


def gemm_epi_run_ws(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux, acc_out,
                    workspace, workspace_bytes, stream) -> int:
    """Pointer-level call of gemm_epi_run_ws (may split K across workgroups,
    stream-K, using the caller's zero-initialised workspace)."""
    sc = (ctypes.c_float * 3)(*[float(v) for v in scalars]) if scalars is not None else None
    return lib().gemm_epi_run_ws(int(L), int(M), int(N), int(K), A, B, C, X, row_bias, col_bias, sc,
                                 _kind_id(epilogue_kind), D, Aux, acc_out, workspace, int(workspace_bytes), stream)


def gemm_epi_run_unfused_typed(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux,
                               acc_out, workspace, workspace_bytes, dtype, stream) -> int:
    """Pointer-level call of gemm_epi_run_unfused_typed: gemm_epi_run_unfused
    with the element type of the 16-bit tensors ("f16" / "bf16" or the enum
    value)."""
    sc = (ctypes.c_float * 3)(*[float(v) for v in scalars]) if scalars is not None else None
    return lib().gemm_epi_run_unfused_typed(int(L), int(M), int(N), int(K), A, B, C, X, row_bias, col_bias, sc,
                                            _kind_id(epilogue_kind), D, Aux, acc_out, workspace,
                                            int(workspace_bytes), _dtype_id(dtype), stream)


def gemm_epi_run_ws_typed(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux, acc_out,
                          workspace, workspace_bytes, dtype, stream) -> int:
    """Pointer-level call of gemm_epi_run_ws_typed: gemm_epi_run_ws with the
    element type of the 16-bit tensors ("f16" / "bf16" or the enum value)."""
    sc = (ctypes.c_float * 3)(*[float(v) for v in scalars]) if scalars is not None else None
    return lib().gemm_epi_run_ws_typed(int(L), int(M), int(N), int(K), A, B, C, X, row_bias, col_bias, sc,
                                       _kind_id(epilogue_kind), D, Aux, acc_out, workspace, int(workspace_bytes),
                                       _dtype_id(dtype), stream)


def gemm_epi_run_ws_static(L, M, N, K, A, B, C, X, row_bias, col_bias, scalars, epilogue_kind, D, Aux, acc_out,
                           dtype, stream) -> int:
    """Pointer-level call of gemm_epi_run_ws_static: gemm_epi_run_ws_typed
    with its split's scratch in the library's per-device static array (no
    workspace argument; allocates nothing)."""
    sc = (ctypes.c_float * 3)(*[float(v) for v in scalars]) if scalars is not None else None
    return lib().gemm_epi_run_ws_static(int(L), int(M), int(N), int(K), A, B, C, X, row_bias, col_bias, sc,
                                        _kind_id(epilogue_kind), D, Aux, acc_out, _dtype_id(dtype), stream)


def gemm_epi_plan_ws(L, M, N, K, A, B, C, X, row_bias, col_bias, epilogue_kind, D, Aux, acc_out):
    """Host-only plan of gemm_epi_run_ws: (status, dict) with the keys of
    gemm_epi_plan plus workspace_bytes (0: no split and no staging)."""
    out = (ctypes.c_int64 * 7)()
    rc = lib().gemm_epi_plan_ws(int(L), int(M), int(N), int(K), A, B, C, X, row_bias, col_bias,
                                _kind_id(epilogue_kind), D, Aux, acc_out, out)
    keys = ("bm", "bn", "bk", "vec", "workgroups", "threads", "workspace_bytes")
    return rc, dict(zip(keys, list(out)))


def gemm_epi_plan_ext(L, M, N, K, A, B, C, X, row_bias, col_bias, epilogue_kind, D, Aux, acc_out):
    """Host-only query of the launch configuration for gemm_epi_run_ext."""
    out = (ctypes.c_int64 * 6)()
    rc = lib().gemm_epi_plan_ext(int(L), int(M), int(N), int(K), A, B, C, X, row_bias, col_bias,
                                 _kind_id(epilogue_kind), D, Aux, acc_out, out)
    keys = ("bm", "bn", "bk", "vec", "workgroups", "threads")
    return rc, dict(zip(keys, list(out)))


def gemm_epi_plan(L, M, N, K, A, B, C, X, epilogue_kind, D, Aux):
    """Host-only query of the launch configuration.  Returns (status, dict)."""
    out = (ctypes.c_int64 * 6)()
    rc = lib().gemm_epi_plan(int(L), int(M), int(N), int(K), A, B, C, X, _kind_id(epilogue_kind), D, Aux, out)
    keys = ("bm", "bn", "bk", "vec", "workgroups", "threads")
    return rc, dict(zip(keys, list(out)))


def _check_tensor(name, t, shape, dtype=None):
    import torch
    dtype = dtype or torch.float16
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (packed row-major)")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _ptr(t):
    return t.data_ptr() if t is not None else None


def run(A, B, C=None, X=None, *, kind, alpha=1.0, beta=0.0, s3=0.0, D, Aux=None, row_bias=None, col_bias=None,
        acc_out=None, stream=None, sync=True, unfused_workspace=None, workspace=None, stream_k_workspace=None):
    """D (and Aux, acc_out) <- fused epilogue of A @ B on torch tensors.

    A (L,M,K), B (L,K,N), C, X, D, Aux (L,M,N): contiguous float16 CUDA
    tensors, or all bfloat16 (then the bfloat16 kernels run; every
    composition below takes either type); or A, B float16 / bfloat16 with
    C, X, D, Aux and the biases all float32 or all of the other 16-bit type
    (gemm_epi_run_mixed, fused call only; D's dtype selects it); row_bias (N,) and col_bias (M,) or (M, 1) of the
    same type for BIAS_ROW_COL; acc_out (L,M,N) float32 for RELU_SCALE_ACC.  s3 is
    extra_scalar (AUX_SCALE), x_factor (LINCOMB_X_ACC) or scale
    (RELU_SCALE_ACC).  The kernel is queued on `stream` (a torch.cuda.Stream;
    default: the current stream); with sync=True the call waits for it.
    With unfused_workspace (a float32 CUDA tensor of at least L*M*N
    elements) the unfused two-launch composition runs instead of the fused
    kernel (for comparison; the outputs are the same).  With workspace (a
    zero-initialised CUDA tensor of at least the workspace_bytes
    gemm_epi_plan_ws reports; stream_k_workspace is the same argument under
    its older name) the call goes through gemm_epi_run_ws: it may split K
    across workgroups, and operands that miss the fast kernel's layout rules
    (K or N not a multiple of 8, a tensor not 16-byte aligned) are staged
    through the workspace so that the fast kernel runs.
    """
    import torch
    if A.dim() != 3 or B.dim() != 3:
        raise ValueError("A and B must be 3-D: (L,M,K) and (L,K,N)")
    L, M, K = A.shape
    N = B.shape[2]
    at = torch.bfloat16 if isinstance(A, torch.Tensor) and A.dtype == torch.bfloat16 else torch.float16
    # the epilogue tensors (C, X, biases, D, Aux) share D's type: A's, the other 16-bit type, or float32
    et = D.dtype if isinstance(D, torch.Tensor) and D.dtype in (torch.float16, torch.bfloat16, torch.float32) else at
    _check_tensor("A", A, (L, M, K), at)
    _check_tensor("B", B, (L, K, N), at)
    _check_tensor("D", D, (L, M, N), et)
    kname = kind if isinstance(kind, str) else {v: k for k, v in KINDS.items()}[int(kind)]
    if kname in READS_C:
        if C is None:
            raise ValueError(f"{kname} reads C")
        _check_tensor("C", C, (L, M, N), et)
    if kname in READS_X:
        if X is None:
            raise ValueError(f"{kname} reads X")
        _check_tensor("X", X, (L, M, N), et)
    if kname in READS_BIAS:
        if row_bias is None or col_bias is None:
            raise ValueError(f"{kname} reads row_bias (N,) and col_bias (M,)")
        _check_tensor("row_bias", row_bias.reshape(-1) if row_bias.dim() == 2 else row_bias, (N,), et)
        _check_tensor("col_bias", col_bias.reshape(-1) if col_bias.dim() == 2 else col_bias, (M,), et)
    if kname in HAS_AUX:
        if Aux is None:
            raise ValueError(f"{kname} writes a second output: pass Aux")
        _check_tensor("Aux", Aux, (L, M, N), et)
    if kname in HAS_ACC:
        if acc_out is None:
            raise ValueError(f"{kname} writes the fp32 accumulator: pass acc_out")
        _check_tensor("acc_out", acc_out, (L, M, N), torch.float32)
    used = [t for t in (A, B, C, D, X, Aux, row_bias, col_bias, acc_out) if t is not None]
    devs = {t.device for t in used}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {devs}")
    dev = A.device
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    ws = unfused_workspace
    if ws is not None and (ws.dtype != torch.float32 or ws.device != dev or not ws.is_contiguous()):
        raise ValueError("unfused_workspace must be a contiguous float32 tensor on the operands' device")
    if workspace is not None and stream_k_workspace is not None:
        raise ValueError("pass workspace or stream_k_workspace (the same argument), not both")
    skw = workspace if workspace is not None else stream_k_workspace
    if skw is not None and (skw.device != dev or not skw.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the operands' device")
    dt = DTYPES["bf16"] if at == torch.bfloat16 else DTYPES["f16"]
    if et != at and (ws is not None or skw is not None):
        raise ValueError("the unfused composition and the workspace call take epilogue tensors of A's type only")
    ops = (L, M, N, K, A.data_ptr(), B.data_ptr(), _ptr(C), _ptr(X), _ptr(row_bias), _ptr(col_bias),
           (alpha, beta, s3), KINDS[kname], D.data_ptr(), _ptr(Aux), _ptr(acc_out))
    with torch.cuda.device(dev):
        if skw is not None:
            rc = gemm_epi_run_ws_typed(*ops, skw.data_ptr(), skw.numel() * skw.element_size(), dt, s.cuda_stream)
        elif ws is not None:
            rc = gemm_epi_run_unfused_typed(*ops, ws.data_ptr(), ws.numel() * 4, dt, s.cuda_stream)
        elif et != at:
            edt = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[et]
            rc = gemm_epi_run_mixed(*ops, dt, DTYPES[edt], s.cuda_stream)
        else:
            rc = gemm_epi_run_typed(*ops, dt, s.cuda_stream)
    if rc != 0:
        msg = gemm_epi_status_string(rc)
        if rc == 6:
            msg += f" (hipError_t {gemm_epi_last_hip_error()})"
        raise GemmEpiError(rc, msg)
    if sync:
        s.synchronize()
    return D, Aux
