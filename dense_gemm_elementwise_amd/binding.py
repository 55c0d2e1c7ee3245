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
}
HAS_AUX = ("AUX_SCALE", "LINCOMB_X_ACC", "SQUARE", "RELU_SQUARE")
READS_X = ("LINCOMB_X_ACC",)

STATUS = {
    0: "GEMM_EPI_OK",
    1: "GEMM_EPI_ERR_SHAPE",
    2: "GEMM_EPI_ERR_NULL_INPUT",
    3: "GEMM_EPI_ERR_NULL_OUTPUT",
    4: "GEMM_EPI_ERR_KIND",
    5: "GEMM_EPI_ERR_ALIGN",
    6: "GEMM_EPI_ERR_HIP",
}

# every function include/gemm_epi.h declares
EXPORTS = ("gemm_epi_run", "gemm_epi_status_string", "gemm_epi_last_hip_error", "gemm_epi_plan")


class GemmEpiError(RuntimeError):
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
    L.gemm_epi_status_string.restype = ctypes.c_char_p
    L.gemm_epi_status_string.argtypes = [ctypes.c_int]
    L.gemm_epi_last_hip_error.restype = ctypes.c_int
    L.gemm_epi_last_hip_error.argtypes = []
    L.gemm_epi_plan.restype = ctypes.c_int
    L.gemm_epi_plan.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.POINTER(i64)]
    _lib = L
    return L


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


def gemm_epi_plan(L, M, N, K, A, B, C, X, epilogue_kind, D, Aux):
    """Host-only query of the launch configuration.  Returns (status, dict)."""
    out = (ctypes.c_int64 * 6)()
    rc = lib().gemm_epi_plan(int(L), int(M), int(N), int(K), A, B, C, X, _kind_id(epilogue_kind), D, Aux, out)
    keys = ("bm", "bn", "bk", "vec", "workgroups", "threads")
    return rc, dict(zip(keys, list(out)))


def _check_tensor(name, t, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float16:
        raise TypeError(f"{name} must be float16, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (packed row-major)")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def run(A, B, C, X=None, *, kind, alpha=1.0, beta=0.0, s3=0.0, D, Aux=None, stream=None, sync=True):
    """D (and Aux) <- fused epilogue of A @ B on torch tensors.

    A (L,M,K), B (L,K,N), C, X, D, Aux (L,M,N): contiguous float16 CUDA
    tensors.  s3 is extra_scalar (AUX_SCALE) or x_factor (LINCOMB_X_ACC).
    The kernel is queued on `stream` (a torch.cuda.Stream; default: the
    current stream); with sync=True the call waits for it.
    """
    import torch
    if A.dim() != 3 or B.dim() != 3:
        raise ValueError("A and B must be 3-D: (L,M,K) and (L,K,N)")
    L, M, K = A.shape
    N = B.shape[2]
    _check_tensor("A", A, (L, M, K))
    _check_tensor("B", B, (L, K, N))
    _check_tensor("C", C, (L, M, N))
    _check_tensor("D", D, (L, M, N))
    kname = kind if isinstance(kind, str) else {v: k for k, v in KINDS.items()}[int(kind)]
    if kname in READS_X:
        if X is None:
            raise ValueError(f"{kname} reads X")
        _check_tensor("X", X, (L, M, N))
    if kname in HAS_AUX:
        if Aux is None:
            raise ValueError(f"{kname} writes a second output: pass Aux")
        _check_tensor("Aux", Aux, (L, M, N))
    devs = {t.device for t in (A, B, C, D, X, Aux) if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {devs}")
    dev = A.device
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        rc = gemm_epi_run(L, M, N, K, A.data_ptr(), B.data_ptr(), C.data_ptr(),
                          X.data_ptr() if X is not None else None, (alpha, beta, s3), KINDS[kname], D.data_ptr(),
                          Aux.data_ptr() if Aux is not None else None, s.cuda_stream)
    if rc != 0:
        msg = gemm_epi_status_string(rc)
        if rc == 6:
            msg += f" (hipError_t {gemm_epi_last_hip_error()})"
        raise GemmEpiError(rc, msg)
    if sync:
        s.synchronize()
    return D, Aux
