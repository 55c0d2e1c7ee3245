"""CPU oracle for the fused fp16 GEMM + elementwise epilogue.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg are the only callers.  The product path (the HIP library and
its binding in dense_gemm_elementwise_amd/) never imports this package, and
this package imports nothing from it.

This module only marshals numpy arrays into liboracle.so (oracle.c), where
the arithmetic lives: exact fp16 decode, an fp64 i-k-j triple loop, the
epilogue in fp64 from the unrounded accumulator, and one round-to-nearest-even
encode per output.  See oracle.c for the definition and its citations.
"""
import ctypes
import os

import numpy as np

from . import build as _build

# The boundary's public epilogue enum, written out here on purpose (the
# oracle shares no header with the HIP library).
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
# element types of the 16-bit tensors, the boundary's enum values
DTYPES = {"f16": 0, "bf16": 1}
HAS_AUX = {"AUX_SCALE", "LINCOMB_X_ACC", "SQUARE", "RELU_SQUARE", "RELU_AUX_STORE", "RELU_SCALE_ACC"}
READS_X = {"LINCOMB_X_ACC"}
READS_C = set(KINDS) - {"BIAS_ROW_COL"}
READS_BIAS = {"BIAS_ROW_COL"}
HAS_ACC = {"RELU_SCALE_ACC"}

_lib = None


def lib():
    """Loads liboracle.so, building it first if it is not there yet."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    L = ctypes.CDLL(_build.LIB)
    i64, u16p, f64p, f32p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    L.oracle_f16_decode.restype = ctypes.c_double
    L.oracle_f16_decode.argtypes = [ctypes.c_uint16]
    L.oracle_f16_encode.restype = ctypes.c_uint16
    L.oracle_f16_encode.argtypes = [ctypes.c_double]
    L.oracle_gemm_epi.restype = ctypes.c_int
    L.oracle_gemm_epi.argtypes = [i64, i64, i64, i64, u16p, u16p, u16p, u16p, f32p, ctypes.c_int,
                                  u16p, u16p, f64p, f64p]
    L.oracle_gemm_epi_ext.restype = ctypes.c_int
    L.oracle_gemm_epi_ext.argtypes = [i64, i64, i64, i64, u16p, u16p, u16p, u16p, u16p, u16p, f32p, ctypes.c_int,
                                      u16p, u16p, f32p, f64p, f64p, f64p]
    L.oracle_gemm_epi_typed.restype = ctypes.c_int
    L.oracle_gemm_epi_typed.argtypes = [i64, i64, i64, i64, u16p, u16p, u16p, u16p, u16p, u16p, f32p, ctypes.c_int,
                                        u16p, u16p, f32p, f64p, f64p, f64p, ctypes.c_int]
    L.oracle_gemm_epi_typed2.restype = ctypes.c_int
    L.oracle_gemm_epi_typed2.argtypes = [i64, i64, i64, i64, u16p, u16p, u16p, u16p, u16p, u16p, f32p, ctypes.c_int,
                                         u16p, u16p, f32p, f64p, f64p, f64p, ctypes.c_int, ctypes.c_int]
    L.oracle_gemm_epi_f32e.restype = ctypes.c_int
    L.oracle_gemm_epi_f32e.argtypes = [i64, i64, i64, i64, u16p, u16p, f32p, f32p, f32p, f32p, f32p, ctypes.c_int,
                                       f32p, f32p, f32p, f64p, f64p, f64p, ctypes.c_int]
    L.oracle_gemm_epi_points_typed.restype = ctypes.c_int
    L.oracle_gemm_epi_points_typed.argtypes = [i64, i64, i64, i64, u16p, u16p, u16p, u16p, u16p, u16p, f32p,
                                               ctypes.c_int, i64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                               u16p, u16p, f32p, f64p, f64p, f64p, ctypes.c_int]
    L.oracle_bf16_decode.restype = ctypes.c_double
    L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
    L.oracle_bf16_encode.restype = ctypes.c_uint16
    L.oracle_bf16_encode.argtypes = [ctypes.c_double]
    L.oracle_bf16_decode_n.restype = None
    L.oracle_bf16_decode_n.argtypes = [u16p, f64p, i64]
    L.oracle_bf16_encode_n.restype = None
    L.oracle_bf16_encode_n.argtypes = [f64p, u16p, i64]
    L.oracle_gemm_epi_points_ext.restype = ctypes.c_int
    L.oracle_gemm_epi_points_ext.argtypes = [i64, i64, i64, i64, u16p, u16p, u16p, u16p, u16p, u16p, f32p,
                                             ctypes.c_int, i64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             u16p, u16p, f32p, f64p, f64p, f64p]
    L.oracle_gemm_epi_points.restype = ctypes.c_int
    L.oracle_gemm_epi_points.argtypes = [i64, i64, i64, i64, u16p, u16p, u16p, u16p, f32p, ctypes.c_int,
                                         i64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         u16p, u16p, f64p, f64p]
    L.oracle_f16_decode_n.restype = None
    L.oracle_f16_decode_n.argtypes = [u16p, f64p, i64]
    L.oracle_f16_encode_n.restype = None
    L.oracle_f16_encode_n.argtypes = [f64p, u16p, i64]
    L.oracle_rounding_mode_is_nearest.restype = ctypes.c_int
    L.oracle_kind_has_aux.restype = ctypes.c_int
    L.oracle_kind_reads_x.restype = ctypes.c_int
    L.oracle_kind_reads_c.restype = ctypes.c_int
    L.oracle_kind_reads_bias.restype = ctypes.c_int
    L.oracle_kind_has_acc_out.restype = ctypes.c_int
    _lib = L
    return L


def _bits(a, dtype="f16"):
    """A float16 (or uint16 bit-pattern) array as a C-contiguous uint16 array.
    bfloat16 tensors are passed as uint16 bit patterns (numpy has no such
    type)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16 and dtype == "f16":
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected {'float16 or ' if dtype == 'f16' else ''}uint16 bits, got {a.dtype}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def f16_decode(bits):
    b = _bits(np.asarray(bits))
    out = np.empty(b.shape, np.float64)
    lib().oracle_f16_decode_n(_ptr(b), _ptr(out), b.size)
    return out


def f16_encode(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f16_encode_n(_ptr(x), _ptr(out), x.size)
    return out


def bf16_decode(bits):
    b = _bits(np.asarray(bits), "bf16")
    out = np.empty(b.shape, np.float64)
    lib().oracle_bf16_decode_n(_ptr(b), _ptr(out), b.size)
    return out


def bf16_encode(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_bf16_encode_n(_ptr(x), _ptr(out), x.size)
    return out


def _shapes(A, B, C):
    if A.ndim != 3 or B.ndim != 3 or (C is not None and C.ndim != 3):
        raise ValueError("A, B, C must be (L,M,K), (L,K,N), (L,M,N)")
    L, M, K = A.shape
    if B.shape[0] != L or B.shape[1] != K or (C is not None and C.shape != (L, M, B.shape[2])):
        raise ValueError(f"shape mismatch A{A.shape} B{B.shape} C{None if C is None else C.shape}")
    return L, M, B.shape[2], K


def _biases(row_bias, col_bias, M, N, dtype="f16"):
    rb = _bits(np.asarray(row_bias).reshape(-1), dtype) if row_bias is not None else None
    cb = _bits(np.asarray(col_bias).reshape(-1), dtype) if col_bias is not None else None
    if rb is not None and rb.size != N:
        raise ValueError(f"row_bias must have N = {N} entries")
    if cb is not None and cb.size != M:
        raise ValueError(f"col_bias must have M = {M} entries")
    return rb, cb


def gemm_epi(A, B, C=None, X=None, *, kind, alpha=1.0, beta=0.0, s3=0.0, row_bias=None, col_bias=None,
             want64=False, dtype="f16", epi_dtype=None):
    """Full fused GEMM + epilogue on host arrays.

    A (L,M,K), B (L,K,N), C and X (L,M,N): float16 arrays (or uint16 bits);
    row_bias (N,) and col_bias (M,) or (M, 1) for BIAS_ROW_COL.  Returns a dict
    with D (and Aux for kinds with a second output) as float16 arrays, Acc
    (float32) for kinds that return the accumulator, plus D64 / Aux64 / Acc64
    (unrounded float64) when want64 is set.  dtype "bf16": the 16-bit tensors
    are bfloat16, passed and returned as uint16 bit patterns.  epi_dtype
    (default: dtype) gives C, X, the biases, D and Aux a 16-bit type of their
    own.
    """
    epi_dtype = epi_dtype or dtype
    A, B = _bits(A, dtype), _bits(B, dtype)
    C = _bits(C, epi_dtype) if C is not None else None
    X = _bits(X, epi_dtype) if X is not None else None
    L, M, N, K = _shapes(A, B, C)
    rb, cb = _biases(row_bias, col_bias, M, N, epi_dtype)
    sc = np.array([alpha, beta, s3], np.float32)
    D = np.empty((L, M, N), np.uint16)
    Aux = np.empty((L, M, N), np.uint16) if kind in HAS_AUX else None
    Acc = np.empty((L, M, N), np.float32) if kind in HAS_ACC else None
    D64 = np.empty((L, M, N), np.float64) if want64 else None
    Aux64 = np.empty((L, M, N), np.float64) if (want64 and kind in HAS_AUX) else None
    Acc64 = np.empty((L, M, N), np.float64) if want64 else None
    rc = lib().oracle_gemm_epi_typed2(L, M, N, K, _ptr(A), _ptr(B), _ptr(C), _ptr(X), _ptr(rb), _ptr(cb), _ptr(sc),
                                      KINDS[kind], _ptr(D), _ptr(Aux), _ptr(Acc), _ptr(D64), _ptr(Aux64),
                                      _ptr(Acc64), DTYPES[dtype], DTYPES[epi_dtype])
    if rc:
        raise ValueError(f"oracle_gemm_epi_typed2 rejected the call (code {rc})")
    view = (lambda a: a.view(np.float16)) if epi_dtype == "f16" else (lambda a: a)
    out = {"D": view(D)}
    if Aux is not None:
        out["Aux"] = view(Aux)
    if Acc is not None:
        out["Acc"] = Acc
    if want64:
        out["D64"] = D64
        out["Acc64"] = Acc64
        if Aux64 is not None:
            out["Aux64"] = Aux64
    return out


def gemm_epi_f32e(A, B, C=None, X=None, *, kind, alpha=1.0, beta=0.0, s3=0.0, row_bias=None, col_bias=None,
                  want64=False, ab_dtype="f16"):
    """gemm_epi with fp32 epilogue tensors: A, B 16-bit of type ab_dtype
    ("f16": float16 arrays or uint16 bits; "bf16": uint16 bits); C, X,
    row_bias, col_bias float32 arrays; D and Aux returned as float32 (one
    round-to-nearest-even from the unrounded double)."""
    A, B = _bits(A, ab_dtype), _bits(B, ab_dtype)
    f32 = (lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float32))
    C, X = f32(C), f32(X)
    L, M, N, K = _shapes(A, B, C)
    rb = f32(np.asarray(row_bias).reshape(-1)) if row_bias is not None else None
    cb = f32(np.asarray(col_bias).reshape(-1)) if col_bias is not None else None
    if rb is not None and rb.size != N:
        raise ValueError(f"row_bias must have N = {N} entries")
    if cb is not None and cb.size != M:
        raise ValueError(f"col_bias must have M = {M} entries")
    sc = np.array([alpha, beta, s3], np.float32)
    D = np.empty((L, M, N), np.float32)
    Aux = np.empty((L, M, N), np.float32) if kind in HAS_AUX else None
    Acc = np.empty((L, M, N), np.float32) if kind in HAS_ACC else None
    D64 = np.empty((L, M, N), np.float64) if want64 else None
    Aux64 = np.empty((L, M, N), np.float64) if (want64 and kind in HAS_AUX) else None
    Acc64 = np.empty((L, M, N), np.float64) if want64 else None
    rc = lib().oracle_gemm_epi_f32e(L, M, N, K, _ptr(A), _ptr(B), _ptr(C), _ptr(X), _ptr(rb), _ptr(cb), _ptr(sc),
                                    KINDS[kind], _ptr(D), _ptr(Aux), _ptr(Acc), _ptr(D64), _ptr(Aux64), _ptr(Acc64),
                                    DTYPES[ab_dtype])
    if rc:
        raise ValueError(f"oracle_gemm_epi_f32e rejected the call (code {rc})")
    out = {"D": D}
    if Aux is not None:
        out["Aux"] = Aux
    if Acc is not None:
        out["Acc"] = Acc
    if want64:
        out["D64"] = D64
        if Aux64 is not None:
            out["Aux64"] = Aux64
        out["Acc64"] = Acc64
    return out


def gemm_epi_points(A, B, C=None, X=None, *, kind, alpha=1.0, beta=0.0, s3=0.0, row_bias=None, col_bias=None,
                    l, i, j, dtype="f16"):
    """The same definition at sampled output points (l[p], i[p], j[p]).

    Returns a dict of 1-D arrays indexed by p: D, Aux (if the kind has one) as
    float16, Acc (float32, if the kind returns it), and D64 / Aux64 / Acc64
    unrounded.  dtype as for gemm_epi.
    """
    A, B = _bits(A, dtype), _bits(B, dtype)
    C = _bits(C, dtype) if C is not None else None
    X = _bits(X, dtype) if X is not None else None
    L, M, N, K = _shapes(A, B, C)
    rb, cb = _biases(row_bias, col_bias, M, N, dtype)
    l = np.ascontiguousarray(l, np.int64)
    i = np.ascontiguousarray(i, np.int64)
    j = np.ascontiguousarray(j, np.int64)
    n = l.size
    if i.size != n or j.size != n:
        raise ValueError("l, i, j must have the same length")
    sc = np.array([alpha, beta, s3], np.float32)
    D = np.empty(n, np.uint16)
    D64 = np.empty(n, np.float64)
    Acc64 = np.empty(n, np.float64)
    Aux = np.empty(n, np.uint16) if kind in HAS_AUX else None
    Aux64 = np.empty(n, np.float64) if kind in HAS_AUX else None
    Acc = np.empty(n, np.float32) if kind in HAS_ACC else None
    rc = lib().oracle_gemm_epi_points_typed(L, M, N, K, _ptr(A), _ptr(B), _ptr(C), _ptr(X), _ptr(rb), _ptr(cb),
                                            _ptr(sc), KINDS[kind], n, _ptr(l), _ptr(i), _ptr(j), _ptr(D), _ptr(Aux),
                                            _ptr(Acc), _ptr(D64), _ptr(Aux64), _ptr(Acc64), DTYPES[dtype])
    if rc:
        raise ValueError(f"oracle_gemm_epi_points_typed rejected the call (code {rc})")
    view = (lambda a: a.view(np.float16)) if dtype == "f16" else (lambda a: a)
    out = {"D": view(D), "D64": D64, "Acc64": Acc64}
    if Aux is not None:
        out["Aux"] = view(Aux)
        out["Aux64"] = Aux64
    if Acc is not None:
        out["Acc"] = Acc
    return out
