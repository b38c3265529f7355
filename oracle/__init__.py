"""CPU oracle for OUT_PROD through a block-quantized weight (ctypes wrapper).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package. It shares no code with the HIP
library and imports nothing from it.

    dst[t][k] = sum_n W[n][k] * G[t][n]

(llama.cpp PR "cuda: out_prod accepts a quantized src0", commit message and
section "What": the backward of mul_mat(W, x) with respect to x.) The
arithmetic lives in oracle.c; this module only marshals numpy arrays.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, F16, Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, BF16 = 0, 1, 2, 3, 6, 7, 8, 10, 11, 12, 13, 14, 30
MXFP4 = 39
NVFP4 = 40

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no FP contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall",
             "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_half_to_float.restype = ctypes.c_float
        lib.oracle_half_to_float.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_float.restype = ctypes.c_float
        lib.oracle_bf16_to_float.argtypes = [ctypes.c_uint16]
        lib.oracle_row_bytes.restype = i64
        lib.oracle_row_bytes.argtypes = [ctypes.c_int, i64]
        lib.oracle_decode_row.restype = ctypes.c_int
        lib.oracle_decode_row.argtypes = [ctypes.c_int, vp, i64, vp]
        lib.oracle_dequantize.restype = ctypes.c_int
        lib.oracle_dequantize.argtypes = [ctypes.c_int, vp, i64, i64, vp]
        lib.oracle_out_prod.restype = ctypes.c_int
        lib.oracle_out_prod.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, vp, i64, vp, vp, vp,
                                        ctypes.c_int]
        lib.oracle_mul_mat.restype = ctypes.c_int
        lib.oracle_mul_mat.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, vp, i64, vp, vp, vp, ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def row_bytes(wtype: int, K: int) -> int:
    return int(_load().oracle_row_bytes(wtype, K))


def half_to_float(bits: np.ndarray) -> np.ndarray:
    """Scalar binary16 decode applied to every uint16 in bits."""
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.array([lib.oracle_half_to_float(int(b)) for b in flat], dtype=np.float32)
    return out.reshape(np.shape(bits))


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.array([lib.oracle_bf16_to_float(int(b)) for b in flat], dtype=np.float32)
    return out.reshape(np.shape(bits))


def dequantize(wtype: int, W: np.ndarray, K: int) -> np.ndarray:
    """Decode W (uint8, N rows of row_bytes) to F32 N x K."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    rb = row_bytes(wtype, K)
    if rb < 0:
        raise ValueError("bad type or K")
    N = W.size // rb if rb else 0
    if W.size != N * rb:
        raise ValueError("W size is not a whole number of rows")
    out = np.empty((N, K), dtype=np.float32)
    if _load().oracle_dequantize(wtype, _ptr(W), K, N, _ptr(out)) != 0:
        raise ValueError("oracle_dequantize failed")
    return out


def out_prod(wtype: int, W: np.ndarray, G: np.ndarray, K: int, rows=None, nthreads: int = 1):
    """Returns (dst F32, acc float64, abssum float64), each len(rows) x K.

    rows selects t rows of the full T x K result (default: all of them).
    """
    W = np.ascontiguousarray(W, dtype=np.uint8)
    G = np.ascontiguousarray(G, dtype=np.float32)
    if G.ndim != 2:
        raise ValueError("G must be T x N")
    T, N = G.shape
    rb = row_bytes(wtype, K)
    if rb < 0 or W.size != N * rb:
        raise ValueError("W does not hold N rows of the given type and K")
    if rows is None:
        nrows, rows_arr, rows_ptr = T, None, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rows_ptr = rows_arr.size, _ptr(rows_arr)
    dst = np.empty((nrows, K), dtype=np.float32)
    acc = np.empty((nrows, K), dtype=np.float64)
    abssum = np.empty((nrows, K), dtype=np.float64)
    rc = _load().oracle_out_prod(wtype, _ptr(W), _ptr(G), K, N, T, rows_ptr, nrows, _ptr(dst),
                                 _ptr(acc), _ptr(abssum), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_out_prod failed")
    return dst, acc, abssum


def mul_mat(wtype: int, W: np.ndarray, X: np.ndarray, K: int, rows=None, nthreads: int = 1):
    """y = mul_mat(W, x): y[t][n] = sum_k W[n][k] x[t][k] (X float32 T x K).

    Returns (y F32, acc float64, abssum float64), each len(rows) x N.
    """
    W = np.ascontiguousarray(W, dtype=np.uint8)
    X = np.ascontiguousarray(X, dtype=np.float32)
    if X.ndim != 2 or X.shape[1] != K:
        raise ValueError("X must be T x K")
    T = X.shape[0]
    rb = row_bytes(wtype, K)
    if rb <= 0 or W.size % rb:
        raise ValueError("W does not hold whole rows of the given type and K")
    N = W.size // rb
    if rows is None:
        nrows, rows_arr, rows_ptr = T, None, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rows_ptr = rows_arr.size, _ptr(rows_arr)
    y = np.empty((nrows, N), dtype=np.float32)
    acc = np.empty((nrows, N), dtype=np.float64)
    abssum = np.empty((nrows, N), dtype=np.float64)
    rc = _load().oracle_mul_mat(wtype, _ptr(W), _ptr(X), K, N, T, rows_ptr, nrows, _ptr(y), _ptr(acc),
                                _ptr(abssum), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_mul_mat failed")
    return y, acc, abssum


def errors(y: np.ndarray, acc: np.ndarray, abssum: np.ndarray) -> dict:
    """Error of a result y against the double oracle.

    nmse    = sum (y - acc)^2 / sum acc^2
    max_rel = max |y - acc| / sum_n |W[n][k] G[t][n]|  (forward-error normaliser
              of a dot product; outputs whose terms are all zero must be exact)
    """
    y = np.asarray(y, dtype=np.float64)
    diff = y - acc
    den = float(np.sum(acc * acc))
    num = float(np.sum(diff * diff))
    nmse = num / den if den > 0 else (0.0 if num == 0 else float("inf"))
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(abssum > 0, np.abs(diff) / abssum, np.where(diff == 0, 0.0, np.inf))
    return {"nmse": nmse, "max_rel": float(np.max(rel)) if rel.size else 0.0,
            "nonfinite": int(np.sum(~np.isfinite(y)))}
