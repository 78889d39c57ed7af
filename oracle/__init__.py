"""CPU oracle for the Q4_K fused dequantize-and-multiply GEMV (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
does and shares no code with it.  The arithmetic lives in ``q4k_oracle.c``
(plain C, built with ``-ffp-contract=off``); this module only builds it with
gcc, loads it with ctypes and marshals numpy arrays.

Functions (names follow the problem's notation: d, dmin, sc_j, m_j, q):
  f16_to_f32(bits)            binary16 decode from its definition
  f32_to_f16_rne(values)      binary16 encode, round-to-nearest-even
  unpack_scales(s12)          12 packed bytes -> (sc[8], m[8])
  pack_scales(sc, m)          the inverse, written from the same bit table
  dequant(w, n, k)            f32 weights [n, k], one rounding per weight
  gemv(w, x)                  y and sum|w||x| in f64, x is [m, k]
  quantize_rows(x)            simple reference quantizer -> Q4_K bytes
  quantize_q8(x), gemv_q8     Q8 activations and the GEMV over them
  q6k_dequant_superblock(b)   one 210-byte Q6_K superblock -> 256 f32
  q6k_dequant(w, n, k)        Q6_K weights [n, k] (exact products)
  q6k_gemv(w, x, n)           the same GEMV over Q6_K weights
  f16_cvt(x)                  f32 -> binary16 bits, nearest even
  mirror_f16(w, fmt, n, k)    fp16 mirror of Q4_K (fmt 4) or Q6_K (fmt 6) rows
  f16_gemm(w16, x16)          y = x16 @ w16^T exactly in f64, and its bound
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4k_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_q4k.so")

QK = 256
SB_BYTES = 144

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, no FP contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oq_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oq_f16_to_f32.restype = ctypes.c_float
        lib.oq_f32_to_f16_rne.argtypes = [ctypes.c_float]
        lib.oq_f32_to_f16_rne.restype = ctypes.c_uint16
        lib.oq_unpack_scales.argtypes = [u8p, u8p, u8p]
        lib.oq_unpack_scales.restype = None
        lib.oq_pack_scales.argtypes = [u8p, u8p, u8p]
        lib.oq_pack_scales.restype = None
        lib.oq_dequant_superblock.argtypes = [u8p, f32p]
        lib.oq_dequant_superblock.restype = None
        lib.oq_dequant.argtypes = [u8p, i64, i64, f32p]
        lib.oq_dequant.restype = ctypes.c_int
        lib.oq_gemv.argtypes = [u8p, f32p, i64, i64, i64, f64p, f64p]
        lib.oq_gemv.restype = ctypes.c_int
        lib.oq_quantize_row.argtypes = [f32p, i64, u8p]
        lib.oq_quantize_row.restype = ctypes.c_int
        i8p = ctypes.POINTER(ctypes.c_int8)
        lib.oq_quantize_q8.argtypes = [f32p, i64, i8p, f32p]
        lib.oq_quantize_q8.restype = ctypes.c_int
        lib.oq_gemv_q8.argtypes = [u8p, i8p, f32p, i64, i64, i64, f64p, f64p]
        lib.oq_gemv_q8.restype = ctypes.c_int
        lib.oq6_dequant_superblock.argtypes = [u8p, f32p]
        lib.oq6_dequant_superblock.restype = None
        lib.oq6_dequant.argtypes = [u8p, i64, i64, i64, f32p]
        lib.oq6_dequant.restype = ctypes.c_int
        lib.oq6_gemv.argtypes = [u8p, f32p, i64, i64, i64, i64, f64p, f64p]
        lib.oq6_gemv.restype = ctypes.c_int
        u16p = ctypes.POINTER(ctypes.c_uint16)
        lib.oq_f16_cvt.argtypes = [f32p, i64, u16p]
        lib.oq_f16_cvt.restype = None
        lib.oq_mirror_f16.argtypes = [u8p, ctypes.c_int, i64, i64, i64, u16p]
        lib.oq_mirror_f16.restype = ctypes.c_int
        lib.oq_f16_gemm.argtypes = [u16p, u16p, i64, i64, i64, f64p, f64p]
        lib.oq_f16_gemm.restype = ctypes.c_int
        lib.oq_num_threads.argtypes = []
        lib.oq_num_threads.restype = ctypes.c_int
        lib.oq_set_num_threads.argtypes = [ctypes.c_int]
        lib.oq_set_num_threads.restype = None
        _lib = lib
        return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u8(w) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(w, dtype=np.uint8)).reshape(-1)
    return a


def num_threads() -> int:
    return int(_load().oq_num_threads())


def set_num_threads(t: int) -> None:
    _load().oq_set_num_threads(int(t))


def f16_to_f32(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).reshape(-1)
    out = np.empty(b.shape, dtype=np.float32)
    for i, v in enumerate(b.tolist()):
        out[i] = lib.oq_f16_to_f32(v)
    return out


def f32_to_f16_rne(values) -> np.ndarray:
    lib = _load()
    v = np.asarray(values, dtype=np.float32).reshape(-1)
    out = np.empty(v.shape, dtype=np.uint16)
    for i, x in enumerate(v.tolist()):
        out[i] = lib.oq_f32_to_f16_rne(x)
    return out


def unpack_scales(s12) -> tuple[np.ndarray, np.ndarray]:
    lib = _load()
    s = _u8(s12)
    assert s.size == 12
    sc = np.zeros(8, dtype=np.uint8)
    m = np.zeros(8, dtype=np.uint8)
    lib.oq_unpack_scales(_ptr(s, ctypes.c_uint8), _ptr(sc, ctypes.c_uint8), _ptr(m, ctypes.c_uint8))
    return sc, m


def pack_scales(sc, m) -> np.ndarray:
    lib = _load()
    a = _u8(sc)
    b = _u8(m)
    assert a.size == 8 and b.size == 8 and int(a.max()) < 64 and int(b.max()) < 64
    s = np.zeros(12, dtype=np.uint8)
    lib.oq_pack_scales(_ptr(a, ctypes.c_uint8), _ptr(b, ctypes.c_uint8), _ptr(s, ctypes.c_uint8))
    return s


def dequant_superblock(blk) -> np.ndarray:
    lib = _load()
    b = _u8(blk)
    assert b.size == SB_BYTES
    out = np.empty(QK, dtype=np.float32)
    lib.oq_dequant_superblock(_ptr(b, ctypes.c_uint8), _ptr(out, ctypes.c_float))
    return out


def _check_shape(w: np.ndarray, n: int, k: int) -> None:
    if k <= 0 or k % QK != 0 or n < 0:
        raise ValueError("bad shape n=%d k=%d" % (n, k))
    if w.size != n * (k // QK) * SB_BYTES:
        raise ValueError("weight bytes %d != n*(k/256)*144 = %d" % (w.size, n * (k // QK) * SB_BYTES))


def dequant(w, n: int, k: int) -> np.ndarray:
    lib = _load()
    wb = _u8(w)
    _check_shape(wb, n, k)
    out = np.empty((n, k), dtype=np.float32)
    rc = lib.oq_dequant(_ptr(wb, ctypes.c_uint8), n, k, _ptr(out, ctypes.c_float))
    if rc != 0:
        raise RuntimeError("oq_dequant rc=%d" % rc)
    return out


def gemv(w, x, n: int) -> tuple[np.ndarray, np.ndarray]:
    """y[b, r] and bound[b, r] = sum_c |w[r,c]| |x[b,c]|, both float64 [m, n]."""
    lib = _load()
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if xa.ndim == 1:
        xa = xa.reshape(1, -1)
    m, k = xa.shape
    wb = _u8(w)
    _check_shape(wb, n, k)
    y = np.empty((m, n), dtype=np.float64)
    bound = np.empty((m, n), dtype=np.float64)
    rc = lib.oq_gemv(_ptr(wb, ctypes.c_uint8), _ptr(xa, ctypes.c_float), n, k, m,
                     _ptr(y, ctypes.c_double), _ptr(bound, ctypes.c_double))
    if rc != 0:
        raise RuntimeError("oq_gemv rc=%d" % rc)
    return y, bound


def quantize_rows(x) -> np.ndarray:
    """Reference quantizer: float32 [n, k] -> Q4_K bytes [n * k/256 * 144]."""
    lib = _load()
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if xa.ndim == 1:
        xa = xa.reshape(1, -1)
    n, k = xa.shape
    if k % QK != 0:
        raise ValueError("k must be a multiple of 256")
    out = np.zeros(n * (k // QK) * SB_BYTES, dtype=np.uint8)
    rb = (k // QK) * SB_BYTES
    for r in range(n):
        row = np.ascontiguousarray(xa[r])
        seg = out[r * rb:(r + 1) * rb]
        rc = lib.oq_quantize_row(_ptr(row, ctypes.c_float), k, _ptr(seg, ctypes.c_uint8))
        if rc != 0:
            raise RuntimeError("oq_quantize_row rc=%d" % rc)
    return out


def quantize_q8(x) -> tuple[np.ndarray, np.ndarray]:
    """Q8 activations: float32 [m, k] -> codes int8 [m, k] and scales
    float32 [m, k/32] (blocks of 32, d = amax/127, nearest-even codes)."""
    lib = _load()
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if xa.ndim == 1:
        xa = xa.reshape(1, -1)
    m, k = xa.shape
    if k % 32 != 0:
        raise ValueError("k must be a multiple of 32")
    q = np.empty((m, k), dtype=np.int8)
    d = np.empty((m, k // 32), dtype=np.float32)
    for b in range(m):
        row = np.ascontiguousarray(xa[b])
        qb = q[b]
        db = d[b]
        rc = lib.oq_quantize_q8(_ptr(row, ctypes.c_float), k, _ptr(qb, ctypes.c_int8),
                                _ptr(db, ctypes.c_float))
        if rc != 0:
            raise RuntimeError("oq_quantize_q8 rc=%d" % rc)
    return q, d


def gemv_q8(w, q, d, n: int) -> tuple[np.ndarray, np.ndarray]:
    """y[b, r] = sum_c w[r, c] * d[b, c/32] * q[b, c] and its bound
    sum |w| |d q|, float64 [m, n]."""
    lib = _load()
    qa = np.ascontiguousarray(np.asarray(q, dtype=np.int8))
    if qa.ndim == 1:
        qa = qa.reshape(1, -1)
    m, k = qa.shape
    da = np.ascontiguousarray(np.asarray(d, dtype=np.float32).reshape(m, k // 32))
    wb = _u8(w)
    _check_shape(wb, n, k)
    y = np.empty((m, n), dtype=np.float64)
    bound = np.empty((m, n), dtype=np.float64)
    rc = lib.oq_gemv_q8(_ptr(wb, ctypes.c_uint8), _ptr(qa, ctypes.c_int8), _ptr(da, ctypes.c_float),
                        n, k, m, _ptr(y, ctypes.c_double), _ptr(bound, ctypes.c_double))
    if rc != 0:
        raise RuntimeError("oq_gemv_q8 rc=%d" % rc)
    return y, bound


Q6K_SB_BYTES = 210


def _q6k_stride(w: np.ndarray, n: int, k: int, row_stride: int) -> int:
    if k <= 0 or k % QK != 0 or n < 0:
        raise ValueError("bad shape n=%d k=%d" % (n, k))
    dense = (k // QK) * Q6K_SB_BYTES
    stride = dense if row_stride == 0 else int(row_stride)
    if stride < dense:
        raise ValueError("row_stride %d below the %d bytes of a row" % (stride, dense))
    if n > 0 and w.size < (n - 1) * stride + dense:
        raise ValueError("weight bytes %d too few for n=%d rows of stride %d" % (w.size, n, stride))
    return stride


def q6k_dequant_superblock(blk) -> np.ndarray:
    lib = _load()
    b = _u8(blk)
    assert b.size == Q6K_SB_BYTES
    out = np.empty(QK, dtype=np.float32)
    lib.oq6_dequant_superblock(_ptr(b, ctypes.c_uint8), _ptr(out, ctypes.c_float))
    return out


def q6k_dequant(w, n: int, k: int, row_stride: int = 0) -> np.ndarray:
    """Q6_K weights as f32 [n, k]; row r starts at byte r * row_stride
    (0: rows packed densely, 210 k / 256 bytes each)."""
    lib = _load()
    wb = _u8(w)
    stride = _q6k_stride(wb, n, k, row_stride)
    out = np.empty((n, k), dtype=np.float32)
    if n == 0:
        return out
    rc = lib.oq6_dequant(_ptr(wb, ctypes.c_uint8), n, k, stride, _ptr(out, ctypes.c_float))
    if rc != 0:
        raise RuntimeError("oq6_dequant rc=%d" % rc)
    return out


def q6k_gemv(w, x, n: int, row_stride: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """y[b, r] and bound[b, r] = sum_c |w[r,c]| |x[b,c]| over Q6_K weights,
    both float64 [m, n]."""
    lib = _load()
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if xa.ndim == 1:
        xa = xa.reshape(1, -1)
    m, k = xa.shape
    wb = _u8(w)
    stride = _q6k_stride(wb, n, k, row_stride)
    y = np.empty((m, n), dtype=np.float64)
    bound = np.empty((m, n), dtype=np.float64)
    if n == 0:
        return y, bound
    rc = lib.oq6_gemv(_ptr(wb, ctypes.c_uint8), _ptr(xa, ctypes.c_float), n, k, stride, m,
                      _ptr(y, ctypes.c_double), _ptr(bound, ctypes.c_double))
    if rc != 0:
        raise RuntimeError("oq6_gemv rc=%d" % rc)
    return y, bound


def f16_cvt(x) -> np.ndarray:
    """binary16 bits (uint16) of float32 values, round to nearest even."""
    lib = _load()
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(xa.shape, dtype=np.uint16)
    lib.oq_f16_cvt(_ptr(xa, ctypes.c_float), xa.size, _ptr(out, ctypes.c_uint16))
    return out


def mirror_f16(w, fmt: int, n: int, k: int, row_stride: int = 0) -> np.ndarray:
    """fp16 mirror (binary16 bits, uint16 [n, k]) of Q4_K rows (fmt 4, dense)
    or Q6_K rows (fmt 6, at row_stride; 0 = dense)."""
    lib = _load()
    wb = _u8(w)
    if fmt == 4:
        _check_shape(wb, n, k)
        stride = 0
    elif fmt == 6:
        stride = _q6k_stride(wb, n, k, row_stride)
    else:
        raise ValueError("fmt must be 4 or 6")
    out = np.empty((n, k), dtype=np.uint16)
    rc = lib.oq_mirror_f16(_ptr(wb, ctypes.c_uint8), fmt, n, k, stride, _ptr(out, ctypes.c_uint16))
    if rc != 0:
        raise RuntimeError("oq_mirror_f16 rc=%d" % rc)
    return out


def f16_gemm(w16, x16) -> tuple[np.ndarray, np.ndarray]:
    """y[b, r] = sum_c w16[r, c] x16[b, c] exactly (f64) and its bound
    sum |w16||x16|; w16 [n, k], x16 [m, k] binary16 bits (uint16)."""
    lib = _load()
    wa = np.ascontiguousarray(np.asarray(w16, dtype=np.uint16))
    xa = np.ascontiguousarray(np.asarray(x16, dtype=np.uint16))
    if xa.ndim == 1:
        xa = xa.reshape(1, -1)
    n, k = wa.shape
    m, k2 = xa.shape
    if k != k2:
        raise ValueError("k mismatch")
    y = np.empty((m, n), dtype=np.float64)
    bound = np.empty((m, n), dtype=np.float64)
    rc = lib.oq_f16_gemm(_ptr(wa, ctypes.c_uint16), _ptr(xa, ctypes.c_uint16), m, n, k,
                         _ptr(y, ctypes.c_double), _ptr(bound, ctypes.c_double))
    if rc != 0:
        raise RuntimeError("oq_f16_gemm rc=%d" % rc)
    return y, bound
