"""Thin ctypes binding of libq4k.so (C ABI in include/q4k.h).

Argument marshalling only: every step of the GEMV runs in the HIP kernels of
libq4k.so.  Arguments may be torch tensors (their data_ptr() is passed) or
plain integers holding device addresses.  ``stream`` defaults to torch's
current HIP stream.  A non-zero status raises Q4KError.  If libq4k.so has not
been built, loading raises immediately -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4k.so")

Q4K_OK = 0
Q4K_ERR_NULL = 1
Q4K_ERR_SHAPE = 2
Q4K_ERR_SIZE = 3
Q4K_ERR_ALIGN = 4
Q4K_ERR_UNSUPPORTED = 5
Q4K_ERR_HIP = 1000

# every symbol include/q4k.h declares
EXPORTED = (
    "q4k_row_bytes",
    "q4k_load",
    "q4k_gemv",
    "q4k_dequantize",
    "q4k_status_string",
    "q4k_gemv_ex",
    "q4k_read_calibrate",
    "q4k_read_calibrate_blocks",
    "q4k_plan",
    "q4k_gemv_q8",
    "q4k_quantize_q8",
    "q6k_row_bytes",
    "q6k_load",
    "q6k_gemv",
    "q6k_gemv_ex",
    "q6k_plan",
    "q6k_dequantize",
    "q4k_mirror_f16",
    "q6k_mirror_f16",
    "q4k_f16_cvt",
    "q4k_f16_gemm",
    "q4k_f16_gemm_f32x",
    "q4k_f16_gemm_f32x_noalloc",
)


class Q4KError(RuntimeError):
    def __init__(self, rc: int, where: str):
        self.rc = rc
        super().__init__("%s failed: status %d (%s)" % (where, rc, status_string(rc)))


class q4k_launch(ctypes.Structure):
    _fields_ = [
        ("variant", ctypes.c_int32),
        ("spans_per_chunk", ctypes.c_int32),
        ("rows_per_block", ctypes.c_int32),
        ("rows_per_wave", ctypes.c_int32),
        ("waves_per_block", ctypes.c_int32),
        ("x_in_registers", ctypes.c_int32),
        ("kernel", ctypes.c_int32),
        ("ring_depth", ctypes.c_int32),
        ("rows_per_task", ctypes.c_int32),
        ("cols_per_task", ctypes.c_int32),
    ]


class q4k_plan_info(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int32),
        ("grid", ctypes.c_int32),
        ("threads", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32),
        ("rows_per_block", ctypes.c_int32),
        ("cols_per_task", ctypes.c_int32),
        ("ring_depth", ctypes.c_int32),
        ("spans_per_chunk", ctypes.c_int32),
    ]


class q6k_launch(ctypes.Structure):
    _fields_ = [
        ("unit_bytes", ctypes.c_int32),
        ("batch_bytes", ctypes.c_int32),
        ("waves_per_block", ctypes.c_int32),
        ("column_groups", ctypes.c_int32),
        ("tiles_per_block", ctypes.c_int32),
    ]


class q6k_plan_info(ctypes.Structure):
    _fields_ = [
        ("unit_bytes", ctypes.c_int32),
        ("batch_bytes", ctypes.c_int32),
        ("waves_per_block", ctypes.c_int32),
        ("column_groups", ctypes.c_int32),
        ("rows_per_block", ctypes.c_int32),
        ("grid", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32),
    ]


VARIANT_AUTO = 0
VARIANT_SINGLE = 1
VARIANT_CHUNKED = 2

_lock = threading.Lock()
_lib = None


def load_library():
    """Load libq4k.so (raises OSError/RuntimeError when it is missing)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libq4k.so is not built (%s); run "
                               "`python -m block_quantized_decode_q4_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.q4k_row_bytes.argtypes = [i64]
        lib.q4k_row_bytes.restype = ctypes.c_size_t
        lib.q4k_load.argtypes = [vp, vp, ctypes.c_size_t, i64, i64, vp]
        lib.q4k_load.restype = ctypes.c_int
        lib.q4k_gemv.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        lib.q4k_gemv.restype = ctypes.c_int
        lib.q4k_gemv_ex.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.POINTER(q4k_launch), vp]
        lib.q4k_gemv_ex.restype = ctypes.c_int
        lib.q4k_dequantize.argtypes = [vp, vp, i64, i64, vp]
        lib.q4k_dequantize.restype = ctypes.c_int
        lib.q4k_gemv_q8.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        lib.q4k_gemv_q8.restype = ctypes.c_int
        lib.q4k_quantize_q8.argtypes = [vp, vp, vp, i64, i64, vp]
        lib.q4k_quantize_q8.restype = ctypes.c_int
        lib.q6k_row_bytes.argtypes = [i64]
        lib.q6k_row_bytes.restype = ctypes.c_size_t
        lib.q6k_load.argtypes = [vp, vp, ctypes.c_size_t, i64, i64, i64, vp]
        lib.q6k_load.restype = ctypes.c_int
        lib.q6k_gemv.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        lib.q6k_gemv.restype = ctypes.c_int
        lib.q6k_gemv_ex.argtypes = [vp, vp, vp, i64, i64, i64, ctypes.POINTER(q6k_launch), vp]
        lib.q6k_gemv_ex.restype = ctypes.c_int
        lib.q6k_plan.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(q6k_launch),
                                 ctypes.c_size_t, ctypes.POINTER(q6k_plan_info)]
        lib.q6k_plan.restype = ctypes.c_int
        lib.q6k_dequantize.argtypes = [vp, vp, i64, i64, i64, vp]
        lib.q6k_dequantize.restype = ctypes.c_int
        lib.q4k_mirror_f16.argtypes = [vp, vp, i64, i64, vp]
        lib.q4k_mirror_f16.restype = ctypes.c_int
        lib.q6k_mirror_f16.argtypes = [vp, vp, i64, i64, i64, vp]
        lib.q6k_mirror_f16.restype = ctypes.c_int
        lib.q4k_f16_cvt.argtypes = [vp, vp, i64, vp]
        lib.q4k_f16_cvt.restype = ctypes.c_int
        lib.q4k_f16_gemm.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        lib.q4k_f16_gemm.restype = ctypes.c_int
        lib.q4k_f16_gemm_f32x.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
        lib.q4k_f16_gemm_f32x.restype = ctypes.c_int
        lib.q4k_f16_gemm_f32x_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        lib.q4k_f16_gemm_f32x_noalloc.restype = ctypes.c_int
        lib.q4k_status_string.argtypes = [ctypes.c_int]
        lib.q4k_status_string.restype = ctypes.c_char_p
        lib.q4k_read_calibrate.argtypes = [vp, ctypes.c_size_t, vp, vp]
        lib.q4k_read_calibrate.restype = ctypes.c_int
        lib.q4k_read_calibrate_blocks.argtypes = []
        lib.q4k_read_calibrate_blocks.restype = ctypes.c_int
        lib.q4k_plan.argtypes = [i64, i64, i64, ctypes.POINTER(q4k_launch), ctypes.c_int,
                                 ctypes.c_size_t, ctypes.POINTER(q4k_plan_info)]
        lib.q4k_plan.restype = ctypes.c_int
        _lib = lib
        return lib


def _addr(a):
    """Device/host address of a torch tensor, numpy array or int (0 for None)."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if hasattr(a, "data_ptr"):
        if not a.is_contiguous():
            raise ValueError("tensor must be contiguous")
        return a.data_ptr()
    if hasattr(a, "ctypes"):
        return a.ctypes.data
    raise TypeError("expected a tensor, an array or an integer address, got %r" % type(a))


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str) -> None:
    if rc != Q4K_OK:
        raise Q4KError(rc, where)


def status_string(rc: int) -> str:
    return load_library().q4k_status_string(int(rc)).decode()


q4k_status_string = status_string


def q4k_row_bytes(k: int) -> int:
    return int(load_library().q4k_row_bytes(int(k)))


def q4k_load(w_dev, src_host, n: int, k: int, stream=None, src_bytes: int | None = None) -> None:
    """Copy Q4_K bytes from host memory into the device buffer w_dev
    (synchronous on stream)."""
    if src_bytes is None:
        src_bytes = src_host.nbytes if hasattr(src_host, "nbytes") else len(src_host)
    _check(load_library().q4k_load(_addr(w_dev), _addr(src_host), int(src_bytes), int(n), int(k),
                                   _stream(stream)), "q4k_load")


def q4k_gemv(w, x, y, n: int, k: int, m: int = 1, stream=None) -> None:
    """y[b*n + r] = sum_c W[r][c] x[b*k + c]; asynchronous on stream."""
    _check(load_library().q4k_gemv(_addr(w), _addr(x), _addr(y), int(n), int(k), int(m),
                                   _stream(stream)), "q4k_gemv")


def q4k_gemv_ex(w, x, y, n: int, k: int, m: int = 1, stream=None, **opts) -> None:
    """q4k_gemv with explicit launch options (fields of q4k_launch)."""
    cfg = q4k_launch(**{f: int(opts.get(f, 0)) for f, _ in q4k_launch._fields_})
    unknown = set(opts) - {f for f, _ in q4k_launch._fields_}
    if unknown:
        raise TypeError("unknown launch options %s" % sorted(unknown))
    _check(load_library().q4k_gemv_ex(_addr(w), _addr(x), _addr(y), int(n), int(k), int(m),
                                      ctypes.byref(cfg), _stream(stream)), "q4k_gemv_ex")


def q4k_dequantize(w, out, n: int, k: int, stream=None) -> None:
    """out[r*k + c] = W[r][c] in f32 (bit-exact); asynchronous on stream."""
    _check(load_library().q4k_dequantize(_addr(w), _addr(out), int(n), int(k), _stream(stream)),
           "q4k_dequantize")


def q4k_gemv_q8(w, x, y, n: int, k: int, m: int = 1, stream=None) -> None:
    """y = W x with x quantized to Q8 inside the kernel (the integer-dot
    variant, its own tolerance: see include/q4k.h); asynchronous."""
    _check(load_library().q4k_gemv_q8(_addr(w), _addr(x), _addr(y), int(n), int(k), int(m),
                                      _stream(stream)), "q4k_gemv_q8")


def q4k_quantize_q8(x, q, d, k: int, m: int = 1, stream=None) -> None:
    """The Q8 codes (int8, m x k) and scales (f32, m x k/32) of x (f32, m x k)
    that q4k_gemv_q8 uses; asynchronous."""
    _check(load_library().q4k_quantize_q8(_addr(x), _addr(q), _addr(d), int(k), int(m),
                                          _stream(stream)), "q4k_quantize_q8")


def q4k_plan(n: int, k: int, m: int = 1, w_aligned128: bool = True, lds_max: int = 0,
             **opts) -> q4k_plan_info:
    """The launch q4k_gemv_ex would make (no launch).  lds_max = 0 asks the
    current device; a nonzero value needs no GPU."""
    cfg = q4k_launch(**opts) if opts else None
    out = q4k_plan_info()
    _check(load_library().q4k_plan(int(n), int(k), int(m), ctypes.byref(cfg) if cfg else None,
                                   1 if w_aligned128 else 0, int(lds_max), ctypes.byref(out)),
           "q4k_plan")
    return out


def q6k_row_bytes(k: int) -> int:
    return int(load_library().q6k_row_bytes(int(k)))


def q6k_load(w_dev, src_host, n: int, k: int, row_stride: int = 0, stream=None,
             src_bytes: int | None = None) -> None:
    """Copy dense Q6_K rows from host memory into w_dev at row_stride
    (synchronous on stream)."""
    if src_bytes is None:
        src_bytes = src_host.nbytes if hasattr(src_host, "nbytes") else len(src_host)
    _check(load_library().q6k_load(_addr(w_dev), _addr(src_host), int(src_bytes), int(n), int(k),
                                   int(row_stride), _stream(stream)), "q6k_load")


def q6k_gemv(w, x, y, n: int, k: int, row_stride: int = 0, stream=None) -> None:
    """y[r] = sum_c W[r][c] x[c] over Q6_K rows; asynchronous on stream."""
    _check(load_library().q6k_gemv(_addr(w), _addr(x), _addr(y), int(n), int(k), int(row_stride),
                                   _stream(stream)), "q6k_gemv")


def q6k_gemv_ex(w, x, y, n: int, k: int, row_stride: int = 0, stream=None, **opts) -> None:
    """q6k_gemv with explicit launch options (fields of q6k_launch)."""
    unknown = set(opts) - {f for f, _ in q6k_launch._fields_}
    if unknown:
        raise TypeError("unknown launch options %s" % sorted(unknown))
    cfg = q6k_launch(**{f: int(opts.get(f, 0)) for f, _ in q6k_launch._fields_})
    _check(load_library().q6k_gemv_ex(_addr(w), _addr(x), _addr(y), int(n), int(k),
                                      int(row_stride), ctypes.byref(cfg), _stream(stream)),
           "q6k_gemv_ex")


def q6k_plan(n: int, k: int, row_stride: int = 0, w_aligned128: bool = True, lds_max: int = 0,
             **opts) -> q6k_plan_info:
    """The launch q6k_gemv_ex would make (no launch); lds_max = 0 asks the
    current device, a nonzero value needs no GPU."""
    cfg = q6k_launch(**opts) if opts else None
    out = q6k_plan_info()
    _check(load_library().q6k_plan(int(n), int(k), int(row_stride), 1 if w_aligned128 else 0,
                                   ctypes.byref(cfg) if cfg else None, int(lds_max),
                                   ctypes.byref(out)), "q6k_plan")
    return out


def q6k_dequantize(w, out, n: int, k: int, row_stride: int = 0, stream=None) -> None:
    """out[r*k + c] = W[r][c] in f32 (bit-exact); asynchronous on stream."""
    _check(load_library().q6k_dequantize(_addr(w), _addr(out), int(n), int(k), int(row_stride),
                                         _stream(stream)), "q6k_dequantize")


def q4k_mirror_f16(w, w16, n: int, k: int, stream=None) -> None:
    """The fp16 mirror (n x k halves) of dense Q4_K rows; asynchronous."""
    _check(load_library().q4k_mirror_f16(_addr(w), _addr(w16), int(n), int(k), _stream(stream)),
           "q4k_mirror_f16")


def q6k_mirror_f16(w, w16, n: int, k: int, row_stride: int = 0, stream=None) -> None:
    """The fp16 mirror (n x k halves) of Q6_K rows; asynchronous."""
    _check(load_library().q6k_mirror_f16(_addr(w), _addr(w16), int(n), int(k), int(row_stride),
                                         _stream(stream)), "q6k_mirror_f16")


def q4k_f16_cvt(x, x16, count: int, stream=None) -> None:
    """x16 = binary16 of x (nearest even); asynchronous."""
    _check(load_library().q4k_f16_cvt(_addr(x), _addr(x16), int(count), _stream(stream)),
           "q4k_f16_cvt")


def q4k_f16_gemm(w16, x16, y, m: int, n: int, k: int, stream=None) -> None:
    """y (m x n, f32) = x16 (m x k) @ w16 (n x k)^T on the matrix cores."""
    _check(load_library().q4k_f16_gemm(_addr(w16), _addr(x16), _addr(y), int(m), int(n), int(k),
                                       _stream(stream)), "q4k_f16_gemm")


def q4k_f16_gemm_f32x(w16, x, xh, y, m: int, n: int, k: int, stream=None) -> None:
    """Convert x (f32, m x k) into the scratch xh, then q4k_f16_gemm."""
    _check(load_library().q4k_f16_gemm_f32x(_addr(w16), _addr(x), _addr(xh), _addr(y), int(m),
                                            int(n), int(k), _stream(stream)),
           "q4k_f16_gemm_f32x")


def q4k_f16_gemm_f32x_noalloc(w16, x, y, m: int, n: int, k: int, stream=None) -> None:
    """q4k_f16_gemm_f32x with the library's static scratch (m*k <= 4 Mi);
    calls on one GPU must not overlap."""
    _check(load_library().q4k_f16_gemm_f32x_noalloc(_addr(w16), _addr(x), _addr(y), int(m),
                                                    int(n), int(k), _stream(stream)),
           "q4k_f16_gemm_f32x_noalloc")


def q4k_read_calibrate_blocks() -> int:
    return int(load_library().q4k_read_calibrate_blocks())


def q4k_read_calibrate(buf, nbytes: int, out, stream=None) -> None:
    _check(load_library().q4k_read_calibrate(_addr(buf), int(nbytes), _addr(out), _stream(stream)),
           "q4k_read_calibrate")
