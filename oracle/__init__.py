"""ctypes wrapper around the CPU oracle (oracle/jetfp8_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by bench.py's CPU-baseline
leg.  The product library never imports it.

Arrays are numpy; bf16 tensors travel as uint16 bit patterns.  Layouts (logical, row-major):
  quantize_rows(x[R,C])   -> codes[R,C], scales[C/128, R]      (1x128 groups along C)
  quantize_cols(x[R,C])   -> codes[R,C], scales[R/128, C]      (128x1 groups along R)
  quantize_blocks(x[R,C]) -> codes[R,C], scales[R/128, C/128]  (128x128 blocks)
  gemm_fwd(xq, xs, wq, ws)      -> y[M,N]   bf16 bits
  gemm_dgrad(dyq, dys, wq, ws)  -> dx[M,K]  (W given in its forward [N,K] layout)
  gemm_wgrad(dyq, dys, xq, xs)  -> dw[N,K]  (dY[M,N], X[M,K] both grouped along M)
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libjetfp8_oracle.so")
_lib = None

EXACT = 0   # group sum = fp32 rounding of the exact 128-term sum (plain definition)
MFMA = 1    # matrix-instruction block model (parity unpinned; see jetfp8_oracle.c)

_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.jo_e4m3_decode.restype = ctypes.c_double
        L.jo_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.jo_e4m3_encode.restype = ctypes.c_uint8
        L.jo_e4m3_encode.argtypes = [ctypes.c_double]
        L.jo_bf16_to_f32.restype = ctypes.c_float
        L.jo_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.jo_f32_to_bf16.restype = ctypes.c_uint16
        L.jo_f32_to_bf16.argtypes = [ctypes.c_float]
        L.jo_code_for.restype = ctypes.c_uint8
        L.jo_code_for.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
        L.jo_requantize_cols.argtypes = [_u8p, _f32p, _i64, _i64, _u8p, _f32p, ctypes.c_int]
        L.jo_requantize_cols.restype = None
        L.jo_dequantize_value.argtypes = [ctypes.c_uint8, ctypes.c_float]
        L.jo_dequantize_value.restype = ctypes.c_float
        for name in ("jo_quantize_rows", "jo_quantize_cols", "jo_quantize_blocks"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [_u16p, _i64, _i64, _u8p, _f32p, ctypes.c_int]
        for name in ("jo_gemm_fwd", "jo_gemm_dgrad", "jo_gemm_wgrad"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [_u8p, _f32p, _u8p, _f32p, _u16p, _i64, _i64, _i64,
                          ctypes.c_void_p, _i64, ctypes.c_int, ctypes.c_int]
        L.jo_group_sum.restype = ctypes.c_float
        L.jo_group_sum.argtypes = [_u8p, _u8p, ctypes.c_int]
        L.jo_gemm_fwd_f64.restype = None
        L.jo_gemm_fwd_f64.argtypes = [_u8p, _f32p, _u8p, _f32p, _f64p, _i64, _i64, _i64]
        _lib = L
    return _lib


def decode(c: int) -> float:
    return lib().jo_e4m3_decode(int(c) & 0xFF)


def encode(v: float) -> int:
    return int(lib().jo_e4m3_encode(float(v)))


def bf16_to_f32(b: int) -> float:
    return lib().jo_bf16_to_f32(int(b) & 0xFFFF)


def f32_to_bf16(f: float) -> int:
    return int(lib().jo_f32_to_bf16(float(f)))


def code_for(x_bits: int, amax_bits: int) -> int:
    return int(lib().jo_code_for(int(x_bits) & 0xFFFF, int(amax_bits) & 0xFFFF))


def _check_bf16(x):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError("expected a 2-D uint16 (bf16 bit pattern) array")
    return x


def quantize_rows(x, threads=None):
    x = _check_bf16(x)
    R, C = x.shape
    if C % 128:
        raise ValueError("columns must be a multiple of 128")
    q = np.empty((R, C), np.uint8)
    s = np.empty((C // 128, R), np.float32)
    lib().jo_quantize_rows(x, R, C, q, s, threads or default_threads())
    return q, s


def quantize_cols(x, threads=None):
    x = _check_bf16(x)
    R, C = x.shape
    if R % 128:
        raise ValueError("rows must be a multiple of 128")
    q = np.empty((R, C), np.uint8)
    s = np.empty((R // 128, C), np.float32)
    lib().jo_quantize_cols(x, R, C, q, s, threads or default_threads())
    return q, s


def requantize_cols(q, s, threads=None):
    """128x1 quantization of the dequantized 1x128 codes of a saved FP8 activation: q uint8 [R, C] with scales
    s float32 [C/128, R] -> codes uint8 [R, C] (logical layout), scales float32 [R/128, C]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    R, C = q.shape
    if R % 128 or C % 128 or s.shape != (C // 128, R):
        raise ValueError("q [R, C] with R, C multiples of 128 and s [C/128, R] expected")
    qo = np.empty((R, C), np.uint8)
    so = np.empty((R // 128, C), np.float32)
    lib().jo_requantize_cols(q, s, R, C, qo, so, threads or default_threads())
    return qo, so


def quantize_blocks(x, threads=None):
    x = _check_bf16(x)
    R, C = x.shape
    if R % 128 or C % 128:
        raise ValueError("both dims must be multiples of 128")
    q = np.empty((R, C), np.uint8)
    s = np.empty((R // 128, C // 128), np.float32)
    lib().jo_quantize_blocks(x, R, C, q, s, threads or default_threads())
    return q, s


def _rows_arg(rows, total):
    if rows is None:
        return None, total, None
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if r.ndim != 1 or (r.size and (r.min() < 0 or r.max() >= total)):
        raise ValueError("row indices out of range")
    return r.ctypes.data_as(ctypes.c_void_p), r.size, r


def _c(a, dt):
    a = np.ascontiguousarray(a)
    if a.dtype != dt:
        raise TypeError(f"expected {dt}, got {a.dtype}")
    return a


def gemm_fwd(xq, xs, wq, ws, rows=None, mode=EXACT, threads=None):
    xq, wq = _c(xq, np.uint8), _c(wq, np.uint8)
    xs, ws = _c(xs, np.float32), _c(ws, np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape == (N, K) and xs.shape == (K // 128, M) and ws.shape == (N // 128, K // 128)
    rp, nr, keep = _rows_arg(rows, M)
    y = np.empty((nr, N), np.uint16)
    lib().jo_gemm_fwd(xq, xs, wq, ws, y, M, N, K, rp, nr, mode, threads or default_threads())
    return y


def gemm_dgrad(dyq, dys, wq, ws, rows=None, mode=EXACT, threads=None):
    dyq, wq = _c(dyq, np.uint8), _c(wq, np.uint8)
    dys, ws = _c(dys, np.float32), _c(ws, np.float32)
    M, N = dyq.shape
    K = wq.shape[1]
    assert wq.shape == (N, K) and dys.shape == (N // 128, M) and ws.shape == (N // 128, K // 128)
    rp, nr, keep = _rows_arg(rows, M)
    dx = np.empty((nr, K), np.uint16)
    lib().jo_gemm_dgrad(dyq, dys, wq, ws, dx, M, N, K, rp, nr, mode, threads or default_threads())
    return dx


def gemm_wgrad(dyq, dys, xq, xs, rows=None, mode=EXACT, threads=None):
    dyq, xq = _c(dyq, np.uint8), _c(xq, np.uint8)
    dys, xs = _c(dys, np.float32), _c(xs, np.float32)
    M, N = dyq.shape
    K = xq.shape[1]
    assert xq.shape == (M, K) and dys.shape == (M // 128, N) and xs.shape == (M // 128, K)
    rp, nr, keep = _rows_arg(rows, N)
    dw = np.empty((nr, K), np.uint16)
    lib().jo_gemm_wgrad(dyq, dys, xq, xs, dw, M, N, K, rp, nr, mode, threads or default_threads())
    return dw


def group_sum(a, b, mode=EXACT) -> float:
    a, b = _c(a, np.uint8), _c(b, np.uint8)
    assert a.size == 128 and b.size == 128
    return float(lib().jo_group_sum(a, b, mode))


def gemm_fwd_f64(xq, xs, wq, ws):
    xq, wq = _c(xq, np.uint8), _c(wq, np.uint8)
    xs, ws = _c(xs, np.float32), _c(ws, np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    y = np.empty((M, N), np.float64)
    lib().jo_gemm_fwd_f64(xq, xs, wq, ws, y, M, N, K)
    return y


def bf16_bits_to_f32(a) -> np.ndarray:
    """Widen an array of bf16 bit patterns (exact)."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32)
