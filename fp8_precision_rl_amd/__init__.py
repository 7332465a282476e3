"""Python binding of libjetfp8 (the MI355X FP8 group-quantize + block-scaled GEMM library).

Argument marshalling only: every step of the quantize / GEMM path runs in the library's gfx950 kernels.
PyTorch supplies device memory (tensors) and the current HIP stream.  The raw entry points carry the C
names (jetfp8_quantize, jetfp8_gemm_fwd, jetfp8_gemm_dgrad, jetfp8_gemm_wgrad) and take caller-allocated
output tensors; the helpers below them (quantize_rows, ..., linear_forward) only allocate outputs and call
the raw entry points.

The library is loaded from fp8_precision_rl_amd/lib/libjetfp8.so.  If it is missing this module raises on
first use; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libjetfp8.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_MODE, ERR_HIP, ERR_VALUE = 0, -1, -2, -3, -4, -5, -6
ROWS_1x128, COLS_128x1_T, BLOCKS_128x128, BLOCKS_128x128_FRAG = 0, 1, 2, 3
EXPORTED = ("jetfp8_quantize", "jetfp8_quantize_dual", "jetfp8_requantize_cols_t", "jetfp8_rmsnorm_quantize",
            "jetfp8_swiglu_quantize", "jetfp8_gemm_fwd", "jetfp8_gemm_fwd_frag", "jetfp8_gemm_dgrad",
            "jetfp8_gemm_wgrad", "jetfp8_status_string", "jetfp8_version")

_lib = None


class JetFP8Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the C entry points.  Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libjetfp8 is not built ({path} missing); run `python -m fp8_precision_rl_amd.build`")
    L = ctypes.CDLL(path)
    vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.jetfp8_quantize.restype = c_int
    L.jetfp8_quantize.argtypes = [vp, i64, i64, c_int, vp, vp, vp, vp]
    L.jetfp8_quantize_dual.restype = c_int
    L.jetfp8_quantize_dual.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
    L.jetfp8_requantize_cols_t.restype = c_int
    L.jetfp8_requantize_cols_t.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    L.jetfp8_rmsnorm_quantize.restype = c_int
    L.jetfp8_rmsnorm_quantize.argtypes = [vp, vp, i64, i64, ctypes.c_float, vp, vp, vp, vp, vp]
    L.jetfp8_swiglu_quantize.restype = c_int
    L.jetfp8_swiglu_quantize.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    for name in ("jetfp8_gemm_fwd", "jetfp8_gemm_fwd_frag", "jetfp8_gemm_dgrad", "jetfp8_gemm_wgrad"):
        f = getattr(L, name)
        f.restype = c_int
        f.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
    L.jetfp8_status_string.restype = ctypes.c_char_p
    L.jetfp8_status_string.argtypes = [c_int]
    L.jetfp8_version.restype = c_int
    L.jetfp8_version.argtypes = []
    _lib = L
    return L


def status_string(status: int) -> str:
    return load_library().jetfp8_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise JetFP8Error(fn, status, status_string(status))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libjetfp8 takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libjetfp8 takes contiguous (row-major) tensors only")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dt(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


_torch = None


def _torch_mod():
    global _torch
    if _torch is None:
        import torch
        _torch = torch
    return _torch


def _need(t, shape, dtype, name, device=None):
    """Host-side check of one operand before its pointer reaches the C ABI (which trusts the sizes it is
    given): a contiguous device tensor of exactly this shape and dtype, on `device` when given.  Kept to a few
    attribute reads (a decode step issues eight calls in well under 100 us)."""
    if t is None:
        raise ValueError(f"{name}: required")
    if not isinstance(t, _torch_mod().Tensor) or not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.shape != shape:                      # torch.Size compares element by element with a tuple
        raise ValueError(f"{name}: expected shape {tuple(int(d) for d in shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, other operands on {device}")


def _bf16_u8_f32():
    torch = _torch_mod()
    return torch.bfloat16, torch.uint8, torch.float32


# ------------------------------------------------------------------------------------------------
# Raw entry points: same names and argument order as the C ABI; outputs are caller-allocated.
# ------------------------------------------------------------------------------------------------
def jetfp8_quantize(src_bf16, rows: int, cols: int, mode: int, dst_codes, dst_scales, dst_codes_t=None,
                    stream=None) -> None:
    L = load_library()
    bf, u8, f32 = _bf16_u8_f32()
    R, C = int(rows), int(cols)
    if R >= 1 and C >= 1 and mode in (ROWS_1x128, COLS_128x1_T, BLOCKS_128x128, BLOCKS_128x128_FRAG):
        _need(src_bf16, (R, C), bf, "src_bf16")
        dev = src_bf16.device
        if mode == ROWS_1x128:
            _need(dst_codes, (R, C), u8, "dst_codes", dev)
            _need(dst_scales, (C // 128, R), f32, "dst_scales", dev)
        elif mode == COLS_128x1_T:
            _need(dst_codes, (C, R), u8, "dst_codes", dev)
            _need(dst_scales, (R // 128, C), f32, "dst_scales", dev)
        else:
            _need(dst_codes, (R, C), u8, "dst_codes", dev)
            _need(dst_scales, (R // 128, C // 128), f32, "dst_scales", dev)
            if dst_codes_t is not None:
                _need(dst_codes_t, (C, R), u8, "dst_codes_t", dev)
    st = L.jetfp8_quantize(_ptr(src_bf16), int(rows), int(cols), int(mode), _ptr(dst_codes), _ptr(dst_scales),
                           _ptr(dst_codes_t), _stream(stream))
    _check("jetfp8_quantize", st)


def jetfp8_quantize_dual(src_bf16, rows: int, cols: int, dst_codes, dst_scales, dst_codes_t, dst_scales_t,
                         stream=None) -> None:
    L = load_library()
    bf, u8, f32 = _bf16_u8_f32()
    R, C = int(rows), int(cols)
    if R >= 1 and C >= 1:
        _need(src_bf16, (R, C), bf, "src_bf16")
        dev = src_bf16.device
        _need(dst_codes, (R, C), u8, "dst_codes", dev)
        _need(dst_scales, (C // 128, R), f32, "dst_scales", dev)
        _need(dst_codes_t, (C, R), u8, "dst_codes_t", dev)
        _need(dst_scales_t, (R // 128, C), f32, "dst_scales_t", dev)
    st = L.jetfp8_quantize_dual(_ptr(src_bf16), int(rows), int(cols), _ptr(dst_codes), _ptr(dst_scales),
                                _ptr(dst_codes_t), _ptr(dst_scales_t), _stream(stream))
    _check("jetfp8_quantize_dual", st)


def jetfp8_requantize_cols_t(codes, scales, rows: int, cols: int, dst_codes_t, dst_scales_t, stream=None) -> None:
    L = load_library()
    bf, u8, f32 = _bf16_u8_f32()
    R, C = int(rows), int(cols)
    if R >= 1 and C >= 1:
        _need(codes, (R, C), u8, "codes")
        dev = codes.device
        _need(scales, (C // 128, R), f32, "scales", dev)
        _need(dst_codes_t, (C, R), u8, "dst_codes_t", dev)
        _need(dst_scales_t, (R // 128, C), f32, "dst_scales_t", dev)
    st = L.jetfp8_requantize_cols_t(_ptr(codes), _ptr(scales), int(rows), int(cols), _ptr(dst_codes_t),
                                    _ptr(dst_scales_t), _stream(stream))
    _check("jetfp8_requantize_cols_t", st)


def jetfp8_rmsnorm_quantize(x_bf16, weight_bf16, rows: int, cols: int, eps: float, dst_codes, dst_scales,
                            dst_rstd=None, dst_y_bf16=None, stream=None) -> None:
    L = load_library()
    bf, u8, f32 = _bf16_u8_f32()
    R, C = int(rows), int(cols)
    if R >= 1 and C >= 1:
        _need(x_bf16, (R, C), bf, "x_bf16")
        dev = x_bf16.device
        _need(weight_bf16, (C,), bf, "weight_bf16", dev)
        _need(dst_codes, (R, C), u8, "dst_codes", dev)
        _need(dst_scales, (C // 128, R), f32, "dst_scales", dev)
        if dst_rstd is not None:
            _need(dst_rstd, (R,), f32, "dst_rstd", dev)
        if dst_y_bf16 is not None:
            _need(dst_y_bf16, (R, C), bf, "dst_y_bf16", dev)
    st = L.jetfp8_rmsnorm_quantize(_ptr(x_bf16), _ptr(weight_bf16), int(rows), int(cols), float(eps),
                                   _ptr(dst_codes), _ptr(dst_scales), _ptr(dst_rstd), _ptr(dst_y_bf16),
                                   _stream(stream))
    _check("jetfp8_rmsnorm_quantize", st)


def jetfp8_swiglu_quantize(gate_up_bf16, rows: int, cols: int, dst_codes, dst_scales, dst_h_bf16=None,
                           stream=None) -> None:
    L = load_library()
    bf, u8, f32 = _bf16_u8_f32()
    R, F = int(rows), int(cols)
    if R >= 1 and F >= 1:
        _need(gate_up_bf16, (R, 2 * F), bf, "gate_up_bf16")
        dev = gate_up_bf16.device
        _need(dst_codes, (R, F), u8, "dst_codes", dev)
        _need(dst_scales, (F // 128, R), f32, "dst_scales", dev)
        if dst_h_bf16 is not None:
            _need(dst_h_bf16, (R, F), bf, "dst_h_bf16", dev)
    st = L.jetfp8_swiglu_quantize(_ptr(gate_up_bf16), int(rows), int(cols), _ptr(dst_codes), _ptr(dst_scales),
                                  _ptr(dst_h_bf16), _stream(stream))
    _check("jetfp8_swiglu_quantize", st)


def _check_gemm_operands(a, sa, b, sb, out, a_shape, sa_shape, b_shape, sb_shape, out_shape):
    bf, u8, f32 = _bf16_u8_f32()
    if min(a_shape + b_shape) < 1:
        return                                  # the C ABI rejects non-positive sizes itself
    _need(a, a_shape, u8, "A codes")
    dev = a.device
    _need(sa, sa_shape, f32, "A scales", dev)
    _need(b, b_shape, u8, "B codes", dev)
    _need(sb, sb_shape, f32, "B scales", dev)
    _need(out, out_shape, bf, "output", dev)


def jetfp8_gemm_fwd(xq, xs, wq, ws, y_bf16, M: int, N: int, K: int, stream=None) -> None:
    L = load_library()
    M, N, K = int(M), int(N), int(K)
    _check_gemm_operands(xq, xs, wq, ws, y_bf16, (M, K), (K // 128, M), (N, K), (N // 128, K // 128), (M, N))
    _check("jetfp8_gemm_fwd", L.jetfp8_gemm_fwd(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(y_bf16),
                                                 int(M), int(N), int(K), _stream(stream)))


def jetfp8_gemm_fwd_frag(xq, xs, wq_frag, ws, y_bf16, M: int, N: int, K: int, stream=None) -> None:
    L = load_library()
    M, N, K = int(M), int(N), int(K)
    _check_gemm_operands(xq, xs, wq_frag, ws, y_bf16, (M, K), (K // 128, M), (N, K), (N // 128, K // 128), (M, N))
    _check("jetfp8_gemm_fwd_frag", L.jetfp8_gemm_fwd_frag(_ptr(xq), _ptr(xs), _ptr(wq_frag), _ptr(ws), _ptr(y_bf16),
                                                           int(M), int(N), int(K), _stream(stream)))


def jetfp8_gemm_dgrad(dyq, dys, wqT, ws, dx_bf16, M: int, N: int, K: int, stream=None) -> None:
    L = load_library()
    M, N, K = int(M), int(N), int(K)
    _check_gemm_operands(dyq, dys, wqT, ws, dx_bf16, (M, N), (N // 128, M), (K, N), (N // 128, K // 128), (M, K))
    _check("jetfp8_gemm_dgrad", L.jetfp8_gemm_dgrad(_ptr(dyq), _ptr(dys), _ptr(wqT), _ptr(ws), _ptr(dx_bf16),
                                                     int(M), int(N), int(K), _stream(stream)))


def jetfp8_gemm_wgrad(dyqT, dysT, xqT, xsT, dw_bf16, M: int, N: int, K: int, stream=None) -> None:
    L = load_library()
    M, N, K = int(M), int(N), int(K)
    _check_gemm_operands(dyqT, dysT, xqT, xsT, dw_bf16, (N, M), (M // 128, N), (K, M), (M // 128, K), (N, K))
    _check("jetfp8_gemm_wgrad", L.jetfp8_gemm_wgrad(_ptr(dyqT), _ptr(dysT), _ptr(xqT), _ptr(xsT), _ptr(dw_bf16),
                                                     int(M), int(N), int(K), _stream(stream)))


# ------------------------------------------------------------------------------------------------
# Allocating helpers (torch tensors in, torch tensors out).
# ------------------------------------------------------------------------------------------------
def quantize_rows(x, stream=None):
    """1x128 groups along the last axis: x bf16 [R, C] -> codes uint8 [R, C], scales fp32 [C/128, R]."""
    import torch
    _dt(x, torch.bfloat16, "x")
    R, C = x.shape
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    s = torch.empty((C // 128, R), dtype=torch.float32, device=x.device)
    jetfp8_quantize(x, R, C, ROWS_1x128, q, s, None, stream)
    return q, s


def quantize_cols_t(x, stream=None):
    """128x1 groups along the first axis, codes transposed: x bf16 [R, C] -> codes [C, R], scales [R/128, C]."""
    import torch
    _dt(x, torch.bfloat16, "x")
    R, C = x.shape
    q = torch.empty((C, R), dtype=torch.uint8, device=x.device)
    s = torch.empty((R // 128, C), dtype=torch.float32, device=x.device)
    jetfp8_quantize(x, R, C, COLS_128x1_T, q, s, None, stream)
    return q, s


def quantize_dual(x, stream=None):
    """Both groupings from one read: x bf16 [R, C] -> (codes [R, C], scales [C/128, R]) as quantize_rows and
    (codes [C, R], scales [R/128, C]) as quantize_cols_t.  R and C multiples of 128."""
    import torch
    _dt(x, torch.bfloat16, "x")
    R, C = x.shape
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    s = torch.empty((C // 128, R), dtype=torch.float32, device=x.device)
    qT = torch.empty((C, R), dtype=torch.uint8, device=x.device)
    sT = torch.empty((R // 128, C), dtype=torch.float32, device=x.device)
    jetfp8_quantize_dual(x, R, C, q, s, qT, sT, stream)
    return q, s, qT, sT


def requantize_cols_t(q, s, stream=None):
    """128x1 groups along the rows from saved 1x128 codes: q uint8 [R, C] with scales fp32 [C/128, R] ->
    codes [C, R], scales [R/128, C] (as quantize_cols_t of the dequantized values)."""
    import torch
    R, C = q.shape
    qT = torch.empty((C, R), dtype=torch.uint8, device=q.device)
    sT = torch.empty((R // 128, C), dtype=torch.float32, device=q.device)
    jetfp8_requantize_cols_t(q, s, R, C, qT, sT, stream)
    return qT, sT


def rmsnorm_quantize(x, weight, eps: float, return_y: bool = False, stream=None):
    """Fused RMSNorm -> 1x128: x bf16 [R, C], weight bf16 [C] -> (codes [R, C], scales [C/128, R], rstd [R])
    and, with return_y, the bf16 normalized activation [R, C] as well."""
    import torch
    _dt(x, torch.bfloat16, "x")
    _dt(weight, torch.bfloat16, "weight")
    R, C = x.shape
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    s = torch.empty((C // 128, R), dtype=torch.float32, device=x.device)
    r = torch.empty((R,), dtype=torch.float32, device=x.device)
    y = torch.empty((R, C), dtype=torch.bfloat16, device=x.device) if return_y else None
    jetfp8_rmsnorm_quantize(x, weight, R, C, eps, q, s, r, y, stream)
    return (q, s, r, y) if return_y else (q, s, r)


def swiglu_quantize(gate_up, return_h: bool = False, stream=None):
    """Fused SwiGLU -> 1x128: gate_up bf16 [R, 2F] (gate first, then up) -> (codes [R, F], scales [F/128, R])
    and, with return_h, the bf16 activation h [R, F] as well."""
    import torch
    _dt(gate_up, torch.bfloat16, "gate_up")
    R, F2 = gate_up.shape
    F = F2 // 2
    q = torch.empty((R, F), dtype=torch.uint8, device=gate_up.device)
    s = torch.empty((F // 128, R), dtype=torch.float32, device=gate_up.device)
    h = torch.empty((R, F), dtype=torch.bfloat16, device=gate_up.device) if return_h else None
    jetfp8_swiglu_quantize(gate_up, R, F, q, s, h, stream)
    return (q, s, h) if return_h else (q, s)


def quantize_blocks(w, transposed: bool = True, stream=None):
    """128x128 blocks: w bf16 [N, K] -> codes [N, K], scales [N/128, K/128], (codes^T [K, N] if transposed)."""
    import torch
    _dt(w, torch.bfloat16, "w")
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
    qT = torch.empty((K, N), dtype=torch.uint8, device=w.device) if transposed else None
    jetfp8_quantize(w, N, K, BLOCKS_128x128, q, s, qT, stream)
    return (q, s, qT) if transposed else (q, s)


def quantize_blocks_frag(w, stream=None):
    """128x128 blocks with the codes in the fragment order of the decode GEMM: w bf16 [N, K] -> codes uint8 [N, K]
    (the same bytes as quantize_blocks, permuted: see JETFP8_BLOCKS_128x128_FRAG), scales [N/128, K/128]."""
    import torch
    _dt(w, torch.bfloat16, "w")
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
    jetfp8_quantize(w, N, K, BLOCKS_128x128_FRAG, q, s, None, stream)
    return q, s


def gemm_fwd_frag(xq, xs, wq_frag, ws, stream=None):
    import torch
    M, K = xq.shape
    N = wq_frag.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    jetfp8_gemm_fwd_frag(xq, xs, wq_frag, ws, y, M, N, K, stream)
    return y


def gemm_fwd(xq, xs, wq, ws, stream=None):
    import torch
    M, K = xq.shape
    N = wq.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    jetfp8_gemm_fwd(xq, xs, wq, ws, y, M, N, K, stream)
    return y


def gemm_dgrad(dyq, dys, wqT, ws, stream=None):
    import torch
    M, N = dyq.shape
    K = wqT.shape[0]
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dyq.device)
    jetfp8_gemm_dgrad(dyq, dys, wqT, ws, dx, M, N, K, stream)
    return dx


def gemm_wgrad(dyqT, dysT, xqT, xsT, stream=None):
    import torch
    N, M = dyqT.shape
    K = xqT.shape[0]
    dw = torch.empty((N, K), dtype=torch.bfloat16, device=dyqT.device)
    jetfp8_gemm_wgrad(dyqT, dysT, xqT, xsT, dw, M, N, K, stream)
    return dw


def linear_forward(x, wq, ws, stream=None):
    """FP8 linear forward (rollout and training share it): quantize x in 1x128 groups, block-scaled GEMM."""
    xq, xs = quantize_rows(x, stream)
    return gemm_fwd(xq, xs, wq, ws, stream), (xq, xs)


def linear_backward(dy, x, wqT, ws, stream=None):
    """DGrad and WGrad of the FP8 linear: dY re-quantized along each GEMM's contraction axis."""
    dyq, dys, dyqT, dysT = quantize_dual(dy, stream)
    dx = gemm_dgrad(dyq, dys, wqT, ws, stream)
    xqT, xsT = quantize_cols_t(x, stream)
    dw = gemm_wgrad(dyqT, dysT, xqT, xsT, stream)
    return dx, dw
