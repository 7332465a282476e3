"""CPU oracle of the fused producers that emit 1x128 FP8 directly: RMSNorm -> quantize and SwiGLU -> quantize.

TEST INFRASTRUCTURE ONLY: imported by tests/ (and available to __graft_entry__.smoke() and bench.py's
CPU-baseline leg).  The product library never imports it.

Source: Jet-RL explainers, "Schema de Quantification" -- the 1x128 activation quantization is fused with the
operator that produces the activation, so the bf16 activation need not make a round trip through memory
before it is quantized.  The pages name no particular operator and give no arithmetic for the producers;
the readings below are the plain ones and are listed with the other readings of the pages:

RMSNorm (x [R][C] bf16, w [C] bf16, eps > 0):
    r[i] = the fp32 value nearest to 1 / sqrt(mean_k x[i][k]^2 + eps), the exact real value rounded once
           (ties to even); eps enters as its fp32 value.  r is also returned (the backward of RMSNorm uses it).
    y[i][k] = bf16( fl32( fl32(x[i][k] * r[i]) * w[k] ) )   -- the unfused fp32 operator with a bf16 output
    codes, scales = the 1x128 quantization of y (the pinned quantize_rows).
SwiGLU (gate_up [R][2F] bf16: gate = columns 0..F-1, up = columns F..2F-1):
    h[i][j] = bf16 nearest to silu(g) * u = g * u / (1 + exp(-g)), the exact real value rounded once (ties
              to even; a nonzero real h is never a tie, since exp of a nonzero rational is irrational).  An
              exact zero takes the sign of the IEEE product g * u / (1 + exp(-g)).
    codes, scales = the 1x128 quantization of h.

Every function here is a plain definition: exact rational arithmetic (Python Fraction / integers) where
the rounding of a real value has to be decided, numpy float64 where its error bound decides it, and
Python's decimal module (correctly rounded exp at 80 digits) for the rare values that fp64 cannot decide.
"""
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

from . import bf16_bits_to_f32, quantize_rows

_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_QUANTUM_SUB = -133          # exponent of the smallest bf16 subnormal


def _bf16_quantum_exp(a):
    """Exponent of the bf16 quantum (spacing) of magnitudes a (float64 array): 8 significant bits in the
    normal range, 2^-133 below 2^-126."""
    _, e = np.frexp(a)            # a = m * 2^e, m in [0.5, 1)
    return np.where(a >= _BF16_MIN_NORMAL, e - 8, _BF16_QUANTUM_SUB)


def round_to_bf16(v) -> np.ndarray:
    """Round float64 values to bfloat16, to nearest with ties to even, subnormals kept, overflow to +-inf;
    returns uint16 bit patterns.  (bf16: 8 significant bits, the exponent range of fp32.)"""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    qe = _bf16_quantum_exp(a)
    n = np.rint(np.ldexp(a, -qe))                     # scaling by a power of two is exact; rint ties to even
    r = np.ldexp(n, qe)
    r = np.where(r >= 2.0 ** 128, np.inf, r)          # 2^128 is past the largest bf16 (255 * 2^120)
    r = np.copysign(r, v)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_midpoint_distance(v) -> np.ndarray:
    """|v - m| / |v| where m is the midpoint between the two bf16 values that enclose |v| (float64 in, float64
    out; 0 for v == 0): how close a value is to a point where its bf16 rounding changes."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    qe = _bf16_quantum_exp(a)
    lo = np.ldexp(np.floor(np.ldexp(a, -qe)), qe)
    mid = lo + np.ldexp(0.5, qe)
    with np.errstate(invalid="ignore", divide="ignore"):
        d = np.abs(a - mid) / a
    return np.where(a > 0, d, np.inf)


# ---------------------------------------------------------------------------------------------- RMSNorm

def _exact_sum_of_squares(row_f64) -> Fraction:
    """Exact sum of squares of bf16 values given as float64 (each value is n / 2^j exactly, j <= 133)."""
    total = 0
    for v in row_f64.tolist():
        if v != 0.0:
            n, d = v.as_integer_ratio()               # d is a power of two <= 2^133
            total += (n * n) << (266 - 2 * (d.bit_length() - 1))
    return Fraction(total, 1 << 266)


def _f32_neighbors(r):
    r = np.float32(r)
    return np.nextafter(r, np.float32(0)), np.nextafter(r, np.float32(np.inf))


def _is_even_f32(r) -> bool:
    return (int(np.float32(r).view(np.uint32)) & 1) == 0


def rstd_exact(T: Fraction, near_rel: float):
    """(r, near): r = fp32 nearest to 1/sqrt(T) (T > 0, ties to even); near = the exact value lies within a
    relative distance near_rel of an fp32 rounding midpoint.  Comparisons are exact: for m > 0,
    1/sqrt(T) >= m  <=>  m^2 T <= 1."""
    r = np.float32(1.0 / np.sqrt(float(T)))                # candidate, then corrected by exact comparisons
    for _ in range(8):
        lo_n, hi_n = _f32_neighbors(r)
        hi_mid = (Fraction(float(r)) + Fraction(float(hi_n))) / 2
        lo_mid = (Fraction(float(r)) + Fraction(float(lo_n))) / 2
        above = hi_mid * hi_mid * T                        # < 1: the value is above hi_mid
        below = lo_mid * lo_mid * T                        # > 1: the value is below lo_mid
        if above < 1:
            r = hi_n
        elif below > 1:
            r = lo_n
        else:
            if above == 1 and not _is_even_f32(r):        # exact tie at hi_mid
                r = hi_n
            elif below == 1 and not _is_even_f32(r):      # exact tie at lo_mid
                r = lo_n
            break
    else:
        raise AssertionError("rstd rounding did not converge")
    lo_n, hi_n = _f32_neighbors(r)
    d = Fraction(near_rel)
    near = False
    for m in ((Fraction(float(r)) + Fraction(float(hi_n))) / 2, (Fraction(float(r)) + Fraction(float(lo_n))) / 2):
        a, b = m * (1 - d), m * (1 + d)
        if a * a * T <= 1 <= b * b * T:
            near = True
    return np.float32(r), near


def rmsnorm_rstd(x_bits, eps: float, near_rel: float = 2.0 ** -46):
    """r [R] float32 and near [R] bool for x [R][C] (bf16 bit patterns); see the module docstring."""
    x = bf16_bits_to_f32(np.ascontiguousarray(x_bits, dtype=np.uint16)).astype(np.float64)
    R, C = x.shape
    eps_q = Fraction(float(np.float32(eps)))
    if not eps_q > 0:
        raise ValueError("eps must be > 0")
    r = np.empty(R, dtype=np.float32)
    near = np.zeros(R, dtype=bool)
    for i in range(R):
        T = _exact_sum_of_squares(x[i]) / C + eps_q
        r[i], near[i] = rstd_exact(T, near_rel)
    return r, near


def rmsnorm_apply(x_bits, w_bits, r) -> np.ndarray:
    """y = bf16(fl32(fl32(x * r) * w)) as bf16 bit patterns [R][C]: two IEEE fp32 products, then one rounding
    to bf16."""
    x = bf16_bits_to_f32(np.ascontiguousarray(x_bits, dtype=np.uint16))
    w = bf16_bits_to_f32(np.ascontiguousarray(w_bits, dtype=np.uint16))
    with np.errstate(over="ignore"):
        y32 = (x * np.asarray(r, dtype=np.float32)[:, None]).astype(np.float32) * w[None, :]
    return round_to_bf16(y32.astype(np.float32).astype(np.float64))


def rmsnorm_quantize(x_bits, w_bits, eps: float, r=None):
    """(codes [R][C], scales [C/128][R], r [R], y bits [R][C], near [R]).  With r given (for instance the rstd
    a kernel returned for a row whose exact value sits next to an fp32 midpoint), y and the codes are formed
    from that r; near is then all False."""
    if r is None:
        r, near = rmsnorm_rstd(x_bits, eps)
    else:
        r = np.asarray(r, dtype=np.float32)
        near = np.zeros(r.shape, dtype=bool)
    y = rmsnorm_apply(x_bits, w_bits, r)
    q, s = quantize_rows(y)
    return q, s, r, y, near


# ----------------------------------------------------------------------------------------------- SwiGLU

def _silu_mul_decimal(g: float, u: float) -> Decimal:
    with localcontext() as ctx:
        ctx.prec = 80
        gd, ud = Decimal(g), Decimal(u)
        return gd * ud / (1 + (-gd).exp())


def _resolve_decimal(g: float, u: float, h64: float) -> np.uint16:
    """bf16 bits of the exact silu(g) * u, for a value whose fp64 estimate h64 is too close to a bf16
    midpoint: the 80-digit value decides the side of that midpoint."""
    a = abs(h64)
    qe = int(_bf16_quantum_exp(np.array([a]))[0])
    lo = np.ldexp(np.floor(np.ldexp(a, -qe)), qe)
    mid = Decimal(float(lo + np.ldexp(0.5, qe)))      # exact: a bf16 midpoint has 9 significant bits
    hd = _silu_mul_decimal(g, u).copy_abs()          # exact (abs() would round to the ambient precision)
    with localcontext() as ctx:
        ctx.prec = 80
        if (hd - mid).copy_abs() > mid * Decimal(10) ** -70:
            below = hd < mid
        elif g > 0 and (Decimal(g) * Decimal(u)).copy_abs() == mid:
            # a large gate: silu(g) = g / (1 + exp(-g)) < g strictly, so |h| lies just below |g u| = mid (by a
            # relative exp(-g), beyond 70 digits here) and rounds to the smaller magnitude
            below = True
        else:
            raise AssertionError(f"silu({g!r}) * {u!r} is a bf16 midpoint to 70 digits")
        mag = float(lo) if below else float(lo + np.ldexp(1.0, qe))
    return round_to_bf16(np.array([np.copysign(mag, h64)]))[0]


def swiglu_h(gu_bits, near_rel: float = 2.0 ** -45):
    """h [R][F] bf16 bit patterns from gate_up [R][2F]; see the module docstring.  Values that float64
    (relative error below 2^-50 here: exp, one add, one divide, one multiply, each within an ulp) places
    within near_rel of a bf16 midpoint are decided at 80 decimal digits."""
    gu = bf16_bits_to_f32(np.ascontiguousarray(gu_bits, dtype=np.uint16)).astype(np.float64)
    R, C2 = gu.shape
    F = C2 // 2
    g, u = gu[:, :F], gu[:, F:]
    with np.errstate(over="ignore", invalid="ignore"):
        h64 = g / (1.0 + np.exp(-g)) * u
    h = round_to_bf16(h64)
    flagged = np.argwhere(bf16_midpoint_distance(h64) <= near_rel)
    for i, j in flagged:
        h[i, j] = _resolve_decimal(float(g[i, j]), float(u[i, j]), float(h64[i, j]))
    return h


def swiglu_quantize(gu_bits):
    """(codes [R][F], scales [F/128][R], h bits [R][F])."""
    h = swiglu_h(gu_bits)
    q, s = quantize_rows(h)
    return q, s, h
