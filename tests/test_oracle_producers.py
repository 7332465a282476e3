"""Pins of the producer oracle (oracle/producers.py) against things other than itself: torch's fp32 -> bf16
conversion, brute-force nearest-value searches with exact arithmetic, decimal square roots and exponentials,
closed forms (constant rows, huge or zero gates) and an exhaustive sweep over every finite bf16 gate value."""
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import producers as P


def _torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_value(bits: int) -> float:
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def _nearest_bf16_brute(exact: Fraction, sign_neg: bool) -> int:
    """bf16 bits of the value nearest to |exact| (ties to the even pattern), found by scanning the bf16
    patterns around the float64 estimate with exact distances."""
    a = abs(exact)
    est = np.array([float(a)], dtype=np.float64).astype(np.float32)
    base = int(est.view(np.uint32)[0] >> 16)
    best = None
    for b in range(max(0, base - 2), min(0x7F80, base + 3) + 1):
        v = Fraction(_bf16_value(b)) if b < 0x7F80 else None
        if v is None:
            continue
        d = abs(v - a)
        if best is None or d < best[0] or (d == best[0] and b % 2 == 0):
            best = (d, b)
    return best[1] | (0x8000 if sign_neg else 0)


# ------------------------------------------------------------------------------------- bf16 rounding

def test_round_to_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 0x7F800000, size=200_000, dtype=np.uint32)       # all finite positive fp32
    bits[:4096] = (bits[:4096] & 0xFFFF0000) | 0x8000                        # exact ties
    bits[4096:8192] &= 0x00FFFFFF                                            # subnormals and tiny normals
    bits[8192:8200] = [0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0, 1, 0x00008000, 0x00018000]
    f = bits.view(np.float32)
    f = np.concatenate([f, -f])
    assert np.array_equal(P.round_to_bf16(f.astype(np.float64)), _torch_bf16_bits(f))


def test_round_to_bf16_on_fp64_values_brute_force():
    rng = np.random.default_rng(2)
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-140, 120, 3000))
    # values that an fp32 intermediate would turn into ties: a bf16 midpoint plus or minus a few fp64 ulps
    mids = (rng.integers(0x3F800000, 0x40000000, 500, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    m64 = mids.view(np.float32).astype(np.float64)
    v = np.concatenate([v, np.nextafter(m64, np.inf), np.nextafter(m64, 0), m64])
    got = P.round_to_bf16(v)
    for x, b in zip(v.tolist(), got.tolist()):
        assert b == _nearest_bf16_brute(Fraction(x), x < 0), x


def test_midpoint_distance_is_zero_at_midpoints():
    mids = np.array([0x3F808000, 0x00008000, 0x7F7F0000 | 0x8000], dtype=np.uint32).view(np.float32)
    assert np.all(P.bf16_midpoint_distance(mids.astype(np.float64)) == 0)
    reps = np.array([0x3F800000, 0x00010000], dtype=np.uint32).view(np.float32).astype(np.float64)
    assert np.all(P.bf16_midpoint_distance(reps) > 2.0 ** -10)


# ----------------------------------------------------------------------------------------- RMSNorm

def _bf16_bits_of(a: np.ndarray) -> np.ndarray:
    return _torch_bf16_bits(np.asarray(a, dtype=np.float32))


def test_rstd_constant_rows_closed_form():
    # x = 2^k everywhere, eps = 3 * 4^k: mean + eps = 4^(k+1), so r = 2^-(k+1) exactly
    for k in (-20, -3, 0, 5, 40):
        x = _bf16_bits_of(np.full((1, 384), 2.0 ** k))
        r, near = P.rmsnorm_rstd(x, eps=float(np.float32(3 * 4.0 ** k)))
        assert r[0] == np.float32(2.0 ** -(k + 1)) and not near[0]


def test_rstd_matches_decimal_sqrt():
    rng = np.random.default_rng(3)
    R, C = 48, 640
    x = rng.standard_normal((R, C)) * np.exp2(rng.integers(-8, 8, (R, 1)))
    x[:, 7] *= 300.0                                                   # outlier channel
    xb = _bf16_bits_of(x)
    eps = 1e-5
    r, near = P.rmsnorm_rstd(xb, eps)
    xf = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    with localcontext() as ctx:
        ctx.prec = 60
        for i in range(R):
            ss = sum(Decimal(v) * Decimal(v) for v in xf[i].tolist())
            T = ss / C + Decimal(float(np.float32(eps)))
            val = 1 / T.sqrt()
            assert not near[i]
            assert r[i] == np.float32(float(val)), i                   # fp64 then fp32: safe away from midpoints


def test_rstd_scales_by_powers_of_two():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16, 256))
    r1, _ = P.rmsnorm_rstd(_bf16_bits_of(x), eps=2.0 ** -20)
    r2, _ = P.rmsnorm_rstd(_bf16_bits_of(x * 8.0), eps=2.0 ** -14)    # x * 8 and eps * 64: r / 8 exactly
    assert np.array_equal(r2, (r1 / np.float32(8.0)).astype(np.float32))


def test_rstd_zero_row_and_validation():
    x = np.zeros((2, 128), dtype=np.uint16)
    r, _ = P.rmsnorm_rstd(x, eps=0.25)
    assert np.all(r == np.float32(2.0))
    with pytest.raises(ValueError):
        P.rmsnorm_rstd(x, eps=0.0)


def test_rmsnorm_apply_matches_torch_and_bound():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((32, 512)) * 3
    w = 1 + 0.2 * rng.standard_normal(512)
    xb, wb = _bf16_bits_of(x), _bf16_bits_of(w)
    r, _ = P.rmsnorm_rstd(xb, 1e-6)
    y = P.rmsnorm_apply(xb, wb, r)
    xt = torch.from_numpy(oracle.bf16_bits_to_f32(xb))
    wt = torch.from_numpy(oracle.bf16_bits_to_f32(wb))
    ref = ((xt * torch.from_numpy(r)[:, None]) * wt).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, ref)
    # and y is x * w / rms to within the bf16 rounding and a few fp32 roundings
    xf, wf = oracle.bf16_bits_to_f32(xb).astype(np.float64), oracle.bf16_bits_to_f32(wb).astype(np.float64)
    exact = xf * wf / np.sqrt((xf ** 2).mean(axis=1, keepdims=True) + float(np.float32(1e-6)))
    yf = oracle.bf16_bits_to_f32(y).astype(np.float64)
    assert np.all(np.abs(yf - exact) <= np.abs(exact) * (2.0 ** -8 + 2.0 ** -21) + 1e-30)


def test_rmsnorm_quantize_composes_with_pinned_quantizer():
    rng = np.random.default_rng(6)
    xb = _bf16_bits_of(rng.standard_normal((8, 384)))
    wb = _bf16_bits_of(1 + 0.1 * rng.standard_normal(384))
    q, s, r, y, near = P.rmsnorm_quantize(xb, wb, 1e-5)
    q2, s2 = oracle.quantize_rows(y)
    assert np.array_equal(q, q2) and np.array_equal(s, s2) and not near.any()
    # with r handed in, the same outputs
    q3, s3, r3, y3, _ = P.rmsnorm_quantize(xb, wb, 1e-5, r=r)
    assert np.array_equal(q3, q) and np.array_equal(y3, y) and np.array_equal(r3, r)


# ------------------------------------------------------------------------------------------ SwiGLU

def _swiglu_brute(gb: np.ndarray, ub: np.ndarray) -> np.ndarray:
    """Per element: 60-digit decimal silu(g) * u, then the nearest bf16 by brute force (exact distances)."""
    out = np.empty(gb.shape, dtype=np.uint16)
    gf, uf = oracle.bf16_bits_to_f32(gb).astype(np.float64), oracle.bf16_bits_to_f32(ub).astype(np.float64)
    with localcontext() as ctx:
        for idx in np.ndindex(gb.shape):
            g, u = float(gf[idx]), float(uf[idx])
            if g == 0.0 or u == 0.0:
                neg = (np.signbit(g) != np.signbit(u))
                out[idx] = 0x8000 if neg else 0
                continue
            if -g > 11000:                                         # e^g below 2^-15000: rounds to zero
                out[idx] = 0 if u < 0 else 0x8000
                continue
            if g >= 300:
                # 0 < g u - h < g u e^-g < g u 2^-432: any value in (g u (1 - 2^-400), g u) has the same
                # nearest bf16 as h, since no bf16 midpoint other than g u itself can lie that close to g u
                h = Fraction(g) * Fraction(u) * (1 - Fraction(1, 2 ** 400))
                if abs(h) >= 2 ** 128:
                    out[idx] = 0xFF80 if h < 0 else 0x7F80
                else:
                    out[idx] = _nearest_bf16_brute(h, h < 0)
                continue
            ctx.prec = 60 if g < 100 else 200                       # e^-g must stay well inside the precision
            h = Decimal(g) * Decimal(u) / (1 + (-Decimal(g)).exp())
            if abs(h) >= Decimal(2) ** 128:
                out[idx] = 0xFF80 if h < 0 else 0x7F80
                continue
            out[idx] = _nearest_bf16_brute(Fraction(h), h < 0)
    return out


def _gu(gb, ub):
    return np.ascontiguousarray(np.concatenate([gb, ub], axis=1))


def test_swiglu_random_pairs_match_decimal():
    rng = np.random.default_rng(7)
    R, F = 8, 256
    g = rng.standard_normal((R, F)) * np.exp2(rng.integers(-6, 6, (R, F)))
    u = rng.standard_normal((R, F)) * np.exp2(rng.integers(-10, 10, (R, F)))
    gb, ub = _bf16_bits_of(g), _bf16_bits_of(u)
    assert np.array_equal(P.swiglu_h(_gu(gb, ub)), _swiglu_brute(gb, ub))


def test_swiglu_every_finite_gate_value():
    # all 65280 finite bf16 gate values (both signs), up = 1 and up = a non-power-of-two: the oracle's
    # float64 path against 60-digit decimal arithmetic
    allb = np.arange(0x10000, dtype=np.uint32)
    finite = ((allb >> 7) & 0xFF) != 0xFF
    gb = allb[finite].astype(np.uint16)
    n = gb.size - gb.size % 128
    gb = gb[:n].reshape(-1, 128)
    for uval in (1.0, -1.6796875):
        ub = np.full(gb.shape, _bf16_bits_of(np.array([uval]))[0], dtype=np.uint16)
        got = P.swiglu_h(_gu(gb, ub))
        assert np.array_equal(got, _swiglu_brute(gb, ub)), uval


def test_swiglu_closed_forms():
    # g = +-0: h = +-0 with the product's sign; g >= 2^8: silu(g) = g to far below bf16 resolution, so h is
    # the bf16 rounding of the exact product g * u; g <= -2^10: h is a zero of sign -sign(u)
    rng = np.random.default_rng(8)
    u = rng.standard_normal(128) * 4
    ub = _bf16_bits_of(u)[None, :]
    zero = np.zeros((1, 128), dtype=np.uint16)
    h = P.swiglu_h(_gu(zero, ub))
    assert np.array_equal(h, np.where(oracle.bf16_bits_to_f32(ub) < 0, 0x8000, 0).astype(np.uint16))
    h = P.swiglu_h(_gu(zero | 0x8000, ub))
    assert np.array_equal(h, np.where(oracle.bf16_bits_to_f32(ub) < 0, 0, 0x8000).astype(np.uint16))
    big = _bf16_bits_of(np.exp2(rng.uniform(8, 60, 128)) * rng.choice([1.0, 1.5, 1.25], 128))[None, :]
    prod = oracle.bf16_bits_to_f32(big).astype(np.float32) * oracle.bf16_bits_to_f32(ub)   # exact: 16 bits
    # where g u is itself a bf16 midpoint, h is just below it in magnitude and rounds toward zero
    pb = prod.view(np.uint32)
    tie = (pb & 0xFFFF) == 0x8000
    expect = np.where(tie, (pb >> 16).astype(np.uint16), _torch_bf16_bits(prod))
    assert tie.any()
    assert np.array_equal(P.swiglu_h(_gu(big, ub)), expect)
    neg = _bf16_bits_of(-np.exp2(rng.uniform(10, 100, 128)))[None, :]
    assert np.array_equal(P.swiglu_h(_gu(neg, ub)),
                          np.where(oracle.bf16_bits_to_f32(ub) < 0, 0, 0x8000).astype(np.uint16))


def test_swiglu_decimal_resolution_agrees_with_float64():
    # flag every value (near_rel = 1): the 80-digit resolution path must reproduce the float64 results
    rng = np.random.default_rng(9)
    gb = _bf16_bits_of(rng.standard_normal((2, 128)) * 3)
    ub = _bf16_bits_of(rng.standard_normal((2, 128)))
    assert np.array_equal(P.swiglu_h(_gu(gb, ub), near_rel=1.0), P.swiglu_h(_gu(gb, ub)))


def test_swiglu_quantize_composes_with_pinned_quantizer():
    rng = np.random.default_rng(10)
    gb = _bf16_bits_of(rng.standard_normal((4, 256)) * 2)
    ub = _bf16_bits_of(rng.standard_normal((4, 256)))
    q, s, h = P.swiglu_quantize(_gu(gb, ub))
    q2, s2 = oracle.quantize_rows(h)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
