"""Pins for the oracle's quantizers (CPU only).

Rule (Jet-RL explainers, "Schema de Quantification" / "Esquema de Quantizacao"): activations and
gradients in 1x128 groups, weights in 128x128 blocks, WGrad operands in 128-groups along the token axis.
Readings: OCP E4M3, s = fl32(amax / 448), code = nearest E4M3 to x / s (ties even, saturating), zero
groups give signed zeros.  Independent pins: the hand-derived fixture file, an exact-rational brute force
written with Python fractions, and invariants of the rule.
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_groups.txt")


def _f32(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def _f32_bits(v) -> int:
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def _bf16_val(b: int) -> float:
    return _f32((b & 0xFFFF) << 16)


def _load_golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            a, x, s, c = (int(t, 16) for t in line.split())
            rows.append((a, x, s, c))
    return rows


def test_golden_hand_groups(orc):
    rows = _load_golden()
    assert len(rows) >= 18
    for a, x, s_bits, code in rows:
        g = np.zeros((1, 128), np.uint16)
        g[0, 0] = a
        g[0, 77] = x
        q, s = orc.quantize_rows(g)
        assert _f32_bits(s[0, 0]) == s_bits, (hex(a), hex(x))
        assert int(q[0, 77]) == code, (hex(a), hex(x), hex(int(q[0, 77])))
        assert orc.code_for(x, a) == code


# --- exact-rational brute force (independent of the oracle's fp64 shortcut) -----------------------
_E4M3 = None


def _e4m3_values():
    global _E4M3
    if _E4M3 is None:
        vals = []
        for e in range(16):
            for m in range(8):
                if e == 15 and m == 7:
                    continue
                vals.append(Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7))
        _E4M3 = vals          # code order 0x00 .. 0x7E, ascending
    return _E4M3


def _brute_code(x: Fraction, s: Fraction) -> int:
    vals = _e4m3_values()
    neg = x < 0
    a = min(abs(x) / s, Fraction(448))
    best = min(range(len(vals)), key=lambda c: (abs(vals[c] - a), c % 2))   # nearest, then even code
    return best | (0x80 if neg else 0)


def test_code_for_matches_exact_rational_brute_force(orc):
    rng = np.random.default_rng(3)
    checked = 0
    # amax spread over the whole bf16 range (normals and subnormals) and x a random fraction of it
    for _ in range(1500):
        a_bits = int(rng.integers(1, 0x7F80))
        a = _bf16_val(a_bits)
        x_bits = int(rng.integers(0, 0x7F80))
        if _bf16_val(x_bits) > a:
            x_bits = int(a_bits * rng.random())  # a smaller bf16 magnitude
        x_bits |= int(rng.integers(0, 2)) << 15
        s = Fraction(_f32(_f32_bits(np.float32(a) / np.float32(448.0))))
        if s == 0:
            continue
        want = _brute_code(Fraction(_bf16_val(x_bits)), s)
        assert orc.code_for(x_bits, a_bits) == want, (hex(x_bits), hex(a_bits))
        checked += 1
    assert checked > 1000


def test_code_for_near_midpoints_brute_force(orc):
    # x chosen so that x / s lands within a hair of an E4M3 rounding midpoint
    vals = _e4m3_values()
    rng = np.random.default_rng(5)
    n = 0
    for _ in range(400):
        c = int(rng.integers(0, 126))
        mid = (vals[c] + vals[c + 1]) / 2
        a_bits = int(rng.integers(0x3800, 0x4400))
        a = _bf16_val(a_bits)
        s = np.float32(a) / np.float32(448.0)
        target = float(mid) * float(s)
        x_bits = _f32_bits(np.float32(target)) >> 16
        for xb in (x_bits - 1, x_bits, x_bits + 1):
            if 0 <= xb < 0x7F80 and _bf16_val(xb) <= a:
                want = _brute_code(Fraction(_bf16_val(xb)), Fraction(float(s)))
                assert orc.code_for(xb, a_bits) == want
                n += 1
    assert n > 300


def test_amax_element_maps_to_448_for_every_bf16_amax(orc):
    # For every positive finite bf16 amax the amax element itself must encode to 0x7E (and -amax to 0xFE):
    # x/s = a / fl32(a/448) stays within [447.5, 464) for all of them.
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    groups = np.zeros((bits.size, 128), np.uint16)
    groups[:, 5] = bits
    groups[:, 99] = bits | 0x8000
    q, s = orc.quantize_rows(groups)
    assert np.all(q[:, 5] == 0x7E)
    assert np.all(q[:, 99] == 0xFE)
    a = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(s[0].view(np.uint32), (a / np.float32(448.0)).view(np.uint32))


def test_power_of_two_scaling_is_equivariant(orc):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    base = (x.view(np.uint32) >> 16).astype(np.uint16)
    q0, s0 = orc.quantize_rows(base)
    for k in (-20, -3, 1, 7, 30):
        xs = ((base.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** k))
        b = (xs.view(np.uint32) >> 16).astype(np.uint16)   # exact: scaling by 2^k keeps bf16 values exact
        q, s = orc.quantize_rows(b)
        assert np.array_equal(q, q0), k
        assert np.array_equal(s, s0 * np.float32(2.0 ** k)), k


def test_negation_flips_only_the_sign_bit(orc):
    rng = np.random.default_rng(10)
    x = rng.standard_normal((4, 384)).astype(np.float32) * 3
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    q, s = orc.quantize_rows(b)
    qn, sn = orc.quantize_rows(b ^ np.uint16(0x8000))
    assert np.array_equal(qn, q ^ np.uint8(0x80))
    assert np.array_equal(s, sn)


def test_zero_group_and_group_locality(orc):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((3, 512)).astype(np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    b[1, 128:256] = 0
    b[1, 130] = 0x8000          # a negative zero inside the zero group
    q, s = orc.quantize_rows(b)
    assert s[1, 1] == 0.0
    assert np.all(q[1, 128:256][np.arange(128) != 2] == 0x00) and q[1, 130] == 0x80
    # changing one group never changes another group's codes or scales
    b2 = b.copy()
    b2[0, 300] = 0x4700        # 32768, the new amax of group 2 of row 0
    q2, s2 = orc.quantize_rows(b2)
    assert np.array_equal(q2[0, :256], q[0, :256]) and np.array_equal(q2[0, 384:], q[0, 384:])
    assert np.array_equal(q2[1:], q[1:]) and s2[2, 0] != s[2, 0]


def test_cols_equal_rows_of_transpose(orc):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((256, 384)).astype(np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    qc, sc = orc.quantize_cols(b)
    qr, sr = orc.quantize_rows(np.ascontiguousarray(b.T))
    assert np.array_equal(qc, qr.T)
    assert np.array_equal(sc, sr)


def test_blocks_use_the_block_amax(orc):
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    x[3, 5] = 1.5     # block (0,0) dominated by one element
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    q, s = orc.quantize_blocks(b)
    assert s.shape == (2, 3)
    xf = (b.astype(np.uint32) << 16).view(np.float32)
    for i in range(2):
        for j in range(3):
            blk = xf[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert s[i, j] == np.float32(np.abs(blk).max()) / np.float32(448.0)
    amax_bits = int(b[3, 5])
    for (r, c) in [(0, 0), (3, 5), (100, 77), (127, 127)]:
        assert q[r, c] == orc.code_for(int(b[r, c]), amax_bits)
    assert q[3, 5] == 0x7E
