"""Pins for the oracle's E4M3 and bf16 codecs (CPU only).

The E4M3 format is OCP FP8 E4M3 ("FN"): the Jet-RL pages only say FP8, the format is the reading taken.
Independent references used here: torch's float8_e4m3fn and bfloat16 conversions (separate
implementations of the same published formats), and facts of the OCP definition (largest finite 448,
smallest normal 2^-6, smallest subnormal 2^-9, NaN at S.1111.111, 8 values per binade).
"""
import math
import struct

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.filterwarnings("ignore")


def _f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def test_decode_all_256_codes_match_torch_e4m3fn(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = orc.decode(c)
        if c & 0x7F == 0x7F:
            assert math.isnan(got) and math.isnan(ref[c])
        else:
            assert got == ref[c], hex(c)
            assert math.copysign(1.0, got) == math.copysign(1.0, ref[c]), hex(c)


def test_decode_landmarks(orc):
    assert orc.decode(0x7E) == 448.0
    assert orc.decode(0x08) == 2.0 ** -6
    assert orc.decode(0x07) == 7 * 2.0 ** -9
    assert orc.decode(0x01) == 2.0 ** -9
    assert orc.decode(0x00) == 0.0 and math.copysign(1, orc.decode(0x80)) == -1
    pos = [orc.decode(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:])), "non-negative codes must be strictly increasing"
    assert len(set(pos)) == 127
    for e in range(1, 15):  # every normal binade holds 8 evenly spaced values
        vals = pos[8 * e: 8 * e + 8]
        step = vals[1] - vals[0]
        assert all(math.isclose(b - a, step) for a, b in zip(vals, vals[1:]))


def test_encode_roundtrips_every_finite_code(orc):
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert orc.encode(orc.decode(c)) == c, hex(c)


def test_encode_midpoints_go_to_even_code(orc):
    for c in range(0x7E):
        lo, hi = orc.decode(c), orc.decode(c + 1)
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert orc.encode(mid) == even, hex(c)
        assert orc.encode(-mid) == even | 0x80, hex(c)
        # just off the midpoint goes to the nearer neighbour
        assert orc.encode(math.nextafter(mid, 0)) == c
        assert orc.encode(math.nextafter(mid, math.inf)) == c + 1


def test_encode_saturates_never_nan(orc):
    for v in (448.0, 449.0, 463.9, 464.0, 480.0, 1e4, 3.4e38, math.inf):
        assert orc.encode(v) == 0x7E
        assert orc.encode(-v) == 0xFE
    assert orc.encode(2.0 ** -11) == 0x00 and orc.encode(-(2.0 ** -11)) == 0x80
    assert orc.encode(-0.0) == 0x80


def test_encode_matches_torch_on_dense_fp32_sweep(orc):
    # torch's fp32 -> float8_e4m3fn is round-to-nearest-even; it does not saturate, so stay <= 448.
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.uniform(-448, 448, 4000),
        np.ldexp(rng.uniform(1, 2, 4000), rng.integers(-14, 9, 4000)) * rng.choice([-1, 1], 4000),
        [orc.decode(c) for c in range(0x7E)],
    ]).astype(np.float32)
    vals = vals[np.abs(vals) <= 448]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.encode(float(v)) for v in vals], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_bf16_widen_all_patterns_match_torch(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    for b in list(range(0, 65536, 97)) + [0x0001, 0x7F7F, 0x8000, 0xFF7F]:
        got = orc.bf16_to_f32(b)
        r = float(ref[b])
        if math.isnan(r):
            assert math.isnan(got)
        else:
            assert _f32_bits(got) == _f32_bits(r)


def test_bf16_narrow_matches_torch_rne(orc):
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    u = u[(u & 0x7F800000) != 0x7F800000]                 # finite only
    ties = (rng.integers(0, 2 ** 15, 2000).astype(np.uint32) << 16) | 0x8000   # exact ties
    ties = ties[(ties & 0x7F800000) != 0x7F800000]
    u = np.concatenate([u, ties, ties | 0x80000000])
    f = u.view(np.float32)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16(float(v)) for v in f], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(hex(int(u[i])), hex(int(got[i])), hex(int(ref[i]))) for i in bad[:5]]
