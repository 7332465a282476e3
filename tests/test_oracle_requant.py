"""Pins of the oracle's requantization of a saved FP8 activation (1x128 codes along K -> 128x1 groups along
the token axis), a CPU-only check: it must reduce to the pinned bf16 128x1 quantizer whenever the dequantized
values are bf16 values, and keep the quantizers' invariants."""
import numpy as np
import pytest

from conftest import f32_to_bits




def _codes(rng, R, C):
    c = rng.integers(0, 0x7F, (R, C), dtype=np.uint8)              # finite codes only (0x7F is NaN)
    return c | (rng.integers(0, 2, (R, C), dtype=np.uint8) << 7)


def _decode_table(orc):
    return np.array([orc.decode(c) for c in range(256)], dtype=np.float64)


@pytest.mark.parametrize("R,C", [(128, 128), (256, 384)])
def test_power_of_two_scales_reduce_to_bf16_cols(orc, R, C):
    """With saved scales 2^k the dequantized values are exact bf16 values (at most 4 significant bits), so the
    requantized codes and scales must equal the 128x1 quantizer's on that bf16 matrix."""
    rng = np.random.default_rng(R * 31 + C)
    q = _codes(rng, R, C)
    k = rng.integers(-20, 11, (C // 128, R))
    s = np.ldexp(np.float32(1.0), k).astype(np.float32)
    dec = _decode_table(orc)[q]                                       # exact values
    x = dec * np.repeat(s.T.astype(np.float64), 128, axis=1)         # [R, C]: s[c // 128][r]
    xb = f32_to_bits(x.astype(np.float32))
    assert np.array_equal(xb.astype(np.uint32) << 16, x.astype(np.float32).view(np.uint32))   # exactly bf16
    qo, so = orc.requantize_cols(q, s)
    qr, sr = orc.quantize_cols(xb)
    assert np.array_equal(so.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(qo, qr)


def test_scale_equivariance_and_sign_symmetry(orc):
    rng = np.random.default_rng(7)
    R, C = 256, 256
    q = _codes(rng, R, C)
    s = (rng.random((C // 128, R)) * 0.05 + 1e-3).astype(np.float32)
    qo, so = orc.requantize_cols(q, s)
    for j in (-3, 5):
        qj, sj = orc.requantize_cols(q, np.ldexp(s, j).astype(np.float32))
        assert np.array_equal(qj, qo)
        assert np.array_equal(sj, np.ldexp(so, j).astype(np.float32))
    qn, sn = orc.requantize_cols(q ^ 0x80, s)
    assert np.array_equal(sn, so)
    assert np.array_equal(qn, qo ^ 0x80)


def test_dequantized_value_is_one_fp32_product(orc):
    rng = np.random.default_rng(3)
    dec = _decode_table(orc)
    for _ in range(200):
        c = int(rng.integers(0, 0x7F)) | (int(rng.integers(0, 2)) << 7)
        sc = np.float32(rng.random() * 10.0 ** int(rng.integers(-6, 3)))
        want = np.float32(np.float32(dec[c]) * sc)                  # numpy's fp32 multiply
        got = np.float32(orc.lib().jo_dequantize_value(c, float(sc)))
        assert got.view(np.uint32) == want.view(np.uint32), (hex(c), sc)


def test_max_element_maps_to_448(orc):
    rng = np.random.default_rng(11)
    R, C = 128, 128
    q = _codes(rng, R, C)
    s = (rng.random((1, R)) + 0.5).astype(np.float32)
    qo, so = orc.requantize_cols(q, s)
    x = np.abs(_decode_table(orc)[q].astype(np.float32) * s[0][:, None])    # fp32 products, [R, C]
    arg = np.argmax(x, axis=0)
    for col in range(C):
        if x[arg[col], col] > 0:
            assert (qo[arg[col], col] & 0x7F) == 0x7E
