import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU check")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


def bits_to_dev(bits, device="cuda"):
    """uint16 bf16 bit patterns (numpy) -> torch bfloat16 device tensor."""
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def dev_to_bits(t):
    """torch bfloat16 tensor -> uint16 bit patterns (numpy)."""
    import numpy as np
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_to_bits(a):
    """fp32 numpy -> bf16 bit patterns, round to nearest even (torch's conversion)."""
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_order(bits):
    """bf16 bit patterns -> integers in the order of the values (+0 and -0 both 0), so two finite values are
    neighbours (one bf16 ulp apart) exactly when their orders differ by 1."""
    import numpy as np
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def compare_bf16(got_bits, ref_bits):
    """Element-wise comparison of two bf16 matrices: bit-match fraction, relative Frobenius error, max-abs
    error / rms(ref), and the same max-abs over the elements that are not exactly one bf16 ulp apart
    (an output whose fp32 accumulator lies next to a bf16 rounding boundary can round either way after any
    change in the last fp32 bits; such single-ulp flips are counted separately)."""
    import numpy as np
    g = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = (ref_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    d = np.abs(g - r)
    rms = max(float(np.sqrt(np.mean(r * r))), 1e-300)
    step = np.abs(bf16_order(got_bits) - bf16_order(ref_bits))
    one_ulp = step == 1
    return {
        "bit_match": float(np.mean(got_bits == ref_bits)),
        "rel_frob": float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)),
        "max_abs_over_rms": float(d.max() / rms) if d.size else 0.0,
        "max_abs_over_rms_beyond_1ulp": float(np.where(one_ulp, 0.0, d).max() / rms) if d.size else 0.0,
        "one_ulp_flips": int(one_ulp.sum()),
        "beyond_1ulp": int((step > 1).sum()),
    }


# GEMM tolerance against the plain definition (the oracle's exact group sums): relative Frobenius error of the
# bf16 outputs, and max |error| / rms(out) over the outputs that are not single-ulp rounding flips.
GEMM_REL_FROB = 1e-3
GEMM_MAX_ABS = 1e-2


def check_gemm_parity(name, got, ref_mfma, ref_exact, model_bitwise=True):
    """Parity of a GPU GEMM output (bf16 bits) with the oracle.

    Against the plain definition (EXACT mode: each group's dot product is the fp32 rounding of its exact
    sum): relative Frobenius <= GEMM_REL_FROB, and max |error| <= GEMM_MAX_ABS * rms(out) once single-ulp
    flips are excluded; the raw max-abs, flips included, is printed.  Hardware-model check (labelled apart):
    bitwise equality with the oracle's matrix-instruction mode, whose group sums follow the FP8 matrix
    instruction's block alignment."""
    e = compare_bf16(got, ref_exact)
    m = compare_bf16(got, ref_mfma)
    print(f"{name}: vs exact group sums: rel_frob={e['rel_frob']:.3e} max_abs/rms raw={e['max_abs_over_rms']:.3e} "
          f"beyond-1ulp={e['max_abs_over_rms_beyond_1ulp']:.3e} (1-ulp flips {e['one_ulp_flips']}, larger "
          f"{e['beyond_1ulp']} of {got.size}); hardware model: bit_match={m['bit_match']:.6f}", flush=True)
    assert e["rel_frob"] <= GEMM_REL_FROB, (name, "relative Frobenius vs exact group sums", e)
    assert e["max_abs_over_rms_beyond_1ulp"] <= GEMM_MAX_ABS, (name, "max-abs beyond 1-ulp flips vs exact", e)
    if model_bitwise:
        assert m["bit_match"] == 1.0, (name, "hardware model (matrix-instruction group sums): not bitwise equal", m)
    return m, e
