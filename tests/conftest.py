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


def compare_bf16(got_bits, ref_bits):
    """Element-wise comparison of two bf16 matrices: bit-match fraction, relative Frobenius error and
    max-abs error / rms(ref)."""
    import numpy as np
    g = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = (ref_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    d = g - r
    rms = float(np.sqrt(np.mean(r * r)))
    return {
        "bit_match": float(np.mean(got_bits == ref_bits)),
        "rel_frob": float(np.linalg.norm(d) / max(np.linalg.norm(r), 1e-300)),
        "max_abs_over_rms": float(np.abs(d).max() / max(rms, 1e-300)),
    }
