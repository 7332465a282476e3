"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to bf16; it holds none of the quantization or GEMM
arithmetic.  It stands in for the models and datasets of the Jet-RL pages (Llama3.1-8B, Qwen2.5-7B,
Qwen3-8B-Base, 32B models; GSM8K / MATH / DeepMATH), which are not available: the tensors take those
models' linear-layer shapes and LLM-like value statistics (outlier activation channels, small weights,
heavy-tailed gradients).

Recipe (host path, numpy PCG64):
  * one SeedSequence(seed) per workload, spawned into independent streams;
  * X  ~ N(0, 1); a fraction of the K columns (round(frac*K), at least 1, chosen without replacement,
        the same columns for every row) is multiplied by 50 before bf16 rounding;
  * W  ~ N(0, 0.02^2)            (0.02 is the standard deviation);
  * dY ~ 1e-3 * Student-t(nu=3) (host: numpy's standard_t; device: Z / sqrt(chi^2_3 / 3) from four
        standard normals);
  * values are drawn in fp32 and rounded to bf16 by torch (round to nearest even).
Large workloads use the device path: the same distributions drawn with a seeded torch generator on the
GPU (fp32 draw, bf16 rounding), because host generation of multi-GB tensors would dominate the run.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

LLAMA3_8B = [("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 28672), ("down", 14336, 4096)]
QWEN25_32B = [("qkv", 5120, 7168), ("o", 5120, 5120), ("gate_up", 5120, 55296), ("down", 27648, 5120)]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    linears: Tuple[Tuple[str, int, int], ...]   # (name, K, N): y[M,N] = x[M,K] . w[N,K]^T
    outlier_frac: float
    seed: int
    backward: bool
    description: str


WORKLOADS = {
    "fp8_linear_64x512x256": Workload(
        "fp8_linear_64x512x256", 64, (("linear", 512, 256),), 0.01, 0, False,
        "single FP8 linear forward, X[64,512] with 1% outlier columns x50, W[256,512]"),
    "llama3_8b_decode_m32": Workload(
        "llama3_8b_decode_m32", 32, tuple(LLAMA3_8B), 0.001, 1, False,
        "rollout decode, 32 tokens through Llama-3-8B-shaped linears"),
    "llama3_8b_prefill_m16384": Workload(
        "llama3_8b_prefill_m16384", 16384, tuple(LLAMA3_8B), 0.001, 2, False,
        "prefill / training forward, 8 x 2048 tokens through Llama-3-8B-shaped linears"),
    "llama3_8b_train_m16384": Workload(
        "llama3_8b_train_m16384", 16384, tuple(LLAMA3_8B), 0.001, 3, True,
        "training step (forward + dgrad + wgrad), 8 x 2048 tokens, Llama-3-8B-shaped linears"),
    "qwen25_32b_train_m65536": Workload(
        "qwen25_32b_train_m65536", 65536, tuple(QWEN25_32B), 0.001, 4, True,
        "long-rollout training step, 4 x 16384 tokens, Qwen2.5-32B-shaped linears"),
}


def outlier_count(frac: float, K: int) -> int:
    """round(frac * K) with halves away from zero, at least one column."""
    return max(1, int(np.floor(frac * K + 0.5)))


def _to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


class HostStreams:
    """Independent numpy PCG64 streams for one workload: one per (linear, tensor)."""

    TENSORS = ("x", "outliers", "w", "dy")

    def __init__(self, seed: int, n_linears: int):
        ss = np.random.SeedSequence(seed)
        kids = ss.spawn(n_linears * len(self.TENSORS))
        self._gens = [np.random.Generator(np.random.PCG64(k)) for k in kids]

    def gen(self, linear: int, tensor: str) -> np.random.Generator:
        return self._gens[linear * len(self.TENSORS) + self.TENSORS.index(tensor)]


def host_x(rng_x: np.random.Generator, rng_cols: np.random.Generator, M: int, K: int, frac: float,
           rows: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """X ~ N(0,1)[M,K] with outlier columns x50; returns (bf16 bits [M,K], outlier column indices)."""
    cols = np.sort(rng_cols.choice(K, size=outlier_count(frac, K), replace=False))
    x = rng_x.standard_normal((M, K), dtype=np.float32)
    x[:, cols] *= np.float32(50.0)
    return _to_bf16_bits(x), cols


def host_w(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    return _to_bf16_bits(w)


def host_dy(rng: np.random.Generator, M: int, N: int) -> np.ndarray:
    dy = (rng.standard_t(3.0, size=(M, N)) * 1e-3).astype(np.float32)
    return _to_bf16_bits(dy)


def host_linear(workload: Workload, index: int, M: Optional[int] = None):
    """Host tensors for one linear of a workload: dict with x, w (and dy when backward)."""
    name, K, N = workload.linears[index]
    M = workload.M if M is None else M
    st = HostStreams(workload.seed, len(workload.linears))
    x, cols = host_x(st.gen(index, "x"), st.gen(index, "outliers"), M, K, workload.outlier_frac)
    out = {"name": name, "M": M, "K": K, "N": N, "x": x, "outlier_cols": cols, "w": host_w(st.gen(index, "w"), N, K)}
    if workload.backward:
        out["dy"] = host_dy(st.gen(index, "dy"), M, N)
    return out


# ------------------------------------------------------------------------------------------------
# Device path (torch on the GPU): same distributions, seeded torch generator.
# ------------------------------------------------------------------------------------------------
def device_linear(workload: Workload, index: int, device="cuda", M: Optional[int] = None):
    import torch
    name, K, N = workload.linears[index]
    M = workload.M if M is None else M
    g = torch.Generator(device=device)
    g.manual_seed(workload.seed * 1000003 + index)
    gc = torch.Generator(device="cpu")
    gc.manual_seed(workload.seed * 1000003 + index)
    ncols = outlier_count(workload.outlier_frac, K)
    cols = torch.randperm(K, generator=gc)[:ncols].sort().values
    x = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    x[:, cols.to(device)] *= 50.0
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * 0.02
    out = {"name": name, "M": M, "K": K, "N": N, "x": x.to(torch.bfloat16), "w": w.to(torch.bfloat16),
           "outlier_cols": cols.numpy()}
    del x, w
    if workload.backward:
        # Student-t(3) = Z / sqrt(V / 3) with V ~ chi^2(3), the sum of three squared standard normals.  Drawn
        # in row chunks of at most 2^26 elements (bounded temporaries, no tensor beyond 2^31 elements in any
        # generator kernel).
        dy = torch.empty((M, N), dtype=torch.bfloat16, device=device)
        rows = max(1, (1 << 26) // N)
        for r0 in range(0, M, rows):
            r1 = min(M, r0 + rows)
            z = torch.randn((4, r1 - r0, N), generator=g, device=device, dtype=torch.float32)
            v = z[1] * z[1] + z[2] * z[2] + z[3] * z[3]
            dy[r0:r1] = (z[0] / torch.sqrt(v / 3.0) * 1e-3).to(torch.bfloat16)
            del z, v
        out["dy"] = dy
    return out


def list_workloads() -> List[str]:
    return list(WORKLOADS)


# ------------------------------------------------------------------------------------------------
# Inputs of the fused producers (RMSNorm -> 1x128 and SwiGLU -> 1x128): same recipes on the host (numpy) and
# on the device (torch), seeded.
# ------------------------------------------------------------------------------------------------
def host_rmsnorm_inputs(seed: int, R: int, C: int, outlier_frac: float = 0.01):
    """Residual-stream rows for an RMSNorm: x = N(0,1) * 2^U(-4,4) per row, outlier channels x50; the norm's
    weight = 1 + 0.1 N(0,1).  Returns (x bits [R,C], w bits [C])."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    x = rng.standard_normal((R, C), dtype=np.float32)
    x *= np.exp2(rng.uniform(-4, 4, size=(R, 1))).astype(np.float32)
    cols = rng.choice(C, size=outlier_count(outlier_frac, C), replace=False)
    x[:, cols] *= np.float32(50.0)
    w = (1.0 + 0.1 * rng.standard_normal(C)).astype(np.float32)
    return _to_bf16_bits(x), _to_bf16_bits(w)


def host_gate_up(seed: int, R: int, F: int, outlier_frac: float = 0.01):
    """Output of a gate/up projection for a SwiGLU: gate = 2 N(0,1) with outlier channels x20 (large positive and
    negative gates, the tails of silu), up = N(0,1).  Returns bits [R, 2F] (gate columns first)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    g = rng.standard_normal((R, F), dtype=np.float32) * np.float32(2.0)
    cols = rng.choice(F, size=outlier_count(outlier_frac, F), replace=False)
    g[:, cols] *= np.float32(20.0)
    u = rng.standard_normal((R, F), dtype=np.float32)
    return _to_bf16_bits(np.concatenate([g, u], axis=1))


def device_rmsnorm_inputs(seed: int, R: int, C: int, device="cuda", outlier_frac: float = 0.01):
    """Device version of host_rmsnorm_inputs (same recipe, torch generator): (x [R,C], w [C]) bf16."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn((R, C), device=device, generator=gen)
    x *= torch.exp2(torch.rand((R, 1), device=device, generator=gen) * 8 - 4)
    cols = torch.randperm(C, device=device, generator=gen)[:outlier_count(outlier_frac, C)]
    x[:, cols] *= 50.0
    w = 1.0 + 0.1 * torch.randn((C,), device=device, generator=gen)
    return x.to(torch.bfloat16), w.to(torch.bfloat16)


def device_gate_up(seed: int, R: int, F: int, device="cuda", outlier_frac: float = 0.01):
    """Device version of host_gate_up: bf16 [R, 2F]."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    gu = torch.empty((R, 2 * F), device=device, dtype=torch.bfloat16)
    g = torch.randn((R, F), device=device, generator=gen) * 2.0
    cols = torch.randperm(F, device=device, generator=gen)[:outlier_count(outlier_frac, F)]
    g[:, cols] *= 20.0
    gu[:, :F] = g.to(torch.bfloat16)
    del g
    gu[:, F:] = torch.randn((R, F), device=device, generator=gen).to(torch.bfloat16)
    return gu
