"""Unified precision flow at the level of a stack of FP8 pre-norm MLP blocks (Jet-RL explainers, "Architecture
Centrale": the rollout graph is a subgraph of the training forward graph, with the same quantization and
precision).  Each block is x + down(SwiGLU(gate_up(RMSNorm(x)))), all on this library's kernels: the fused
RMSNorm->1x128 producer, the FP8 gate/up GEMM (128x128 weight blocks), the fused SwiGLU->1x128 producer and the
FP8 down GEMM; only the residual add is torch (row-local bf16).

  * A token decoded alone (M = 1) or in a decode batch (M = 32) gets bitwise the same hidden state at every
    depth as the same token inside a prefill of the whole sequence (M = 96): no rollout/training mismatch.
  * Against a bf16 reference of the same stack (fp32 math on the bf16 tensors), each FP8 block adds a
    quantization error of a few percent that does not grow with depth.
Weights are random and seeded; no trained model is involved.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

D, F, LAYERS, S = 1024, 2816, 4, 96


@pytest.fixture(scope="module")
def stack():
    import torch
    import fp8_precision_rl_amd as jf
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    jf.load_library()
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    layers = []
    for _ in range(LAYERS):
        w_gu = (torch.randn((2 * F, D), device="cuda", generator=g) * D ** -0.5).to(torch.bfloat16)
        w_dn = (torch.randn((D, F), device="cuda", generator=g) * F ** -0.5).to(torch.bfloat16)
        w_nm = (1.0 + 0.1 * torch.randn((D,), device="cuda", generator=g)).to(torch.bfloat16)
        gq, gs, _ = jf.quantize_blocks(w_gu)
        dq, ds, _ = jf.quantize_blocks(w_dn)
        layers.append(dict(w_gu=w_gu, w_dn=w_dn, w_nm=w_nm, gq=gq, gs=gs, dq=dq, ds=ds))
    x0 = torch.randn((S, D), device="cuda", generator=g).to(torch.bfloat16)
    x0[:, 17] *= 30                                                   # an outlier channel
    return jf, layers, x0


EPS = 1e-5


def _fp8_block(jf, L, x):
    """FP8 branch y of one block (the residual is added by the caller)."""
    xq, xs, _ = jf.rmsnorm_quantize(x, L["w_nm"], EPS)
    gu = jf.gemm_fwd(xq, xs, L["gq"], L["gs"])
    hq, hs = jf.swiglu_quantize(gu)
    return jf.gemm_fwd(hq, hs, L["dq"], L["ds"])


def _bf16_block(L, x):
    import torch
    xf = x.float()
    n = (xf * torch.rsqrt(xf.pow(2).mean(dim=1, keepdim=True) + EPS) * L["w_nm"].float()).to(torch.bfloat16)
    gu = (n.float() @ L["w_gu"].float().t()).to(torch.bfloat16)
    g, u = gu.float().chunk(2, dim=-1)
    h = (torch.nn.functional.silu(g) * u).to(torch.bfloat16)
    return h.float() @ L["w_dn"].float().t()


def _fp8_stack(jf, layers, x):
    outs = []
    for L in layers:
        x = (x.float() + _fp8_block(jf, L, x).float()).to(x.dtype)
        outs.append(x)
    return outs


def _bf16_stack(layers, x):
    outs = []
    for L in layers:
        x = (x.float() + _bf16_block(L, x)).to(x.dtype)
        outs.append(x)
    return outs


def test_decode_and_prefill_hidden_states_are_bitwise_equal(stack):
    import torch
    jf, layers, x0 = stack
    prefill = _fp8_stack(jf, layers, x0)
    batch = _fp8_stack(jf, layers, x0[32:64].contiguous())
    singles = {t: _fp8_stack(jf, layers, x0[t:t + 1].contiguous()) for t in (0, 33, 95)}
    torch.cuda.synchronize()
    for depth in range(LAYERS):
        full = prefill[depth].view(torch.int16)
        assert torch.equal(batch[depth].view(torch.int16), full[32:64]), f"decode batch, depth {depth}"
        for t, outs in singles.items():
            assert torch.equal(outs[depth].view(torch.int16)[0], full[t]), f"token {t}, depth {depth}"


def test_fp8_block_error_against_bf16(stack):
    """Each block fed the same input on both sides (teacher forcing): the FP8 block's output branch y differs
    from the bf16 one by the quantization error of two GEMMs, a few percent in relative Frobenius norm (E4M3
    keeps 3 fraction bits: a relative rounding error of at most 2^-4 per operand element, about 2^-4 / sqrt(3)
    in rms), and that error does not grow with depth.  Run free, a random stack amplifies perturbations, so
    the end-to-end distance grows with depth; it is printed, not bounded."""
    import torch
    jf, layers, x0 = stack
    per_block = []
    x = x0
    for L in layers:
        y8, y_r = _fp8_block(jf, L, x).float(), _bf16_block(L, x)
        per_block.append(float((y8 - y_r).norm() / y_r.norm()))
        x = (x.float() + y_r).to(x.dtype)                              # continue on the bf16 trajectory
    free = [float((a.float() - b.float()).norm() / b.float().norm())
            for a, b in zip(_fp8_stack(jf, layers, x0), _bf16_stack(layers, x0))]
    print("per-block relative error (teacher-forced):", [f"{r:.3e}" for r in per_block], flush=True)
    print("free-running relative distance by depth:", [f"{r:.3e}" for r in free], flush=True)
    assert all(np.isfinite(per_block)) and all(np.isfinite(free))
    assert max(per_block) < 0.08, per_block
    assert max(per_block) < 1.5 * min(per_block), per_block
