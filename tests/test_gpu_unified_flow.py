"""Unified precision flow at the level of a stack of FP8 pre-norm decoder blocks (Jet-RL explainers, "Architecture
Centrale": the rollout graph is a subgraph of the training forward graph, with the same quantization and
precision).  Each block is

    h  = x + O(attn(QKV(RMSNorm(x))))
    x' = h + down(SwiGLU(gate_up(RMSNorm(h))))

with every linear and producer on this library's kernels: the fused RMSNorm->1x128 and SwiGLU->1x128 producers,
the 1x128 quantizer for the attention output, and the FP8 GEMMs with 128x128 weight blocks.  The attention
mixing itself (causal softmax over the cached keys) is a deterministic fp64 CPU stand-in that computes each query
row with the same call whatever the mode, so any difference between the modes can only come from the FP8 path.

  * Prefill of 96 tokens (M = 96), incremental decode of the same tokens one at a time (M = 1, with a key/value
    cache) and chunked decode (M = 32 per step) give bitwise the same hidden state for every token at every depth:
    no rollout/training mismatch.
  * The prefill hidden states equal, bit for bit at every depth, the same stack run through the CPU oracle
    (its RMSNorm->1x128 and SwiGLU->1x128 producers, its 1x128 quantizer, its block quantizer and its forward GEMM
    in the matrix-instruction mode), with the same attention stand-in and the same fp32 residual adds.
  * Against a bf16 reference of the same stack (fp32 math on the bf16 tensors, same attention stand-in), each FP8
    block adds a quantization error of a few percent that does not grow with depth (teacher forcing).
Weights are random and seeded; no trained model is involved.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

D, HEADS, F, LAYERS, S = 1024, 8, 2816, 3, 96
HD = D // HEADS
EPS = 1e-5


@pytest.fixture(scope="module")
def stack():
    import torch
    import fp8_precision_rl_amd as jf
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    jf.load_library()
    g = torch.Generator(device="cuda")
    g.manual_seed(7)

    def lin(n, k):
        return (torch.randn((n, k), device="cuda", generator=g) * k ** -0.5).to(torch.bfloat16)

    def norm_w():
        return (1.0 + 0.1 * torch.randn((D,), device="cuda", generator=g)).to(torch.bfloat16)

    layers = []
    for _ in range(LAYERS):
        L = dict(w_qkv=lin(3 * D, D), w_o=lin(D, D), w_gu=lin(2 * F, D), w_dn=lin(D, F), n1=norm_w(), n2=norm_w())
        for k in ("qkv", "o", "gu", "dn"):
            L[k + "_q"], L[k + "_s"], _ = jf.quantize_blocks(L["w_" + k])
        layers.append(L)
    x0 = torch.randn((S, D), device="cuda", generator=g).to(torch.bfloat16)
    x0[:, 17] *= 30                                                   # an outlier channel
    return jf, layers, x0


# --------------------------------------------------------------------------- attention stand-in (CPU, fp64)

def _attn_row(q, K, V):
    """One query row against its visible keys: q [D], K, V [t+1, D] (float64) -> [D].  Per head: softmax of
    q.k / sqrt(HD) over the keys, then the weighted sum of the values."""
    out = np.empty(D)
    for h in range(HEADS):
        sl = slice(h * HD, (h + 1) * HD)
        s = K[:, sl] @ q[sl] / np.sqrt(HD)
        p = np.exp(s - s.max())
        out[sl] = (p / p.sum()) @ V[:, sl]
    return out


def _f32(bits):
    """bf16 bit patterns (numpy uint16) -> float32, exact."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _to_bf16_bits(a32):
    """float32 (numpy) -> bf16 bit patterns, round to nearest even (torch's conversion, on the CPU)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _attention_bits(qkv_bits, cache, start):
    """qkv_bits: bf16 bits [m, 3D] for tokens start .. start+m-1; cache: dict of K, V float64 lists (appended
    here).  Returns the attention output rows as bf16 bits [m, D] (fp64 -> fp32 -> bf16, each rounding to
    nearest even)."""
    a = _f32(qkv_bits).astype(np.float64)
    outs = []
    for i in range(a.shape[0]):
        cache["K"].append(a[i, D:2 * D])
        cache["V"].append(a[i, 2 * D:])
        t = start + i
        outs.append(_attn_row(a[i, :D], np.array(cache["K"][:t + 1]), np.array(cache["V"][:t + 1])))
    return _to_bf16_bits(np.array(outs, dtype=np.float32))


def _attention(qkv_rows, cache, start):
    """Device wrapper of _attention_bits: bf16 [m, 3D] on the GPU -> bf16 [m, D] on the GPU."""
    import torch
    bits = qkv_rows.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    out = _attention_bits(bits, cache, start)
    return torch.from_numpy(out.view(np.int16)).to("cuda").view(torch.bfloat16)


# --------------------------------------------------------------------------------------------- blocks

def _fp8_block(jf, L, x, cache, start):
    import torch
    xq, xs, _ = jf.rmsnorm_quantize(x, L["n1"], EPS)
    qkv = jf.gemm_fwd(xq, xs, L["qkv_q"], L["qkv_s"])
    att = _attention(qkv, cache, start)
    aq, as_ = jf.quantize_rows(att)
    h = (x.float() + jf.gemm_fwd(aq, as_, L["o_q"], L["o_s"]).float()).to(torch.bfloat16)
    hq, hs, _ = jf.rmsnorm_quantize(h, L["n2"], EPS)
    gu = jf.gemm_fwd(hq, hs, L["gu_q"], L["gu_s"])
    sq, ss = jf.swiglu_quantize(gu)
    return (h.float() + jf.gemm_fwd(sq, ss, L["dn_q"], L["dn_s"]).float()).to(torch.bfloat16)


def _rmsnorm_ref(x, w):
    import torch
    xf = x.float()
    return (xf * torch.rsqrt(xf.pow(2).mean(dim=1, keepdim=True) + EPS) * w.float()).to(torch.bfloat16)


def _mm(a, w):
    import torch
    return (a.float() @ w.float().t()).to(torch.bfloat16)


def _bf16_block(L, x, cache, start):
    import torch
    qkv = _mm(_rmsnorm_ref(x, L["n1"]), L["w_qkv"])
    h = (x.float() + _mm(_attention(qkv, cache, start), L["w_o"]).float()).to(torch.bfloat16)
    gu = _mm(_rmsnorm_ref(h, L["n2"]), L["w_gu"])
    g, u = gu.float().chunk(2, dim=-1)
    act = (torch.nn.functional.silu(g) * u).to(torch.bfloat16)
    return (h.float() + _mm(act, L["w_dn"]).float()).to(torch.bfloat16)


def _run_fp8(jf, layers, x0, chunk):
    """Hidden states [layer][token] of the stack fed `chunk` tokens per call (S = prefill, 1 = decode)."""
    import torch
    caches = [{"K": [], "V": []} for _ in layers]
    outs = [[] for _ in layers]
    for start in range(0, S, chunk):
        x = x0[start:start + chunk].contiguous()
        for li, L in enumerate(layers):
            x = _fp8_block(jf, L, x, caches[li], start)
            outs[li].append(x)
    torch.cuda.synchronize()
    return [torch.cat(o).view(torch.int16).cpu().numpy() for o in outs]


def test_decode_and_prefill_hidden_states_are_bitwise_equal(stack):
    jf, layers, x0 = stack
    prefill = _run_fp8(jf, layers, x0, S)
    for chunk in (32, 1):
        print(f"unified flow: {S // chunk} calls of M = {chunk} against one prefill of M = {S}", flush=True)
        dec = _run_fp8(jf, layers, x0, chunk)
        for depth in range(LAYERS):
            diff = np.flatnonzero((dec[depth] != prefill[depth]).any(axis=1))
            assert diff.size == 0, f"M = {chunk}: tokens {diff[:8]} differ at depth {depth}"


def _oracle_block(orc, prod, Lq, x, cache):
    """One block on the CPU oracle (prefill of every token at once): bf16 bits in, bf16 bits out."""
    xq, xs, _, _, _ = prod.rmsnorm_quantize(x, Lq["n1"], EPS)
    qkv = orc.gemm_fwd(xq, xs, Lq["qkv_q"], Lq["qkv_s"], mode=orc.MFMA)
    aq, as_ = orc.quantize_rows(_attention_bits(qkv, cache, 0))
    h = _to_bf16_bits(_f32(x) + _f32(orc.gemm_fwd(aq, as_, Lq["o_q"], Lq["o_s"], mode=orc.MFMA)))
    hq, hs, _, _, _ = prod.rmsnorm_quantize(h, Lq["n2"], EPS)
    gu = orc.gemm_fwd(hq, hs, Lq["gu_q"], Lq["gu_s"], mode=orc.MFMA)
    sq, ss, _ = prod.swiglu_quantize(gu)
    return _to_bf16_bits(_f32(h) + _f32(orc.gemm_fwd(sq, ss, Lq["dn_q"], Lq["dn_s"], mode=orc.MFMA)))


def test_prefill_hidden_states_equal_the_oracle_stack(stack, orc):
    """The GPU prefill (M = 96) against the same three blocks run through the CPU oracle from the same bf16
    weights and inputs: every hidden state bitwise equal at every depth."""
    import torch
    from oracle import producers as prod
    jf, layers, x0 = stack
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    gpu = _run_fp8(jf, layers, x0, S)
    x = bits(x0)
    for depth, L in enumerate(layers):
        Lq = {"n1": bits(L["n1"]), "n2": bits(L["n2"])}
        for k in ("qkv", "o", "gu", "dn"):
            Lq[k + "_q"], Lq[k + "_s"] = orc.quantize_blocks(bits(L["w_" + k]))
            assert np.array_equal(Lq[k + "_q"], L[k + "_q"].cpu().numpy()), (depth, k, "weight codes")
        x = _oracle_block(orc, prod, Lq, x, {"K": [], "V": []})
        diff = np.flatnonzero((x.view(np.int16) != gpu[depth]).any(axis=1))
        print(f"depth {depth}: GPU prefill vs oracle stack, {diff.size} of {S} token rows differ", flush=True)
        assert diff.size == 0, f"depth {depth}: tokens {diff[:8]} differ from the oracle"


def test_fp8_block_error_against_bf16(stack):
    """Each block fed the same input on both sides (teacher forcing): the FP8 block's residual update differs
    from the bf16 one by the quantization error of its FP8 linears, a few percent in relative Frobenius norm
    (E4M3 keeps 3 fraction bits: a relative rounding error of at most 2^-4 per operand element), and that
    error does not grow with depth.  Run free, the end-to-end distance is printed, not bounded."""
    import torch
    jf, layers, x0 = stack
    per_block = []
    x = x0
    for L in layers:
        y8 = _fp8_block(jf, L, x, {"K": [], "V": []}, 0).float() - x.float()
        yr = _bf16_block(L, x, {"K": [], "V": []}, 0).float() - x.float()
        per_block.append(float((y8 - yr).norm() / yr.norm()))
        x = (x.float() + yr).to(torch.bfloat16)                        # continue on the bf16 trajectory
    x8, xr = x0, x0
    free = []
    for L in layers:
        x8 = _fp8_block(jf, L, x8, {"K": [], "V": []}, 0)
        xr = _bf16_block(L, xr, {"K": [], "V": []}, 0)
        free.append(float((x8.float() - xr.float()).norm() / xr.float().norm()))
    print("per-block relative error (teacher-forced):", [f"{r:.3e}" for r in per_block], flush=True)
    print("free-running relative distance by depth:", [f"{r:.3e}" for r in free], flush=True)
    assert all(np.isfinite(per_block)) and all(np.isfinite(free))
    assert max(per_block) < 0.08, per_block
    assert max(per_block) < 1.5 * min(per_block), per_block
