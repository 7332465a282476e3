"""Every entry point writes only inside its outputs.  Each output buffer sits between two 4 KiB canary regions
(byte 0xA5) of one allocation; after the call the canaries must be intact and the output must equal that of the
same call on plain tensors.  Shapes are ragged where the ABI allows it (token counts that are not a multiple of
the tiles, a column count that leaves half a 256-wide GEMM tile, a 128x1 width that is a multiple of 64 only),
and the GEMMs run on both the small-M kernel (1, 2 and 4 row tiles) and the large-tile kernel."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

PAD = 4096
CANARY = 0xA5


@pytest.fixture(scope="module")
def jf():
    import torch
    import fp8_precision_rl_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.load_library()
    return m


class Padded:
    """An output tensor inside one allocation with PAD canary bytes before and after it."""

    def __init__(self, shape, dtype):
        import torch
        self.n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((PAD + self.n + PAD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[PAD:PAD + self.n].view(dtype).view(shape)

    def intact(self):
        import torch
        torch.cuda.synchronize()
        return bool((self.buf[:PAD] == CANARY).all()) and bool((self.buf[PAD + self.n:] == CANARY).all())


def _bf16(shape, seed, scale=1.0):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn(shape, device="cuda", generator=g) * scale).to(torch.bfloat16)


def _check(name, outs, refs):
    import torch
    for i, (o, r) in enumerate(zip(outs, refs)):
        assert o.intact(), f"{name}: output {i} wrote outside its buffer"
        assert torch.equal(o.t, r), f"{name}: output {i} differs from the plain call"


@pytest.mark.parametrize("R,C", [(37, 384), (100, 640)])
def test_quantize_rows(jf, R, C):
    import torch
    x = _bf16((R, C), 1)
    q, s = Padded((R, C), torch.uint8), Padded((C // 128, R), torch.float32)
    jf.jetfp8_quantize(x, R, C, jf.ROWS_1x128, q.t, s.t)
    _check("rows", (q, s), jf.quantize_rows(x))


def test_quantize_cols_t_half_tile(jf):
    import torch
    R, C = 256, 192
    x = _bf16((R, C), 2)
    q, s = Padded((C, R), torch.uint8), Padded((R // 128, C), torch.float32)
    jf.jetfp8_quantize(x, R, C, jf.COLS_128x1_T, q.t, s.t)
    _check("cols_t", (q, s), jf.quantize_cols_t(x))


def test_quantize_blocks_dual_requant(jf):
    import torch
    R, C = 256, 384
    x = _bf16((R, C), 3)
    q, s, qT = Padded((R, C), torch.uint8), Padded((R // 128, C // 128), torch.float32), Padded((C, R), torch.uint8)
    jf.jetfp8_quantize(x, R, C, jf.BLOCKS_128x128, q.t, s.t, qT.t)
    _check("blocks", (q, s, qT), jf.quantize_blocks(x))
    d = [Padded((R, C), torch.uint8), Padded((C // 128, R), torch.float32), Padded((C, R), torch.uint8),
         Padded((R // 128, C), torch.float32)]
    jf.jetfp8_quantize_dual(x, R, C, *(p.t for p in d))
    _check("dual", d, jf.quantize_dual(x))
    xq, xs = jf.quantize_rows(x)
    rq = [Padded((C, R), torch.uint8), Padded((R // 128, C), torch.float32)]
    jf.jetfp8_requantize_cols_t(xq, xs, R, C, rq[0].t, rq[1].t)
    _check("requantize", rq, jf.requantize_cols_t(xq, xs))


def test_producers(jf):
    import torch
    R, C, F = 37, 384, 384
    x, w = _bf16((R, C), 4), (1.0 + 0.1 * _bf16((C,), 5).float()).to(torch.bfloat16)
    o = [Padded((R, C), torch.uint8), Padded((C // 128, R), torch.float32), Padded((R,), torch.float32),
         Padded((R, C), torch.bfloat16)]
    jf.jetfp8_rmsnorm_quantize(x, w, R, C, 1e-5, *(p.t for p in o))
    _check("rmsnorm", o, jf.rmsnorm_quantize(x, w, 1e-5, return_y=True))
    gu = _bf16((R, 2 * F), 6, 2.0)
    o = [Padded((R, F), torch.uint8), Padded((F // 128, R), torch.float32), Padded((R, F), torch.bfloat16)]
    jf.jetfp8_swiglu_quantize(gu, R, F, *(p.t for p in o))
    _check("swiglu", o, jf.swiglu_quantize(gu, return_h=True))


@pytest.mark.parametrize("M", [1, 20, 40, 300])
def test_gemms(jf, M):
    """M = 1, 20, 40: the small-M kernel with 1, 2 and 4 row tiles; M = 300: the large-tile kernel (a ragged
    second row of tiles).  N = 384 leaves half of the second 256-wide column tile outside the matrix."""
    import torch
    N, K = 384, 512
    x, w, dy = _bf16((M, K), 7), _bf16((N, K), 8, 0.02), _bf16((M, N), 9, 1e-3)
    wq, ws, wqT = jf.quantize_blocks(w)
    xq, xs = jf.quantize_rows(x)
    y = Padded((M, N), torch.bfloat16)
    jf.jetfp8_gemm_fwd(xq, xs, wq, ws, y.t, M, N, K)
    _check("fwd", (y,), (jf.gemm_fwd(xq, xs, wq, ws),))
    dyq, dys = jf.quantize_rows(dy)
    dx = Padded((M, K), torch.bfloat16)
    jf.jetfp8_gemm_dgrad(dyq, dys, wqT, ws, dx.t, M, N, K)
    _check("dgrad", (dx,), (jf.gemm_dgrad(dyq, dys, wqT, ws),))
    if M % 128 == 0 or M == 300:
        Mw = M // 128 * 128
        dyqT, dysT = jf.quantize_cols_t(dy[:Mw].contiguous())
        xqT, xsT = jf.quantize_cols_t(x[:Mw].contiguous())
        dw = Padded((N, K), torch.bfloat16)
        jf.jetfp8_gemm_wgrad(dyqT, dysT, xqT, xsT, dw.t, Mw, N, K)
        _check("wgrad", (dw,), (jf.gemm_wgrad(dyqT, dysT, xqT, xsT),))
