"""GPU parity of the block-scaled FP8 GEMMs (forward, dgrad, wgrad) against the oracle, plus the
kernel-level unified-flow property: an output row's bits do not depend on how many rows are computed.

Tolerance: against the plain definition (the oracle's EXACT mode, each group's dot product the fp32 rounding
of its exact sum), relative Frobenius error <= 1e-3 and max |error| <= 1e-2 * rms(out) over the outputs that
are not single-bf16-ulp rounding flips (the raw max-abs, flips included, is printed).  Separately, as a
hardware-model check, the outputs are bitwise equal to the oracle's matrix-instruction mode (see
conftest.check_gemm_parity).
"""
import numpy as np
import pytest

from conftest import bits_to_dev, check_gemm_parity, dev_to_bits, f32_to_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jf():
    import torch
    import fp8_precision_rl_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.load_library()
    return m


def _x(M, K, seed, frac=0.01):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, int(round(frac * K))), replace=False)] *= 50
    return f32_to_bits(x)


def _w(N, K, seed):
    rng = np.random.default_rng(seed)
    return f32_to_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))


def _dy(M, N, seed):
    rng = np.random.default_rng(seed)
    return f32_to_bits((rng.standard_t(3, (M, N)) * 1e-3).astype(np.float32))


@pytest.mark.parametrize("M,N,K", [(64, 256, 512), (300, 384, 640), (1, 128, 128), (129, 256, 1024)])
def test_forward_parity(jf, orc, M, N, K):
    import torch
    xb, wb = _x(M, K, M + K), _w(N, K, N + K)
    wq, ws, _ = jf.quantize_blocks(bits_to_dev(wb))
    y, _ = jf.linear_forward(bits_to_dev(xb), wq, ws)
    torch.cuda.synchronize()
    oxq, oxs = orc.quantize_rows(xb)
    owq, ows = orc.quantize_blocks(wb)
    got = dev_to_bits(y)
    check_gemm_parity(f"fwd {M}x{N}x{K}", got, orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.MFMA),
                   orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.EXACT))


@pytest.mark.parametrize("M,N,K", [(64, 256, 512), (300, 384, 256)])
def test_dgrad_parity(jf, orc, M, N, K):
    import torch
    dyb, wb = _dy(M, N, M + N), _w(N, K, N + K + 1)
    wq, ws, wqT = jf.quantize_blocks(bits_to_dev(wb))
    dyq, dys = jf.quantize_rows(bits_to_dev(dyb))
    dx = jf.gemm_dgrad(dyq, dys, wqT, ws)
    torch.cuda.synchronize()
    odq, ods = orc.quantize_rows(dyb)
    owq, ows = orc.quantize_blocks(wb)
    check_gemm_parity(f"dgrad {M}x{N}x{K}", dev_to_bits(dx), orc.gemm_dgrad(odq, ods, owq, ows, mode=orc.MFMA),
                   orc.gemm_dgrad(odq, ods, owq, ows, mode=orc.EXACT))


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (384, 128, 384)])
def test_wgrad_parity(jf, orc, M, N, K):
    import torch
    dyb, xb = _dy(M, N, M + N + 2), _x(M, K, M + K + 3)
    dyqT, dysT = jf.quantize_cols_t(bits_to_dev(dyb))
    xqT, xsT = jf.quantize_cols_t(bits_to_dev(xb))
    dw = jf.gemm_wgrad(dyqT, dysT, xqT, xsT)
    torch.cuda.synchronize()
    odq, ods = orc.quantize_cols(dyb)
    oxq, oxs = orc.quantize_cols(xb)
    check_gemm_parity(f"wgrad {M}x{N}x{K}", dev_to_bits(dw), orc.gemm_wgrad(odq, ods, oxq, oxs, mode=orc.MFMA),
                   orc.gemm_wgrad(odq, ods, oxq, oxs, mode=orc.EXACT))


def test_rows_are_bitwise_independent_of_M(jf):
    """Decode (M=1), decode batches (M=20, 32, 48, 64: the small-M kernel with 1, 2 and 4 row tiles; M=96, 128: the
    small-M kernel on rows 0-63 and then on the rest, fewer output columns than contraction) and a training batch
    (M=300: 128 x 128 quarter tiles) produce bitwise identical rows."""
    import torch
    M, N, K = 300, 256, 512
    xb, wb = _x(M, K, 41), _w(N, K, 42)
    wq, ws, _ = jf.quantize_blocks(bits_to_dev(wb))
    x = bits_to_dev(xb)
    y_all, _ = jf.linear_forward(x, wq, ws)
    batches = {m: jf.linear_forward(x[100:100 + m].contiguous(), wq, ws)[0] for m in (20, 32, 48, 64, 96, 128)}
    ones = [jf.linear_forward(x[r:r + 1].contiguous(), wq, ws)[0] for r in (0, 131, 299)]
    torch.cuda.synchronize()
    full = dev_to_bits(y_all)
    for m, yb in batches.items():
        assert np.array_equal(dev_to_bits(yb), full[100:100 + m]), f"M={m}"
    for r, y1 in zip((0, 131, 299), ones):
        assert np.array_equal(dev_to_bits(y1)[0], full[r])


def test_dgrad_equals_forward_on_transposed_blocks(jf):
    import torch
    M, N, K = 96, 256, 384
    dyb, wb = _dy(M, N, 51), _w(N, K, 52)
    wq, ws, wqT = jf.quantize_blocks(bits_to_dev(wb))
    dyq, dys = jf.quantize_rows(bits_to_dev(dyb))
    dx = jf.gemm_dgrad(dyq, dys, wqT, ws)
    dx_fwd = jf.gemm_fwd(dyq, dys, wqT, ws.t().contiguous())
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_bits(dx), dev_to_bits(dx_fwd))


def test_repeat_runs_are_bitwise_identical(jf):
    import torch
    M, N, K = 256, 512, 1024
    xb, wb = _x(M, K, 61), _w(N, K, 62)
    wq, ws, _ = jf.quantize_blocks(bits_to_dev(wb))
    x = bits_to_dev(xb)
    outs = [dev_to_bits(jf.linear_forward(x, wq, ws)[0]) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("m_small", [1, 17, 33, 100, 128])
def test_decode_ragged_chunks_many_slices(jf, orc, m_small):
    """Small-M kernel (1, 2 and 4 row tiles) on a contraction of 11 groups (a full chunk of 8 and a partial
    one of 3) and 520 column slices (more than the persistent blocks, so the operand stream crosses slice
    boundaries); 100 and 128 rows run on the upper 128 x 128 quarter tiles (more output columns than
    contraction).  Forward and DGrad rows are bitwise equal to the same rows of a 300-row call, and the forward
    matches the oracle within the stated tolerance."""
    import torch
    big, n_wide, k_ragged = 300, 8320, 1408
    xb, wb = _x(big, k_ragged, 71), _w(n_wide, k_ragged, 72)
    wq, ws, _ = jf.quantize_blocks(bits_to_dev(wb))
    x = bits_to_dev(xb)
    y_big, _ = jf.linear_forward(x, wq, ws)
    y_small, _ = jf.linear_forward(x[:m_small].contiguous(), wq, ws)
    # DGrad: the contraction (N) is the ragged one, the output columns (K) the wide one
    dyb, w2b = _dy(big, k_ragged, 73), _w(k_ragged, n_wide, 74)
    w2q, w2s, w2qT = jf.quantize_blocks(bits_to_dev(w2b))
    dyq, dys = jf.quantize_rows(bits_to_dev(dyb))
    dx_big = jf.gemm_dgrad(dyq, dys, w2qT, w2s)
    dyq_s, dys_s = jf.quantize_rows(bits_to_dev(dyb[:m_small]))
    dx_small = jf.gemm_dgrad(dyq_s, dys_s, w2qT, w2s)
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_bits(y_small), dev_to_bits(y_big)[:m_small])
    assert np.array_equal(dev_to_bits(dx_small), dev_to_bits(dx_big)[:m_small])
    oxq, oxs = orc.quantize_rows(xb[:m_small])
    owq, ows = orc.quantize_blocks(wb)
    check_gemm_parity(f"decode fwd {m_small}x{n_wide}x{k_ragged}", dev_to_bits(y_small),
                   orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.MFMA), orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.EXACT))


def test_degenerate_groups_fwd_dgrad_wgrad(jf, orc):
    """All-zero activation rows and groups (scale 0), an all-zero 128x128 weight block, negative zeros and
    full-scale groups (every element +-amax) in the forward, DGrad and WGrad GEMMs on the large-tile and the
    small-M kernels: outputs equal the oracle's (matrix-instruction mode) bit for bit, and rows whose
    activations are all zero come out as +0."""
    import torch
    M, N, K = 200, 384, 512
    x = np.random.default_rng(81).standard_normal((M, K)).astype(np.float32)
    x[5] = 0.0                                   # an all-zero row
    x[7, 128:256] = -0.0                         # a group of negative zeros
    x[9, 256:384] = np.where(np.arange(128) % 2 == 0, 3.0, -3.0)   # every element at +-amax
    x[:, 384:512][x[:, 384:512] < -1.0] = 0.0    # sparse tail groups
    w = (np.random.default_rng(82).standard_normal((N, K)) * 0.02).astype(np.float32)
    w[128:256, 0:128] = 0.0                      # an all-zero weight block
    xb, wb = f32_to_bits(x), f32_to_bits(w)
    dyb = f32_to_bits(np.where(np.arange(N) < 128, 0.0, np.random.default_rng(83).standard_t(3, (M, N)) * 1e-3)
                      .astype(np.float32))       # dY's first 128 columns all zero (one zero group per row)
    wq, ws, wqT = jf.quantize_blocks(bits_to_dev(wb))
    owq, ows = orc.quantize_blocks(wb)
    for m in (M, 24):                            # large-tile kernel, then the small-M kernel
        y, _ = jf.linear_forward(bits_to_dev(xb[:m]), wq, ws)
        dyq, dys = jf.quantize_rows(bits_to_dev(dyb[:m]))
        dx = jf.gemm_dgrad(dyq, dys, wqT, ws)
        torch.cuda.synchronize()
        oxq, oxs = orc.quantize_rows(xb[:m])
        odq, ods = orc.quantize_rows(dyb[:m])
        assert np.array_equal(dev_to_bits(y), orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.MFMA)), m
        assert np.array_equal(dev_to_bits(dx), orc.gemm_dgrad(odq, ods, owq, ows, mode=orc.MFMA)), m
        assert not dev_to_bits(y)[5].any()
    xqT, xsT = jf.quantize_cols_t(bits_to_dev(xb[:M // 128 * 128]))
    dyqT, dysT = jf.quantize_cols_t(bits_to_dev(dyb[:M // 128 * 128]))
    dw = jf.gemm_wgrad(dyqT, dysT, xqT, xsT)
    torch.cuda.synchronize()
    odc, odsc = orc.quantize_cols(dyb[:M // 128 * 128])
    oxc, oxsc = orc.quantize_cols(xb[:M // 128 * 128])
    got = dev_to_bits(dw)
    assert np.array_equal(got, orc.gemm_wgrad(odc, odsc, oxc, oxsc, mode=orc.MFMA))
    assert not got[:128].any()                   # dW rows of the all-zero dY columns


def _tiles_and_rounds(M, N):
    T = ((M + 255) // 256) * ((N + 255) // 256)
    return T, T % 256


def test_large_tiles_and_tail_round_equal_quarter_tiles(jf, orc):
    """Schedules of the large-M kernels against each other, bit for bit (each output element goes through the same
    operation sequence in all of them):
      * M = 8192, N = 2048: 256 tiles of 256 x 256, one full round (no quarter tiles);
      * M = 4352, N = 4096: 272 tiles, one full round and a last round of 16 tiles run as 64 quarter tiles;
    both against the same rows computed 128 at a time (quarter tiles only) and, on sampled rows, the oracle."""
    import torch
    K = 512
    for M, N, seed in ((8192, 2048, 91), (4352, 4096, 93)):
        T, R = _tiles_and_rounds(M, N)
        print(f"M={M} N={N}: {T} tiles of 256 x 256, last round {R}", flush=True)
        xb, wb = _x(M, K, seed), _w(N, K, seed + 1)
        wq, ws, _ = jf.quantize_blocks(bits_to_dev(wb))
        x = bits_to_dev(xb)
        y, (xq, xs) = jf.linear_forward(x, wq, ws)
        parts = [jf.gemm_fwd(xq[r:r + 128].contiguous(), xs[:, r:r + 128].contiguous(), wq, ws) for r in range(0, M, 128)]
        torch.cuda.synchronize()
        full = dev_to_bits(y)
        assert np.array_equal(full, np.concatenate([dev_to_bits(p) for p in parts])), (M, N)
        rows = np.array([0, 1, 2047, M - 129, M - 1])
        oxq, oxs = orc.quantize_rows(xb[rows])
        owq, ows = orc.quantize_blocks(wb)
        check_gemm_parity(f"large-M fwd {M}x{N}x{K} sampled rows", full[rows],
                          orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.MFMA), orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.EXACT))
        del y, parts, x


def test_wgrad_tail_round_equal_row_slabs(jf, orc):
    """WGrad with N = 4352, K = 4096 (272 tiles: a full round and 16 tiles as quarter tiles) against the same dW
    rows computed 128 at a time (quarter tiles only), bit for bit, and sampled dW rows against the oracle."""
    import torch
    M, N, K = 256, 4352, 4096
    dyb, xb = _dy(M, N, 95), _x(M, K, 96)
    dyqT, dysT = jf.quantize_cols_t(bits_to_dev(dyb))
    xqT, xsT = jf.quantize_cols_t(bits_to_dev(xb))
    dw = jf.gemm_wgrad(dyqT, dysT, xqT, xsT)
    slabs = [jf.gemm_wgrad(dyqT[n:n + 128].contiguous(), dysT[:, n:n + 128].contiguous(), xqT, xsT)
             for n in range(0, N, 128)]
    torch.cuda.synchronize()
    full = dev_to_bits(dw)
    assert np.array_equal(full, np.concatenate([dev_to_bits(p) for p in slabs]))
    rows = np.array([0, 129, N - 1])
    odq, ods = orc.quantize_cols(dyb)
    oxq, oxs = orc.quantize_cols(xb)
    check_gemm_parity(f"wgrad {M}x{N}x{K} sampled dW rows", full[rows],
                      orc.gemm_wgrad(odq, ods, oxq, oxs, rows=rows, mode=orc.MFMA),
                      orc.gemm_wgrad(odq, ods, oxq, oxs, rows=rows, mode=orc.EXACT))


@pytest.mark.parametrize("K", [128, 1152])
def test_alternating_phase_kernel_edges(jf, orc, K):
    """Forward and DGrad on 256 x 256 tiles (the alternating-phase schedule) at M = 20000 rows (79 row tiles, the
    last 32 rows deep) and 1152 output columns (5 column tiles, the last 128 wide): 395 tiles, so blocks take one or
    two tiles.  Forward contracts over K: one group (K = 128: a tile's first and last group coincide, so its rows
    are stored across the next tile's phases) or nine.  DGrad contracts over the 1152 columns (nine groups) into K
    outputs: at K = 1152 the same 395 tiles; at K = 128, 79 tiles on the quarter-tile schedule.  Bit for bit
    against the same rows computed 128 at a time (the quarter-tile schedule) and, on sampled rows, against the
    oracle."""
    import torch
    M, N = 20000, 1152
    T, R = _tiles_and_rounds(M, N)
    print(f"M={M} N={N} K={K}: {T} tiles of 256 x 256, last round {R} (no quarter-tile tail)", flush=True)
    assert T > 256 and 2 * R > 256
    xb, wb, dyb = _x(M, K, 201 + K), _w(N, K, 202 + K), _dy(M, N, 203 + K)
    wq, ws, wqT = jf.quantize_blocks(bits_to_dev(wb))
    xq, xs = jf.quantize_rows(bits_to_dev(xb))
    y = jf.gemm_fwd(xq, xs, wq, ws)
    y_parts = [jf.gemm_fwd(xq[r:r + 128].contiguous(), xs[:, r:r + 128].contiguous(), wq, ws) for r in range(0, M, 128)]
    # DGrad: dY [M, N] against W [N, K]; its 1x128 groups run along N
    dyq, dys = jf.quantize_rows(bits_to_dev(dyb))
    dx = jf.gemm_dgrad(dyq, dys, wqT, ws)
    dx_parts = [jf.gemm_dgrad(dyq[r:r + 128].contiguous(), dys[:, r:r + 128].contiguous(), wqT, ws)
                for r in range(0, M, 128)]
    torch.cuda.synchronize()
    yb, dxb = dev_to_bits(y), dev_to_bits(dx)
    assert np.array_equal(yb, np.concatenate([dev_to_bits(p) for p in y_parts])), ("fwd", K)
    assert np.array_equal(dxb, np.concatenate([dev_to_bits(p) for p in dx_parts])), ("dgrad", K)
    rows = np.array([0, 255, 256, 9999, M - 33, M - 32, M - 1])
    owq, ows = orc.quantize_blocks(wb)
    oxq, oxs = orc.quantize_rows(xb[rows])
    check_gemm_parity(f"alternating-phase fwd {M}x{N}x{K} sampled rows", yb[rows],
                      orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.MFMA), orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.EXACT))
    odq, ods = orc.quantize_rows(dyb[rows])
    check_gemm_parity(f"alternating-phase dgrad {M}x{N}x{K} sampled rows", dxb[rows],
                      orc.gemm_dgrad(odq, ods, owq, ows, mode=orc.MFMA),
                      orc.gemm_dgrad(odq, ods, owq, ows, mode=orc.EXACT))
