"""Rollout decode over fragment-ordered weights (JETFP8_BLOCKS_128x128_FRAG + jetfp8_gemm_fwd_frag).

The fragment order is a pure permutation of the 128x128 block codes (Jet-RL explainers, "Schema de Quantification":
weights in 128x128 blocks), chosen so the small-M GEMM kernel reads whole 128-byte lines.  Checked here:
  * the quantizer's fragment-ordered codes equal the oracle's row-major block codes moved by the permutation the
    header states (computed independently with numpy index arithmetic), and its scales and transposed codes equal
    the row-major mode's;
  * jetfp8_gemm_fwd_frag is bitwise equal to jetfp8_gemm_fwd on the row-major codes for every small-M row-tile
    count (1, 16, 17, 32, 33, 64 rows), on a ragged contraction (11 groups) with more column slices than blocks and
    on a Llama-3-8B-shaped linear, and matches the oracle;
  * the small-M schedules for fragment-ordered weights (wide outputs: a wave per slice, the activations in LDS at
    once or in windows; fewer slices: a block per one or two slices, or producer and consumer waves; otherwise the
    slice-sharing schedule) each equal the row-major call bitwise and the oracle on sampled column blocks;
  * more than 64 rows is a shape error.
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


def _frag_index(N, K):
    """Destination byte of each row-major code (n, k) in the fragment order."""
    n = np.arange(N, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    return (((n // 16) * (K // 128) + k // 128) * 2048 + ((k % 32) // 16) * 1024 + 16 * (n % 16 + 16 * ((k % 128) // 32))
            + k % 16)


def _w(N, K, seed):
    rng = np.random.default_rng(seed)
    return f32_to_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))


def _x(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.integers(K)] *= 50
    return f32_to_bits(x)


def test_frag_index_is_a_permutation():
    for N, K in ((128, 128), (256, 1408), (384, 512)):
        idx = _frag_index(N, K).ravel()
        assert np.array_equal(np.sort(idx), np.arange(N * K))


@pytest.mark.parametrize("N,K", [(256, 1408), (384, 512)])
def test_frag_codes_are_the_permuted_block_codes(jf, orc, N, K):
    import torch
    wb = _w(N, K, N + K)
    w = bits_to_dev(wb)
    qf, sf = jf.quantize_blocks_frag(w)
    q, s, qT = jf.quantize_blocks(w)
    qTf = torch.empty_like(qT)
    jf.jetfp8_quantize(w, N, K, jf.BLOCKS_128x128_FRAG, torch.empty_like(q), torch.empty_like(s), qTf)
    torch.cuda.synchronize()
    oq, os_ = orc.quantize_blocks(wb)
    want = np.empty(N * K, np.uint8)
    want[_frag_index(N, K).ravel()] = oq.ravel()
    assert np.array_equal(qf.cpu().numpy().ravel(), want)
    assert np.array_equal(sf.cpu().numpy(), os_) and torch.equal(sf, s)
    assert torch.equal(qTf, qT)


@pytest.mark.parametrize("N,K", [(8320, 1408), (6144, 4096)])
def test_frag_gemm_equals_row_major_gemm(jf, orc, N, K):
    import torch
    wb = _w(N, K, 7 + N)
    w = bits_to_dev(wb)
    wq, ws = jf.quantize_blocks(w, transposed=False)
    wqf, wsf = jf.quantize_blocks_frag(w)
    xb = _x(64, K, 8 + K)
    x = bits_to_dev(xb)
    for M in (1, 16, 17, 32, 33, 64):
        xq, xs = jf.quantize_rows(x[:M].contiguous())
        y = jf.gemm_fwd(xq, xs, wq, ws)
        yf = jf.gemm_fwd_frag(xq, xs, wqf, wsf)
        torch.cuda.synchronize()
        assert np.array_equal(dev_to_bits(yf), dev_to_bits(y)), (N, K, M)
    oxq, oxs = orc.quantize_rows(xb[:33])
    owq, ows = orc.quantize_blocks(wb)
    xq, xs = jf.quantize_rows(x[:33].contiguous())
    yf = jf.gemm_fwd_frag(xq, xs, wqf, wsf)
    torch.cuda.synchronize()
    check_gemm_parity(f"fwd_frag 33x{N}x{K}", dev_to_bits(yf), orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.MFMA),
                      orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.EXACT))


def test_frag_gemm_rejects_more_than_64_rows(jf):
    import torch
    N, K, M = 256, 512, 65
    wqf = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    ws = torch.ones((N // 128, K // 128), dtype=torch.float32, device="cuda")
    xq = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.ones((K // 128, M), dtype=torch.float32, device="cuda")
    with pytest.raises(jf.JetFP8Error) as e:
        jf.gemm_fwd_frag(xq, xs, wqf, ws)
    assert e.value.status == jf.ERR_SHAPE


@pytest.mark.parametrize("M", [1, 16, 17, 32])
def test_wide_schedule_equals_row_major(jf, orc, M):
    """Gate/up-shaped forward (28672 output columns, 1792 slices, K = 4096) over fragment-ordered weights runs the
    wide small-M schedule (each wave owns whole slices, activations held in LDS): bitwise equal to the row-major
    weights on the slice-sharing schedule, and sampled columns against the oracle."""
    import torch
    N, K = 28672, 4096
    wb = _w(N, K, 11 + M)
    w = bits_to_dev(wb)
    wq, ws = jf.quantize_blocks(w, transposed=False)
    wqf, wsf = jf.quantize_blocks_frag(w)
    xb = _x(M, K, 12 + M)
    xq, xs = jf.quantize_rows(bits_to_dev(xb))
    y = jf.gemm_fwd(xq, xs, wq, ws)
    yf = jf.gemm_fwd_frag(xq, xs, wqf, wsf)
    torch.cuda.synchronize()
    yb, yfb = dev_to_bits(y), dev_to_bits(yf)
    assert np.array_equal(yfb, yb), M
    cols = np.r_[0:128, 14336:14464, N - 128:N]
    oxq, oxs = orc.quantize_rows(xb)
    owq, ows = orc.quantize_blocks(wb[cols])
    check_gemm_parity(f"wide decode {M}x{N}x{K} sampled column blocks", yfb[:, cols],
                      orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.MFMA), orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.EXACT))


@pytest.mark.parametrize("M,N,K", [
    (1, 4096, 4096),      # one slice per block, one round of 32 groups, 16-row tile
    (16, 6144, 4096),     # more slices than CUs, 16-row tile: still one slice per block
    (17, 4096, 4096),     # 32-row tile (row-contiguous activation loads), one slice per block
    (32, 6144, 4096),     # more slices than CUs, 32-row tile: two slices per block
    (29, 2048, 640),      # 5 groups: three waves of the round idle
    (32, 4096, 14336),    # down projection: producer and consumer waves, 14 rounds of 8 groups
    (5, 1024, 4736),      # 37 groups (producers and consumers): a ragged last round (5 groups)
    (32, 128, 16384),     # 128 groups, the most the per-slice schedules take; 8 slices
    (32, 256, 16512),     # 129 groups: back on the slice-sharing schedule
    (17, 6144, 8192),     # 64 groups, 1.5 slices per CU (on 256 CUs): producer and consumer waves
    (32, 8192, 8192),     # 64 groups, 2 slices per CU: producer and consumer waves
    (32, 8192, 5120),     # 40 groups, 2 slices per CU: the slice-sharing schedule
    (16, 12288, 5120),    # 40 groups, 3 slices per CU, too few for the wide schedule: the slice-sharing schedule
    (48, 4096, 14336),    # 48 rows (4 row tiles), 112 groups: producer and consumer waves, two outputs per consumer
    (64, 4096, 4096),     # 64 rows, 32 groups, one slice per CU: producer and consumer waves
    (40, 2048, 640),      # 40 rows, 5 groups: one ragged round, rows 40-63 empty
    (48, 6144, 4096),     # 48 rows, 1.5 slices per CU and 32 groups: producer and consumer waves
    (48, 12288, 4096),    # 48 rows, 3 slices per CU, too few for the wide schedules: the slice-sharing schedule
])
def test_per_slice_schedule_equals_row_major(jf, orc, M, N, K):
    """Forward GEMMs with fewer 16-column slices than the wide schedule needs (QKV, O, down shapes) run the
    per-slice small-M schedules over fragment-ordered weights (up to 32 groups: a block per one or two slices, the
    groups dealt out to the waves, products promoted after one barrier; longer contractions: producer waves form
    rounds of 8 group products while consumer waves promote the round before): bitwise equal to the row-major
    weights on the slice-sharing schedule, and the first and last column blocks against the oracle."""
    import torch
    wb = _w(N, K, 21 + M + N)
    w = bits_to_dev(wb)
    wq, ws = jf.quantize_blocks(w, transposed=False)
    wqf, wsf = jf.quantize_blocks_frag(w)
    del w
    xb = _x(M, K, 22 + M)
    xq, xs = jf.quantize_rows(bits_to_dev(xb))
    y = jf.gemm_fwd(xq, xs, wq, ws)
    yf = jf.gemm_fwd_frag(xq, xs, wqf, wsf)
    torch.cuda.synchronize()
    yb, yfb = dev_to_bits(y), dev_to_bits(yf)
    assert np.array_equal(yfb, yb), (M, N, K)
    cols = np.r_[0:128, N - 128:N] if N > 128 else np.r_[0:128]
    oxq, oxs = orc.quantize_rows(xb)
    owq, ows = orc.quantize_blocks(wb[cols])
    check_gemm_parity(f"per-slice decode {M}x{N}x{K} first/last column blocks", yfb[:, cols],
                      orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.MFMA), orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.EXACT))


@pytest.mark.parametrize("M,N,K", [
    (48, 16384, 4096),    # 48 rows (4 row tiles), at least 4 slices per CU: activation windows
    (64, 16384, 1152),    # 64 rows, 9 groups: a ragged last window (6 + 3)
    (32, 16384, 5120),    # 32 rows whose activations (160 KB) do not fit in LDS at once
    (3, 16384, 8320),     # 65 groups, too many for the unwindowed wide schedule, at 3 rows
    (33, 16384, 2048),    # 33 rows: 4 row tiles, rows 33-63 empty
])
def test_windowed_wide_schedule_equals_row_major(jf, orc, M, N, K):
    """Wide outputs whose activations do not fit in LDS at once (more than 32 rows, or a long contraction) run the
    wide small-M schedule with the activations streamed through LDS in windows of 6 groups: bitwise equal to the
    row-major weights on the slice-sharing or large-tile schedules, and the first and last column blocks against
    the oracle."""
    import torch
    wb = _w(N, K, 31 + M + K)
    w = bits_to_dev(wb)
    wq, ws = jf.quantize_blocks(w, transposed=False)
    wqf, wsf = jf.quantize_blocks_frag(w)
    del w
    xb = _x(M, K, 32 + M)
    xq, xs = jf.quantize_rows(bits_to_dev(xb))
    y = jf.gemm_fwd(xq, xs, wq, ws)
    yf = jf.gemm_fwd_frag(xq, xs, wqf, wsf)
    torch.cuda.synchronize()
    yb, yfb = dev_to_bits(y), dev_to_bits(yf)
    assert np.array_equal(yfb, yb), (M, N, K)
    cols = np.r_[0:128, N - 128:N]
    oxq, oxs = orc.quantize_rows(xb)
    owq, ows = orc.quantize_blocks(wb[cols])
    check_gemm_parity(f"windowed wide decode {M}x{N}x{K} first/last column blocks", yfb[:, cols],
                      orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.MFMA), orc.gemm_fwd(oxq, oxs, owq, ows, mode=orc.EXACT))
