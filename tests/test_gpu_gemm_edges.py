"""GPU parity of the W4A4 product on operand bytes no encoder would produce for smooth data, on
every kernel the dispatch can choose, and on mid-size problems compared in full.

* Raw bytes (``workloads.random_nvfp4_bytes``): every E2M1 nibble including the signed zero 0x8,
  block scales drawn from all 127 finite E4M3 codes (zero, the seven subnormals 0x01..0x07, every
  normal up to 0x7E = 448), all-zero blocks made by zero codes and by a zero scale.  Each product
  kernel decodes block scales its own way (a hardware fp8 conversion in the tiled, one-pass decode
  and streaming kernels, a bit-level decode in the general one), so each is driven over the whole
  scale range: general (K % 64 != 0), tiled (every count of 64-element sub-chunks left after its
  loop over pairs of 256-element chunks), the
  one-pass decode kernel with one and two 16-column tiles per workgroup, its long-K form with one
  and two tiles and its many-column form, the streaming kernel's cached and column-pair forms, and
  K split into pieces that add into C.
* Mid-size problems compared element by element over the whole output: more tiles than compute
  units with a tile count that is not a multiple of 8 (the persistent kernel's plain tile order),
  partial edge tiles, and K ending in a lone 64-element sub-chunk (read after the last barrier,
  before the next tile's first copies are issued); larger K, where each tile also runs the loop
  over pairs of chunks, on sampled rows of every tile row.

Tolerance as everywhere (stated for FP32 accumulation of exact products): per element
``|C_gpu - C_ref| <= 1e-4 * sum_k |a*w| / (gA gW[seg])``, relative Frobenius error <= 1e-5.  The
reference is the oracle's exact int64 product of the same bytes (ai.info summary, "Methodology in
Plain English": an E4M3 scale per 16-element block of E2M1 values)."""

import numpy as np
import pytest

from workloads import random_matrix, random_nvfp4_bytes

import oracle

from .gpu_util import DEV, check_gemm, log, oracle_product, scalar

pytestmark = pytest.mark.gpu


def _up(arr):
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def _run(ac, as_, ga, wc, ws, gw, segs, what):
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    log(f"{what}: M={ac.shape[0]} N={wc.shape[0]} K={ac.shape[1] * 2}")
    C = nv.fused_nvfp4_gemm(_up(ac), _up(as_), scalar(ga), _up(wc), _up(ws),
                            _up(np.asarray(gw, np.float32)), segs)
    torch.cuda.synchronize()
    C = C.cpu().numpy()
    R, B = oracle_product(ac, as_, ga, wc, ws, gw, segs)
    worst = check_gemm(C, R, B, what)
    log(f"{what}: worst err / sum|ab| = {worst:.2e}")
    return C, R


# (M, N, K, kernel the dispatch picks)
RAW_SHAPES = [
    (40, 300, 2064, "general"),
    (33, 65, 48, "general, K = 48"),
    (300, 260, 256, "tiled 256 x 192, 4 K sub-chunks: one pass of the two-chunk loop"),
    (257, 513, 320, "tiled 256 x 192, 5 K sub-chunks: the loop, then a lone sub-chunk"),
    (129, 200, 384, "tiled 256 x 192, 6 K sub-chunks: the loop, then one whole chunk"),
    (300, 260, 448, "tiled 256 x 192, 7 K sub-chunks: the loop, a chunk and a lone sub-chunk"),
    (65, 130, 192, "tiled 256 x 192, 3 K sub-chunks: no loop pass"),
    (17, 1000, 2048, "tiled 256 x 192, 17 rows"),
    (4096, 4096, 128, "tiled 256 x 256, one full round, one K chunk"),
    (2048, 8232, 64, "tiled, split: 256 x 256 tiles over 8192 columns, 64 x 64 over the last 40"),
    (1990, 8200, 192, "tiled, split, partial last tile row in both launches, 3 K sub-chunks"),
    (1, 3000, 2048, "one-pass decode, one tile per workgroup"),
    (16, 6000, 2048, "one-pass decode, two tiles per workgroup"),
    (3, 8100, 8192, "one-pass decode, K = 8192"),
    (4, 9000, 2048, "many-column decode form"),
    (4, 9000, 8192, "streaming, cached form"),
    (2, 1000, 9216, "long-K decode, one tile per workgroup"),
    (3, 4500, 10240, "long-K decode, two tiles per workgroup"),
    (8, 4500, 10240, "long-K decode, two tiles, 8 rows"),
    (3, 8500, 10240, "streaming, column-pair form"),
    (2, 40, 33792, "K pieces adding into C"),
]


@pytest.mark.parametrize("M,N,K,path", RAW_SHAPES)
def test_raw_bytes_every_scale_code(M, N, K, path):
    ac, as_ = random_nvfp4_bytes(1000 + M + K, M, K)
    wc, ws = random_nvfp4_bytes(2000 + N + K, N, K)
    # every nibble appears in both operands, and every scale code too (the smallest shape, with
    # three blocks per row, holds only some of them)
    for c, s in ((ac, as_), (wc, ws)):
        assert len(np.unique(np.concatenate([c & 15, c >> 4]))) == 16
        assert K == 48 or len(np.unique(s)) == 0x7F
    segs = [0, N // 3, N] if N >= 3 else [0, N]
    gw = np.array([1.7, 0.03125][: len(segs) - 1], np.float32)
    _run(ac, as_, np.float32(2.5), wc, ws, gw, segs, f"raw bytes, {path}")


@pytest.mark.parametrize("M,N,K", [(300, 260, 256), (1, 3000, 1024), (4, 9000, 2048),
                                   (3, 4500, 10240), (40, 70, 80)])
def test_zero_operands_give_zero(M, N, K):
    """All-zero activations (zero scales) against random weights, and the signed-zero code 0x8
    everywhere under the largest scale: every output is exactly +0 or -0 equal to 0."""
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    wc, ws = random_nvfp4_bytes(3000 + N, N, K)
    for codes, scale in ((0x00, 0x00), (0x88, 0x7E)):
        ac = np.full((M, K // 2), codes, np.uint8)
        as_ = np.full((M, K // 16), scale, np.uint8)
        C = nv.nvfp4_gemm(_up(ac), _up(as_), scalar(1.0), _up(wc), _up(ws), scalar(3.0))
        torch.cuda.synchronize()
        assert np.all(C.cpu().numpy() == 0.0)


def test_small_scales_under_a_static_activation_scale():
    """Activations with quiet tokens: rows scaled by 1e-2, 2e-3, 5e-4 and 1e-6, and exact zero rows,
    encoded by the oracle under a static scale calibrated on the loud rows, so low and subnormal
    E4M3 block scales (codes 0x01..0x07) and underflowed (zero) blocks appear, as in zero-padded or
    quiet tokens of real prefill batches."""
    M, N, K = 96, 384, 1024
    a = random_matrix(77, M, K, outlier_cols=4, outlier_gain=100.0)
    for i, f in enumerate((1e-2, 2e-3, 5e-4, 1e-6)):
        a[1 + i::5] *= np.float32(f)
    a[2::11] = 0.0
    a[5, :16] = -0.0
    ga = oracle.dynamic_global_scale(a[0::5])
    ac, as_, _ = oracle.quantize(a, ga)
    assert (as_ == 0).mean() > 0.1 and ((as_ > 0) & (as_ < 8)).mean() > 0.1
    assert set(range(8)) <= set(np.unique(as_).tolist())
    wt = random_matrix(78, N, K, std=0.02)
    wc, ws, gw = oracle.quantize_segments(wt, [0, N])
    _run(ac, as_, ga, wc, ws, gw, [0, N], "quiet tokens, tiled")
    for m in (1, 16):  # the same rows through the decode-shaped kernels
        _run(ac[:m], as_[:m], ga, wc, ws, gw, [0, N], f"quiet tokens, {m} rows")


@pytest.mark.parametrize("M,N,K,what", [
    (2304, 8485, 128, "405 tiles of 256 x 192 (not a multiple of 8), partial last tile column"),
    (2304, 7936, 192, "378 tiles of 256 x 192, 3 K sub-chunks per tile (odd)"),
    (1100, 16400, 320, "430 tiles of 256 x 192, 5 K sub-chunks, partial last tile row"),
    (1100, 19653, 192, "385 tiles of 256 x 256, 3 K sub-chunks, partial last tile row and column"),
])
def test_mid_size_full_output(M, N, K, what):
    """Every output element of problems with more tiles than compute units, so each persistent
    workgroup runs several tiles back to back (plain tile order, since the tile count is not a
    multiple of 8), in both tile shapes the dispatch picks between, compared with the oracle."""
    a = random_matrix(90 + K, M, K, outlier_cols=3)
    wt = random_matrix(91 + K, N, K, std=0.02)
    segs = [0, N // 2 + 3, N]
    ac, as_, ga = oracle.quantize(a)
    wc, ws, gw = oracle.quantize_segments(wt, segs)
    _run(ac, as_, ga, wc, ws, gw, segs, f"full output, {what}")


def test_split_launch_full_output_and_segment_calls():
    """A problem split into two launches: 256 tiles of 256 x 256 over the first 8192 columns (one
    round) and 32 tiles of 64 x 64 over the last 40, with a module boundary inside those 40 columns
    (the second launch sees its columns' part of the segment table, rebased).  Every element is
    compared with the oracle, and the fused result equals the per-module calls (which run single
    launches of other tile shapes) bit for bit."""
    M, N, K = 2048, 8232, 320
    segs = [0, 3000, 8212, N]
    a = random_matrix(97, M, K, outlier_cols=3)
    wt = random_matrix(98, N, K, std=0.02)
    ac, as_, ga = oracle.quantize(a)
    wc, ws, gw = oracle.quantize_segments(wt, segs)
    fused, _ = _run(ac, as_, ga, wc, ws, gw, segs, "split launch, 5 K sub-chunks")
    parts = []
    for j in range(len(segs) - 1):
        lo, hi = segs[j], segs[j + 1]
        C, _ = _run(ac, as_, ga, wc[lo:hi], ws[lo:hi], gw[j:j + 1], [0, hi - lo],
                    f"split launch, module {j} alone")
        parts.append(C)
    assert np.array_equal(fused, np.concatenate(parts, axis=1))


@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_split_launch_into_output_view(odt):
    """The split launch writing into a column window of a wider buffer (row pitch N + 11 elements,
    so rows are not 16-byte aligned; window starting 8 elements in): the second launch's columns
    start at the window's column 8192.  Elements outside the window keep their sentinel; the f32
    result is within the product tolerance, the bf16 one within one more rounding."""
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    M, N, K = 2048, 8232, 64
    segs = [0, 4100, 8200, N]
    a = random_matrix(99, M, K, outlier_cols=3)
    wt = random_matrix(100, N, K, std=0.02)
    ac, as_, ga = oracle.quantize(a)
    wc, ws, gw = oracle.quantize_segments(wt, segs)
    dt = torch.float32 if odt == "f32" else torch.bfloat16
    buf = torch.full((M, N + 11), -7.0, dtype=dt, device=DEV)
    out = buf[:, 8:8 + N]
    log(f"split launch into a view ({odt}): M={M} N={N} K={K}")
    nv.fused_nvfp4_gemm(_up(ac), _up(as_), scalar(ga), _up(wc), _up(ws),
                        _up(np.asarray(gw, np.float32)), segs, out=out)
    torch.cuda.synchronize()
    hb = buf.float().cpu().numpy()
    assert np.all(hb[:, :8] == -7.0) and np.all(hb[:, 8 + N:] == -7.0)
    C = hb[:, 8:8 + N].astype(np.float64)
    R, B = oracle_product(ac, as_, ga, wc, ws, gw, segs)
    if odt == "f32":
        check_gemm(C, R, B, "split launch into a view")
    else:  # one extra rounding of the FP32 result to bf16
        assert np.all(np.abs(C - R) <= 2.0 ** -8 * np.abs(R) + 1e-4 * B)


@pytest.mark.parametrize("M,N,K,what", [
    (48, 320, 65600, "tiled, K = 65600: 128 passes of the two-chunk loop and a lone sub-chunk"),
    (40, 8232, 16448, "tiled 256 x 192, K = 16448: 32 passes of the two-chunk loop and a lone sub-chunk"),
])
def test_tiled_long_k_full_output(M, N, K, what):
    """The tiled product far along K (the longest K of the parity tests above is 17408 at full
    size): FP32 accumulation over thousands of MFMA steps stays within the tolerance, and the
    K loop's bookkeeping holds over hundreds of chunks.  Every element against the oracle."""
    a = random_matrix(101, M, K, outlier_cols=5)
    wt = random_matrix(102, N, K, std=0.02)
    segs = [0, N // 2 + 1, N]
    ac, as_, ga = oracle.quantize(a)
    wc, ws, gw = oracle.quantize_segments(wt, segs)
    _run(ac, as_, ga, wc, ws, gw, segs, what)


def test_mid_size_raw_bytes_full_output():
    M, N, K = 2304, 7936, 192
    ac, as_ = random_nvfp4_bytes(5, M, K)
    wc, ws = random_nvfp4_bytes(6, N, K)
    _run(ac, as_, np.float32(0.75), wc, ws, np.array([3.0], np.float32), [0, N],
         "raw bytes, full output, 378 tiles, odd K sub-chunks")


@pytest.mark.parametrize("M,N,K,what", [
    (2304, 7936, 576, "378 tiles of 256 x 192; per tile one pass of the two-chunk loop and a lone "
                      "sub-chunk"),
    (1100, 19653, 704, "385 tiles of 256 x 256; per tile one loop pass, a chunk and a lone "
                       "sub-chunk"),
    (2048, 8232, 704, "split: 256 tiles of 256 x 256, then 32 of 64 x 64; per tile one loop pass, "
                      "a chunk and a lone sub-chunk"),
])
def test_mid_size_loop_sampled_rows(M, N, K, what):
    """Several tiles per persistent workgroup with K long enough for the K loop itself: the GPU
    computes the whole output; the oracle checks the first and last rows of every 256-row tile
    row, and every ninth row, over all columns."""
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    a = random_matrix(95 + K, M, K, outlier_cols=3)
    wt = random_matrix(96 + K, N, K, std=0.02)
    segs = [0, N // 3 + 5, N]
    ac, as_, ga = oracle.quantize(a)
    wc, ws, gw = oracle.quantize_segments(wt, segs)
    log(f"{what}: M={M} N={N} K={K}")
    C = nv.fused_nvfp4_gemm(_up(ac), _up(as_), scalar(ga), _up(wc), _up(ws),
                            _up(np.asarray(gw, np.float32)), segs)
    torch.cuda.synchronize()
    C = C.cpu().numpy()
    bands = [r for t in range(0, M, 256) for r in (t, t + 1, min(t + 255, M - 1))]
    rows = np.unique(np.concatenate([np.arange(0, M, 9), bands, [M - 1]]))
    R, B = oracle_product(ac[rows], as_[rows], ga, wc, ws, gw, segs)
    worst = check_gemm(C[rows], R, B, f"{what}, {len(rows)} rows")
    log(f"{what}: worst err / sum|ab| = {worst:.2e}")
