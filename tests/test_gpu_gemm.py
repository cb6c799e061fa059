"""GPU parity of nvfp4_gemm and fused_nvfp4_gemm against the oracle's exact product.

Tolerance (stated for FP32 accumulation of exactly decoded products):
  |C_gpu - C_ref| <= 1e-4 * sum_k |a*w| / (gA gW[seg])  per element, and
  ||C_gpu - C_ref||_F <= 1e-5 ||C_ref||_F.
Operands are always encoded by the oracle on the host (never taken from the GPU encoder), uploaded,
and multiplied on the GPU.  Full-size workloads are checked on sampled rows and columns."""

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, activations, gate_up, random_matrix, weights

from .gpu_util import DEV, check_gemm, log, oracle_product, scalar

pytestmark = pytest.mark.gpu


def _up(arr):
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def _gpu_product(ac, as_, ga, wc, ws, seg_g, segs, out_dtype="f32"):
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    C = nv.fused_nvfp4_gemm(_up(ac), _up(as_), scalar(ga), _up(wc), _up(ws),
                            _up(np.asarray(seg_g, np.float32)), segs, out_dtype=odt)
    torch.cuda.synchronize()
    return C.float().cpu().numpy()


def _encode(a, w, segs, seg_g=None, ga=None):
    ac, as_, ga = oracle.quantize(a, ga)
    wc, ws, gw = oracle.quantize_segments(w, segs, seg_g)
    return ac, as_, ga, wc, ws, gw


def _check(ac, as_, ga, wc, ws, gw, segs, what):
    C = _gpu_product(ac, as_, ga, wc, ws, gw, segs)
    R = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, segs)
    B = oracle.gemm_abs_bound(ac, as_, ga, wc, ws, gw, segs)
    worst = check_gemm(C, R, B, what)
    log(f"{what}: worst err / sum|ab| = {worst:.2e}")
    return C, R


def test_workload1_full():
    w = WORKLOADS[1]
    a, wt = activations(w), weights(w)
    enc = _encode(a, wt, w.seg_offsets)
    _check(*enc, w.seg_offsets, "workload 1")


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 16), (1, 37, 64), (5, 70, 48), (33, 65, 80), (31, 129, 128), (64, 64, 64),
    (129, 130, 192), (200, 300, 1024), (257, 255, 320), (96, 160, 5120), (70, 90, 384),
    (65, 200, 448),
    # decode-shaped (M <= 16): the skinny kernel for K a multiple of 1024 (in pieces above 8192),
    # the tiled or general kernel otherwise
    (1, 100, 512), (3, 77, 1536), (16, 40, 1024), (7, 33, 512), (16, 16, 2048), (5, 3, 16384),
    (2, 300, 17408), (1, 19, 384),
])
def test_ragged_shapes(M, N, K):
    a = random_matrix(M * 7 + K, M, K, outlier_cols=max(1, K // 100))
    wt = random_matrix(N * 5 + K, N, K, std=0.02)
    enc = _encode(a, wt, [0, N])
    _check(*enc, [0, N], f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 48, 9216), (16, 320, 17408), (7, 130, 15360), (4, 40, 31744),
                                   (2, 40, 33792), (3, 50, 65536)])
def test_decode_long_k(M, N, K):
    # at most 16 rows and K above 8192, at most 16 columns per compute unit: the decode kernel's
    # long-K form up to K = 32768 (9 to 31 phases of 1024), beyond that pieces of at most 8 phases
    # (5 at K = 33792, 8 at K = 65536) through the streaming kernel's cached form, each later piece
    # adding into C; three fused modules
    a = random_matrix(M * 11 + K, M, K, outlier_cols=max(1, K // 200))
    wt = random_matrix(N * 3 + K, N, K, std=0.02)
    segs = [0, N // 3, N // 2, N]
    _check(*_encode(a, wt, segs), segs, f"long K M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 9000, 2048), (16, 8250, 1024), (5, 12345, 3072),
                                   (3, 8500, 4096), (16, 8250, 8192)])
def test_decode_many_columns(M, N, K):
    # more than 32 columns per compute unit: the decode kernel's many-column form walks several
    # 16-column tiles per workgroup (ragged last tile) up to 5 phases of K, the streaming kernel's
    # cached form beyond (8 phases), two fused modules
    a = random_matrix(M * 13 + N, M, K, outlier_cols=3)
    wt = random_matrix(N + K, N, K, std=0.02)
    segs = [0, N // 2 + 5, N]
    _check(*_encode(a, wt, segs), segs, f"many columns M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(3, 4200, 9216), (16, 8250, 10240), (1, 5120, 17408),
                                   (2, 4500, 10240), (16, 5120, 17408), (5, 4500, 10240)])
def test_decode_even_column_share(M, N, K):
    # K above 8192 and more than 16 columns per compute unit (256 of them): workgroups own equal
    # column ranges (17 columns and a last workgroup of one; 33; 20, the MLP down projection's
    # shape; 18), three fused modules.  Up to 32 columns: the decode kernel's long-K form with two
    # tiles; 33 columns: the streaming kernel's column-pair form, groups of 32 columns whose 20
    # units of one group-phase end in a closing run of 2 units
    a = random_matrix(M * 17 + N, M, K, outlier_cols=max(1, K // 300))
    wt = random_matrix(N * 5 + K, N, K, std=0.02)
    segs = [0, N // 3 + 7, N // 2 + 1, N]
    _check(*_encode(a, wt, segs), segs, f"even column share M={M} N={N} K={K}")


def test_decode_even_column_share_bf16_output():
    # the same form with bf16 C (one rounding of the FP32 result)
    a = random_matrix(81, 5, 9216, outlier_cols=30)
    wt = random_matrix(82, 4500, 9216, std=0.02)
    ac, as_, ga, wc, ws, gw = _encode(a, wt, [0, 4500])
    C = _gpu_product(ac, as_, ga, wc, ws, gw, [0, 4500], out_dtype="bf16")
    R = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, [0, 4500])
    assert np.all(np.abs(C - R) <= 2.0 ** -8 * np.abs(R) + 1e-4 * oracle.gemm_abs_bound(
        ac, as_, ga, wc, ws, gw, [0, 4500]))


def test_decode_long_k_bf16_output():
    # bf16 C with a long K: the long-K decode form (one pass over K, so no partial sums are rounded)
    a = random_matrix(71, 3, 17408, outlier_cols=40)
    wt = random_matrix(72, 96, 17408, std=0.02)
    ac, as_, ga, wc, ws, gw = _encode(a, wt, [0, 96])
    C = _gpu_product(ac, as_, ga, wc, ws, gw, [0, 96], out_dtype="bf16")
    R = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, [0, 96])
    assert np.all(np.abs(C - R) <= 2.0 ** -8 * np.abs(R) + 1e-4 * oracle.gemm_abs_bound(
        ac, as_, ga, wc, ws, gw, [0, 96]))


def test_bf16_output():
    a = random_matrix(3, 100, 256, outlier_cols=3)
    wt = random_matrix(4, 72, 256, std=0.02)
    ac, as_, ga, wc, ws, gw = _encode(a, wt, [0, 72])
    C = _gpu_product(ac, as_, ga, wc, ws, gw, [0, 72], out_dtype="bf16")
    R = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, [0, 72])
    # bf16 output: one extra rounding of the FP32 result (relative 2^-9)
    assert np.all(np.abs(C - R) <= 2.0 ** -8 * np.abs(R) + 1e-4 * oracle.gemm_abs_bound(
        ac, as_, ga, wc, ws, gw, [0, 72]))


@pytest.mark.parametrize("M,N,K", [(300, 260, 256), (3, 70, 1024), (40, 33, 80), (1, 70, 1024),
                                   (2, 45, 2048)])
@pytest.mark.parametrize("pad", [3, 8])
@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_output_view_with_row_pitch(M, N, K, pad, odt):
    """C written into a column window of a wider buffer: row pitch N + pad elements (not a multiple
    of 4 for pad = 3, so rows are not 16-byte aligned), window starting 8 elements in.  Elements
    outside the window keep their sentinel value."""
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    a = random_matrix(M + 3 * K, M, K, outlier_cols=2)
    wt = random_matrix(N + 5 * K, N, K, std=0.02)
    ac, as_, ga, wc, ws, gw = _encode(a, wt, [0, N])
    dt = torch.float32 if odt == "f32" else torch.bfloat16
    buf = torch.full((M, N + pad + 8), -7.0, dtype=dt, device=DEV)
    out = buf[:, 8:8 + N]
    nv.nvfp4_gemm(_up(ac), _up(as_), scalar(ga), _up(wc), _up(ws), _up(np.asarray([gw], np.float32)),
                  out=out)
    torch.cuda.synchronize()
    hb = buf.float().cpu().numpy()
    assert np.all(hb[:, :8] == -7.0) and np.all(hb[:, 8 + N:] == -7.0)
    C = hb[:, 8:8 + N].astype(np.float64)
    R = oracle.gemm_exact(ac, as_, ga, wc, ws, [gw], [0, N])
    B = oracle.gemm_abs_bound(ac, as_, ga, wc, ws, [gw], [0, N])
    if odt == "f32":
        check_gemm(C, R, B, f"view M={M} N={N} K={K} pad={pad}")
    else:  # one extra rounding of the FP32 result to bf16
        assert np.all(np.abs(C - R) <= 2.0 ** -8 * np.abs(R) + 1e-4 * B)


@pytest.mark.parametrize("M,N,K", [
    (1, 5000, 1024), (4, 4100, 2048), (16, 8100, 1024), (3, 9000, 1024), (8, 3000, 7168),
    (2, 4500, 8192), (16, 5123, 1024),
    # one or two activation rows: padding of 15 or 14 MFMA rows
    (1, 5120, 5120), (2, 3001, 7168), (1, 7, 1024), (2, 33, 3072), (2, 9000, 2048),
    (1, 16, 4096), (2, 40000, 1024),
])
def test_skinny_column_split(M, N, K):
    """Decode-shaped products whose columns are split evenly over the compute units: workgroups of
    more than 16 columns (two MFMA tiles, the second partly empty), more than 32 columns per compute
    unit, ragged last workgroups, one column per workgroup, and K up to the largest the skinny
    kernels take."""
    a = random_matrix(M * 11 + K, M, K, outlier_cols=max(1, K // 100))
    wt = random_matrix(N * 3 + K, N, K, std=0.02)
    enc = _encode(a, wt, [0, N])
    _check(*enc, [0, N], f"skinny M={M} N={N} K={K}")


def test_skinny_fused_equals_per_segment_calls_bitwise():
    """On the decode path the fused product (two tiles per workgroup) and the per-segment products
    (one tile) must agree bit for bit: every column is accumulated the same way."""
    M, K = 4, 2048
    sizes = [2048, 2048, 48, 48]
    segs = list(np.cumsum([0] + sizes))
    a = random_matrix(40, M, K, outlier_cols=20)
    wt = random_matrix(41, segs[-1], K, std=0.02)
    ac, as_, ga, wc, ws, gw = _encode(a, wt, segs)
    fused = _gpu_product(ac, as_, ga, wc, ws, gw, segs)
    parts = [_gpu_product(ac, as_, ga, wc[segs[j]:segs[j + 1]], ws[segs[j]:segs[j + 1]], [gw[j]],
                          [0, sizes[j]]) for j in range(len(sizes))]
    assert np.array_equal(fused, np.concatenate(parts, axis=1))


@pytest.mark.parametrize("M", [1, 2])
def test_single_row_fused_equals_per_segment_calls_bitwise(M):
    """One or two activation rows on the decode path: the fused product and the per-segment
    products use different column splits and must agree bit for bit."""
    K = 3072
    sizes = [2048, 2048, 48, 48, 5]
    segs = list(np.cumsum([0] + sizes))
    a = random_matrix(50 + M, M, K, outlier_cols=20)
    wt = random_matrix(51, segs[-1], K, std=0.02)
    ac, as_, ga, wc, ws, gw = _encode(a, wt, segs)
    fused = _gpu_product(ac, as_, ga, wc, ws, gw, segs)
    parts = [_gpu_product(ac, as_, ga, wc[segs[j]:segs[j + 1]], ws[segs[j]:segs[j + 1]], [gw[j]],
                          [0, sizes[j]]) for j in range(len(sizes))]
    assert np.array_equal(fused, np.concatenate(parts, axis=1))
    R = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, segs)
    check_gemm(fused, R, oracle.gemm_abs_bound(ac, as_, ga, wc, ws, gw, segs), f"decode M={M}")


@pytest.mark.parametrize("M", [2, 16])
def test_long_k_fused_equals_per_segment_calls_bitwise(M):
    """Long K on the decode path (the long-K form, two tiles per workgroup fused, one per segment):
    the fused product and the per-segment products agree bit for bit."""
    K = 10240
    sizes = [2048, 2048, 48, 48]
    segs = list(np.cumsum([0] + sizes))
    a = random_matrix(60 + M, M, K, outlier_cols=20)
    wt = random_matrix(61, segs[-1], K, std=0.02)
    ac, as_, ga, wc, ws, gw = _encode(a, wt, segs)
    fused = _gpu_product(ac, as_, ga, wc, ws, gw, segs)
    parts = [_gpu_product(ac, as_, ga, wc[segs[j]:segs[j + 1]], ws[segs[j]:segs[j + 1]], [gw[j]],
                          [0, sizes[j]]) for j in range(len(sizes))]
    assert np.array_equal(fused, np.concatenate(parts, axis=1))
    R = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, segs)
    bound = oracle.gemm_abs_bound(ac, as_, ga, wc, ws, gw, segs)
    check_gemm(fused, R, bound, f"long K fused M={M}")
    check_gemm(np.concatenate(parts, axis=1), R, bound, f"long K per segment M={M}")


@pytest.mark.parametrize("M", [1, 16])
def test_many_column_fused_equals_per_segment_calls_bitwise(M):
    """More than 32 columns per compute unit fused (the many-column form), at most 32 per segment
    (the one-pass form): every element is accumulated the same way, so the two agree bit for bit."""
    K = 2048
    sizes = [4096, 4096, 808]
    segs = list(np.cumsum([0] + sizes))
    a = random_matrix(70 + M, M, K, outlier_cols=20)
    wt = random_matrix(71, segs[-1], K, std=0.02)
    ac, as_, ga, wc, ws, gw = _encode(a, wt, segs)
    fused = _gpu_product(ac, as_, ga, wc, ws, gw, segs)
    parts = [_gpu_product(ac, as_, ga, wc[segs[j]:segs[j + 1]], ws[segs[j]:segs[j + 1]], [gw[j]],
                          [0, sizes[j]]) for j in range(len(sizes))]
    assert np.array_equal(fused, np.concatenate(parts, axis=1))
    R = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, segs)
    check_gemm(fused, R, oracle.gemm_abs_bound(ac, as_, ga, wc, ws, gw, segs), f"many columns M={M}")


def test_fused_equals_per_segment_calls_bitwise():
    M, K = 96, 512
    sizes = [64, 64, 128, 48, 48, 7]
    segs = list(np.cumsum([0] + sizes))
    N = segs[-1]
    a = random_matrix(10, M, K, outlier_cols=5)
    wt = random_matrix(11, N, K, std=0.02)
    ac, as_, ga, wc, ws, gw = _encode(a, wt, segs)
    fused = _gpu_product(ac, as_, ga, wc, ws, gw, segs)
    parts = [_gpu_product(ac, as_, ga, wc[segs[j]:segs[j + 1]], ws[segs[j]:segs[j + 1]], [gw[j]],
                          [0, sizes[j]]) for j in range(len(sizes))]
    assert np.array_equal(fused, np.concatenate(parts, axis=1))
    R = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, segs)
    check_gemm(fused, R, oracle.gemm_abs_bound(ac, as_, ga, wc, ws, gw, segs), "fused")


def test_defective_fused_scale_reproduced_on_gpu():
    """The pages' defect (largest global scale for every segment) versus the per-segment repair,
    at the paired ratios 1.82 (qkv/z) and 2.75 (b/a)."""
    M, K, n = 64, 5120, 96
    a = random_matrix(20, M, K, outlier_cols=51, outlier_gain=50.0)
    for ratio in (1.82, 2.75):
        wt = random_matrix(21, 2 * n, K, std=0.02)
        g0 = np.float32(20000.0)
        g1 = np.float32(g0 * np.float32(ratio))
        segs = [0, n, 2 * n]
        ac, as_, ga, wc, ws, gw = _encode(a, wt, segs, [g0, g1])
        good = _gpu_product(ac, as_, ga, wc, ws, gw, segs)
        bad = _gpu_product(ac, as_, ga, wc, ws, oracle.fused_scale_defect(gw), segs)
        R = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, segs)
        check_gemm(good, R, oracle.gemm_abs_bound(ac, as_, ga, wc, ws, gw, segs), "repaired")
        assert np.array_equal(bad[:, n:], good[:, n:])
        rel = np.linalg.norm(bad[:, :n] - R[:, :n]) / np.linalg.norm(R[:, :n])
        assert abs(rel - (1 - 1 / ratio)) < 1e-5, rel
        log(f"ratio {ratio}: defective segment relative error {rel:.4f}")


def test_determinism():
    a = random_matrix(30, 256, 1024, outlier_cols=5)
    wt = random_matrix(31, 384, 1024, std=0.02)
    enc = _encode(a, wt, [0, 384])
    c1 = _gpu_product(*enc, [0, 384])
    c2 = _gpu_product(*enc, [0, 384])
    assert np.array_equal(c1, c2)


def _sampled_full_size(wid, M=None):
    """Full-size product on the GPU (inputs encoded on the GPU from the same seeded tensors, then
    checked bit for bit against the oracle's encoding on the sampled rows), sampled outputs
    compared with the oracle's exact product."""
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    from .gpu_util import to_device

    w = WORKLOADS[wid]
    M = w.M if M is None else M
    log(f"workload {wid}: generating A {M}x{w.K}, W {w.N}x{w.K}")
    wt = weights(w)
    segs = w.seg_offsets
    gw = np.array([oracle.dynamic_global_scale(wt[segs[j]:segs[j + 1]])
                   for j in range(len(segs) - 1)], np.float32)
    wd = to_device(wt, w.w_dtype)
    log(f"workload {wid}: encode on GPU")
    if w.silu_mul:
        # the activation is SiLU(g) * u, encoded by the fused encoder with its dynamic scale
        g, u = gate_up(w, M)
        gd, ud = to_device(g, w.act_dtype), to_device(u, w.act_dtype)
        ac_d, as_d, ga_d = nv.nvfp4_silu_mul_quantize(gd, ud)
        torch.cuda.synchronize()
        ga = np.float32(ga_d.item())
        del gd, ud

        def encode_rows(rows):
            return oracle.silu_mul_quantize(g[rows], u[rows], ga)[:2]
    else:
        a = activations(w, M)
        ga = oracle.dynamic_global_scale(a)
        ad = to_device(a, w.act_dtype)
        ac_d, as_d, _ = nv.nvfp4_quantize(ad, scalar(ga))
        del ad

        def encode_rows(rows):
            return oracle.quantize(a[rows], ga)[:2]
    wc_d = torch.empty((w.N, w.K // 2), dtype=torch.uint8, device=DEV)
    ws_d = torch.empty((w.N, w.K // 16), dtype=torch.uint8, device=DEV)
    for j in range(len(segs) - 1):
        nv.nvfp4_quantize(wd[segs[j]:segs[j + 1]], scalar(gw[j]), wc_d[segs[j]:segs[j + 1]],
                          ws_d[segs[j]:segs[j + 1]])
    del wd
    log(f"workload {wid}: product on GPU")
    C = nv.fused_nvfp4_gemm(ac_d, as_d, scalar(ga), wc_d, ws_d, _up(gw), segs)
    torch.cuda.synchronize()

    # stratified sample: one random row in every band of 256 rows and one random column in every
    # band of 256 columns (so every 256 x 256 output tile holds a checked element), the first and
    # last row and column of the matrix and of every segment, and 30 rows / 40 columns per segment
    # more at random
    rng = np.random.Generator(np.random.PCG64(100 + wid))

    def bands(n):
        return [int(rng.integers(lo, min(n, lo + 256))) for lo in range(0, n, 256)]

    rows = np.unique(np.concatenate([[0, M - 1], bands(M),
                                     rng.choice(M, min(30, M), replace=False)]))
    cols = [0, w.N - 1] + bands(w.N)
    for j in range(len(segs) - 1):
        cols += [segs[j], segs[j + 1] - 1]
        cols += list(rng.choice(np.arange(segs[j], segs[j + 1]), min(40, segs[j + 1] - segs[j]),
                                replace=False))
    cols = np.unique(np.array(cols))
    assert len(np.unique(rows // 256)) == -(-M // 256) and len(np.unique(cols // 256)) == -(-w.N // 256)
    log(f"workload {wid}: oracle on {len(rows)} rows x {len(cols)} cols")
    ac, as_ = encode_rows(rows)
    assert np.array_equal(ac, ac_d[rows].cpu().numpy()) and np.array_equal(as_, as_d[rows].cpu().numpy())
    seg_of = np.searchsorted(segs, cols, side="right") - 1
    wc = np.zeros((len(cols), w.K // 2), np.uint8)
    ws = np.zeros((len(cols), w.K // 16), np.uint8)
    for i, (cidx, j) in enumerate(zip(cols, seg_of)):
        c1, s1, _ = oracle.quantize(wt[cidx:cidx + 1], gw[j])
        wc[i], ws[i] = c1[0], s1[0]
    assert np.array_equal(wc, wc_d[cols].cpu().numpy()) and np.array_equal(ws, ws_d[cols].cpu().numpy())
    # per-column global scales: treat each sampled column as its own one-column segment
    one = list(range(len(cols) + 1))
    R, B = oracle_product(ac, as_, ga, wc, ws, gw[seg_of], one)
    got = C[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].cpu().numpy()
    worst = check_gemm(got, R, B, f"workload {wid}")
    log(f"workload {wid}: worst err / sum|ab| = {worst:.2e}")
    del C, ac_d, as_d, wc_d, ws_d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wid", [2, 3, 5])
def test_full_size_sampled(wid):
    _sampled_full_size(wid)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_shapes(M):
    _sampled_full_size(4, M)


@pytest.mark.parametrize("wid,M", [(3, 1), (3, 16), (5, 1), (5, 16)])
def test_mlp_decode_shapes_full_size(wid, M):
    # decode steps on the full MLP weights: gate+up (34816 x 5120, two modules: the decode kernel's
    # many-column form) and down (5120 x 17408 behind the fused SiLU(g) * u encode: its long-K
    # form), every 256-column band sampled
    _sampled_full_size(wid, M)


def test_fused_equals_per_segment_calls_across_tile_shapes():
    """The GDN in_proj's shape (M = 4096, modules of 2048, 2048, 4096, 48 and 48 columns): the fused
    product runs as two launches, 256 x 256 tiles over the first 8192 columns (two full rounds)
    and 64 x 64 tiles over the last 96 (instead of 528 tiles of 256 x 256 whose third round is 1/16
    full, or three rounds of 704 tiles of 256 x 192); the 4096-column module alone runs 256 x 256
    tiles and the others 256 x 192.  Every element is accumulated the same way in every shape, so
    the fused result equals the per-module results bit for bit; sampled rows are checked against
    the oracle."""
    from workloads import random_nvfp4_bytes

    from .gpu_util import oracle_product

    M, K = 4096, 128
    sizes = [2048, 2048, 4096, 48, 48]
    segs = list(np.cumsum([0] + sizes))
    ac, as_ = random_nvfp4_bytes(71, M, K)
    wc, ws = random_nvfp4_bytes(72, segs[-1], K)
    gw = np.array([0.5, 2.0, 1.25, 3.0, 0.75], np.float32)
    ga = np.float32(1.5)
    fused = _gpu_product(ac, as_, ga, wc, ws, gw, segs)
    parts = [_gpu_product(ac, as_, ga, wc[segs[j]:segs[j + 1]], ws[segs[j]:segs[j + 1]], [gw[j]],
                          [0, sizes[j]]) for j in range(len(sizes))]
    assert np.array_equal(fused, np.concatenate(parts, axis=1))
    rows = np.arange(0, M, 64)
    R, B = oracle_product(ac[rows], as_[rows], ga, wc, ws, gw, segs)
    check_gemm(fused[rows], R, B, "fused GDN in_proj shape, sampled rows")
