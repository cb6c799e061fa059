"""GPU parity of nvfp4_linear, the linear layer on a raw activation: the activation's codes and
scales must equal the oracle's encoding under the same static scale bit for bit, and C must equal
fused_nvfp4_gemm on those codes bit for bit (same kernels, same accumulation) and the oracle's exact
product within the stated tolerance.  Decode shapes with at most 6 rows (K a multiple of 1024 up
to 8192, M * K / 1024 <= 32) run encode and product in one launch; the other shapes, decode shapes
of 7 to 16 rows and of 5 or 6 rows with longer K included, run them as two."""

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, activations, random_matrix, weights

from .gpu_util import DEV, check_gemm, log, oracle_product, scalar, to_device

pytestmark = pytest.mark.gpu


def _up(arr):
    import torch

    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def _run(x, dtype, wt, segs, what, ga=None, out_dtype="f32"):
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    M, K = x.shape
    ga = oracle.dynamic_global_scale(x) if ga is None else np.float32(ga)
    wc, ws, gw = oracle.quantize_segments(wt, segs)
    xd = to_device(x, dtype)
    wcd, wsd, gwd = _up(wc), _up(ws), _up(gw)
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    C, ac_d, as_d = nv.nvfp4_linear(xd, scalar(ga), wcd, wsd, gwd, segs, out_dtype=odt)
    ref = nv.fused_nvfp4_gemm(ac_d, as_d, scalar(ga), wcd, wsd, gwd, segs, out_dtype=odt)
    torch.cuda.synchronize()
    ac, as_, _ = oracle.quantize(x, ga)
    got_c, got_s = ac_d.cpu().numpy(), as_d.cpu().numpy()
    assert np.array_equal(got_s, as_), f"{what}: scale bytes differ"
    assert np.array_equal(got_c, ac), f"{what}: code bytes differ"
    C = C.float().cpu().numpy()
    assert np.array_equal(C, ref.float().cpu().numpy()), f"{what}: differs from fused_nvfp4_gemm"
    if out_dtype == "f32":
        R, B = oracle_product(ac, as_, ga, wc, ws, gw, segs)
        worst = check_gemm(C, R, B, what)
        log(f"{what}: codes bit-exact, worst err / sum|ab| = {worst:.2e}")
    return C


@pytest.mark.parametrize("M,N,K", [(1, 5120, 1024), (4, 3000, 2048), (6, 5120, 5120),
                                   (2, 8100, 8192), (5, 40, 3072), (4, 4096, 8192), (1, 16, 1024)])
@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_decode_shapes_one_launch(M, N, K, dtype):
    # one or two 16-column tiles per workgroup, 1 to 8 phases of K, every input type; 4 rows at
    # K = 8192 fill the encode's one batch of blocks exactly (f32 input above K = 5120: two launches)
    x = random_matrix(M * 31 + K, M, K, outlier_cols=max(1, K // 100), dtype="bf16")
    if dtype == "f16":
        x = np.asarray(np.float16(x / 64), np.float32)  # exactly representable in f16
    wt = random_matrix(N + K, N, K, std=0.02)
    segs = [0, N // 3, N] if N >= 3 else [0, N]
    _run(x, dtype, wt, segs, f"linear {dtype} M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(64, 300, 512), (17, 100, 1024), (5, 70, 48), (3, 9000, 1024),
                                   (2, 40, 17408), (7, 40, 3072), (16, 5120, 5120), (6, 4096, 7168),
                                   (5, 300, 7168)])
def test_two_launch_shapes(M, N, K):
    # more than 16 rows, K not a multiple of 1024, more than 32 columns per compute unit, long K,
    # 7 to 16 rows, 5 or 6 rows whose raw blocks exceed the encode's one batch
    x = random_matrix(M * 37 + K, M, K, outlier_cols=3, dtype="bf16")
    wt = random_matrix(N * 3 + K, N, K, std=0.02)
    _run(x, "bf16", wt, [0, N], f"linear two launches M={M} N={N} K={K}")


def test_static_scale_saturation_and_quiet_rows():
    """An under-calibrated static scale (a quarter of the dynamic one's inverse: block scales
    saturate at 448) and quiet or zero rows (subnormal and zero block scales), one launch."""
    M, N, K = 6, 5120, 5120
    x = random_matrix(501, M, K, outlier_cols=51, outlier_gain=50.0, dtype="bf16")
    x[2] *= np.float32(2.0 ** -20)
    x[4] = 0.0
    x[5, :32] = -0.0
    ga = np.float32(oracle.dynamic_global_scale(x) * np.float32(4.0))
    wt = random_matrix(502, N, K, std=0.02)
    _run(x, "bf16", wt, [0, N], "linear saturated static scale", ga=ga)


def test_bf16_output():
    x = random_matrix(601, 4, 4096, outlier_cols=40, dtype="bf16")
    wt = random_matrix(602, 4000, 4096, std=0.02)
    _run(x, "bf16", wt, [0, 2000, 4000], "linear bf16 out", out_dtype="bf16")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_workload_full_size(M):
    """The decode workload (K = N = 5120, N(0, 0.02) weights, activations with 1% hot channels)
    at full size, every output compared."""
    w = WORKLOADS[4]
    _run(activations(w, M), "bf16", weights(w), w.seg_offsets, f"decode workload M={M}")


def test_empty_weight_encodes_only():
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    x = random_matrix(701, 3, 1024, outlier_cols=2, dtype="bf16")
    ga = oracle.dynamic_global_scale(x)
    wc = torch.empty((0, 512), dtype=torch.uint8, device=DEV)
    ws = torch.empty((0, 64), dtype=torch.uint8, device=DEV)
    C, ac_d, as_d = nv.nvfp4_linear(to_device(x, "bf16"), scalar(ga), wc, ws, scalar(1.0))
    torch.cuda.synchronize()
    ac, as_, _ = oracle.quantize(x, ga)
    assert C.shape == (3, 0)
    assert np.array_equal(ac_d.cpu().numpy(), ac) and np.array_equal(as_d.cpu().numpy(), as_)
