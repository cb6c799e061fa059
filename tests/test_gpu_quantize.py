"""GPU parity of nvfp4_quantize: codes, scale bytes and the global scale must be bit-identical to
the oracle's, for every input dtype, static and dynamic global scales, ragged and strided shapes,
the numeric edge cases, dense sweeps of both codecs, and sampled rows of the full-size workloads."""

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, activations, random_matrix, round_bf16, weights

from .gpu_util import assert_codes_equal, gpu_quantize, log, scalar, to_device

pytestmark = pytest.mark.gpu


def _both(x, dtype, g=None):
    got = gpu_quantize(x, dtype, g)
    ref = oracle.quantize(x, g)
    return got, ref


def _cast(x, dtype):
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    return x


def test_workload1_single_dynamic():
    w = WORKLOADS[1]
    a, wt = activations(w), weights(w)
    log("workload 1: A", a.shape, "W", wt.shape)
    assert_codes_equal(*_both(a, "f32"), "A dynamic")
    assert_codes_equal(*_both(wt, "f32"), "W dynamic")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (17, 80), (64, 512), (130, 1040)])
def test_ragged_shapes_all_dtypes(dtype, shape):
    x = _cast(random_matrix(sum(shape), *shape, outlier_cols=max(1, shape[1] // 64)), dtype)
    log("ragged", dtype, shape)
    assert_codes_equal(*_both(x, dtype), f"{dtype} {shape} dynamic")
    assert_codes_equal(*_both(x, dtype, np.float32(37.5)), f"{dtype} {shape} static")


@pytest.mark.parametrize("block", [0, 3 * 65536 + 5, 131111, 4099 * 64 - 1])
def test_dynamic_scale_wherever_the_maximum_sits(block):
    # 4099 x 1024 (262336 blocks): on 256 compute units the max pass takes four blocks per step
    # for the first 262144 and one at a time for the rest, so the planted maximum lands in the
    # first or fourth slot of a step, mid-tensor, or in the last block
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    x = round_bf16(random_matrix(41, 4099, 1024, outlier_cols=3))
    r, c = divmod(block * 16, 1024)
    x[r, c + 7] = np.float32(-32768.0)  # exact in bf16
    g = oracle.dynamic_global_scale(x)
    codes, scales, gg = nv.nvfp4_quantize(to_device(x, "bf16"))
    torch.cuda.synchronize()
    assert np.float32(gg.item()) == g, f"planted max in block {block}"
    rows = np.unique([0, r, 4098])
    ref = oracle.quantize(x[rows], g)
    got = (codes[rows].cpu().numpy(), scales[rows].cpu().numpy(), np.float32(gg.item()))
    assert_codes_equal(got, ref, f"planted max in block {block}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_rows(dtype):
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    x = _cast(random_matrix(5, 33, 96, outlier_cols=2), dtype)
    big = np.zeros((33, 160), np.float32)
    big[:, :96] = x
    xd = to_device(big, dtype)[:, :96]
    assert xd.stride(0) == 160
    c, s, g = nv.nvfp4_quantize(xd, scalar(11.0))
    torch.cuda.synchronize()
    assert_codes_equal((c.cpu().numpy(), s.cpu().numpy(), np.float32(g.item())),
                       oracle.quantize(x, 11.0), "strided")


def test_edge_cases():
    rows = []
    z = np.zeros(16, np.float32)
    rows.append(z)                                   # zero block
    rows.append(-z)                                  # signed zeros
    rows.append(np.full(16, 3.0, np.float32))        # constant
    rows.append(np.full(16, -0.37, np.float32))      # negative constant
    r = z.copy(); r[0] = 6.0; r[1] = -0.1; r[2] = 0.1  # negatives rounding to zero keep the sign
    rows.append(r)
    rows.append(np.full(16, 1e-4, np.float32))       # scale underflows to 0
    r = np.full(16, 3e-3, np.float32); r[5] = -7e-3  # subnormal E4M3 scale
    rows.append(r)
    r = np.array([12, 5, -10, 1.5, 0.5, 3.5, 7] + [0] * 9, np.float32)  # ties
    rows.append(r)
    r = np.array([1.0, -0.3] + [0] * 14, np.float32)
    rows.append(r)
    r = np.zeros(16, np.float32); r[7] = 1e30; r[8] = -1e-30  # huge dynamic range in a block
    rows.append(r)
    r = np.linspace(-6, 6, 16).astype(np.float32)
    rows.append(r)
    x = np.stack(rows)
    for g in (1.0, 4.0, 1e-3, 1e6, None):
        log("edge cases g =", g)
        assert_codes_equal(*_both(x, "f32", g), f"edge g={g}")


def test_saturation_under_calibrated_scale():
    x = round_bf16(random_matrix(7, 64, 256, outlier_cols=4))
    g_cal = oracle.dynamic_global_scale(x)
    got, ref = _both(x, "bf16", np.float32(g_cal * 4))
    assert np.any(ref[1] == 0x7E)
    assert_codes_equal(got, ref, "under-calibrated")


def test_e2m1_sweep():
    # blocks [6.0, y1..y15] with g = 1: s = fl(6 * fl(1/6)) = 1, sd = 1, r = 1, so the encoder
    # rounds y directly; y sweeps dense fp32 windows around every E2M1 threshold plus random values
    centres = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    ys = []
    for c in centres:
        b = np.float32(c).view(np.uint32)
        ys.append(np.arange(b - 3000, b + 3001, dtype=np.uint32).view(np.float32))
    # every binary32 magnitude in [0, 6] whose low 12 pattern bits are zero: each binade from the
    # subnormals up, so no stretch of the grid is left to the random values alone
    ys.append((np.arange(0, 0x40C01, dtype=np.uint32) << 12).view(np.float32))
    rng = np.random.Generator(np.random.PCG64(99))
    ys.append(rng.uniform(0, 6, 150_000).astype(np.float32))
    y = np.concatenate(ys)
    y = y[(y >= 0) & (y <= 6)]
    y = np.concatenate([y, np.zeros((-len(y)) % 15, np.float32)])
    sign = np.where(rng.random(len(y)) < 0.5, -1, 1).astype(np.float32)
    body = (y * sign).reshape(-1, 15)
    x = np.concatenate([np.full((len(body), 1), 6.0, np.float32), body], axis=1)
    x = x.reshape(-1, 64 * 16) if len(x) % 64 == 0 else x.reshape(-1, 16)
    assert_codes_equal(*_both(x, "f32", 1.0), "e2m1 sweep")


def test_e4m3_sweep():
    # g = 6: gs6 = 1, so the block scale is amax itself; amax sweeps every bf16 value in
    # [2^-12, 460] and dense fp32 windows around E4M3 rounding midpoints
    v = oracle.E4M3_VALUES
    mids = np.concatenate([(v[:-1] + v[1:]) / 2.0, v[1:]])
    parts = [np.arange(0x3980, 0x43E6, dtype=np.uint32) << 16]
    for c in mids:
        b = np.float32(c).view(np.uint32)
        parts.append(np.arange(b - 300, b + 301, dtype=np.uint32))
    amax = np.concatenate(parts).view(np.float32)
    amax = amax[(amax > 0) & (amax < 1000)]
    rng = np.random.Generator(np.random.PCG64(98))
    frac = rng.random((len(amax), 15)).astype(np.float32)
    body = (frac * amax[:, None]).astype(np.float32)
    x = np.concatenate([amax[:, None], body], axis=1).astype(np.float32)
    x = np.concatenate([x, np.zeros(((-len(x)) % 4, 16), np.float32)]).reshape(-1, 64)
    assert_codes_equal(*_both(x, "f32", 6.0), "e4m3 sweep")


def test_determinism():
    x = round_bf16(random_matrix(8, 256, 1024, outlier_cols=8))
    a = gpu_quantize(x, "bf16")
    b = gpu_quantize(x, "bf16")
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


@pytest.mark.parametrize("wid", [2, 3, 4])
def test_full_size_activations_sampled_rows(wid):
    """Full-size activation tensor quantised on the GPU with the static scale the benchmark uses
    (2688 / amax, computed on the host from the generated tensor) and with the dynamic scale;
    sampled rows compared bit for bit."""
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    w = WORKLOADS[wid]
    log(f"workload {wid}: generating A {w.M}x{w.K}")
    a = activations(w)
    g = oracle.dynamic_global_scale(a)
    xd = to_device(a, w.act_dtype)
    rng = np.random.Generator(np.random.PCG64(wid))
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.choice(w.M, min(62, w.M), replace=False)]))
    for dyn in (False, True):
        log(f"workload {wid}: quantize dynamic={dyn}")
        c, s, gg = nv.nvfp4_quantize(xd, None if dyn else scalar(g))
        torch.cuda.synchronize()
        assert np.float32(gg.item()) == g
        ref = oracle.quantize(a[rows], g)
        got = (c[rows].cpu().numpy(), s[rows].cpu().numpy(), np.float32(gg.item()))
        assert_codes_equal(got, ref, f"workload {wid} dynamic={dyn}")
    del xd
    torch.cuda.empty_cache()
