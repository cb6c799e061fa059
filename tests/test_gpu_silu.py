"""GPU parity of nvfp4_silu_mul_quantize (the fused SiLU(gate) * up -> NVFP4 encoder) against the
oracle (oracle/activation.py): codes, scale bytes and the dynamic global scale bit for bit.

Inputs are seeded; besides N(0, 1) gate/up pairs the cases cover |gate| > 16 (binary64 path),
signed zeros, subnormals, products far out of range, and pairs built so that SiLU(gate) * up lies
next to a bfloat16 rounding midpoint (the cases the binary32 path must hand to binary64)."""

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, gate_up, random_matrix, round_bf16

from .gpu_util import DEV, assert_codes_equal, log, scalar, to_device

pytestmark = pytest.mark.gpu


def _gpu(g, u, dtype, ga=None, pad=0):
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    def dev(x):
        if pad:
            x = np.concatenate([x, np.zeros((x.shape[0], pad), np.float32)], axis=1)
        t = to_device(x, dtype)
        return t[:, :t.shape[1] - pad] if pad else t

    c, s, gg = nv.nvfp4_silu_mul_quantize(dev(g), dev(u), None if ga is None else scalar(ga))
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy(), np.float32(gg.item())


def _check(g, u, dtype, what, pad=0):
    for ga in (None, np.float32(123.5)):
        got = _gpu(g, u, dtype, ga, pad)
        ref = oracle.silu_mul_quantize(g, u, ga)
        assert_codes_equal(got, ref, f"{what} dtype={dtype} static={ga is not None}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_normal_inputs(dtype):
    rows, cols = 96, 1024
    g = random_matrix(51, rows, cols, std=1.0)
    u = random_matrix(52, rows, cols, std=1.0)
    if dtype == "bf16":
        g, u = round_bf16(g), round_bf16(u)
    elif dtype == "f16":
        g, u = g.astype(np.float16).astype(np.float32), u.astype(np.float16).astype(np.float32)
    _check(g, u, dtype, "normal")


def test_special_values():
    rng = np.random.default_rng(53)
    rows, cols = 64, 512
    g = round_bf16(rng.normal(0, 1, (rows, cols)).astype(np.float32))
    u = round_bf16(rng.normal(0, 1, (rows, cols)).astype(np.float32))
    # |g| beyond the binary32 path, signed zeros, subnormal and huge magnitudes
    g[0, :64] = round_bf16(rng.uniform(16, 200, 64).astype(np.float32) * rng.choice([-1, 1], 64))
    g[1, :16], u[1, :16] = 0.0, 1.0
    g[1, 16:32], u[1, 16:32] = -0.0, 1.0
    g[1, 32:48], u[1, 32:48] = 1.0, -0.0
    g[2, :32] = round_bf16(np.float32(1e-39) * rng.uniform(1, 9, 32).astype(np.float32))
    u[2, :32] = round_bf16(np.float32(1e-30) * rng.uniform(1, 9, 32).astype(np.float32))
    g[3, :16] = 3.0
    u[3, :16] = round_bf16(np.float32(1e30) * rng.uniform(1, 9, 16).astype(np.float32))
    g[4, :16] = -90.0  # silu(-90) ~ -7e-38: tiny times ordinary u
    _check(g, u, "bf16", "special")


def test_near_bfloat16_midpoints():
    """Pairs with SiLU(g) * u within a few binary32 ulps of a bfloat16 midpoint."""
    rng = np.random.default_rng(54)
    n = 16 * 4096
    g = round_bf16(rng.normal(0, 1.5, n).astype(np.float32))
    a = oracle.silu(g)
    # pick a target midpoint near a random magnitude, solve u = target / silu(g), round u to
    # bf16 (so the product lands near, not exactly on, the midpoint), keep those that land close
    t = rng.uniform(0.1, 4.0, n) * rng.choice([-1, 1], n)
    step = np.exp2(np.floor(np.log2(np.abs(t))) - 7)
    mid = (np.floor(np.abs(t) / step) + 0.5) * step * np.sign(t)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = round_bf16(np.clip(mid / np.where(a == 0, 1.0, a), -1e30, 1e30).astype(np.float32))
    y = a * u.astype(np.float64)
    ulp32 = np.exp2(np.floor(np.log2(np.abs(y) + 1e-300)) - 23)
    near = np.abs(np.abs(y) - np.abs(mid)) < 200 * ulp32
    log(f"midpoint cases within 200 binary32 ulps: {near.sum()} of {n}")
    assert near.sum() > 100
    _check(g.reshape(-1, 1024), u.reshape(-1, 1024), "bf16", "midpoints")


def test_strided_rows():
    g = round_bf16(random_matrix(55, 40, 256, std=2.0))
    u = round_bf16(random_matrix(56, 40, 256, std=1.0))
    _check(g, u, "bf16", "strided", pad=24)


def test_full_size_sampled_rows():
    """The long-prefill activation (32768 x 17408): dynamic scale against the oracle's max over
    the whole tensor, codes and scales on sampled rows."""
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    w = WORKLOADS[5]
    log(f"generating gate/up {w.M}x{w.K}")
    g, u = gate_up(w)
    gd, ud = to_device(g, "bf16"), to_device(u, "bf16")
    c, s, gg = nv.nvfp4_silu_mul_quantize(gd, ud)
    torch.cuda.synchronize()
    ga = np.float32(gg.item())
    log("oracle amax over the full tensor")
    amax = np.float32(0.0)
    for r0 in range(0, w.M, 2048):
        amax = max(amax, np.abs(oracle.silu_mul_activation(g[r0:r0 + 2048], u[r0:r0 + 2048])).max())
    assert ga == np.float32(np.float32(2688.0) / amax)
    rng = np.random.Generator(np.random.PCG64(57))
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.choice(w.M, 62, replace=False)]))
    ref = oracle.silu_mul_quantize(g[rows], u[rows], ga)
    assert_codes_equal((c[rows].cpu().numpy(), s[rows].cpu().numpy(), ga), ref, "full size")
    del gd, ud, c, s
    torch.cuda.empty_cache()
