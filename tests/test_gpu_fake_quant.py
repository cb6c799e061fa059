"""GPU parity of fake quantization, the quantization-error statistics, requantization and
checkpoint-side harmonization against the oracle (oracle/fake_quant.py).

* nvfp4_fake_quantize: every output bit equal to the oracle's fl32(V * sd / g) (and its bf16
  rounding), static and dynamic scales, all input dtypes, ragged shapes, strided rows, the encoder's
  edge cases (signed zeros, underflowed and subnormal scales, ties, saturation).
* nvfp4_quant_error_stats: dominated-block counts and the dynamic scale exact; the binary64 sums
  within 1e-12 relative (their summation order is unspecified) -- on ragged shapes and on sampled
  rows of the full-size prefill activations.
* nvfp4_requantize / nvfp4_harmonize_segments: every byte equal to the oracle's, in place and out
  of place; the fused GDN in_proj weight (five modules, 8288 x 5120) at full size.
"""

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, activations, random_matrix, round_bf16, weights

from .gpu_util import DEV, assert_codes_equal, log, scalar, to_device

pytestmark = pytest.mark.gpu


def _fake(x, dtype, g=None, out="f32", pitch=None):
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    if pitch is None:
        xd = to_device(x, dtype)
    else:
        big = np.zeros((x.shape[0], pitch), np.float32)
        big[:, :x.shape[1]] = x
        xd = to_device(big, dtype)[:, :x.shape[1]]
    od = torch.float32 if out == "f32" else torch.bfloat16
    xh, gg = nv.nvfp4_fake_quantize(xd, None if g is None else scalar(g), od)
    torch.cuda.synchronize()
    return xh.float().cpu().numpy(), np.float32(gg.item())


def _ref_fake(x, g, out):
    xh, gg = oracle.fake_quantize(x, g)
    if out == "bf16":
        xh = oracle.round_to_bf16(xh.astype(np.float64))
    return xh, gg


def _assert_bits(got, ref, what):
    gb, rb = got.view(np.uint32), ref.view(np.uint32)
    bad = np.argwhere(gb != rb)
    assert bad.size == 0, (f"{what}: {len(bad)} values differ, first at {bad[0].tolist()}: "
                           f"{got[tuple(bad[0])]!r} vs {ref[tuple(bad[0])]!r}")


def _edge_rows():
    z = np.zeros(16, np.float32)
    rows = [z, -z, np.full(16, 3.0, np.float32), np.full(16, -0.37, np.float32)]
    r = z.copy(); r[0] = 6.0; r[1] = -0.1; r[2] = 0.1
    rows.append(r)
    rows.append(np.full(16, 1e-4, np.float32))
    r = np.full(16, 3e-3, np.float32); r[5] = -7e-3
    rows.append(r)
    rows.append(np.array([12, 5, -10, 1.5, 0.5, 3.5, 7] + [0] * 9, np.float32))
    r = np.zeros(16, np.float32); r[7] = 1e30; r[8] = -1e-30
    rows.append(r)
    rows.append(np.linspace(-6, 6, 16).astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fake_quantize_edge_cases(out):
    x = _edge_rows()
    for g in (1.0, 4.0, 1e-3, 1e6, None):
        log(f"fake quantize edge cases g={g} out={out}")
        got, gg = _fake(x, "f32", g, out)
        ref, rg = _ref_fake(x, g, out)
        assert gg == rg
        _assert_bits(got, ref, f"edge g={g} out={out}")


def test_fake_quantize_extreme_scales():
    """Blocks whose dequantized values leave the binary32 normal range (tiny values under a huge
    scale, huge values under a tiny one): the kernel divides each element there instead of scaling
    two per-block quotients."""
    rng = np.random.default_rng(91)
    tiny = (rng.uniform(-1, 1, (8, 32)) * 2.3e-38).astype(np.float32)
    huge = (rng.uniform(-1, 1, (8, 32)) * 3e38).astype(np.float32)
    mixed = np.concatenate([tiny[:, :16], huge[:, :16]], axis=1)
    for x, g in ((tiny, 1e36), (huge, 1e-36), (mixed, 1e-36), (mixed, 1e36), (huge, 8.9e-36)):
        log(f"fake quantize extreme g={g}")
        for out in ("f32", "bf16"):
            got, _ = _fake(x, "f32", np.float32(g), out)
            ref, _ = _ref_fake(x, np.float32(g), out)
            _assert_bits(got, ref, f"extreme g={g} out={out}")
    c, s_, gg = oracle.quantize(huge, np.float32(1e-36))
    for g_out in (np.float32(2e-36), np.float32(1e-37)):
        import torch

        import bit_block_scaled_nvfp4_amd as nv

        rc, rs = oracle.requantize(c, s_, gg, g_out)
        oc, os_ = nv.nvfp4_requantize(torch.from_numpy(c).to(DEV), torch.from_numpy(s_).to(DEV),
                                      scalar(gg), scalar(g_out))
        torch.cuda.synchronize()
        assert_codes_equal((oc.cpu().numpy(), os_.cpu().numpy(), 0), (rc, rs, 0), "extreme requantize")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 16), (37, 144), (300, 1024), (64, 5120)])
def test_fake_quantize_ragged(dtype, shape):
    x = random_matrix(shape[0] * 3 + shape[1], *shape, outlier_cols=3,
                      dtype="bf16" if dtype == "bf16" else "f32")
    if dtype == "f16":
        x = x.astype(np.float16).astype(np.float32)
    for g in (None, np.float32(123.25)):
        for out in ("f32", "bf16"):
            log(f"fake quantize {dtype} {shape} g={g} out={out}")
            got, gg = _fake(x, dtype, g, out)
            ref, rg = _ref_fake(x, g, out)
            assert gg == rg
            _assert_bits(got, ref, f"{dtype} {shape} g={g} out={out}")


def test_fake_quantize_strided_and_saturating():
    x = round_bf16(random_matrix(17, 50, 256, outlier_cols=4))
    g_sat = np.float32(oracle.dynamic_global_scale(x) * 4)  # under-calibrated: scales saturate
    got, _ = _fake(x, "bf16", g_sat, "f32", pitch=384)
    ref, _ = _ref_fake(x, g_sat, "f32")
    _assert_bits(got, ref, "strided, saturating")


def _stats(x, dtype, g=None):
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    e2, n2, dom, gg = nv.nvfp4_quant_error_stats(to_device(x, dtype), None if g is None else scalar(g))
    torch.cuda.synchronize()
    return e2.cpu().numpy(), n2.cpu().numpy(), dom.cpu().numpy(), np.float32(gg.item())


def _check_stats(got, ref, what):
    e2, n2, dom, g = got
    re2, rn2, rdom, rg = ref
    assert g == rg, what
    assert np.array_equal(dom, rdom), f"{what}: dominated counts differ"
    for a, b, nm in ((e2, re2, "err2"), (n2, rn2, "norm2")):
        lim = 1e-12 * np.abs(b)
        assert np.all(np.abs(a - b) <= lim), f"{what}: {nm} max rel diff " \
            f"{np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-300)):.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 16), (5, 1040), (133, 512), (7, 17408)])
def test_error_stats_ragged(dtype, shape):
    x = random_matrix(shape[0] + 7 * shape[1], *shape, outlier_cols=max(1, shape[1] // 100),
                      outlier_gain=60.0, dtype="bf16" if dtype == "bf16" else "f32")
    for g in (None, np.float32(77.0)):
        log(f"error stats {dtype} {shape} g={g}")
        _check_stats(_stats(x, dtype, g), oracle.quant_error_stats(x, g), f"{dtype} {shape} g={g}")


def test_error_stats_edge_rows():
    x = _edge_rows()
    x = np.concatenate([x, np.zeros((2, 16), np.float32)])
    x[-1, :2] = 1.0  # 2 * 1 > 2 is false: not dominated
    _check_stats(_stats(x, "f32", 1.0), oracle.quant_error_stats(x, 1.0), "edge rows")


@pytest.mark.parametrize("wid", [2, 3])
def test_error_stats_full_size_sampled_rows(wid):
    """The whole prefill activation tensor on the GPU (dynamic scale over all of it), the
    statistics of sampled rows against the oracle with the same scale."""
    w = WORKLOADS[wid]
    log(f"workload {wid}: generating A {w.M}x{w.K}")
    a = activations(w)
    got = _stats(a, w.act_dtype)
    g = oracle.dynamic_global_scale(a)
    assert got[3] == g
    rng = np.random.Generator(np.random.PCG64(40 + wid))
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.choice(w.M, 62, replace=False)]))
    ref = oracle.quant_error_stats(a[rows], g)
    _check_stats((got[0][rows], got[1][rows], got[2][rows], got[3]), ref, f"workload {wid}")


def _encoded(seed, rows, cols, g=None, std=1.0):
    x = random_matrix(seed, rows, cols, std=std, outlier_cols=2)
    return oracle.quantize(x, g)


def test_requantize_matches_oracle_in_and_out_of_place():
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    for (rows, cols), seed in (((1, 16), 1), ((37, 144), 2), ((256, 1024), 3)):
        c, s, g = _encoded(seed, rows, cols)
        for g_out in (g, g / np.float32(2.75), g / np.float32(1.82), g * np.float32(3.1)):
            log(f"requantize {rows}x{cols} {g} -> {g_out}")
            rc, rs = oracle.requantize(c, s, g, g_out)
            cd, sd = torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV)
            oc, os_ = nv.nvfp4_requantize(cd, sd, scalar(g), scalar(g_out))
            torch.cuda.synchronize()
            assert_codes_equal((oc.cpu().numpy(), os_.cpu().numpy(), 0), (rc, rs, 0), "out of place")
            nv.nvfp4_requantize(cd, sd, scalar(g), scalar(g_out), cd, sd)  # in place
            torch.cuda.synchronize()
            assert_codes_equal((cd.cpu().numpy(), sd.cpu().numpy(), 0), (rc, rs, 0), "in place")


def test_harmonize_small_fused_weight():
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    rng = np.random.default_rng(90)
    segs = [48, 16, 80]
    w = np.concatenate([rng.standard_normal((n, 256)).astype(np.float32) * np.float32(m)
                        for n, m in zip(segs, (0.02, 0.02 * 1.82, 0.02 / 2.75))])
    offs = list(np.cumsum([0] + segs))
    c, s, gw = oracle.quantize_segments(w, offs)
    gw = np.asarray(gw, np.float32)
    rc, rs, rg = oracle.harmonize_segments(c, s, gw, offs)
    cd, sd = torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV)
    gd = torch.from_numpy(gw).to(DEV)
    log("harmonize small fused weight")
    hc, hs, hg = nv.nvfp4_harmonize_segments(cd, sd, gd, offs)
    torch.cuda.synchronize()
    assert np.float32(hg.item()) == rg == gw.min()
    assert_codes_equal((hc.cpu().numpy(), hs.cpu().numpy(), 0), (rc, rs, 0), "harmonize")
    nv.nvfp4_harmonize_segments(cd, sd, gd, offs, cd, sd)  # in place
    torch.cuda.synchronize()
    assert_codes_equal((cd.cpu().numpy(), sd.cpu().numpy(), 0), (rc, rs, 0), "harmonize in place")


def test_harmonize_full_size_gdn_in_proj():
    """The five-module fused GDN input projection (8288 x 5120, modules calibrated separately, the
    decay gate's weights 2.75x wider), harmonized on the GPU: every byte against the oracle."""
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    w = WORKLOADS[2]
    log(f"workload 2: generating W {w.N}x{w.K}")
    wt = weights(w)
    offs = w.seg_offsets
    c, s, gw = oracle.quantize_segments(wt, offs)
    del wt
    gw = np.asarray(gw, np.float32)
    rc, rs, rg = oracle.harmonize_segments(c, s, gw, offs)
    cd, sd = torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV)
    hc, hs, hg = nv.nvfp4_harmonize_segments(cd, sd, torch.from_numpy(gw).to(DEV), offs)
    torch.cuda.synchronize()
    assert np.float32(hg.item()) == rg
    assert_codes_equal((hc.cpu().numpy(), hs.cpu().numpy(), 0), (rc, rs, 0), "harmonize full size")
