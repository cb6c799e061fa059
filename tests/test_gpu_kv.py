"""GPU parity of the FP8 E4M3 KV cache (nvfp4_kv_fp8_store / nvfp4_kv_fp8_load) against the oracle
(oracle/kv_cache.py): every cache byte bit for bit, decoded rows bit for bit.

Cases: every finite E4M3 value, the midpoints between neighbours (ties) and one binary32 ulp either
side, the subnormal range, signed zeros, the saturation region; random rows in f32/bf16/f16 under
power-of-two and arbitrary scales; ragged token counts and widths that leave lanes idle or span
several workgroups along the row; padded row pitches (keys and values as column slices of one qkv
tensor, a cache with a wider pitch); slot mappings with padding (-1) and out-of-range slots, whose
rows must stay untouched; keys-only calls; and the 32K-token, 1024-wide paged prefill at full size
(sampled rows against the oracle, every row against a decode round trip)."""

import numpy as np
import pytest

import oracle
from workloads import KV_WORKLOADS, kv_slot_mapping, kv_tokens, random_matrix

from .gpu_util import DEV, log, scalar, to_device

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A  # pre-fill of cache bytes that must not be written


def _cache(num_slots, width, pitch=None):
    import torch

    pitch = width if pitch is None else pitch
    c = torch.full((num_slots, pitch), SENTINEL, dtype=torch.uint8, device=DEV)
    return c[:, :width] if pitch != width else c


def _store(k, v, dtype, ks, vs, num_slots, slots=None, pitch=None, cache_pitch=None):
    """Run the store on the GPU; returns (key_cache, value_cache) as full-pitch numpy arrays."""
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    tokens, width = k.shape

    def dev(x):
        if pitch is None:
            return to_device(x, dtype)
        big = np.zeros((x.shape[0], pitch), np.float32)
        big[:, :width] = x
        return to_device(big, dtype)[:, :width]

    kc = _cache(num_slots, width, cache_pitch)
    vc = _cache(num_slots, width, cache_pitch) if v is not None else None
    sd = None if slots is None else torch.from_numpy(np.asarray(slots, np.int64)).to(DEV)
    nv.nvfp4_kv_fp8_store(dev(k), None if v is None else dev(v), scalar(ks),
                          None if v is None else scalar(vs), kc, vc, sd)
    torch.cuda.synchronize()
    base = lambda c: c.as_strided((num_slots, c.stride(0)), (c.stride(0), 1)).cpu().numpy()
    return base(kc), (base(vc) if vc is not None else None)


def _expected_cache(x, scale, num_slots, width, slots, pitch=None):
    pitch = width if pitch is None else pitch
    out = np.full((num_slots, pitch), SENTINEL, np.uint8)
    codes = oracle.kv_fp8_encode(x, scale)
    slots = np.arange(x.shape[0]) if slots is None else np.asarray(slots)
    for t, s in enumerate(slots):
        if 0 <= s < num_slots:
            out[s, :width] = codes[t]
    return out


def _assert_bytes(got, ref, what):
    bad = np.argwhere(got != ref)
    assert bad.size == 0, (f"{what}: {len(bad)} bytes differ, first at {bad[0].tolist()}: "
                           f"got {got[tuple(bad[0])]:#04x}, expected {ref[tuple(bad[0])]:#04x}")


def _e4m3_probe_values():
    """Finite E4M3 values (both signs), neighbour midpoints, midpoints +- 1 ulp, tiny values and
    the saturation region, as float32."""
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    vals = oracle.kv_fp8_decode(codes, 1.0).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2  # exact in binary32 (one more significant bit)
    m32 = mids.astype(np.float32)
    up = np.nextafter(m32, np.float32(np.inf))
    dn = np.nextafter(m32, np.float32(0))
    extra = np.array([448.0, 449.0, 463.9, 464.0, 464.1, 480.0, 1e4, 3e38, 2.0 ** -10, 2.0 ** -11,
                      2.0 ** -10 * 1.0000001, 1e-30, 1e-45, 2.0 ** -9 * 0.75, 2.0 ** -9 * 1.5],
                     dtype=np.float32)
    pos = np.concatenate([vals.astype(np.float32), m32, up, dn, extra])
    allv = np.concatenate([pos, -pos, np.array([0.0, -0.0], np.float32)])
    n = (len(allv) + 15) // 16 * 16
    return np.resize(allv, n).astype(np.float32)


def test_every_e4m3_value_tie_and_saturation():
    x = _e4m3_probe_values().reshape(-1, 32)
    for scale in (1.0, 0.25, 4.0):
        log(f"kv probe values scale={scale} shape={x.shape}")
        kc, _ = _store(x, None, "f32", scale, None, x.shape[0])
        ref = _expected_cache(x, scale, x.shape[0], x.shape[1], None)
        _assert_bytes(kc, ref, f"probe values scale={scale}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("tokens,width", [(1, 16), (37, 144), (300, 1024), (70, 1040), (5, 4096)])
def test_store_random_rows_with_slots(dtype, tokens, width):
    rng = np.random.default_rng(tokens * 7 + width)
    k = random_matrix(1000 + tokens, tokens, width, std=3.0, outlier_cols=2, outlier_gain=40.0,
                      dtype="bf16" if dtype == "bf16" else "f32")
    v = random_matrix(2000 + tokens, tokens, width, std=0.5, dtype="bf16" if dtype == "bf16" else "f32")
    if dtype == "f16":
        k, v = k.astype(np.float16).astype(np.float32), v.astype(np.float16).astype(np.float32)
    num_slots = 2 * tokens + 5
    slots = rng.permutation(num_slots)[:tokens].astype(np.int64)
    if tokens > 3:
        slots[1] = -1  # padding token
        slots[2] = num_slots + 7  # out of range: skipped
    ks, vs = np.float32(np.abs(k).max() / 448.0), np.float32(0.0371)
    log(f"kv store dtype={dtype} tokens={tokens} width={width}")
    kc, vc = _store(k, v, dtype, ks, vs, num_slots, slots)
    _assert_bytes(kc, _expected_cache(k, ks, num_slots, width, slots), f"keys {dtype} {tokens}x{width}")
    _assert_bytes(vc, _expected_cache(v, vs, num_slots, width, slots), f"values {dtype} {tokens}x{width}")


def test_store_padded_pitches_and_identity_slots():
    tokens, width = 50, 256
    k = random_matrix(31, tokens, width, std=2.0, dtype="bf16")
    v = random_matrix(32, tokens, width, std=2.0, dtype="bf16")
    log("kv store padded pitches")
    kc, vc = _store(k, v, "bf16", 0.01, 0.02, tokens + 3, None, pitch=width * 3, cache_pitch=width + 48)
    _assert_bytes(kc, _expected_cache(k, 0.01, tokens + 3, width, None, width + 48), "keys padded")
    _assert_bytes(vc, _expected_cache(v, 0.02, tokens + 3, width, None, width + 48), "values padded")


def test_keys_only_and_empty():
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    k = random_matrix(41, 20, 64, dtype="f32")
    log("kv keys only")
    kc, vc = _store(k, None, "f32", 0.003, None, 20)
    assert vc is None
    _assert_bytes(kc, _expected_cache(k, 0.003, 20, 64, None), "keys only")
    # zero tokens: nothing written
    c = _cache(4, 64)
    empty = torch.zeros((1, 64), dtype=torch.bfloat16, device=DEV)[:0]  # valid pointer, 0 rows
    nv.nvfp4_kv_fp8_store(empty, None, scalar(1.0), None, c, None)
    torch.cuda.synchronize()
    assert bool((c == SENTINEL).all())


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_load_matches_oracle(out_dtype):
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    rng = np.random.default_rng(77)
    num_slots, width = 300, 160
    cache = rng.integers(0, 256, (num_slots, width), dtype=np.uint8)
    cache[(cache & 0x7F) == 0x7F] = 0x11  # the store never writes NaN codes
    slots = rng.integers(0, num_slots, 97).astype(np.int64)
    slots[3] = -1
    slots[5] = num_slots
    scale = np.float32(0.0713)
    td = torch.float32 if out_dtype == "f32" else torch.bfloat16
    log(f"kv load out={out_dtype}")
    out = nv.nvfp4_kv_fp8_load(torch.from_numpy(cache).to(DEV), scalar(scale),
                               torch.from_numpy(slots).to(DEV), td)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    ref = np.zeros((len(slots), width), np.float32)
    ok = (slots >= 0) & (slots < num_slots)
    ref[ok] = oracle.kv_fp8_decode(cache[slots[ok]], scale, out_dtype)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_full_size_paged_prefill():
    """The 32768-token, 1024-wide K and V prefill into a shuffled paged cache, in the launch
    configuration the benchmark times: 2048 sampled tokens against the oracle, every stored row
    against a decode round trip bound, untouched slots unchanged."""
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    w = KV_WORKLOADS[6]
    k, v = kv_tokens(w)
    kcal, vcal = kv_tokens(w, 4096, calibration=True)
    ks, vs = oracle.kv_calibrated_scale(kcal), oracle.kv_calibrated_scale(vcal)
    slots = kv_slot_mapping(w)
    log(f"kv full size {w.name} scales {ks} {vs}")
    kd, vd = to_device(k, "bf16"), to_device(v, "bf16")
    kc, vc = _cache(w.num_slots, w.width), _cache(w.num_slots, w.width)
    sd = torch.from_numpy(slots).to(DEV)
    nv.nvfp4_kv_fp8_store(kd, vd, scalar(ks), scalar(vs), kc, vc, sd)
    torch.cuda.synchronize()
    kcn, vcn = kc.cpu().numpy(), vc.cpu().numpy()
    pick = np.sort(np.random.default_rng(5).choice(w.tokens, 2048, replace=False))
    for x, c, s, nm in ((k, kcn, ks, "keys"), (v, vcn, vs, "values")):
        _assert_bytes(c[slots[pick]], oracle.kv_fp8_encode(x[pick], s), f"{nm} sampled rows")
        untouched = np.ones(w.num_slots, bool)
        untouched[slots] = False
        assert np.all(c[untouched] == SENTINEL), nm
        # every row: the decoded code is within half an E4M3 step of x (relative 2^-4), or x is
        # below the subnormal range's half step, or saturated
        xh = oracle.kv_fp8_decode(c[slots], s)
        err = np.abs(xh - x)
        bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-6)
        sat = np.abs(x) / s >= 448
        assert np.all((err <= bound) | sat), nm
