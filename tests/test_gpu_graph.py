"""The library's calls under HIP graph capture.

One captured sequence covers both product kernels and the encoders:
- a dynamic activation encode;
- a two-module fused product (tiled kernel) and a decode-shaped product (M = 4, skinny kernel);
- a decode-shaped product with K = 9216 and 4500 columns (M = 2, the decode kernel's long-K form,
  two tiles per workgroup);
- a dynamic SiLU-mul encode;
- an FP8 KV store into paged slots;
- a dynamic fake quantisation.

The graph is replayed several times. Before each replay, new input values are copied into the
captured input buffers and the same calls run eagerly on those values in other buffers, with a
synchronisation in between. Every replay must equal those eager calls bit for bit. The dynamic
encodes clear their max cell with a fill kernel, never `hipMemsetAsync`, so replays after the first
start from zero too.
"""

import numpy as np
import pytest

from workloads import random_matrix

from .gpu_util import DEV, log, scalar, to_device

pytestmark = pytest.mark.gpu

SEGS = [0, 256, 640]
SLOTS = 128


def _inputs(seed):
    shapes = [(300, 1024, 8), (4, 1024, 0), (96, 512, 0), (96, 512, 0), (64, 256, 0), (64, 256, 0),
              (2, 9216, 3)]
    return [to_device(random_matrix(seed + i, r, c, outlier_cols=o, dtype="bf16"), "bf16")
            for i, (r, c, o) in enumerate(shapes)]


def _weights():
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    w = to_device(random_matrix(900, SEGS[-1], 1024, std=0.02, dtype="bf16"), "bf16")
    parts = [nv.nvfp4_quantize(w[lo:hi]) for lo, hi in zip(SEGS[:-1], SEGS[1:])]
    wc = torch.cat([p[0] for p in parts])
    ws = torch.cat([p[1] for p in parts])
    gw = torch.cat([p[2] for p in parts])
    long_w = nv.nvfp4_quantize(
        to_device(random_matrix(901, 4500, 9216, std=0.02, dtype="bf16"), "bf16"))
    return wc, ws, gw, long_w


def _sequence(ins, wts, kv):
    """The calls under test; returns every output tensor (the caches are written in place)."""
    import bit_block_scaled_nvfp4_amd as nv

    a, ad, gate, up, k, v, al = ins
    ks, vs, slots, key_cache, value_cache = kv
    wc, ws, gw, (lc, ls, lg) = wts
    ac, as_, ga = nv.nvfp4_quantize(a)
    c = nv.fused_nvfp4_gemm(ac, as_, ga, wc, ws, gw, SEGS)
    dc, ds, dg = nv.nvfp4_quantize(ad, ga)  # decode rows under the prefill's scale
    cd = nv.nvfp4_gemm(dc, ds, dg, wc, ws, gw[:1])
    lac, las, lag = nv.nvfp4_quantize(al)
    cl = nv.nvfp4_gemm(lac, las, lag, lc, ls, lg)
    sc, ss, sg = nv.nvfp4_silu_mul_quantize(gate, up)
    nv.nvfp4_kv_fp8_store(k, v, ks, vs, key_cache, value_cache, slots)
    xh, fg = nv.nvfp4_fake_quantize(a)
    return [ac, as_, ga, c, dc, ds, cd, cl, sc, ss, sg, xh, fg]


def test_captured_sequence_replays_bitwise():
    import torch

    wts = _weights()
    perm = np.random.Generator(np.random.PCG64(77)).permutation(SLOTS)[:64].astype(np.int64)
    slots = torch.from_numpy(perm).to(DEV)
    ks, vs = scalar(0.05), scalar(0.04)  # made before capture: creating them copies from the host

    def caches():
        return (torch.full((SLOTS, 256), 0x5A, dtype=torch.uint8, device=DEV),
                torch.full((SLOTS, 256), 0x5A, dtype=torch.uint8, device=DEV))

    # eager warm-up, then capture on static buffers
    static_in = _inputs(1000)
    kc_g, vc_g = caches()
    _sequence(static_in, wts, (ks, vs, slots, kc_g, vc_g))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs_g = _sequence(static_in, wts, (ks, vs, slots, kc_g, vc_g))
    torch.cuda.synchronize()

    prev_ga = None
    for rep in range(3):
        seed = 2000 + 100 * rep
        log("graph replay", rep, "inputs seed", seed)
        fresh = _inputs(seed)
        for dst, src in zip(static_in, fresh):
            dst.copy_(src)
        kc_g.fill_(0x5A)
        vc_g.fill_(0x5A)
        kc_e, vc_e = caches()
        outs_e = _sequence(fresh, wts, (ks, vs, slots, kc_e, vc_e))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        names = ["a codes", "a scales", "gA", "fused product", "decode codes", "decode scales",
                 "decode product", "long-K decode product", "silu codes", "silu scales", "silu g", "fake quant", "fake g"]
        for name, e, g in zip(names, outs_e, outs_g):
            assert torch.equal(e, g), f"replay {rep}: {name} differs from the eager call"
        assert torch.equal(kc_e, kc_g) and torch.equal(vc_e, vc_g), f"replay {rep}: KV caches differ"
        # the dynamic scale follows each replay's inputs (its max cell starts from zero each time)
        ga = outs_g[2].item()
        assert ga != prev_ga
        prev_ga = ga
