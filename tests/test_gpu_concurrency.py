"""Concurrent calls: the library keeps no mutable state, so calls from several host threads, each on
its own stream (default priority), give the same bytes as the same calls made one after another."""

import threading

import pytest

from workloads import random_matrix

from .gpu_util import DEV, log, to_device

pytestmark = pytest.mark.gpu

SEGS = [0, 192, 512]


def _work(seed):
    """Inputs of one thread's sequence: activations, a fused two-module weight, gate and up, and
    two activation rows for a long-K decode product."""
    return (to_device(random_matrix(seed, 257, 1024, outlier_cols=4, dtype="bf16"), "bf16"),
            to_device(random_matrix(seed + 1, SEGS[-1], 1024, std=0.02, dtype="bf16"), "bf16"),
            to_device(random_matrix(seed + 2, 64, 768, dtype="bf16"), "bf16"),
            to_device(random_matrix(seed + 3, 64, 768, dtype="bf16"), "bf16"),
            to_device(random_matrix(seed + 4, 2, 9216, outlier_cols=3, dtype="bf16"), "bf16"))


_LONG = {}


def _long_weight():
    """One NVFP4 weight of 4500 x 9216 shared (read only) by every thread: its decode products take
    the decode kernel's long-K form with two tiles per workgroup."""
    import bit_block_scaled_nvfp4_amd as nv

    if "w" not in _LONG:
        _LONG["w"] = nv.nvfp4_quantize(
            to_device(random_matrix(3999, 4500, 9216, std=0.02, dtype="bf16"), "bf16"))
    return _LONG["w"]


def _sequence(a, w, gate, up, al, reps):
    """Dynamic encodes, the fused product and two decode-shaped products, `reps` times over."""
    import torch

    import bit_block_scaled_nvfp4_amd as nv

    outs = []
    for _ in range(reps):
        parts = [nv.nvfp4_quantize(w[lo:hi]) for lo, hi in zip(SEGS[:-1], SEGS[1:])]
        wc = torch.cat([p[0] for p in parts])
        ws = torch.cat([p[1] for p in parts])
        gw = torch.cat([p[2] for p in parts])
        ac, as_, ga = nv.nvfp4_quantize(a)
        c = nv.fused_nvfp4_gemm(ac, as_, ga, wc, ws, gw, SEGS)
        dc, ds, dg = nv.nvfp4_quantize(a[:3], ga)
        cd = nv.nvfp4_gemm(dc, ds, dg, wc, ws, gw[:1])
        sc, ss, sg = nv.nvfp4_silu_mul_quantize(gate, up)
        lc, ls, lg = _LONG["w"]
        lac, las, lag = nv.nvfp4_quantize(al)
        cl = nv.nvfp4_gemm(lac, las, lag, lc, ls, lg)
        outs.append([wc, ws, gw, ac, as_, ga, c, cd, sc, ss, sg, lac, las, lag, cl])
    return outs


def test_threads_on_their_own_streams_match_sequential_calls():
    import torch

    seeds = [3100, 3200, 3300, 3400]
    inputs = [_work(s) for s in seeds]
    _long_weight()
    torch.cuda.synchronize()
    ref = [_sequence(*ins, reps=1)[0] for ins in inputs]
    torch.cuda.synchronize()

    results = [None] * len(seeds)
    errors = []

    def run(i):
        try:
            stream = torch.cuda.Stream(device=DEV)  # default priority
            with torch.cuda.stream(stream):
                results[i] = _sequence(*inputs[i], reps=3)
            stream.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(seeds))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, seed in enumerate(seeds):
        log("thread", i, "seed", seed)
        for rep, outs in enumerate(results[i]):
            for k, (x, y) in enumerate(zip(ref[i], outs)):
                assert torch.equal(x, y), f"thread {i} rep {rep}: output {k} differs"
