"""Benchmark of the NVFP4 W4A4 linear-layer hot path on one MI355X.

One step = the whole hot path over one batch of the fused MLP gate+up workload (M = 8192 tokens,
K = 5120, N = 2 x 17408, two calibrated modules): encode the bf16 activations to NVFP4 with the
static (calibrated) global scale, then the fused W4A4 product with the per-module epilogue, FP32
output.  Weights are encoded once before timing (offline step).  Inputs are seeded synthetic
tensors resident in HBM before the timed region starts.

Printed: one JSON line with the prefill throughput (TFLOP/s = 2MNK / step time), the roofline of
the dominant kernel (the product; its average duration from HIP events recorded on the stream it
is launched on), the activation encode with the static and with the dynamic global scale, the
decode-shaped product throughput (GB/s of algorithmic bytes) on a 5120 x 5120 weight and on the
MLP weights, and the CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense f16/bf16
MFMA_FP4_PEAK_TFLOPS = 10066.0  # dense MXFP4, context only
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _encode_weights(torch, nv, W, w, dev):
    """Offline step: encode each calibrated module of the weight with its own dynamic scale."""
    segs = w.seg_offsets
    wc = torch.empty((w.N, w.K // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty((w.N, w.K // 16), dtype=torch.uint8, device=dev)
    gw = torch.empty(len(segs) - 1, dtype=torch.float32, device=dev)
    for j in range(len(segs) - 1):
        wd = W.device_weights(w, dev, slice(segs[j], segs[j + 1]))
        _, _, g = nv.nvfp4_quantize(wd, None, wc[segs[j]:segs[j + 1]], ws[segs[j]:segs[j + 1]])
        gw[j:j + 1].copy_(g)
        del wd
    return wc, ws, gw


def prefill(args, torch, nv, W, wid=3):
    """One prefill-shaped linear layer: the activation encode (or, for the down projection, the
    fused SiLU(g) * u encode) with the static calibrated scale, then the fused product with the
    per-module epilogue, f32 output.  Times: the whole step (`steps` steps between events), the
    product alone (events around each launch, on its stream), and for the headline shape the encode
    alone over rotating inputs and the vendor bf16 GEMM of the same shape."""
    w = W.WORKLOADS[wid]
    dev = "cuda:0"
    log(f"[bench] prefill {w.name}: drawing inputs on the device")
    wc, ws, gw = _encode_weights(torch, nv, W, w, dev)
    segs = w.seg_offsets
    ac = torch.empty((w.M, w.K // 2), dtype=torch.uint8, device=dev)
    as_ = torch.empty((w.M, w.K // 16), dtype=torch.uint8, device=dev)
    C = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    if w.silu_mul:
        gd, ud = W.device_gate_up(w, dev)
        _, _, ga = nv.nvfp4_silu_mul_quantize(gd, ud, None, ac, as_)  # calibration stand-in

        def encode():
            nv.nvfp4_silu_mul_quantize(gd, ud, ga, ac, as_)
    else:
        ad = W.device_activations(w, dev)
        # calibration stand-in: the static scale 2688 / amax of this batch
        ga = torch.tensor([2688.0], device=dev) / ad.float().abs().max().reshape(1)

        def encode():
            nv.nvfp4_quantize(ad, ga, ac, as_)
    torch.cuda.synchronize()

    def product():
        nv.fused_nvfp4_gemm(ac, as_, ga, wc, ws, gw, segs, out=C)

    def step():
        encode()
        product()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    ms_step = _timed(torch, args.steps, lambda i: step())
    # the product alone: events around each launch (it runs for milliseconds)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    for i in range(args.steps):
        encode()
        evs[2 * i].record()
        product()
        evs[2 * i + 1].record()
    torch.cuda.synchronize()
    g_ms = sum(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(args.steps)) / args.steps
    res = dict(w=w, ms_step=ms_step, gemm_ms=g_ms, flops=w.flops)
    if wid != 3:
        return res

    # the encode alone, `steps` launches back to back over 4 rotating input/output sets (430 MB,
    # beyond the 256 MB last-level cache), static and dynamic scale
    R = 4
    sets = [(W.device_activations(w, dev) if i else ad, torch.empty_like(ac), torch.empty_like(as_))
            for i in range(R)]
    for i in range(R):
        nv.nvfp4_quantize(sets[i][0], ga, sets[i][1], sets[i][2])
    torch.cuda.synchronize()
    q_ms = _timed(torch, args.steps, lambda i: nv.nvfp4_quantize(sets[i % R][0], ga, sets[i % R][1],
                                                                 sets[i % R][2]))
    # the dynamic scale: clearing the max cell, the max pass over A, the encode and the scale's
    # finalisation (A is read twice)
    qd_ms = _timed(torch, args.steps, lambda i: nv.nvfp4_quantize(sets[i % R][0], None, sets[i % R][1],
                                                                  sets[i % R][2]))
    del sets
    res.update(quant_ms=q_ms, q_bytes=w.M * w.K * (2 + 9 / 16), quant_dyn_ms=qd_ms,
               qd_bytes=w.M * w.K * (2 + 2 + 9 / 16), quant_sets=R)
    # the vendor dense bf16 GEMM of the same shape (torch.matmul -> hipBLASLt), timed in turns with
    # the NVFP4 product so both see the same clock and temperature
    nv.nvfp4_quantize(ad, ga, ac, as_)
    wb = torch.randn(w.N, w.K, device=dev, dtype=torch.bfloat16)
    for _ in range(2):
        ad @ wb.t()
    torch.cuda.synchronize()
    ours, vend = [], []
    for _ in range(3):
        ours.append(_timed(torch, args.steps, lambda i: product()))
        vend.append(_timed(torch, args.steps, lambda i: ad @ wb.t()))
    del wb
    torch.cuda.empty_cache()
    flops = w.flops
    res["vendor"] = {"ms": round(min(vend), 4), "TFLOP/s": round(flops / min(vend) / 1e9, 1),
                     "frac_of_peak": round(flops / min(vend) / 1e9 / MFMA_F16_PEAK_TFLOPS, 4),
                     "nvfp4_product_ms_same_turns": round(min(ours), 4),
                     "nvfp4_product_over_vendor": round(min(vend) / min(ours), 4)}
    return res


def prefill_summary(p):
    """Sub-object of the JSON line for one prefill shape."""
    w = p["w"]
    prod = p["flops"] / (p["gemm_ms"] * 1e-3) / 1e12
    stp = p["flops"] / (p["ms_step"] * 1e-3) / 1e12
    return {"workload": w.name, "M": w.M, "K": w.K, "N": w.N, "segments": list(w.seg_sizes),
            "encode": "fused SiLU(g)*u -> NVFP4" if w.silu_mul else "NVFP4 (static scale)",
            "step_ms": round(p["ms_step"], 4), "step_TFLOP/s": round(stp, 1),
            "product_ms": round(p["gemm_ms"], 4), "product_TFLOP/s": round(prod, 1),
            "frac": round(prod / MFMA_F16_PEAK_TFLOPS, 4), "bound": "mfma",
            "peak": MFMA_F16_PEAK_TFLOPS}


def decode(args, torch, nv, W):
    """Decode-shaped products M in {1, 4, 16}, K = N = 5120, NVFP4 weights resident in HBM and
    rotated over 24 byte-identical copies (354 MB, beyond the 256 MB last-level cache); the
    activations are encoded per call.

    Two timings per M: ``call_us``, the median over single calls (encode + product) between HIP
    events, launch latency included; ``kernel_us``, the product kernels alone, 24 of them (one per
    weight copy) replayed back to back from a HIP graph, total / 24.  The algorithmic bytes of the
    product are the NVFP4 weights (codes + scales), the encoded activations and the f32 output.
    ``linear``: the same step through nvfp4_linear (call and graph-replay timings as above): encode
    and product in one launch up to 6 rows at this K (M * K / 1024 <= 32), two launches above
    (where every workgroup's encode of all the rows costs more than the separate encode launch)."""
    import numpy as np

    w = W.WORKLOADS[4]
    dev = "cuda:0"
    wt = W.weights(w)
    wd = torch.from_numpy(wt).to(torch.bfloat16).to(dev)
    wc0, ws0, gw = nv.nvfp4_quantize(wd)
    del wd
    R = 24
    copies = [(wc0.clone(), ws0.clone()) for _ in range(R)]
    res = {}
    for M in (1, 4, 16):
        a = W.activations(w, M)
        ga = torch.tensor([np.float32(2688.0 / np.abs(a).max())], dtype=torch.float32, device=dev)
        ad = torch.from_numpy(a).to(torch.bfloat16).to(dev)
        ac = torch.empty((M, w.K // 2), dtype=torch.uint8, device=dev)
        as_ = torch.empty((M, w.K // 16), dtype=torch.uint8, device=dev)
        C = torch.empty((M, w.N), dtype=torch.float32, device=dev)
        for i in range(2 * R):
            nv.nvfp4_quantize(ad, ga, ac, as_)
            wc, ws = copies[i % R]
            nv.nvfp4_gemm(ac, as_, ga, wc, ws, gw, out=C)
        torch.cuda.synchronize()
        n = 10 * R
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for i in range(n):
            wc, ws = copies[i % R]
            evs[2 * i].record()
            nv.nvfp4_quantize(ad, ga, ac, as_)
            nv.nvfp4_gemm(ac, as_, ga, wc, ws, gw, out=C)
            evs[2 * i + 1].record()
        torch.cuda.synchronize()
        call_ms = sorted(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(n))[n // 2]

        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for wc, ws in copies:
                nv.nvfp4_gemm(ac, as_, ga, wc, ws, gw, out=C)
        graph.replay()
        torch.cuda.synchronize()
        reps = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        k_ms = e0.elapsed_time(e1) / (reps * R)
        del graph
        nbytes = w.N * w.K * 9 // 16 + M * w.K * 9 // 16 + M * w.N * 4
        gbs = nbytes / (k_ms * 1e-3) / 1e9
        # the same step through nvfp4_linear: the activation encode and the product in one launch
        # up to 6 rows at this K (one call per step; bytes: the bf16 activation read instead of its
        # codes)
        for i in range(2 * R):
            wc, ws = copies[i % R]
            nv.nvfp4_linear(ad, ga, wc, ws, gw, out=C, a_codes=ac, a_scales=as_)
        torch.cuda.synchronize()
        for i in range(n):
            wc, ws = copies[i % R]
            evs[2 * i].record()
            nv.nvfp4_linear(ad, ga, wc, ws, gw, out=C, a_codes=ac, a_scales=as_)
            evs[2 * i + 1].record()
        torch.cuda.synchronize()
        lcall_ms = sorted(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(n))[n // 2]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for wc, ws in copies:
                nv.nvfp4_linear(ad, ga, wc, ws, gw, out=C, a_codes=ac, a_scales=as_)
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        lk_ms = e0.elapsed_time(e1) / (reps * R)
        del graph
        lbytes = w.N * w.K * 9 // 16 + M * w.K * 2 + M * w.K * 9 // 16 + M * w.N * 4
        res[f"M{M}"] = {"kernel_us": round(k_ms * 1e3, 3), "call_us": round(call_ms * 1e3, 3),
                        "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                        "bytes": nbytes,
                        "linear": {"kernel_us": round(lk_ms * 1e3, 3),
                                   "call_us": round(lcall_ms * 1e3, 3),
                                   "GB/s": round(lbytes / (lk_ms * 1e-3) / 1e9, 1),
                                   "bytes": lbytes,
                                   "launches": 1 if M <= 6 and M * w.K <= 32 * 1024 else 2}}
    res["ceilings"] = _decode_ceilings(torch, copies, R)
    return res


def _graph_us(torch, launch, R, reps=20):
    """`launch(i)` for i = 0..R-1 captured in one HIP graph and replayed `reps` times back to back:
    microseconds per i."""
    for i in range(R):
        launch(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(R):
            launch(i)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * R)
    del graph
    return us


def _ceiling_lib():
    """The benchmark's reference kernels (a plain read in the decode kernel's launch shape, and an
    empty launch), built beside libnvfp4.so."""
    import ctypes

    path = os.path.join(ROOT, "bit_block_scaled_nvfp4_amd", "libnvfp4_ceiling.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    c_vp, c_i64 = ctypes.c_void_p, ctypes.c_int64
    lib.nvfp4_ceiling_stream_read.argtypes = [c_vp, c_i64, c_vp, c_i64, c_vp, ctypes.c_int, c_vp]
    lib.nvfp4_ceiling_stream_read.restype = ctypes.c_int
    lib.nvfp4_ceiling_empty_launch.argtypes = [c_vp]
    lib.nvfp4_ceiling_empty_launch.restype = ctypes.c_int
    return lib


def _decode_ceilings(torch, copies, R):
    """What the hardware gives for one decode weight at this size, each over the same R rotated
    copies from a HIP graph like the product:
    ``read``: a plain read of the weight's codes and scales (14.75 MB) in the decode kernel's launch
    shape (one workgroup of 512 lanes per compute unit, 16-byte loads, all in flight), folded to one
    word per wavefront -- the bytes the product reads, with no decode, product or output;
    ``empty_launch``: a kernel that does nothing, the fixed cost of one launch in a graph;
    ``vendor_copy``: torch's device copy of the codes and of the scales (reads and writes them)."""
    lib = _ceiling_lib()
    dev = copies[0][0].device
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(cus * 8, dtype=torch.int32, device=dev)
    nbytes = copies[0][0].numel() + copies[0][1].numel()

    def read(i):
        wc, ws = copies[i]
        st = lib.nvfp4_ceiling_stream_read(wc.data_ptr(), wc.numel(), ws.data_ptr(), ws.numel(),
                                           out.data_ptr(), cus, torch.cuda.current_stream().cuda_stream)
        assert st == 0, st

    def empty(i):
        st = lib.nvfp4_ceiling_empty_launch(torch.cuda.current_stream().cuda_stream)
        assert st == 0, st

    dst_c = torch.empty_like(copies[0][0])
    dst_s = torch.empty_like(copies[0][1])

    def copy(i):
        dst_c.copy_(copies[i][0])
        dst_s.copy_(copies[i][1])

    r_us = _graph_us(torch, read, R)
    e_us = _graph_us(torch, empty, R)
    c_us = _graph_us(torch, copy, R)
    return {"bytes_read": nbytes,
            "read": {"us_per_weight": round(r_us, 3), "read_GB/s": round(nbytes / r_us / 1e3, 1),
                     "workgroups": cus},
            "empty_launch_us": round(e_us, 3),
            "vendor_copy": {"us_per_weight": round(c_us, 3), "read_GB/s": round(nbytes / c_us / 1e3, 1),
                            "launches": 2}}


def decode_mlp(args, torch, nv, W):
    """Decode-shaped products on the MLP weights, M in {1, 16}: gate+up (N = 2 x 17408, K = 5120,
    two modules) and down (N = 5120, K = 17408), each one launch of the streaming kernel.  NVFP4
    weights encoded from seeded N(0, 0.02) draws, rotated over copies of about 300 MB in total
    (beyond the last-level cache); kernel time per product from HIP-graph replays, as in
    `decode`.  ``<name>_read``: a plain read of the same weight bytes over the same copies (the
    reference kernel of `decode`'s ceilings)."""
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    out = {}
    for name, N, K, segs, R in (("gate_up", 34816, 5120, [0, 17408, 34816], 3),
                                ("down", 5120, 17408, [0, 5120], 6)):
        log(f"[bench] decode on the MLP {name} weights {N}x{K}")
        wb = (torch.randn(N, K, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        parts = [nv.nvfp4_quantize(wb[lo:hi]) for lo, hi in zip(segs[:-1], segs[1:])]
        wc = torch.cat([q[0] for q in parts])
        ws = torch.cat([q[1] for q in parts])
        gw = torch.cat([q[2] for q in parts])
        del wb, parts
        copies = [(wc.clone(), ws.clone()) for _ in range(R)]
        del wc, ws
        for M in (1, 16):
            a = torch.randn(M, K, generator=gen, device=dev).to(torch.bfloat16)
            ac, as_, ga = nv.nvfp4_quantize(a)
            C = torch.empty((M, N), dtype=torch.float32, device=dev)
            for wc, ws in copies:
                nv.fused_nvfp4_gemm(ac, as_, ga, wc, ws, gw, segs, out=C)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for wc, ws in copies:
                    nv.fused_nvfp4_gemm(ac, as_, ga, wc, ws, gw, segs, out=C)
            graph.replay()
            torch.cuda.synchronize()
            reps = 10
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            k_ms = e0.elapsed_time(e1) / (reps * R)
            del graph
            nbytes = N * K * 9 // 16 + M * K * 9 // 16 + M * N * 4
            gbs = nbytes / (k_ms * 1e-3) / 1e9
            out[f"{name}_M{M}"] = {"N": N, "K": K, "kernel_us": round(k_ms * 1e3, 3),
                                   "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                   "bytes": nbytes}
        # a plain read of the same weight bytes in one launch of the decode kernels' shape
        cl = _ceiling_lib()
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        sink = torch.empty(cus * 8, dtype=torch.int32, device=dev)

        def read(i):
            wc_i, ws_i = copies[i]
            st = cl.nvfp4_ceiling_stream_read(wc_i.data_ptr(), wc_i.numel(), ws_i.data_ptr(),
                                              ws_i.numel(), sink.data_ptr(), cus,
                                              torch.cuda.current_stream().cuda_stream)
            assert st == 0, st

        r_us = _graph_us(torch, read, R, reps=10)
        wbytes = N * K * 9 // 16
        out[f"{name}_read"] = {"us": round(r_us, 3), "bytes": wbytes,
                               "read_GB/s": round(wbytes / r_us / 1e3, 1)}
        del copies
        torch.cuda.empty_cache()
    return out


def silu_quantize(args, torch, nv, W):
    """The fused SiLU(g) * u -> NVFP4 encoder on the long-prefill down projection's input
    (32768 x 17408 bf16 gate and up), static global scale.  Timed over `steps` launches back to
    back between HIP events; bytes = bf16 gate + up read, codes + scales written."""
    import numpy as np

    w = W.WORKLOADS[5]
    dev = "cuda:0"
    log(f"[bench] drawing gate/up {w.M}x{w.K} on the device")
    gd, ud = W.device_gate_up(w, dev)
    codes = torch.empty((w.M, w.K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((w.M, w.K // 16), dtype=torch.uint8, device=dev)
    _, _, ga = nv.nvfp4_silu_mul_quantize(gd, ud, None, codes, scales)  # calibration stand-in
    for _ in range(args.warmup):
        nv.nvfp4_silu_mul_quantize(gd, ud, ga, codes, scales)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        nv.nvfp4_silu_mul_quantize(gd, ud, ga, codes, scales)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = w.M * w.K * (2 + 2) + w.M * w.K * 9 // 16
    gbs = nbytes / (ms * 1e-3) / 1e9
    del gd, ud, codes, scales
    torch.cuda.empty_cache()
    return {"bound": "hbm", "shape": [w.M, w.K], "ms": round(ms, 4), "GB/s": round(gbs, 1),
            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": nbytes}


def kv_store(args, torch, nv, W):
    """The FP8 KV-cache store on a 32768-token prefill: keys and values [32768, 1024] bf16 encoded
    under static per-tensor scales (amax / 448 of an independent calibration sample, computed
    before timing) and scattered into a shuffled paged cache of 65536 slots.  Timed over `steps`
    launches back to back between HIP events, rotating over 3 copies of inputs and caches (605 MB,
    beyond the 256 MB last-level cache); bytes = bf16 keys + values read, the slot mapping read,
    the FP8 rows written.  Then the decode direction: both caches gathered back to bf16 through the
    same slots (two launches per call; bytes = FP8 rows and slots read, bf16 rows written)."""
    import numpy as np

    w = W.KV_WORKLOADS[6]
    dev = "cuda:0"
    log(f"[bench] generating {w.name}")
    k, v = W.kv_tokens(w)
    kcal, vcal = W.kv_tokens(w, 4096, calibration=True)
    ks = torch.tensor([np.float32(np.abs(kcal).max()) / np.float32(448.0)], device=dev)
    vs = torch.tensor([np.float32(np.abs(vcal).max()) / np.float32(448.0)], device=dev)
    kd = torch.from_numpy(k).to(torch.bfloat16).to(dev)
    vd = torch.from_numpy(v).to(torch.bfloat16).to(dev)
    slots = torch.from_numpy(W.kv_slot_mapping(w)).to(dev)
    R = 3
    sets = []
    for _ in range(R):
        kc = torch.zeros((w.num_slots, w.width), dtype=torch.uint8, device=dev)
        sets.append((kd.clone(), vd.clone(), kc, torch.zeros_like(kc), slots.clone()))
    del k, v, kcal, vcal, kd, vd
    for i in range(args.warmup):
        nv.nvfp4_kv_fp8_store(sets[i % R][0], sets[i % R][1], ks, vs, *sets[i % R][2:])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        nv.nvfp4_kv_fp8_store(sets[i % R][0], sets[i % R][1], ks, vs, *sets[i % R][2:])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = 2 * w.tokens * w.width * (2 + 1) + w.tokens * 8
    gbs = nbytes / (ms * 1e-3) / 1e9
    # the decode direction: gather the sequence's K and V rows back from the paged caches as bf16
    outs = [(torch.empty((w.tokens, w.width), dtype=torch.bfloat16, device=dev),
             torch.empty((w.tokens, w.width), dtype=torch.bfloat16, device=dev)) for _ in range(R)]

    def load(i):
        s_ = sets[i % R]
        nv.nvfp4_kv_fp8_load(s_[2], ks, s_[4], out=outs[i % R][0])
        nv.nvfp4_kv_fp8_load(s_[3], vs, s_[4], out=outs[i % R][1])

    for i in range(args.warmup):
        load(i)
    lms = _timed(torch, args.steps, load)
    lbytes = 2 * w.tokens * w.width * (1 + 2) + 2 * w.tokens * 8
    lgbs = lbytes / (lms * 1e-3) / 1e9
    del sets, slots, outs
    torch.cuda.empty_cache()
    return {"bound": "hbm", "tokens": w.tokens, "width": w.width, "us": round(ms * 1e3, 3),
            "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": nbytes,
            "load": {"us": round(lms * 1e3, 3), "GB/s": round(lgbs, 1),
                     "frac_hbm": round(lgbs / HBM_PEAK_GBS, 4), "bytes": lbytes,
                     "launches": 2}}


def _timed(torch, steps, fn):
    """Mean milliseconds per call of fn(i) over `steps` calls back to back between HIP events."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def error_tools(args, torch, nv, W):
    """Fake quantization, error statistics and harmonization: their throughput, and the error
    figures they produce on the synthetic workloads next to the bands the pages report.

    * fake_quantize: the 8192 x 5120 bf16 prefill activations -> f32, static scale (bytes: bf16 in,
      f32 out); 3 rotating input/output sets (755 MB, beyond the last-level cache).
    * error_stats: the same activations, 3 rotating inputs (bytes: bf16 in).
    * harmonize: the five-module GDN in_proj weight (8288 x 5120 NVFP4), 8 rotating sets (bytes:
      codes + scales read and written).
    * statistics: per-token activation error (mean over tokens of sqrt(err2 / norm2)) and the share
      of dominated blocks for the GDN in_proj and MLP gate+up activations; the weight error of each
      GDN in_proj module; the fused GDN in_proj product (M = 4096) with the exact per-module
      epilogue, after harmonization with one shared scale, and with the defective maximum scale,
      as relative Frobenius errors against the exact per-module product."""
    import numpy as np

    dev = "cuda:0"
    out = {}
    w3 = W.WORKLOADS[3]
    a = W.activations(w3)
    ga = torch.tensor([np.float32(2688.0 / np.abs(a).max())], device=dev)
    R = 3
    ins = [torch.from_numpy(a).to(torch.bfloat16).to(dev) for _ in range(R)]
    outs = [torch.empty((w3.M, w3.K), dtype=torch.float32, device=dev) for _ in range(R)]
    del a
    for i in range(args.warmup):
        nv.nvfp4_fake_quantize(ins[i % R], ga, out=outs[i % R])
    torch.cuda.synchronize()
    ms = _timed(torch, args.steps, lambda i: nv.nvfp4_fake_quantize(ins[i % R], ga, out=outs[i % R]))
    nbytes = w3.M * w3.K * (2 + 4)
    out["fake_quantize"] = {"bound": "hbm", "shape": [w3.M, w3.K], "us": round(ms * 1e3, 2),
                            "GB/s": round(nbytes / ms / 1e6, 1),
                            "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "bytes": nbytes}
    del outs
    for i in range(args.warmup):
        nv.nvfp4_quant_error_stats(ins[i % R], ga)
    torch.cuda.synchronize()
    ms = _timed(torch, args.steps, lambda i: nv.nvfp4_quant_error_stats(ins[i % R], ga))
    nbytes = w3.M * w3.K * 2
    # bound by vector-ALU work (the fake quantisation plus binary64 sums per element), not by its
    # 2 bytes per element of reads: the HBM fraction is context
    out["error_stats"] = {"bound": "valu", "shape": [w3.M, w3.K], "us": round(ms * 1e3, 2),
                          "GB/s": round(nbytes / ms / 1e6, 1),
                          "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "bytes": nbytes}
    stats = {}
    e2, n2, dom, _ = nv.nvfp4_quant_error_stats(ins[0], None)
    stats["mlp_gate_up_act_per_token_err"] = round(float(torch.sqrt(e2 / n2).mean()), 4)
    stats["mlp_gate_up_dominated_block_share"] = round(float(dom.sum()) / (w3.M * w3.K / 16), 4)
    del ins

    w2 = W.WORKLOADS[2]
    a2 = torch.from_numpy(W.activations(w2)).to(torch.bfloat16).to(dev)
    e2, n2, dom, _ = nv.nvfp4_quant_error_stats(a2, None)
    stats["gdn_in_proj_act_per_token_err"] = round(float(torch.sqrt(e2 / n2).mean()), 4)
    stats["gdn_in_proj_dominated_block_share"] = round(float(dom.sum()) / (w2.M * w2.K / 16), 4)
    segs = w2.seg_offsets
    wc = torch.empty((w2.N, w2.K // 2), dtype=torch.uint8, device=dev)
    wsc = torch.empty((w2.N, w2.K // 16), dtype=torch.uint8, device=dev)
    gw = torch.empty(len(segs) - 1, dtype=torch.float32, device=dev)
    werr = []
    for j in range(len(segs) - 1):
        wd = torch.from_numpy(W.weights(w2, slice(segs[j], segs[j + 1]))).to(torch.bfloat16).to(dev)
        _, _, g = nv.nvfp4_quantize(wd, None, wc[segs[j]:segs[j + 1]], wsc[segs[j]:segs[j + 1]])
        gw[j:j + 1].copy_(g)
        e2, n2, _, _ = nv.nvfp4_quant_error_stats(wd, g)
        werr.append(round(float(torch.sqrt(e2.sum() / n2.sum())), 4))
        del wd
    stats["gdn_in_proj_weight_err_per_module"] = werr
    ac, as_, gA = nv.nvfp4_quantize(a2)
    exact = nv.fused_nvfp4_gemm(ac, as_, gA, wc, wsc, gw, segs)
    hc, hs, gs = nv.nvfp4_harmonize_segments(wc, wsc, gw, segs)
    harm = nv.fused_nvfp4_gemm(ac, as_, gA, hc, hs, gs.repeat(len(segs) - 1), segs)
    bug = nv.fused_nvfp4_gemm(ac, as_, gA, wc, wsc, gw.max().repeat(len(segs) - 1), segs)
    nrm = torch.linalg.vector_norm(exact)
    stats["gdn_in_proj_fused_product_rel_err"] = {
        "per_module_epilogue": 0.0,
        "harmonized_shared_scale": round(float(torch.linalg.vector_norm(harm - exact) / nrm), 5),
        "defective_max_scale": round(float(torch.linalg.vector_norm(bug - exact) / nrm), 5)}
    stats["pages_bands"] = {"per_token_act_err": [0.075, 0.092], "weight_err": [0.105, 0.119],
                            "dominated_block_share": [0.10, 0.32]}
    out["statistics"] = stats
    del a2, ac, as_, exact, harm, bug, hc, hs

    RH = 8
    sets = [(wc.clone(), wsc.clone(), torch.empty_like(wc), torch.empty_like(wsc),
             torch.empty(1, dtype=torch.float32, device=dev)) for _ in range(RH)]
    for i in range(args.warmup):
        c, sc, co, so, g1 = sets[i % RH]
        nv.nvfp4_harmonize_segments(c, sc, gw, segs, co, so, g1)
    torch.cuda.synchronize()

    def harm_call(i):
        c, sc, co, so, g1 = sets[i % RH]
        nv.nvfp4_harmonize_segments(c, sc, gw, segs, co, so, g1)

    ms = _timed(torch, args.steps, harm_call)
    nbytes = 2 * w2.N * w2.K * 9 // 16
    # bound by vector-ALU work (decode, three divisions and re-encode per block): the HBM fraction
    # is context
    out["harmonize"] = {"bound": "valu", "shape": [w2.N, w2.K], "us": round(ms * 1e3, 2),
                        "GB/s": round(nbytes / ms / 1e6, 1),
                        "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "bytes": nbytes}
    del sets, wc, wsc
    torch.cuda.empty_cache()
    return out


def vendor_bf16_gemm(args, torch, W):
    """The vendor dense bf16 GEMM (torch.matmul -> hipBLASLt) on the prefill shape, M = 8192,
    K = 5120, N = 34816, operands already bf16 in HBM: a calibration of the MFMA rate this GPU
    sustains under its power limit, beside the NVFP4 product (which also decodes its operands)."""
    w = W.WORKLOADS[3]
    a = torch.randn(w.M, w.K, device="cuda:0", dtype=torch.bfloat16)
    b = torch.randn(w.N, w.K, device="cuda:0", dtype=torch.bfloat16)
    for _ in range(max(args.warmup, 2)):
        c = a @ b.t()
    torch.cuda.synchronize()
    ms = _timed(torch, args.steps, lambda i: a @ b.t())
    del a, b, c
    torch.cuda.empty_cache()
    tf = w.flops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "TFLOP/s": round(tf, 1), "frac_of_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}


def copy_calibration(args, torch):
    """A plain device-to-device copy of 1 GiB, the reference for scaling HBM byte counters:
    it reads and writes exactly 2^30 bytes per launch."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(max(args.steps, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copied {n} bytes x {max(args.steps, 1)}")


def traffic_from_profile(kernel_files, summary):
    """HBM bytes per launch recorded in a committed counter summary, or None when the summary is
    missing or the kernel's sources have changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in kernel_files:
        with open(os.path.join(ROOT, "bit_block_scaled_nvfp4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#", "|")):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != h.hexdigest():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(rows: int = 112):
    """The oracle as it stands, on a bounded sample of the same workload: encode `rows` activation
    rows and form their exact product with all 34816 output columns (the weights are encoded
    beforehand, untimed, as on the GPU).  NumPy's int64 matmul runs on one thread."""
    import numpy as np

    import oracle
    import workloads as W

    w = W.WORKLOADS[3]
    a = W.activations(w, rows)
    segs = w.seg_offsets
    wt = W.weights(w)
    wc, ws, gw = oracle.quantize_segments(wt, segs)
    del wt
    g_a = np.float32(2688.0 / np.abs(a).max())
    t0 = time.perf_counter()
    ac, as_, _ = oracle.quantize(a, g_a)
    oracle.gemm_exact(ac, as_, g_a, wc, ws, gw, segs)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    # the decode shape: one activation row encoded and multiplied by the 5120 x 5120 weight (the
    # weight encoded beforehand, untimed), as GB/s of the same algorithmic bytes as the GPU figure
    w4 = W.WORKLOADS[4]
    a4 = W.activations(w4, 1)
    wc4, ws4, gw4 = oracle.quantize(W.weights(w4))
    g4 = np.float32(2688.0 / np.abs(a4).max())
    reps = 3
    t0 = time.perf_counter()
    for _ in range(reps):
        c4, s4, _ = oracle.quantize(a4, g4)
        oracle.gemm_exact(c4, s4, g4, wc4, ws4, [gw4])
    dt4 = (time.perf_counter() - t0) / reps
    nbytes4 = w4.N * w4.K * 9 // 16 + w4.K * 9 // 16 + w4.N * 4
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "host_cpus_usable": len(os.sched_getaffinity(0)),
            "sample": f"{rows} of {w.M} activation rows x all {w.N} columns, K={w.K} "
                      f"(encode + exact int64 product), {dt:.1f} s, one thread",
            "decode": {"value": round(nbytes4 / dt4 / 1e9, 4), "unit": "GB/s", "cores": 1,
                       "sample": f"M=1 x {w4.K} x {w4.N}: encode + exact int64 product, "
                                 f"{dt4 * 1e3:.1f} ms per call, mean of {reps}"}}


# Sources of the tiled product kernel: its committed HBM counter summary is valid while they are
# unchanged.
TILED_SOURCES = ("gemm.hip", "gemm_common.h")
TILED_TRAFFIC = "gemm_tiled_mlp_gate_up_8192x5120x34816_traffic.txt"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--only", choices=("all", "prefill", "prefill_gdn", "prefill_down", "decode",
                                      "silu", "kv", "errors", "vendor", "copy"),
                    default="all",
                    help="run one part (for profiler runs); 'copy' is the counter calibration copy")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the hot path here is the single-GPU W4A4 linear "
              "layer, and multi-GPU runs are not part of this build (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_block_scaled_nvfp4_amd as nv
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    nv.load_library()

    if args.only == "copy":
        copy_calibration(args, torch)
        return
    if args.only == "decode":
        print(json.dumps({"decode": decode(args, torch, nv, W),
                          "decode_mlp": decode_mlp(args, torch, nv, W)}), flush=True)
        return
    if args.only == "silu":
        print(json.dumps({"silu_mul_quantize": silu_quantize(args, torch, nv, W)}), flush=True)
        return
    if args.only == "kv":
        print(json.dumps({"kv_fp8_store": kv_store(args, torch, nv, W)}), flush=True)
        return
    if args.only == "errors":
        print(json.dumps(error_tools(args, torch, nv, W)), flush=True)
        return
    if args.only == "vendor":
        print(json.dumps({"vendor_bf16_gemm": vendor_bf16_gemm(args, torch, W)}), flush=True)
        return

    if args.only == "prefill_gdn":
        print(json.dumps({"prefill_gdn": prefill_summary(prefill(args, torch, nv, W, 2))}), flush=True)
        return
    if args.only == "prefill_down":
        print(json.dumps({"prefill_down": prefill_summary(prefill(args, torch, nv, W, 5))}), flush=True)
        return

    p = prefill(args, torch, nv, W, 3)
    run_rest = args.only == "all"
    gdn = prefill_summary(prefill(args, torch, nv, W, 2)) if run_rest else None
    down = prefill_summary(prefill(args, torch, nv, W, 5)) if run_rest else None
    dec = decode(args, torch, nv, W) if run_rest and not args.no_decode else None
    dec_mlp = decode_mlp(args, torch, nv, W) if run_rest and not args.no_decode else None
    silu = silu_quantize(args, torch, nv, W) if run_rest else None
    kv = kv_store(args, torch, nv, W) if run_rest else None
    errs = error_tools(args, torch, nv, W) if run_rest else None
    cpu = cpu_baseline() if run_rest and not args.no_cpu_baseline else None

    w = p["w"]
    value = p["flops"] / (p["ms_step"] * 1e-3) / 1e12
    achieved = p["flops"] / (p["gemm_ms"] * 1e-3) / 1e12
    q_gbs = p["q_bytes"] / (p["quant_ms"] * 1e-3) / 1e9
    qd_gbs = p["qd_bytes"] / (p["quant_dyn_ms"] * 1e-3) / 1e9
    line = {
        "metric": "NVFP4 W4A4 GEMM TFLOP/s (prefill M=8192) + decode GB/s, % of MI355X roofline",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(p["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1 + e4m3/16) operands decoded exactly to f16, f16 MFMA, f32 accumulate",
        "data": "synthetic (seeded, drawn on the device; bf16 N(0,1) activations with 1% "
                "Student-t(3)x50 channels, N(0,0.02) weights)",
        "config": {"workload": w.name, "M": w.M, "K": w.K, "N": w.N,
                   "segments": list(w.seg_sizes), "act_scale": "static", "output": "f32"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profile(TILED_SOURCES, TILED_TRAFFIC),
                     "kernel": "gemm_tiled_kernel (fused_nvfp4_gemm)",
                     "kernel_ms": round(p["gemm_ms"], 4),
                     "frac_of_mxfp4_peak": round(achieved / MFMA_FP4_PEAK_TFLOPS, 4)},
        "prefill_gdn": gdn,
        "prefill_down": down,
        "quantize": {"bound": "hbm", "ms": round(p["quant_ms"], 4), "GB/s": round(q_gbs, 1),
                     "frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4), "bytes": int(p["q_bytes"]),
                     "rotating_sets": p["quant_sets"],
                     "dynamic": {"ms": round(p["quant_dyn_ms"], 4), "GB/s": round(qd_gbs, 1),
                                 "frac_hbm": round(qd_gbs / HBM_PEAK_GBS, 4),
                                 "bytes": int(p["qd_bytes"])}},
        "decode": dec,
        "decode_mlp": dec_mlp,
        "silu_mul_quantize": silu,
        "kv_fp8_store": kv,
        "fake_quantize": errs and errs["fake_quantize"],
        "error_stats": errs and errs["error_stats"],
        "harmonize": errs and errs["harmonize"],
        "error_statistics": errs and errs["statistics"],
        "vendor_bf16_gemm": p["vendor"],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
