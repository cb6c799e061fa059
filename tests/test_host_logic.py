"""Host-side logic that needs no GPU: the seeded input generators' reproducibility guarantees, the
benchmark's counter-summary check and its refusal of multi-GPU runs, and the binding's argument
checks that happen before any library call."""

import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_activation_rows_reproduce_from_any_offset():
    w = W.WORKLOADS[2]
    full = W.activations(w, 600)
    part = W.activations(w, 300, row0=250)
    assert np.array_equal(part, full[250:550])
    assert W.activations(w, 0).shape == (0, w.K)


def test_weight_rows_reproduce_and_segments_carry_their_spread():
    w = W.WORKLOADS[2]
    rows = W.weights(w, slice(8190, 8288))  # the last (decay- and write-gate) segments
    assert np.array_equal(rows, W.weights(w, slice(8000, 8288))[190:])
    a_seg = rows[50:98]  # segment 4 (write gate): std x1
    b_seg = rows[2:50]   # segment 3 (decay gate): std x2.75
    ratio = np.abs(b_seg).max() / np.abs(a_seg).max()
    assert 1.8 < ratio < 4.0


def test_gate_up_and_kv_tokens_reproduce_from_any_offset():
    w5 = W.WORKLOADS[5]
    g, u = W.gate_up(w5, 300)
    g2, u2 = W.gate_up(w5, 100, row0=200)
    assert np.array_equal(g2, g[200:300]) and np.array_equal(u2, u[200:300])
    kw = W.KV_WORKLOADS[6]
    k, v = W.kv_tokens(kw, 600)
    k2, v2 = W.kv_tokens(kw, 200, row0=300)
    assert np.array_equal(k2, k[300:500]) and np.array_equal(v2, v[300:500])
    kc, _ = W.kv_tokens(kw, 600, calibration=True)
    assert not np.array_equal(kc, k)  # the calibration sample is an independent draw


def test_kv_slot_mapping_is_a_paged_injection():
    kw = W.KV_WORKLOADS[6]
    s = W.kv_slot_mapping(kw)
    assert len(s) == kw.tokens and len(np.unique(s)) == kw.tokens
    assert s.min() >= 0 and s.max() < kw.num_slots
    # consecutive tokens of a block sit in consecutive slots of one cache block
    assert np.all((s[1:16] - s[0]) == np.arange(1, 16))
    assert np.all(s % kw.block_size == np.arange(kw.tokens) % kw.block_size)
    with pytest.raises(ValueError):
        W.kv_slot_mapping(kw, kw.num_slots + 1)


def test_silu_workload_refuses_to_draw_its_activation():
    with pytest.raises(ValueError):
        W.activations(W.WORKLOADS[5], 4)


def test_bf16_inputs_are_exact_bf16_values():
    x = W.activations(W.WORKLOADS[3], 64)
    assert np.all((x.view(np.uint32) & 0xFFFF) == 0)


def test_traffic_summary_is_used_only_while_the_kernel_sources_match(tmp_path, monkeypatch):
    import bench

    h = hashlib.sha256()
    for f in bench.TILED_SOURCES:
        with open(os.path.join(ROOT, "bit_block_scaled_nvfp4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    fake = tmp_path / "profiles"
    fake.mkdir()
    # sources are read relative to ROOT: link them in so only the summary differs
    (tmp_path / "bit_block_scaled_nvfp4_amd").symlink_to(os.path.join(ROOT, "bit_block_scaled_nvfp4_amd"))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    body = "# summary\ncommand: x\ntraffic_bytes_per_launch: 2446000000\nkernel_source_sha256: {}\n"
    (fake / bench.TILED_TRAFFIC).write_text(body.format(h.hexdigest()))
    assert bench.traffic_from_profile(bench.TILED_SOURCES, bench.TILED_TRAFFIC) == 2446000000.0
    # a summary whose hash does not match the sources is ignored
    (fake / bench.TILED_TRAFFIC).write_text(body.format("0" * 64))
    assert bench.traffic_from_profile(bench.TILED_SOURCES, bench.TILED_TRAFFIC) is None
    assert bench.traffic_from_profile(bench.TILED_SOURCES, "missing.txt") is None


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_binding_checks_shapes_before_calling_the_library():
    torch = pytest.importorskip("torch")
    import bit_block_scaled_nvfp4_amd as nv

    if not os.path.exists(nv.LIB_PATH):
        pytest.skip("libnvfp4.so not built")

    x = torch.zeros(4, 32)
    with pytest.raises(ValueError):
        nv.nvfp4_quantize(x)  # CPU tensor
    with pytest.raises(ValueError):
        nv.nvfp4_silu_mul_quantize(torch.zeros(4, 32), torch.zeros(4, 48))
    with pytest.raises(ValueError):
        nv.nvfp4_kv_fp8_store(torch.zeros(4, 32), None, torch.ones(1), None, torch.zeros(4, 32,
                              dtype=torch.uint8), None)


def test_binding_rejects_malformed_operands_before_the_device_check():
    """Every shape, dtype and layout check of the binding fires on CPU tensors, before the device
    check: a wrongly sized or strided operand never reaches the library, which takes bare pointers
    and would read or write out of bounds."""
    torch = pytest.importorskip("torch")
    import bit_block_scaled_nvfp4_amd as nv

    if not os.path.exists(nv.LIB_PATH):
        pytest.skip("libnvfp4.so not built")
    u8, f32 = torch.uint8, torch.float32
    M, N, K = 4, 24, 64
    ac, as_ = torch.zeros(M, K // 2, dtype=u8), torch.zeros(M, K // 16, dtype=u8)
    wc, ws = torch.zeros(N, K // 2, dtype=u8), torch.zeros(N, K // 16, dtype=u8)
    g1, g2 = torch.ones(1), torch.ones(2)

    def gemm_raises(match, **kw):
        a = dict(a_codes=ac, a_scales=as_, a_gscale=g1, w_codes=wc, w_scales=ws, w_gscale=g1)
        a.update(kw)
        with pytest.raises(ValueError, match=match):
            nv.nvfp4_gemm(**a)

    gemm_raises("a_scales must have shape", a_scales=torch.zeros(M, K // 16 + 1, dtype=u8))
    gemm_raises("w_scales must have shape", w_scales=torch.zeros(N - 1, K // 16, dtype=u8))
    gemm_raises("w_codes must be uint8", w_codes=torch.zeros(N, K // 2, dtype=torch.int8))
    gemm_raises("a_codes must be row-contiguous",
                a_codes=torch.zeros(M, K, dtype=u8)[:, : K // 2])
    gemm_raises("disagree on K", w_codes=torch.zeros(N, K // 2 + 8, dtype=u8))
    gemm_raises("multiple of 16", a_codes=torch.zeros(M, 36, dtype=u8),
                w_codes=torch.zeros(N, 36, dtype=u8))
    gemm_raises("a_gscale must be float32", a_gscale=torch.ones(1, dtype=torch.float64))
    gemm_raises("out must have shape", out=torch.zeros(M, N + 1))
    gemm_raises("out must have dtype", out=torch.zeros(M, N, dtype=torch.float16))
    gemm_raises("out must have contiguous rows", out=torch.zeros(N, M).t())
    gemm_raises("tensors must live on the GPU")  # well formed, but on the host

    def fused_raises(match, segs=(0, 8, N), seg_g=g2, **kw):
        with pytest.raises(ValueError, match=match):
            nv.fused_nvfp4_gemm(ac, as_, g1, wc, ws, seg_g, list(segs), **kw)

    fused_raises("segment global scales must hold 3", segs=(0, 8, 16, N))
    fused_raises("segment global scales must hold 2", seg_g=torch.ones(4)[::2])
    fused_raises("between 1 and 16 segments", segs=tuple(range(0, 18)) + (N,), seg_g=torch.ones(18))
    fused_raises("tensors must live on the GPU")

    x = torch.zeros(M, K)
    with pytest.raises(ValueError, match="codes must have shape"):
        nv.nvfp4_quantize(x, g1, torch.zeros(M, K // 2 - 1, dtype=u8))
    with pytest.raises(ValueError, match="scales must be row-contiguous"):
        nv.nvfp4_quantize(x, g1, torch.zeros(M, K // 2, dtype=u8),
                          torch.zeros(M, K // 8, dtype=u8)[:, ::2])
    with pytest.raises(ValueError, match="multiple of 16 columns"):
        nv.nvfp4_quantize(torch.zeros(M, 40))
    with pytest.raises(ValueError, match="x must be float32, bfloat16 or float16"):
        nv.nvfp4_quantize(torch.zeros(M, K, dtype=torch.float64))
    with pytest.raises(ValueError, match="global_scale must be float32"):
        nv.nvfp4_quantize(x, torch.ones(1, dtype=torch.float16))
    with pytest.raises(ValueError, match="codes must have shape"):
        nv.nvfp4_silu_mul_quantize(x, x, g1, torch.zeros(M + 1, K // 2, dtype=u8))
    with pytest.raises(ValueError, match="out must have shape"):
        nv.nvfp4_fake_quantize(x, g1, out=torch.zeros(M, K - 16))
    with pytest.raises(ValueError, match="scales must have shape"):
        nv.nvfp4_requantize(ac, torch.zeros(M, K // 32, dtype=u8), g1, g1)
    with pytest.raises(ValueError, match="codes_out must have shape"):
        nv.nvfp4_requantize(ac, as_, g1, g1, codes_out=torch.zeros(M, K // 4, dtype=u8))
    with pytest.raises(ValueError, match="seg_gscale must hold 2"):
        nv.nvfp4_harmonize_segments(wc, ws, g1, [0, 8, N])
    with pytest.raises(ValueError, match="cache must be 2-D uint8"):
        nv.nvfp4_kv_fp8_load(torch.zeros(8, 32), g1)
    with pytest.raises(ValueError, match="exceeds the cache row"):
        nv.nvfp4_kv_fp8_load(torch.zeros(8, 32, dtype=u8), g1, width=48)
    with pytest.raises(ValueError, match="value needs value_scale"):
        nv.nvfp4_kv_fp8_store(x, x, g1, None, torch.zeros(8, K, dtype=u8), None)
