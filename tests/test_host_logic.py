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

    val = bench.traffic_from_profile(bench.TILED_SOURCES, bench.TILED_TRAFFIC)
    assert val is not None and val > 1e9
    # a summary whose hash does not match the sources is ignored
    fake = tmp_path / "profiles"
    fake.mkdir()
    with open(os.path.join(ROOT, "profiles", bench.TILED_TRAFFIC)) as fh:
        text = fh.read()
    h = hashlib.sha256()
    for f in bench.TILED_SOURCES:
        with open(os.path.join(ROOT, "bit_block_scaled_nvfp4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    assert h.hexdigest() in text
    (fake / bench.TILED_TRAFFIC).write_text(text.replace(h.hexdigest(), "0" * 64))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # sources are read relative to ROOT: link them in so only the summary differs
    (tmp_path / "bit_block_scaled_nvfp4_amd").symlink_to(os.path.join(ROOT, "bit_block_scaled_nvfp4_amd"))
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
