"""Helpers for the GPU parity tests: upload seeded inputs, call the C ABI through the binding,
compare against the oracle with the stated tolerance."""

from __future__ import annotations

import sys

import numpy as np

import bit_block_scaled_nvfp4_amd as nv
import oracle

DEV = "cuda:0"

# GEMM acceptance: per element |C_gpu - C_ref| <= ELEM_TOL * sum_k |a*w| / (gA gW), and
# ||C_gpu - C_ref||_F <= FRO_TOL * ||C_ref||_F.
ELEM_TOL = 1e-4
FRO_TOL = 1e-5


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, dtype: str):
    """float32 array holding values of ``dtype`` -> device tensor of that dtype (exact)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    t = t.to(tdt)
    if not np.array_equal(t.to(torch.float32).numpy(), x):
        raise ValueError(f"values are not exactly representable in {dtype}")
    return t.to(DEV)


def scalar(v: float):
    import torch

    return torch.tensor([np.float32(v)], dtype=torch.float32, device=DEV)


def gpu_quantize(x: np.ndarray, dtype: str, g=None):
    """Quantise on the GPU; returns numpy (codes, scales, g)."""
    import torch

    xd = to_device(x, dtype)
    gd = None if g is None else scalar(g)
    c, s, gg = nv.nvfp4_quantize(xd, gd)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy(), np.float32(gg.cpu().numpy()[0])


def assert_codes_equal(got, ref, what):
    gc, gs, gg = got
    rc, rs, rg = ref
    assert gg == rg, f"{what}: global scale {gg!r} != {rg!r}"
    bad = np.argwhere(gs != rs)
    assert bad.size == 0, (f"{what}: {len(bad)} scale bytes differ, first at {bad[0].tolist()}: "
                           f"{gs[tuple(bad[0])]:#x} vs {rs[tuple(bad[0])]:#x}")
    bad = np.argwhere(gc != rc)
    assert bad.size == 0, (f"{what}: {len(bad)} code bytes differ, first at {bad[0].tolist()}: "
                           f"{gc[tuple(bad[0])]:#x} vs {rc[tuple(bad[0])]:#x}")


def check_gemm(C_gpu: np.ndarray, C_ref: np.ndarray, B_ref: np.ndarray, what: str,
               elem_tol=ELEM_TOL, fro_tol=FRO_TOL):
    C_gpu = C_gpu.astype(np.float64)
    assert C_gpu.shape == C_ref.shape
    assert np.all(np.isfinite(C_gpu)), f"{what}: non-finite output"
    err = np.abs(C_gpu - C_ref)
    lim = elem_tol * B_ref
    bad = np.argwhere(err > lim)
    assert bad.size == 0, (f"{what}: {len(bad)} elements out of tolerance, first {bad[0].tolist()}: "
                           f"gpu={C_gpu[tuple(bad[0])]!r} ref={C_ref[tuple(bad[0])]!r} "
                           f"bound={lim[tuple(bad[0])]!r}")
    nref = np.linalg.norm(C_ref)
    if nref > 0:
        rel = np.linalg.norm(C_gpu - C_ref) / nref
        assert rel <= fro_tol, f"{what}: relative Frobenius error {rel:.3e} > {fro_tol}"
    else:
        assert np.all(C_gpu == 0)
    return float(np.max(err / np.maximum(B_ref, 1e-300))) if err.size else 0.0


def oracle_product(ac, as_, ga, wc, ws, seg_g, segs, threads: int = 16):
    """The oracle's exact product and its tolerance scale, ``(gemm_exact, gemm_abs_bound)``, formed
    over blocks of rows in a thread pool (NumPy's int64 matmul runs on one core but releases the
    interpreter lock); each block is exactly the oracle's own call on those rows."""
    from concurrent.futures import ThreadPoolExecutor

    M = ac.shape[0]
    step = max(1, -(-M // threads))
    blocks = [(r, min(M, r + step)) for r in range(0, M, step)]

    def run(b):
        lo, hi = b
        return (oracle.gemm_exact(ac[lo:hi], as_[lo:hi], ga, wc, ws, seg_g, segs),
                oracle.gemm_abs_bound(ac[lo:hi], as_[lo:hi], ga, wc, ws, seg_g, segs))

    with ThreadPoolExecutor(max_workers=min(threads, len(blocks))) as ex:
        parts = list(ex.map(run, blocks))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
