"""Seeded synthetic inputs for the NVFP4 W4A4 linear layer.

Shared by the tests, the benchmark and the smoke check: the oracle and the HIP path are fed the same
bits from here.  This module holds no arithmetic of the method (no quantisation, no product); it
only draws random tensors with the shapes, value distributions and outlier structure of the five
workloads below, and rounds them once to bf16 with PyTorch's CPU round-to-nearest-even cast where
the workload is bf16.

Random streams: ``numpy.random.Generator(PCG64(1000 * workload + tensor_id))`` with tensor ids
1 = activations, 2 = weights, 3 = outlier-channel indices, 4 = second activation factor / t draws.

Statistics imitated (ai.info summary of arXiv 2609.04098, "Main Findings"): residual-stream inputs
carry extreme outliers on a few hot channels (hot channels about 100x the median channel), and a
sizeable share of 16-element blocks is dominated by a single value.  The workload shapes follow the
hybrid model's projections named on the same page (fused GDN in_proj, MLP gate+up and down
projections, decode GEMV).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WEIGHT_STD = np.float32(0.02)


@dataclass(frozen=True)
class Workload:
    """Shape and recipe of one synthetic workload."""

    wid: int
    name: str
    M: int
    K: int
    N: int
    seg_sizes: tuple  # output-column segments, one per calibrated module
    act_dtype: str  # "f32" or "bf16" (what the quantiser reads)
    w_dtype: str
    outlier_frac: float
    outlier_gain: float
    outlier_kind: str  # "scale" (N(0,1) * gain) or "t3" (gain * Student-t, 3 dof) or "none"
    seg_std_mult: tuple = field(default=())  # per-segment weight std multipliers
    silu_mul: bool = False  # activations = SiLU(g) * u

    @property
    def seg_offsets(self):
        off = [0]
        for s in self.seg_sizes:
            off.append(off[-1] + s)
        return off

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    # Single quantise + W4A4 GEMM, fp32 inputs, 0.5% of K-channels x100.
    1: Workload(1, "single_64x512x256", 64, 512, 256, (256,), "f32", "f32", 0.005, 100.0, "scale"),
    # Fused GDN input projection q,k,v,decay-gate,write-gate; a/b pair with a 2.75x scale ratio.
    2: Workload(2, "gdn_in_proj_4096x5120x8288", 4096, 5120, 8288, (2048, 2048, 4096, 48, 48),
                "bf16", "bf16", 0.01, 50.0, "scale", seg_std_mult=(1.0, 1.0, 1.0, 2.75, 1.0)),
    # Fused MLP gate+up, heavy-tailed outlier channels.
    3: Workload(3, "mlp_gate_up_8192x5120x34816", 8192, 5120, 34816, (17408, 17408),
                "bf16", "bf16", 0.01, 50.0, "t3"),
    # Decode-shaped skinny GEMM (M is 1, 4 or 16).
    4: Workload(4, "decode_Mx5120x5120", 16, 5120, 5120, (5120,), "bf16", "bf16", 0.01, 50.0,
                "scale"),
    # Long-prefill MLP down projection on SiLU(g)*u activations.
    5: Workload(5, "mlp_down_32768x17408x5120", 32768, 17408, 5120, (5120,), "bf16", "bf16",
                0.0, 1.0, "none", silu_mul=True),
}


def _rng(wid: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * wid + tensor_id))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (PyTorch CPU cast, nearest-even) and widen back exactly."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def outlier_channels(w: Workload) -> np.ndarray:
    n = int(round(w.outlier_frac * w.K))
    if n == 0 or w.outlier_kind == "none":
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(w.wid, 3).choice(w.K, size=n, replace=False))


def activations(w: Workload, M: int | None = None, row0: int = 0) -> np.ndarray:
    """Activation rows ``[row0, row0 + M)`` of workload ``w`` as float32 holding values of the
    workload's dtype.  Rows are drawn in fixed 256-row chunks so any row range reproduces the same
    values as the full tensor."""
    M = w.M if M is None else M
    if M == 0:
        return np.zeros((0, w.K), dtype=np.float32)
    chunk = 256
    c0, c1 = row0 // chunk, (row0 + M + chunk - 1) // chunk
    parts = [_activation_chunk(w, c, chunk) for c in range(c0, c1)]
    full = np.concatenate(parts, axis=0)
    off = row0 - c0 * chunk
    return np.ascontiguousarray(full[off:off + M])


def _activation_chunk(w: Workload, c: int, chunk: int) -> np.ndarray:
    # One independent substream per 256-row chunk (jumped PCG64), so chunks are reproducible alone.
    bitgen = np.random.PCG64(1000 * w.wid + 1).jumped(c)
    rng = np.random.Generator(bitgen)
    rows = chunk
    if w.silu_mul:
        raise ValueError(
            f"workload {w.name}: its activation is SiLU(g) * u, a step of the method -- draw the "
            "inputs with gate_up() and form the activation with the encoder under test")
    else:
        x = rng.standard_normal((rows, w.K), dtype=np.float32)
        ch = outlier_channels(w)
        if len(ch):
            if w.outlier_kind == "scale":
                x[:, ch] *= np.float32(w.outlier_gain)
            elif w.outlier_kind == "t3":
                trng = np.random.Generator(np.random.PCG64(1000 * w.wid + 4).jumped(c))
                x[:, ch] = np.float32(w.outlier_gain) * trng.standard_t(3, (rows, len(ch))).astype(
                    np.float32)
    x = x.astype(np.float32)
    return round_bf16(x) if w.act_dtype == "bf16" else x


def gate_up(w: Workload, M: int | None = None, row0: int = 0):
    """Gate and up projections ``(g, u)`` (rows ``[row0, row0 + M)``, float32 arrays holding
    bfloat16 values, each element drawn N(0, 1)) of a workload whose activation is SiLU(g) * u.
    Rows are drawn in fixed 256-row chunks so any row range reproduces the full tensors."""
    if not w.silu_mul:
        raise ValueError(f"workload {w.name} has no gate/up inputs")
    M = w.M if M is None else M
    if M == 0:
        z = np.zeros((0, w.K), dtype=np.float32)
        return z, z.copy()
    chunk = 256
    c0, c1 = row0 // chunk, (row0 + M + chunk - 1) // chunk
    gs, us = [], []
    for c in range(c0, c1):
        rng = np.random.Generator(np.random.PCG64(1000 * w.wid + 1).jumped(c))
        gs.append(rng.standard_normal((chunk, w.K), dtype=np.float32))
        us.append(rng.standard_normal((chunk, w.K), dtype=np.float32))
    off = row0 - c0 * chunk
    g = np.concatenate(gs, axis=0)[off:off + M]
    u = np.concatenate(us, axis=0)[off:off + M]
    return round_bf16(np.ascontiguousarray(g)), round_bf16(np.ascontiguousarray(u))


def weights(w: Workload, rows: slice | None = None) -> np.ndarray:
    """Weight matrix ``[N, K]`` (nn.Linear layout) as float32 holding values of the weight dtype.
    ``rows`` selects a row range without drawing the whole matrix (256-row substreams)."""
    rows = slice(0, w.N) if rows is None else rows
    r0, r1 = rows.start or 0, w.N if rows.stop is None else rows.stop
    chunk = 256
    c0, c1 = r0 // chunk, (r1 + chunk - 1) // chunk
    parts = []
    mult = _row_std_mult(w)
    for c in range(c0, c1):
        rng = np.random.Generator(np.random.PCG64(1000 * w.wid + 2).jumped(c))
        lo, hi = c * chunk, min((c + 1) * chunk, w.N)
        x = rng.standard_normal((chunk, w.K), dtype=np.float32)[: hi - lo]
        x *= (WEIGHT_STD * mult[lo:hi])[:, None]
        parts.append(x)
    full = np.concatenate(parts, axis=0) if parts else np.zeros((0, w.K), np.float32)
    out = np.ascontiguousarray(full[r0 - c0 * chunk: r1 - c0 * chunk])
    return round_bf16(out) if w.w_dtype == "bf16" else out


def _row_std_mult(w: Workload) -> np.ndarray:
    mult = np.ones(w.N, dtype=np.float32)
    if w.seg_std_mult:
        off = w.seg_offsets
        for j, m in enumerate(w.seg_std_mult):
            mult[off[j]:off[j + 1]] = np.float32(m)
    return mult


def random_matrix(seed: int, rows: int, cols: int, std: float = 1.0, outlier_cols: int = 0,
                  outlier_gain: float = 50.0, dtype: str = "f32") -> np.ndarray:
    """Small seeded N(0, std^2) matrix with optional hot columns, for ragged/edge-case tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    if outlier_cols and cols:
        ch = rng.choice(cols, size=min(outlier_cols, cols), replace=False)
        x[:, ch] *= np.float32(outlier_gain)
    return round_bf16(x) if dtype == "bf16" else x


# ---- FP8 KV cache --------------------------------------------------------------------------


@dataclass(frozen=True)
class KvWorkload:
    """Keys and values of new tokens written into a paged FP8 KV cache.

    Shape (reading; the pages give the attention layers' count, 16, and the context, 32K, but no
    head shape): a prefill of ``tokens`` tokens, rows of ``width`` = heads * head_dim elements for
    each of K and V, a paged cache of ``num_blocks`` blocks of ``block_size`` slots whose blocks the
    sequence occupies in a shuffled order.  Keys carry a few hot channels; values do not."""

    wid: int
    name: str
    tokens: int
    width: int
    block_size: int
    num_blocks: int
    key_outlier_frac: float
    key_outlier_gain: float

    @property
    def num_slots(self) -> int:
        return self.num_blocks * self.block_size


KV_WORKLOADS = {
    # 32K-token prefill, 4 KV heads x 256 dims, bf16 keys/values, 2% of key channels x8.
    6: KvWorkload(6, "kv_fp8_store_32768x1024", 32768, 1024, 16, 4096, 0.02, 8.0),
}


def kv_key_channels(w: KvWorkload) -> np.ndarray:
    n = int(round(w.key_outlier_frac * w.width))
    return np.sort(_rng(w.wid, 3).choice(w.width, size=n, replace=False))


def kv_tokens(w: KvWorkload, tokens: int | None = None, row0: int = 0, calibration=False):
    """Keys and values ``(k, v)`` of tokens ``[row0, row0 + tokens)`` as float32 arrays holding
    bfloat16 values: N(0, 1), key hot channels times the gain.  ``calibration=True`` draws an
    independent sample of the same distribution (the calibration set).  256-token chunks, so any
    range reproduces the full tensors."""
    tokens = w.tokens if tokens is None else tokens
    if tokens == 0:
        z = np.zeros((0, w.width), dtype=np.float32)
        return z, z.copy()
    chunk = 256
    c0, c1 = row0 // chunk, (row0 + tokens + chunk - 1) // chunk
    ch = kv_key_channels(w)
    ks, vs = [], []
    for c in range(c0, c1):
        rng = np.random.Generator(np.random.PCG64(1000 * w.wid + (5 if calibration else 1)).jumped(c))
        k = rng.standard_normal((chunk, w.width), dtype=np.float32)
        k[:, ch] *= np.float32(w.key_outlier_gain)
        ks.append(k)
        vs.append(rng.standard_normal((chunk, w.width), dtype=np.float32))
    off = row0 - c0 * chunk
    k = np.concatenate(ks, axis=0)[off:off + tokens]
    v = np.concatenate(vs, axis=0)[off:off + tokens]
    return round_bf16(np.ascontiguousarray(k)), round_bf16(np.ascontiguousarray(v))


def kv_slot_mapping(w: KvWorkload, tokens: int | None = None) -> np.ndarray:
    """Cache slot of each token (int64): token t sits at position t % block_size of the
    sequence's (t // block_size)-th block, and the sequence's blocks are a seeded random choice of
    the cache's blocks."""
    tokens = w.tokens if tokens is None else tokens
    nblk = (tokens + w.block_size - 1) // w.block_size
    if nblk > w.num_blocks:
        raise ValueError("the cache is too small for this many tokens")
    table = _rng(w.wid, 2).permutation(w.num_blocks)[:nblk].astype(np.int64)
    t = np.arange(tokens, dtype=np.int64)
    return table[t // w.block_size] * w.block_size + t % w.block_size


def random_nvfp4_bytes(seed: int, rows: int, cols: int, zero_block_frac: float = 0.05):
    """Random encoded operand bytes, not produced by any encoder: ``codes [rows, cols/2]`` uint8
    with every nibble 0x0..0xF equally likely (0x8 is the signed zero), and ``scales
    [rows, cols/16]`` uint8 drawn uniformly from the 127 finite non-negative E4M3 codes 0x00..0x7E
    (zero, the seven subnormals and every normal value up to 448).  A ``zero_block_frac`` share of
    blocks is then made all zero: half of them by zero codes under a random scale (mixing 0x0 and
    0x8), half by a zero scale under random codes.  The first row holds every scale code in turn
    (none of its blocks is zeroed)."""
    if cols % 16 != 0:
        raise ValueError("cols must be a multiple of 16")
    rng = np.random.Generator(np.random.PCG64(seed))
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (rows, cols // 16), dtype=np.uint8)
    nb = cols // 16
    if rows > 0:
        scales[0] = np.arange(nb) % 0x7F
    pick = rng.random((rows, nb)) < zero_block_frac
    pick[:1] = False
    by_codes = pick & (rng.random((rows, nb)) < 0.5)
    by_scale = pick & ~by_codes
    zc = rng.choice(np.array([0x00, 0x08, 0x80, 0x88], np.uint8), size=(rows, cols // 2))
    codes = np.where(np.repeat(by_codes, 8, axis=1), zc, codes)
    scales = np.where(by_scale, np.uint8(0), scales)
    return np.ascontiguousarray(codes, np.uint8), np.ascontiguousarray(scales, np.uint8)


# ---- the same recipes drawn on the device ----------------------------------------------------
#
# The benchmark draws its large inputs directly on the GPU with torch's seeded generator, so that a
# run does not spend most of its time generating gigabytes on the host.  The distributions are the
# ones above (same outlier channels, gains, segment spreads, bf16 rounding by torch's
# nearest-even cast); the random streams differ from the host draws, which the parity tests use.


def _device_gen(device, seed: int):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_activations(w: Workload, device, M: int | None = None):
    """Activations ``[M, K]`` bf16 (or f32) on ``device``: N(0,1), the workload's outlier channels
    scaled by its gain (``scale``) or replaced by gain * Student-t(3) draws (``t3``)."""
    import torch

    if w.silu_mul:
        raise ValueError("this workload's activation is SiLU(g) * u: draw gate and up instead")
    M = w.M if M is None else M
    gen = _device_gen(device, 1000 * w.wid + 11)
    x = torch.randn((M, w.K), generator=gen, device=device, dtype=torch.float32)
    ch = torch.from_numpy(outlier_channels(w)).to(device)
    if len(ch):
        if w.outlier_kind == "scale":
            x[:, ch] *= w.outlier_gain
        elif w.outlier_kind == "t3":
            z = torch.randn((M, len(ch)), generator=gen, device=device)
            chi2 = (torch.randn((M, len(ch), 3), generator=gen, device=device) ** 2).sum(-1)
            x[:, ch] = w.outlier_gain * z / torch.sqrt(chi2 / 3.0)
    return x.to(torch.bfloat16) if w.act_dtype == "bf16" else x


def device_gate_up(w: Workload, device, M: int | None = None):
    """Gate and up inputs ``[M, K]`` of a SiLU(g) * u workload on ``device``, bf16 N(0,1)."""
    import torch

    M = w.M if M is None else M
    gen = _device_gen(device, 1000 * w.wid + 14)
    g = torch.randn((M, w.K), generator=gen, device=device).to(torch.bfloat16)
    u = torch.randn((M, w.K), generator=gen, device=device).to(torch.bfloat16)
    return g, u


def device_weights(w: Workload, device, rows: slice | None = None):
    """Weight rows ``[N, K]`` on ``device``: N(0, 0.02) times the segment spread, bf16 (or f32)."""
    import torch

    rows = slice(0, w.N) if rows is None else rows
    r0, r1 = rows.start or 0, w.N if rows.stop is None else rows.stop
    gen = _device_gen(device, 1000 * w.wid + 12 + 7919 * r0)
    x = torch.randn((r1 - r0, w.K), generator=gen, device=device, dtype=torch.float32)
    mult = torch.from_numpy(_row_std_mult(w)[r0:r1] * WEIGHT_STD).to(device)
    x *= mult[:, None]
    return x.to(torch.bfloat16) if w.w_dtype == "bf16" else x
