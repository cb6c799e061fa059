"""The C-ABI library (CPU side): it loads, exports every function include/nvfp4.h declares, and
rejects every malformed call with the documented status before touching the device.

These tests pass fake but aligned device addresses: every call here fails validation (or is an
empty problem), so no HIP call is made and no GPU is needed.
"""

import ctypes
import os
import re
import subprocess

import pytest

import bit_block_scaled_nvfp4_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")



def _gpu_visible() -> bool:
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


# The calls below pass fake device addresses; should a check ever let one through, it must not
# reach a real GPU, so on a machine with one these host-only tests do not run.
pytestmark = [
    pytest.mark.skipif(not os.path.exists(nv.LIB_PATH),
                       reason="libnvfp4.so not built (run __graft_entry__.build())"),
    pytest.mark.skipif(_gpu_visible(), reason="host-only checks with fake device addresses"),
]

P = 0x10000  # a fake, 256-byte aligned device address (never dereferenced here)


def _declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^\n(]*?\b(nvfp4_\w+|fused_nvfp4_\w+)\s*\(", src, re.M)))


def test_header_declares_the_three_entry_points():
    names = _declared_functions()
    for n in ("nvfp4_quantize", "nvfp4_gemm", "fused_nvfp4_gemm", "nvfp4_status_string"):
        assert n in names
    assert sorted(nv.EXPORTED_SYMBOLS) == names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", nv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in _declared_functions():
        assert name in exported, name
    lib = nv.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name)


def test_benchmark_reference_library_exports_its_two_kernels():
    """The benchmark's reference kernels (a plain read and an empty launch) are built beside the
    product library, outside its ABI: the product library exports neither."""
    path = os.path.join(os.path.dirname(os.path.abspath(nv.__file__)), "libnvfp4_ceiling.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert {"nvfp4_ceiling_stream_read", "nvfp4_ceiling_empty_launch"} <= exported
    lib = ctypes.CDLL(path)
    lib.nvfp4_ceiling_stream_read.restype = ctypes.c_int
    lib.nvfp4_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                              ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_void_p]
    # rejected on the host before any HIP call: sizes that are not whole 16-byte pieces, no blocks
    assert lib.nvfp4_ceiling_stream_read(None, 8, None, 0, ctypes.c_void_p(16), 1, None) != 0
    assert lib.nvfp4_ceiling_stream_read(None, 0, None, 0, ctypes.c_void_p(16), 0, None) != 0
    prod = subprocess.run(["nm", "-D", "--defined-only", nv.LIB_PATH], capture_output=True,
                          text=True, check=True).stdout
    assert "nvfp4_ceiling" not in prod


def test_status_strings_and_version():
    for s in range(5):
        assert nv.status_string(s).startswith("NVFP4")
    assert "unknown" in nv.status_string(99)
    assert nv.load_library().nvfp4_version() >= 100


def _q(**kw):
    a = dict(x=P, dt=nv.NVFP4_BF16, rows=4, cols=32, ldx=32, g=P, dyn=0, codes=P, scales=P, s=None)
    a.update(kw)
    return nv.load_library().nvfp4_quantize(a["x"], a["dt"], a["rows"], a["cols"], a["ldx"], a["g"],
                                            a["dyn"], a["codes"], a["scales"], a["s"])


def test_quantize_validation():
    assert _q(x=None) == nv.NVFP4_EINVAL
    assert _q(g=None) == nv.NVFP4_EINVAL
    assert _q(codes=None) == nv.NVFP4_EINVAL
    assert _q(scales=None) == nv.NVFP4_EINVAL
    assert _q(dt=7) == nv.NVFP4_EINVAL
    assert _q(dyn=2) == nv.NVFP4_EINVAL
    assert _q(cols=24, ldx=24) == nv.NVFP4_ESHAPE
    assert _q(rows=-1) == nv.NVFP4_ESHAPE
    assert _q(ldx=16) == nv.NVFP4_ESHAPE
    assert _q(x=P + 8) == nv.NVFP4_EALIGN
    assert _q(ldx=36) == nv.NVFP4_EALIGN  # 72-byte bf16 row pitch
    assert _q(codes=P + 4) == nv.NVFP4_EALIGN
    assert _q(rows=1 << 28, cols=1 << 8, ldx=1 << 8) == nv.NVFP4_ESHAPE  # 2^32 blocks
    # empty static problems are valid and enqueue nothing
    assert _q(rows=0) == nv.NVFP4_OK
    assert _q(cols=0, ldx=16) == nv.NVFP4_OK


def _sq(**kw):
    a = dict(gate=P, up=P + 4096, dt=nv.NVFP4_BF16, rows=4, cols=32, ldg=32, ldu=32, g=P, dyn=0,
             codes=P, scales=P, s=None)
    a.update(kw)
    return nv.load_library().nvfp4_silu_mul_quantize(
        a["gate"], a["up"], a["dt"], a["rows"], a["cols"], a["ldg"], a["ldu"], a["g"], a["dyn"],
        a["codes"], a["scales"], a["s"])


def test_silu_mul_quantize_validation():
    assert _sq(gate=None) == nv.NVFP4_EINVAL
    assert _sq(up=None) == nv.NVFP4_EINVAL
    assert _sq(g=None) == nv.NVFP4_EINVAL
    assert _sq(codes=None) == nv.NVFP4_EINVAL
    assert _sq(scales=None) == nv.NVFP4_EINVAL
    assert _sq(dt=7) == nv.NVFP4_EINVAL
    assert _sq(dyn=2) == nv.NVFP4_EINVAL
    assert _sq(cols=24, ldg=24, ldu=24) == nv.NVFP4_ESHAPE
    assert _sq(rows=-1) == nv.NVFP4_ESHAPE
    assert _sq(ldg=16) == nv.NVFP4_ESHAPE
    assert _sq(ldu=16) == nv.NVFP4_ESHAPE
    assert _sq(gate=P + 8) == nv.NVFP4_EALIGN
    assert _sq(up=P + 8) == nv.NVFP4_EALIGN
    assert _sq(ldu=36) == nv.NVFP4_EALIGN  # 72-byte bf16 row pitch
    assert _sq(codes=P + 4) == nv.NVFP4_EALIGN
    assert _sq(rows=1 << 28, cols=1 << 8, ldg=1 << 8, ldu=1 << 8) == nv.NVFP4_ESHAPE
    assert _sq(rows=0) == nv.NVFP4_OK
    assert _sq(cols=0, ldg=16, ldu=16) == nv.NVFP4_OK


def _g(fused=False, **kw):
    a = dict(ac=P, as_=P, ga=P, wc=P, ws=P, gw=P, M=64, N=96, K=512, c=P, cdt=nv.NVFP4_F32, ldc=96,
             offs=None, nseg=None, s=None)
    a.update(kw)
    lib = nv.load_library()
    if not fused:
        return lib.nvfp4_gemm(a["ac"], a["as_"], a["ga"], a["wc"], a["ws"], a["gw"], a["M"], a["N"],
                              a["K"], a["c"], a["cdt"], a["ldc"], a["s"])
    offs = a["offs"] if a["offs"] is not None else [0, a["N"]]
    nseg = a["nseg"] if a["nseg"] is not None else len(offs) - 1
    arr = (ctypes.c_int64 * max(len(offs), 1))(*offs)
    return lib.fused_nvfp4_gemm(a["ac"], a["as_"], a["ga"], a["wc"], a["ws"], a["gw"], arr, nseg,
                                a["M"], a["N"], a["K"], a["c"], a["cdt"], a["ldc"], a["s"])


@pytest.mark.parametrize("fused", [False, True])
def test_gemm_validation(fused):
    E = nv
    for k in ("ac", "as_", "ga", "wc", "ws", "gw", "c"):
        assert _g(fused, **{k: None}) == E.NVFP4_EINVAL, k
    assert _g(fused, cdt=E.NVFP4_F16) == E.NVFP4_EINVAL
    assert _g(fused, K=40) == E.NVFP4_ESHAPE
    assert _g(fused, K=0) == E.NVFP4_ESHAPE
    assert _g(fused, M=-1) == E.NVFP4_ESHAPE
    assert _g(fused, ldc=95) == E.NVFP4_ESHAPE
    assert _g(fused, K=1 << 24) == E.NVFP4_ESHAPE
    assert _g(fused, ac=P + 8) == E.NVFP4_EALIGN
    assert _g(fused, ws=P + 4) == E.NVFP4_EALIGN
    assert _g(fused, c=P + 4) == E.NVFP4_EALIGN
    assert _g(fused, M=0) == E.NVFP4_OK  # empty: nothing enqueued
    assert _g(fused, M=0, ac=None, as_=None, c=None) == E.NVFP4_OK  # no storage when empty
    assert _g(fused, M=0, ga=None) == E.NVFP4_EINVAL  # global scales are always required


def _lin(**kw):
    a = dict(x=P, xdt=nv.NVFP4_BF16, ldx=512, ga=P, ac=P, as_=P, wc=P, ws=P, gw=P, offs=None,
             nseg=None, M=4, N=96, K=512, c=P, cdt=nv.NVFP4_F32, ldc=96, s=None)
    a.update(kw)
    offs = a["offs"] if a["offs"] is not None else [0, a["N"]]
    nseg = a["nseg"] if a["nseg"] is not None else len(offs) - 1
    arr = (ctypes.c_int64 * max(len(offs), 1))(*offs)
    return nv.load_library().nvfp4_linear(a["x"], a["xdt"], a["ldx"], a["ga"], a["ac"], a["as_"],
                                          a["wc"], a["ws"], a["gw"], arr, nseg, a["M"], a["N"],
                                          a["K"], a["c"], a["cdt"], a["ldc"], a["s"])


def test_linear_validation():
    """nvfp4_linear checks the activation as nvfp4_quantize does and the product as
    fused_nvfp4_gemm does, before any launch."""
    E = nv
    for k in ("x", "ga", "ac", "as_", "wc", "ws", "gw", "c"):
        assert _lin(**{k: None}) == E.NVFP4_EINVAL, k
    assert _lin(xdt=7) == E.NVFP4_EINVAL
    assert _lin(cdt=E.NVFP4_F16) == E.NVFP4_EINVAL
    assert _lin(ldx=500) == E.NVFP4_ESHAPE  # row pitch below K
    assert _lin(K=40, ldx=40) == E.NVFP4_ESHAPE
    assert _lin(offs=[0, 32, 95]) == E.NVFP4_ESHAPE
    assert _lin(x=P + 8) == E.NVFP4_EALIGN
    assert _lin(ldx=516) == E.NVFP4_EALIGN  # 1032-byte bf16 rows are not 16-byte multiples
    assert _lin(ac=P + 8) == E.NVFP4_EALIGN
    assert _lin(M=0, x=None, ac=None, as_=None, c=None) == E.NVFP4_OK  # empty: nothing enqueued


def test_fused_segment_validation():
    E = nv
    assert _g(True, offs=[0, 32, 96], nseg=0) == E.NVFP4_EINVAL
    assert _g(True, offs=list(range(0, 96, 5)) + [96], nseg=20) == E.NVFP4_EINVAL  # > 16 segments
    assert _g(True, offs=[1, 32, 96]) == E.NVFP4_ESHAPE  # must start at 0
    assert _g(True, offs=[0, 32, 95]) == E.NVFP4_ESHAPE  # must end at N
    assert _g(True, offs=[0, 32, 32, 96]) == E.NVFP4_ESHAPE  # strictly rising
    assert _g(True, offs=[0, 64, 32, 96]) == E.NVFP4_ESHAPE
    assert _g(True, offs=[0, 0], N=0, ldc=1) == E.NVFP4_OK  # empty problem


def test_binding_refuses_cpu_tensors():
    import torch

    with pytest.raises(ValueError):
        nv.nvfp4_quantize(torch.zeros(4, 32))


def _kvs(**kw):
    a = dict(k=P, v=P + 4096, dt=nv.NVFP4_BF16, tokens=4, width=32, ldk=32, ldv=32, ks=P, vs=P,
             slots=P, kc=P, vc=P, num_slots=8, cache_ld=32, s=None)
    a.update(kw)
    return nv.load_library().nvfp4_kv_fp8_store(
        a["k"], a["v"], a["dt"], a["tokens"], a["width"], a["ldk"], a["ldv"], a["ks"], a["vs"],
        a["slots"], a["kc"], a["vc"], a["num_slots"], a["cache_ld"], a["s"])


def test_kv_store_validation():
    assert _kvs(k=None) == nv.NVFP4_EINVAL
    assert _kvs(ks=None) == nv.NVFP4_EINVAL
    assert _kvs(kc=None) == nv.NVFP4_EINVAL
    assert _kvs(v=None) == nv.NVFP4_EINVAL  # value scale and cache given without values
    assert _kvs(vc=None) == nv.NVFP4_EINVAL
    assert _kvs(vs=None) == nv.NVFP4_EINVAL
    assert _kvs(dt=7) == nv.NVFP4_EINVAL
    assert _kvs(width=24, ldk=24, ldv=24, cache_ld=32) == nv.NVFP4_ESHAPE
    assert _kvs(tokens=-1) == nv.NVFP4_ESHAPE
    assert _kvs(num_slots=-1) == nv.NVFP4_ESHAPE
    assert _kvs(ldk=16) == nv.NVFP4_ESHAPE
    assert _kvs(ldv=16) == nv.NVFP4_ESHAPE
    assert _kvs(cache_ld=16) == nv.NVFP4_ESHAPE
    assert _kvs(width=1 << 25, ldk=1 << 25, ldv=1 << 25, cache_ld=1 << 25) == nv.NVFP4_ESHAPE
    assert _kvs(k=P + 8) == nv.NVFP4_EALIGN
    assert _kvs(v=P + 8) == nv.NVFP4_EALIGN
    assert _kvs(ldk=36) == nv.NVFP4_EALIGN  # 72-byte bf16 row pitch
    assert _kvs(kc=P + 4) == nv.NVFP4_EALIGN
    assert _kvs(cache_ld=40) == nv.NVFP4_EALIGN
    assert _kvs(slots=P + 4) == nv.NVFP4_EALIGN
    assert _kvs(ks=P + 2) == nv.NVFP4_EALIGN
    # keys only, and empty problems, are valid (nothing enqueued for empty ones)
    assert _kvs(tokens=0) == nv.NVFP4_OK
    assert _kvs(width=0, ldk=16, ldv=16, cache_ld=16) == nv.NVFP4_OK
    assert _kvs(tokens=0, v=None, vs=None, vc=None) == nv.NVFP4_OK


def _kvl(**kw):
    a = dict(c=P, num_slots=8, cache_ld=32, width=32, scale=P, slots=P, tokens=4, out=P,
             odt=nv.NVFP4_F32, ld_out=32, s=None)
    a.update(kw)
    return nv.load_library().nvfp4_kv_fp8_load(
        a["c"], a["num_slots"], a["cache_ld"], a["width"], a["scale"], a["slots"], a["tokens"],
        a["out"], a["odt"], a["ld_out"], a["s"])


def test_kv_load_validation():
    assert _kvl(c=None) == nv.NVFP4_EINVAL
    assert _kvl(scale=None) == nv.NVFP4_EINVAL
    assert _kvl(out=None) == nv.NVFP4_EINVAL
    assert _kvl(odt=nv.NVFP4_F16) == nv.NVFP4_EINVAL
    assert _kvl(width=24, cache_ld=32, ld_out=32) == nv.NVFP4_ESHAPE
    assert _kvl(tokens=-1) == nv.NVFP4_ESHAPE
    assert _kvl(cache_ld=16) == nv.NVFP4_ESHAPE
    assert _kvl(ld_out=16) == nv.NVFP4_ESHAPE
    assert _kvl(c=P + 8) == nv.NVFP4_EALIGN
    assert _kvl(out=P + 8) == nv.NVFP4_EALIGN
    assert _kvl(cache_ld=40) == nv.NVFP4_EALIGN
    assert _kvl(ld_out=33) == nv.NVFP4_EALIGN  # 132-byte f32 row pitch
    assert _kvl(slots=P + 4) == nv.NVFP4_EALIGN
    assert _kvl(tokens=0) == nv.NVFP4_OK


def test_empty_problems_accept_null_data_pointers():
    lib = nv.load_library()
    assert _q(x=None, codes=None, scales=None, rows=0) == nv.NVFP4_OK
    assert _q(x=None, codes=None, scales=None, rows=4) == nv.NVFP4_EINVAL
    assert _kvs(k=None, v=None, kc=None, vc=None, slots=None, tokens=0) == nv.NVFP4_OK
    assert _kvl(c=None, out=None, slots=None, tokens=0) == nv.NVFP4_OK
    assert lib.nvfp4_requantize(None, None, P, P, 0, 32, None, None, None) == nv.NVFP4_OK


def _fk(**kw):
    a = dict(x=P, dt=nv.NVFP4_BF16, rows=4, cols=32, ldx=32, g=P, dyn=0, out=P,
             odt=nv.NVFP4_F32, ldo=32, s=None)
    a.update(kw)
    return nv.load_library().nvfp4_fake_quantize(a["x"], a["dt"], a["rows"], a["cols"], a["ldx"],
                                                 a["g"], a["dyn"], a["out"], a["odt"], a["ldo"],
                                                 a["s"])


def test_fake_quantize_validation():
    assert _fk(x=None) == nv.NVFP4_EINVAL
    assert _fk(g=None) == nv.NVFP4_EINVAL
    assert _fk(out=None) == nv.NVFP4_EINVAL
    assert _fk(dt=7) == nv.NVFP4_EINVAL
    assert _fk(odt=nv.NVFP4_F16) == nv.NVFP4_EINVAL
    assert _fk(dyn=3) == nv.NVFP4_EINVAL
    assert _fk(cols=24, ldx=24, ldo=24) == nv.NVFP4_ESHAPE
    assert _fk(ldo=16) == nv.NVFP4_ESHAPE
    assert _fk(ldx=16) == nv.NVFP4_ESHAPE
    assert _fk(out=P + 8) == nv.NVFP4_EALIGN
    assert _fk(ldo=33) == nv.NVFP4_EALIGN
    assert _fk(x=P + 4) == nv.NVFP4_EALIGN
    assert _fk(rows=0) == nv.NVFP4_OK


def _st(**kw):
    a = dict(x=P, dt=nv.NVFP4_F32, rows=4, cols=32, ldx=32, g=P, dyn=0, e=P, n=P, d=P, s=None)
    a.update(kw)
    return nv.load_library().nvfp4_quant_error_stats(a["x"], a["dt"], a["rows"], a["cols"], a["ldx"],
                                                     a["g"], a["dyn"], a["e"], a["n"], a["d"],
                                                     a["s"])


def test_quant_error_stats_validation():
    for k in ("x", "g", "e", "n", "d"):
        assert _st(**{k: None}) == nv.NVFP4_EINVAL, k
    assert _st(dt=9) == nv.NVFP4_EINVAL
    assert _st(cols=8, ldx=8) == nv.NVFP4_ESHAPE
    assert _st(rows=-2) == nv.NVFP4_ESHAPE
    assert _st(e=P + 4) == nv.NVFP4_EALIGN
    assert _st(d=P + 2) == nv.NVFP4_EALIGN
    assert _st(ldx=33) == nv.NVFP4_EALIGN  # 132-byte f32 row pitch
    assert _st(rows=0, e=None, n=None, d=None, x=None) == nv.NVFP4_OK


def test_requantize_and_harmonize_validation():
    lib = nv.load_library()
    rq = lambda **kw: lib.nvfp4_requantize(*[kw.get(k, v) for k, v in (
        ("c", P), ("sc", P), ("gi", P), ("go", P), ("rows", 4), ("cols", 32), ("co", P),
        ("so", P), ("s", None))])
    assert rq(gi=None) == nv.NVFP4_EINVAL
    assert rq(go=None) == nv.NVFP4_EINVAL
    assert rq(c=None) == nv.NVFP4_EINVAL
    assert rq(so=None) == nv.NVFP4_EINVAL
    assert rq(cols=20) == nv.NVFP4_ESHAPE
    assert rq(rows=-1) == nv.NVFP4_ESHAPE
    assert rq(c=P + 4) == nv.NVFP4_EALIGN
    assert rq(co=P + 2) == nv.NVFP4_EALIGN
    assert rq(rows=0) == nv.NVFP4_OK

    def hz(offs=(0, 16, 32), nseg=None, N=32, K=64, g=P, sh=P + 256, **kw):
        arr = (ctypes.c_int64 * len(offs))(*offs)
        nseg = len(offs) - 1 if nseg is None else nseg
        return lib.nvfp4_harmonize_segments(kw.get("c", P), kw.get("sc", P), g, arr, nseg, N, K, sh,
                                            kw.get("co", P), kw.get("so", P), None)
    assert hz(g=None) == nv.NVFP4_EINVAL
    assert hz(sh=None) == nv.NVFP4_EINVAL
    assert hz(sh=P + 4) == nv.NVFP4_EINVAL  # inside the segment-scale table
    assert hz(nseg=0) == nv.NVFP4_EINVAL
    assert hz(nseg=17) == nv.NVFP4_EINVAL
    assert hz(offs=(0, 16, 16)) == nv.NVFP4_ESHAPE
    assert hz(offs=(0, 40, 32)) == nv.NVFP4_ESHAPE
    assert hz(offs=(1, 16, 32)) == nv.NVFP4_ESHAPE
    assert hz(K=40) == nv.NVFP4_ESHAPE
    assert hz(c=P + 4) == nv.NVFP4_EALIGN
    assert hz(g=P + 2) == nv.NVFP4_EALIGN
    assert hz(N=0, offs=(0, 0), c=None, sc=None, co=None, so=None) == nv.NVFP4_OK
