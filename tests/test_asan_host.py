"""The host layer of the C ABI (argument validation, kernel selection, segment tables) built with
AddressSanitizer and UndefinedBehaviorSanitizer for the CPU, the kernel launchers replaced by
host-only stand-ins (``tests/asan/launch_stubs.cpp``), and the C-ABI tests of ``test_abi.py`` run
against that build in a child process with the sanitizer runtime preloaded.  Any out-of-bounds
read of an argument (for instance of the host segment-offset array), use of freed memory or
undefined arithmetic in the host layer aborts the child and fails this test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_block_scaled_nvfp4_amd", "csrc")


def _gpu_visible() -> bool:
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


pytestmark = pytest.mark.skipif(_gpu_visible(), reason="host-only build with stubbed launchers")


def _asan_runtime():
    if shutil.which("g++") is None:
        return None
    p = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_host_layer_under_address_and_ub_sanitizers(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("g++ with libasan is not available")
    lib = tmp_path / "libnvfp4_host_asan.so"
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}",
             f"-I{CSRC}"]
    objs = []
    for src, lang in ((os.path.join(CSRC, "api.hip"), "c++"),
                      (os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"), "c++")):
        obj = tmp_path / (os.path.basename(src) + ".o")
        subprocess.run(["g++", "-x", lang, *flags, "-c", src, "-o", str(obj)], check=True,
                       capture_output=True, text=True)
        objs.append(str(obj))
    subprocess.run(["g++", "-shared", "-fsanitize=address,undefined", "-o", str(lib), *objs],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "asan", "run_abi_tests.py"),
                          str(lib)], capture_output=True, text=True, env=env, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out
