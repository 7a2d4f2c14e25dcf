"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer: abi.hip is
rebuilt with both sanitizers on its host side (device code unchanged), linked with the
library's other objects into a separate copy, and tests/test_abi_cpu.py (every declared
symbol, every validation path and status code) runs against that copy in a subprocess
with the sanitizer runtime preloaded. Any report fails the test. CPU only."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

from fp8_block_scaled_quant_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def sanitized_library(tmp_path_factory):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rt = _asan_runtime()
    others = [os.path.join(B.BUILD, os.path.basename(src) + ".o") for src in sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))
              if os.path.basename(src) != "abi.hip"]
    others = [o for o in others if os.path.exists(o)]
    if rt is None or not others:
        pytest.skip("sanitizer runtime or the library's objects are missing (build the library first)")
    d = str(tmp_path_factory.mktemp("san"))
    obj = os.path.join(d, "abi.hip.o")
    flags = [f for f in B.CFLAGS if f != "-Wall"]
    r = subprocess.run([hipcc, *flags, *SAN, "-c", os.path.join(B.CSRC, "abi.hip"), "-o", obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = os.path.join(d, "libfp8rl_san.so")
    r = subprocess.run([hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libsan", *SAN, "-o", lib,
                        obj, *others], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    yield lib, rt
    shutil.rmtree(d, ignore_errors=True)


def test_abi_validation_paths_under_sanitizers(sanitized_library):
    lib, rt = sanitized_library
    env = dict(os.environ, FP8RL_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_cpu.py", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, out
    assert " passed" in r.stdout, out
