"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

`tests/sanitize/okv_abi_driver.cpp` is built together with `okv_host.cpp`, with every
kernel launcher replaced by a stub, and exercises the C ABI's GPU-free paths:
configuration layout and validation at the edges of every field, the 4 GiB slice limit,
pointer and rotation-parameter refusals, calls on a null handle and the status strings.
The sanitizers apply to host code only (each `-fsanitize=` follows `-Xarch_host`); no
call reaches the GPU. CPU only."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_host_abi_under_asan_ubsan():
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "okv_abi_driver")
        cmd = [hipcc, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"),
               "-I", os.path.join(ROOT, "decode_attention_okv_amd", "csrc"),
               "-Xarch_host", "-fsanitize=address,undefined",
               "-Xarch_host", "-fno-sanitize-recover=all",
               "-Xarch_host", "-fno-omit-frame-pointer",
               "-x", "hip", os.path.join(ROOT, "decode_attention_okv_amd", "csrc", "okv_host.cpp"),
               os.path.join(ROOT, "tests", "sanitize", "okv_abi_driver.cpp"), "-o", exe]
        b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        assert b.returncode == 0, b.stderr[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
        assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout + r.stderr)[-4000:]
