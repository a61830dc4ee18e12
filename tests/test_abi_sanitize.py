"""The host side of the C ABI (tests/sanitize/abi_driver.cpp over
csrc/attn_api.cpp, the kernel launchers replaced by the checking stand-ins of
tests/sanitize/abi_stubs.cpp) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU: every entry point's checks,
its packed launch parameters, and sizes at and past every limit (int64
extremes included) must run without undefined behaviour and return the
documented codes ("ops-transformer：Transformer算子融合与推理加速实战" §6.2:
out-of-bounds bugs show as random crashes; §4.4: debug builds)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "transformer_attention_06_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_host_path_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", SAN,
           os.path.join(CSRC, "attn_api.cpp"), os.path.join(SAN, "abi_stubs.cpp"),
           os.path.join(SAN, "abi_driver.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    # verify_asan_link_order=0: a library the environment preloads may come
    # before the ASan runtime in the load order
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert r.stdout.strip().endswith("0 failed")
