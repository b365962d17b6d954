"""The host-side entry points (kivi_api.cpp: argument validation, sizing,
stream counters, layer runs, image layout) built on the CPU with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, with launchers that
enqueue nothing (tests/host_sanitize/stub_launchers.cpp), and the CPU test
modules of the C ABI run against that build in a child process: any
out-of-bounds access, signed overflow, misaligned access or other undefined
behaviour in the checks aborts the child and fails this test.  CPU only;
no GPU code is built."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "kv_cache_quantization_codec_amd", "csrc", "kivi_api.cpp"),
       os.path.join(ROOT, "tests", "host_sanitize", "stub_launchers.cpp")]
MODULES = ["tests/test_abi_cpu.py", "tests/test_attention_cpu.py", "tests/test_layers_cpu.py",
           "tests/test_payload_cpu.py", "tests/test_abi_extremes_cpu.py"]


def _gxx():
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    return gxx


def _runtime(gxx, name):
    path = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_abi_modules_clean_under_asan_and_ubsan(tmp_path):
    gxx = _gxx()
    asan = _runtime(gxx, "libasan.so")
    if asan is None:
        pytest.skip("the AddressSanitizer runtime is not installed")
    lib = tmp_path / "libkivi_host_sanitized.so"
    build = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-shared", "-fPIC",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-I", os.path.join(ROOT, "include"), *SRC, "-o", str(lib)]
    res = subprocess.run(build, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ)
    env.update({
        "KIVI_HOST_SANITIZED_LIB": str(lib),
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *MODULES],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout[-4000:] + res.stderr[-4000:]
    assert res.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert " passed" in out
