"""The host side of the C ABI (include/mla.h, csrc/mla_api.cpp) compiled for
the CPU with AddressSanitizer and UndefinedBehaviorSanitizer and driven by
tests/abi_sanitized/driver.cpp: the HIP runtime and the kernel launchers are
stubs, so every entry point's descriptor checks and launch-parameter
arithmetic run on the host — directed cases with the status each broken
argument must give, 200,000 calls with random descriptors, 50,000 valid calls
with one or two fields changed.  No GPU, no kernel code."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _clang():
    for cand in ("/opt/rocm/lib/llvm/bin/clang++", shutil.which("clang++")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_clang() is None, reason="clang++ with the sanitizer runtimes is not installed")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "abi_driver"
    cmd = [_clang(), "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(ROOT, "tests", "abi_sanitized", "driver.cpp"),
           os.path.join(ROOT, "mla_latent_kv_39_amd", "csrc", "mla_api.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0 and out.rstrip().endswith("OK"), out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
