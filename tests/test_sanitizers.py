"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C ABI's argument validation (kda_api.cpp) is built with g++ against
  stub launchers (tests/sanitize/api_driver.cpp): every entry point's valid
  calls reach one launch, invalid ones return their status and launch
  nothing, with no memory error or undefined behaviour.
* The oracle is rebuilt instrumented and its pins (tests/test_oracle.py) run
  against it in a child process with the ASan runtime preloaded.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _runtime():
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc/g++ not available")
    lib = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(lib) or not os.path.exists(lib):
        pytest.skip("the ASan runtime is not installed")
    return lib


def test_api_validation_under_sanitizers(tmp_path):
    _runtime()
    exe = str(tmp_path / "api_driver")
    cmd = ["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                                          "-I" + os.path.join(ROOT, "include"),
                                          "-I" + os.path.join(ROOT, "kimi_delta_attention_amd", "csrc"),
                                          os.path.join(ROOT, "kimi_delta_attention_amd", "csrc", "kda_api.cpp"),
                                          os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "0 failures" in r.stdout


def test_oracle_pins_under_sanitizers():
    asan = _runtime()
    env = dict(os.environ, KDA_ORACLE_SANITIZE="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=900)
    print(r.stdout[-1500:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-4000:]
