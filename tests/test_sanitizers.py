"""The host code under the compilers' sanitizers (CPU only, no GPU needed):
  * the fp64 oracle (oracle/gdn_oracle.c) built with AddressSanitizer + UndefinedBehaviorSanitizer
    and, separately, ThreadSanitizer (it splits work over threads), driven over packed
    workloads with empty, one-token and ragged sequences (tests/sanitize/oracle_driver.c);
  * the C ABI's host validation (gdn_api.hip, compiled as host C++ against stubbed kernel
    launchers) with AddressSanitizer + UndefinedBehaviorSanitizer and leak checking, driven over
    every entry point with valid and invalid arguments (tests/sanitize/api_driver.cpp).
A sanitizer report ends the program with a non-zero status."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gated_deltanet_recurrence_chunked_amd", "csrc")


def _run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ...: rc {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


def _env(**kw):
    env = dict(os.environ)
    env.pop("LD_PRELOAD", None)
    env.update(kw)
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_oracle_under_sanitizers(tmp_path, san):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", f"-fsanitize={san}", "-fno-sanitize-recover=all",
          "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "oracle", "gdn_oracle.c"), os.path.join(SAN, "oracle_driver.c"),
          "-o", exe, "-lm", "-lpthread"])
    r = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=1", TSAN_OPTIONS="halt_on_error=1"))
    assert "oracle driver done" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_abi_host_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_driver")
    _run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-x", "c++", os.path.join(CSRC, "gdn_api.hip"),
          "-x", "c++", os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "api_driver.cpp"),
          "-o", exe])
    r = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=1"))
    assert r.stdout.startswith("0 failures")
