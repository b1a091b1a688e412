"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

abi.cpp (the C-ABI's argument checks, size arithmetic, device check, stream
workspaces and call locks, the fixed-scratch path) is built host-only against a
fake HIP runtime and stub launchers (tests/sanitize/fake_hip.cpp) that touch
exactly the bytes the real kernels would, and driven by tests/sanitize/abi_driver.cpp.
The CPU oracle (oracle/oracle.cpp) is built with the same sanitizers and driven
by tests/sanitize/oracle_driver.cpp. Any sanitizer report, or an unexpected
status from a driver, fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "deterministic_invariant_gemm_det_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SANITIZERS = "-fsanitize=address,undefined"
COMMON = ["-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _check_clean(r):
    for marker in ("ERROR: AddressSanitizer", "ERROR: LeakSanitizer", "runtime error:"):
        assert marker not in r.stderr, r.stderr


def _abi_driver(tmp_path, sanitizers):
    objs = []
    for src in (os.path.join(CSRC, "abi.cpp"), os.path.join(SAN, "fake_hip.cpp"), os.path.join(SAN, "abi_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        # host-only HIP compilation: the sanitizers apply to host code only
        _run([CLANG, "-x", "hip", "--offload-host-only", *COMMON, "-Xarch_host", sanitizers,
              "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_sanitized")
    _run([CLANG, sanitizers, "-pthread", *objs, "-o", exe])
    return exe


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not installed")
def test_abi_host_code_sanitized(tmp_path):
    r = _run([_abi_driver(tmp_path, SANITIZERS)], env=ENV)
    _check_clean(r)
    assert "abi driver: 0 failures" in r.stdout


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not installed")
def test_abi_host_code_threads(tmp_path):
    """The same driver under ThreadSanitizer: four threads on two streams share
    the slot map, the per-stream locks and workspaces and the device cache."""
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    r = _run([_abi_driver(tmp_path, "-fsanitize=thread")], env=env)
    assert "WARNING: ThreadSanitizer" not in r.stderr, r.stderr
    assert "abi driver: 0 failures" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_oracle_sanitized(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    _run(["g++", *COMMON, SANITIZERS, "-mfma", "-ffp-contract=off", "-fno-fast-math",
          os.path.join(ROOT, "oracle", "oracle.cpp"), os.path.join(SAN, "oracle_driver.cpp"), "-o", exe])
    r = _run([exe], env=ENV)
    _check_clean(r)
    assert "oracle driver: 0 failures" in r.stdout
