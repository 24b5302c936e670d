"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

The planner, the C ABI's host paths (argument checks, plan life cycle, getters,
fault injection, tuning's candidate planning) and the front-end's matrix
builders are built with gcc's -fsanitize=address,undefined into a library of
their own; the kernels' launchers are replaced by stand-ins
(tests/sanitize/launch_stubs.cpp), which no CPU test reaches.  The CPU suites
of the planner (tests/test_plan.py: exports, errors, F2 algebra, host replay
of every kernel table against the oracle), of the random option cases and of
the front-end then run in a child process against that library.  Any
sanitizer report fails the test.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bmmc_affine_index_amd", "csrc")
SUITES = ["tests/test_plan.py", "tests/test_random_cases.py", "tests/test_frontend.py"]


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _build(out_dir):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.cpp"))) + [
        os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp")]
    lib = os.path.join(out_dir, "libbmmc_host_san.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           *srcs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=600)
    return lib


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/lib"),
                    reason="needs g++ and the ROCm runtime library")
@pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")),
                    reason="the host already preloads a library; the sanitizer runtime "
                           "must come first and this test does not displace it")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = _build(str(tmp_path))
    env = dict(os.environ)
    env.update(BMMC_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: a sanitizer report ends the child at once, before pytest could
    # print what it captured
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *SUITES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
