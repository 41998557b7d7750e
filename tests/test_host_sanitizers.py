"""The library's host C++ (dispatch guard, argument checks, workspace
carving, metadata validation, page allocator) built with g++ under
AddressSanitizer + UndefinedBehaviorSanitizer and, for the allocator shared
by eight threads, under ThreadSanitizer; tests/host/harness.cpp holds the
checks and the stubs that stand in for the HIP runtime and the kernels.
The PA_DEBUG_VALIDATE switch (metadata checked before every launch that
reads a page table) is tested in a process of its own, since the library
reads the variable once.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_02_amd", "csrc")
SRCS = [os.path.join(ROOT, "tests", "host", "harness.cpp"), os.path.join(CSRC, "api.cpp"),
        os.path.join(CSRC, "pool.cpp")]
COMMON = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
          "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-pthread"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                                reason="needs g++ and the ROCm headers")


def build_and_run(tmp_path, flags, mode, env_extra):
    exe = str(tmp_path / f"harness_{mode}")
    cmd = ["g++", *COMMON, *flags, *SRCS, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    env = {k: v for k, v in os.environ.items() if k != "PA_DEBUG_VALIDATE"}
    env.update(env_extra)
    run = subprocess.run([exe, mode], capture_output=True, text=True, timeout=300, env=env)
    print(run.stdout, run.stderr[-3000:])
    assert run.returncode == 0, run.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in run.stderr
    assert "runtime error" not in run.stderr
    assert "WARNING: ThreadSanitizer" not in run.stderr
    return run.stdout


def test_host_code_under_address_and_undefined_sanitizers(tmp_path):
    out = build_and_run(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"],
                        "asan", {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0"})
    assert "asan mode ok" in out


def test_page_pool_under_thread_sanitizer(tmp_path):
    out = build_and_run(tmp_path, ["-fsanitize=thread"], "tsan", {"TSAN_OPTIONS": "halt_on_error=1"})
    assert "tsan mode ok" in out


def test_debug_validation_switch(tmp_path):
    out = build_and_run(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"],
                        "debug", {"PA_DEBUG_VALIDATE": "1", "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0"})
    assert "debug mode ok" in out
