"""The host runtime (runtime.cpp) built with AddressSanitizer and UndefinedBehaviorSanitizer
and driven through the C ABI on the CPU; the kernel launchers are stand-ins
(tests/host/stub_launchers.cpp) and no GPU is used.

* the paged KV bookkeeping (allocator, sliding-window rings, slot counts per KV mode,
  truncation, release, refusals for lack of pages) against a model of its page counts
  (tests/host/allocator_main.cpp), with the HIP runtime library;
* the error contract (tests/host/rollback_main.cpp), with a stand-in HIP runtime that
  records the uploads (tests/host/fake_hip.cpp): calls made to fail after committing
  leave the context unchanged, and their retries upload exactly what a context that
  never failed uploads."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
                    reason="needs g++ and the HIP runtime library")
def test_allocator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "allocator")
    src = [os.path.join(ROOT, "looped_ngpt_transformer_amd", "csrc", "runtime.cpp"),
           os.path.join(ROOT, "tests", "host", "stub_launchers.cpp"),
           os.path.join(ROOT, "tests", "host", "allocator_main.cpp")]
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", *src, f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib",
           "-lamdhip64", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "allocator checks passed" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_rollback_under_sanitizers(tmp_path):
    exe = str(tmp_path / "rollback")
    src = [os.path.join(ROOT, "looped_ngpt_transformer_amd", "csrc", "runtime.cpp"),
           os.path.join(ROOT, "tests", "host", "stub_launchers.cpp"),
           os.path.join(ROOT, "tests", "host", "fake_hip.cpp"),
           os.path.join(ROOT, "tests", "host", "rollback_main.cpp")]
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", *src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "rollback checks passed" in r.stdout
