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


def _trace_run(exe, env_extra):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("DORY_TRACE", None)
    env.update(env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "trace main done" in r.stdout
    return [l.split(" ", 3)[1:] for l in r.stdout.splitlines() if l.startswith("roctx ")]


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_trace_ranges(tmp_path):
    """DORY_TRACE=1: every boundary call opens one range, with the input block, each loop
    and the output block nested in it and one range per layer call inside those; pushes
    and pops balance. Unset: no range at all. The marker library is a stand-in that prints
    the ranges (tests/host/roctx_stub.cpp), loaded through DORY_TRACE_LIB."""
    stub = str(tmp_path / "libroctx_stub.so")
    r = subprocess.run(["g++", "-std=c++17", "-shared", "-fPIC", "-o", stub,
                        os.path.join(ROOT, "tests", "host", "roctx_stub.cpp")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = str(tmp_path / "trace")
    src = [os.path.join(ROOT, "looped_ngpt_transformer_amd", "csrc", "runtime.cpp"),
           os.path.join(ROOT, "tests", "host", "stub_launchers.cpp"),
           os.path.join(ROOT, "tests", "host", "fake_hip.cpp"),
           os.path.join(ROOT, "tests", "host", "trace_main.cpp")]
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", *src, "-ldl", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]

    assert _trace_run(exe, {"DORY_TRACE_LIB": stub}) == []
    assert _trace_run(exe, {"DORY_TRACE": "0", "DORY_TRACE_LIB": stub}) == []
    ev = _trace_run(exe, {"DORY_TRACE": "1", "DORY_TRACE_LIB": stub})
    # rebuild the tree of ranges from the pushes and pops
    stack, calls = [], []
    for e in ev:
        if e[0] == "push":
            assert int(e[1]) == len(stack), e
            node = {"name": e[2], "kids": []}
            (stack[-1]["kids"] if stack else calls).append(node)
            stack.append(node)
        else:
            assert e[0] == "pop" and stack and int(e[1]) == len(stack) - 1, e
            stack.pop()
    assert not stack
    assert [c["name"] for c in calls] == ["dory_prefill: 2 sequences", "dory_decode_step: 2 sequences"]
    for call in calls:
        blocks = [b["name"] for b in call["kids"]]
        assert blocks == ["input block", "loop 1 of 2", "loop 2 of 2", "output block"], blocks
        layers = [[k["name"] for k in b["kids"]] for b in call["kids"]]
        assert [len(x) for x in layers] == [2, 4, 4, 2]
        assert all(not k["kids"] for b in call["kids"] for k in b["kids"])
        assert layers[0][0].startswith("layer 0, KV slot 0")
        assert layers[1][0].startswith("layer 2, KV slot 0") and layers[2][0].startswith("layer 2, KV slot 1")
        assert layers[3][-1].startswith("layer 7, KV slot 0")
    assert calls[0]["kids"][0]["kids"][0]["name"].endswith("130 rows")
    assert calls[1]["kids"][0]["kids"][0]["name"].endswith("2 rows")
