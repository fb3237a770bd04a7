"""The library's host code (the planner, workspace sizing, argument checks of
every entry point) built for the CPU with AddressSanitizer and
UndefinedBehaviorSanitizer, its device launchers replaced by stubs, and the
host tests of ``test_host.py`` run against that build in a child process.

Any out-of-bounds access, use after free, integer overflow, misaligned access
or other undefined behaviour in the host code aborts the child, which fails
this test.  Test infrastructure only (g++, no GPU)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_sliding_amd", "csrc")
STUBS = os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("g++ has no sanitizer runtimes")
    lib = str(tmp_path / "libpkvs_host_sanitized.so")
    cmd = ["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           f"-I{os.path.join(ROOT, 'include')}", "-O1", "-g", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "run.cpp"), STUBS, f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{ROCM}/lib", "-o", lib]
    subprocess.run(cmd, check=True)
    env = dict(os.environ)
    env.update({
        "PKVS_LIBRARY": lib,
        "LD_PRELOAD": f"{asan}:{ubsan}",
        # the interpreter and torch are not instrumented: their allocations
        # are not checked for leaks or mismatched frees
        "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:"
                        "abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HIP_VISIBLE_DEVICES": "",
    })
    # the child loads the instrumented build, not the in-tree library
    probe = subprocess.run([sys.executable, "-c", "from paged_kv_sliding_amd import pkvs as P; "
                            "print(P.LIB_PATH, P._lib._name)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.split() == [lib, lib], probe.stdout
    # (-s: a sanitizer report goes straight to the child's stderr)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                          "-m", "not gpu", os.path.join(ROOT, "tests", "test_host.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout[-2000:] + res.stderr[-4000:])
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "failed" not in res.stdout, tail
