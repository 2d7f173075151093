"""The library's host code -- argument validation and operation objects
(csrc/api.cpp) and the launch planners (csrc/planner.cpp) -- built with g++,
AddressSanitizer and UndefinedBehaviorSanitizer (kernel launchers replaced by
tests/sanitizer_launch_stubs.cpp, which no CPU-only run reaches), and the CPU
ABI / planner tests run against that build in a child process: any invalid
memory access or undefined behaviour on those paths fails the test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "masked_paged_attention_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_abi_and_planner_tests_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("g++ sanitizer runtimes not installed")
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}"]
    objs = []
    for src in [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "planner.cpp"),
                os.path.join(ROOT, "tests", "sanitizer_launch_stubs.cpp")]:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run(["g++"] + flags + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    lib = str(tmp_path / "libmpa_sanitized.so")
    r = subprocess.run(["g++", "-shared", "-fsanitize=address,undefined", "-o", lib] + objs +
                       [f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ)
    env.update(MPA_LIBRARY=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert " passed" in out
