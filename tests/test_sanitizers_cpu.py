"""The C-ABI validation layer under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

api.cpp (argument checks, workspace arithmetic, dispatch) and the split
planning are compiled host-only with g++ -fsanitize=address,undefined
(every report fatal) and linked against launch stand-ins that report no
device (sanitizer_launch_stubs.cpp).  The CPU ABI and binding tests then run
in a child process against that library, with the ASan runtime preloaded
into the interpreter.  Any sanitizer report aborts the child and fails this
test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int2_rotated_kv_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _asan_runtime():
    if shutil.which("g++") is None:
        return None
    path = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized_library(tmp_path_factory):
    if _asan_runtime() is None:
        pytest.skip("g++ with AddressSanitizer is not available")
    out = str(tmp_path_factory.mktemp("asan") / "libkvq.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "kvq_plan.cpp"),
           os.path.join(ROOT, "tests", "sanitizer_launch_stubs.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return out


def test_abi_checks_under_sanitizers(sanitized_library):
    env = dict(os.environ)
    env.update(LD_PRELOAD=_asan_runtime(), KVQ_TEST_LIBRARY=sanitized_library,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi_cpu.py"), os.path.join(ROOT, "tests", "test_binding_checks_cpu.py")]
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail, tail
