"""The host layer of the C ABI (argument checks, workspace sizing, the decode
split plan: api.cpp and plan.cpp) built on the CPU with AddressSanitizer and
UndefinedBehaviorSanitizer (plain g++, no device code; the kernel launchers
are stand-ins), and the CPU boundary tests of test_abi.py run against it in
a child process with the sanitizer runtimes preloaded.  Any report of either
sanitizer aborts the child, so the run fails."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_attn_fwd_amd", "csrc")


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("no sanitizer runtimes for g++")
    out = str(tmp_path_factory.mktemp("san") / "libgptoss_attn_host_san.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "stub_launchers.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return out, asan, ubsan


def test_boundary_checks_under_sanitizers(sanitized_lib):
    lib, asan, ubsan = sanitized_lib
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join([asan, ubsan] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else []))
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["GPTOSS_ATTN_LIBRARY"] = lib
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail, tail
