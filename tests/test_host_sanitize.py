"""The C ABI's host code (argument validation, workspace layouts, the launch
sequences of every entry point) built for the host alone with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, every kernel launcher a
no-op stub, and run through valid and invalid calls (tests/host_sanitize).
No GPU and no device code: the HIP runtime library is linked only for its
host calls (error strings, device queries that fail without a GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fine_grained_mixture_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "lib")),
                    reason="needs g++ and the ROCm host libraries")
def test_host_code_under_asan_and_ubsan(tmp_path):
    import sys
    sys.path.insert(0, HERE)
    from make_stubs import stubs
    (tmp_path / "stubs.cpp").write_text(stubs(open(os.path.join(CSRC, "moe_internal.h")).read()))
    exe = tmp_path / "host_checks"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g", "-O1"]
    cmd = ["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *san,
           os.path.join(CSRC, "api.cpp"), str(tmp_path / "stubs.cpp"),
           os.path.join(HERE, "driver.cpp"), f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failures" in r.stdout and "runtime error" not in r.stderr
