"""The C ABI's host code (validation, workspace sizing, launch sequencing of every entry point
over every band class and engine) built with AddressSanitizer and UndefinedBehaviorSanitizer
by the host compiler, with counting stubs in place of the kernel launchers
(tests/asan/capi_driver.cpp); no GPU and no device code are involved."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "entropic_ot_attention_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs the host C++ compiler")
def test_capi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "capi_driver"
    sanitize = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                "-fno-omit-frame-pointer"]
    cmd = ["g++", "-std=c++17", "-O1", "-g", *sanitize, "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "asan", "capi_driver.cpp"),
           os.path.join(CSRC, "ska_capi.cpp"), os.path.join(CSRC, "ska_geometry.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "failures 0" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
