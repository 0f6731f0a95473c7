"""The C ABI's host code (argument checks, argument packing, error messages)
built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and run
against a driver whose kernel launchers are stubs (tests/host_sanitize).  The
driver calls every entry point with valid arguments (exactly one launch each,
with the arguments the header promises) and with invalid or extreme ones (no
launch, a status and a message); any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefill_causal_attention_amd", "csrc")
ROCM = "/opt/rocm"


def test_abi_host_code_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP headers")
    # the host source is compiled as plain C++ (it holds no device code)
    src = tmp_path / "pca_api.cpp"
    shutil.copyfile(os.path.join(CSRC, "pca_api.hip"), src)
    exe = tmp_path / "abi_driver"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = [gxx, "-std=c++17", "-O1", "-g", *san, "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           str(src), os.path.join(ROOT, "tests", "host_sanitize", "abi_driver.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-6000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert out.startswith("OK:"), out[-2000:]
