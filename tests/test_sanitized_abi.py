"""The C ABI layer's argument checks, built for the host with
AddressSanitizer and UndefinedBehaviorSanitizer (g++; the kernel side is
replaced by host-only stubs, so no device is needed) and driven through
every rejection path, the size arithmetic near the int64 limits included."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(f"{ROCM}/lib/libamdhip64.so"),
                                reason="needs g++ and the HIP runtime library")


def test_argument_checks_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include",
           f"-I{ROOT}/linear_attention_rnn_amd/csrc", os.path.join(HERE, "abi_driver.cpp"),
           os.path.join(HERE, "kernel_stub.cpp"), os.path.join(ROOT, "linear_attention_rnn_amd", "csrc", "wkv6_api.cpp"),
           f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib", "-lamdhip64", "-lpthread", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "all argument checks hold" in out
