"""The host code of liblores (csrc/lores_api.cpp) built with AddressSanitizer
and UndefinedBehaviorSanitizer (g++, host only) against stand-in kernel
launchers (tests/host/launch_stubs.cpp), and driven by tests/host/host_check.cpp:
layout planning over many shapes, validation, launch grouping, the windowed
states' step bookkeeping and the precision assignment.  No GPU is used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "host_check"
    srcs = [os.path.join(ROOT, "quantized_linear_recurrence_amd", "csrc", "lores_api.cpp"),
            os.path.join(ROOT, "tests", "host", "launch_stubs.cpp"),
            os.path.join(ROOT, "tests", "host", "host_check.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *srcs, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # the ASan runtime need not be the first library loaded in this environment
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "host check ok" in r.stdout, (r.stdout[-3000:], r.stderr[-3000:])
