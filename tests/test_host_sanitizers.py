"""The host layer of libflce under AddressSanitizer and UndefinedBehaviorSanitizer.

flce_api.cpp (the C ABI: validation, plans, workspace layouts, launch
sequences) is built with g++ and both sanitizers, against host-only
stand-ins of the kernel launchers (tests/host/flce_host_stubs.cpp) that
launch nothing: each checks that every workspace pointer it receives, over
the extent its kernel touches, lies inside the caller's workspace, and that
the named workspace buffers of one pass do not overlap.  The driver
(tests/host/flce_host_driver.cpp) calls every entry point over the five
workloads and a sweep of dtypes, shapes, options, plan overrides and strided
token layouts, with fake device addresses, plus invalid calls that must be
refused before any launch.  No GPU and no HIP runtime are used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "linear_cross_entropy_fwd_amd", "csrc", "flce_api.cpp"),
           os.path.join(ROOT, "tests", "host", "flce_host_stubs.cpp"),
           os.path.join(ROOT, "tests", "host", "flce_host_driver.cpp")]
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the HIP headers")
def test_host_layer_under_asan_ubsan(tmp_path):
    exe = tmp_path / "flce_host_driver"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INCLUDE}",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROOT, 'linear_cross_entropy_fwd_amd', 'csrc')}",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           *SOURCES, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-6000:])
    words = r.stdout.split()
    assert words[:1] == ["ok"], r.stdout
    calls, launches = int(words[1]), int(words[2])
    # every configuration of the sweep ran (not an early return)
    assert calls > 10000 and launches > 100000, r.stdout
