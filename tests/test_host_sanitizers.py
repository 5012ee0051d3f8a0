"""Host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

`host_sanitize/driver.cpp` calls every entry point with arguments that
validation must reject (so no kernel is launched and no GPU is needed) and
checks the host-only threshold DP against exhaustive enumeration.  The C-ABI
layer and the driver are compiled by g++ with both sanitizers and linked
against the library's kernel objects from `_build/` (their host parts
uninstrumented); a sanitizer report fails the run.  CPU only.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_long_stride_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
KERNEL_OBJECTS = ["calib.hip.o", "flash_bf16.hip.o", "flash_fp32.hip.o", "score_bf16.hip.o",
                  "score_fp32.hip.o", "select.hip.o"]


def test_c_abi_host_code_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    objs = [os.path.join(BUILD, o) for o in KERNEL_OBJECTS]
    if gxx is None or not all(os.path.exists(o) for o in objs):
        pytest.skip("needs g++ and the kernel objects of a library build in _build/")
    # g++ compiles the HIP runtime headers as plain host C++ once told the platform
    flags = ["-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("api.o", "driver.o", "driver"))
    for src, obj in ((os.path.join(CSRC, "xattn_api.cpp"), api_o),
                     (os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp"), drv_o)):
        r = subprocess.run([gxx] + flags + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([gxx, "-fsanitize=address,undefined", drv_o, api_o] + objs +
                       [f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",   # the HIP runtime's own allocations are not ours
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert "all checks passed" in r.stdout
