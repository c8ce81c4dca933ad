"""The C ABI's host code (irreps parser, plan and CG table builder, argument
validation) under AddressSanitizer, LeakSanitizer and
UndefinedBehaviorSanitizer: capi.cpp is recompiled with the sanitizers on its
host pass only, linked with the library's other objects and a host driver
(tests/host/abi_sanitizer_driver.cpp) that runs no kernel, and the driver
must finish clean.  Needs the objects of a library build (skipped without)."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_abi_host_code_is_sanitizer_clean(tmp_path):
    objs = [o for o in glob.glob(os.path.join(ROOT, "_build", "*.o")) if not o.endswith("capi.cpp.o")]
    if not objs or not os.path.exists(HIPCC) or shutil.which("g++") is None:
        pytest.skip("needs a library build, hipcc and g++")
    inc = os.path.join(ROOT, "include")
    capi = str(tmp_path / "capi_san.o")
    drv = str(tmp_path / "driver.o")
    exe = str(tmp_path / "driver")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-fconstexpr-steps=100000000", "-Wno-unused-command-line-argument", f"-I{inc}",
                    *san, "-Xarch_host", "-fno-omit-frame-pointer", "-c",
                    os.path.join(ROOT, "tensor_product_convolution_amd", "csrc", "capi.cpp"), "-o", capi],
                   check=True, capture_output=True, timeout=600)
    subprocess.run(["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{inc}", "-c",
                    os.path.join(ROOT, "tests", "host", "abi_sanitizer_driver.cpp"), "-o", drv],
                   check=True, capture_output=True, timeout=300)
    subprocess.run([HIPCC, "--offload-arch=gfx950", *san, drv, capi, *objs, "-o", exe],
                   check=True, capture_output=True, timeout=600)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "OK (0 failures)" in r.stdout, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
