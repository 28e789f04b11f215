"""The C-ABI host layer under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

tests/abi_asan_driver.cpp calls every entry point of include/attn.h with
invalid arguments (and one valid call, which must fail the device check on a
machine without a GPU).  Here the host layer (attn_api.hip) and the driver are
compiled with the sanitizers on the host side only, linked against the
library's kernel objects, and run; any sanitizer report or wrong status fails
the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    import torch

    if torch.cuda.is_available():
        pytest.skip("the driver's last call expects a machine without a GPU")
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from exact_io_aware_75_amd import build as b

    objs = [os.path.join(b.BUILD, os.path.splitext(s)[0] + ".o") for s in b.SOURCES if s != "attn_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        b.build()
    out = tmp_path_factory.mktemp("asan")
    common = [f"--offload-arch={b.ARCH}", "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include")]
    api_o = str(out / "attn_api_asan.o")
    r = subprocess.run([HIPCC, *common, *SAN, "-c", os.path.join(b.CSRC, "attn_api.hip"), "-o", api_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    drv_o = str(out / "abi_asan_driver.o")
    r = subprocess.run([HIPCC, *common, *SAN, "-c", os.path.join(ROOT, "tests", "abi_asan_driver.cpp"), "-o", drv_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(out / "abi_asan_driver")
    r = subprocess.run([HIPCC, f"--offload-arch={b.ARCH}", *SAN, drv_o, api_o, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    yield exe
    shutil.rmtree(out, ignore_errors=True)


def test_host_layer_is_clean_under_sanitizers(driver):
    env = dict(os.environ)
    # the HIP runtime's own allocations are not the library's: leak checking off
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([driver], capture_output=True, text=True, timeout=300, env=env)
    assert "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert r.stdout.strip().endswith("0 failures")
