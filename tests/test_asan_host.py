"""The host-side argument validation of every C-ABI entry point under
AddressSanitizer (CPU only, no GPU touched).

Every HIP source of the library is compiled with the host half instrumented
(the device code is built as usual) and linked with tests/asan/abi_driver.cpp,
which calls each entry point with invalid and valid arguments.  Every device
pointer it passes is the address of a freed heap block, so a host-side read
through one is reported as a use-after-free; every error message is read in
full.  The build is cached under block_scaled_fp4_moe_amd/_build_asan and
redone when a source, header, the driver or the flags change.
"""

import concurrent.futures
import glob
import hashlib
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_scaled_fp4_moe_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
DRIVER = os.path.join(ROOT, "tests", "asan", "abi_driver.cpp")
OUT = os.path.join(PKG, "_build_asan")
# host code instrumented, device code untouched; no packed fp32 in device code
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
         "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]


def _inputs():
    return (sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip"))),
            sorted(glob.glob(os.path.join(PKG, "csrc", "*.h"))) +
            [os.path.join(ROOT, "include", "fp4moe.h")])


def _build():
    srcs, headers = _inputs()
    h = hashlib.sha256(" ".join(FLAGS).encode())
    for f in srcs + headers + [DRIVER]:
        h.update(f.encode())
        h.update(open(f, "rb").read())
    key = h.hexdigest()
    exe = os.path.join(OUT, "abi_driver")
    stamp = os.path.join(OUT, "stamp")
    if os.path.exists(exe) and os.path.exists(stamp) and open(stamp).read() == key:
        return exe
    os.makedirs(OUT, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        r = subprocess.run([HIPCC] + FLAGS + ["-c", src, "-o", obj], capture_output=True,
                           text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr[-3000:]}"
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, srcs + [DRIVER]))
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address"] +
                       objs + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    open(stamp, "w").write(key)
    return exe


def test_host_validation_under_address_sanitizer():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert " 0 failures" in r.stdout, r.stdout
