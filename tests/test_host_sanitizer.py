"""The C ABI's host code (argument checks, error messages; csrc/ttt_api.cpp) built with
AddressSanitizer and UndefinedBehaviorSanitizer for the host and driven through every entry
point's rejection paths by tests/host_sanitizer_driver.cpp, on one thread and on four at
once.  Every call is rejected before any HIP call, so it needs no GPU: the sanitized
ttt_api.cpp is linked with the kernels' objects of the ordinary build."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "test_sequence_layers_amd")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")


@pytest.mark.skipif(HIPCC is None, reason="hipcc not found")
def test_c_abi_host_code_under_asan_and_ubsan(tmp_path):
    from test_sequence_layers_amd import build as B
    objs = [o for o in glob.glob(os.path.join(B.OUT_DIR, "*.hip.o"))]
    if len(objs) < len(glob.glob(os.path.join(B.CSRC, "*.hip"))):
        B.build()
        objs = glob.glob(os.path.join(B.OUT_DIR, "*.hip.o"))
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    api = tmp_path / "ttt_api_san.o"
    common = [HIPCC, f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
              "-I", os.path.join(ROOT, "include")]
    r = subprocess.run(common + san + ["-x", "hip", "-c", os.path.join(B.CSRC, "ttt_api.cpp"), "-o", str(api)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    drv = tmp_path / "driver_san.o"
    r = subprocess.run(common + san + ["-x", "c++", "-c", os.path.join(ROOT, "tests", "host_sanitizer_driver.cpp"),
                                       "-o", str(drv)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "abi_san"
    r = subprocess.run(common + san + [str(drv), str(api), *objs, "-o", str(exe), "-lpthread"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert "OK: 0 failure(s)" in out
