"""The host layer of libattnq.so under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only: every -fsanitize= applies to the
host compilation through -Xarch_host; device code is built as usual),
driven through every entry point's argument validation by
tests/csrc/abi_sanitize.c.  CPU only: every call fails validation or has
nothing to do, so no kernel is launched.  The other sources' objects come
from the regular build (paged_kv_amd/_build)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
BUILD = os.path.join(ROOT, "paged_kv_amd", "_build")
SRC = os.path.join(ROOT, "paged_kv_amd", "csrc")


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain missing")
def test_host_layer_under_asan_and_ubsan(tmp_path):
    objs = sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD) if f.endswith(".o") and f != "api.o") \
        if os.path.isdir(BUILD) else []
    if not objs:
        pytest.skip("library objects not built (python -m paged_kv_amd.build)")
    api_o = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libattnq_san.so")
    drv = str(tmp_path / "abi_sanitize")
    san_host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           *san_host, "-c", os.path.join(SRC, "api.hip"), "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", api_o, *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    driver_cmd = [CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                  os.path.join(ROOT, "tests", "csrc", "abi_sanitize.c"), lib, "-Wl,-rpath," + str(tmp_path),
                  "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lm", "-o", drv]
    r = subprocess.run(driver_cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([drv], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert "all statuses as expected" in out
