"""The C ABI's host code under AddressSanitizer (CPU only).

api.cpp is compiled with host-side AddressSanitizer (device code untouched) and linked with
the library's other objects and tests/asan_abi_main.cpp, which calls every entry point with
invalid arguments (documented status, nothing launched) and with valid ones whose placeholder
device addresses reach the launchers.  Run only where no GPU is visible: there every launch
fails with NM_ERR_HIP before touching memory.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None or shutil.which("g++") is None, reason="hipcc and g++ are needed")
@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="runs only where no GPU is visible")
def test_abi_host_code_under_asan(tmp_path):
    from sparse_matmul_ffns_amd import build
    build.build()
    objs = [os.path.join(build.BUILD, os.path.splitext(s)[0] + ".o") for s in build.SOURCES if s != "api.cpp"]
    inc = os.path.join(ROOT, "include")
    api_o, main_o, exe = tmp_path / "api_asan.o", tmp_path / "main.o", tmp_path / "abi_asan"
    flags = [f for f in build.FLAGS if not f.startswith("-O")]
    res = subprocess.run([_hipcc(), "-x", "hip", *flags, "-O1", "-g", "-Xarch_host", "-fsanitize=address",
                          "-c", os.path.join(ROOT, "sparse_matmul_ffns_amd", "csrc", "api.cpp"), "-o", str(api_o)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    res = subprocess.run(["g++", "-std=c++17", "-g", "-fsanitize=address", f"-I{inc}", "-c",
                          os.path.join(ROOT, "tests", "asan_abi_main.cpp"), "-o", str(main_o)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    res = subprocess.run([_hipcc(), f"--offload-arch={build.ARCH}", "-Xarch_host", "-fsanitize=address", str(main_o),
                          str(api_o), *objs, "-o", str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0 and "asan abi ok" in res.stdout, (res.returncode, res.stdout[-2000:],
                                                                 res.stderr[-4000:])
