"""Host code under AddressSanitizer (CPU only, no GPU needed).

Every csrc/*.hip is compiled with its host half instrumented (each sanitizer
flag passed to hipcc behind -Xarch_host, so the device code is built as
usual), linked with tests/host_abi_driver.cpp by clang++ with the ASan
runtime, and run.  The driver calls every C-ABI entry point with arguments
the library rejects before any HIP call and reads every error string; ASan
aborts on any invalid host memory access in that code.  A second run makes
the driver overflow a heap array on purpose, which must be reported, so a
build without instrumentation cannot pass unnoticed."""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_55_amd", "csrc")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
ROCM_LIB = "/opt/rocm/lib"
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics",
         "-Wno-inline-asm", "-I", os.path.join(ROOT, "include")]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="needs hipcc and the ROCm clang++")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    out = tmp_path_factory.mktemp("asan")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(ROOT, "tests", "host_abi_driver.cpp")]

    def compile_one(src):
        obj = str(out / (os.path.basename(src) + ".o"))
        extra = ["-mllvm", "-amdgpu-mfma-vgpr-form"] if os.path.basename(src) in ("fa_bwd.hip", "fa_calib.hip") else []
        res = subprocess.run([HIPCC, *FLAGS, *extra, *HOST_ASAN, "-c", src, "-o", obj],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(out / "host_abi_driver")
    res = subprocess.run([CLANG, "-fsanitize=address", *objs, f"-L{ROCM_LIB}", "-lamdhip64",
                          f"-Wl,-rpath,{ROCM_LIB}", "-o", exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return exe


def test_abi_validation_is_clean_under_asan(driver):
    res = subprocess.run([driver], capture_output=True, text=True, env=ENV, timeout=120)
    assert "AddressSanitizer" not in res.stderr, res.stderr[-3000:]
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout + res.stderr[-2000:]


def test_asan_is_live_in_the_build(driver):
    res = subprocess.run([driver, "--selftest-overflow"], capture_output=True, text=True, env=ENV,
                         timeout=120)
    assert res.returncode != 0
    assert "heap-buffer-overflow" in res.stderr, res.stderr[-2000:]
