"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every source of the library is compiled with the sanitizers on its host side (device code at -O0, never
run), linked with tests/sanitize/validation_driver.cpp, and run: the driver makes every entry point fail
validation on fake pointers, and runs the pure host code (workspace sizes and layout, the sampler
schedule, error strings).  No GPU is touched: on a machine without one the device check itself takes
the HIP-error path."""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not installed")
def test_validation_layer_under_asan_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(ROOT, "quantized_video_diffusion_amd", "csrc", "*.hip")))
    assert srcs

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-Xarch_device", "-O0", "-g0", "-std=c++17", "-fPIC",
               *HOST_SAN, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr[-3000:]}"
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "driver.o")
    san = "-fsanitize=address,undefined"
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c++17", san, "-fno-sanitize-recover=undefined",
                        "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "sanitize", "validation_driver.cpp"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "driver")
    r = subprocess.run([CLANG, san, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    nm = shutil.which("nm")
    if nm:
        syms = subprocess.run([nm, exe], capture_output=True, text=True).stdout
        assert "__asan_report_load" in syms and "__ubsan_handle" in syms, "sanitizers not linked in"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "all checks passed" in out
