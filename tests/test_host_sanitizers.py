"""The library's host code (argument validation, workspace planning, status
text) built with AddressSanitizer and UndefinedBehaviorSanitizer, driven on
the CPU by tests/host_validation_driver.c: every entry point is called with
arguments it must refuse before touching a device, and the workspace queries
with valid and extreme sizes.  Nothing is launched, so no GPU is needed; the
device code of this build is compiled as usual (the sanitizers apply to the
host pass only)."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "visual_kv_pruning_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="needs hipcc and the ROCm clang")


def test_host_validation_under_asan_and_ubsan(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(f):
        extra = ["-mllvm", "-amdgpu-mfma-vgpr-form"] if f == "score.hip" else []
        out = str(tmp_path / (f[:-4] + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", *san, "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", *extra, f"-I{ROOT}/include", f"-I{CSRC}", "-c",
               os.path.join(CSRC, f), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return out

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libsvlm_san.so")
    clangxx = CLANG + "++"
    r = subprocess.run([clangxx, "-shared", "-fPIC", "-fsanitize=address,undefined", "-o", lib, *objs,
                        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    drv = str(tmp_path / "drv")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", f"-I{ROOT}/include",
                        os.path.join(ROOT, "tests", "host_validation_driver.c"), f"-L{tmp_path}", "-lsvlm_san",
                        f"-Wl,-rpath,{tmp_path}", "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([drv], capture_output=True, text=True, env=env, timeout=120)
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, r.stderr[-3000:]
