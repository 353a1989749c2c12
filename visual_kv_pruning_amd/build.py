"""Build libsvlm.so (all HIP sources under csrc/) for gfx950 with hipcc, in-tree.

Usage: python -m visual_kv_pruning_amd.build   (or call build()).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsvlm.so")
# the same sources with -DSVLM_DEBUG: kernels also record violated device
# preconditions, read back with svlm_debug_flags()
DEBUG_LIB = os.path.join(PKG, "libsvlm_debug.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}",
]
# per-source additions: the score passes keep their matrix-core accumulators in
# ordinary VGPRs (the exponentials read every one of them; accumulator
# registers would cost a move per element)
EXTRA = {
    "score.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(job) -> str:
    src, debug = job
    out_dir = os.path.join(BUILD, "debug") if debug else BUILD
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DSVLM_DEBUG"] if debug else []), *EXTRA.get(os.path.basename(src), []),
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}{' (SVLM_DEBUG)' if debug else ''}:\n{r.stderr[-4000:]}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    # -z defs: a symbol left undefined (a kernel launch stub the compiler did
    # not emit, say) fails the link here instead of the library's first load
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libsvlm.so and libsvlm_debug.so;
    always rebuilds.  Returns the path of libsvlm.so."""
    os.makedirs(os.path.join(BUILD, "debug"), exist_ok=True)
    srcs = sources()
    jobs = [(s, False) for s in srcs] + [(s, True) for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], DEBUG_LIB)
    if verbose:
        print(f"built {LIB} and {os.path.basename(DEBUG_LIB)} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
