"""ctypes loader for libsvlm.so: the C ABI declared in include/svlm.h.

Argument marshalling only.  Loading fails loudly when the library is missing;
there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SVLM_LIB", os.path.join(_HERE, "libsvlm.so"))
# the same library built with SVLM_DEBUG (device preconditions checked in the kernels)
DEBUG_LIB_PATH = os.environ.get("SVLM_DEBUG_LIB", os.path.join(_HERE, "libsvlm_debug.so"))

SVLM_OK, SVLM_E_INVALID, SVLM_E_UNSUPPORTED, SVLM_E_WORKSPACE, SVLM_E_HIP = range(5)
SVLM_BF16, SVLM_F32 = 0, 1
SVLM_AGG_QHEAD, SVLM_AGG_KVHEAD, SVLM_AGG_ALL = 0, 1, 2
SVLM_VERIFY_GREEDY, SVLM_VERIFY_REJECT = 0, 1
SVLM_NOALLOC_SCRATCH_BYTES = 16 << 20
(SVLM_DBG_KV_LEN, SVLM_DBG_KV_INDEX, SVLM_DBG_GATHER_INDEX, SVLM_DBG_DRAFT_TOKEN, SVLM_DBG_PROB_RANGE,
 SVLM_DBG_SCORE_RANGE) = (1, 2, 4, 8, 16, 32)

vp, i64, i32, f32, f64, sz = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_double, C.c_size_t

# name -> (restype, argtypes), in the order of include/svlm.h
SIGNATURES = {
    "svlm_abi_version": (i32, []),
    "svlm_status_string": (C.c_char_p, [i32]),
    "svlm_last_error": (C.c_char_p, []),
    "svlm_score_workspace": (sz, [i32, i32, i32, i32, i32]),
    "svlm_score": (i32, [vp, i64, i64, vp, i64, i64, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                         f32, i32, f32, f32, vp, vp, sz, vp]),
    "svlm_score_layers_workspace": (sz, [i32, i32, i32, i32, i32, i32]),
    "svlm_score_layers": (i32, [vp, i64, i64, i64, vp, i64, i64, i64, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                i32, f32, i32, i32, f32, f32, vp, vp, sz, vp]),
    "svlm_select_workspace": (sz, [i32, i32, i32, f64]),
    "svlm_select": (i32, [vp, i64, i32, i32, i32, i32, f64, i32, vp, vp, vp, vp, sz, vp]),
    "svlm_gather_kv": (i32, [vp, vp, i64, i64, i32, vp, i64, i32, i32, i32, vp, vp, i64, i64, i32, i32, i32, vp]),
    "svlm_decode_attn_workspace": (sz, [i32, i32, i32, i32, i32, i32, i32]),
    "svlm_decode_attn": (i32, [vp, i64, vp, vp, i64, i64, i64, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                               vp, vp, i32, vp, sz, vp]),
    "svlm_decode_attn_noalloc": (i32, [vp, i64, vp, vp, i64, i64, i64, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                       i32, vp, vp, i32, vp]),
    "svlm_decode_attn_indexed_workspace": (sz, [i32, i32, i32, i32, i32, i32, i32]),
    "svlm_decode_attn_indexed": (i32, [vp, i64, vp, vp, i64, i64, i64, i32, vp, i64, i64, vp, i64, i64, i32, i32,
                                       i32, i32, i32, i32, i32, f32, i32, vp, vp, i32, vp, sz, vp]),
    "svlm_uvprune_workspace": (sz, [i32, i32]),
    "svlm_uvprune_score": (i32, [vp, vp, i64, i32, vp, vp, i64, i32, i32, i32, f32, f32, vp, vp, sz, vp]),
    "svlm_verify_workspace": (sz, [i32, i32, i32]),
    "svlm_verify": (i32, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
    "svlm_stream_read": (i32, [vp, i64, i32, vp, vp]),
    "svlm_debug_flags": (i32, [C.POINTER(C.c_uint)]),
}

ABI_VERSION = 4  # SVLM_ABI_VERSION of include/svlm.h

_lib = None
_debug_lib = None


class SvlmError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


def _open(path: str) -> C.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{os.path.basename(path)} not found at {path}: build it with `python -m visual_kv_pruning_amd.build` "
            "(there is no non-HIP fallback)")
    lib = C.CDLL(path)
    lib.svlm_abi_version.restype = C.c_int
    if lib.svlm_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {lib.svlm_abi_version()}, these bindings expect "
                          f"{ABI_VERSION}: rebuild it")
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load() -> C.CDLL:
    """Load libsvlm.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


def load_debug() -> C.CDLL:
    """Load libsvlm_debug.so (once): the same calls, with the kernels also
    recording violated device preconditions (svlm_debug_flags)."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _open(DEBUG_LIB_PATH)
    return _debug_lib


def debug_flags(lib: C.CDLL) -> int:
    """Flags recorded by `lib` since the previous read (which clears them)."""
    v = C.c_uint(0)
    st = lib.svlm_debug_flags(C.byref(v))
    if st != SVLM_OK:
        raise SvlmError("svlm_debug_flags", st, lib.svlm_last_error().decode(errors="replace"))
    return int(v.value)


def call(name: str, *args) -> None:
    """Invoke an svlm_* entry point that returns a status; raise SvlmError unless SVLM_OK."""
    lib = load()
    st = getattr(lib, name)(*args)
    if st != SVLM_OK:
        raise SvlmError(name, st, lib.svlm_last_error().decode(errors="replace"))
