"""The C ABI library loads and exports every symbol include/svlm.h declares;
host-side validation rejects bad arguments before touching a device."""
import ctypes as C
import os

import pytest

from tests._util import declared_symbols
from visual_kv_pruning_amd import _lib as L


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libsvlm.so is not built (run python -m visual_kv_pruning_amd.build)")
    return L.load()


def test_header_declares_the_five_calls():
    syms = declared_symbols()
    for name in ("svlm_score", "svlm_select", "svlm_gather_kv", "svlm_decode_attn", "svlm_verify"):
        assert name in syms


def test_every_declared_symbol_is_exported(lib):
    syms = declared_symbols()
    assert len(syms) >= 12
    for name in syms:
        assert hasattr(lib, name), name
        assert name in L.SIGNATURES, f"{name} has no ctypes signature"


def test_version_and_status_strings(lib):
    assert lib.svlm_abi_version() == L.ABI_VERSION == 4
    for st in range(5):
        assert lib.svlm_status_string(st)
    assert b"unknown" in lib.svlm_status_string(99)


def test_workspace_queries_are_host_only(lib):
    assert lib.svlm_select_workspace(4, 1000, 100, 1.0) == 0
    # the split top-K form needs a workspace: pure top-K on rows past 32768 tokens
    assert lib.svlm_select_workspace(112, 141120, 1024, 1.0) > 0
    assert lib.svlm_select_workspace(112, 141120, 1024, 0.5) == 0
    assert lib.svlm_select_workspace(1, 32768, 1024, 1.0) == 0
    assert lib.svlm_select_workspace(0, 141120, 1024, 1.0) == 0


def test_split_select_plan(lib):
    """The split top-K plan, seen through its workspace (2 x R x C x 4 bytes,
    each half rounded up to 256; C = segments x budget).  Without a GPU the
    chip is taken as 256 CUs."""
    def ws(R, C):
        half = (R * C * 4 + 255) // 256 * 256
        return 2 * half
    # 112 rows of 141120: 6 segments of ~24576 would need a third round of
    # 1024-thread workgroups, so the fewest possible, 4 of 35280, are taken
    assert lib.svlm_select_workspace(112, 141120, 1024, 1.0) == ws(112, 4 * 1024)
    # 4 rows: 6 segments of 23520 fit one round
    assert lib.svlm_select_workspace(4, 141120, 1024, 1.0) == ws(4, 6 * 1024)
    # 2 segments of 19600 for 39200 tokens; 2 x 16384 candidates still fit
    # one register-resident row, 2 x 16385 do not (one-workgroup form)
    assert lib.svlm_select_workspace(3, 39200, 16384, 1.0) == ws(3, 2 * 16384)
    assert lib.svlm_select_workspace(3, 39200, 16385, 2.0) == 0
    # rows that fit one workgroup's registers are never split
    assert lib.svlm_select_workspace(500, 32768, 10, 1.0) == 0
    assert lib.svlm_select_workspace(100, 32769, 10, 1.0) == ws(100, 2 * 10)
    # 500 such rows: two segments each would double the rounds of workgroups,
    # and one segment is no split
    assert lib.svlm_select_workspace(500, 32769, 10, 1.0) == 0
    assert lib.svlm_verify_workspace(1, 5, 152064) > 0
    assert lib.svlm_verify_workspace(0, 5, 10) == 0


def test_verify_workspace_layout(lib):
    """The acceptance workspace opens with 256 KB of arrival counters (one per
    sequence index, the same place for every call shape), then the chunk
    results of the larger of the two forms: greedy 8 bytes per (row, 16384
    vocabulary entries), rejection 24 bytes per 1024 entries."""
    def expect(batch, gamma, V):
        greedy = batch * (gamma + 1) * (-(-V // 16384)) * 8
        reject = batch * (-(-V // 1024)) * 24
        return 256 * 1024 + max(greedy, reject)
    for batch, gamma, V in ((1, 5, 152064), (4, 9, 152064), (3, 70, 5000), (1, 1, 1), (2, 63, 1_100_000)):
        assert lib.svlm_verify_workspace(batch, gamma, V) == expect(batch, gamma, V)
    # every shape of a smaller call fits the workspace of a larger one
    assert lib.svlm_verify_workspace(1, 5, 152064) <= lib.svlm_verify_workspace(4, 9, 152064)


NULL = None


def _attn(lib, **kw):
    args = dict(q=NULL, q_sb=0, k=NULL, v=NULL, kv_sb=0, kv_sh=0, kv_sn=128, kv_len=NULL, max_kv_len=10,
                dtype=L.SVLM_BF16, batch=1, nq=1, Hq=8, Hkv=2, D=128, scale=0.1, causal=0, out=NULL, lse=NULL,
                num_splits=0, ws=NULL, ws_bytes=0, stream=NULL)
    args.update(kw)
    return lib.svlm_decode_attn(*args.values())


def test_decode_attn_rejects_bad_arguments(lib):
    fake = C.c_void_p(4096)   # never dereferenced: validation fails first
    ok = dict(q=fake, k=fake, v=fake, kv_len=fake, out=fake)
    assert _attn(lib, D=96, **ok) == L.SVLM_E_UNSUPPORTED
    assert _attn(lib, dtype=7, **ok) == L.SVLM_E_UNSUPPORTED
    # fp32 operands: rows of 16-byte multiples (4 elements), so 100 passes and 102 fails
    assert _attn(lib, dtype=L.SVLM_F32, kv_sn=102, **ok) == L.SVLM_E_INVALID
    assert _attn(lib) == L.SVLM_E_INVALID                              # null pointers
    assert _attn(lib, Hq=6, Hkv=4, **ok) == L.SVLM_E_INVALID          # Hq % Hkv
    assert _attn(lib, nq=0, **ok) == L.SVLM_E_INVALID
    assert _attn(lib, scale=float("inf"), **ok) == L.SVLM_E_INVALID
    assert _attn(lib, scale=0.0, **ok) == L.SVLM_E_INVALID             # the row maxima assume scale > 0
    assert _attn(lib, scale=-0.1, **ok) == L.SVLM_E_INVALID
    assert _attn(lib, nq=4096, Hq=4096, Hkv=4096, **ok) == L.SVLM_E_UNSUPPORTED   # queries past a 32-bit range
    assert _attn(lib, max_kv_len=1 << 23, num_splits=1, **ok) == L.SVLM_E_UNSUPPORTED  # one split past 2^31 bytes
    assert b"2^31" in lib.svlm_last_error()
    assert _attn(lib, causal=2, **ok) == L.SVLM_E_INVALID
    assert _attn(lib, kv_sn=100, **ok) == L.SVLM_E_INVALID            # row stride not a multiple of 8
    assert _attn(lib, q=C.c_void_p(4098), k=fake, v=fake, kv_len=fake, out=fake) == L.SVLM_E_INVALID  # misaligned
    assert b"16-byte" in lib.svlm_last_error()


def _attn_idx(lib, **kw):
    args = dict(q=NULL, q_sb=0, k=NULL, v=NULL, kv_sb=0, kv_sh=0, kv_sn=128, kv_rows=100, kv_idx=NULL, idx_sb=0,
                idx_sh=0, n_idx=NULL, n_sb=1, n_sh=0, max_n_idx=10, dtype=L.SVLM_BF16, batch=1, nq=1, Hq=8, Hkv=2, D=128,
                scale=0.1, causal=0, out=NULL, lse=NULL, num_splits=0, ws=NULL, ws_bytes=0, stream=NULL)
    args.update(kw)
    return lib.svlm_decode_attn_indexed(*args.values())


def test_decode_attn_indexed_rejects_bad_arguments(lib):
    fake = C.c_void_p(4096)   # never dereferenced: validation fails first
    ok = dict(q=fake, k=fake, v=fake, kv_idx=fake, n_idx=fake, out=fake)
    assert _attn_idx(lib, **dict(ok, kv_idx=NULL)) == L.SVLM_E_INVALID
    assert b"index" in lib.svlm_last_error()
    assert _attn_idx(lib, kv_rows=0, **ok) == L.SVLM_E_INVALID
    assert _attn_idx(lib, kv_rows=1 << 24, **ok) == L.SVLM_E_INVALID   # 2^24 rows x 256 B > 2^31
    assert _attn_idx(lib, idx_sh=-1, **ok) == L.SVLM_E_INVALID
    assert _attn_idx(lib, n_sh=-1, **ok) == L.SVLM_E_INVALID
    assert b"length" in lib.svlm_last_error()
    assert _attn_idx(lib, D=96, **ok) == L.SVLM_E_UNSUPPORTED
    # a long list needs more splits than asked for: the split length is capped
    # (the split's list is staged on chip), so the workspace is never zero
    assert lib.svlm_decode_attn_indexed_workspace(1, 1, 8, 2, 128, 10000, 1) > 0
    assert lib.svlm_decode_attn_workspace(1, 1, 8, 2, 128, 10000, 1) == 0


def test_uvprune_rejects_bad_arguments(lib):
    fake = C.c_void_p(4096)
    f = lib.svlm_uvprune_score
    assert f(fake, fake, 256, 10, fake, fake, 256, 4, 256, L.SVLM_F32, 1.0, 0.0, fake, fake, 1 << 20, NULL) \
        == L.SVLM_E_UNSUPPORTED
    assert f(fake, fake, 256, 10, fake, fake, 256, 4, 250, L.SVLM_BF16, 1.0, 0.0, fake, fake, 1 << 20, NULL) \
        == L.SVLM_E_UNSUPPORTED                                       # d % 8
    assert f(fake, fake, 256, 10, fake, fake, 256, 4, 32768, L.SVLM_BF16, 1.0, 0.0, fake, fake, 1 << 20, NULL) \
        == L.SVLM_E_UNSUPPORTED                                       # d too large
    assert f(fake, fake, 128, 10, fake, fake, 256, 4, 256, L.SVLM_BF16, 1.0, 0.0, fake, fake, 1 << 20, NULL) \
        == L.SVLM_E_INVALID                                           # stride < d
    assert f(fake, fake, 256, 10, fake, fake, 256, 4, 256, L.SVLM_BF16, float("nan"), 0.0, fake, fake, 1 << 20,
             NULL) == L.SVLM_E_INVALID
    assert f(fake, fake, 256, 10, fake, fake, 256, 4, 256, L.SVLM_BF16, 1.0, 0.0, fake, fake, 16, NULL) \
        == L.SVLM_E_WORKSPACE
    assert lib.svlm_uvprune_workspace(128, 8192) >= 2 * 8192 * 4


def test_verify_select_gather_score_reject_bad_arguments(lib):
    fake = C.c_void_p(4096)
    assert lib.svlm_verify(7, 1, 1, 10, fake, fake, fake, fake, fake, fake, fake, 1 << 20, NULL) == L.SVLM_E_INVALID
    assert lib.svlm_verify(0, 1, 0, 10, fake, fake, fake, fake, fake, fake, fake, 1 << 20, NULL) == L.SVLM_E_INVALID
    assert lib.svlm_verify(1, 1, 2, 10, fake, fake, NULL, fake, fake, fake, fake, 1 << 20, NULL) == L.SVLM_E_INVALID
    assert lib.svlm_verify(0, 1, 2, 10, fake, fake, NULL, NULL, fake, fake, NULL, 0, NULL) == L.SVLM_E_WORKSPACE
    # select: budget beyond n_vis, bad grid, too long rows
    assert lib.svlm_select(fake, 20, 1, 2, 2, 5, 0.5, 21, fake, fake, NULL, NULL, 0, NULL) == L.SVLM_E_INVALID
    assert lib.svlm_select(fake, 20, 1, 0, 2, 5, 0.5, 2, fake, fake, NULL, NULL, 0, NULL) == L.SVLM_E_INVALID
    assert lib.svlm_select(fake, 1 << 20, 1, 1024, 16, 17, 0.5, 2, fake, fake, NULL, NULL, 0, NULL) == L.SVLM_E_UNSUPPORTED
    assert lib.svlm_select(fake, 20, 1, 2, 2, 5, float("nan"), 2, fake, fake, NULL, NULL, 0, NULL) == L.SVLM_E_INVALID
    assert lib.svlm_select(fake, 10, 1, 2, 2, 5, 0.5, 2, fake, fake, NULL, NULL, 0, NULL) == L.SVLM_E_INVALID  # stride
    # select: the split top-K form (pure top-K, rows past 32768 tokens, no tags)
    # needs its workspace; with tags it takes the one-workgroup form and none
    need = lib.svlm_select_workspace(2, 141120, 1024, 1.0)
    assert lib.svlm_select(fake, 141120, 2, 720, 14, 14, 1.0, 1024, fake, fake, NULL, NULL, 0, NULL) \
        == L.SVLM_E_WORKSPACE
    assert lib.svlm_select(fake, 141120, 2, 720, 14, 14, 1.0, 1024, fake, fake, NULL, fake, need - 1, NULL) \
        == L.SVLM_E_WORKSPACE
    # select with no rows is a no-op (nothing is launched, pointers may be null)
    assert lib.svlm_select(NULL, 20, 0, 2, 2, 5, 0.5, 2, NULL, NULL, NULL, NULL, 0, NULL) == L.SVLM_OK
    # gather: tail past the source, unsupported D
    assert lib.svlm_gather_kv(fake, fake, 0, 128, 10, fake, 0, 3, 8, 3, fake, fake, 0, 128, 1, 128, 0, NULL) == L.SVLM_E_INVALID
    assert lib.svlm_gather_kv(fake, fake, 0, 128, 10, fake, 0, 3, 0, 3, fake, fake, 0, 128, 1, 80, 0, NULL) == L.SVLM_E_UNSUPPORTED
    assert lib.svlm_gather_kv(fake, fake, 0, 128, 10, fake, 0, 3, 0, 3, fake, fake, 0, 128, 1, 128, 5, NULL) == L.SVLM_E_UNSUPPORTED
    # fp32 rows: a row stride of 68 elements is 272 bytes (a 16-byte multiple), 66 is not
    assert lib.svlm_gather_kv(fake, fake, 0, 66, 10, fake, 0, 3, 0, 3, fake, fake, 0, 64, 1, 64, 1, NULL) == L.SVLM_E_INVALID
    # score: T too large, visual range beyond what text sees, non-positive scale
    args = [fake, 1024, 128, fake, 1 << 16, 128, 0, 200, 300, 100, 0, 50, 8, 2, 128, 0.1, 2, 1.0, 0.0, fake, fake, 1 << 20, NULL]
    assert lib.svlm_score(*args) == L.SVLM_E_UNSUPPORTED
    args[7] = 16
    args[11] = 150
    assert lib.svlm_score(*args) == L.SVLM_E_INVALID
    args[11] = 50
    args[15] = -0.1
    assert lib.svlm_score(*args) == L.SVLM_E_INVALID
    args[15] = 0.1
    args[16] = 9
    assert lib.svlm_score(*args) == L.SVLM_E_INVALID
    args[16] = 2
    args[1] = 1 << 27                        # one head's queries past a 32-bit buffer range
    assert lib.svlm_score(*args) == L.SVLM_E_UNSUPPORTED
    # score_layers: layer count, layer-mean flag, per-head rows under the layer
    # mean, a short workspace; the workspace of one layer is svlm_score's
    la = [fake, 1024, 128, 1 << 20, fake, 1 << 16, 128, 1 << 22, 2, 0, 16, 300, 100, 0, 50, 8, 2, 128, 0.1, 2, 1,
          1.0, 0.0, fake, fake, 1 << 30, NULL]
    for i, val, want in ((8, 0, L.SVLM_E_INVALID), (20, 2, L.SVLM_E_INVALID), (19, 0, L.SVLM_E_UNSUPPORTED),
                         (25, 16, L.SVLM_E_WORKSPACE), (3, 3, L.SVLM_E_INVALID)):
        bad = list(la)
        bad[i] = val
        assert lib.svlm_score_layers(*bad) == want, (i, val)
    one = lib.svlm_score_workspace(16, 8, 2, 100, 50)
    assert lib.svlm_score_layers_workspace(1, 16, 8, 2, 100, 50) == one > 0
    assert lib.svlm_score_layers_workspace(3, 16, 8, 2, 100, 50) >= 3 * one
    assert lib.svlm_score_layers_workspace(0, 16, 8, 2, 100, 50) == 0


def test_noalloc_refuses_state_beyond_its_scratch_on_the_host(lib):
    """The no-allocation attention call checks its split-K state against the
    static scratch before anything else touches the device."""
    fake = C.c_void_p(4096)
    need = lib.svlm_decode_attn_workspace(1, 64, 64, 8, 128, 1 << 20, 256)
    assert need > L.SVLM_NOALLOC_SCRATCH_BYTES
    st = lib.svlm_decode_attn_noalloc(fake, 64 * 64 * 128, fake, fake, 0, 128 << 20, 128, fake, 1 << 20,
                                      L.SVLM_BF16, 1, 64, 64, 8, 128, C.c_float(0.1), 1, fake, fake, 256, None)
    assert st == L.SVLM_E_UNSUPPORTED
    assert b"scratch" in lib.svlm_last_error()


def test_debug_library_exports_every_symbol():
    """libsvlm_debug.so (SVLM_DEBUG: kernels record violated device
    preconditions) carries the same ABI."""
    if not os.path.exists(L.DEBUG_LIB_PATH):
        pytest.fail("libsvlm_debug.so is not built (run python -m visual_kv_pruning_amd.build)")
    dbg = L.load_debug()
    assert dbg.svlm_abi_version() == L.ABI_VERSION
    for name in declared_symbols():
        assert hasattr(dbg, name), name


def test_debug_flags_outside_a_debug_build(lib):
    v = C.c_uint(7)
    assert lib.svlm_debug_flags(C.byref(v)) == L.SVLM_E_UNSUPPORTED and v.value == 0
    assert b"SVLM_DEBUG" in lib.svlm_last_error()
    assert lib.svlm_debug_flags(None) == L.SVLM_E_INVALID


def test_debug_flags_of_the_debug_build_without_work():
    """Reading the flags launches nothing: OK (flags 0) where a device is
    present, SVLM_E_HIP where none is."""
    dbg = L.load_debug()
    v = C.c_uint(7)
    st = dbg.svlm_debug_flags(C.byref(v))
    assert st in (L.SVLM_OK, L.SVLM_E_HIP)
    assert v.value == 0 or st == L.SVLM_OK
    assert dbg.svlm_debug_flags(None) == L.SVLM_E_INVALID


def _workspace_in_subprocess(env_value):
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("from visual_kv_pruning_amd import _lib as L; lib = L.load(); "
            "print(lib.svlm_decode_attn_workspace(1, 6, 64, 8, 128, 25222, 0), "
            "lib.svlm_decode_attn_workspace(1, 6, 64, 8, 128, 25222, 5), "
            "lib.svlm_decode_attn_indexed_workspace(1, 1, 64, 8, 128, 2638, 0), "
            "lib.svlm_decode_attn_indexed_workspace(1, 1, 64, 8, 128, 2638, 5))")
    env = dict(os.environ)
    env.pop("SVLM_NUM_SPLITS", None)
    if env_value is not None:
        env["SVLM_NUM_SPLITS"] = env_value
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, cwd=root, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    return [int(x) for x in r.stdout.split()]


def test_num_splits_environment_override():
    """SVLM_NUM_SPLITS replaces the planner's split count for calls that
    leave it to the library (num_splits = 0), in the workspace queries as in
    the launches (one planner); invalid values are ignored."""
    auto, five, iauto, ifive = _workspace_in_subprocess("5")
    assert auto == five > 0 and iauto == ifive > 0
    default = _workspace_in_subprocess(None)
    assert _workspace_in_subprocess("abc")[0] == default[0]
    assert _workspace_in_subprocess("-3")[0] == default[0]
    assert default[1] == five
