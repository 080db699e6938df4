"""CPU-only checks of the C-ABI library: it loads, exports every function
include/jfa.h declares, and rejects bad arguments on the host before any
HIP call (no compute is attempted here)."""
import ctypes
import math
import os
import re

import pytest

import jagged_flashattention_fwd_amd as jfa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(jfa.LIB_PATH):
        from jagged_flashattention_fwd_amd import build
        build.build()
    return jfa.lib()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "jfa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jfa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_calls():
    assert _declared_functions() == sorted([
        "jfa_bwd", "jfa_debug_schedule", "jfa_fwd", "jfa_kernel_name", "jfa_schedule_params",
        "jfa_status_string", "jfa_timing_enable", "jfa_timing_read", "jfa_timing_reset",
        "jfa_workspace_size", "jfa_workspace_size_gqa", "jfa_fwd_ex", "jfa_bwd_ex", "jfa_debug_schedule_ex", "jfa_fwd_noalloc",
        "jfa_fwd_mxfp8", "jfa_mxfp8_t_pad", "jfa_bwd_mxfp8"])


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(jfa.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(raw, name), name
    assert set(jfa._SIGS) == set(_declared_functions())


def test_status_strings(lib):
    for code, name in jfa.STATUS_NAMES.items():
        assert jfa.status_string(code).startswith(name)
    assert "unknown" in jfa.status_string(99)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def _fwd(lib, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, off=FAKE, B=2, H=2, Lq=8, d=128, scale=0.1, causal=0, bq=1,
                out=FAKE, lse=FAKE, T=10, ws=FAKE, wsb=1 << 30)
    args.update(kw)
    vp = ctypes.c_void_p
    return lib.jfa_fwd(vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["off"]), args["B"],
                       args["H"], args["Lq"], args["d"], args["scale"], args["causal"], args["bq"],
                       vp(args["out"]), vp(args["lse"]), args["T"], vp(args["ws"]), args["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(off=0), 1), (dict(out=0), 1), (dict(ws=0), 1),
    (dict(q=FAKE + 2), 1), (dict(lse=FAKE + 1), 1), (dict(off=FAKE + 4), 1),
    (dict(scale=math.inf), 1), (dict(scale=math.nan), 1),
    (dict(B=0), 1), (dict(H=0), 1), (dict(T=-1), 1), (dict(Lq=0), 1),
    (dict(d=96), 2), (dict(d=256), 2), (dict(B=8193), 2),
])
def test_fwd_rejects_bad_arguments_before_any_hip_call(lib, kw, code):
    assert _fwd(lib, **kw) == code


def test_bwd_rejects_null_gradient(lib):
    vp = ctypes.c_void_p
    rc = lib.jfa_bwd(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 2, 2, 8, 128, 0.1, 0, 1, vp(FAKE),
                     vp(FAKE), vp(FAKE), None, vp(FAKE), vp(FAKE), 10, vp(FAKE), 1 << 30, None)
    assert rc == 1


def test_workspace_size_argument_checks(lib):
    # rejected sizes give 0 bytes (a valid workspace is never empty)
    assert lib.jfa_workspace_size(10, 2, 2, 8, 96, 0, 1, 0) == 0
    assert lib.jfa_workspace_size(10, 0, 2, 8, 128, 0, 1, 0) == 0
    assert lib.jfa_workspace_size(10, 2, 2, 8, 128, 0, 1, 7) == 0
    assert lib.jfa_workspace_size(-1, 2, 2, 8, 128, 0, 1, 0) == 0
    assert lib.jfa_workspace_size_gqa(10, 2, 4, 3, 8, 128, 0, 1, 1) == 0


def _bwd(lib, scale, **kw):
    vp = ctypes.c_void_p
    args = dict(B=2, H=2, Lq=8, d=128, causal=0, bq=1, T=10)
    args.update(kw)
    return lib.jfa_bwd(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), args["B"], args["H"], args["Lq"], args["d"],
                       scale, args["causal"], args["bq"], vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                       vp(FAKE), args["T"], vp(FAKE), 1 << 30, None)


@pytest.mark.parametrize("scale", [0.0, -0.0, 1e-31, -1e-35, 2.0 ** -101, math.inf, math.nan])
def test_bwd_rejects_zero_and_tiny_scale(lib, scale):
    """The backward folds -lse / scale into its score products: |scale| below
    2^-100 (scale = 0 included) is an argument error, found on the host."""
    assert _bwd(lib, scale) == 1
    vp = ctypes.c_void_p
    assert lib.jfa_bwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 2, 2, 1, 8, 128, scale, 0, 0, 1, vp(FAKE),
                          vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 10, vp(FAKE), 1 << 30, None) == 1


@pytest.mark.parametrize("scale", [2.0 ** -100, -(2.0 ** -100), -0.3, 1e30])
def test_bwd_accepts_scales_from_the_minimum(lib, scale):
    # past the scale check the next failure is the missing device (HIP error),
    # or success where a GPU is present -- never an argument error
    assert _bwd(lib, scale, d=96) == 2  # unsupported head dim is still reported
    assert _bwd(lib, scale, B=0) == 1


@pytest.mark.parametrize("kw", [dict(list_=3), dict(list_=-1), dict(list_=2, bq=1), dict(H_kv=3),
                                dict(cap=-1), dict(tiles=0)])
def test_debug_schedule_ex_argument_checks(lib, kw):
    vp = ctypes.c_void_p
    a = dict(H=4, H_kv=2, bq=0, list_=1, cap=16, tiles=FAKE)
    a.update(kw)
    assert lib.jfa_debug_schedule_ex(vp(FAKE), 2, a["H"], a["H_kv"], 8, 0, a["bq"], a["list_"], 10,
                                     vp(a["tiles"]), a["cap"], vp(FAKE), vp(FAKE), 1 << 30, None) == 1


@pytest.mark.parametrize("H,H_kv", [(4, 3), (4, 0), (2, 4), (6, -1)])
def test_gqa_calls_reject_heads_that_do_not_split(lib, H, H_kv):
    vp = ctypes.c_void_p
    assert lib.jfa_workspace_size_gqa(10, 2, H, H_kv, 8, 128, 0, 1, 1) == 0
    assert lib.jfa_fwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 2, H, H_kv, 8, 128, 0.1, 0, 0, 1, vp(FAKE),
                          vp(FAKE), 10, vp(FAKE), 1 << 30, None) == 1
    assert lib.jfa_bwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 2, H, H_kv, 8, 128, 0.1, 0, 0, 1, vp(FAKE),
                          vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 10, vp(FAKE), 1 << 30, None) == 1


def test_gqa_calls_check_sizes_like_the_plain_ones(lib):
    vp = ctypes.c_void_p
    assert lib.jfa_fwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 2, 4, 2, 8, 96, 0.1, 0, 0, 1, vp(FAKE),
                          vp(FAKE), 10, vp(FAKE), 1 << 30, None) == 2
    assert lib.jfa_fwd_ex(vp(FAKE), vp(0), vp(FAKE), vp(FAKE), 2, 4, 2, 8, 128, 0.1, 0, 0, 1, vp(FAKE),
                          vp(FAKE), 10, vp(FAKE), 1 << 30, None) == 1


@pytest.mark.parametrize("causal,window,code", [(0, 5, 2), (1, -1, 1), (0, -3, 1)])
def test_window_argument_checks(lib, causal, window, code):
    vp = ctypes.c_void_p
    assert lib.jfa_fwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 2, 2, 2, 8, 128, 0.1, causal, window, 1,
                          vp(FAKE), vp(FAKE), 10, vp(FAKE), 1 << 30, None) == code
    assert lib.jfa_bwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 2, 2, 2, 8, 128, 0.1, causal, window, 1,
                          vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 10, vp(FAKE), 1 << 30,
                          None) == code


def test_kernel_names(lib):
    names = []
    k = 0
    while jfa.jfa_kernel_name(k) is not None:
        names.append(jfa.jfa_kernel_name(k))
        k += 1
    assert "fwd_kernel" in names and "dkdv_kernel" in names and len(names) == len(set(names))
    assert lib.jfa_timing_read(-1, None, None) == 1


def test_noalloc_forward_host_checks(lib):
    """jfa_fwd_noalloc checks its arguments, and its size against the static
    scratch, before any HIP call."""
    vp = ctypes.c_void_p

    def call(B=2, H=2, H_kv=2, Lq=8, d=128, scale=0.1, q=FAKE, T=10):
        return lib.jfa_fwd_noalloc(vp(q), vp(FAKE), vp(FAKE), vp(FAKE), B, H, H_kv, Lq, d, scale, 0, 0, 0,
                                   vp(FAKE), vp(FAKE), T, None)
    assert call(q=0) == 1
    assert call(d=96) == 2
    assert call(scale=math.nan) == 1
    assert call(H_kv=3) == 1
    # 1000 heads x (8192 sequences + 2^30 / 256 rows) tiles: far beyond the 16 MiB scratch
    assert call(B=8192, H=1000, H_kv=1000, T=1 << 30) == 3


def test_mxfp8_forward_host_checks(lib):
    """jfa_fwd_mxfp8 rejects bad arguments before any HIP call: missing or
    misaligned scale arrays, a head dim other than 128, the forward's own
    checks, a missing workspace."""
    vp = ctypes.c_void_p

    def call(qs=FAKE, ks=FAKE, vs=FAKE, d=128, q=FAKE, H_kv=2, scale=0.1, ws=FAKE):
        return lib.jfa_fwd_mxfp8(vp(q), vp(qs), vp(FAKE), vp(ks), vp(FAKE), vp(vs), vp(FAKE), 2, 2, H_kv, 8, d,
                                 scale, 0, 1, vp(FAKE), vp(FAKE), 10, vp(ws), 1 << 20, None)
    assert call(qs=0) == 1 and call(ks=0) == 1 and call(vs=0) == 1
    assert call(qs=FAKE + 1) == 1 and call(ks=FAKE + 2) == 1 and call(vs=FAKE + 3) == 1
    assert call(q=0) == 1 and call(q=FAKE + 8) == 1
    assert call(d=64) == 2 and call(d=96) == 2
    assert call(H_kv=3) == 1 and call(scale=math.inf) == 1
    assert call(ws=0) == 1 and call(ws=FAKE + 4) == 1
    # transposed rows past (2^31 - 1) / 32 keys
    assert lib.jfa_fwd_mxfp8(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 2, 2, 2, 8, 128,
                             0.1, 0, 1, vp(FAKE), vp(FAKE), 1 << 27, vp(FAKE), 1 << 40, None) == 2


def test_mxfp8_t_pad(lib):
    assert [lib.jfa_mxfp8_t_pad(n) for n in (0, 1, 63, 64, 65, 1000)] == [64, 64, 64, 64, 128, 1024]
    assert lib.jfa_mxfp8_t_pad(-5) == -1


def test_mxfp8_backward_host_checks(lib):
    """jfa_bwd_mxfp8 rejects bad arguments before any HIP call: any missing
    or misaligned encoding, scale array or output, a head dim other than
    128, heads that do not split, a non-finite scale."""
    vp = ctypes.c_void_p

    def call(over=None, d=128, H_kv=2, scale=0.1):
        ptrs = [FAKE] * 15 + [FAKE] * 5 + [FAKE]  # 14 encodings, offsets; out, lse, dq, dk, dv; workspace
        for i, v in (over or {}).items():
            ptrs[i] = v
        enc, offs, outs, ws = ptrs[:14], ptrs[14], ptrs[15:20], ptrs[20]
        return lib.jfa_bwd_mxfp8(*[vp(x) for x in enc], vp(offs), 2, 2, H_kv, 8, d, scale, 0, 1,
                                 *[vp(x) for x in outs], 10, vp(ws), 1 << 30, None)
    for i in range(21):
        assert call({i: 0}) == 1, i
    for i in (0, 2, 4, 6, 8, 10, 12, 15, 17, 18, 19, 20):   # codes, out, dq, dk, dv, workspace: 16 bytes
        assert call({i: FAKE + 4}) == 1, i
    for i in (1, 3, 5, 7, 9, 11, 13, 16):                    # scale arrays, lse: 4 bytes
        assert call({i: FAKE + 2}) == 1, i
    assert call({14: FAKE + 4}) == 1                         # offsets: 8 bytes
    assert call(d=64) == 2 and call(d=96) == 2
    assert call(H_kv=3) == 1 and call(scale=math.nan) == 1 and call(scale=-math.inf) == 1
    ptrs = [vp(FAKE)] * 15
    assert lib.jfa_bwd_mxfp8(*ptrs, 2, 2, 2, 8, 128, 0.1, 0, 1, *[vp(FAKE)] * 5, 1 << 27, vp(FAKE), 1 << 40,
                             None) == 2
