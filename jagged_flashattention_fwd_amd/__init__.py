"""Python binding of libjfa.so, the gfx950 jagged flash-attention library.

Argument marshalling only: every step of the computation runs in the
library's HIP kernels.  torch provides device memory and the current stream.
The C functions keep their names (jfa_fwd, jfa_bwd, ...); `attention_fwd` and
`attention_bwd` additionally allocate outputs and the workspace with torch.
If the library is missing, or no GPU is present, calls raise RuntimeError;
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libjfa.so")

JFA_OK = 0
STATUS_NAMES = {0: "JFA_OK", 1: "JFA_ERR_INVALID_ARG", 2: "JFA_ERR_UNSUPPORTED",
                3: "JFA_ERR_WORKSPACE", 4: "JFA_ERR_HIP"}

# Symbols declared in include/jfa.h, with their ctypes signatures.
_c = ctypes
_SIGS = {
    "jfa_workspace_size": (_c.c_size_t, [_c.c_int64, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                         _c.c_int, _c.c_int]),
    "jfa_fwd": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int,
                           _c.c_int, _c.c_int, _c.c_float, _c.c_int, _c.c_int, _c.c_void_p,
                           _c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "jfa_bwd": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int,
                           _c.c_int, _c.c_int, _c.c_float, _c.c_int, _c.c_int, _c.c_void_p,
                           _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                           _c.c_int64, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "jfa_workspace_size_gqa": (_c.c_size_t, [_c.c_int64, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                             _c.c_int, _c.c_int, _c.c_int]),
    "jfa_fwd_ex": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int,
                              _c.c_int, _c.c_int, _c.c_int, _c.c_float, _c.c_int, _c.c_int, _c.c_int,
                              _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "jfa_bwd_ex": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int,
                              _c.c_int, _c.c_int, _c.c_int, _c.c_float, _c.c_int, _c.c_int, _c.c_int,
                              _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                              _c.c_int64, _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "jfa_fwd_noalloc": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int,
                                   _c.c_int, _c.c_int, _c.c_int, _c.c_float, _c.c_int, _c.c_int, _c.c_int,
                                   _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p]),
    "jfa_fwd_mxfp8": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                 _c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_float,
                                 _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p,
                                 _c.c_size_t, _c.c_void_p]),
    "jfa_mxfp8_t_pad": (_c.c_int64, [_c.c_int64]),
    "jfa_bwd_mxfp8": (_c.c_int, [_c.c_void_p] * 15 + [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_float,
                                                      _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                                      _c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_void_p,
                                                      _c.c_size_t, _c.c_void_p]),
    "jfa_schedule_params": (_c.c_int, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.POINTER(_c.c_int),
                                       _c.POINTER(_c.c_int)]),
    "jfa_debug_schedule": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                      _c.c_int, _c.c_int64, _c.c_void_p, _c.c_int64, _c.c_void_p,
                                      _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "jfa_debug_schedule_ex": (_c.c_int, [_c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
                                         _c.c_int, _c.c_int, _c.c_int64, _c.c_void_p, _c.c_int64, _c.c_void_p,
                                         _c.c_void_p, _c.c_size_t, _c.c_void_p]),
    "jfa_status_string": (_c.c_char_p, [_c.c_int]),
    "jfa_timing_enable": (_c.c_int, [_c.c_int]),
    "jfa_timing_reset": (_c.c_int, []),
    "jfa_timing_read": (_c.c_int, [_c.c_int, _c.POINTER(_c.c_int64), _c.POINTER(_c.c_double)]),
    "jfa_kernel_name": (_c.c_char_p, [_c.c_int]),
}

_lib = None


def lib():
    """The loaded library (raises RuntimeError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m jagged_flashattention_fwd_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(rc: int) -> str:
    return lib().jfa_status_string(rc).decode()


def _check(rc: int, what: str):
    if rc != JFA_OK:
        raise RuntimeError(f"{what}: {status_string(rc)}")


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ------------------------------------------------------- C names ---------
def jfa_workspace_size(total_len, B, H, Lq, d, causal, broadcast_q, pass_) -> int:
    n = lib().jfa_workspace_size(int(total_len), B, H, Lq, d, int(causal), int(broadcast_q), pass_)
    if n == 0:
        raise RuntimeError("jfa_workspace_size: arguments rejected")
    return n


def jfa_workspace_size_gqa(total_len, B, H, H_kv, Lq, d, causal, broadcast_q, pass_) -> int:
    n = lib().jfa_workspace_size_gqa(int(total_len), B, H, H_kv, Lq, d, int(causal), int(broadcast_q), pass_)
    if n == 0:
        raise RuntimeError("jfa_workspace_size_gqa: arguments rejected")
    return n


def jfa_fwd_ex(q, k, v, offsets, B, H, H_kv, Lq, d, scale, causal, window, broadcast_q, out, lse, total_len,
               workspace, stream=None):
    _check(lib().jfa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(offsets), B, H, H_kv, Lq, d, float(scale),
                            int(causal), int(window), int(broadcast_q), _ptr(out), _ptr(lse), int(total_len),
                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream(stream)), "jfa_fwd_ex")


def jfa_bwd_ex(q, k, v, offsets, B, H, H_kv, Lq, d, scale, causal, window, broadcast_q, out, lse, dout, dq,
               dk, dv, total_len, workspace, stream=None):
    _check(lib().jfa_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(offsets), B, H, H_kv, Lq, d, float(scale),
                            int(causal), int(window), int(broadcast_q), _ptr(out), _ptr(lse), _ptr(dout),
                            _ptr(dq), _ptr(dk), _ptr(dv), int(total_len), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream)), "jfa_bwd_ex")


def jfa_fwd_noalloc(q, k, v, offsets, B, H, H_kv, Lq, d, scale, causal, window, broadcast_q, out, lse, total_len,
                    stream=None):
    _check(lib().jfa_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(offsets), B, H, H_kv, Lq, d, float(scale),
                                 int(causal), int(window), int(broadcast_q), _ptr(out), _ptr(lse),
                                 int(total_len), _stream(stream)), "jfa_fwd_noalloc")


def jfa_fwd_mxfp8(q8, q_scale, k8, k_scale, vt8, vt_scale, offsets, B, H, H_kv, Lq, d, scale, causal,
                  broadcast_q, out, lse, total_len, workspace, stream=None):
    _check(lib().jfa_fwd_mxfp8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(vt8), _ptr(vt_scale),
                               _ptr(offsets), B, H, H_kv, Lq, d, float(scale), int(causal), int(broadcast_q),
                               _ptr(out), _ptr(lse), int(total_len), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)), "jfa_fwd_mxfp8")


def jfa_bwd_mxfp8(t, offsets, B, H, H_kv, Lq, d, scale, causal, broadcast_q, out, lse, dq, dk, dv, total_len,
                  workspace, stream=None):
    """t: the uint8 encodings by their header names (q8, q_scale, qt8,
    qt_scale, k8, k_scale, kt8, kt_scale, v8, v_scale, do8, do_scale, dot8,
    dot_scale)."""
    enc = [_ptr(t[n]) for n in ("q8", "q_scale", "qt8", "qt_scale", "k8", "k_scale", "kt8", "kt_scale", "v8",
                                "v_scale", "do8", "do_scale", "dot8", "dot_scale")]
    _check(lib().jfa_bwd_mxfp8(*enc, _ptr(offsets), B, H, H_kv, Lq, d, float(scale), int(causal),
                               int(broadcast_q), _ptr(out), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                               int(total_len), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream)), "jfa_bwd_mxfp8")


def jfa_mxfp8_t_pad(total_len) -> int:
    return int(lib().jfa_mxfp8_t_pad(int(total_len)))


def jfa_schedule_params(pass_, causal, broadcast_q, d):
    br, w = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().jfa_schedule_params(pass_, int(causal), int(broadcast_q), d, ctypes.byref(br),
                                     ctypes.byref(w)), "jfa_schedule_params")
    return br.value, w.value


def jfa_fwd(q, k, v, offsets, B, H, Lq, d, scale, causal, broadcast_q, out, lse, total_len,
            workspace, stream=None):
    _check(lib().jfa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(offsets), B, H, Lq, d, float(scale),
                         int(causal), int(broadcast_q), _ptr(out), _ptr(lse), int(total_len),
                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                         _stream(stream)), "jfa_fwd")


def jfa_bwd(q, k, v, offsets, B, H, Lq, d, scale, causal, broadcast_q, out, lse, dout, dq, dk, dv,
            total_len, workspace, stream=None):
    _check(lib().jfa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(offsets), B, H, Lq, d, float(scale),
                         int(causal), int(broadcast_q), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                         _ptr(dk), _ptr(dv), int(total_len), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream(stream)), "jfa_bwd")


def jfa_debug_schedule(offsets, B, H, Lq, causal, broadcast_q, pass_, total_len, tiles, n_tiles,
                       workspace, stream=None):
    _check(lib().jfa_debug_schedule(_ptr(offsets), B, H, Lq, int(causal), int(broadcast_q), pass_,
                                    int(total_len), _ptr(tiles), tiles.shape[0], _ptr(n_tiles),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "jfa_debug_schedule")


def jfa_debug_schedule_ex(offsets, B, H, H_kv, Lq, causal, broadcast_q, list_, total_len, tiles, n_tiles,
                          workspace, stream=None):
    _check(lib().jfa_debug_schedule_ex(_ptr(offsets), B, H, H_kv, Lq, int(causal), int(broadcast_q), list_,
                                       int(total_len), _ptr(tiles), tiles.shape[0], _ptr(n_tiles),
                                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(stream)), "jfa_debug_schedule_ex")


def jfa_timing_enable(capacity: int):
    _check(lib().jfa_timing_enable(int(capacity)), "jfa_timing_enable")


def jfa_timing_reset():
    _check(lib().jfa_timing_reset(), "jfa_timing_reset")


def jfa_timing_read(kernel: int):
    n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
    _check(lib().jfa_timing_read(int(kernel), ctypes.byref(n), ctypes.byref(ms)), "jfa_timing_read")
    return n.value, ms.value


def jfa_kernel_name(kernel: int):
    r = lib().jfa_kernel_name(int(kernel))
    return None if r is None else r.decode()


def kernel_times():
    """{kernel name: (launches, total ms)} of every kernel timed since the last reset."""
    out = {}
    k = 0
    while True:
        name = jfa_kernel_name(k)
        if name is None:
            return out
        out[name] = jfa_timing_read(k)
        k += 1


# --------------------------------------------- allocating helpers --------
def _shape_args(q, k, offsets, broadcast_q):
    """(B, H, H_kv, Lq, d, T): query heads from q, key / value heads from k."""
    T, H_kv, d = k.shape
    B = offsets.numel() - 1
    H = q.shape[0] if broadcast_q else q.shape[1]
    Lq = q.shape[1] if broadcast_q else 0
    return B, H, H_kv, Lq, d, T


def workspace(total_len, B, H, Lq, d, causal, broadcast_q, pass_, device, H_kv=None):
    import torch
    n = jfa_workspace_size_gqa(total_len, B, H, H if H_kv is None else H_kv, Lq, d, causal, broadcast_q, pass_)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def attention_fwd(q, k, v, offsets, scale, causal=False, broadcast_q=True, ws=None, window=0):
    """(out bf16, lse fp32) of jagged attention; see include/jfa.h for layouts
    (k / v with fewer heads than q: grouped-query attention; window > 0 with
    causal: sliding window)."""
    import torch
    B, H, H_kv, Lq, d, T = _shape_args(q, k, offsets, broadcast_q)
    if broadcast_q:
        out = torch.empty((B, H, Lq, d), dtype=torch.bfloat16, device=k.device)
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=k.device)
    else:
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device=k.device)
        lse = torch.empty((T, H), dtype=torch.float32, device=k.device)
    if ws is None:
        ws = workspace(T, B, H, Lq, d, causal, broadcast_q, 0, k.device, H_kv)
    jfa_fwd_ex(q, k, v, offsets, B, H, H_kv, Lq, d, scale, causal, window, broadcast_q, out, lse, T, ws)
    return out, lse


def attention_bwd(q, k, v, offsets, scale, causal, broadcast_q, out, lse, dout, ws=None, window=0):
    """(dq, dk, dv) fp32 of jagged attention; see include/jfa.h for layouts
    (dk / dv with k's head count)."""
    import torch
    B, H, H_kv, Lq, d, T = _shape_args(q, k, offsets, broadcast_q)
    dq = torch.empty(q.shape, dtype=torch.float32, device=k.device)
    dk = torch.empty((T, H_kv, d), dtype=torch.float32, device=k.device)
    dv = torch.empty((T, H_kv, d), dtype=torch.float32, device=k.device)
    if ws is None:
        ws = workspace(T, B, H, Lq, d, causal, broadcast_q, 1, k.device, H_kv)
    jfa_bwd_ex(q, k, v, offsets, B, H, H_kv, Lq, d, scale, causal, window, broadcast_q, out, lse, dout, dq, dk,
               dv, T, ws)
    return dq, dk, dv


def attention_fwd_mxfp8(q8, q_scale, k8, k_scale, vt8, vt_scale, offsets, scale, causal=False, broadcast_q=True,
                        ws=None):
    """(out bf16, lse fp32) of the MXFP8 forward on uint8 E4M3 / E8M0 codes;
    see include/jfa.h (jfa_fwd_mxfp8) for layouts."""
    import torch
    B, H, H_kv, Lq, d, T = _shape_args(q8, k8, offsets, broadcast_q)
    if broadcast_q:
        out = torch.empty((B, H, Lq, d), dtype=torch.bfloat16, device=k8.device)
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=k8.device)
    else:
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device=k8.device)
        lse = torch.empty((T, H), dtype=torch.float32, device=k8.device)
    if ws is None:
        ws = workspace(T, B, H, Lq, d, causal, broadcast_q, 0, k8.device, H_kv)
    jfa_fwd_mxfp8(q8, q_scale, k8, k_scale, vt8, vt_scale, offsets, B, H, H_kv, Lq, d, scale, causal, broadcast_q,
                  out, lse, T, ws)
    return out, lse


def attention_bwd_mxfp8(t, offsets, scale, causal, broadcast_q, out, lse, ws=None):
    """(dq, dk, dv) fp32 of the MXFP8 backward; t holds the uint8 encodings
    by their header names (include/jfa.h, jfa_bwd_mxfp8), out / lse are the
    MXFP8 forward's outputs."""
    import torch
    q8, k8 = t["q8"], t["k8"]
    B, H, H_kv, Lq, d, T = _shape_args(q8, k8, offsets, broadcast_q)
    dev = k8.device
    dq = torch.empty(q8.shape, dtype=torch.float32, device=dev)
    dk = torch.empty((T, H_kv, d), dtype=torch.float32, device=dev)
    dv = torch.empty((T, H_kv, d), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(T, B, H, Lq, d, causal, broadcast_q, 1, dev, H_kv)
    jfa_bwd_mxfp8(t, offsets, B, H, H_kv, Lq, d, scale, causal, broadcast_q, out, lse, dq, dk, dv, T, ws)
    return dq, dk, dv
