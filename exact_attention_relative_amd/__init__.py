"""Python binding of the relpos_attn C ABI (argument marshalling only).

Every function here forwards device pointers and sizes to librelpos_attn.so; all arithmetic
runs in the library's HIP kernels.  The library is loaded on first use and a missing build is
an error, never a fallback.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librelpos_attn.so")

RELPOS_T5, RELPOS_SHAW, RELPOS_TXL, RELPOS_DEBERTA, RELPOS_ALIBI = 0, 1, 2, 3, 4
RELPOS_BF16, RELPOS_FP32 = 0, 1
MECH_IDS = {"t5": RELPOS_T5, "shaw": RELPOS_SHAW, "txl": RELPOS_TXL, "deberta": RELPOS_DEBERTA,
            "alibi": RELPOS_ALIBI}

RELPOS_OK = 0
RELPOS_E_INVALID = -1
RELPOS_E_UNSUPPORTED = -2
RELPOS_E_WORKSPACE = -3
RELPOS_E_LAUNCH = -4

EXPORTED = ("relpos_attn_workspace_size", "relpos_attn_fwd", "relpos_attn_fwd_noalloc", "relpos_attn_bwd",
            "relpos_index_map", "relpos_profile_events", "relpos_status_string", "relpos_version",
            "relpos_project_fwd", "relpos_project_workspace_size", "relpos_project_bwd")
RELPOS_PROF_OFF, RELPOS_PROF_FWD, RELPOS_PROF_BWD_DQ, RELPOS_PROF_BWD_DKDV = 0, 1, 2, 3


class relpos_desc(ctypes.Structure):
    _fields_ = [("mech", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("batch", ctypes.c_int64), ("heads", ctypes.c_int64),
                ("seqlen", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
                ("rel_span", ctypes.c_int32), ("num_buckets", ctypes.c_int32),
                ("max_distance", ctypes.c_int32), ("bidirectional", ctypes.c_int32),
                ("scale", ctypes.c_float), ("max_partial_bytes", ctypes.c_int64),
                ("rel_head_stride", ctypes.c_int64)]


class relpos_proj_desc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("in_features", ctypes.c_int64), ("heads", ctypes.c_int64),
                ("head_dim", ctypes.c_int64)]


class RelposError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {relpos_status_string(status)} ({status})")
        self.status = status


_lib = None


def load_library(path: str | None = None):
    """Load librelpos_attn.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m exact_attention_relative_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dp = ctypes.POINTER(relpos_desc)
    lib.relpos_attn_workspace_size.argtypes = [dp, i32, ctypes.POINTER(sz)]
    lib.relpos_attn_workspace_size.restype = i32
    lib.relpos_attn_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.relpos_attn_fwd.restype = i32
    lib.relpos_attn_fwd_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.relpos_attn_fwd_noalloc.restype = i32
    lib.relpos_attn_bwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    vp, vp, vp, sz, vp]
    lib.relpos_attn_bwd.restype = i32
    lib.relpos_index_map.argtypes = [dp, vp, vp, vp]
    lib.relpos_index_map.restype = i32
    lib.relpos_profile_events.argtypes = [vp, vp, i32]
    lib.relpos_profile_events.restype = i32
    lib.relpos_status_string.argtypes = [i32]
    lib.relpos_status_string.restype = ctypes.c_char_p
    pp = ctypes.POINTER(relpos_proj_desc)
    lib.relpos_project_fwd.argtypes = [pp, vp, vp, vp, vp]
    lib.relpos_project_fwd.restype = i32
    lib.relpos_project_workspace_size.argtypes = [pp, ctypes.POINTER(sz)]
    lib.relpos_project_workspace_size.restype = i32
    lib.relpos_project_bwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.relpos_project_bwd.restype = i32
    lib.relpos_version.argtypes = []
    lib.relpos_version.restype = i32
    if path is None:
        _lib = lib
    return lib


def default_rel_head_stride(mech, seqlen, head_dim=64, window=(-1, -1)):
    """The relation-table layout of the pages' workloads: T-XL one r [Nrel, d] per head, Shaw's w
    and DeBERTa's Kr / Qr shared by every head (stride 0)."""
    m = MECH_IDS[mech] if isinstance(mech, str) else int(mech)
    if m != RELPOS_TXL:
        return 0
    nrel = seqlen if window[1] == 0 else max(2 * seqlen - 1, 0)
    return nrel * head_dim


def make_desc(mech, batch, heads, seqlen, head_dim=64, dtype="bf16", window=(-1, -1),
              rel_span=0, num_buckets=32, max_distance=128, bidirectional=True, scale=0.0,
              max_partial_bytes=0, rel_head_stride=None):
    """Descriptor for the attention calls.  rel_head_stride None = default_rel_head_stride."""
    if rel_head_stride is None:
        rel_head_stride = default_rel_head_stride(mech, seqlen, head_dim, window)
    return relpos_desc(MECH_IDS[mech] if isinstance(mech, str) else int(mech),
                       RELPOS_FP32 if dtype in ("fp32", RELPOS_FP32) else RELPOS_BF16,
                       int(batch), int(heads), int(seqlen), int(head_dim),
                       int(window[0]), int(window[1]), int(rel_span), int(num_buckets),
                       int(max_distance), 1 if bidirectional else 0, float(scale),
                       int(max_partial_bytes), int(rel_head_stride))


def make_proj_desc(rows, in_features, heads, head_dim, dtype="bf16"):
    return relpos_proj_desc(RELPOS_FP32 if dtype in ("fp32", RELPOS_FP32) else RELPOS_BF16,
                            int(rows), int(in_features), int(heads), int(head_dim))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != RELPOS_OK:
        raise RelposError(status, what)


def relpos_status_string(status: int) -> str:
    return load_library().relpos_status_string(int(status)).decode()


def relpos_version() -> int:
    return load_library().relpos_version()


def relpos_attn_workspace_size(desc: relpos_desc, pass_: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().relpos_attn_workspace_size(ctypes.byref(desc), int(pass_), ctypes.byref(out)),
           "relpos_attn_workspace_size")
    return out.value


def relpos_attn_fwd(desc, q, k, v, rel_a, rel_b, bias_a, bias_b, o, lse, workspace,
                    workspace_bytes=None, stream=None, check=True) -> int:
    wsb = workspace_bytes if workspace_bytes is not None else (
        0 if workspace is None else workspace.numel() * workspace.element_size())
    st = load_library().relpos_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(rel_a),
                                        _ptr(rel_b), _ptr(bias_a), _ptr(bias_b), _ptr(o), _ptr(lse),
                                        _ptr(workspace), wsb, _stream(stream))
    if check:
        _check(st, "relpos_attn_fwd")
    return st


NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024   # RELPOS_NOALLOC_SCRATCH_BYTES


def relpos_attn_fwd_noalloc(desc, q, k, v, rel_a, rel_b, bias_a, bias_b, o, lse, stream=None,
                            check=True) -> int:
    st = load_library().relpos_attn_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                                _ptr(rel_a), _ptr(rel_b), _ptr(bias_a),
                                                _ptr(bias_b), _ptr(o), _ptr(lse), _stream(stream))
    if check:
        _check(st, "relpos_attn_fwd_noalloc")
    return st


def relpos_attn_bwd(desc, q, k, v, o, lse, dout, rel_a, rel_b, bias_a, bias_b, dq, dk, dv,
                    drel_a, drel_b, dbias_a, dbias_b, workspace, workspace_bytes=None, stream=None,
                    check=True) -> int:
    wsb = workspace_bytes if workspace_bytes is not None else (
        0 if workspace is None else workspace.numel() * workspace.element_size())
    st = load_library().relpos_attn_bwd(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(rel_a),
        _ptr(rel_b), _ptr(bias_a), _ptr(bias_b), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(drel_a),
        _ptr(drel_b), _ptr(dbias_a), _ptr(dbias_b), _ptr(workspace), wsb, _stream(stream))
    if check:
        _check(st, "relpos_attn_bwd")
    return st


def relpos_index_map(desc, out_a, out_b=None, stream=None, check=True) -> int:
    st = load_library().relpos_index_map(ctypes.byref(desc), _ptr(out_a), _ptr(out_b), _stream(stream))
    if check:
        _check(st, "relpos_index_map")
    return st


def relpos_profile_events(start_event, stop_event, kernel: int) -> int:
    """start_event / stop_event: torch.cuda.Event(enable_timing=True) (or raw hipEvent_t ints)."""
    def raw(e):
        if e is None or isinstance(e, int):
            return e
        return e.cuda_event
    st = load_library().relpos_profile_events(raw(start_event), raw(stop_event), int(kernel))
    _check(st, "relpos_profile_events")
    return st


def relpos_project_fwd(desc, X, W, rel, stream=None, check=True) -> int:
    st = load_library().relpos_project_fwd(ctypes.byref(desc), _ptr(X), _ptr(W), _ptr(rel),
                                           _stream(stream))
    if check:
        _check(st, "relpos_project_fwd")
    return st


def relpos_project_workspace_size(desc) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().relpos_project_workspace_size(ctypes.byref(desc), ctypes.byref(out)),
           "relpos_project_workspace_size")
    return out.value


def relpos_project_bwd(desc, X, W, drel, dX, dW, workspace, workspace_bytes=None, stream=None,
                       check=True) -> int:
    wsb = workspace_bytes if workspace_bytes is not None else (
        0 if workspace is None else workspace.numel() * workspace.element_size())
    st = load_library().relpos_project_bwd(ctypes.byref(desc), _ptr(X), _ptr(W), _ptr(drel),
                                           _ptr(dX), _ptr(dW), _ptr(workspace), wsb,
                                           _stream(stream))
    if check:
        _check(st, "relpos_project_bwd")
    return st
