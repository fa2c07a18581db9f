"""ctypes binding of libpoetx (C ABI in include/poetx.h).

Argument marshalling only: tensors become device pointers, the current
torch stream becomes the hipStream_t, a status other than POETX_OK becomes a
PoetxError. Every computation runs in the library's HIP kernels; there is no
fallback. Importing this module fails loudly if libpoetx.so is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first, so libpoetx binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
# POETX_LIBRARY may name another build of the same library (the host
# sanitizer build of the CPU tests); by default the in-tree libpoetx.so
LIB_PATH = os.environ.get("POETX_LIBRARY") or os.path.join(_HERE, "libpoetx.so")

POETX_OK = 0
POETX_ERR_NULL = 1
POETX_ERR_SHAPE = 2
POETX_ERR_DTYPE = 3
POETX_ERR_ALIGN = 4
POETX_ERR_WORKSPACE = 5
POETX_ERR_HIP = 6
POETX_ERR_ALIAS = 7

POETX_F32 = 0
POETX_BF16 = 1

POETX_ABI_VERSION = 7
POETX_RECOMPUTE_Z = 1
POETX_CAYLEY_NEUMANN = 2
POETX_SAVED_Y = 4

EXPORTS = (
    "poetx_abi_version", "poetx_status_string", "poetx_num_blocks", "poetx_theta_count",
    "poetx_build_workspace_size", "poetx_build_orthogonal", "poetx_build_cnp_workspace_size",
    "poetx_build_cnp", "poetx_fold_weight", "poetx_quantize_weight", "poetx_fwd_workspace_size",
    "poetx_bwd_workspace_size", "poetx_linear_fwd", "poetx_linear_fwd_noalloc", "poetx_linear_bwd",
    "poetx_event_create", "poetx_event_destroy", "poetx_event_record",
    "poetx_event_synchronize", "poetx_event_elapsed_ms",
)


class PoetxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class LinearDesc(ctypes.Structure):
    _fields_ = [
        ("tokens", ctypes.c_int64),
        ("d_in", ctypes.c_int64),
        ("d_out", ctypes.c_int64),
        ("b_in", ctypes.c_int32),
        ("b_out", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("n_events", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("events", ctypes.POINTER(ctypes.c_void_p)),
        ("perm_in", ctypes.c_void_p),
        ("perm_out", ctypes.c_void_p),
        ("w_scale", ctypes.c_void_p),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m orthogonal_equivalence_amd.build` "
            "(the POET-X path has no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    dp = ctypes.POINTER(LinearDesc)
    sig = {
        "poetx_abi_version": (ctypes.c_int, []),
        "poetx_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "poetx_num_blocks": (i64, [i64, i32]),
        "poetx_theta_count": (i64, [i64, i32]),
        "poetx_build_workspace_size": (sz, [i64, i32]),
        "poetx_build_orthogonal": (ctypes.c_int, [vp, i64, i32, vp, vp, i32, vp, sz, vp]),
        "poetx_build_cnp_workspace_size": (sz, [i64, i32]),
        "poetx_build_cnp": (ctypes.c_int, [vp, i64, i32, vp, vp, vp, i32, vp, sz, vp]),
        "poetx_fold_weight": (ctypes.c_int, [vp, i64, i64, vp, vp, i32, vp, vp]),
        "poetx_quantize_weight": (ctypes.c_int, [vp, i64, i64, i32, vp, vp, vp]),
        "poetx_fwd_workspace_size": (sz, [dp]),
        "poetx_bwd_workspace_size": (sz, [dp]),
        "poetx_linear_fwd": (ctypes.c_int, [dp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "poetx_linear_fwd_noalloc": (ctypes.c_int, [dp, vp, vp, vp, vp, vp, vp, vp]),
        "poetx_linear_bwd": (ctypes.c_int, [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "poetx_event_create": (ctypes.c_int, [ctypes.POINTER(vp)]),
        "poetx_event_destroy": (ctypes.c_int, [vp]),
        "poetx_event_record": (ctypes.c_int, [vp, vp]),
        "poetx_event_synchronize": (ctypes.c_int, [vp]),
        "poetx_event_elapsed_ms": (ctypes.c_int, [vp, vp, ctypes.POINTER(ctypes.c_float)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _ptr(t):
    """Device address of a tensor (or a raw int address, or None for NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t or None
    if not t.is_contiguous():
        raise ValueError("libpoetx takes contiguous tensors")
    return t.data_ptr() or None


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != POETX_OK:
        raise PoetxError(status, where)


def _nbytes(t):
    return 0 if t is None or isinstance(t, int) else t.numel() * t.element_size()


def status_string(status: int) -> str:
    return _lib.poetx_status_string(status).decode()


def poetx_abi_version() -> int:
    return _lib.poetx_abi_version()


def poetx_num_blocks(d: int, b: int) -> int:
    return _lib.poetx_num_blocks(d, b)


def poetx_theta_count(d: int, b: int) -> int:
    return _lib.poetx_theta_count(d, b)


def poetx_build_workspace_size(d: int, b: int) -> int:
    return _lib.poetx_build_workspace_size(d, b)


def poetx_build_cnp_workspace_size(d: int, b: int) -> int:
    return _lib.poetx_build_cnp_workspace_size(d, b)


def make_desc(tokens, d_in, d_out, b_in, b_out, act, events=None, flags=0, perm_in=None,
              perm_out=None, w_scale=None) -> LinearDesc:
    desc = LinearDesc(tokens, d_in, d_out, b_in, b_out, act, 0, flags, 0, None,
                      _ptr(perm_in), _ptr(perm_out), _ptr(w_scale))
    if events:
        arr = (ctypes.c_void_p * len(events))(*events)
        desc.n_events = len(events)
        desc.events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        desc._events_keepalive = arr
    return desc


def poetx_fwd_workspace_size(desc: LinearDesc) -> int:
    return _lib.poetx_fwd_workspace_size(ctypes.byref(desc))


def poetx_bwd_workspace_size(desc: LinearDesc) -> int:
    return _lib.poetx_bwd_workspace_size(ctypes.byref(desc))


def poetx_build_orthogonal(theta, d, b, blocks_f32, blocks_act, act, ws, stream=None, raw=False):
    st = _lib.poetx_build_orthogonal(_ptr(theta), d, b, _ptr(blocks_f32), _ptr(blocks_act), act,
                                     _ptr(ws), _nbytes(ws), _stream(stream))
    if raw:
        return st
    _check(st, "poetx_build_orthogonal")


def poetx_build_cnp(theta, d, b, q_f32, blocks_f32, blocks_act, act, ws, stream=None, raw=False):
    st = _lib.poetx_build_cnp(_ptr(theta), d, b, _ptr(q_f32), _ptr(blocks_f32), _ptr(blocks_act),
                              act, _ptr(ws), _nbytes(ws), _stream(stream))
    if raw:
        return st
    _check(st, "poetx_build_cnp")


def poetx_fold_weight(W0, d_out, d_in, perm_out, perm_in, act, W0_folded, stream=None, raw=False):
    st = _lib.poetx_fold_weight(_ptr(W0), d_out, d_in, _ptr(perm_out), _ptr(perm_in), act,
                                _ptr(W0_folded), _stream(stream))
    if raw:
        return st
    _check(st, "poetx_fold_weight")


def poetx_quantize_weight(W0, d_out, d_in, act, q, scale, stream=None, raw=False):
    st = _lib.poetx_quantize_weight(_ptr(W0), d_out, d_in, act, _ptr(q), _ptr(scale),
                                    _stream(stream))
    if raw:
        return st
    _check(st, "poetx_quantize_weight")


def poetx_linear_fwd(desc, x, W0, R_act, P_act, y, z_save, ws, stream=None, raw=False):
    st = _lib.poetx_linear_fwd(ctypes.byref(desc), _ptr(x), _ptr(W0), _ptr(R_act), _ptr(P_act),
                               _ptr(y), _ptr(z_save), _ptr(ws), _nbytes(ws), _stream(stream))
    if raw:
        return st
    _check(st, "poetx_linear_fwd")


POETX_NOALLOC_SCRATCH_BYTES = 64 << 20


def poetx_linear_fwd_noalloc(desc, x, W0, R_act, P_act, y, z_save, stream=None, raw=False):
    st = _lib.poetx_linear_fwd_noalloc(ctypes.byref(desc), _ptr(x), _ptr(W0), _ptr(R_act),
                                       _ptr(P_act), _ptr(y), _ptr(z_save), _stream(stream))
    if raw:
        return st
    _check(st, "poetx_linear_fwd_noalloc")


def poetx_linear_bwd(desc, g_y, x, W0, R_f32, P_f32, R_act, P_act, z_saved, g_x, g_theta_R,
                     g_theta_P, ws, stream=None, raw=False):
    st = _lib.poetx_linear_bwd(ctypes.byref(desc), _ptr(g_y), _ptr(x), _ptr(W0), _ptr(R_f32),
                               _ptr(P_f32), _ptr(R_act), _ptr(P_act), _ptr(z_saved), _ptr(g_x),
                               _ptr(g_theta_R), _ptr(g_theta_P), _ptr(ws), _nbytes(ws),
                               _stream(stream))
    if raw:
        return st
    _check(st, "poetx_linear_bwd")


class Event:
    """A hipEvent_t owned through the library's event helpers."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(_lib.poetx_event_create(ctypes.byref(h)), "poetx_event_create")
        self.handle = h.value

    def record(self, stream=None):
        _check(_lib.poetx_event_record(self.handle, _stream(stream)), "poetx_event_record")

    def synchronize(self):
        _check(_lib.poetx_event_synchronize(self.handle), "poetx_event_synchronize")

    def elapsed_ms(self, end: "Event") -> float:
        ms = ctypes.c_float()
        _check(_lib.poetx_event_elapsed_ms(self.handle, end.handle, ctypes.byref(ms)),
               "poetx_event_elapsed_ms")
        return ms.value

    def __del__(self):
        if getattr(self, "handle", None):
            _lib.poetx_event_destroy(self.handle)
            self.handle = None
