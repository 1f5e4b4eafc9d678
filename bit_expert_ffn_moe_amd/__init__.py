"""Thin ctypes binding of libbefmoe.so, the gfx950 routed-expert MoE FFN library.

Every function has the name and argument order of its C counterpart in
include/moe.h and only marshals arguments: device buffers may be passed as
integers (device addresses) or as objects with ``data_ptr()`` (torch tensors);
``stream`` may be an integer hipStream_t, a torch stream, or None (the current
torch stream when torch is loaded, else the default stream).  A negative
status raises :class:`MoeError`.  All computation happens in the library's
HIP kernels; there is no fallback path, and importing this module fails when
the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_PKG, "libbefmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_EALIGN, MOE_EWORKSPACE, MOE_ELAUNCH = 0, -1, -2, -3, -4, -5
MOE_W_FP4_E2M1_UE8M0_K32, MOE_W_FP8_E4M3_F32_B128 = 1, 2
MOE_DT_BF16, MOE_DT_F32 = 1, 2
MOE_STATUS_BAD_EXPERT_ID, MOE_STATUS_SYNC_TIMEOUT = 1, 2
MOE_KERNEL_GEMV_GATE_UP, MOE_KERNEL_GEMM_GATE_UP, MOE_KERNEL_GEMV_DOWN, MOE_KERNEL_GEMM_DOWN = 1, 2, 3, 4
MOE_KERNEL_DECODE_FFN = 5
MOE_NOALLOC_SCRATCH_BYTES = 16 << 20

if not os.path.exists(_SO):
    raise ImportError(
        f"{_SO} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
# torch first: its HIP runtime (libamdhip64.so.7) must be the one the library
# binds to.  Loaded the other way round, torch's own libraries (which ask for
# the unversioned name) would bring in a second runtime beside ours, and
# device pointers and streams of one would be invalid in the other.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(_SO)
LIBRARY_PATH = _SO


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {moe_status_string(status)} ({status})")
        self.status = status


class moe_weights(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("gate_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("up_q", ctypes.c_void_p), ("up_s", ctypes.c_void_p),
                ("down_q", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


class moe_expert_cache(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("n_slots", ctypes.c_int32),
                ("slot_of", ctypes.c_void_p), ("expert_of", ctypes.c_void_p),
                ("last_use", ctypes.c_void_p), ("calls", ctypes.c_uint64),
                ("shared_resident", ctypes.c_int32), ("pad_", ctypes.c_int32),
                ("hits", ctypes.c_uint64), ("misses", ctypes.c_uint64),
                ("bytes_copied", ctypes.c_uint64)]


_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_W = ctypes.POINTER(moe_weights)
_C = ctypes.POINTER(moe_expert_cache)
_sigs = {
    "moe_workspace_bytes": ([_W, _i32, _i32], _sz),
    "moe_workspace_init": ([_vp, _sz, _vp], ctypes.c_int),
    "moe_route": ([_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "act_quant_fp8": ([_vp, _i32, _i64, _i32, _vp, _vp, _vp], ctypes.c_int),
    "moe_permute": ([_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe_expert_ffn": ([_W, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe_expert_gate_up": ([_W, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "moe_expert_down": ([_W, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp],
                        ctypes.c_int),
    "moe_combine": ([_vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp], ctypes.c_int),
    "dsv4_moe_forward": ([_W, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _i32, _vp, _sz, _vp],
                         ctypes.c_int),
    "dsv4_moe_forward_noalloc": ([_W, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _i32, _vp],
                                 ctypes.c_int),
    "moe_host_experts_workspace_bytes": ([_W, _i32, _i32], _sz),
    "moe_host_experts_scratch_bytes": ([_i32, _i32, _i32], _sz),
    "moe_forward_host_experts": ([_W, _W, _C, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _sz, _vp, _sz,
                                  _vp, _vp, _vp], ctypes.c_int),
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_device_status": ([_vp, _vp, ctypes.POINTER(ctypes.c_uint32), ctypes.c_int],
                          ctypes.c_int),
    "moe_debug_intermediates": ([_W, _i32, _i32, _vp, _sz, ctypes.POINTER(_vp),
                                 ctypes.POINTER(_vp), ctypes.POINTER(_vp)], ctypes.c_int),
    "moe_debug_time_kernel": ([_i32, _vp, _vp], ctypes.c_int),
    "moe_debug_set_decode_fused": ([_i32], ctypes.c_int),
    "moe_debug_store_h": ([_vp, _sz], ctypes.c_int),
    "moe_debug_stream_read": ([_vp, _sz, _vp, _i32, _vp], ctypes.c_int),
    "moe_debug_routing": ([_W, _i32, _i32, _vp, _sz, ctypes.POINTER(_vp), ctypes.POINTER(_vp)],
                          ctypes.c_int),
}
for _name, (_args, _res) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_sigs)


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(s):
    if s is None:
        import sys
        torch = sys.modules.get("torch")
        if torch is not None and torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc: int, where: str) -> int:
    if rc != MOE_OK:
        raise MoeError(rc, where)
    return rc


def make_weights(fmt, n_experts, hidden, inter, gate_q, gate_s, up_q, up_s, down_q, down_s):
    """Build the C weight descriptor from device buffers (ints or tensors).
    The returned object keeps references to tensors passed in."""
    w = moe_weights(fmt, n_experts, hidden, inter, _ptr(gate_q), _ptr(gate_s), _ptr(up_q),
                    _ptr(up_s), _ptr(down_q), _ptr(down_s))
    w._keep = (gate_q, gate_s, up_q, up_s, down_q, down_s)
    return w


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def moe_workspace_bytes(w: moe_weights, max_tokens: int, top_k: int) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(w), max_tokens, top_k)


def moe_workspace_init(ws, ws_bytes: int, stream=None) -> int:
    return _check(_lib.moe_workspace_init(_ptr(ws), ws_bytes, _stream(stream)), "moe_workspace_init")


def moe_route(x, w_router, T, H, E, k, topk_ids, topk_w, ws, ws_bytes, stream=None) -> int:
    return _check(_lib.moe_route(_ptr(x), _ptr(w_router), T, H, E, k, _ptr(topk_ids),
                                 _ptr(topk_w), _ptr(ws), ws_bytes, _stream(stream)), "moe_route")


def act_quant_fp8(x, x_dtype, rows, cols, q, scales, stream=None) -> int:
    return _check(_lib.act_quant_fp8(_ptr(x), x_dtype, rows, cols, _ptr(q), _ptr(scales),
                                     _stream(stream)), "act_quant_fp8")


def moe_permute(topk_ids, T, k, E, offsets, row_token, row_of, ws, ws_bytes, stream=None) -> int:
    return _check(_lib.moe_permute(_ptr(topk_ids), T, k, E, _ptr(offsets), _ptr(row_token),
                                   _ptr(row_of), _ptr(ws), ws_bytes, _stream(stream)),
                  "moe_permute")


def moe_expert_ffn(w, xq, xs, T, k, offsets, row_token, y_rows, ws, ws_bytes, stream=None) -> int:
    return _check(_lib.moe_expert_ffn(ctypes.byref(w), _ptr(xq), _ptr(xs), T, k, _ptr(offsets),
                                      _ptr(row_token), _ptr(y_rows), _ptr(ws), ws_bytes,
                                      _stream(stream)), "moe_expert_ffn")


def moe_expert_gate_up(w, xq, xs, T, k, offsets, row_token, ws, ws_bytes, stream=None) -> int:
    return _check(_lib.moe_expert_gate_up(ctypes.byref(w), _ptr(xq), _ptr(xs), T, k,
                                          _ptr(offsets), _ptr(row_token), _ptr(ws), ws_bytes,
                                          _stream(stream)), "moe_expert_gate_up")


def moe_expert_down(w, T, k, offsets, row_of, topk_w, y_rows, out, out_dtype, ws, ws_bytes,
                    stream=None) -> int:
    return _check(_lib.moe_expert_down(ctypes.byref(w), T, k, _ptr(offsets), _ptr(row_of),
                                       _ptr(topk_w), _ptr(y_rows), _ptr(out), out_dtype,
                                       _ptr(ws), ws_bytes, _stream(stream)), "moe_expert_down")


def moe_combine(y_rows, row_of, topk_w, T, k, H, out, out_dtype, stream=None) -> int:
    return _check(_lib.moe_combine(_ptr(y_rows), _ptr(row_of), _ptr(topk_w), T, k, H, _ptr(out),
                                   out_dtype, _stream(stream)), "moe_combine")


def dsv4_moe_forward(w, w_router, x, T, k, routing_ids, routing_w, out, out_dtype, ws, ws_bytes,
                     stream=None) -> int:
    return _check(_lib.dsv4_moe_forward(ctypes.byref(w), _ptr(w_router), _ptr(x), T, k,
                                        _ptr(routing_ids), _ptr(routing_w), _ptr(out), out_dtype,
                                        _ptr(ws), ws_bytes, _stream(stream)), "dsv4_moe_forward")


def dsv4_moe_forward_noalloc(w, w_router, x, T, k, routing_ids, routing_w, out, out_dtype,
                             stream=None) -> int:
    return _check(_lib.dsv4_moe_forward_noalloc(ctypes.byref(w), _ptr(w_router), _ptr(x), T, k,
                                                _ptr(routing_ids), _ptr(routing_w), _ptr(out),
                                                out_dtype, _stream(stream)),
                  "dsv4_moe_forward_noalloc")


class ExpertCache:
    """Host-side LRU state of one layer's expert cache (the moe_expert_cache
    of include/moe.h) in numpy arrays, in its initial (empty) state."""

    def __init__(self, n_experts: int, n_slots: int):
        import numpy as np
        self.slot_of = np.full(n_experts, -1, np.int32)
        self.expert_of = np.full(n_slots, -1, np.int32)
        self.last_use = np.zeros(n_slots, np.uint64)
        self.c = moe_expert_cache(n_experts, n_slots, self.slot_of.ctypes.data,
                                  self.expert_of.ctypes.data, self.last_use.ctypes.data,
                                  0, 0, 0, 0, 0, 0)


def moe_host_experts_workspace_bytes(host_w, max_tokens, top_k) -> int:
    return _lib.moe_host_experts_workspace_bytes(ctypes.byref(host_w), max_tokens, top_k)


def moe_host_experts_scratch_bytes(n_experts, max_tokens, top_k) -> int:
    return _lib.moe_host_experts_scratch_bytes(n_experts, max_tokens, top_k)


def moe_forward_host_experts(host_w, slot_w, cache, w_router, x, T, k, out, out_dtype, ws,
                             ws_bytes, host_scratch, host_scratch_bytes, copies_done,
                             stream=None, copy_stream=None) -> int:
    c = cache.c if isinstance(cache, ExpertCache) else cache
    return _check(_lib.moe_forward_host_experts(
        ctypes.byref(host_w), ctypes.byref(slot_w), ctypes.byref(c), _ptr(w_router), _ptr(x),
        T, k, _ptr(out), out_dtype, _ptr(ws), ws_bytes, _ptr(host_scratch), host_scratch_bytes,
        _ptr(copies_done), _stream(stream), _stream(copy_stream)), "moe_forward_host_experts")


def moe_device_status(ws, stream=None, clear: bool = False) -> int:
    st = ctypes.c_uint32(0)
    _check(_lib.moe_device_status(_ptr(ws), _stream(stream), ctypes.byref(st), int(clear)),
           "moe_device_status")
    return st.value


def moe_debug_set_decode_fused(fused) -> int:
    """1: the one-token FP4 path runs the fused expert kernel where it fits; 0: separate kernels."""
    return _check(_lib.moe_debug_set_decode_fused(int(fused)), "moe_debug_set_decode_fused")


def moe_debug_time_kernel(which, start_event, stop_event) -> int:
    """Time kernel `which` with two hipEvent_t handles (None, None clears)."""
    return _check(_lib.moe_debug_time_kernel(which, start_event, stop_event),
                  "moe_debug_time_kernel")


def moe_debug_intermediates(w, T, k, ws, ws_bytes):
    """Device addresses (h or None, hq, hs) of the intermediates in ws."""
    h, hq, hs = _vp(), _vp(), _vp()
    _check(_lib.moe_debug_intermediates(ctypes.byref(w), T, k, _ptr(ws), ws_bytes,
                                        ctypes.byref(h), ctypes.byref(hq), ctypes.byref(hs)),
           "moe_debug_intermediates")
    return h.value, hq.value, hs.value


def moe_debug_stream_read(src, nbytes, sink, blocks, stream=None):
    _check(_lib.moe_debug_stream_read(_ptr(src), nbytes, _ptr(sink), blocks, _stream(stream)),
           "moe_debug_stream_read")


def moe_debug_store_h(h, n_floats):
    """Set (or clear with None, 0) the MFMA gate+up kernels' fp32 h sink."""
    _check(_lib.moe_debug_store_h(_ptr(h) if h is not None else None, n_floats),
           "moe_debug_store_h")


def moe_debug_routing(w, T, k, ws, ws_bytes):
    """Device addresses (ids, weights) the last forward's router left in ws."""
    ids, tw = _vp(), _vp()
    _check(_lib.moe_debug_routing(ctypes.byref(w), T, k, _ptr(ws), ws_bytes, ctypes.byref(ids),
                                  ctypes.byref(tw)), "moe_debug_routing")
    return ids.value, tw.value


def raw_call(name: str, *args) -> int:
    """Call a C entry point with already-marshalled arguments and return its
    status without raising (used by tests of the error paths)."""
    return getattr(_lib, name)(*args)
