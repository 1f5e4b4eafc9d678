"""Helpers for the GPU parity tests: upload seeded layers to the device and
run the library's entry points through the C ABI (via the ctypes binding)."""
from __future__ import annotations

import numpy as np
import torch

import bit_expert_ffn_moe_amd as moe

DEV = "cuda:0"


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


class DevLayer:
    """A synth.Layer resident on the GPU, with its weight descriptor."""

    def __init__(self, layer, max_tokens=None):
        wl = layer.wl
        self.layer, self.wl = layer, wl
        self.x = to_dev(layer.x)
        self.wr = to_dev(layer.wr)
        self.t = {n: to_dev(getattr(layer, n)) for n in
                  ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")}
        fmt = moe.MOE_W_FP4_E2M1_UE8M0_K32 if wl.fmt == "fp4" else moe.MOE_W_FP8_E4M3_F32_B128
        self.w = moe.make_weights(fmt, wl.E, wl.H, wl.I, self.t["gate_q"], self.t["gate_s"],
                                  self.t["up_q"], self.t["up_s"], self.t["down_q"],
                                  self.t["down_s"])
        self.ids = to_dev(layer.ids) if layer.ids is not None else None
        self.rw = to_dev(layer.w) if layer.w is not None else None
        self.max_tokens = max_tokens or wl.T
        self.ws_bytes = moe.moe_workspace_bytes(self.w, self.max_tokens, wl.k)
        assert self.ws_bytes > 0
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=DEV)
        moe.moe_workspace_init(self.ws, self.ws_bytes)

    def forward(self, x=None, T=None, out_dtype=moe.MOE_DT_F32, ids=None, rw=None,
                injected=True):
        wl = self.wl
        x = self.x if x is None else x
        T = x.shape[0] if T is None else T
        if ids is None and injected and self.ids is not None:
            ids, rw = self.ids[:T], self.rw[:T]
        dt = torch.float32 if out_dtype == moe.MOE_DT_F32 else torch.uint16
        out = torch.empty((T, wl.H), dtype=dt, device=DEV)
        moe.dsv4_moe_forward(self.w, self.wr, x, T, wl.k, ids, rw, out, out_dtype, self.ws,
                             self.ws_bytes)
        return out


_hip = None


def d2h(ptr: int, shape, dtype) -> np.ndarray:
    """Copy a device buffer (raw address) to a new host array with hipMemcpy."""
    import ctypes
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch loaded
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    torch.cuda.synchronize()
    out = np.empty(shape, dtype)
    rc = _hip.hipMemcpy(out.ctypes.data, ptr, out.nbytes, 2)  # 2 = device to host
    assert rc == 0, rc
    return out


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even) -- computed
    exactly: go through float32 only when that cannot double-round, i.e. by
    rounding the float64 significand directly."""
    v = np.asarray(v, np.float64)
    m, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= |m| < 1
    scaled = np.ldexp(m, 8)                  # 8 significant bits of bf16
    r = np.round(scaled)                     # numpy rounds half to even
    out = np.ldexp(r, e - 8).astype(np.float32)  # exact: r has <= 9 bits
    return (out.view(np.uint32) >> 16).astype(np.uint16)
