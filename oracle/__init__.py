"""ctypes wrapper of the plain C oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the GPU library and its
Python binding never do.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
# a build of the oracle to load instead (the pins' mutation test points this
# at copies of moe_oracle.c with a planted mistake)
_SO_OVERRIDE = os.environ.get("BEF_ORACLE_LIB")
FMT_FP4, FMT_FP8 = 1, 2


def build(compiler: str = "gcc", out: str | None = None, extra=(), src: str | None = None) -> str:
    """Compile moe_oracle.c (C99, -O2, no fast-math, no FP contraction)."""
    out = out or _SO
    src = src or os.path.join(_HERE, "moe_oracle.c")
    cmd = [compiler, "-O2", "-std=c99", "-Wall", "-Wextra", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", f"-I{_HERE}", *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class _W(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("E", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32), ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p),
                ("down_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


_lib = None


def _load(path: str | None = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if _SO_OVERRIDE:
            _lib = _bind(ctypes.CDLL(_SO_OVERRIDE))
            return _lib
        if not os.path.exists(_SO):
            build()
        _lib = _bind(ctypes.CDLL(_SO))
    return _lib


def _bind(lib):
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.orc_e2m1_value.argtypes = [ctypes.c_uint]
    lib.orc_e2m1_value.restype = ctypes.c_double
    lib.orc_ue8m0_value.argtypes = [ctypes.c_uint]
    lib.orc_ue8m0_value.restype = ctypes.c_double
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_value.restype = ctypes.c_double
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode.restype = ctypes.c_uint
    lib.orc_e4m3_encode_n.argtypes = [vp, i64, vp]
    lib.orc_act_quant_f32.argtypes = [vp, i64, i32, vp, vp]
    lib.orc_act_quant_bf16.argtypes = [vp, i64, i32, vp, vp]
    lib.orc_router_logits.argtypes = [vp, vp, i32, i32, i32, vp]
    lib.orc_topk.argtypes = [vp, i32, i32, i32, vp, vp]
    lib.orc_topk_weights.argtypes = [vp, i32, i32, i32, vp, vp]
    lib.orc_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.orc_permute.restype = ctypes.c_int
    lib.orc_weight.argtypes = [ctypes.POINTER(_W), ctypes.c_int, i32, i32, i32]
    lib.orc_weight.restype = ctypes.c_double
    lib.orc_gate_up.argtypes = [ctypes.POINTER(_W), i32, vp, vp, vp, vp]
    lib.orc_swiglu.argtypes = [vp, vp, i32, vp]
    lib.orc_down.argtypes = [ctypes.POINTER(_W), i32, vp, vp, vp]
    lib.orc_expert_row.argtypes = [ctypes.POINTER(_W), i32, vp, vp, vp, vp, vp, vp]
    lib.orc_moe_forward.argtypes = [ctypes.POINTER(_W), vp, vp, i32, i32, vp, vp, vp, i32, vp,
                                    i32]
    lib.orc_moe_forward.restype = ctypes.c_int
    return lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


class Weights:
    """Holds numpy weight arrays and the C descriptor pointing at them."""

    def __init__(self, fmt, E, H, I, gate_q, gate_s, up_q, up_s, down_q, down_s):
        self.arrays = [np.ascontiguousarray(a) for a in (gate_q, gate_s, up_q, up_s, down_q, down_s)]
        gq, gs, uq, us, dq, ds = self.arrays
        self.fmt, self.E, self.H, self.I = fmt, E, H, I
        self.c = _W(fmt, E, H, I, _p(gq), _p(uq), _p(dq), _p(gs), _p(us), _p(ds))

    @classmethod
    def from_layer(cls, layer):
        wl = layer.wl
        fmt = FMT_FP4 if wl.fmt == "fp4" else FMT_FP8
        return cls(fmt, wl.E, wl.H, wl.I, layer.gate_q, layer.gate_s, layer.up_q, layer.up_s,
                   layer.down_q, layer.down_s)


class Oracle:
    def __init__(self, so_path: str | None = None):
        self.lib = _load(so_path)

    # ---- codecs --------------------------------------------------------
    def e2m1(self, c):
        return self.lib.orc_e2m1_value(c)

    def ue8m0(self, b):
        return self.lib.orc_ue8m0_value(b)

    def e4m3(self, b):
        return self.lib.orc_e4m3_value(b)

    def e4m3_table(self):
        return np.array([self.e4m3(b) for b in range(256)], np.float64)

    def e4m3_encode(self, v: np.ndarray) -> np.ndarray:
        v = np.ascontiguousarray(v, np.float32)
        out = np.empty(v.shape, np.uint8)
        self.lib.orc_e4m3_encode_n(_p(v), v.size, _p(out))
        return out

    # ---- S3 ------------------------------------------------------------
    def act_quant(self, x: np.ndarray):
        """x: [rows][cols] float32 or uint16 (bf16 bits)."""
        x = np.ascontiguousarray(x)
        rows, cols = x.shape
        q = np.empty((rows, cols), np.uint8)
        s = np.empty((rows, cols // 128), np.float32)
        if x.dtype == np.float32:
            self.lib.orc_act_quant_f32(_p(x), rows, cols, _p(q), _p(s))
        elif x.dtype == np.uint16:
            self.lib.orc_act_quant_bf16(_p(x), rows, cols, _p(q), _p(s))
        else:
            raise TypeError(x.dtype)
        return q, s

    # ---- S1/S2 ---------------------------------------------------------
    def router_logits(self, x, wr):
        x, wr = np.ascontiguousarray(x, np.uint16), np.ascontiguousarray(wr, np.uint16)
        T, H = x.shape
        E = wr.shape[1]
        z = np.empty((T, E), np.float32)
        self.lib.orc_router_logits(_p(x), _p(wr), T, H, E, _p(z))
        return z

    def topk(self, z, k):
        z = np.ascontiguousarray(z, np.float32)
        T, E = z.shape
        ids = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float64)
        self.lib.orc_topk(_p(z), T, E, k, _p(ids), _p(w))
        return ids, w

    def topk_weights(self, z, ids):
        """Renormalised sigmoid weights of a given selection ids [T][k]."""
        z = np.ascontiguousarray(z, np.float32)
        ids = np.ascontiguousarray(ids, np.int32)
        T, E = z.shape
        k = ids.shape[1]
        assert ids.min() >= 0 and ids.max() < E
        w = np.empty((T, k), np.float64)
        self.lib.orc_topk_weights(_p(z), T, E, k, _p(ids), _p(w))
        return w

    def route(self, x, wr, k):
        return self.topk(self.router_logits(x, wr), k)

    # ---- S4 ------------------------------------------------------------
    def permute(self, ids, E):
        ids = np.ascontiguousarray(ids, np.int32)
        T, k = ids.shape
        offsets = np.empty(E + 2, np.int32)
        row_token = np.full(T * k + T, -1, np.int32)
        row_of = np.empty((T, k + 1), np.int32)
        dropped = self.lib.orc_permute(_p(ids), T, k, E, _p(offsets), _p(row_token), _p(row_of))
        return offsets, row_token, row_of, dropped

    # ---- S5/S6 ---------------------------------------------------------
    def weight(self, W: Weights, mat, e, row, col):
        return self.lib.orc_weight(ctypes.byref(W.c), mat, e, row, col)

    def gate_up(self, W: Weights, e, xq, xs):
        xq, xs = np.ascontiguousarray(xq, np.uint8), np.ascontiguousarray(xs, np.float32)
        g = np.empty(W.I, np.float64)
        u = np.empty(W.I, np.float64)
        self.lib.orc_gate_up(ctypes.byref(W.c), e, _p(xq), _p(xs), _p(g), _p(u))
        return g, u

    def swiglu(self, g, u):
        g, u = np.ascontiguousarray(g, np.float64), np.ascontiguousarray(u, np.float64)
        h = np.empty(g.shape, np.float32)
        self.lib.orc_swiglu(_p(g), _p(u), g.size, _p(h))
        return h

    def down(self, W: Weights, e, hq, hs):
        hq, hs = np.ascontiguousarray(hq, np.uint8), np.ascontiguousarray(hs, np.float32)
        y = np.empty(W.H, np.float64)
        self.lib.orc_down(ctypes.byref(W.c), e, _p(hq), _p(hs), _p(y))
        return y

    def expert_row(self, W: Weights, e, xq, xs):
        xq, xs = np.ascontiguousarray(xq, np.uint8), np.ascontiguousarray(xs, np.float32)
        h = np.empty(W.I, np.float32)
        hq = np.empty(W.I, np.uint8)
        hs = np.empty(W.I // 128, np.float32)
        y = np.empty(W.H, np.float64)
        self.lib.orc_expert_row(ctypes.byref(W.c), e, _p(xq), _p(xs), _p(h), _p(hq), _p(hs), _p(y))
        return h, hq, hs, y

    # ---- whole layer ---------------------------------------------------
    def forward(self, W: Weights, wr, x, k, ids=None, w=None, tokens=None, threads=0):
        x = np.ascontiguousarray(x, np.uint16)
        wr = np.ascontiguousarray(wr, np.uint16)
        T = x.shape[0]
        if ids is not None:
            ids = np.ascontiguousarray(ids, np.int32)
            w = np.ascontiguousarray(w, np.float32)
        tok = None if tokens is None else np.ascontiguousarray(tokens, np.int32)
        n = T if tok is None else tok.size
        out = np.empty((n, W.H), np.float64)
        rc = self.lib.orc_moe_forward(ctypes.byref(W.c), _p(wr), _p(x), T, k, _p(ids), _p(w),
                                      _p(tok), n, _p(out), threads)
        if rc != 0:
            raise ValueError("oracle: expert id out of range")
        return out
