"""An independent, dense reference of the MoE FFN layer, used only to pin the
oracle.  It shares nothing with the oracle's C code: element values come from
the golden tables (the OCP format specifications) or from PyTorch's
float8_e4m3fn conversions, every matrix is expanded to dense float64 first,
and products are numpy matmuls -- a deliberately different path.
"""
from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_table(name, hexkey=False):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            out[int(k, 16) if hexkey else int(k)] = float(v)
    return out


E2M1 = _read_table("e2m1_values.txt")
E2M1_ARR = np.array([E2M1[c] for c in range(16)], np.float64)
# code 8 is negative zero
E2M1_ARR[8] = -0.0
# all 256 E4M3 values from the library's own decode
E4M3_ARR = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b).astype(np.uint32) << 16).view(np.float32)


def dense_fp4(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """[rows][cols/2] packed codes + [rows][cols/32] UE8M0 -> dense float64."""
    rows = q.shape[0]
    lo = (q & 0xF).astype(np.int64)
    hi = (q >> 4).astype(np.int64)
    codes = np.stack([lo, hi], axis=-1).reshape(rows, -1)
    vals = E2M1_ARR[codes]
    scale = np.exp2(s.astype(np.float64) - 127.0)
    return vals * np.repeat(scale, 32, axis=1)


def dense_fp8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """[rows][cols] E4M3 codes + [rows/128][cols/128] fp32 -> dense float64."""
    vals = E4M3_ARR[q.astype(np.int64)]
    sc = np.repeat(np.repeat(s.astype(np.float64), 128, axis=0), 128, axis=1)
    return vals * sc


def quant_torch(x: np.ndarray):
    """E4M3 per 128 with s = fl32(amax / 448), codes from torch's conversion."""
    x = np.ascontiguousarray(x, np.float32)
    rows, cols = x.shape
    b = x.reshape(rows, cols // 128, 128)
    amax = np.abs(b).max(axis=2)
    s = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    t = (b / safe[:, :, None]).astype(np.float32)
    q = torch.from_numpy(np.ascontiguousarray(t)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    q = np.where((s > 0)[:, :, None], q, np.uint8(0)).astype(np.uint8)
    return q.reshape(rows, cols), s


def dequant_act(q, s):
    rows, cols = q.shape
    v = E4M3_ARR[q.astype(np.int64)].reshape(rows, cols // 128, 128)
    return (v * s.astype(np.float64)[:, :, None]).reshape(rows, cols)


def dense_expert(layer, e):
    if layer.wl.fmt == "fp4":
        f = dense_fp4
    else:
        f = dense_fp8
    return f(layer.gate_q[e], layer.gate_s[e]), f(layer.up_q[e], layer.up_s[e]), \
        f(layer.down_q[e], layer.down_s[e])


def route_fp64(x_bf16, wr_bf16, k):
    z = bf16_to_f32(x_bf16).astype(np.float64) @ bf16_to_f32(wr_bf16).astype(np.float64)
    ids = np.argsort(-z, axis=1, kind="stable")[:, :k].astype(np.int32)
    zs = np.take_along_axis(z, ids, axis=1)
    sg = 1.0 / (1.0 + np.exp(-zs))
    return ids, sg / sg.sum(axis=1, keepdims=True), z


def forward(layer, ids, w):
    """out[t] = FFN_shared(x_t) + sum_j w_j FFN_{ids_j}(x_t), dense float64."""
    wl = layer.wl
    x = bf16_to_f32(layer.x)
    xq, xs = quant_torch(x)
    xd = dequant_act(xq, xs)
    T = x.shape[0]
    out = np.zeros((T, wl.H), np.float64)
    cache = {}

    def ffn(e, rows):
        if e not in cache:
            cache[e] = dense_expert(layer, e)
        G, U, D = cache[e]
        g = xd[rows] @ G.T
        u = xd[rows] @ U.T
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
        hq, hs = quant_torch(h)
        return dequant_act(hq, hs) @ D.T

    out += ffn(wl.E, np.arange(T))
    for t in range(T):
        for j in range(ids.shape[1]):
            out[t] += float(w[t, j]) * ffn(int(ids[t, j]), np.array([t]))[0]
    return out
