"""Seeded synthetic inputs for the routed-expert MoE FFN layer.

The shapes, formats and value distributions follow the workload definitions
that accompany the pages (hidden 4096, expert intermediate 2048, 256 routed
experts top-6 plus one shared expert; FP4 E2M1 codes uniform over the 16
values with UE8M0 scale exponents uniform in [-8, -4]; bf16 activations
~N(0,1); bf16 router ~N(0,0.02); an FP8-weight variant whose weights are
~N(0,0.02) quantised per 128x128 block).  No page publishes a dataset or
weights for this layer, so these seeded tensors stand in for all of them.

This module holds no arithmetic of the layer itself: it draws random numbers
(``synth.c``) and, for the FP8-weight variant only, turns drawn fp32 weights
into E4M3 codes with PyTorch's own ``float8_e4m3fn`` conversion -- input
preparation done by a library routine that neither the oracle nor the GPU
library uses.

Streams: 1 x, 2 router, 3/4 gate codes/scales (3 = gate values for FP8),
5/6 up, 7/8 down, 9 routing Gumbel draws, 10 routing weights, 11 rank
permutation.
"""
from __future__ import annotations

import ctypes
import dataclasses
import functools
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")


def build() -> str:
    """Compile synth.c into libsynth.so (gcc, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           os.path.join(_HERE, "synth.c"), "-o", _SO, "-lm"]
    subprocess.run(cmd, check=True)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        u64, i64, u32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_uint32
        vp = ctypes.c_void_p
        lib.synth_bytes.argtypes = [u64, u64, u64, i64, u32, u32, vp]
        lib.synth_normal_f32.argtypes = [u64, u64, u64, i64, ctypes.c_double, vp]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, i64, ctypes.c_double, vp]
        lib.synth_uniform.argtypes = [u64, u64, u64, i64, vp]
        lib.synth_draw.argtypes = [u64, u64, u64]
        lib.synth_draw.restype = u64
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def bytes_uniform(seed, stream, shape, lo, span, offset=0) -> np.ndarray:
    out = np.empty(shape, np.uint8)
    _load().synth_bytes(seed, stream, offset, out.size, lo, span, _ptr(out))
    return out


def normal_f32(seed, stream, shape, sigma, offset=0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _load().synth_normal_f32(seed, stream, offset, out.size, sigma, _ptr(out))
    return out


def normal_bf16(seed, stream, shape, sigma, offset=0) -> np.ndarray:
    out = np.empty(shape, np.uint16)
    _load().synth_normal_bf16(seed, stream, offset, out.size, sigma, _ptr(out))
    return out


def uniform(seed, stream, shape, offset=0) -> np.ndarray:
    out = np.empty(shape, np.float64)
    _load().synth_uniform(seed, stream, offset, out.size, _ptr(out))
    return out


def permutation(seed, stream, n) -> np.ndarray:
    """Fisher-Yates shuffle of 0..n-1 driven by the counter stream."""
    u = uniform(seed, stream, (n,))
    p = np.arange(n, dtype=np.int32)
    for i in range(n - 1, 0, -1):
        j = int(u[i] * (i + 1))
        p[i], p[j] = p[j], p[i]
    return p


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    fmt: str            # "fp4" (E2M1 + UE8M0/32) or "fp8" (E4M3 + fp32 per 128x128)
    routing: str        # "router" (router on x) or "zipf" (drawn, injected)
    zipf_s: float = 0.0
    seed: int = 0


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_t8", 8, 256, 128, 8, 2, "fp4", "router", seed=1000),
        Workload("decode_t1", 1, 4096, 2048, 256, 6, "fp4", "router", seed=1001),
        Workload("verify_t32", 32, 4096, 2048, 256, 6, "fp4", "zipf", 1.0, seed=1002),
        Workload("prefill_fp4_t4096", 4096, 4096, 2048, 256, 6, "fp4", "zipf", 1.2, seed=1003),
        Workload("prefill_fp8_t8192", 8192, 4096, 2048, 256, 6, "fp8", "router", seed=1004),
    ]
}


@dataclasses.dataclass
class Layer:
    wl: Workload
    x: np.ndarray          # [T][H] uint16 (bf16 bits)
    wr: np.ndarray         # [H][E] uint16 (bf16 bits)
    gate_q: np.ndarray
    gate_s: np.ndarray
    up_q: np.ndarray
    up_s: np.ndarray
    down_q: np.ndarray
    down_s: np.ndarray
    ids: np.ndarray | None  # [T][k] int32 when routing is injected
    w: np.ndarray | None    # [T][k] float32 when routing is injected


def _fp4_matrix(seed, stream_q, stream_s, n_exp, rows, cols):
    q = bytes_uniform(seed, stream_q, (n_exp, rows, cols // 2), 0, 256)
    s = bytes_uniform(seed, stream_s, (n_exp, rows, cols // 32), 119, 5)
    return q, s


def _fp8_matrix(seed, stream, n_exp, rows, cols, sigma=0.02):
    """~N(0, sigma) weights, one fp32 scale per 128x128 block = amax / 448,
    codes = torch's float8_e4m3fn conversion of w / scale (torch on the CPU
    for the block maxima and the fp32 division too, for its threads)."""
    import torch
    q = np.empty((n_exp, rows, cols), np.uint8)
    s = np.empty((n_exp, rows // 128, cols // 128), np.float32)
    per = rows * cols
    for e in range(n_exp):
        w = torch.from_numpy(normal_f32(seed, stream, (rows, cols), sigma, offset=e * per))
        blk = w.view(rows // 128, 128, cols // 128, 128)
        sc = blk.abs().amax(dim=(1, 3)) / 448.0
        s[e] = sc.numpy()
        safe = torch.where(sc > 0, sc, torch.ones_like(sc))
        scaled = (blk / safe[:, None, :, None]).reshape(rows, cols)
        q[e] = scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, s


@functools.lru_cache(maxsize=2)
def _weights(fmt, seed, E, H, I):
    """The stacked expert weights of a layer; they depend on neither T, k
    nor the routing, so layers of one (fmt, seed, E, H, I) share them (the
    caller must not modify them)."""
    if fmt == "fp4":
        gq, gs = _fp4_matrix(seed, 3, 4, E + 1, I, H)
        uq, us = _fp4_matrix(seed, 5, 6, E + 1, I, H)
        dq, ds = _fp4_matrix(seed, 7, 8, E + 1, H, I)
    elif fmt == "fp8":
        gq, gs = _fp8_matrix(seed, 3, E + 1, I, H)
        uq, us = _fp8_matrix(seed, 5, E + 1, I, H)
        dq, ds = _fp8_matrix(seed, 7, E + 1, H, I)
    else:
        raise ValueError(fmt)
    return gq, gs, uq, us, dq, ds


def zipf_routing(seed, T, E, k, s):
    """Plackett-Luce draw of k distinct experts per token with weight
    proportional to rank^-s (Gumbel-top-k), rank -> id by a seeded
    permutation; gate weights drawn uniform in [0.2, 1], sorted descending,
    normalised to sum 1."""
    g = uniform(seed, 9, (T, E))
    ranks = np.arange(1, E + 1, dtype=np.float64)
    keys = -s * np.log(ranks)[None, :] - np.log(-np.log(g))
    order = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    perm = permutation(seed, 11, E)
    ids = perm[order].astype(np.int32)
    v = 0.2 + 0.8 * uniform(seed, 10, (T, k))
    v = -np.sort(-v, axis=1)
    w = (v / v.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(w)


def make_layer(wl: Workload | str, **over) -> Layer:
    """Build a layer's inputs.  ``over`` may change T, H, I, E, k, seed,
    fmt, routing or zipf_s (parity tests use smaller shapes)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    wl = dataclasses.replace(wl, **over) if over else wl
    T, H, I, E, k, seed = wl.T, wl.H, wl.I, wl.E, wl.k, wl.seed
    x = normal_bf16(seed, 1, (T, H), 1.0)
    wr = normal_bf16(seed, 2, (H, E), 0.02)
    gq, gs, uq, us, dq, ds = _weights(wl.fmt, seed, E, H, I)
    ids = w = None
    if wl.routing == "zipf":
        ids, w = zipf_routing(seed, T, E, k, wl.zipf_s)
    return Layer(wl, x, wr, gq, gs, uq, us, dq, ds, ids, w)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)
