"""Helpers for the GPU parity tests: upload seeded layers to the device and
run the library's entry points through the C ABI (via the ctypes binding)."""
from __future__ import annotations

import numpy as np
import torch

import bit_expert_ffn_moe_amd as moe
from route_check import check_selection

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


def check_gpu_selection(orc, x, wr, k, ids_g, w_g, exact=False, what=""):
    """The GPU's expert ids must be a valid top-k of the oracle's logits
    (route_check: equal to the oracle's, or differing only between logits
    within the near-tie band), bit-exact when `exact`; its weights must match
    the oracle's renormalised sigmoids of the GPU's own ids to 1e-5.
    Returns (oracle ids, number of tokens whose ids differ)."""
    z = orc.router_logits(x, wr)
    ids_ref, _ = orc.topk(z, k)
    valid, sub = check_selection(ids_g, z, ids_ref)
    n_sub = int(sub.sum())
    print(f"routing {what}: {ids_g.shape[0]} tokens, {n_sub} near-tie substitutions", flush=True)
    assert valid.all(), np.nonzero(~valid)[0][:8]
    if exact:
        assert n_sub == 0
    w_ref = orc.topk_weights(z, ids_g)
    assert np.allclose(w_g, w_ref, rtol=1e-5, atol=0, equal_nan=True)
    return ids_ref, n_sub


def gpu_routing(D, T):
    """ids and weights the last dsv4_moe_forward's router left in D's workspace."""
    ip, wp = moe.moe_debug_routing(D.w, T, D.wl.k, D.ws, D.ws_bytes)
    return d2h(ip, (T, D.wl.k), np.int32), d2h(wp, (T, D.wl.k), np.float32)


def routed_reference(orc, W, L, ids_g=None, w_g=None, tok=None, threads=0):
    """Oracle output of tokens `tok` (all when None).  With drawn routing
    the oracle takes it as well.  With the router on x, the GPU's selection
    ids_g / w_g [T][k] (read back from the workspace, or from moe_route) is
    first checked against the oracle's logits; the oracle's layer then runs
    its own router, except on tokens where the GPU chose differently inside
    the near-tie band: those take the GPU's ids with the oracle's weights of
    them."""
    k = L.wl.k
    if L.ids is not None:
        return orc.forward(W, L.wr, L.x, k, ids=L.ids, w=L.w, tokens=tok, threads=threads)
    T = L.x.shape[0]
    sel = np.arange(T) if tok is None else np.asarray(tok)
    ids_ref, _ = check_gpu_selection(orc, L.x[sel], L.wr, k, ids_g[sel], w_g[sel],
                                     what=f"T={T}")
    ref = orc.forward(W, L.wr, L.x, k, tokens=tok, threads=threads)
    diff = np.nonzero((ids_g[sel] != ids_ref).any(axis=1))[0]
    if diff.size:
        z = orc.router_logits(L.x[sel[diff]], L.wr)
        ids_all = np.zeros((T, k), np.int32)
        w_all = np.zeros((T, k), np.float32)
        ids_all[sel[diff]] = ids_g[sel[diff]]
        w_all[sel[diff]] = orc.topk_weights(z, ids_g[sel[diff]]).astype(np.float32)
        ref[diff] = orc.forward(W, L.wr, L.x, k, ids=ids_all, w=w_all,
                                tokens=sel[diff].astype(np.int32), threads=threads)
    return ref


def grouped_gemm_tile(T, k, E):
    """Tokens per M-tile of the grouped GEMM for this shape: the tile size
    the library's launcher picks from the routed rows per expert (256 from
    128 rows per expert on average, 128 from 32, else 64)."""
    rows = T * k
    return 256 if rows >= 128 * E else 128 if rows >= 32 * E else 64


def tile_cover_tokens(orc, ids, E, TM):
    """A small set of tokens whose rows touch every (group, M-tile) work item
    of the grouped GEMM (groups in the stable counting-sort order, the shared
    group E holding every token, M-tiles of TM rows) and include the last
    row of every partly filled tile: those last rows first, then greedily the
    token that covers the most work items still uncovered."""
    T, k = ids.shape
    offsets, row_token, row_of, _ = orc.permute(ids, E)
    grp = np.searchsorted(offsets, np.arange(offsets[-1]), side="right") - 1
    tile_base = np.zeros(E + 2, np.int64)
    n_tiles = (np.diff(offsets) + TM - 1) // TM
    tile_base[1:] = np.cumsum(n_tiles)
    tile_of_row = tile_base[grp] + (np.arange(offsets[-1]) - offsets[grp]) // TM
    cover = np.where(row_of >= 0, tile_of_row[np.maximum(row_of, 0)], -1)   # [T][k+1]
    uncovered = np.ones(int(tile_base[-1]), bool)
    pick = set()
    for g in range(E + 1):
        n = offsets[g + 1] - offsets[g]
        if n % TM:
            pick.add(int(row_token[offsets[g + 1] - 1]))
    for t in pick:
        uncovered[cover[t][cover[t] >= 0]] = False
    while uncovered.any():
        score = np.where(cover >= 0, uncovered[np.maximum(cover, 0)], False).sum(axis=1)
        t = int(np.argmax(score))
        pick.add(t)
        uncovered[cover[t][cover[t] >= 0]] = False
    return np.array(sorted(pick), np.int32)
