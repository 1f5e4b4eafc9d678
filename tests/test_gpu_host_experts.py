"""Routed experts resident in host memory (moe_forward_host_experts): an LRU
cache of expert slots in HBM, misses copied on a second stream and computed
on arrival.  Each call's output is checked against the oracle (with the
GPU's own selection, as for dsv4_moe_forward) and against dsv4_moe_forward
on device-resident weights; the cache's slot tables and hit / miss counts
are checked against a plain model of the same LRU policy."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import Oracle, Weights

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_expert_ffn_moe_amd as moe  # noqa: E402
from gpu_util import DevLayer, d2h, rel_l2, routed_reference, to_host  # noqa: E402

orc = Oracle()
NAMES = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")


def _hip_event():
    hip = ctypes.CDLL("libamdhip64.so.7")
    e = ctypes.c_void_p()
    assert hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(2)) == 0  # no timing
    return e.value


class LruModel:
    """The cache policy written out plainly: hits keep their slots; each
    miss (in order of first appearance in the call's ids) takes the slot
    with the smallest last use among those no expert of this call needs."""

    def __init__(self, E, NS):
        self.slot_of = np.full(E, -1)
        self.expert_of = np.full(NS, -1)
        self.last = np.zeros(NS, np.int64)
        self.calls = self.hits = self.misses = 0

    def call(self, ids):
        self.calls += 1
        now = self.calls
        for e in ids.ravel():
            s = self.slot_of[e]
            if s >= 0 and self.last[s] != now:
                self.last[s] = now
                self.hits += 1
        for e in ids.ravel():
            if self.slot_of[e] >= 0:
                continue
            cand = [s for s in range(len(self.last)) if self.last[s] != now]
            v = min(cand, key=lambda s: (self.last[s], s))
            if self.expert_of[v] >= 0:
                self.slot_of[self.expert_of[v]] = -1
            self.expert_of[v] = e
            self.slot_of[e] = v
            self.last[v] = now
            self.misses += 1


class HostLayer:
    def __init__(self, L, n_slots, max_tokens):
        wl = L.wl
        self.L, self.wl, self.NS = L, wl, n_slots
        self.D = DevLayer(L, max_tokens=max_tokens)      # device-resident reference layer
        fmt = self.D.w.format
        self.host = {n: torch.from_numpy(np.ascontiguousarray(getattr(L, n))).pin_memory()
                     for n in NAMES}
        self.host_w = moe.make_weights(fmt, wl.E, wl.H, wl.I, *[self.host[n] for n in NAMES])
        self.slots = {n: torch.zeros((n_slots + 1,) + tuple(self.host[n].shape[1:]),
                                     dtype=self.host[n].dtype, device="cuda:0") for n in NAMES}
        self.slot_w = moe.make_weights(fmt, n_slots, wl.H, wl.I, *[self.slots[n] for n in NAMES])
        self.cache = moe.ExpertCache(wl.E, n_slots)
        self.ws_b = moe.moe_host_experts_workspace_bytes(self.host_w, max_tokens, wl.k)
        self.ws = torch.empty(self.ws_b, dtype=torch.uint8, device="cuda:0")
        moe.moe_workspace_init(self.ws, self.ws_b)
        self.sc_b = moe.moe_host_experts_scratch_bytes(wl.E, max_tokens, wl.k)
        self.scratch = torch.empty(self.sc_b, dtype=torch.uint8, pin_memory=True)
        self.ev = _hip_event()
        self.copy_stream = torch.cuda.Stream()
        self.model = LruModel(wl.E, n_slots)

    def forward(self, x, T):
        out = torch.empty((T, self.wl.H), dtype=torch.float32, device="cuda:0")
        moe.moe_forward_host_experts(self.host_w, self.slot_w, self.cache, self.D.wr, x, T,
                                     self.wl.k, out, moe.MOE_DT_F32, self.ws, self.ws_b,
                                     self.scratch, self.sc_b, self.ev,
                                     copy_stream=self.copy_stream)
        got = to_host(out)
        ip, wp = moe.moe_debug_routing(self.host_w, T, self.wl.k, self.ws, self.ws_b)
        ids = d2h(ip, (T, self.wl.k), np.int32)
        w = d2h(wp, (T, self.wl.k), np.float32)
        self.model.call(ids)
        c = self.cache
        assert np.array_equal(c.slot_of, self.model.slot_of)
        assert np.array_equal(c.expert_of, self.model.expert_of)
        assert (c.c.hits, c.c.misses) == (self.model.hits, self.model.misses)
        return got, ids, w


def _check(got, ref, what, tol=2e-3):
    e = rel_l2(got, ref)
    m = np.abs(got - ref).max() / np.abs(ref).max()
    print(f"{what}: rel_l2={e:.3e} max_rel={m:.3e}", flush=True)
    assert e <= tol and m <= 1e-2


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_decode_tokens_through_a_small_cache(fmt):
    """One token per call at decode shapes (32 experts, 8 slots): hits,
    misses and evictions; each output matches the oracle and the
    device-resident forward."""
    L = synth.make_layer("decode_t1", T=12, E=32, fmt=fmt, seed=2101)
    HL = HostLayer(L, 8, 1)
    W = Weights.from_layer(L)
    for t in range(L.wl.T):
        x = HL.D.x[t:t + 1]
        got, ids, w = HL.forward(x, 1)
        res = to_host(HL.D.forward(x=x, T=1))
        Lt = synth.make_layer("decode_t1", T=1, E=32, fmt=fmt, seed=2101)
        Lt.x = L.x[t:t + 1]
        ref = routed_reference(orc, W, Lt, ids, w)
        _check(got, ref, f"token {t}: oracle")
        _check(got, res, f"token {t}: resident forward", tol=1e-5)
    print("cache", HL.cache.c.hits, "hits", HL.cache.c.misses, "misses",
          HL.cache.c.bytes_copied, "bytes", flush=True)
    assert HL.cache.c.hits > 0 and HL.cache.c.misses > 8


def test_batches_on_both_expert_paths():
    """4 tokens (VALU path) and 40 tokens (grouped GEMM) through a cache of
    all 16 experts of a small layer, then a repeated batch (all hits)."""
    L = synth.make_layer("tiny_t8", T=40, E=16, k=2, seed=2102)
    HL = HostLayer(L, 16, 40)
    W = Weights.from_layer(L)
    for T in (4, 40, 40):
        got, ids, w = HL.forward(HL.D.x[:T], T)
        Lt = synth.make_layer("tiny_t8", T=T, E=16, k=2, seed=2102)
        ref = routed_reference(orc, W, Lt, ids, w)
        _check(got, ref, f"T={T}: oracle")
    assert HL.cache.c.misses <= 16


def test_refuses_a_call_whose_experts_do_not_fit():
    L = synth.make_layer("tiny_t8", T=8, E=16, k=2, seed=2103)
    HL = HostLayer(L, 4, 8)
    out = torch.empty((8, L.wl.H), dtype=torch.float32, device="cuda:0")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_host_experts(HL.host_w, HL.slot_w, HL.cache, HL.D.wr, HL.D.x, 8, 2, out,
                                     moe.MOE_DT_F32, HL.ws, HL.ws_b, HL.scratch, HL.sc_b, HL.ev)
    assert ei.value.status == moe.MOE_ENOTSUP
    assert HL.cache.c.calls == 0
