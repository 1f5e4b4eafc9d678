"""The fused one-token expert kernel (routed gate+up, down of all k + 1 rows
and the combine in one persistent launch, FP4 weights) against the separate
gate+up and down+combine kernels of the same path: same arithmetic in the
same order, so the outputs and the intermediate h rows must agree bit for
bit; and against the oracle with the GPU's own selection.  Consecutive calls
exercise the launch tags of its exchange words, which are never cleared."""
import numpy as np
import pytest
import torch

import synth
from oracle import Oracle, Weights

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_expert_ffn_moe_amd as moe  # noqa: E402
from gpu_util import DevLayer, d2h, gpu_routing, rel_l2, routed_reference, to_host  # noqa: E402

orc = Oracle()


def _print(*a):
    print(*a, flush=True)


def _forward(D, t, out_dtype, fused):
    moe.moe_debug_set_decode_fused(fused)
    try:
        out = to_host(D.forward(x=D.x[t:t + 1], T=1, out_dtype=out_dtype))
        ids, w = gpu_routing(D, 1)
        k, I = D.wl.k, D.wl.I
        hp, hqp, hsp = moe.moe_debug_intermediates(D.w, 1, k, D.ws, D.ws_bytes)
        inter = (d2h(hp, (k + 1, I), np.float32), d2h(hqp, (k + 1, I), np.uint8),
                 d2h(hsp, (k + 1, I // 128), np.float32))
    finally:
        moe.moe_debug_set_decode_fused(0)
    return out, ids, w, inter


@pytest.mark.parametrize("name,over,n_tok", [
    ("decode_t1", dict(T=8), 8),                         # hidden 4096, 256 experts top-6: 256 blocks
    ("decode_t1", dict(T=3, H=2048, seed=2301), 3),      # 128 blocks, one activation chunk per lane
    ("decode_t1", dict(T=3, I=1024, seed=2302), 3),
    ("decode_t1", dict(T=3, E=64, k=7, seed=2303), 3),  # k + 1 = 8 rows: the LDS at its limit
    ("tiny_t8", dict(T=4), 4),                           # hidden 256: 16 blocks, intermediate 128
])
def test_fused_equals_separate_kernels(name, over, n_tok):
    _print("fused decode", name, over)
    L = synth.make_layer(name, **over)
    D = DevLayer(L, max_tokens=1)
    W = Weights.from_layer(L)
    outs, ids_all, w_all = [], [], []
    for t in range(n_tok):
        for dt in (moe.MOE_DT_F32, moe.MOE_DT_BF16):
            of, idf, wf, inf = _forward(D, t, dt, 1)
            os_, ids_, ws_, ins = _forward(D, t, dt, 0)
            assert np.array_equal(idf, ids_) and np.array_equal(wf, ws_), t
            assert np.array_equal(of, os_), (t, dt)
            for a, b in zip(inf, ins):
                assert np.array_equal(a, b), t
            if dt == moe.MOE_DT_F32:
                outs.append(of[0])
                ids_all.append(idf[0])
                w_all.append(wf[0])
    assert moe.moe_device_status(D.ws) == 0
    ref = routed_reference(orc, W, L, np.stack(ids_all), np.stack(w_all))
    out = np.stack(outs)
    e = rel_l2(out, ref)
    m = np.abs(out - ref).max() / np.abs(ref).max()
    _print(f"  vs oracle: rel_l2={e:.3e} max_rel={m:.3e}")
    assert e <= 2e-3 and m <= 1e-2


def test_fused_many_calls_in_a_row():
    """200 fused calls on one workspace (the exchange words keep the tags of
    earlier calls): each equals the separate kernels' output for its token."""
    L = synth.make_layer("decode_t1", T=4, seed=2304)
    D = DevLayer(L, max_tokens=1)
    ref = [_forward(D, t, moe.MOE_DT_F32, 0)[0] for t in range(4)]
    outs = [torch.empty((1, L.wl.H), dtype=torch.float32, device="cuda:0") for _ in range(200)]
    moe.moe_debug_set_decode_fused(1)
    try:
        for i, o in enumerate(outs):
            moe.dsv4_moe_forward(D.w, D.wr, D.x[i % 4:i % 4 + 1], 1, L.wl.k, None, None, o,
                                 moe.MOE_DT_F32, D.ws, D.ws_bytes)
    finally:
        moe.moe_debug_set_decode_fused(0)
    for i, o in enumerate(outs):
        assert np.array_equal(to_host(o), ref[i % 4]), i
    assert moe.moe_device_status(D.ws) == 0


def test_fused_kernel_is_timed():
    """The kernel-timing hook sees the fused kernel on the one-token FP4 path."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    evs = []
    for _ in range(2):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    L = synth.make_layer("decode_t1", T=1, seed=2305)
    D = DevLayer(L, max_tokens=1)
    moe.moe_debug_time_kernel(moe.MOE_KERNEL_DECODE_FFN, evs[0], evs[1])
    moe.moe_debug_set_decode_fused(1)
    try:
        D.forward(x=D.x[:1], T=1)
        torch.cuda.synchronize()
    finally:
        moe.moe_debug_set_decode_fused(0)
        moe.moe_debug_time_kernel(moe.MOE_KERNEL_DECODE_FFN, None, None)
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(evs[0]),
                                   ctypes.c_void_p(evs[1])) == 0
    _print(f"fused kernel {ms.value * 1e3:.1f} us")
    assert 0 < ms.value < 10
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))
