"""End-to-end GPU parity of the whole layer (dsv4_moe_forward) against the
oracle, on every workload shape; at the full prefill sizes the oracle runs on
a sample of tokens (chosen to include the most- and least-loaded experts and
the ragged tails).  Tolerances: relative L2 <= 2e-3 and max-abs <=
1e-2 * max|ref| on the fp32 output."""
import numpy as np
import pytest
import torch

import synth
from oracle import Oracle, Weights

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_expert_ffn_moe_amd as moe  # noqa: E402
from gpu_util import (DevLayer, bf16_bits_to_f32, check_gpu_selection, d2h,  # noqa: E402
                      f64_to_bf16_bits, gpu_routing, grouped_gemm_tile, max_rel, rel_l2,
                      routed_reference, tile_cover_tokens, to_dev, to_host)

orc = Oracle()
REL_L2, MAX_ABS = 2e-3, 1e-2


def _print(*a):
    print(*a, flush=True)


def _check(out, ref, what):
    e1, e2 = rel_l2(out, ref), max_rel(out, ref)
    _print(f"{what}: rel_l2={e1:.3e} max_rel={e2:.3e}")
    assert e1 <= REL_L2, (what, e1)
    assert e2 <= MAX_ABS, (what, e2)


def _sample_tokens(ids, T, n, seed=0):
    """Tokens touching the most and least loaded experts, the first/last
    tokens, and random ones."""
    rng = np.random.default_rng(seed)
    pick = {0, T - 1}
    if ids is not None:
        cnt = np.bincount(ids.ravel(), minlength=ids.max() + 1)
        hot, cold = int(np.argmax(cnt)), int(np.argmin(np.where(cnt > 0, cnt, 1 << 30)))
        for e in (hot, cold):
            ts = np.nonzero((ids == e).any(axis=1))[0]
            pick.update(ts[:2].tolist())
            pick.update(ts[-1:].tolist())
    while len(pick) < min(n, T):
        pick.add(int(rng.integers(0, T)))
    return np.array(sorted(pick), np.int32)


def _run(name, sample=None, threads=0, **over):
    """Forward on the GPU, then the oracle on all tokens, on `sample` random
    ones, or (sample="tiles") on tokens whose rows cover every (group,
    M-tile) work item of the grouped GEMM and the last row of every partly
    filled tile."""
    L = synth.make_layer(name, **over)
    wl = L.wl
    D = DevLayer(L)
    _print("layer", name, over, "T", wl.T, "fmt", wl.fmt, "routing", wl.routing)
    out = to_host(D.forward())
    W = Weights.from_layer(L)
    ids_g, w_g = gpu_routing(D, wl.T) if L.ids is None else (None, None)
    if sample == "tiles":
        ids = L.ids if L.ids is not None else ids_g
        TM = grouped_gemm_tile(wl.T, wl.k, wl.E)
        tok = np.union1d(tile_cover_tokens(orc, ids, wl.E, TM), [0, wl.T - 1]).astype(np.int32)
        _print(f"  {tok.size} tokens cover every work item of {TM}-token tiles")
    elif sample is not None:
        tok = _sample_tokens(L.ids, wl.T, sample)
    else:
        tok = None
    ref = routed_reference(orc, W, L, ids_g, w_g, tok=tok, threads=threads)
    got = out if tok is None else out[tok]
    _check(got, ref, f"{name} {over}")
    assert moe.moe_device_status(D.ws) == 0
    return L, D, out, ref, tok


@pytest.mark.parametrize("over", [dict(), dict(fmt="fp8"), dict(T=1), dict(T=1, fmt="fp8"),
                                  dict(T=2), dict(T=3, E=3, k=3), dict(T=4, fmt="fp8"),
                                  dict(T=5), dict(T=130, routing="zipf", zipf_s=1.0),
                                  dict(E=1, k=1, T=9), dict(E=3, k=3, T=17),
                                  dict(T=3, H=384), dict(T=3, H=384, fmt="fp8"),
                                  dict(T=5, H=384), dict(T=5, H=384, fmt="fp8"),
                                  dict(T=1, H=384), dict(T=40, H=640, fmt="fp8"),
                                  # scale rings: one K step per scale load (K not a multiple
                                  # of 512) in 128- and 256-token tiles, and a single group of
                                  # four steps (K = 512)
                                  dict(T=130, routing="zipf", zipf_s=1.0, fmt="fp8", H=384),
                                  dict(T=520, fmt="fp8", H=640),
                                  dict(T=130, routing="zipf", zipf_s=1.0, H=512),
                                  dict(T=130, routing="zipf", zipf_s=1.0, fmt="fp8", H=512,
                                       I=512)])
def test_tiny_layer(over):
    _run("tiny_t8", **over)


def test_tiny_layer_bf16_output_and_determinism():
    L = synth.make_layer("tiny_t8", T=40)
    D = DevLayer(L)
    a = to_host(D.forward(out_dtype=moe.MOE_DT_BF16))
    b = to_host(D.forward(out_dtype=moe.MOE_DT_BF16))
    assert np.array_equal(a, b)
    f1 = to_host(D.forward())
    f2 = to_host(D.forward())
    assert np.array_equal(f1, f2)
    ref = orc.forward(Weights.from_layer(L), L.wr, L.x, L.wl.k)
    refb = bf16_bits_to_f32(f64_to_bf16_bits(ref))
    got = bf16_bits_to_f32(a)
    assert rel_l2(got, refb) <= 3e-3
    assert max_rel(got, refb) <= 1.5e-2


def test_decode_t1_full_shapes_many_tokens():
    """One token per call at hidden 4096 / intermediate 2048 / 256 experts top-6."""
    L = synth.make_layer("decode_t1", T=24)
    D = DevLayer(L, max_tokens=1)
    outs, ids_g, w_g = [], [], []
    for t in range(L.wl.T):
        outs.append(to_host(D.forward(x=D.x[t:t + 1], T=1))[0])
        i1, w1 = gpu_routing(D, 1)
        ids_g.append(i1[0])
        w_g.append(w1[0])
    out = np.stack(outs)
    ids_g, w_g = np.stack(ids_g), np.stack(w_g)
    ref = routed_reference(orc, Weights.from_layer(L), L, ids_g, w_g)
    _check(out, ref, "decode_t1 x24")
    assert moe.moe_device_status(D.ws) == 0
    ids = torch.empty((L.wl.T, 6), dtype=torch.int32, device="cuda")
    w = torch.empty((L.wl.T, 6), dtype=torch.float32, device="cuda")
    # the router for all 24 tokens at once: a workspace sized for T = 24
    rb = moe.moe_workspace_bytes(D.w, L.wl.T, 6)
    rws = torch.zeros(rb, dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(rws, rb)
    moe.moe_route(D.x, D.wr, L.wl.T, 4096, 256, 6, ids, w, rws, rb)
    check_gpu_selection(orc, L.x, L.wr, 6, to_host(ids), to_host(w), what="24 tokens at once")


def test_decode_t1_repeated_expert_ids():
    """One token whose injected ids repeat experts: a group then holds
    several rows, and the gate+up blocks publish h for each of them in turn;
    a second shape (I = 1024) on the same workspace follows."""
    L = synth.make_layer("decode_t1", T=1, routing="zipf", zipf_s=1.0)
    L.ids[0] = np.array([7, 7, 7, 100, 100, 9], np.int32)
    D = DevLayer(L)
    ref = orc.forward(Weights.from_layer(L), L.wr, L.x, 6, ids=L.ids, w=L.w)
    for _ in range(3):
        _check(to_host(D.forward()), ref, "decode repeated ids")
    # another intermediate size through the same workspace, then back
    L2 = synth.make_layer("decode_t1", T=1, I=1024, seed=2001)
    D2 = DevLayer(L2)
    assert D2.ws_bytes <= D.ws_bytes
    out2 = torch.empty((1, 4096), dtype=torch.float32, device="cuda")
    for _ in range(2):
        moe.dsv4_moe_forward(D2.w, D2.wr, D2.x, 1, 6, None, None, out2, moe.MOE_DT_F32, D.ws,
                             D.ws_bytes)
        ip, wp = moe.moe_debug_routing(D2.w, 1, 6, D.ws, D.ws_bytes)
        ref2 = routed_reference(orc, Weights.from_layer(L2), L2, d2h(ip, (1, 6), np.int32),
                                d2h(wp, (1, 6), np.float32))
        _check(to_host(out2), ref2, "decode I=1024")
    _check(to_host(D.forward()), ref, "decode repeated ids, after I=1024")
    assert moe.moe_device_status(D.ws) == 0


@pytest.mark.parametrize("name,over", [("decode_t1", dict(T=1)), ("tiny_t8", dict(T=1)),
                                       ("decode_t1", dict(T=1, I=1024, seed=2002)),
                                       ("decode_t1", dict(T=4)),
                                       ("decode_t1", dict(T=3, seed=2003)),
                                       ("decode_t1", dict(T=1, fmt="fp8", E=16)),
                                       ("decode_t1", dict(T=2, fmt="fp8", E=16)),
                                       ("tiny_t8", dict(T=4, fmt="fp8"))])
def test_decode_layer_matches_stagewise_kernels(name, over):
    """The router's small-T VALU path (front kernel with the shared expert's
    gate+up, gate+up kernel, down+combine kernel; FP4 or FP8 weights, 1 to 4
    tokens) against the oracle's h rows and the act_quant of its own h, and
    bit for bit against the separate gate+up and down+combine calls on the
    same routing (same arithmetic in the same order); three calls in a row
    reuse the workspace."""
    _print("decode vs stagewise", name, over)
    L = synth.make_layer(name, **over)
    wl = L.wl
    T, k, E, H, I = wl.T, wl.k, wl.E, wl.H, wl.I
    R = T * k + T
    D = DevLayer(L)
    W = Weights.from_layer(L)
    # the separate kernels, on a workspace of their own; the GPU's selection
    # (a valid top-k of the oracle's logits) is the routing of the oracle's rows
    ws2 = torch.zeros(D.ws_bytes, dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws2, D.ws_bytes)
    gids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(D.x, D.wr, T, H, E, k, gids, gw, ws2, D.ws_bytes)
    ids, tw = to_host(gids), to_host(gw)
    check_gpu_selection(orc, L.x, L.wr, k, ids, tw)
    xq, xs = orc.act_quant(L.x)
    offsets, row_token, row_of, _ = orc.permute(ids, E)
    grp = np.searchsorted(offsets, np.arange(R), side="right") - 1
    rows_ref = [orc.expert_row(W, int(grp[r]), xq[row_token[r]], xs[row_token[r]])
                for r in range(R)]
    ref = routed_reference(orc, W, L, ids, tw)
    moe.moe_expert_gate_up(D.w, to_dev(xq), to_dev(xs), T, k, to_dev(offsets), to_dev(row_token),
                           ws2, D.ws_bytes)
    out2 = torch.empty((T, H), dtype=torch.float32, device="cuda")
    moe.moe_expert_down(D.w, T, k, to_dev(offsets), to_dev(row_of), gw, None, out2,
                        moe.MOE_DT_F32, ws2, D.ws_bytes)
    o2 = to_host(out2)
    for call in range(3):
        out = to_host(D.forward())
        _check(out, ref, f"decode {name} {over} call {call}")
        assert np.array_equal(out, o2), call
        assert np.array_equal(gpu_routing(D, T)[0], ids), call
        hp, hqp, hsp = moe.moe_debug_intermediates(D.w, T, k, D.ws, D.ws_bytes)
        assert hp is not None          # the VALU path ran
        h = d2h(hp, (R, I), np.float32)
        hq = d2h(hqp, (R, I), np.uint8)
        hs = d2h(hsp, (R, I // 128), np.float32)
        for r in range(R):
            assert rel_l2(h[r], rows_ref[r][0]) <= 1e-5, (call, r)
            q2, s2 = orc.act_quant(h[r][None, :])
            assert np.array_equal(hq[r], q2[0]) and np.array_equal(hs[r], s2[0]), (call, r)
    assert moe.moe_device_status(D.ws) == 0
    assert moe.moe_device_status(ws2) == 0


@pytest.mark.parametrize("fmt,T", [("fp4", 2), ("fp4", 4), ("fp8", 4)])
def test_small_batch_drawn_routing(fmt, T):
    """2 to 4 tokens with drawn routing (Zipf s=1.0: tokens share experts,
    so groups hold several rows) through the VALU path at decode shapes."""
    over = dict(T=T, routing="zipf", zipf_s=1.0, fmt=fmt)
    if fmt == "fp8":
        over["E"] = 16
    L, D, out, ref, _ = _run("decode_t1", **over)
    hp, _, _ = moe.moe_debug_intermediates(D.w, T, L.wl.k, D.ws, D.ws_bytes)
    assert hp is not None


def test_verify_t32_full_shapes():
    _run("verify_t32")


def test_prefill_fp4_partial_batch():
    _run("prefill_fp4_t4096", T=512, sample="tiles", threads=16)     # 64-token tiles


def test_prefill_fp4_full_tiles():
    _run("prefill_fp4_t4096", sample="tiles", threads=16)            # 128-token tiles


def test_prefill_fp4_256_token_tiles():
    """6144 tokens: 256-token FP4 tiles with hidden 4096 (32 K steps through
    the stage ring from rotated starts), hot groups of many M-tiles."""
    _run("prefill_fp4_t4096", T=6144, sample="tiles", threads=16)


def test_prefill_fp8_full_tiles():
    _run("prefill_fp8_t8192", sample="tiles", threads=16)            # 256-token tiles


def test_prefill_fp8_128_token_tiles():
    _run("prefill_fp8_t8192", T=4096, sample="tiles", threads=16)


def test_all_tokens_on_the_same_experts():
    L = synth.make_layer("tiny_t8", T=300, routing="zipf", zipf_s=1.0)
    L.ids[:] = np.array([5, 2], np.int32)
    D = DevLayer(L)
    out = to_host(D.forward())
    ref = orc.forward(Weights.from_layer(L), L.wr, L.x, 2, ids=L.ids, w=L.w)
    _check(out, ref, "one group")


def test_bad_expert_id_is_skipped_and_flagged():
    L = synth.make_layer("tiny_t8", T=20, routing="zipf", zipf_s=1.0)
    L.ids[3, 1] = 99
    D = DevLayer(L)
    out = to_host(D.forward())
    assert moe.moe_device_status(D.ws, clear=True) & moe.MOE_STATUS_BAD_EXPERT_ID
    assert moe.moe_device_status(D.ws) == 0
    ids = L.ids.copy()
    w = L.w.copy()
    w[3, 1] = 0.0
    ids[3, 1] = 0          # weight 0: same as skipping the slot
    ref = orc.forward(Weights.from_layer(L), L.wr, L.x, 2, ids=ids, w=w)
    _check(out, ref, "bad id")


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_empty_batch_then_a_real_one(fmt):
    """T = 0 enqueues nothing: the output buffer keeps its contents and the
    workspace stays clean; the next call with tokens is unaffected."""
    L = synth.make_layer("tiny_t8", fmt=fmt)
    D = DevLayer(L)
    sentinel = torch.full((1, L.wl.H), 7.0, dtype=torch.float32, device="cuda:0")
    moe.dsv4_moe_forward(D.w, D.wr, D.x, 0, L.wl.k, None, None, sentinel, moe.MOE_DT_F32, D.ws,
                         D.ws_bytes)
    xq = torch.full((1, L.wl.H), 5, dtype=torch.uint8, device="cuda:0")
    xs = torch.full((1, L.wl.H // 128), 3.0, dtype=torch.float32, device="cuda:0")
    moe.act_quant_fp8(D.x, moe.MOE_DT_BF16, 0, L.wl.H, xq, xs)
    assert (to_host(sentinel) == 7.0).all()
    assert (to_host(xq) == 5).all() and (to_host(xs) == 3.0).all()
    assert moe.moe_device_status(D.ws) == 0
    out = to_host(D.forward(injected=False))
    ref = orc.forward(Weights.from_layer(L), L.wr, L.x, L.wl.k)
    _check(out, ref, f"after an empty batch ({fmt})")


@pytest.mark.parametrize("over", [
    dict(fmt="fp4", T=1, H=8192, I=4096),   # the one-token VALU path at its largest shape
    dict(fmt="fp4", T=3, H=8192, I=8192),   # the MFMA path at the ABI's limits
    dict(fmt="fp8", T=3, H=8192, I=8192),
])
def test_maximum_hidden_and_intermediate(over):
    """H and I at the largest values the ABI accepts (two routed experts keep
    the weights and the oracle small); the router runs on x."""
    _run("tiny_t8", E=2, k=2, threads=16, **over)


def test_more_tokens_than_a_grid_row():
    """70,000 tokens (past 65,535, the largest grid y extent): the router,
    permute, grouped GEMM and combine launches index tokens where the grid
    allows that many; checked on a sample that includes the last token."""
    _run("tiny_t8", T=70000, sample=16, threads=16)
