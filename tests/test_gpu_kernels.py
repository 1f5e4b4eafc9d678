"""GPU parity of each step against the oracle, through the C ABI.

Bit-exact: activation codes/scales (S3), expert ids (S2), permutation tables
(S4).  Float: router weights <= 1e-5 relative; stage-wise FFN checks on the
intermediate h (see test_expert_ffn_stagewise)."""
import numpy as np
import pytest
import torch

import synth
from oracle import Oracle, Weights

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_expert_ffn_moe_amd as moe  # noqa: E402
from gpu_util import DevLayer, check_gpu_selection, d2h, rel_l2, to_dev, to_host  # noqa: E402

orc = Oracle()


def _print(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ S3 ----

def _act_inputs(rows, cols, seed):
    x = synth.normal_bf16(seed, 1, (rows, cols), 1.0)
    if rows >= 3 and cols >= 256:
        x[1, 128:256] = 0                   # a zero block
        x[2, :128] = np.uint16(0x8000)      # a block of -0
        x[2, 130] = np.uint16(0x0001)       # tiny subnormal bf16 in an otherwise normal block
        x[0, 5] = np.uint16(0x7F00)         # a huge finite value
    return x


@pytest.mark.parametrize("rows,cols", [(1, 128), (3, 256), (33, 4096), (1000, 4096), (17, 8192)])
def test_act_quant_bf16_bitexact(rows, cols):
    _print("act_quant bf16", rows, cols)
    x = _act_inputs(rows, cols, 77 + rows)
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 128), dtype=torch.float32, device="cuda")
    moe.act_quant_fp8(to_dev(x), moe.MOE_DT_BF16, rows, cols, q, s)
    qr, sr = orc.act_quant(x)
    assert np.array_equal(to_host(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(to_host(q), qr)


def test_act_quant_f32_random_bitexact():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((257, 512)) * np.exp(rng.uniform(-30, 30, (257, 1)))).astype(np.float32)
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    s = torch.empty((257, 4), dtype=torch.float32, device="cuda")
    moe.act_quant_fp8(to_dev(x), moe.MOE_DT_F32, 257, 512, q, s)
    qr, sr = orc.act_quant(x)
    assert np.array_equal(to_host(s).view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(to_host(q), qr)


def test_act_quant_encoder_exhaustive_sweep():
    """Every fp32 with |v| <= 448 through the real kernel: blocks of
    [448, v_1..v_127] have scale exactly 1, so each code is E4M3(v_i)."""
    _print("encoder sweep")
    n_pos = np.uint32(0x43E00000) + np.uint32(1)   # bit patterns 0 .. 448.0
    per = 127 * (1 << 21)                           # values per chunk
    total = int(n_pos) * 2
    done = 0
    mism = 0
    while done < total:
        cnt = min(per, total - done)
        idx = np.arange(done, done + cnt, dtype=np.uint32)
        neg = idx >= n_pos
        idx[neg] -= n_pos
        idx[neg] |= np.uint32(0x80000000)
        vals = idx.view(np.float32)
        nb = (cnt + 126) // 127
        blk = np.zeros((nb, 128), np.float32)
        blk[:, 0] = 448.0
        flat = blk[:, 1:].reshape(-1)
        flat[:cnt] = vals
        blk[:, 1:] = flat.reshape(nb, 127)
        q = torch.empty((nb, 128), dtype=torch.uint8, device="cuda")
        s = torch.empty((nb, 1), dtype=torch.float32, device="cuda")
        moe.act_quant_fp8(to_dev(blk), moe.MOE_DT_F32, nb, 128, q, s)
        qg = to_host(q)[:, 1:].reshape(-1)[:cnt]
        assert np.all(to_host(s) == 1.0)
        qr = orc.e4m3_encode(vals)
        mism += int(np.count_nonzero(qg != qr))
        done += cnt
    _print("encoder sweep values", total, "mismatches", mism)
    assert mism == 0


# ------------------------------------------------------------ S1 / S2 -----

@pytest.mark.parametrize("T,H,E,k", [(1, 256, 8, 2), (3, 256, 8, 2), (8, 256, 8, 2),
                                     (64, 256, 8, 2), (1, 4096, 256, 6), (4, 4096, 256, 6),
                                     (5, 4096, 256, 6), (37, 4096, 256, 6),
                                     (300, 4096, 256, 6), (40, 1024, 100, 16),
                                     (4, 8192, 256, 16), (2, 8192, 200, 11),
                                     (33, 8192, 200, 11), (257, 4096, 256, 6),
                                     (3, 384, 256, 6), (1024, 4096, 256, 6),
                                     (300, 384, 200, 11), (256, 8192, 100, 16)])
def test_route_ids_valid_topk(T, H, E, k):
    """The GPU's ids are a top-k of the oracle's logits: equal to the
    oracle's, except between logits within the near-tie band (the kernels
    sum the same products in an order of their own); bit-exact where both
    orders coincide (H <= 256: at most four 64-wide chunks).  Weights match
    the oracle's renormalised sigmoids of the GPU's ids."""
    _print("route", T, H, E, k)
    x = synth.normal_bf16(900 + T, 1, (T, H), 1.0)
    wr = synth.normal_bf16(900 + T, 2, (H, E), 0.02)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    # control block + group sums (+ the transposed router from 256 tokens on)
    ws_b = (1 << 22) + ((H // 64 + 3) // 4) * T * E * 4 + (E * H * 2 if T >= 256 else 0)
    ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws, ws_b)
    moe.moe_route(to_dev(x), to_dev(wr), T, H, E, k, ids, w, ws, ws_b)
    ig, wg = to_host(ids), to_host(w)
    check_gpu_selection(orc, x, wr, k, ig, wg, exact=H <= 256)
    # a second call (the arrival counters were reset) gives the same result
    moe.moe_route(to_dev(x), to_dev(wr), T, H, E, k, ids, w, ws, ws_b)
    assert np.array_equal(to_host(ids), ig)
    assert np.array_equal(to_host(w), wg)


@pytest.mark.parametrize("T", [1, 7, 64])
def test_route_ties_pick_lower_ids(T):
    H, E, k = 256, 16, 4
    x = synth.normal_bf16(31, 1, (T, H), 1.0)
    wr = synth.normal_bf16(31, 2, (H, E), 0.02)
    wr[:, 9] = wr[:, 3]          # exact ties between experts 3 and 9
    wr[:, 12] = wr[:, 3]
    zero = np.zeros_like(wr)
    ws_b = 1 << 22
    ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws, ws_b)
    for W in (wr, zero):
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        moe.moe_route(to_dev(x), to_dev(W), T, H, E, k, ids, w, ws, ws_b)
        ir, wref = orc.route(x, W, k)
        assert np.array_equal(to_host(ids), ir)
        assert np.allclose(to_host(w), wref, rtol=1e-5, atol=0)
    assert np.array_equal(ir, np.tile(np.arange(k), (T, 1)))


@pytest.mark.parametrize("T", [1, 4, 9])
def test_route_ties_within_and_across_lanes(T):
    """Experts 3, 67, 131, 195 (one wave lane owns all four) and 10 tie at
    the top; the lower ids must win, in order."""
    H, E, k = 256, 256, 8
    x = synth.normal_bf16(33, 1, (T, H), 1.0) & np.uint16(0x7FFF)   # |x|: sign bit cleared
    wr = synth.normal_bf16(33, 2, (H, E), 0.02)
    big = np.full(H, 0x3F80, np.uint16)    # 1.0: far above every other column's logit
    for e in (3, 10, 67, 131, 195):
        wr[:, e] = big
    ws_b = 1 << 22
    ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws, ws_b)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(to_dev(x), to_dev(wr), T, H, E, k, ids, w, ws, ws_b)
    ir, wref = orc.route(x, wr, k)
    assert np.array_equal(ir[:, :5], np.tile([3, 10, 67, 131, 195], (T, 1)))
    assert np.array_equal(to_host(ids), ir)
    assert np.allclose(to_host(w), wref, rtol=1e-5, atol=0)


@pytest.mark.parametrize("T", [1, 4, 9])
@pytest.mark.parametrize("E,k", [(256, 8), (12, 12)])
def test_route_nan_and_inf_logits(T, E, k):
    """0 * inf makes a NaN logit, 1 * (+-inf) an infinite one: +inf ranks
    first, -inf after every finite logit, NaN after every number (lower ids
    first among equals), as the oracle orders them."""
    _print("route nan/inf", T, E, k)
    H = 256
    x = synth.normal_bf16(35, 1, (T, H), 1.0) & np.uint16(0x7FFF)
    x[:, 0] = 0x0000                      # 0.0
    x[:, 1] = 0x3F80                      # 1.0
    wr = synth.normal_bf16(35, 2, (H, E), 0.02)
    for e in (2, 5):
        wr[0, e] = 0x7F80                 # +inf * 0 -> NaN
    wr[1, 9] = 0x7F80                     # +inf
    wr[1, 3] = 0xFF80                     # -inf
    if E > 130:
        wr[0, 200] = 0x7F80
        wr[1, 130] = 0x7F80
    ws_b = 1 << 22
    ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws, ws_b)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(to_dev(x), to_dev(wr), T, H, E, k, ids, w, ws, ws_b)
    ir, wref = orc.route(x, wr, k)
    assert ir[0, 0] == 9
    if E == 12:
        assert ir[0, -3:].tolist() == [3, 2, 5]
    assert np.array_equal(to_host(ids), ir)
    assert np.allclose(to_host(w), wref, rtol=1e-5, atol=0, equal_nan=True)


# ----------------------------------------------------------------- S4 -----

def _permute_gpu(ids, E):
    T, k = ids.shape
    offsets = torch.empty(E + 2, dtype=torch.int32, device="cuda")
    row_token = torch.full((T * k + T,), -7, dtype=torch.int32, device="cuda")
    row_of = torch.empty((T, k + 1), dtype=torch.int32, device="cuda")
    ws_b = 1 << 24
    ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
    moe.moe_workspace_init(ws, ws_b)
    moe.moe_permute(to_dev(ids), T, k, E, offsets, row_token, row_of, ws, ws_b)
    st = moe.moe_device_status(ws)
    return to_host(offsets), to_host(row_token), to_host(row_of), st


@pytest.mark.parametrize("T,k,E,kind", [(1, 6, 256, "uniform"), (32, 6, 256, "zipf"),
                                        (300, 6, 256, "uniform"), (341, 8, 64, "zipf"),
                                        (4096, 6, 256, "zipf"), (8192, 6, 256, "uniform"),
                                        (1000, 6, 256, "one_group"), (2600, 6, 200, "zipf")])
def test_permute_bitexact(T, k, E, kind):
    _print("permute", T, k, E, kind)
    if kind == "zipf":
        ids, _ = synth.zipf_routing(44, T, E, k, 1.2)
    elif kind == "one_group":
        ids = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    else:
        u = synth.uniform(45, 9, (T, E))
        ids = np.argsort(u, axis=1)[:, :k].astype(np.int32)
    off, rt, ro, st = _permute_gpu(ids, E)
    o2, rt2, ro2, dropped = orc.permute(ids, E)
    assert st == 0 and dropped == 0
    assert np.array_equal(off, o2)
    assert np.array_equal(rt, rt2)
    assert np.array_equal(ro, ro2)


@pytest.mark.parametrize("T", [5, 700])
def test_permute_bad_ids_set_status_and_are_dropped(T):
    k, E = 4, 32
    u = synth.uniform(46, 9, (T, E))
    ids = np.argsort(u, axis=1)[:, :k].astype(np.int32)
    ids[1, 2] = E + 3
    ids[T - 1, 0] = -1
    off, rt, ro, st = _permute_gpu(ids, E)
    o2, rt2, ro2, dropped = orc.permute(ids, E)
    assert dropped == 2
    assert st & moe.MOE_STATUS_BAD_EXPERT_ID
    assert np.array_equal(off, o2)
    n = o2[E + 1]
    assert np.array_equal(rt[:n], rt2[:n])
    assert np.array_equal(ro, ro2)


# ------------------------------------------------------------ S5 / S6 -----

# Stage tolerances.  The VALU GEMV path sums exact fp16 products in fp32
# (error ~1e-7 relative), so an h code may differ from the oracle's only when
# h/s lies within 2^-14 (relative) of a rounding midpoint, and y must match
# the oracle's down projection of the GPU's own codes to 1e-5.  The f8f6f4 MFMA
# does not round its 128-term reduction exactly: a one-MFMA probe on random
# full-range E4M3 x E2M1 and E4M3 x E4M3 operands measured
# |err| <= 2.1e-4 * sum|products| (rel-L2 ~5e-5).  On that path each element's
# allowed h error is that bound (doubled: MFMA_EPS) applied to sum|products|
# of g and u, carried through SwiGLU, and y matches to 2e-4.
BAND_GEMV, MFMA_EPS = 2.0 ** -14, 4.2e-4
YTOL_GEMV, YTOL_MFMA = 1e-5, 2e-4


def _tie_band(h, hs, hq, hq_ref, band, h_err=None):
    """Codes may differ only where h/s lies within `band` (relative) of an
    E4M3 rounding midpoint, widened by the bound h_err on |h_gpu - h| when
    given."""
    tab = orc.e4m3_table()
    s = np.repeat(hs.astype(np.float64), 128, axis=-1)
    t = np.abs(h.astype(np.float64) / s)
    a = np.abs(tab[hq_ref.astype(int)])
    b = np.abs(tab[hq.astype(int)])
    mid = (a + b) / 2
    diff = hq != hq_ref
    tol = band * np.maximum(mid, 1e-30)
    if h_err is not None:
        tol = tol + h_err / s
    near = np.abs(t - mid) <= tol
    return diff, near


def _mfma_h_error_bound(L, e, xq, xs):
    """Bound on |h_gpu - h| per element from the MFMA error bound: |dg| <=
    MFMA_EPS * sum|g products|, likewise u, through h = silu(g) u; the
    block scale (amax) error is folded in as the largest element bound."""
    import dense_ref
    G, U, _ = dense_ref.dense_expert(L, e)
    xd = dense_ref.dequant_act(xq[None, :], xs[None, :])[0]
    g, u = G @ xd, U @ xd
    dg = MFMA_EPS * (np.abs(G) @ np.abs(xd))
    du = MFMA_EPS * (np.abs(U) @ np.abs(xd))
    sg = 1.0 / (1.0 + np.exp(-g))
    silu, dsilu = g * sg, sg * (1.0 + g * (1.0 - sg))
    dh = np.abs(dsilu * u) * dg + np.abs(silu) * du + np.abs(silu * u) * 2.0 ** -22
    h = np.abs(silu * u)
    rel_amax = dh.reshape(-1, 128).max(axis=1) / np.maximum(h.reshape(-1, 128).max(axis=1), 1e-300)
    return dh + h * np.repeat(rel_amax, 128)


@pytest.mark.parametrize("name,over", [
    ("tiny_t8", dict(T=1)),
    ("tiny_t8", dict(T=8)),
    ("tiny_t8", dict(T=8, fmt="fp8")),
    ("tiny_t8", dict(T=200, routing="zipf", zipf_s=0.5)),
    ("tiny_t8", dict(T=1, fmt="fp8")),
    ("tiny_t8", dict(T=5, H=384)),            # MFMA down: half an N-block at the end of H
    ("tiny_t8", dict(T=5, H=384, fmt="fp8")),
    ("tiny_t8", dict(T=3, H=384)),            # VALU path, 3 tokens
    ("tiny_t8", dict(T=4, fmt="fp8")),
])
def test_expert_ffn_stagewise(name, over):
    _print("expert_ffn stagewise", name, over)
    L = synth.make_layer(name, **over)
    wl = L.wl
    T, k, E, H, I = wl.T, wl.k, wl.E, wl.H, wl.I
    W = Weights.from_layer(L)
    D = DevLayer(L)
    if L.ids is None:
        ids, wts = orc.route(L.x, L.wr, k)
    else:
        ids, wts = L.ids, L.w
    xq, xs = orc.act_quant(L.x)
    offsets, row_token, row_of, _ = orc.permute(ids, E)
    R = T * k + T
    y = torch.zeros((R, H), dtype=torch.float32, device="cuda")
    # the MFMA path's fp32 h goes to a debug sink (the VALU path keeps it in ws)
    sink = torch.full((R, I), np.nan, dtype=torch.float32, device="cuda")
    moe.moe_debug_store_h(sink, R * I)
    try:
        moe.moe_expert_ffn(D.w, to_dev(xq), to_dev(xs), T, k, to_dev(offsets), to_dev(row_token),
                           y, D.ws, D.ws_bytes)
        yg = to_host(y)
    finally:
        moe.moe_debug_store_h(None, 0)
    hp, hqp, hsp = moe.moe_debug_intermediates(D.w, T, k, D.ws, D.ws_bytes)
    hq = d2h(hqp, (R, I), np.uint8)
    hs = d2h(hsp, (R, I // 128), np.float32)
    gemv = hp is not None
    h = d2h(hp, (R, I), np.float32) if gemv else to_host(sink)
    assert np.isfinite(h).all()
    grp = np.searchsorted(offsets, np.arange(R), side="right") - 1
    y_err, y_ref_all, y_own_all = [], [], []
    for r in range(R):
        e, t = int(grp[r]), int(row_token[r])
        h_ref, hq_ref, hs_ref, y_ref = orc.expert_row(W, e, xq[t], xs[t])
        # the act_quant rule applied to the GPU's own h, bit for bit (both paths)
        q2, s2 = orc.act_quant(h[r][None, :])
        assert np.array_equal(hq[r], q2[0]) and np.array_equal(hs[r], s2[0]), r
        h_err = None if gemv else _mfma_h_error_bound(L, e, xq[t], xs[t])
        if gemv:
            assert rel_l2(h[r], h_ref) <= 1e-5, r
        else:
            assert np.all(np.abs(h[r].astype(np.float64) - h_ref) <= h_err), r
        diff, near = _tie_band(h_ref, hs[r], hq[r], hq_ref, BAND_GEMV, h_err)
        assert np.all(near[diff]), (r, int(diff.sum()))
        assert np.allclose(hs[r], hs_ref, rtol=1e-5 if gemv else 2e-4, atol=0), r
        y_own = orc.down(W, e, hq[r], hs[r])
        assert rel_l2(yg[r], y_own) <= (YTOL_GEMV if gemv else YTOL_MFMA), r
        y_ref_all.append(y_ref)
        y_own_all.append(yg[r])
    assert rel_l2(np.array(y_own_all), np.array(y_ref_all)) <= 2e-3


def test_combine_matches_fp64_sum():
    T, k, H = 50, 6, 512
    rng = np.random.default_rng(8)
    R = T * k + T
    y = rng.standard_normal((R, H)).astype(np.float32)
    perm = rng.permutation(R).astype(np.int32)
    row_of = perm.reshape(T, k + 1)
    row_of[3, 2] = -1
    w = rng.uniform(0.05, 0.5, (T, k)).astype(np.float32)
    for dt in (moe.MOE_DT_F32, moe.MOE_DT_BF16):
        out = torch.empty((T, H), dtype=torch.float32 if dt == moe.MOE_DT_F32 else torch.uint16,
                          device="cuda")
        moe.moe_combine(to_dev(y), to_dev(row_of), to_dev(w), T, k, H, out, dt)
        ref = np.zeros((T, H))
        for t in range(T):
            ref[t] = y[row_of[t, k]]
            for j in range(k):
                if row_of[t, j] >= 0:
                    ref[t] += float(w[t, j]) * y[row_of[t, j]]
        o = to_host(out)
        if dt == moe.MOE_DT_BF16:
            o = (o.astype(np.uint32) << 16).view(np.float32)
            assert np.allclose(o, ref, rtol=2 ** -8, atol=1e-6)
        else:
            assert np.allclose(o, ref, rtol=1e-5, atol=1e-5)
