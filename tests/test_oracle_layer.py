"""Pins of the oracle's router (S1/S2), permutation (S4), expert FFN (S5/S6)
and whole layer (S7) against brute force, closed forms, invariants and an
independent dense float64 path."""
import itertools

import numpy as np
import pytest

import dense_ref
import synth
from oracle import FMT_FP4, Oracle, Weights

orc = Oracle()


def _tiny(**over):
    return synth.make_layer("tiny_t8", **over)


# ---------------------------------------------------------------- S1 -----

def test_router_logits_within_fp32_bound_of_exact_sum():
    L = _tiny(T=16)
    z = orc.router_logits(L.x, L.wr)
    xf = dense_ref.bf16_to_f32(L.x).astype(np.float64)
    wf = dense_ref.bf16_to_f32(L.wr).astype(np.float64)
    exact = xf @ wf                 # products are exact; fp64 sum error is negligible here
    bound = (np.abs(xf) @ np.abs(wf)) * (L.wl.H + 8) * 2.0 ** -24
    assert np.all(np.abs(z - exact) <= bound)


def test_router_sum_order_is_one_ascending_chain():
    """Worked case of the fixed order: x = 1, H = 512 (8 chunks of 64).
    Expert 0: chunk 0 sums to 2^24 and chunks 4..7 to 1 each.  One running
    sum over the chunk partials in ascending order meets 2^24 first, and
    2^24 + 1 rounds back to 2^24 (a tie, to the even significand), so every
    +1 is dropped: z = 2^24 (a sum of the last four chunks first would keep
    them: 2^24 + 4).  Expert 1 holds the same values in the reverse order:
    1 + 1 + 1 + 1 = 4 first, then 4 + 2^24 = 2^24 + 4 exactly.  Expert 2:
    inside chunk 0, h = 0 holds 2^24 and h = 1..4 hold 1: ascending h drops
    each 1, z = 2^24.  Expert 3: the same inside chunk 0 in the reverse
    order (h = 0..3 hold 1, h = 4 holds 2^24): z = 2^24 + 4."""
    H, E = 512, 4
    one, big = 0x3F80, 0x4B80                          # bf16 1.0 and 2^24
    x = np.full((1, H), one, np.uint16)
    wr = np.zeros((H, E), np.uint16)
    wr[5, 0] = big
    for c in range(4, 8):
        wr[64 * c + 7, 0] = one
    for c in range(4):
        wr[64 * c + 3, 1] = one
    wr[64 * 6 + 1, 1] = big
    wr[0, 2] = big
    wr[1:5, 2] = one
    wr[0:4, 3] = one
    wr[4, 3] = big
    z = orc.router_logits(x, wr)
    assert z[0].tolist() == [2.0 ** 24, 2.0 ** 24 + 4, 2.0 ** 24, 2.0 ** 24 + 4]


def test_topk_weights_of_a_given_selection():
    """Renormalised sigmoids of the chosen logits, in the order given:
    z = 0 gives sigmoid 1/2 for every expert, so the weights are 1/k."""
    z = np.array([[0.0, 0.0, 0.0, 0.0], [2.0, -1.0, 0.5, 3.0]], np.float32)
    ids = np.array([[3, 0], [3, 1]], np.int32)
    w = orc.topk_weights(z, ids)
    assert np.allclose(w[0], 0.5, rtol=0, atol=1e-15)
    s3, s1 = 1 / (1 + np.exp(-3.0)), 1 / (1 + np.exp(1.0))
    assert np.allclose(w[1], [s3 / (s3 + s1), s1 / (s3 + s1)], rtol=1e-15, atol=0)
    ids2, w2 = orc.topk(z, 2)
    assert np.array_equal(w2, orc.topk_weights(z, ids2))


def test_router_zero_weights_give_lowest_ids_and_equal_weights():
    L = _tiny()
    z = orc.router_logits(L.x, np.zeros_like(L.wr))
    assert not z.any()
    ids, w = orc.topk(z, 2)
    assert np.array_equal(ids, np.tile([0, 1], (L.wl.T, 1)))
    assert np.allclose(w, 0.5, rtol=0, atol=1e-15)


def test_router_scale_by_power_of_two_keeps_ids():
    L = _tiny(T=32)
    z = orc.router_logits(L.x, L.wr)
    ids, _ = orc.topk(z, 2)
    wr2 = (L.wr.astype(np.uint32) + (3 << 7)).astype(np.uint16)  # exponent + 3: W * 8
    z2 = orc.router_logits(L.x, wr2)
    assert np.array_equal(z2, z * np.float32(8))
    ids2, _ = orc.topk(z2, 2)
    assert np.array_equal(ids, ids2)


def _brute_topk(zt, k):
    best = None
    for sub in itertools.combinations(range(zt.size), k):
        key = sorted(((-float(zt[e]), e) for e in sub))
        if best is None or key < best[0]:
            best = (key, [e for _, e in key])
    return best[1]


def test_topk_nan_ranks_after_every_number():
    # no order is given for NaN logits; the reading ranks them below -inf,
    # lower id first among themselves, and keeps -0 == +0
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    z = np.array([[nan, 1.0, nan, -inf, 0.5, nan],
                  [nan, nan, nan, nan, nan, nan],
                  [-0.0, 0.0, nan, -0.0, inf, -inf],
                  [nan, -inf, -inf, nan, 2.0, 2.0]], dtype=np.float32)
    expect = {1: [[1], [0], [4], [4]],
              3: [[1, 4, 3], [0, 1, 2], [4, 0, 1], [4, 5, 1]],
              6: [[1, 4, 3, 0, 2, 5], [0, 1, 2, 3, 4, 5], [4, 0, 1, 3, 5, 2],
                  [4, 5, 1, 2, 0, 3]]}
    for k, rows in expect.items():
        ids, _ = orc.topk(z, k)
        assert ids.tolist() == rows


def test_topk_matches_brute_force_over_all_subsets():
    rng = np.random.default_rng(11)
    z = rng.standard_normal((50, 8)).astype(np.float32)
    z[::5, 3] = z[::5, 5]           # exact ties between ids 3 and 5
    z[1::7, :] = 0.25               # all-equal rows
    for k in (1, 2, 3, 8):
        ids, w = orc.topk(z, k)
        for t in range(z.shape[0]):
            assert list(ids[t]) == _brute_topk(z[t], k)
        s = 1.0 / (1.0 + np.exp(-np.take_along_axis(z, ids, 1).astype(np.float64)))
        assert np.allclose(w, s / s.sum(1, keepdims=True), rtol=1e-15, atol=0)
        assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)


def test_route_agrees_with_fp64_routing_away_from_ties():
    L = _tiny(T=64)
    ids, w = orc.route(L.x, L.wr, 2)
    ids64, w64, z64 = dense_ref.route_fp64(L.x, L.wr, 2)
    srt = -np.sort(-z64, axis=1)
    gap = np.minimum(srt[:, 0] - srt[:, 1], srt[:, 1] - srt[:, 2])
    clear = gap > 1e-4 * np.abs(z64).max()
    assert clear.mean() > 0.9
    assert np.array_equal(ids[clear], ids64[clear])
    assert np.allclose(w[clear], w64[clear], rtol=1e-6)


# ---------------------------------------------------------------- S4 -----

def test_permute_is_stable_counting_sort():
    rng = np.random.default_rng(12)
    T, k, E = 300, 6, 40
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    offsets, row_token, row_of, dropped = orc.permute(ids, E)
    assert dropped == 0
    flat_e = ids.ravel()
    flat_t = np.repeat(np.arange(T), k)
    order = np.argsort(flat_e, kind="stable")      # library stable sort
    assert np.array_equal(row_token[:T * k], flat_t[order])
    counts = np.bincount(flat_e, minlength=E)
    assert np.array_equal(np.diff(offsets[:E + 1]), counts)
    assert offsets[E] == T * k and offsets[E + 1] == T * k + T
    assert np.array_equal(row_token[T * k:], np.arange(T))
    for t in range(T):
        for j in range(k):
            r = row_of[t, j]
            assert row_token[r] == t and offsets[ids[t, j]] <= r < offsets[ids[t, j] + 1]
        assert row_of[t, k] == T * k + t
    assert sorted(row_of.ravel().tolist()) == list(range(T * k + T))


def test_permute_drops_out_of_range_ids():
    ids = np.array([[0, 5], [7, 2], [-1, 3]], np.int32)
    offsets, row_token, row_of, dropped = orc.permute(ids, 6)
    assert dropped == 2
    assert row_of[1, 0] == -1 and row_of[2, 0] == -1
    assert offsets[6] == 4 and offsets[7] == 7


# ---------------------------------------------------------------- S5/S6 --

@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_expert_ffn_matches_dense_matmul(fmt):
    L = _tiny(fmt=fmt, T=4, E=3)
    W = Weights.from_layer(L)
    x = dense_ref.bf16_to_f32(L.x)
    xq, xs = orc.act_quant(x)
    xd = dense_ref.dequant_act(xq, xs)
    for e in range(L.wl.E + 1):
        G, U, D = dense_ref.dense_expert(L, e)
        for t in range(L.wl.T):
            g, u = orc.gate_up(W, e, xq[t], xs[t])
            assert np.allclose(g, G @ xd[t], rtol=1e-12, atol=1e-14 * np.abs(g).max())
            assert np.allclose(u, U @ xd[t], rtol=1e-12, atol=1e-14 * np.abs(u).max())
            h, hq, hs, y = orc.expert_row(W, e, xq[t], xs[t])
            assert np.array_equal(h, orc.swiglu(g, u))
            hq2, hs2 = orc.act_quant(h[None, :])
            assert np.array_equal(hq, hq2[0]) and np.array_equal(hs, hs2[0])
            hd = dense_ref.dequant_act(hq[None, :], hs[None, :])[0]
            assert np.allclose(y, D @ hd, rtol=1e-12, atol=1e-14 * np.abs(y).max())


def test_weight_element_decode_nibble_order_and_scale():
    E, H, I = 1, 128, 128
    gq = np.zeros((E + 1, I, H // 2), np.uint8)
    gs = np.full((E + 1, I, H // 32), 127, np.uint8)
    gq[0, 3, 5] = 0x72          # element 10 = code 2 (1.0), element 11 = code 7 (6.0)
    gs[0, 3, 0] = 125           # elements 0..31 of row 3 scaled by 1/4
    W = Weights(FMT_FP4, E, H, I, gq, gs, gq, gs, gq.reshape(E + 1, H, I // 2), gs)
    assert orc.weight(W, 0, 0, 3, 10) == 0.25
    assert orc.weight(W, 0, 0, 3, 11) == 1.5
    assert orc.weight(W, 0, 0, 3, 12) == 0.0


def test_exact_integer_cross_check_of_one_block():
    """E4M3 * 2^9 and E2M1 * 2 are integers, so a 32-element block dot with
    scale 2^0 can be checked in exact integer arithmetic."""
    L = _tiny(T=1, E=1)
    W = Weights.from_layer(L)
    xq, xs = orc.act_quant(dense_ref.bf16_to_f32(L.x))
    gq = L.gate_q[0].copy()
    ones = np.full_like(L.gate_s[0], 127)
    W1 = Weights(FMT_FP4, 1, L.wl.H, L.wl.I, gq[None].repeat(2, 0), ones[None].repeat(2, 0),
                 L.up_q, L.up_s, L.down_q, L.down_s)
    g, _ = orc.gate_up(W1, 0, xq[0], np.ones_like(xs[0]))
    xi = (dense_ref.E4M3_ARR[xq[0].astype(int)] * 512).astype(np.int64)
    lo = (gq & 0xF).astype(int)
    hi = (gq >> 4).astype(int)
    wc = np.stack([lo, hi], -1).reshape(L.wl.I, L.wl.H)
    wi = (dense_ref.E2M1_ARR[wc] * 2).astype(np.int64)
    exact = (wi * xi[None, :]).sum(1)
    assert np.array_equal(g * 1024, exact.astype(np.float64))


# ---------------------------------------------------------------- layer --

@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_layer_matches_dense_reference(fmt):
    L = _tiny(fmt=fmt)
    W = Weights.from_layer(L)
    out = orc.forward(W, L.wr, L.x, L.wl.k)
    ids, w = orc.route(L.x, L.wr, L.wl.k)
    ids64, _, _ = dense_ref.route_fp64(L.x, L.wr, L.wl.k)
    assert np.array_equal(ids, ids64)
    ref = dense_ref.forward(L, ids, w)
    err = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert err < 1e-9, err


def test_layer_with_injected_zipf_routing_matches_dense_reference():
    L = _tiny(routing="zipf", zipf_s=1.0, T=12)
    W = Weights.from_layer(L)
    out = orc.forward(W, L.wr, L.x, L.wl.k, ids=L.ids, w=L.w)
    ref = dense_ref.forward(L, L.ids, L.w.astype(np.float64))
    assert np.linalg.norm(out - ref) / np.linalg.norm(ref) < 1e-9


def test_topk_all_with_zero_router_equals_mean_of_all_experts():
    L = _tiny(T=4)
    E = L.wl.E
    W = Weights.from_layer(L)
    out = orc.forward(W, np.zeros_like(L.wr), L.x, E)
    x = dense_ref.bf16_to_f32(L.x)
    xq, xs = dense_ref.quant_torch(x)
    ref = np.zeros_like(out)
    for e in range(E + 1):
        for t in range(L.wl.T):
            _, _, _, y = orc.expert_row(W, e, xq[t], xs[t])
            ref[t] += y if e == E else y / E
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14 * np.abs(ref).max())


def test_single_expert_top1_is_dense_ffn_plus_shared():
    L = _tiny(E=1, T=3)
    W = Weights.from_layer(L)
    out = orc.forward(W, L.wr, L.x, 1)
    ids = np.zeros((3, 1), np.int32)
    ref = dense_ref.forward(L, ids, np.ones((3, 1)))
    assert np.linalg.norm(out - ref) / np.linalg.norm(ref) < 1e-9


def test_expert_permutation_invariance_is_bit_exact():
    L = _tiny(T=8)
    E = L.wl.E
    W = Weights.from_layer(L)
    out = orc.forward(W, L.wr, L.x, L.wl.k)
    perm = np.array([5, 2, 7, 0, 3, 6, 1, 4])
    full = np.concatenate([perm, [E]])
    P = Weights(W.fmt, E, W.H, W.I, L.gate_q[full], L.gate_s[full], L.up_q[full], L.up_s[full],
                L.down_q[full], L.down_s[full])
    wr = np.ascontiguousarray(L.wr[:, perm])
    # ties never occur here, so the permuted router selects the same experts
    out2 = orc.forward(P, wr, L.x, L.wl.k)
    assert np.array_equal(out, out2)


def test_token_subset_equals_full_forward():
    L = _tiny(T=8)
    W = Weights.from_layer(L)
    full = orc.forward(W, L.wr, L.x, 2)
    sub = orc.forward(W, L.wr, L.x, 2, tokens=[6, 1])
    assert np.array_equal(sub, full[[6, 1]])
