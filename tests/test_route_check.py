"""CPU pins of the selection-validity check the GPU router tests use."""
import numpy as np

import synth
from oracle import Oracle
from route_check import BAND_REL, check_selection

orc = Oracle()


def _z():
    x = synth.normal_bf16(61, 1, (16, 1024), 1.0)
    wr = synth.normal_bf16(61, 2, (1024, 64), 0.02)
    return orc.router_logits(x, wr)


def test_oracle_selection_is_valid_and_not_substituted():
    z = _z()
    ids, _ = orc.topk(z, 6)
    valid, sub = check_selection(ids, z, ids)
    assert valid.all() and not sub.any()


def test_far_apart_swaps_and_wrong_members_are_rejected():
    z = _z()
    ids, _ = orc.topk(z, 6)
    bad = ids.copy()
    bad[0, [0, 5]] = bad[0, [5, 0]]                 # rank 1 and rank 6 swapped
    order = np.argsort(-z[1], kind="stable")
    bad[1, 5] = order[40]                           # a far lower expert in slot 6
    bad[2, 1] = bad[2, 0]                           # a repeated id
    bad[3, 0] = 64                                  # out of range
    valid, sub = check_selection(bad, z, ids)
    assert not valid[:4].any() and sub[:4].all()
    assert valid[4:].all() and not sub[4:].any()


def test_swaps_inside_the_band_are_accepted():
    z = _z()
    ids, _ = orc.topk(z, 6)
    z2 = z.copy()
    t = 5
    a, b = ids[t, 2], ids[t, 3]
    z2[t, b] = z2[t, a] - 0.25 * BAND_REL * np.abs(z2[t]).max()   # ranks 3, 4 now nearly tie
    ids2, _ = orc.topk(z2, 6)
    swapped = ids2.copy()
    swapped[t, [2, 3]] = swapped[t, [3, 2]]
    valid, sub = check_selection(swapped, z2, ids2)
    assert valid.all() and sub[t] and sub.sum() == 1
    # the k-th and (k+1)-th in a near tie: the other one may be chosen
    z3 = z.copy()
    nxt = np.argsort(-z3[t], kind="stable")[6]
    z3[t, nxt] = z3[t, ids[t, 5]] - 0.25 * BAND_REL * np.abs(z3[t]).max()
    ids3, _ = orc.topk(z3, 6)
    alt = ids3.copy()
    alt[t, 5] = nxt
    valid, sub = check_selection(alt, z3, ids3)
    assert valid.all() and sub[t]
    # the same exchange without the near tie is rejected
    valid, _ = check_selection(alt, z, ids)
    assert not valid[t]
