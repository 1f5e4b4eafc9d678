"""Pins of the oracle's element codecs and of S3 (activation quantisation)
against what the format specifications and the mathematics fix."""
import math

import numpy as np
import pytest
import torch

import dense_ref
from oracle import Oracle

orc = Oracle()


def _golden(name, hexkey=False):
    return dense_ref._read_table(name, hexkey)


def test_e2m1_all_16_codes_match_spec_table():
    tab = _golden("e2m1_values.txt")
    assert len(tab) == 16
    for c, v in tab.items():
        got = orc.e2m1(c)
        assert got == v, (c, got, v)
        assert math.copysign(1.0, got) == math.copysign(1.0, v), c  # -0 for code 8


def test_ue8m0_values_match_spec_and_double_per_step():
    for b, v in _golden("ue8m0_values.txt").items():
        got = orc.ue8m0(b)
        if math.isnan(v):
            assert math.isnan(got)
        else:
            assert got == v, (b, got, v)
    for b in range(0, 254):
        assert orc.ue8m0(b + 1) == 2.0 * orc.ue8m0(b)


def test_e4m3_selected_values_match_spec():
    for c, v in _golden("e4m3_values.txt", hexkey=True).items():
        got = orc.e4m3(c)
        if math.isnan(v):
            assert math.isnan(got), hex(c)
        else:
            assert got == v and math.copysign(1, got) == math.copysign(1, v), (hex(c), got, v)


def test_e4m3_decode_all_256_codes_match_library():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = orc.e4m3_table()
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(mine))
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(lib[~nan], mine[~nan])
    assert np.array_equal(np.signbit(lib[~nan]), np.signbit(mine[~nan]))


def test_e4m3_roundtrip_every_finite_code():
    tab = orc.e4m3_table()
    codes = [c for c in range(256) if not math.isnan(tab[c])]
    vals = np.array([tab[c] for c in codes], np.float32)
    enc = orc.e4m3_encode(vals)
    assert list(enc) == codes  # includes 0x80 (-0) -> 0x80


def test_e4m3_encode_saturates_and_keeps_sign():
    v = np.array([448.0, 449.0, 463.99, 464.0, 500.0, 1e30, np.inf, -449.0, -np.inf,
                  -0.0, -1e-30, 1e-30, -2.0 ** -11], np.float32)
    enc = list(orc.e4m3_encode(v))
    assert enc == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE,
                   0x80, 0x80, 0x00, 0x80]


def _brute_nearest(v: np.ndarray) -> np.ndarray:
    """Nearest non-negative finite E4M3 value by exhaustive search over the
    127 values; exact ties go to the even code (= even mantissa)."""
    tab = dense_ref.E4M3_ARR[:0x7F]  # codes 0x00..0x7E, ascending
    a = np.abs(v.astype(np.float64))
    d = np.abs(a[:, None] - tab[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.arange(0x7F)[None, :]
    even = np.where(cand & (idx % 2 == 0), idx, 10 ** 6).min(axis=1)
    any_ = np.where(cand, idx, 10 ** 6).min(axis=1)
    code = np.where(cand.sum(axis=1) > 1, even, any_)
    code = np.where(a >= 448.0, 0x7E, code)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def _boundary_probe_values():
    tab = dense_ref.E4M3_ARR[:0x7F]
    mids = ((tab[1:] + tab[:-1]) / 2).astype(np.float32)
    out = [mids]
    for k in range(1, 4):
        out.append(np.nextafter(mids, np.float32(np.inf)))
        out.append(np.nextafter(mids, np.float32(0)))
        mids = out[-2]
    base = np.concatenate(out + [tab.astype(np.float32)])
    return np.concatenate([base, -base]).astype(np.float32)


def test_e4m3_encode_matches_brute_force_at_every_midpoint():
    v = _boundary_probe_values()
    assert np.array_equal(orc.e4m3_encode(v), _brute_nearest(v))


def test_e4m3_encode_matches_brute_force_random():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(orc.e4m3_encode(v), _brute_nearest(v))


def test_e4m3_encode_matches_library_on_dense_sweep():
    """Every fp32 whose exponent lies in [2^-12, 2^9) with the 16 low mantissa
    bits sampled (all 128 patterns of the top 7 mantissa bits, which decide
    the rounding, crossed with 64 low patterns), both signs, |x| < 464
    (above 464 the library returns NaN while the layer saturates)."""
    exps = np.arange(127 - 12, 127 + 9, dtype=np.uint32)
    hi7 = np.arange(128, dtype=np.uint32) << 16
    lo = np.concatenate([np.arange(32, dtype=np.uint32),
                         (np.uint32(0xFFFF) - np.arange(32, dtype=np.uint32))])
    mant = (hi7[:, None] | lo[None, :]).ravel()
    bits = (exps[:, None] << 23 | mant[None, :]).ravel()
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    v = bits.view(np.float32)
    v = v[np.abs(v) < 464]
    lib = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(v), lib)


# ---------------------------------------------------------------- S3 ------

def test_act_quant_matches_library_quantiser():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((37, 512)) * np.exp(rng.uniform(-8, 8, (37, 1)))).astype(np.float32)
    q, s = orc.act_quant(x)
    q2, s2 = dense_ref.quant_torch(x)
    assert np.array_equal(s, s2)
    assert np.array_equal(q, q2)


def test_act_quant_power_of_two_invariance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((9, 384)).astype(np.float32)
    q, s = orc.act_quant(x)
    for j in (-20, -3, 1, 5, 30):
        qj, sj = orc.act_quant((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(qj, q)
        assert np.array_equal(sj, (s * np.float32(2.0 ** j)).astype(np.float32))


def test_act_quant_zero_block_and_amax_element():
    x = np.zeros((2, 256), np.float32)
    x[1, 128:] = np.linspace(-3, 2, 128, dtype=np.float32)
    x[0, 130] = -0.0
    q, s = orc.act_quant(x)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    assert not q[0].any() and not q[1, :128].any()
    assert s[1, 1] == np.float32(3.0) / np.float32(448.0)
    assert q[1, 128] == 0xFE  # the amax element maps to -448


def test_act_quant_bf16_equals_f32_of_same_values():
    rng = np.random.default_rng(5)
    xb = (rng.integers(0, 2 ** 16, (6, 256), dtype=np.uint32)).astype(np.uint16)
    xb &= np.uint16(0xBFFF)  # clear the top exponent bit: finite, moderate values
    xf = dense_ref.bf16_to_f32(xb)
    q1, s1 = orc.act_quant(xb)
    q2, s2 = orc.act_quant(xf)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("compiler", ["clang"])
def test_oracle_builds_and_agrees_with_second_compiler(tmp_path, compiler):
    """The oracle is portable C99: a Clang build gives bit-identical codes."""
    import shutil

    import oracle as om
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    so = om.build(compiler=compiler, out=str(tmp_path / "liboracle_clang.so"))
    other = om.Oracle(so)
    v = _boundary_probe_values()
    assert np.array_equal(other.e4m3_encode(v), orc.e4m3_encode(v))
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 256)).astype(np.float32)
    a, b = other.act_quant(x), orc.act_quant(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
