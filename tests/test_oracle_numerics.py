"""Pins for the oracle's number-format helpers and stochastic rounding (CPU only)."""
import numpy as np
import torch

import oracle as orc


def _special_f32():
    vals = [0.0, -0.0, 1.0, -1.0, 1.5, 3.0e38, -3.0e38, 3.3895314e38, 1e-40, -1e-40, 1.17549435e-38,
            np.inf, -np.inf, 65504.0, 1.0 + 2**-8, 1.0 + 2**-9, 1.0 + 3 * 2**-9, 2**-126, 2**-149]
    return np.array(vals, dtype=np.float32)


def test_bf16_rne_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        _special_f32(),
        rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 200000).astype(np.float32),
        orc.bits_f32(rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)),
    ])
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f32_to_bf16_rne(x), ref)


def test_bf16_rne_ties_to_even():
    # 1 + 2^-8 is exactly halfway between bf16 1.0 and 1.0078125: ties to even (1.0)
    assert orc.f32_to_bf16_rne(np.float32(1.0 + 2**-8)) == 0x3F80
    # 1 + 3*2^-8 lies halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> even
    assert orc.f32_to_bf16_rne(np.float32(1.0 + 3 * 2**-8)) == 0x3F82
    nan = orc.f32_to_bf16_rne(orc.bits_f32(np.uint32(0xFF800001)))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0 and (nan & 0x8000)


def test_bf16_roundtrip_exact():
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = orc.bf16_to_f64(b)
    finite = np.isfinite(v)
    assert np.array_equal(orc.f32_to_bf16_rne(v[finite].astype(np.float32)), b[finite])


def _sr_sum_and_ups(v):
    r16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    out = orc.stochastic_round(np.full(r16.shape, v, dtype=np.float32), r16)
    vals = orc.bf16_to_f64(out)
    down = orc.bf16_to_f64(orc.f32_bits(np.float32(v)) >> 16)
    ups = int(np.count_nonzero(vals != down))
    return float(np.sum(vals)), ups, vals, down


def test_stochastic_rounding_exhaustively_unbiased():
    """Over all 2^16 random words, the rounded values sum to exactly 2^16 * v and
    the number of round-ups equals the dropped low half (the pages' "fraction of
    the gap, that often")."""
    rng = np.random.default_rng(3)
    vs = list(rng.standard_normal(40).astype(np.float32) * np.float32(0.02))
    vs += [np.float32(1e-40), np.float32(-3e-39), np.float32(1.0), np.float32(-2.0 + 2**-20),
           np.float32(1.9999999), np.float32(-0.0), np.float32(3.0e38)]
    for v in vs:
        total, ups, vals, down = _sr_sum_and_ups(v)
        assert total == float(v) * 65536.0, (v, total)
        assert ups == int(orc.f32_bits(np.float32(v)).item() & 0xFFFF), v
        # every result is one of the two bf16 neighbours of v (no overshoot)
        lo, hi = sorted([float(down[0]), float(vals.max() if v >= 0 else vals.min())])
        assert np.all((vals == down[0]) | (np.abs(vals) > np.abs(down[0])))


def test_stochastic_rounding_specials():
    r16 = np.array([0, 1, 0x7FFF, 0x8000, 0xFFFF], dtype=np.uint16)
    for v in (np.inf, -np.inf):
        out = orc.stochastic_round(np.full(5, v, dtype=np.float32), r16)
        assert np.all(out == (orc.f32_bits(np.float32(v)) >> 16))
    nan = orc.bits_f32(np.full(5, 0xFFC00001, dtype=np.uint32))
    out = orc.stochastic_round(nan, r16)
    assert np.all((out & 0x7FC0) == 0x7FC0) and np.all(out & 0x8000)
    # exact bf16 values never move
    exact = orc.bf16_to_f64(np.array([0x3F80, 0xBF80, 0x0001, 0x8000, 0x7F7F], dtype=np.uint16)).astype(np.float32)
    for e in exact:
        out = orc.stochastic_round(np.full(5, e, dtype=np.float32), r16)
        assert np.all(out == (orc.f32_bits(e) >> 16))
    # the largest finite values can carry into infinity, as the rule allows
    top = orc.bits_f32(np.uint32(0x7F7FFFFF))
    assert orc.stochastic_round(np.float32(top), np.uint16(1)) == 0x7F80


def test_pre_round_value_is_two_roundings_without_fma():
    w = np.array([0x3C23], dtype=np.uint16)  # ~0.00995
    h = np.array([[1.2345678]], dtype=np.float32)
    s = np.float32(3.3e-4)
    v = orc.pre_round_values(w.reshape(1, 1), h, s)
    prod = np.float32(s * h[0, 0])
    expect = np.float32(np.float32(orc.bf16_to_f64(w)[0]) - prod)
    assert v[0, 0] == expect
