"""Pins for the oracle's number formats against library routines, closed
forms and brute force (CPU only)."""
import numpy as np
import pytest
import torch

import oracle

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_f16_decode_all_codes_match_numpy():
    ours = oracle.decode16(ALL16, oracle.F16)
    ref = ALL16.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_all_codes_match_torch():
    ours = oracle.decode16(ALL16, oracle.BF16)
    ref = torch.from_numpy(ALL16.view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_encode16_round_trips_every_finite_code(dtype):
    vals = oracle.decode16(ALL16, dtype)
    fin = np.isfinite(vals)
    back = oracle.encode16_n(vals[fin], dtype)
    assert np.array_equal(back, ALL16[fin])


def _random_doubles(rng, n):
    """Magnitudes from deep subnormal to overflow, both signs."""
    e = rng.uniform(-30, 17, n)
    v = np.exp2(e) * rng.choice([-1.0, 1.0], n)
    return v


def test_f16_encode_matches_numpy_rne():
    rng = np.random.default_rng(1)
    v = _random_doubles(rng, 200000)
    ours = oracle.encode16_n(v, oracle.F16)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_encode_ties_go_to_even():
    # midpoints between consecutive positive float16 values (normal and
    # subnormal): the result must be the neighbour with an even code
    codes = np.arange(1, 0x7BFF, 37, dtype=np.uint16)
    lo = oracle.decode16(codes, oracle.F16)
    hi = oracle.decode16(codes + 1, oracle.F16)
    mid = (lo + hi) / 2
    got = oracle.encode16_n(mid, oracle.F16)
    want = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(got, want)


def test_bf16_encode_matches_torch_rne_on_float32_inputs():
    rng = np.random.default_rng(2)
    v = _random_doubles(rng, 200000).astype(np.float32)
    # add float32 values that sit exactly on bfloat16 midpoints
    bits = rng.integers(0x0080, 0x7F00, 20000).astype(np.uint32) << 16
    bits |= 0x8000
    v = np.concatenate([v, bits.view(np.float32)])
    ours = oracle.encode16_n(v.astype(np.float64), oracle.BF16)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_overflow_and_nan():
    assert oracle.f16_encode(65504.0) == 0x7BFF
    assert oracle.f16_encode(65519.99) == 0x7BFF
    assert oracle.f16_encode(65520.0) == 0x7C00        # RNE overflow -> inf
    assert oracle.f16_encode(-1e9) == 0xFC00
    assert oracle.f16_encode(-0.0) == 0x8000
    assert oracle.f16_encode(2.0 ** -25) == 0x0000      # tie to even (zero)
    assert oracle.f16_encode(1.5 * 2.0 ** -24) == 0x0002
    assert np.isnan(oracle.f16_decode(oracle.f16_encode(float("nan"))))


# ---- e4m3 ------------------------------------------------------------------

def test_e4m3_decode_all_codes_match_torch_float8():
    ours = oracle.e4m3_table()
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # landmarks of the format
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x08] == 2.0 ** -6            # smallest normal
    assert ours[0x01] == 2.0 ** -9            # smallest subnormal
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]


def _nearest_e4m3_brute(v):
    """Brute force: nearest finite e4m3 value after clamping to +-448,
    ties to the even code, the sign kept for zero."""
    table = oracle.e4m3_table()
    pos = np.arange(0, 0x7F)                 # codes 0x00..0x7E, ascending
    vals = table[pos]
    a = np.minimum(np.abs(v), 448.0)
    i = np.clip(np.searchsorted(vals, a), 1, len(vals) - 1)
    lo, hi = vals[i - 1], vals[i]
    dlo, dhi = a - lo, hi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (pos[i] % 2 == 0))
    code = np.where(pick_hi, pos[i], pos[i - 1])
    code = np.where(a <= vals[0], 0, code)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def test_e4m3_encode_brute_force_dense_float32_sweep():
    # every 97th float32 bit pattern in [0, 500], both signs, plus all exact
    # midpoints between neighbouring codes
    bits = np.arange(0, 0x43FA0000, 97, dtype=np.uint32)
    v = bits.view(np.float32).astype(np.float64)
    table = oracle.e4m3_table()
    fin = table[:0x7F]
    mids = (fin[:-1] + fin[1:]) / 2
    v = np.concatenate([v, -v, mids, -mids, [0.0, -0.0]])
    ours = oracle.e4m3_encode_n(v)
    assert np.array_equal(ours, _nearest_e4m3_brute(v))


def test_e4m3_encode_matches_torch_below_464():
    rng = np.random.default_rng(3)
    v = rng.uniform(-463.9, 463.9, 100000).astype(np.float32)
    v = np.concatenate([v, (rng.standard_normal(100000) * 1e-2)
                        .astype(np.float32)])
    ours = oracle.e4m3_encode_n(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8) \
        .numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturation_nan_and_signed_zero():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(464.0) == 0x7E
    assert oracle.e4m3_encode(480.0) == 0x7E          # saturates, not NaN
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(float("inf")) == 0x7E
    assert oracle.e4m3_encode(-float("inf")) == 0xFE
    assert oracle.e4m3_encode(float("nan")) == 0x7F
    assert oracle.e4m3_encode(-1e-9) == 0x80
    assert oracle.e4m3_encode(1.0625) == 0x38          # tie -> even mantissa
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00      # tie -> zero
    assert oracle.e4m3_encode(1.5 * 2.0 ** -10) == 0x01


def test_e4m3_round_trip_error_bound():
    rng = np.random.default_rng(4)
    v = np.exp2(rng.uniform(-12, np.log2(448), 100000))
    q = oracle.e4m3_encode_n(v)
    d = oracle.e4m3_table()[q]
    normal = v >= 2.0 ** -6
    assert np.all(np.abs(d - v)[normal] <= 2.0 ** -4 * v[normal])
    assert np.all(np.abs(d - v)[~normal] <= 2.0 ** -10)
