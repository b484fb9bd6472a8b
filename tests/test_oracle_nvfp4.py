"""Pins for the oracle's NVFP4 quantiser and the residual-RMSNorm -> NVFP4
producer built from it (CPU only).  NVFP4 (the format's published
definition; the pages only name it): E2M1 elements in blocks of 16, each
block with an E4M3 scale chosen so that the block maximum maps to 6, and one
fp32 dequantisation scale g for the tensor; value = e2m1 * e4m3 * g."""
import math

import numpy as np
import pytest

import oracle
import workloads

EPS = 1e-6
MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]      # E2M1 magnitudes by code
E4M3 = None


def _e4m3_values():
    global E4M3
    if E4M3 is None:
        E4M3 = oracle.e4m3_table()
    return E4M3


def _nearest_e4m3(v):
    """Brute force over the 127 non-negative finite E4M3 codes: the nearest
    value, ties to the even code, above 448 saturating."""
    vals = _e4m3_values()[:127]
    if v >= 448.0:
        return 0x7E
    d = np.abs(vals - v)
    cands = np.flatnonzero(d == d.min())
    return int(cands[0]) if len(cands) == 1 else int([c for c in cands if c % 2 == 0][0])


def _nearest_e2m1(v):
    a = abs(v)
    if a >= 6.0:
        m = 7
    else:
        d = [abs(a - x) for x in MAGS]
        cands = [c for c in range(8) if d[c] == min(d)]
        m = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return m | (8 if math.copysign(1.0, v) < 0 else 0)


def _unpack(packed):
    return oracle.unpack_fp4(packed)


def test_nvfp4_worked_block():
    # y = 0, 0.25, ..., 3.75 with g = 1/64: amax / (6 g) = 40 = 1.25 * 2^5
    # -> E4M3 code 0x62; S = 40 / 64 = 0.625; y / S = 0, 0.4, 0.8, ... 6.0
    y = np.arange(16) * 0.25
    packed, scales = oracle.quant_nvfp4(y, 1.0 / 64)
    assert list(scales) == [0x62]
    assert list(_unpack(packed)) == [0, 1, 2, 2, 3, 4, 4, 5, 5, 6, 6, 6, 6, 7, 7, 7]
    assert list(packed) == [0x10, 0x22, 0x43, 0x54, 0x65, 0x66, 0x76, 0x77]


def test_nvfp4_signs_zero_block_and_saturation():
    y = np.array([-3.0, 3.0, -0.0, 0.0] + [0.0] * 12)
    p, s = oracle.quant_nvfp4(y, 0.5)             # amax / (6 g) = 1 -> code 0x38, S = 0.5
    assert list(s) == [0x38]
    assert list(_unpack(p)[:4]) == [8 | 7, 7, 8, 0]     # -6, 6, -0, +0
    p, s = oracle.quant_nvfp4(np.zeros(16), 1.0)    # all-zero block: scale code 0, zero codes
    assert list(s) == [0] and not p.any()
    # a scale below the smallest E4M3 subnormal decodes to 0: zero codes, signs kept
    y = np.full(16, -1e-6)
    p, s = oracle.quant_nvfp4(y, 1.0)
    assert list(s) == [0] and list(_unpack(p)) == [8] * 16
    # amax / (6 g) above 448 saturates the scale at 448; elements saturate at 6
    y = np.full(16, 1e6)
    p, s = oracle.quant_nvfp4(y, 1.0)
    assert list(s) == [0x7E] and list(_unpack(p)) == [7] * 16


@pytest.mark.parametrize("g", [1.0 / 64, 0.37 / 448, 3.0e-3, 1.7])
def test_nvfp4_brute_force(g):
    """Against the definition evaluated by search: the block code is the
    nearest E4M3 value to amax / (6 g) (ties to the even code), each element
    the nearest E2M1 value to y / S (ties to even, saturating, sign kept)."""
    rng = np.random.default_rng(int(g * 1e6) + 7)
    y = np.concatenate([rng.standard_normal(16 * 300) * np.exp2(rng.integers(-12, 8, 16 * 300)),
                        np.repeat(np.exp2(rng.integers(-14, 10, 30)), 16) * rng.standard_normal(16 * 30)])
    p, s = oracle.quant_nvfp4(y, g)
    codes = _unpack(p)
    tab = _e4m3_values()
    for b in range(y.size // 16):
        yb = y[16 * b: 16 * b + 16]
        amax = np.abs(yb).max()
        assert s[b] == _nearest_e4m3(amax / (6.0 * g)), b
        S = tab[s[b]] * g
        for i in range(16):
            want = _nearest_e2m1(yb[i] / S) if S > 0 else (8 if math.copysign(1, yb[i]) < 0 else 0)
            assert codes[16 * b + i] == want, (b, i)


def test_nvfp4_block_maximum_maps_to_six():
    """With the scale neither saturated nor underflowed, S is within 1/16 of
    amax / 6, so the block maximum's code is the E2M1 maximum (6)."""
    rng = np.random.default_rng(11)
    y = rng.standard_normal(16 * 2000) * 3.0
    g = 1.0 / 448
    p, s = oracle.quant_nvfp4(y, g)
    codes = _unpack(p).reshape(-1, 16)
    yb = y.reshape(-1, 16)
    arg = np.abs(yb).argmax(axis=1)
    assert np.all((codes[np.arange(len(arg)), arg] & 7) == 7)


def test_nvfp4_power_of_two_invariance_and_error_bound():
    rng = np.random.default_rng(12)
    y = rng.standard_normal(16 * 500)
    g = 0.01
    p1, s1 = oracle.quant_nvfp4(y, g)
    p2, s2 = oracle.quant_nvfp4(y * 8.0, g * 8.0)
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2)
    # dequantised error: at most half the E2M1 spacing at the value (<= 1 S
    # in [4, 6]), plus the saturation at 6 S (S >= amax / 6 / (1 + 2^-4))
    tab = _e4m3_values()
    S = np.repeat(tab[s1] * g, 16)
    deq = np.array([oracle.e2m1_decode(c) for c in _unpack(p1)]) * S
    err = np.abs(deq - y)
    assert np.all(err <= np.maximum(0.25 * S, np.where(np.abs(y) / S > 4, S, 0.5 * S)) + 1e-15)


@pytest.mark.parametrize("wmode", [oracle.W_NONE, oracle.W_MUL, oracle.W_ONE_PLUS])
def test_resid_rmsnorm_nvfp4_is_the_composition(wmode):
    T, H, dt = 5, 96, workloads.BF16
    inp = workloads.resid_rmsnorm_inputs(T, H, dt, 330 + wmode)
    g = 2.5e-3
    ro, q, sc = oracle.resid_rmsnorm_nvfp4(inp["x"], inp["residual"], inp["weight"], wmode,
                                           EPS, g, dt)
    ro8, _, _ = oracle.resid_rmsnorm_fp8(inp["x"], inp["residual"], inp["weight"], wmode, EPS,
                                         oracle.Q_STATIC, 1.0, dt)
    assert np.array_equal(ro, ro8)                  # the same new residual as op (a)
    w = oracle.decode16(inp["weight"], dt)
    for t in range(T):
        y = oracle.rmsnorm(oracle.decode16(ro[t], dt), w, wmode, EPS)
        p, s = oracle.quant_nvfp4(y, np.float32(g))
        assert np.array_equal(q[t], p) and np.array_equal(sc[t], s)
