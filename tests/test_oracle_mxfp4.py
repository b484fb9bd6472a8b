"""Pins for the oracle's MX FP4 pieces (E2M1 codec, E8M0 block scale, block
quantiser) and the two FP4 producer ops built from them (CPU only).  The
format is the OCP Microscaling MXFP4: E2M1 elements in blocks of 32 with a
power-of-two E8M0 scale."""
import math

import numpy as np
import pytest

import oracle
import workloads

EPS = 1e-6
MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]      # E2M1 magnitudes by code


def test_e2m1_decode_all_codes():
    for c in range(16):
        v = oracle.e2m1_decode(c)
        want = MAGS[c & 7] * (-1.0 if c & 8 else 1.0)
        assert v == want and math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)


def _nearest_code(v):
    """Brute force: nearest magnitude, ties to the even code, |v| >= 6 -> 7."""
    a = abs(v)
    if a >= 6.0:
        m = 7
    else:
        d = [abs(a - x) for x in MAGS]
        best = min(d)
        cands = [c for c in range(8) if d[c] == best]
        m = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return m | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_encode_brute_force_sweep():
    grid = np.arange(-8 * 512, 8 * 512 + 1) / 512.0
    mids = [(a + b) / 2 for a, b in zip(MAGS, MAGS[1:])]
    vals = list(grid) + mids + [-m for m in mids] + [-0.0, 1e-300, -1e-300, 1e30, -1e30]
    for v in vals:
        assert oracle.e2m1_encode(v) == _nearest_code(v), v


def test_e2m1_ties_and_saturation():
    # midpoints go to the even mantissa; 5 -> 4 (not 6); beyond 6 saturates
    assert [oracle.e2m1_encode(v) for v in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)] == \
        [0, 2, 2, 4, 4, 6, 6]
    assert oracle.e2m1_encode(6.5) == 7 and oracle.e2m1_encode(-1e9) == 15
    assert oracle.e2m1_encode(float("inf")) == 7
    assert oracle.e2m1_encode(-0.1) == 8            # sign kept when rounding to 0
    for c in range(16):
        assert oracle.e2m1_encode(oracle.e2m1_decode(c)) == c


def test_mx_scale_code_worked_values():
    cases = {1.0: 125, 6.0: 127, 7.99: 127, 8.0: 128, 0.5: 124, 4.0: 127,
             3.99: 126, 0.0: 0, 2.0 ** -130: 0, 2.0 ** -125: 0, 2.0 ** -124: 1,
             2.0 ** 200: 254}
    for amax, code in cases.items():
        assert oracle.mx_scale_code(amax) == code, amax


def test_mx_scale_puts_block_max_in_4_to_8():
    rng = np.random.default_rng(5)
    for amax in 2.0 ** rng.uniform(-100, 100, 2000):
        X = 2.0 ** (oracle.mx_scale_code(amax) - 127)
        assert 4.0 <= amax / X < 8.0


def test_quant_mxfp4_worked_block():
    y = np.zeros(64)
    y[:6] = [1.0, -0.5, 3.0, 7.0, 0.25, 0.75]
    y[32:36] = [0.0, -0.0, 2.0 ** -20, -3 * 2.0 ** -21]   # second block
    packed, scales = oracle.quant_mxfp4(y)
    assert scales[0] == 127                          # amax 7 -> 2^(2-2)
    assert list(packed[:4]) == [0x92, 0x75, 0x20, 0x00]
    # block 2: amax 2^-20 -> scale 2^-22; values / scale: 0, -0, 4, -6
    assert scales[1] == 127 - 22
    assert list(packed[16:18]) == [0x80, 0xF6]


def test_quant_mxfp4_scale_invariance_and_error_bound():
    rng = np.random.default_rng(6)
    y = rng.standard_normal(32 * 64) * np.repeat(2.0 ** rng.uniform(-20, 20, 64), 32)
    y[::97] *= 50.0                                  # outliers
    p1, s1 = oracle.quant_mxfp4(y)
    p2, s2 = oracle.quant_mxfp4(y * 2.0 ** -7)
    assert np.array_equal(p1, p2) and np.array_equal(s1.astype(int) - 7, s2.astype(int))
    codes = oracle.unpack_fp4(p1)
    X = np.repeat(2.0 ** (s1.astype(np.int64) - 127), 32)
    dq = np.array([oracle.e2m1_decode(c) for c in codes]) * X
    r = np.abs(y) / X
    spacing = np.where(r < 2, 0.5, np.where(r < 4, 1.0, 2.0))
    bound = np.maximum(spacing / 2, r - 6.0) * X     # saturation above 6
    assert np.all(np.abs(dq - y) <= bound * (1 + 1e-12))
    assert np.all(np.abs(codes & 7).reshape(-1, 32).max(axis=1) >= 6)   # max in {4, 6}


@pytest.mark.parametrize("wmode", [oracle.W_NONE, oracle.W_MUL, oracle.W_ONE_PLUS])
def test_resid_rmsnorm_mxfp4_composes_pinned_pieces(wmode):
    dt = oracle.BF16
    inp = workloads.resid_rmsnorm_inputs(3, 256, dt, seed=41, outliers=True)
    ro, q, sc = oracle.resid_rmsnorm_mxfp4(inp["x"], inp["residual"], inp["weight"],
                                          wmode, EPS, dt)
    ro8, _, _ = oracle.resid_rmsnorm_fp8(inp["x"], inp["residual"], inp["weight"],
                                         wmode, EPS, oracle.Q_STATIC, 1.0, dt)
    assert np.array_equal(ro, ro8)
    w = oracle.decode16(inp["weight"], dt)
    for t in range(3):
        y = oracle.rmsnorm(oracle.decode16(ro[t], dt), w, wmode, EPS)
        pw, sw = oracle.quant_mxfp4(y)
        assert np.array_equal(q[t], pw) and np.array_equal(sc[t], sw)


def test_gated_act_mxfp4_worked_example_and_composition():
    g = np.zeros(32)
    g[:4] = [1.0, -1.0, 2.0, 0.0]
    u = np.zeros(32)
    u[:4] = 1.0
    gu = np.empty(64)
    gu[0::2], gu[1::2] = g, u
    q, s = oracle.gated_act_mxfp4(workloads.to16(gu[None, :], workloads.BF16),
                                  oracle.ACT_SWIGLU, oracle.BF16)
    # silu: 0.7311, -0.2689, 1.7616, 0 -> scale 2^-2 -> 2.92, -1.08, 7.05, 0
    assert s[0, 0] == 125 and list(q[0, :2]) == [0xA5, 0x07]
    inp = workloads.gated_act_inputs(2, 256, workloads.F16, seed=42, outliers=True)
    for act in (oracle.ACT_SWIGLU, oracle.ACT_GEGLU_TANH, oracle.ACT_SQRELU):
        q, s = oracle.gated_act_mxfp4(inp["gate_up"], act, workloads.F16)
        for t in range(2):
            v = oracle.decode16(inp["gate_up"][t], workloads.F16)
            h = np.array([oracle.act(x, act) for x in v[0::2]]) * v[1::2]
            pw, sw = oracle.quant_mxfp4(h)
            assert np.array_equal(q[t], pw) and np.array_equal(s[t], sw)
