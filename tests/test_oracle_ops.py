"""Pins for the oracle's building blocks and fused ops (CPU only).

The pages print no worked numeric example for any of these kernels, so the
oracle is pinned by hand-computed closed forms, invariants, special cases
that reduce to a library routine, and brute force.  Each test names the
mistake it is there to catch.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads

EPS = 1e-6


# ---- RMSNorm ------------------------------------------------------------------

def test_rstd_worked_example():
    # [1,2,3,4]: mean of squares 30/4 = 7.5 -> 1/sqrt(7.500001)
    assert oracle.rms_rstd([1, 2, 3, 4], EPS) == pytest.approx(
        0.36514834732689, rel=1e-12)
    # sum instead of mean would give 1/sqrt(30); eps outside the root differs
    # visibly for a small vector: mean 1e-6 -> 1/sqrt(2e-6)
    assert oracle.rms_rstd([1e-3] * 4, EPS) == pytest.approx(
        707.10678118654755, rel=1e-12)


def test_rmsnorm_unit_rms_invariant():
    rng = np.random.default_rng(10)
    v = rng.standard_normal(1024)
    y = oracle.rmsnorm(v, None, oracle.W_NONE, EPS)
    ms = np.mean(v * v)
    assert np.mean(y * y) == pytest.approx(ms / (ms + EPS), rel=1e-12)
    # scale invariance with eps = 0
    y1 = oracle.rmsnorm(v, None, oracle.W_NONE, 0.0)
    y2 = oracle.rmsnorm(v * 37.5, None, oracle.W_NONE, 0.0)
    assert np.allclose(y1, y2, rtol=1e-13, atol=0)


def test_rmsnorm_weight_modes_and_fold_identity():
    rng = np.random.default_rng(11)
    n = 64
    v = rng.standard_normal(n)
    w = rng.standard_normal(n) * 0.3
    y_none = oracle.rmsnorm(v, None, oracle.W_NONE, EPS)
    y_mul = oracle.rmsnorm(v, w, oracle.W_MUL, EPS)
    y_one = oracle.rmsnorm(v, w, oracle.W_ONE_PLUS, EPS)
    assert np.array_equal(oracle.rmsnorm(v, np.ones(n), oracle.W_MUL, EPS),
                          y_none)
    assert np.array_equal(oracle.rmsnorm(v, np.zeros(n), oracle.W_ONE_PLUS,
                                         EPS), y_none)
    # folding (1+w) into the next projection W: W (n(x) * (1+w)) equals
    # (W diag(1+w)) n(x) -- the "_noweight" pre-fold
    Wm = rng.standard_normal((32, n))
    lhs = Wm @ y_one
    rhs = (Wm * (1.0 + w)[None, :]) @ y_none
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    lhs = Wm @ y_mul
    rhs = (Wm * w[None, :]) @ y_none
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    assert not np.allclose(y_one, y_mul)


def test_adarms_worked_example():
    h = np.array([1.0, 2.0, 3.0, 4.0])
    y = oracle.adarms(h, [0.1, 0, -0.1, 0], [0, 0.1, 0, -0.1], EPS)
    # rstd = 0.36514834732689; y = [1.1 rstd, 2 rstd + 0.1, 2.7 rstd,
    # 4 rstd - 0.1]
    assert np.allclose(y, [0.401663182059579, 0.83029669465378,
                           0.98590053778260, 1.36059338930756], rtol=1e-12)


# ---- quantisation ------------------------------------------------------------

def test_quant_static_worked_example():
    y = oracle.rmsnorm([1, 2, 3, 4], None, oracle.W_NONE, EPS)
    q = oracle.quant_static(y, 56.0)
    # y*56 = 20.45, 40.90, 61.35, 81.79 -> e4m3 20, 40, 60, 80
    assert list(q) == [0x5A, 0x62, 0x67, 0x6A]
    tab = oracle.e4m3_table()
    assert list(tab[q]) == [20.0, 40.0, 60.0, 80.0]
    # saturation and subnormal range
    assert list(oracle.quant_static([10.0, -10.0], 56.0)) == [0x7E, 0xFE]
    assert list(oracle.quant_static([2.0 ** -9], 1.0)) == [0x01]


def test_quant_dynamic_worked_example_and_invariants():
    y = oracle.rmsnorm([1, 2, 3, 4], None, oracle.W_NONE, EPS)
    q, s = oracle.quant_dynamic(y)
    assert s == np.float32(1.4605933893075536 / 448.0)
    # y/s = 112, 224, 336 (a tie between 320 and 352), 448
    assert q[0] == 0x6E and q[1] == 0x76 and q[3] == 0x7E
    assert q[2] in (0x7A, 0x7B)
    # zero group: floored scale, zero codes
    q0, s0 = oracle.quant_dynamic(np.zeros(8))
    assert s0 == np.float32(np.float32(1e-10) / 448.0) and not q0.any()
    # random groups: the largest magnitude maps to 448; bounded error
    rng = np.random.default_rng(12)
    tab = oracle.e4m3_table()
    for _ in range(50):
        v = rng.standard_normal(128) * 10.0 ** rng.uniform(-3, 3)
        q, s = oracle.quant_dynamic(v)
        assert np.max(np.abs(tab[q])) == 448.0
        assert abs(float(s) - np.max(np.abs(v)) / 448.0) <= \
            2.0 ** -24 * float(s)
        d = tab[q] * float(s)
        big = np.abs(v) >= 2.0 ** -6 * float(s)
        assert np.all(np.abs(d - v)[big] <= 2.0 ** -4 * np.abs(v)[big] * 1.0001)
        assert np.all(np.abs(d - v)[~big] <= 2.0 ** -10 * float(s) * 1.0001)


# ---- activations -------------------------------------------------------------

def test_activation_worked_values():
    assert oracle.act(1.0, oracle.ACT_SWIGLU) == pytest.approx(0.7310585786300049, rel=1e-14)
    assert oracle.act(-1.0, oracle.ACT_SWIGLU) == pytest.approx(-0.2689414213699951, rel=1e-14)
    assert oracle.act(1.0, oracle.ACT_GEGLU_TANH) == pytest.approx(0.8411919906082768, rel=1e-12)
    assert oracle.act(-1.0, oracle.ACT_GEGLU_TANH) == pytest.approx(-0.15880800939172324, rel=1e-12)
    assert oracle.act(2.0, oracle.ACT_GEGLU_TANH) == pytest.approx(1.9545976940871754, rel=1e-12)
    assert oracle.act(2.0, oracle.ACT_SQRELU) == 4.0
    assert oracle.act(-3.0, oracle.ACT_SQRELU) == 0.0


def test_activations_match_library_routines():
    rng = np.random.default_rng(13)
    g = np.concatenate([rng.standard_normal(2000) * 4, [0.0, -30.0, 30.0]])
    silu = np.array([oracle.act(x, oracle.ACT_SWIGLU) for x in g])
    assert np.allclose(silu, g * scipy.special.expit(g), rtol=1e-14, atol=1e-300)
    gelu = np.array([oracle.act(x, oracle.ACT_GEGLU_TANH) for x in g])
    ref = torch.nn.functional.gelu(torch.from_numpy(g), approximate="tanh").numpy()
    assert np.allclose(gelu, ref, rtol=1e-12, atol=1e-15)
    # the tanh form stays within 1e-3 of the exact (erf) GELU
    exact = torch.nn.functional.gelu(torch.from_numpy(g)).numpy()
    assert np.max(np.abs(gelu - exact)) < 1e-3
    sq = np.array([oracle.act(x, oracle.ACT_SQRELU) for x in g])
    assert np.array_equal(sq, np.maximum(g, 0) ** 2)


# ---- RoPE ------------------------------------------------------------------------

def test_rope_worked_examples():
    # D=4, theta=1e4: inverse frequencies 1 and 1e4^(-1/2) = 0.01
    c1, s1, c2, s2 = math.cos(1), math.sin(1), math.cos(0.01), math.sin(0.01)
    out = oracle.rope([1, 0, 0, 0], 1, 1e4)
    assert np.allclose(out, [c1, 0, s1, 0], rtol=0, atol=1e-15)
    out = oracle.rope([1, 2, 3, 4], 1, 1e4)
    assert np.allclose(out, [-1.9841106485860646, 1.9599006675066357,
                             2.4623779023910066, 4.0197996683000016],
                       rtol=1e-13)
    out = oracle.rope([1, 2, 3, 4], 1, 1e4, oracle.ROPE_INTERLEAVED)
    assert np.allclose(out, [c1 - 2 * s1, 2 * c1 + s1,
                             3 * c2 - 4 * s2, 4 * c2 + 3 * s2], rtol=1e-13)


def test_rope_equals_complex_rotation():
    # rotate-half RoPE is multiplication of z_i = v_i + j v_{i+D/2} by
    # exp(j * pos * theta^(-2i/D))
    rng = np.random.default_rng(14)
    D, pos, theta = 128, 797, 1e6
    v = rng.standard_normal(D)
    z = v[: D // 2] + 1j * v[D // 2:]
    f = theta ** (-np.arange(0, D, 2) / D)
    zr = z * np.exp(1j * pos * f)
    got = oracle.rope(v, pos, theta)
    assert np.allclose(got[: D // 2], zr.real, rtol=0, atol=1e-12)
    assert np.allclose(got[D // 2:], zr.imag, rtol=0, atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(15)
    D, theta = 64, 1e4
    v = rng.standard_normal(D)
    for style in (oracle.ROPE_HALF, oracle.ROPE_INTERLEAVED):
        assert np.array_equal(oracle.rope(v, 0, theta, style), v)
        a = oracle.rope(v, 123, theta, style)
        # pair norms are preserved
        if style == oracle.ROPE_HALF:
            pn = lambda u: u[: D // 2] ** 2 + u[D // 2:] ** 2
        else:
            pn = lambda u: u[0::2] ** 2 + u[1::2] ** 2
        assert np.allclose(pn(a), pn(v), rtol=1e-12)
        # composition R_a R_b = R_(a+b)
        ab = oracle.rope(oracle.rope(v, 40, theta, style), 83, theta, style)
        assert np.allclose(ab, a, rtol=0, atol=1e-12)
        # relative position: <R_m q, R_n k> = <q, R_(n-m) k>
        q, k = rng.standard_normal(D), rng.standard_normal(D)
        lhs = oracle.rope(q, 17, theta, style) @ oracle.rope(k, 50, theta, style)
        rhs = q @ oracle.rope(k, 33, theta, style)
        assert lhs == pytest.approx(rhs, rel=1e-12)
    # the interleaved layout is rotate-half on de-interleaved elements
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
    inter = oracle.rope(v, 77, theta, oracle.ROPE_INTERLEAVED)
    half = oracle.rope(v[perm], 77, theta, oracle.ROPE_HALF)
    assert np.allclose(inter[perm], half, rtol=0, atol=1e-12)


# ---- paged KV slots -----------------------------------------------------------------

def test_kv_slot_identity_table_is_contiguous():
    P, pages = 16, 8
    table = np.arange(pages, dtype=np.int32)
    for p in range(P * pages):
        assert oracle.kv_slot(p, table, P, pages) == p


def test_kv_slot_brute_force_bijection_and_range():
    P, pages = 16, 32
    rng = np.random.default_rng(16)
    table = rng.permutation(pages).astype(np.int32)
    slots = [oracle.kv_slot(p, table, P, pages) for p in range(P * pages)]
    assert sorted(slots) == list(range(P * pages))
    for p in range(P * pages):
        s = slots[p]
        assert s // P == table[p // P] and s % P == p % P
    # out of range: negative, past the table, page id out of range
    assert oracle.kv_slot(-1, table, P, pages) == -1
    assert oracle.kv_slot(P * pages, table, P, pages) == -1
    bad = table.copy()
    bad[3] = pages
    assert oracle.kv_slot(3 * P + 1, bad, P, pages) == -1
    bad[3] = -2
    assert oracle.kv_slot(3 * P + 1, bad, P, pages) == -1


# ---- fused ops: compositions of the pinned pieces ----------------------------------

def _dec(bits, dt):
    return oracle.decode16(bits, dt)


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_resid_rmsnorm_residual_out_is_correctly_rounded_sum(dt):
    inp = workloads.resid_rmsnorm_inputs(8, 256, dt, seed=20)
    ro, _, _ = oracle.resid_rmsnorm_fp8(inp["x"], inp["residual"], None,
                                        oracle.W_NONE, EPS, oracle.Q_STATIC,
                                        56.0, dt)
    # the exact sum of two 16-bit floats rounded once: float16 addition in
    # numpy / bfloat16 addition in torch (both compute in float32, which is
    # wide enough that the double rounding is harmless)
    if dt == oracle.F16:
        ref = (inp["x"].view(np.float16) + inp["residual"].view(np.float16)) \
            .view(np.uint16)
    else:
        a = torch.from_numpy(inp["x"].view(np.int16)).view(torch.bfloat16)
        b = torch.from_numpy(inp["residual"].view(np.int16)).view(torch.bfloat16)
        ref = (a + b).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ro, ref)


def test_resid_rmsnorm_worked_example_fp16():
    x = workloads.to16(np.array([[0.5, 1.0, 1.5, 2.0]]), workloads.F16)
    r = workloads.to16(np.array([[0.5, 1.0, 1.5, 2.0]]), workloads.F16)
    ro, q, _ = oracle.resid_rmsnorm_fp8(x, r, None, oracle.W_NONE, EPS,
                                        oracle.Q_STATIC, 56.0, oracle.F16)
    assert list(_dec(ro[0], oracle.F16)) == [1.0, 2.0, 3.0, 4.0]
    assert list(q[0]) == [0x5A, 0x62, 0x67, 0x6A]
    _, q, s = oracle.resid_rmsnorm_fp8(x, r, None, oracle.W_NONE, EPS,
                                       oracle.Q_TOKEN, 0.0, oracle.F16)
    assert s[0] == np.float32(1.4605933893075536 / 448.0)
    assert q[0, 0] == 0x6E and q[0, 1] == 0x76 and q[0, 3] == 0x7E


def test_resid_rmsnorm_norm_reads_the_rounded_residual():
    # x + r is not representable in bfloat16; the norm must see the rounded
    # sum (the stored residual), not the exact one
    dt = oracle.BF16
    x = workloads.to16(np.array([[1.0, 1.0, 1.0, 1.0]]), dt)
    r = workloads.to16(np.array([[2.0 ** -9 * 3, 0.0, 0.0, 0.0]]), dt)
    ro, q, s = oracle.resid_rmsnorm_fp8(x, r, None, oracle.W_NONE, 0.0,
                                        oracle.Q_TOKEN, 0.0, dt)
    stored = _dec(ro[0], dt)
    assert stored[0] == 1.0 + 2.0 ** -7        # 1 + 3*2^-9 rounds up
    y = oracle.rmsnorm(stored, None, oracle.W_NONE, 0.0)
    qq, ss = oracle.quant_dynamic(y)
    assert np.array_equal(q[0], qq) and s[0] == ss


def test_adarms_op_worked_example_and_reduction_to_plain_norm():
    dt = oracle.F16
    f = lambda a: workloads.to16(np.array([a]), dt)
    ro, q, _ = oracle.adarms_gate_res_fp8(
        f([1, 1, 1, 1]), f([0.5] * 4), f([0.5, 1.5, 2.5, 3.5]),
        f([0.1, 0, -0.1, 0]), f([0, 0.1, 0, -0.1]), EPS, oracle.Q_STATIC,
        56.0, dt)
    assert list(_dec(ro[0], dt)) == [1.0, 2.0, 3.0, 4.0]
    # y = [0.40166, 0.83030, 0.98590, 1.36059]; *56 -> 22.5, 46.5, 55.2, 76.2
    # the scale/shift are fp16-rounded (0.1 -> 0.0999755859375), which
    # does not move any code
    assert list(q[0]) == [0x5B, 0x64, 0x66, 0x6A]
    # gate = 0, scale = shift = 0 is the plain residual norm with x = 0
    inp = workloads.adarms_inputs(6, 128, dt, seed=21)
    z = np.zeros_like(inp["x"])
    ro1, q1, s1 = oracle.adarms_gate_res_fp8(inp["x"], z, inp["residual"], z,
                                             z, EPS, oracle.Q_TOKEN, 0.0, dt)
    ro2, q2, s2 = oracle.resid_rmsnorm_fp8(z, inp["residual"], None,
                                           oracle.W_NONE, EPS, oracle.Q_TOKEN,
                                           0.0, dt)
    assert np.array_equal(ro1, ro2) and np.array_equal(q1, q2)
    assert np.array_equal(s1, s2)


@pytest.mark.parametrize("style", [oracle.ROPE_HALF, oracle.ROPE_INTERLEAVED])
def test_qkv_op_composes_pinned_pieces(style):
    dt = oracle.BF16
    T, Hq, Hkv, D, P, pages = 5, 4, 2, 32, 4, 6
    inp = workloads.qkv_inputs(T, Hq, Hkv, D, dt, seed=22, page_size=P,
                               num_pages=pages,
                               positions=np.array([0, 3, 4, 9, 22]))
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    q_out, err = oracle.qkv_normrope_kvwrite(
        inp["qkv"], inp["q_norm_w"], inp["k_norm_w"], EPS, inp["positions"],
        1e6, style, kc, vc, inp["page_table"], P, Hq, Hkv, D, dt)
    assert err == 0
    qkv = _dec(inp["qkv"], dt).reshape(T, Hq + 2 * Hkv, D)
    qw, kw = _dec(inp["q_norm_w"], dt), _dec(inp["k_norm_w"], dt)
    touched = set()
    for t in range(T):
        pos = int(inp["positions"][t])
        slot = oracle.kv_slot(pos, inp["page_table"], P, pages)
        pg, off = divmod(slot, P)
        touched.add((pg, off))
        for h in range(Hq + Hkv):
            w = qw if h < Hq else kw
            y = oracle.rope(oracle.rmsnorm(qkv[t, h], w, oracle.W_MUL, EPS),
                            pos, 1e6, style)
            want = oracle.encode16_n(y, dt)
            got = q_out[t, h] if h < Hq else kc[pg, off, h - Hq]
            assert np.array_equal(got, want)
        for g in range(Hkv):
            assert np.array_equal(
                vc[pg, off, g],
                inp["qkv"][t].reshape(Hq + 2 * Hkv, D)[Hq + Hkv + g])
    for pg in range(pages):
        for off in range(P):
            if (pg, off) not in touched:
                assert np.all(kc[pg, off] == workloads.SENTINEL)
                assert np.all(vc[pg, off] == workloads.SENTINEL)


def test_qkv_op_without_norm_and_out_of_range_positions():
    dt = oracle.F16
    T, Hq, Hkv, D, P, pages = 4, 2, 1, 16, 4, 2
    inp = workloads.qkv_inputs(T, Hq, Hkv, D, dt, seed=23, page_size=P,
                               num_pages=pages, norm=False,
                               positions=np.array([1, -1, 8, 5]))
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    q_out, err = oracle.qkv_normrope_kvwrite(
        inp["qkv"], None, None, EPS, inp["positions"], 1e4,
        oracle.ROPE_HALF, kc, vc, inp["page_table"], P, Hq, Hkv, D, dt)
    assert err == 1
    qkv = _dec(inp["qkv"], dt).reshape(T, Hq + 2 * Hkv, D)
    for t in range(T):
        for h in range(Hq):
            y = oracle.rope(qkv[t, h], int(inp["positions"][t]), 1e4)
            assert np.array_equal(q_out[t, h], oracle.encode16_n(y, dt))
    # only positions 1 and 5 were in range (2 pages of 4 slots)
    written = (kc != workloads.SENTINEL).any(axis=(2, 3))
    assert written.sum() == 2


def test_qkv_op_q_prescale():
    """Q pre-scale folded into RoPE ([HY] 04 step 10): Q only, K/V untouched;
    a power-of-two scale commutes with rounding (exact); any scale gives the
    correctly rounded s * y of the pinned composition."""
    dt = oracle.BF16
    T, Hq, Hkv, D, P, pages = 6, 4, 2, 64, 4, 4
    inp = workloads.qkv_inputs(T, Hq, Hkv, D, dt, seed=24, page_size=P,
                               num_pages=pages)
    outs = {}
    for qs in (1.0, 0.25, 64 ** -0.5):
        kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
        q_out, _ = oracle.qkv_normrope_kvwrite(
            inp["qkv"], inp["q_norm_w"], inp["k_norm_w"], EPS,
            inp["positions"], 1e6, oracle.ROPE_HALF, kc, vc,
            inp["page_table"], P, Hq, Hkv, D, dt, q_scale=qs)
        outs[qs] = (q_out, kc, vc)
    base = outs[1.0]
    for qs in (0.25, 64 ** -0.5):
        assert np.array_equal(outs[qs][1], base[1])
        assert np.array_equal(outs[qs][2], base[2])
    # power of two: exactly a quarter of the unscaled values (no subnormals here)
    assert np.array_equal(_dec(outs[0.25][0], dt), 0.25 * _dec(base[0], dt))
    # general scale: the correctly rounded product of the float64 composition
    qkv = _dec(inp["qkv"], dt).reshape(T, Hq + 2 * Hkv, D)
    qw = _dec(inp["q_norm_w"], dt)
    s = 64 ** -0.5
    got = _dec(outs[s][0], dt)
    for t in range(T):
        for h in range(Hq):
            y = s * oracle.rope(oracle.rmsnorm(qkv[t, h], qw, oracle.W_MUL, EPS),
                                int(inp["positions"][t]), 1e6)
            mag = outs[s][0][t, h] & 0x7FFF               # spacing above |got|
            ulp = _dec(mag + 1, dt) - _dec(mag, dt)
            assert np.all(np.abs(got[t, h] - y) <= 0.5 * ulp)


@pytest.mark.parametrize("kind", [oracle.ACT_SWIGLU, oracle.ACT_GEGLU_TANH,
                                  oracle.ACT_SQRELU])
def test_gated_act_block_worked_example(kind):
    # g = [1, -1, 2, 0], u = 1, rest of the 128-block zero
    g = np.zeros(128)
    g[:4] = [1, -1, 2, 0]
    u = np.zeros(128)
    u[:4] = 1
    gu = np.empty(256)
    gu[0::2], gu[1::2] = g, u
    bits = workloads.to16(gu[None, :], workloads.BF16)
    q, s = oracle.gated_act_fp8(bits, kind, oracle.BF16)
    want = {
        oracle.ACT_SWIGLU: ([0x74, 0xE9, 0x7E, 0x00], 1.7615941559557649 / 448),
        oracle.ACT_GEGLU_TANH: ([0x74, 0xE1, 0x7E, 0x00], 1.9545976940871754 / 448),
        oracle.ACT_SQRELU: ([0x6E, 0x00, 0x7E, 0x00], 4.0 / 448),
    }[kind]
    assert list(q[0, :4]) == want[0]
    assert not q[0, 4:].any()
    assert s[0, 0] == np.float32(want[1])


def test_gated_act_op_blocks_and_interleave():
    dt = oracle.BF16
    T, I = 3, 384
    inp = workloads.gated_act_inputs(T, I, dt, seed=24)
    q, s = oracle.gated_act_fp8(inp["gate_up"], oracle.ACT_SWIGLU, dt)
    gu = _dec(inp["gate_up"], dt)
    for t in range(T):
        g, u = gu[t, 0::2], gu[t, 1::2]
        h = np.array([oracle.act(a, oracle.ACT_SWIGLU) for a in g]) * u
        for b in range(I // 128):
            qq, ss = oracle.quant_dynamic(h[b * 128:(b + 1) * 128])
            assert np.array_equal(q[t, b * 128:(b + 1) * 128], qq)
            assert s[t, b] == ss
    # u = 0 gives zero codes (+0 or -0: act(g) * +0 keeps act(g)'s sign)
    z = inp["gate_up"].copy()
    z[:, 1::2] = 0
    qz, _ = oracle.gated_act_fp8(z, oracle.ACT_GEGLU_TANH, dt)
    assert not (qz & 0x7F).any()
