"""Pins for the oracle's Q/K norm + RoPE variants: LayerNorm, 3D RoPE, and
the general packed-QKV op over norm kind, norm scope and RoPE layout (CPU
only)."""
import numpy as np
import pytest
import torch

import oracle
import workloads

EPS = 1e-6


def test_layernorm_matches_torch_and_worked_values():
    rng = np.random.default_rng(31)
    v = rng.standard_normal(96) * 3 + 1.5
    w = rng.standard_normal(96)
    b = rng.standard_normal(96)
    want = torch.nn.functional.layer_norm(torch.from_numpy(v), (96,), torch.from_numpy(w),
                                          torch.from_numpy(b), EPS).numpy()
    assert np.allclose(oracle.layernorm(v, w, b, EPS), want, rtol=1e-13, atol=1e-13)
    y = oracle.layernorm(np.array([1.0, 2.0, 3.0, 4.0]), eps=EPS)
    r = 1.0 / np.sqrt(1.25 + EPS)
    assert np.allclose(y, np.array([-1.5, -0.5, 0.5, 1.5]) * r, rtol=1e-15)


def test_layernorm_invariants():
    rng = np.random.default_rng(32)
    v = rng.standard_normal(200)
    y = oracle.layernorm(v, eps=0.0)
    assert abs(y.mean()) < 1e-14 and abs(y.var() - 1.0) < 1e-13
    assert np.allclose(oracle.layernorm(v + 7.25, eps=EPS), oracle.layernorm(v, eps=EPS),
                       rtol=1e-11, atol=1e-12)


def test_rope3d_reduces_to_1d_and_keeps_axes_apart():
    rng = np.random.default_rng(33)
    D = 96
    v = rng.standard_normal(D)
    for style in (oracle.ROPE_HALF, oracle.ROPE_INTERLEAVED):
        got = oracle.rope3d(v, [37, 5, 9], [D // 2, 0, 0], 1e4, style)
        assert np.array_equal(got, oracle.rope(v, 37, 1e4, style))
        assert np.array_equal(oracle.rope3d(v, [0, 0, 0], [16, 16, 16], 1e4, style), v)
    sec = [16, 16, 16]
    a = oracle.rope3d(v, [3, 4, 5], sec, 1e4)
    b = oracle.rope3d(v, [3, 11, 5], sec, 1e4)
    pairs = lambda x: np.stack([x[:D // 2], x[D // 2:]], axis=1)   # rotate-half pairs
    same = np.all(pairs(a) == pairs(b), axis=1)
    assert same[:16].all() and not same[16:32].any() and same[32:].all()
    assert np.allclose(np.linalg.norm(pairs(a), axis=1), np.linalg.norm(pairs(v), axis=1),
                       rtol=1e-14)


def test_rope3d_relative_position():
    rng = np.random.default_rng(34)
    D, sec = 64, [12, 10, 10]
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    p, p2 = np.array([5, 17, 2]), np.array([9, 3, 30])
    for style in (oracle.ROPE_HALF, oracle.ROPE_INTERLEAVED):
        lhs = oracle.rope3d(q, p, sec, 1e4, style) @ oracle.rope3d(k, p2, sec, 1e4, style)
        rhs = q @ oracle.rope3d(k, p2 - p, sec, 1e4, style)
        assert abs(lhs - rhs) < 1e-12 * (np.abs(q).sum() * np.abs(k).sum())


def _inputs(T, Hq, Hkv, D, dt, seed):
    rng = np.random.default_rng(seed)
    qkv = workloads.to16(rng.standard_normal((T, (Hq + 2 * Hkv) * D), dtype=np.float32), dt)
    return rng, qkv


def test_rms_head_1d_equals_the_paged_op():
    T, Hq, Hkv, D, dt = 5, 4, 2, 64, oracle.BF16
    inp = workloads.qkv_inputs(T, Hq, Hkv, D, dt, seed=35, page_size=8, num_pages=1,
                               random_pages=False)
    q, k, v = oracle.qk_norm_rope(inp["qkv"], oracle.NORM_RMS, oracle.SCOPE_HEAD,
                                  inp["q_norm_w"], None, inp["k_norm_w"], None, EPS,
                                  inp["positions"], 1, None, 1e6, oracle.ROPE_HALF, 0.5,
                                  Hq, Hkv, D, dt)
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    q2, _ = oracle.qkv_normrope_kvwrite(inp["qkv"], inp["q_norm_w"], inp["k_norm_w"], EPS,
                                        inp["positions"], 1e6, oracle.ROPE_HALF, kc, vc,
                                        inp["page_table"], 8, Hq, Hkv, D, dt, q_scale=0.5)
    assert np.array_equal(q, q2)
    assert np.array_equal(k, kc[0, :T]) and np.array_equal(v, vc[0, :T])


@pytest.mark.parametrize("kind,scope,dims", [
    (oracle.NORM_LAYER, oracle.SCOPE_HEAD, 1),
    (oracle.NORM_RMS, oracle.SCOPE_FULL, 3),
    (oracle.NORM_LAYER, oracle.SCOPE_FULL, 3),
    (oracle.NORM_NONE, oracle.SCOPE_HEAD, 3),
])
def test_op_composes_pinned_pieces(kind, scope, dims):
    T, Hq, Hkv, D, dt = 3, 3, 2, 32, oracle.F16
    rng, qkv = _inputs(T, Hq, Hkv, D, dt, 36 + kind + 3 * scope + dims)
    wq, wk = (Hq * D, Hkv * D) if scope == oracle.SCOPE_FULL else (D, D)
    mk = lambda n, m: workloads.to16(m + 0.1 * rng.standard_normal(n).astype(np.float32), dt)
    qw, qb, kw, kb = mk(wq, 1.0), mk(wq, 0.0), mk(wk, 1.0), mk(wk, 0.0)
    if dims == 3:
        pos = rng.integers(0, 50, (T, 3)).astype(np.int32)
        sec = np.array([6, 5, 5], np.int32)
    else:
        pos = np.arange(T, dtype=np.int32) + 11
        sec = None
    q, k, v = oracle.qk_norm_rope(qkv, kind, scope, qw, qb, kw, kb, EPS, pos, dims, sec,
                                  1e4, oracle.ROPE_INTERLEAVED, 1.0, Hq, Hkv, D, dt)
    dec = lambda a: oracle.decode16(a, dt)
    for t in range(T):
        row = dec(qkv[t])
        for part, H0, H, w, b, out in ((0, 0, Hq, qw, qb, q), (1, Hq, Hkv, kw, kb, k)):
            x = row[H0 * D:(H0 + H) * D]
            if kind == oracle.NORM_NONE:
                y = x.copy()
            elif scope == oracle.SCOPE_FULL:
                y = (oracle.rmsnorm(x, dec(w), oracle.W_MUL, EPS) if kind == oracle.NORM_RMS
                     else oracle.layernorm(x, dec(w), dec(b), EPS))
            else:
                y = np.concatenate([
                    oracle.rmsnorm(x[h * D:(h + 1) * D], dec(w), oracle.W_MUL, EPS)
                    if kind == oracle.NORM_RMS else
                    oracle.layernorm(x[h * D:(h + 1) * D], dec(w), dec(b), EPS)
                    for h in range(H)])
            for h in range(H):
                yh = y[h * D:(h + 1) * D]
                r = (oracle.rope3d(yh, pos[t], sec, 1e4, oracle.ROPE_INTERLEAVED) if dims == 3
                     else oracle.rope(yh, int(pos[t]), 1e4, oracle.ROPE_INTERLEAVED))
                assert np.array_equal(out[t, h], oracle.encode16_n(r, dt))
        assert np.array_equal(v[t].reshape(-1), qkv[t, (Hq + Hkv) * D:])


@pytest.mark.parametrize("out_kind,qmode", [(0, oracle.Q_STATIC), (0, oracle.Q_TOKEN), (1, 0)])
def test_resid_layernorm_composes_pinned_pieces(out_kind, qmode):
    dt = oracle.BF16
    T, H = 3, 256
    inp = workloads.resid_rmsnorm_inputs(T, H, dt, seed=40, outliers=True)
    rng = np.random.default_rng(41)
    bias = workloads.to16(0.1 * rng.standard_normal(H).astype(np.float32), dt)
    ro, q, sc = oracle.resid_layernorm(inp["x"], inp["residual"], inp["weight"], bias, EPS,
                                       out_kind, qmode, 56.0, dt)
    ro8, _, _ = oracle.resid_rmsnorm_fp8(inp["x"], inp["residual"], None, oracle.W_NONE,
                                         EPS, oracle.Q_STATIC, 1.0, dt)
    assert np.array_equal(ro, ro8)
    w, b = oracle.decode16(inp["weight"], dt), oracle.decode16(bias, dt)
    for t in range(T):
        y = oracle.layernorm(oracle.decode16(ro[t], dt), w, b, EPS)
        if out_kind == 1:
            pw, sw = oracle.quant_mxfp4(y)
            assert np.array_equal(q[t], pw) and np.array_equal(sc[t], sw)
        elif qmode == oracle.Q_STATIC:
            assert np.array_equal(q[t], oracle.e4m3_encode_n(y * 56.0))
        else:
            s = np.float32(max(np.abs(y).max(), np.float32(1e-10)) / 448.0)
            assert sc[t] == s
            assert np.array_equal(q[t], oracle.e4m3_encode_n(y / np.float64(s)))


@pytest.mark.parametrize("with_bias,g", [(True, 3.7e-2), (False, 2.5e-4), (True, 400.0)])
def test_resid_layernorm_nvfp4_composes_pinned_pieces(with_bias, g):
    """Add + LayerNorm -> NVFP4 is the pinned NVFP4 quantiser applied to the
    pinned LayerNorm of the same new residual as the FP8 producer; the tensor
    scales include one that saturates block scales (2.5e-4) and one that
    sends most blocks' scales to zero (400)."""
    dt = oracle.BF16
    T, H = 3, 256
    inp = workloads.resid_rmsnorm_inputs(T, H, dt, seed=42, outliers=True)
    rng = np.random.default_rng(43)
    bias = workloads.to16(0.1 * rng.standard_normal(H).astype(np.float32), dt) if with_bias else None
    ro, q, sc = oracle.resid_layernorm_nvfp4(inp["x"], inp["residual"], inp["weight"], bias,
                                             EPS, g, dt)
    ro8, _, _ = oracle.resid_rmsnorm_fp8(inp["x"], inp["residual"], None, oracle.W_NONE,
                                         EPS, oracle.Q_STATIC, 1.0, dt)
    assert np.array_equal(ro, ro8)
    w = oracle.decode16(inp["weight"], dt)
    b = oracle.decode16(bias, dt) if with_bias else np.zeros(H)
    for t in range(T):
        y = oracle.layernorm(oracle.decode16(ro[t], dt), w, b, EPS)
        pw, sw = oracle.quant_nvfp4(y, g)
        assert np.array_equal(q[t], pw) and np.array_equal(sc[t], sw)
