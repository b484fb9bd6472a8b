"""GPU parity of the FP8 gate_up GEMM fused with the gated activation and
block-128 FP8 output, against the oracle (dequantise, float64 matmul,
activation, block quantisation) on the same seeded codes and scales.

Acceptance (derived from the arithmetic; the matrix instruction's own error
is measured by test_mfma_block_error_bound below).  The kernel forms each
128-wide K block's partial sum p_b with two e4m3 matrix instructions
(v_mfma_scale_f32_32x32x64_f8f6f4) starting from zero, then folds
acc = fma(p_b, a_s * w_s, acc) in fp32.  The products of e4m3 codes are
exact, but the instruction does not add them exactly: its error on one
block is bounded by C_MFMA times the block's largest product magnitude,
|p_b - P_b| <= C_MFMA * max_k |a_k w_k|, with C_MFMA = 2^-10 (the probe
test asserts it on six operand classes; the largest ratio seen on MI355X is
2^-10.7).  Relative to the sum of magnitudes the same error is 2^-15 on the
GEMM's N(0,1)-shaped codes but 2^-12 on codes of wide dynamic range, so a
bound in the sum of magnitudes would depend on the data; the maximum-based
one does not.  Bounding each block's largest product by the product of the
two operands' block maxima (amax_b, wmax_b, dequantised), and adding the
fp32 fold (the scale product and one fma per block, 2^-24 each, against the
running sum <= S = sum_k |A_k W_k|), every accumulator lies within
  E_acc = C_MFMA * sum_b amax_b(m) wmax_b(n) + (K/128 + 2) 2^-24 S(m, n)
of the exact dequantised sum.  With g, u the oracle's exact gate and up
values and dg, du their E_acc:
  E_h = |act'|max * dg * (|u| + du) + (|act(g)| + |act'|max * dg) * du,
  |act'| <= 1.2 for SiLU and GELU-tanh, 2 (|g| + dg) for ReLU^2.
Every GPU code must lie in the e4m3 code interval of (h_o -+ E_h) / s_gpu,
and every GPU scale within max_block(E_h) / 448 (+ 4 ulp) of the oracle's.
So the fp8 rule of the element-wise ops (>= 99.9% identical codes, scales
within 1e-6) is replaced here by this interval rule: where the interval
holds one code the GPU code must be that code; the identical fraction and
the fraction of codes whose interval holds a single code are reported."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import announce, check_fp8, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fr():
    import memory_bound_amd
    return memory_bound_amd


C_MFMA = 2.0 ** -10          # per 128-wide K block, times the largest |product|


def _act(g, act):
    if act == oracle.ACT_SWIGLU:
        return g / (1.0 + np.exp(-g))
    if act == oracle.ACT_GEGLU_TANH:
        return 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3)))
    return np.maximum(g, 0.0) ** 2


def _ord(c):
    c = c.astype(np.int32)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def accumulator_bound(inp):
    """E_acc of every output (see the module docstring): [M, 2I] float64."""
    tab = oracle.e4m3_table()
    a, w = inp["a"], inp["w"]
    M, K = a.shape
    N = w.shape[0]
    KB = K // 128
    amax = np.abs(tab[a]).reshape(M, KB, 128).max(axis=2) * inp["a_scales"]
    wmax = np.abs(tab[w]).reshape(N, KB, 128).max(axis=2) \
        * np.repeat(inp["w_scales"].astype(np.float64), 128, axis=0)
    A = oracle.dequant_blocks(a, inp["a_scales"], 1)
    W = oracle.dequant_blocks(w, inp["w_scales"], 128)
    S = np.abs(A) @ np.abs(W).T
    return C_MFMA * (amax @ wmax.T) + (KB + 2) * 2.0 ** -24 * S, A @ W.T


def check_gemm_interval(q_g, s_g, q_o, s_o, inp, act):
    """Interval parity (see the module docstring); returns (identical
    fraction, fraction of single-code intervals, max scale relative
    error)."""
    E_acc, acc = accumulator_bound(inp)
    g, u = acc[:, 0::2], acc[:, 1::2]
    dg, du = E_acc[:, 0::2], E_acc[:, 1::2]
    h = _act(g, act) * u
    dmax = 2.0 * (np.abs(g) + dg) if act == oracle.ACT_SQRELU else 1.2
    E = dmax * dg * (np.abs(u) + du) + (np.abs(_act(g, act)) + dmax * dg) * du
    M, I = h.shape
    s_g64 = s_g.astype(np.float64)
    assert np.all(np.isfinite(s_g64)) and np.all(s_g64 > 0), "unwritten scales"
    # scales: the block maximum moves by at most max(E) over the block
    Eb = E.reshape(M, I // 128, 128).max(axis=2)
    ulp = np.spacing(s_o.astype(np.float32)).astype(np.float64)
    bad = np.abs(s_g64 - s_o) > Eb / 448.0 * 1.001 + 4 * ulp
    assert not bad.any(), f"{bad.sum()} scales outside their bound"
    # codes: inside the rounding interval of the perturbed exact value
    sfull = np.repeat(s_g64, 128, axis=1)
    lo = oracle.e4m3_encode_n((h - E) / sfull).reshape(M, I)
    hi = oracle.e4m3_encode_n((h + E) / sfull).reshape(M, I)
    og = _ord(q_g)
    nan = (q_g & 0x7F) == 0x7F
    assert not nan.any(), f"{nan.sum()} NaN / unwritten codes"
    out = (og < _ord(lo)) | (og > _ord(hi))
    if out.any():
        i = np.argwhere(out)[0]
        raise AssertionError(f"{out.sum()} codes outside their interval; first {tuple(i)}: "
                             f"got {q_g[tuple(i)]:#04x} interval [{lo[tuple(i)]:#04x}, "
                             f"{hi[tuple(i)]:#04x}] oracle {q_o[tuple(i)]:#04x}")
    same = lambda x, y: (x == y) | (((x | y) & 0x7F) == 0)       # +-0 identified
    ident = float(np.mean(same(q_g, q_o)))
    single = float(np.mean(same(lo, hi)))
    return ident, single, float((np.abs(s_g64 - s_o) / s_o).max())


# ---------------------------------------------------------------------------
# The matrix instruction's accumulation error, measured against exact sums
# ---------------------------------------------------------------------------

def _probe_tiles(kind, n, rng):
    """n operand tile pairs [n, 32, 128] of e4m3 codes of one class."""
    shape = (n, 32, 128)
    if kind == "workload":            # the GEMM inputs' class: N(0,1) x 32
        draw = lambda: workloads.e4m3_codes(workloads.normal(rng, shape) * np.float32(32.0))
    elif kind == "positive":          # no cancellation
        draw = lambda: workloads.e4m3_codes(np.abs(workloads.normal(rng, shape)) * np.float32(32.0))
    elif kind == "uniform_codes":     # every finite code equally likely
        fin = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
        draw = lambda: fin[rng.integers(0, fin.size, shape)]
    elif kind == "log_uniform":       # magnitudes 2^-9 .. 2^8.8, random signs
        def draw():
            mag = np.exp2(rng.uniform(-9.0, 8.8, shape)).astype(np.float32)
            sign = np.where(rng.random(shape) < 0.5, -1.0, 1.0).astype(np.float32)
            return workloads.e4m3_codes(mag * sign)
    elif kind == "dominant":          # one large product among small ones
        def draw():
            c = workloads.e4m3_codes(workloads.normal(rng, shape) * np.float32(0.01))
            c[:, :, 5] = 0x7E
            return c
    else:                             # small integers: every sum exact in fp32
        vals = np.array([0x00, 0x38, 0x40, 0x48, 0xB8, 0xC0, 0xC8], dtype=np.uint8)
        draw = lambda: vals[rng.integers(0, vals.size, shape)]
    return draw(), draw()


def _probe(x, y, ninstr):
    import gpu_support
    lib = gpu_support.load()
    n = x.shape[0]
    xd, yd = to_dev(x), to_dev(y)
    out = torch.full((n, 32, 32), float("nan"), dtype=torch.float32, device="cuda")
    assert lib.mfma_probe_e4m3(xd.data_ptr(), yd.data_ptr(), out.data_ptr(), n, ninstr,
                               None) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kind", ["workload", "positive", "uniform_codes", "log_uniform",
                                  "dominant", "small_int"])
def test_mfma_block_error_bound(kind):
    """One 128-wide K block of the GEMM (two chained instructions from a
    zero accumulator) and one instruction alone: |hardware - exact| <=
    C_MFMA * max_k |x_k y_k| for every output of 1024 tiles; small-integer
    operands (all partial sums exact in fp32) must give exact sums, which
    also pins the probe's lane layout."""
    n = 1024
    announce(f"mfma block error bound, class {kind}, {n} tiles")
    rng = np.random.default_rng(["workload", "positive", "uniform_codes", "log_uniform",
                                 "dominant", "small_int"].index(kind) + 9100)
    x, y = _probe_tiles(kind, n, rng)
    tab = oracle.e4m3_table()
    for ninstr in (2, 1):
        K = 64 * ninstr
        X, Y = tab[x[:, :, :K]], tab[y[:, :, :K]]
        exact = np.einsum("nik,njk->nij", X, Y)          # exact: <= 51 significant bits
        mx = np.concatenate([np.max(np.abs(X[i:i + 64])[:, :, None, :]
                                    * np.abs(Y[i:i + 64])[:, None, :, :], axis=3)
                             for i in range(0, n, 64)])
        err = np.abs(_probe(x, y, ninstr) - exact)
        assert np.all(np.isfinite(err)), "unwritten probe outputs"
        if kind == "small_int":
            assert np.all(err == 0.0), f"{np.sum(err != 0)} inexact small-integer sums"
            continue
        ratio = float(np.max(err / mx))
        announce(f"  {ninstr} instruction(s): max |err| / max|product| = 2^{np.log2(ratio):.2f}")
        assert ratio <= C_MFMA, f"block error 2^{np.log2(ratio):.2f} above the bound"


def pack_reference(w):
    """The packed weight layout, written out from its definition in the
    library header: unit u = ((G * KB + kb) * 4 + c) * 64 + lane holds
    w[32 G + lane % 32, 128 kb + off : +16] with
    off = 64 (c // 2) + 32 (lane // 32) + 16 (c % 2)."""
    N, K = w.shape
    G, kb, c, lane = np.meshgrid(np.arange(N // 32), np.arange(K // 128),
                                 np.arange(4), np.arange(64), indexing="ij")
    row = 32 * G + lane % 32
    col = 128 * kb + 64 * (c // 2) + 32 * (lane // 32) + 16 * (c % 2)
    idx = (row * K + col)[..., None] + np.arange(16)
    return np.ascontiguousarray(w).reshape(-1)[idx.reshape(-1)]


def pack_dev(fr, w):
    N, K = w.shape
    wp = torch.full((N * K,), 0x7F, dtype=torch.uint8, device="cuda")
    fr.fr_gemm_pack_weights(to_dev(w), wp, N, K)
    return wp


def run_gemm(fr, inp, act):
    M, K = inp["a"].shape
    I = inp["w"].shape[0] // 2
    q = torch.full((M, I), 0x7F, dtype=torch.uint8, device="cuda")
    sc = torch.full((M, I // 128), float("nan"), dtype=torch.float32, device="cuda")
    wp = pack_dev(fr, inp["w"])
    fr.fr_gemm_gated_act_fp8(to_dev(inp["a"]), to_dev(inp["a_scales"]),
                             wp, to_dev(inp["w_scales"]), act, q, sc, M, K, I)
    torch.cuda.synchronize()
    return to_host(q, np.uint8), to_host(sc, np.float32)


@pytest.mark.parametrize("N,K", [(32, 128), (64, 384), (12288, 2048)])
def test_pack_weights_layout(fr, N, K):
    announce(f"gemm pack weights N={N} K={K}")
    rng = np.random.default_rng(N + K)
    w = rng.integers(0, 256, (N, K), dtype=np.uint8)
    got = to_host(pack_dev(fr, w), np.uint8)
    assert np.array_equal(got, pack_reference(w))


GEMM_CASES = [
    # (M, K, I, act, seed)
    (1, 128, 128, oracle.ACT_SWIGLU, 701),
    (37, 256, 384, oracle.ACT_GEGLU_TANH, 702),          # ragged M, several tiles
    (64, 2048, 256, oracle.ACT_SQRELU, 703),
    (128, 2048, 6144, oracle.ACT_SWIGLU, 704),           # 2B gate_up, S=128
    (192, 2048, 6144, oracle.ACT_SWIGLU, 705),           # 2B gate_up, S=192
    (192, 2048, 6144, oracle.ACT_GEGLU_TANH, 705),
    (128, 4096, 12288, oracle.ACT_SWIGLU, 706),          # 8B gate_up, S=128
    (390, 2048, 6144, oracle.ACT_SWIGLU, 708),           # 128-row tiles (one round), ragged
    (1000, 2048, 6144, oracle.ACT_SQRELU, 709),          # 64-row tiles (768), ragged
    (1024, 4096, 6144, oracle.ACT_SWIGLU, 710),          # 64-row tiles, K = 4096
    (96, 16384, 256, oracle.ACT_SWIGLU, 711),            # largest K
    (100, 256, 17920, oracle.ACT_GEGLU_TANH, 712),       # 128-row tile with M < 128 (140 tiles)
    (33, 512, 2048, oracle.ACT_SQRELU, 713),             # one row past a 32-row tile
    (250, 1024, 1024, oracle.ACT_GEGLU_TANH, 714),       # ragged 64-row tiles
    (129, 128, 16384, oracle.ACT_SWIGLU, 715),           # 128 output blocks, ragged
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: f"M{c[0]}_K{c[1]}_I{c[2]}_act{c[3]}")
def test_gemm_gated_act(fr, case):
    M, K, I, act, seed = case
    announce(f"gemm_gated_act M={M} K={K} I={I} act={act} seed={seed}")
    inp = workloads.gemm_inputs(M, K, I, seed)
    q_g, s_g = run_gemm(fr, inp, act)
    q_o, s_o, _ = oracle.gemm_gated_act_fp8(inp["a"], inp["a_scales"], inp["w"],
                                            inp["w_scales"], act)
    ident, single, rel = check_gemm_interval(q_g, s_g, q_o, s_o, inp, act)
    announce(f"  fp8 identical {ident:.6f} (single-code intervals {single:.6f}), "
             f"scale max rel err {rel:.2e}")


def test_gemm_bench_shapes(fr):
    """The two larger shapes the benchmark times, in its launch configuration:
    1024 x 2048 x 6144 in full, 4096 x 4096 x 12288 on 16 sampled rows (rows
    are independent, so the oracle runs on those rows only)."""
    announce("gemm_gated_act bench shape M=1024 K=2048 I=6144")
    inp = workloads.gemm_inputs(1024, 2048, 6144, 1824)
    q_g, s_g = run_gemm(fr, inp, oracle.ACT_SWIGLU)
    q_o, s_o, _ = oracle.gemm_gated_act_fp8(inp["a"], inp["a_scales"], inp["w"],
                                            inp["w_scales"], oracle.ACT_SWIGLU)
    check_gemm_interval(q_g, s_g, q_o, s_o, inp, oracle.ACT_SWIGLU)

    M, K, I = 4096, 4096, 12288
    announce(f"gemm_gated_act bench shape M={M} K={K} I={I}, 16 sampled rows")
    inp = workloads.gemm_inputs(M, K, I, 4896)
    q_g, s_g = run_gemm(fr, inp, oracle.ACT_SWIGLU)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 2047, M - 2, M - 1],
                                     np.random.default_rng(4896).integers(0, M, 9)]))
    sub = {"a": inp["a"][rows], "a_scales": inp["a_scales"][rows],
           "w": inp["w"], "w_scales": inp["w_scales"]}
    q_o, s_o, _ = oracle.gemm_gated_act_fp8(sub["a"], sub["a_scales"], sub["w"],
                                            sub["w_scales"], oracle.ACT_SWIGLU)
    ident, single, rel = check_gemm_interval(q_g[rows], s_g[rows], q_o, s_o, sub,
                                             oracle.ACT_SWIGLU)
    announce(f"  sampled rows {len(rows)}: fp8 identical {ident:.6f} (single-code "
             f"{single:.6f}), scale max rel err {rel:.2e}")


def test_gemm_large_batch_tile_ragged(fr):
    """The 128-row, 8-wave tile (taken at >= 768 tiles of 128 rows) with a
    ragged last row tile: M = 2000 = 15 x 128 + 80, checked on sampled rows
    (rows are independent) including both sides of every tile edge."""
    M, K, I = 2000, 512, 6144
    announce(f"gemm_gated_act large-batch tile M={M} K={K} I={I}, sampled rows")
    inp = workloads.gemm_inputs(M, K, I, 2000)
    for act in (oracle.ACT_SWIGLU, oracle.ACT_GEGLU_TANH, oracle.ACT_SQRELU):
        q_g, s_g = run_gemm(fr, inp, act)
        rows = np.unique(np.concatenate([[0, 1, 31, 32, 63, 64, 127, 128, 1919, 1920,
                                          1951, 1952, M - 2, M - 1],
                                         np.random.default_rng(2000).integers(0, M, 10)]))
        sub = {"a": inp["a"][rows], "a_scales": inp["a_scales"][rows],
               "w": inp["w"], "w_scales": inp["w_scales"]}
        q_o, s_o, _ = oracle.gemm_gated_act_fp8(sub["a"], sub["a_scales"], sub["w"],
                                                sub["w_scales"], act)
        ident, single, rel = check_gemm_interval(q_g[rows], s_g[rows], q_o, s_o, sub, act)
        announce(f"  act {act}: sampled rows {len(rows)}: fp8 identical {ident:.6f} "
                 f"(single-code {single:.6f})")


def test_gemm_worked_example(fr):
    announce("gemm worked example")
    K, I = 128, 128
    a = np.full((1, K), 0x38, dtype=np.uint8)
    w = np.zeros((2 * I, K), dtype=np.uint8)
    w[0::2, 0] = 0x38
    for j in range(I):
        w[2 * j + 1, : [1, 2, 4, 8][j % 4]] = 0x38
    inp = {"a": a, "a_scales": np.ones((1, 1), np.float32), "w": w,
           "w_scales": np.ones((2, 1), np.float32)}
    q, s = run_gemm(fr, inp, oracle.ACT_SWIGLU)
    assert list(q[0, :8]) == [0x66, 0x6E, 0x76, 0x7E] * 2


def test_gemm_determinism(fr):
    announce("gemm determinism x3")
    inp = workloads.gemm_inputs(96, 1024, 1024, 707)
    first = run_gemm(fr, inp, oracle.ACT_SWIGLU)
    for _ in range(2):
        again = run_gemm(fr, inp, oracle.ACT_SWIGLU)
        assert np.array_equal(first[0], again[0])
        assert np.array_equal(first[1].view(np.uint32), again[1].view(np.uint32))


def test_gemm_two_streams(fr):
    """Launches on two streams that overlap give the outputs of one launch at
    a time (the kernel keeps no state between launches)."""
    announce("gemm two streams, overlapping launches")
    M, K, I = 128, 1024, 4096
    inps = [workloads.gemm_inputs(M, K, I, 720 + i) for i in range(2)]
    refs = [run_gemm(fr, inp, oracle.ACT_SWIGLU) for inp in inps]
    bufs = []
    for inp in inps:
        bufs.append({
            "a": to_dev(inp["a"]), "a_s": to_dev(inp["a_scales"]),
            "w": pack_dev(fr, inp["w"]), "w_s": to_dev(inp["w_scales"]),
            "q": torch.full((M, I), 0x7F, dtype=torch.uint8, device="cuda"),
            "sc": torch.full((M, I // 128), float("nan"), dtype=torch.float32,
                             device="cuda")})
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(4):
        for b, st in zip(bufs, streams):
            fr.fr_gemm_gated_act_fp8(b["a"], b["a_s"], b["w"], b["w_s"], oracle.ACT_SWIGLU,
                                     b["q"], b["sc"], M, K, I, stream=st)
    torch.cuda.synchronize()
    for b, (q_r, s_r) in zip(bufs, refs):
        assert np.array_equal(to_host(b["q"], np.uint8), q_r)
        assert np.array_equal(to_host(b["sc"], np.float32).view(np.uint32), s_r.view(np.uint32))
