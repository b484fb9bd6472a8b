"""GPU parity: every fused op through the C ABI against the CPU oracle on the
same seeded inputs, at the pages' workload shapes (including the full
8192-token bandwidth shapes the benchmark times), ragged and edge shapes, and
every mode."""
import numpy as np
import pytest

import oracle
import workloads
from parity import (announce, check16, check_exact, check_fp8, check_scales,
                    run_adarms, run_gated_act, run_qkv, run_resid_rmsnorm)

pytestmark = pytest.mark.gpu

F16, BF16 = 0, 1
EPS = 1e-6


@pytest.fixture(scope="module")
def fr():
    import memory_bound_amd
    return memory_bound_amd


# ---------------------------------------------------------------------------
# (a) residual add + RMSNorm + FP8
# ---------------------------------------------------------------------------

RMS_CASES = [
    # (T, H, dtype, wmode, qmode, static_scale, outliers, seed)
    (10, 1024, F16, oracle.W_NONE, oracle.Q_STATIC, 56.0, False, 101),   # decode boundary
    (37, 1040, BF16, oracle.W_MUL, oracle.Q_TOKEN, 0.0, False, 201),      # ragged width
    (5, 16, F16, oracle.W_ONE_PLUS, oracle.Q_TOKEN, 0.0, False, 202),     # smallest width
    (3, 32768, BF16, oracle.W_MUL, oracle.Q_TOKEN, 0.0, True, 203),       # largest width
    (1, 4096, F16, oracle.W_ONE_PLUS, oracle.Q_STATIC, 56.0, False, 204),
    (3000, 4096, BF16, oracle.W_MUL, oracle.Q_TOKEN, 0.0, True, 205),     # bandwidth shape path
    (2049, 1040, F16, oracle.W_NONE, oracle.Q_TOKEN, 0.0, False, 206),
    (8192, 4096, BF16, oracle.W_MUL, oracle.Q_TOKEN, 0.0, True, 105),     # full bandwidth config
    (8192, 4096, BF16, oracle.W_NONE, oracle.Q_TOKEN, 0.0, True, 105),
    # bandwidth path with rows over several waves, each workgroup taking rows in
    # turn: (1 + w) weights with static scale, three waves per row
    (2304, 2048, F16, oracle.W_ONE_PLUS, oracle.Q_STATIC, 56.0, False, 210),
    (4100, 3072, BF16, oracle.W_ONE_PLUS, oracle.Q_TOKEN, 0.0, True, 211),
    (16, 256, F16, oracle.W_NONE, oracle.Q_STATIC, 1000.0, False, 207),   # saturating multiplier
    (16, 256, F16, oracle.W_NONE, oracle.Q_STATIC, 2.0 ** -8, False, 208),  # subnormal codes
]


@pytest.mark.parametrize("case", RMS_CASES, ids=lambda c: f"T{c[0]}_H{c[1]}_dt{c[2]}_w{c[3]}_q{c[4]}_s{c[5]}")
def test_resid_rmsnorm(fr, case):
    T, H, dt, wmode, qmode, s, outl, seed = case
    announce(f"resid_rmsnorm T={T} H={H} dtype={dt} wmode={wmode} qmode={qmode} seed={seed}")
    inp = workloads.resid_rmsnorm_inputs(T, H, dt, seed, outliers=outl)
    ro_g, q_g, sc_g = run_resid_rmsnorm(fr, inp, wmode, EPS, qmode, s, dt)
    ro_o, q_o, sc_o = oracle.resid_rmsnorm_fp8(
        inp["x"], inp["residual"], inp["weight"], wmode, EPS, qmode, s, dt)
    check_exact(ro_g, ro_o, "residual_out")
    ident = check_fp8(q_g, q_o, "out_fp8")
    announce(f"  fp8 identical fraction {ident:.7f}")
    if qmode == oracle.Q_TOKEN:
        check_scales(sc_g, sc_o, "out_scales")


@pytest.mark.parametrize("T,H,dt", [(64, 2048, F16), (2100, 4096, BF16)],
                         ids=["T64_H2048", "T2100_H4096_bandwidth"])
def test_resid_rmsnorm_in_place(fr, T, H, dt):
    announce(f"resid_rmsnorm in place T={T} H={H}")
    inp = workloads.resid_rmsnorm_inputs(T, H, dt, 209)
    ro_g, q_g, sc_g = run_resid_rmsnorm(fr, inp, oracle.W_MUL, EPS,
                                        oracle.Q_TOKEN, 0.0, dt, inplace=True)
    ro_o, q_o, sc_o = oracle.resid_rmsnorm_fp8(
        inp["x"], inp["residual"], inp["weight"], oracle.W_MUL, EPS,
        oracle.Q_TOKEN, 0.0, dt)
    check_exact(ro_g, ro_o, "residual_out (in place)")
    check_fp8(q_g, q_o, "out_fp8")
    check_scales(sc_g, sc_o, "out_scales")


def test_resid_rmsnorm_worked_example(fr):
    announce("resid_rmsnorm worked example")
    x = workloads.to16(np.array([[0.5, 1.0, 1.5, 2.0] * 4]), F16)
    inp = {"x": x, "residual": x.copy(), "weight": np.zeros(16, np.uint16)}
    ro, q, _ = run_resid_rmsnorm(fr, inp, oracle.W_NONE, EPS, oracle.Q_STATIC,
                                 56.0, F16)
    # the row [1,2,3,4]*4 has the same mean square (7.5) as [1,2,3,4]
    assert list(q[0, :4]) == [0x5A, 0x62, 0x67, 0x6A]
    _, q, s = run_resid_rmsnorm(fr, inp, oracle.W_NONE, EPS, oracle.Q_TOKEN,
                                0.0, F16)
    assert q[0, 0] == 0x6E and q[0, 1] == 0x76 and q[0, 3] == 0x7E
    assert q[0, 2] in (0x7A, 0x7B)
    assert abs(s[0] - 1.4605933893075536 / 448) <= 1e-6 * s[0]


# ---------------------------------------------------------------------------
# (a') gate + residual + AdaRMSNorm + FP8
# ---------------------------------------------------------------------------

ADA_CASES = [
    # (T, H, dtype, qmode, static_scale, seed)
    (10, 1024, F16, oracle.Q_STATIC, 56.0, 102),        # decode boundary
    (33, 1040, BF16, oracle.Q_TOKEN, 0.0, 301),         # ragged width
    (2, 16, F16, oracle.Q_TOKEN, 0.0, 302),
    (2500, 4096, BF16, oracle.Q_TOKEN, 0.0, 303),       # bandwidth shape path
    (8192, 1024, F16, oracle.Q_STATIC, 56.0, 102),      # bandwidth config
    (8192, 1024, F16, oracle.Q_TOKEN, 0.0, 102),
    (4, 20000, BF16, oracle.Q_TOKEN, 0.0, 304),         # wide row
    # bandwidth path (two single-wave rows per workgroup) with a ragged
    # width and an odd token count: the last workgroup's second row is a
    # duplicate that stores nothing
    (2049, 1040, F16, oracle.Q_TOKEN, 0.0, 305),
    (3001, 528, BF16, oracle.Q_STATIC, 56.0, 306),
]


@pytest.mark.parametrize("case", ADA_CASES, ids=lambda c: f"T{c[0]}_H{c[1]}_dt{c[2]}_q{c[3]}")
def test_adarms(fr, case):
    T, H, dt, qmode, s, seed = case
    announce(f"adarms T={T} H={H} dtype={dt} qmode={qmode} seed={seed}")
    inp = workloads.adarms_inputs(T, H, dt, seed)
    ro_g, q_g, sc_g = run_adarms(fr, inp, EPS, qmode, s, dt)
    ro_o, q_o, sc_o = oracle.adarms_gate_res_fp8(
        inp["x"], inp["gate"], inp["residual"], inp["ada_scale"],
        inp["ada_shift"], EPS, qmode, s, dt)
    check_exact(ro_g, ro_o, "residual_out")
    ident = check_fp8(q_g, q_o, "out_fp8")
    announce(f"  fp8 identical fraction {ident:.7f}")
    if qmode == oracle.Q_TOKEN:
        check_scales(sc_g, sc_o, "out_scales")


def test_adarms_in_place_and_reduction(fr):
    announce("adarms in place; gate = scale = shift = 0")
    inp = workloads.adarms_inputs(12, 1024, BF16, 305)
    z = np.zeros_like(inp["x"])
    zin = {"x": inp["x"], "gate": z, "residual": inp["residual"],
           "ada_scale": z, "ada_shift": z}
    ro_g, q_g, sc_g = run_adarms(fr, zin, EPS, oracle.Q_TOKEN, 0.0, BF16,
                                 inplace=True)
    ro_o, q_o, sc_o = oracle.resid_rmsnorm_fp8(
        z, inp["residual"], None, oracle.W_NONE, EPS, oracle.Q_TOKEN, 0.0, BF16)
    check_exact(ro_g, ro_o, "residual_out")
    check_fp8(q_g, q_o, "out_fp8")
    check_scales(sc_g, sc_o, "out_scales")


# ---------------------------------------------------------------------------
# (b) packed QKV split + Q/K RMSNorm + RoPE + paged KV write
# ---------------------------------------------------------------------------

QKV_CASES = [
    # (name, T, Hq, Hkv, D, dtype, norm, theta, style, P, pages, random_pages, positions, seed)
    ("prefill_qwen3", 128, 32, 8, 128, BF16, True, 1e6, 0, 16, 512, True, None, 103),
    ("decode_pi05", 10, 8, 1, 256, F16, False, 1e4, 0, 1024, 1, False,
     np.arange(790, 800), 102),
    ("interleaved", 20, 4, 2, 64, BF16, True, 1e4, 1, 8, 8, True, None, 401),
    ("d16", 9, 3, 1, 16, F16, True, 1e4, 0, 4, 4, True, None, 402),
    ("d32_interleaved", 9, 5, 1, 32, F16, True, 1e4, 1, 4, 4, True, None, 403),
    ("d96_padded_lanes", 11, 6, 2, 96, BF16, True, 1e6, 0, 4, 8, True, None, 404),
    ("d256_norm", 7, 2, 2, 256, BF16, True, 1e6, 1, 16, 1, False, None, 405),
    ("far_positions", 16, 4, 1, 128, BF16, True, 1e6, 0, 4096, 64, True,
     np.arange(200000, 200016), 406),
    # a small batch whose page-table indices reach past the 64 entries the
    # kernel holds in registers (indices 0..255 of a 256-entry table)
    ("long_page_table", 12, 4, 2, 64, BF16, True, 1e4, 0, 16, 256, True,
     np.array([3, 63 * 16 + 15, 64 * 16, 64 * 16 + 1, 100 * 16 + 7, 127 * 16 + 15,
               128 * 16, 200 * 16 + 3, 255 * 16 + 15, 17, 1000, 4000]), 409),
    ("bench_8192", 8192, 32, 8, 128, BF16, True, 1e6, 0, 16, 512, True, None, 103),
    # bandwidth regime, 80 heads = 10 groups of 8: the token's last wave
    # takes fewer groups than the others
    ("wide_heads_2048", 2048, 64, 8, 128, BF16, True, 1e6, 0, 16, 128, True, None, 410),
    # the bandwidth-regime kernel with interleaved RoPE pairs, fp16, D = 64
    ("interleaved_2048_f16", 2048, 8, 2, 64, F16, True, 1e4, 1, 16, 128, True, None, 413),
    # the bandwidth-regime kernel at D = 256 (16 lanes per head) and D = 16
    ("d256_2048", 2048, 8, 1, 256, BF16, True, 1e4, 0, 16, 128, True, None, 414),
    ("d16_2048_interleaved", 2048, 6, 2, 16, F16, True, 1e4, 1, 16, 128, True, None, 415),
]


def _check_cache(got, want, dt, what):
    written = want != workloads.SENTINEL
    check_exact(got[~written], want[~written], what + " untouched slots")
    if written.any():
        check16(got[written], want[written], dt, what)


@pytest.mark.parametrize("case", QKV_CASES, ids=lambda c: c[0])
def test_qkv_normrope_kvwrite(fr, case):
    name, T, Hq, Hkv, D, dt, norm, theta, style, P, pages, rnd, pos, seed = case
    announce(f"qkv {name} T={T} Hq={Hq} Hkv={Hkv} D={D} dtype={dt} seed={seed}")
    inp = workloads.qkv_inputs(T, Hq, Hkv, D, dt, seed, page_size=P,
                               num_pages=pages, positions=pos, norm=norm,
                               random_pages=rnd)
    q_g, kc_g, vc_g, err_g = run_qkv(fr, inp, EPS, theta, style, Hq, Hkv, D,
                                     P, dt)
    kc_o, vc_o = inp["k_cache"].copy(), inp["v_cache"].copy()
    q_o, err_o = oracle.qkv_normrope_kvwrite(
        inp["qkv"], inp["q_norm_w"], inp["k_norm_w"], EPS, inp["positions"],
        theta, style, kc_o, vc_o, inp["page_table"], P, Hq, Hkv, D, dt)
    assert err_g == err_o == 0
    same = check16(q_g, q_o, dt, "q_out")
    announce(f"  q_out bit-identical fraction {same:.6f}")
    _check_cache(kc_g, kc_o, dt, "k_cache")
    check_exact(vc_g, vc_o, "v_cache")


@pytest.mark.parametrize("T", [128, 2048], ids=["T128", "T2048_bandwidth"])
@pytest.mark.parametrize("qs", [0.0625, 128 ** -0.5, 3.0])
def test_qkv_q_prescale(fr, qs, T):
    """Q pre-scale folded into RoPE (the attention's Q preparation):
    Qwen3 prefill shape (and the bandwidth-regime kernel at 2048 tokens); a
    power of two, 1/sqrt(D) and a scale above 1."""
    Hq, Hkv, D, P, pages = 32, 8, 128, 16, 512
    announce(f"qkv q_scale={qs:.6g} T={T}")
    inp = workloads.qkv_inputs(T, Hq, Hkv, D, BF16, 408, page_size=P,
                               num_pages=pages)
    q_g, kc_g, vc_g, _ = run_qkv(fr, inp, EPS, 1e6, 0, Hq, Hkv, D, P, BF16,
                                 q_scale=qs)
    kc_o, vc_o = inp["k_cache"].copy(), inp["v_cache"].copy()
    q_o, _ = oracle.qkv_normrope_kvwrite(
        inp["qkv"], inp["q_norm_w"], inp["k_norm_w"], EPS, inp["positions"],
        1e6, 0, kc_o, vc_o, inp["page_table"], P, Hq, Hkv, D, BF16, q_scale=qs)
    same = check16(q_g, q_o, BF16, "q_out")
    announce(f"  q_out bit-identical fraction {same:.6f}")
    _check_cache(kc_g, kc_o, BF16, "k_cache")
    check_exact(vc_g, vc_o, "v_cache")


def test_qkv_bandwidth_k_norm_only_and_out_of_range(fr):
    """Bandwidth regime (T >= 2048): K norm only (each lane loads its own
    head's weight; Q heads take none), a head group that mixes K and V
    heads (16/4 x 128: group 2 = K heads 0..3 and V heads 0..3), and two
    tokens whose positions map to no slot (their K/V writes are skipped and
    the error bit set)."""
    T, Hq, Hkv, D, P, pages = 2048, 16, 4, 128, 16, 128
    announce("qkv bandwidth regime, k_norm only, out-of-range positions")
    pos = np.arange(T, dtype=np.int32)
    pos[5], pos[1000] = -1, P * pages                      # no slot
    inp = workloads.qkv_inputs(T, Hq, Hkv, D, BF16, 412, page_size=P,
                               num_pages=pages, positions=pos)
    inp["q_norm_w"] = None
    q_g, kc_g, vc_g, err_g = run_qkv(fr, inp, EPS, 1e6, 0, Hq, Hkv, D, P, BF16)
    kc_o, vc_o = inp["k_cache"].copy(), inp["v_cache"].copy()
    q_o, err_o = oracle.qkv_normrope_kvwrite(
        inp["qkv"], None, inp["k_norm_w"], EPS, pos, 1e6, 0, kc_o, vc_o,
        inp["page_table"], P, Hq, Hkv, D, BF16)
    assert err_o == 1 and err_g == 1
    check16(q_g, q_o, BF16, "q_out")
    _check_cache(kc_g, kc_o, BF16, "k_cache")
    check_exact(vc_g, vc_o, "v_cache")


def test_qkv_only_q_norm_and_out_of_range(fr):
    T, Hq, Hkv, D, P, pages = 6, 4, 2, 64, 4, 3
    announce("qkv out-of-range positions / q_norm only")
    pos = np.array([0, -1, 11, 12, 5, 2], dtype=np.int32)   # -1 and 12 invalid
    inp = workloads.qkv_inputs(T, Hq, Hkv, D, BF16, 407, page_size=P,
                               num_pages=pages, positions=pos)
    inp["k_norm_w"] = None
    q_g, kc_g, vc_g, err_g = run_qkv(fr, inp, EPS, 1e4, 0, Hq, Hkv, D, P, BF16)
    kc_o, vc_o = inp["k_cache"].copy(), inp["v_cache"].copy()
    q_o, err_o = oracle.qkv_normrope_kvwrite(
        inp["qkv"], inp["q_norm_w"], None, EPS, pos, 1e4, 0, kc_o, vc_o,
        inp["page_table"], P, Hq, Hkv, D, BF16)
    assert err_o == 1 and err_g == 1
    check16(q_g, q_o, BF16, "q_out")
    _check_cache(kc_g, kc_o, BF16, "k_cache")
    check_exact(vc_g, vc_o, "v_cache")
    # a page id outside the pool is also an error
    inp2 = dict(inp)
    inp2["page_table"] = np.array([0, 7, 1], dtype=np.int32)
    inp2["positions"] = np.array([0, 1, 4, 5, 8, 9], dtype=np.int32)
    _, kc_g, vc_g, err_g = run_qkv(fr, inp2, EPS, 1e4, 0, Hq, Hkv, D, P, BF16)
    kc_o, vc_o = inp["k_cache"].copy(), inp["v_cache"].copy()
    _, err_o = oracle.qkv_normrope_kvwrite(
        inp["qkv"], inp["q_norm_w"], None, EPS, inp2["positions"], 1e4, 0,
        kc_o, vc_o, inp2["page_table"], P, Hq, Hkv, D, BF16)
    assert err_o == 1 and err_g == 1
    _check_cache(kc_g, kc_o, BF16, "k_cache")
    check_exact(vc_g, vc_o, "v_cache")


# ---------------------------------------------------------------------------
# (c) gated activation + block-128 FP8
# ---------------------------------------------------------------------------

ACT_CASES = [
    # (T, I, dtype, act, outliers, seed)
    (128, 6144, BF16, oracle.ACT_SWIGLU, False, 104),
    (128, 6144, BF16, oracle.ACT_GEGLU_TANH, False, 104),
    (128, 6144, BF16, oracle.ACT_SQRELU, False, 104),
    (192, 6144, BF16, oracle.ACT_SWIGLU, False, 104),
    (192, 6144, BF16, oracle.ACT_GEGLU_TANH, False, 104),
    (1024, 6144, BF16, oracle.ACT_SWIGLU, False, 104),
    (1024, 6144, BF16, oracle.ACT_GEGLU_TANH, False, 104),
    (7, 384, F16, oracle.ACT_SWIGLU, False, 501),        # 3 blocks: partial wave
    (7, 384, F16, oracle.ACT_GEGLU_TANH, False, 501),
    (7, 384, F16, oracle.ACT_SQRELU, False, 501),
    (3, 128, BF16, oracle.ACT_SWIGLU, False, 502),       # one block
    (5, 1152, BF16, oracle.ACT_GEGLU_TANH, True, 503),   # 9 blocks: crosses waves
    (8192, 12288, BF16, oracle.ACT_SWIGLU, True, 105),   # full bandwidth config
    (8192, 12288, BF16, oracle.ACT_GEGLU_TANH, True, 105),
    # bandwidth launch shape (T >= 2048) with a ragged last wave per row
    (2048, 1152, BF16, oracle.ACT_SWIGLU, True, 506),    # 9 blocks: 8 + 1
    (2048, 640, F16, oracle.ACT_SQRELU, False, 507),     # 5 blocks: one partial wave
]


@pytest.mark.parametrize("case", ACT_CASES, ids=lambda c: f"T{c[0]}_I{c[1]}_dt{c[2]}_act{c[3]}")
def test_gated_act(fr, case):
    T, I, dt, act, outl, seed = case
    announce(f"gated_act T={T} I={I} dtype={dt} act={act} seed={seed}")
    inp = workloads.gated_act_inputs(T, I, dt, seed, outliers=outl)
    q_g, sc_g = run_gated_act(fr, inp, act, dt)
    q_o, sc_o = oracle.gated_act_fp8(inp["gate_up"], act, dt)
    ident = check_fp8(q_g, q_o, "out_fp8")
    rel = check_scales(sc_g, sc_o, "out_scales")
    announce(f"  fp8 identical fraction {ident:.7f}, scale max rel err {rel:.2e}")


def test_gated_act_worked_block(fr):
    announce("gated_act worked block")
    g = np.zeros(128)
    g[:4] = [1, -1, 2, 0]
    u = np.zeros(128)
    u[:4] = 1
    gu = np.empty(256)
    gu[0::2], gu[1::2] = g, u
    inp = {"gate_up": workloads.to16(gu[None, :], BF16)}
    for act, codes in ((oracle.ACT_SWIGLU, [0x74, 0xE9, 0x7E, 0x00]),
                       (oracle.ACT_GEGLU_TANH, [0x74, 0xE1, 0x7E, 0x00]),
                       (oracle.ACT_SQRELU, [0x6E, 0x00, 0x7E, 0x00])):
        q, s = run_gated_act(fr, inp, act, BF16)
        assert list(q[0, :4]) == codes
        assert not (q[0, 4:] & 0x7F).any()


# ---------------------------------------------------------------------------
# determinism: repeated calls are bit-identical
# ---------------------------------------------------------------------------

def test_determinism_five_runs(fr):
    announce("determinism x5")
    ri = workloads.resid_rmsnorm_inputs(1024, 4096, BF16, 601, outliers=True)
    ai = workloads.adarms_inputs(256, 1024, F16, 602)
    qi = workloads.qkv_inputs(128, 32, 8, 128, BF16, 603, page_size=16,
                              num_pages=512)
    gi = workloads.gated_act_inputs(512, 6144, BF16, 604)
    first = None
    for _ in range(5):
        out = (run_resid_rmsnorm(fr, ri, oracle.W_MUL, EPS, oracle.Q_TOKEN, 0.0, BF16)
               + run_adarms(fr, ai, EPS, oracle.Q_TOKEN, 0.0, F16)
               + run_qkv(fr, qi, EPS, 1e6, 0, 32, 8, 128, 16, BF16)
               + run_gated_act(fr, gi, oracle.ACT_SWIGLU, BF16))
        if first is None:
            first = out
        else:
            for a, b in zip(first, out):
                if a is None:
                    assert b is None
                elif isinstance(a, int):
                    assert a == b
                else:
                    assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
