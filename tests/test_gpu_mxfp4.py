"""GPU parity of the MX FP4 producers (residual RMSNorm -> MXFP4, gated
activation -> MXFP4) against the oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
import workloads
from parity import (announce, check_exact, check_fp4, check16,
                    run_gated_act_mxfp4, run_resid_rmsnorm_mxfp4)

pytestmark = pytest.mark.gpu
F16, BF16 = workloads.F16, workloads.BF16
EPS = 1e-6


@pytest.fixture(scope="module")
def fr():
    import memory_bound_amd
    return memory_bound_amd


NORM_CASES = [
    # (name, T, H, dtype, wmode, outliers, seed)
    ("decode_t10", 10, 1024, F16, oracle.W_NONE, False, 501),
    ("prefill_4096_mul", 128, 4096, BF16, oracle.W_MUL, True, 502),
    ("one_plus", 33, 2048, BF16, oracle.W_ONE_PLUS, True, 503),
    ("ragged_1056", 17, 1056, F16, oracle.W_MUL, False, 504),
    ("smallest_32", 5, 32, BF16, oracle.W_NONE, False, 505),
    ("largest_32768", 3, 32768, BF16, oracle.W_MUL, True, 506),
    ("t1", 1, 4096, F16, oracle.W_ONE_PLUS, False, 507),
    ("bench_8192", 8192, 4096, BF16, oracle.W_MUL, True, 101),
]


@pytest.mark.parametrize("case", NORM_CASES, ids=lambda c: c[0])
def test_resid_rmsnorm_mxfp4(fr, case):
    name, T, H, dt, wmode, outl, seed = case
    announce(f"resid_rmsnorm_mxfp4 {name} T={T} H={H} dtype={dt} wmode={wmode}")
    inp = workloads.resid_rmsnorm_inputs(T, H, dt, seed, outliers=outl)
    ro_g, q_g, s_g = run_resid_rmsnorm_mxfp4(fr, inp, wmode, EPS, dt)
    ro_o, q_o, s_o = oracle.resid_rmsnorm_mxfp4(inp["x"], inp["residual"],
                                                inp["weight"], wmode, EPS, dt)
    check_exact(ro_g, ro_o, "residual_out")
    check_exact(s_g, s_o, "scales (E8M0)")
    check_exact(q_g, q_o, "codes (E2M1)")


def test_resid_rmsnorm_mxfp4_in_place_and_every_byte_written(fr):
    announce("resid_rmsnorm_mxfp4 in place, two poisons")
    inp = workloads.resid_rmsnorm_inputs(19, 1056, BF16, 508)
    a = run_resid_rmsnorm_mxfp4(fr, inp, oracle.W_MUL, EPS, BF16, inplace=True, poison=0x00)
    b = run_resid_rmsnorm_mxfp4(fr, inp, oracle.W_MUL, EPS, BF16, poison=0xFF)
    for x, y in zip(a, b):
        check_exact(x, y, "poison-independent output")


ACT_CASES = [
    # (name, T, I, dtype, act, outliers, seed)
    ("decode_t10", 10, 6144, BF16, oracle.ACT_SWIGLU, False, 511),
    ("prefill_gelu", 128, 12288, BF16, oracle.ACT_GEGLU_TANH, True, 512),
    ("sqrelu_f16", 64, 6144, F16, oracle.ACT_SQRELU, True, 513),
    ("ragged_384", 7, 384, F16, oracle.ACT_SWIGLU, False, 514),
    ("smallest_128", 3, 128, BF16, oracle.ACT_GEGLU_TANH, False, 515),
    ("bench_8192", 8192, 12288, BF16, oracle.ACT_SWIGLU, True, 105),
    ("bandwidth_ragged_1152", 2048, 1152, BF16, oracle.ACT_GEGLU_TANH, False, 517),
]


@pytest.mark.parametrize("case", ACT_CASES, ids=lambda c: c[0])
def test_gated_act_mxfp4(fr, case):
    name, T, I, dt, act, outl, seed = case
    announce(f"gated_act_mxfp4 {name} T={T} I={I} dtype={dt} act={act}")
    inp = workloads.gated_act_inputs(T, I, dt, seed, outliers=outl)
    q_g, s_g = run_gated_act_mxfp4(fr, inp, act, dt)
    q_o, s_o = oracle.gated_act_mxfp4(inp["gate_up"], act, dt)
    ident, frac = check_fp4(q_g, s_g, q_o, s_o, "gated_act_mxfp4")
    announce(f"  codes identical {ident:.6f}, block scales differing {frac:.2e}")


def test_gated_act_mxfp4_every_byte_written(fr):
    announce("gated_act_mxfp4 two poisons")
    inp = workloads.gated_act_inputs(9, 384, BF16, 516)
    a = run_gated_act_mxfp4(fr, inp, oracle.ACT_SWIGLU, BF16, poison=0x00)
    b = run_gated_act_mxfp4(fr, inp, oracle.ACT_SWIGLU, BF16, poison=0xFF)
    for x, y in zip(a, b):
        check_exact(x, y, "poison-independent output")


# ---------------------------------------------------------------------------
# residual add + LayerNorm producers (FP8 and MXFP4)
# ---------------------------------------------------------------------------

LN_CASES = [
    # (name, T, H, dtype, out_kind, qmode, bias, seed)
    ("vit_mx_1024", 64, 1024, BF16, 1, 0, True, 521),
    ("vit_mx_nobias_f16", 10, 2048, F16, 1, 0, False, 522),
    ("fp8_token_4096", 128, 4096, BF16, 0, 1, True, 523),
    ("fp8_static_1056", 17, 1056, F16, 0, 0, True, 524),
    ("mx_32768", 3, 32768, BF16, 1, 0, True, 525),
    ("mx_bench_8192", 8192, 4096, BF16, 1, 0, True, 526),
]


@pytest.mark.parametrize("case", LN_CASES, ids=lambda c: c[0])
def test_resid_layernorm(fr, case):
    import torch
    from parity import POISON16, check_fp8, check_scales, to_dev, to_host
    name, T, H, dt, kind, qmode, has_b, seed = case
    announce(f"resid_layernorm {name} T={T} H={H} kind={kind} qmode={qmode}")
    inp = workloads.resid_rmsnorm_inputs(T, H, dt, seed, outliers=True)
    rng = np.random.default_rng(seed + 1)
    bias = workloads.to16(0.1 * rng.standard_normal(H).astype(np.float32), dt) if has_b else None
    x, r, w = to_dev(inp["x"]), to_dev(inp["residual"]), to_dev(inp["weight"])
    b = to_dev(bias) if has_b else None
    ro = torch.full((T, H), POISON16, dtype=torch.int16, device="cuda")
    if kind == 1:
        q = torch.full((T, H // 2), 0xAA, dtype=torch.uint8, device="cuda")
        sc = torch.full((T, H // 32), 0xFF, dtype=torch.uint8, device="cuda")
        fr.fr_resid_layernorm_mxfp4(x, r, ro, w, b, EPS, q, sc, T, H, dt)
    else:
        q = torch.full((T, H), 0x7F, dtype=torch.uint8, device="cuda")
        sc = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
        fr.fr_resid_layernorm_fp8(x, r, ro, w, b, EPS, q, qmode, 40.0, sc, T, H, dt)
    torch.cuda.synchronize()
    ro_o, q_o, s_o = oracle.resid_layernorm(inp["x"], inp["residual"], inp["weight"], bias,
                                            EPS, kind, qmode, 40.0, dt)
    check_exact(to_host(ro, np.uint16), ro_o, "residual_out")
    if kind == 1:
        ident, frac = check_fp4(to_host(q, np.uint8), to_host(sc, np.uint8), q_o, s_o,
                                "resid_layernorm_mxfp4")
        announce(f"  codes identical {ident:.6f}, block scales differing {frac:.2e}")
    else:
        ident = check_fp8(to_host(q, np.uint8), q_o, "out_fp8")
        if qmode == 1:
            check_scales(to_host(sc, np.float32), s_o, "out_scales")
        announce(f"  fp8 identical {ident:.6f}")
