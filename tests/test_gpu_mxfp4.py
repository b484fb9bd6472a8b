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
