"""GPU parity of the residual RMSNorm -> NVFP4 producer against the oracle,
through the C ABI.  The kernel takes both decisions on the exact value (the
block scale on a double-precision amax / (6 g), the elements as round-to-odd
products), so residual, E4M3 block scales and E2M1 codes must be
bit-identical to the oracle's."""
import numpy as np
import pytest

import oracle
import workloads
from parity import announce, check_exact, run_resid_rmsnorm_nvfp4

pytestmark = pytest.mark.gpu
F16, BF16 = workloads.F16, workloads.BF16
EPS = 1e-6
G = 3.7e-2          # a calibrated-style tensor scale: amax ~ 100 over 6 * 448


@pytest.fixture(scope="module")
def fr():
    import memory_bound_amd
    return memory_bound_amd


CASES = [
    # (name, T, H, dtype, wmode, outliers, g, seed)
    ("decode_t10", 10, 1024, F16, oracle.W_NONE, False, G, 521),
    ("prefill_4096_mul", 128, 4096, BF16, oracle.W_MUL, True, G, 522),
    ("one_plus", 33, 2048, BF16, oracle.W_ONE_PLUS, True, G, 523),
    ("ragged_1040", 17, 1040, F16, oracle.W_MUL, False, G, 524),
    ("smallest_16", 5, 16, BF16, oracle.W_NONE, False, G, 525),
    ("largest_32768", 3, 32768, BF16, oracle.W_MUL, True, G, 526),
    ("t1_one_plus", 1, 4096, F16, oracle.W_ONE_PLUS, False, G, 527),
    ("saturated_scales", 64, 1024, BF16, oracle.W_MUL, True, 1e-5, 528),   # codes 0x7E, elements at 6
    ("subnormal_scales", 64, 1024, BF16, oracle.W_MUL, False, 400.0, 529),  # E4M3 subnormal and zero scales
    ("bench_8192", 8192, 4096, BF16, oracle.W_MUL, True, G, 105),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_resid_rmsnorm_nvfp4(fr, case):
    name, T, H, dt, wmode, outl, g, seed = case
    announce(f"resid_rmsnorm_nvfp4 {name} T={T} H={H} dtype={dt} wmode={wmode} g={g}")
    inp = workloads.resid_rmsnorm_inputs(T, H, dt, seed, outliers=outl)
    ro_g, q_g, s_g = run_resid_rmsnorm_nvfp4(fr, inp, wmode, EPS, g, dt)
    ro_o, q_o, s_o = oracle.resid_rmsnorm_nvfp4(inp["x"], inp["residual"], inp["weight"],
                                                wmode, EPS, g, dt)
    check_exact(ro_g, ro_o, "residual_out")
    check_exact(s_g, s_o, "block scales (E4M3)")
    check_exact(q_g, q_o, "codes (E2M1)")
    if name == "saturated_scales":
        assert np.mean(s_o == 0x7E) > 0.99
    if name == "subnormal_scales":                     # subnormal and zero scale codes exercised
        assert np.any((s_o > 0) & (s_o < 0x08)) and np.any(s_o == 0)


def test_resid_rmsnorm_nvfp4_in_place_and_every_byte_written(fr):
    announce("resid_rmsnorm_nvfp4 in place, two poisons")
    inp = workloads.resid_rmsnorm_inputs(19, 1040, BF16, 530)
    a = run_resid_rmsnorm_nvfp4(fr, inp, oracle.W_MUL, EPS, G, BF16, inplace=True, poison=0x00)
    b = run_resid_rmsnorm_nvfp4(fr, inp, oracle.W_MUL, EPS, G, BF16, poison=0xFF)
    for x, y in zip(a, b):
        check_exact(x, y, "poison-independent output")
