"""GPU parity of the NVFP4 producers against the oracle, through the C ABI.
Residual RMSNorm -> NVFP4: the kernel takes both decisions on the exact value
(the block scale on a double-precision amax / (6 g), the elements as
round-to-odd products), so residual, E4M3 block scales and E2M1 codes must be
bit-identical to the oracle's.  Residual add + LayerNorm -> NVFP4: the
LayerNorm output is fp32 on the GPU (float64 in the oracle), so its codes and
scales follow the FP4 tolerance rule of parity.py (residual bit-exact)."""
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


LN_CASES = [
    # (name, T, H, dtype, bias, g, seed)
    ("vit_1024", 64, 1024, BF16, True, G, 531),
    ("nobias_f16_1040", 17, 1040, F16, False, G, 532),
    ("smallest_16", 5, 16, BF16, True, G, 533),
    ("largest_32768", 3, 32768, BF16, True, G, 534),
    ("saturated_scales", 64, 1024, BF16, True, 2.5e-4, 535),
    ("zero_scales", 64, 1024, BF16, True, 400.0, 536),
    ("bench_8192", 8192, 4096, BF16, True, G, 537),
]


def _run_ln_nvfp4(fr, inp, bias, g, dt, poison):
    import torch
    from parity import POISON16, to_dev, to_host
    T, H = inp["x"].shape
    ro = torch.full((T, H), POISON16, dtype=torch.int16, device="cuda")
    q = torch.full((T, H // 2), poison, dtype=torch.uint8, device="cuda")
    sc = torch.full((T, H // 16), 0xFF, dtype=torch.uint8, device="cuda")
    fr.fr_resid_layernorm_nvfp4(to_dev(inp["x"]), to_dev(inp["residual"]), ro,
                                to_dev(inp["weight"]), None if bias is None else to_dev(bias),
                                EPS, g, q, sc, T, H, dt)
    torch.cuda.synchronize()
    return to_host(ro, np.uint16), to_host(q, np.uint8), to_host(sc, np.uint8)


@pytest.mark.parametrize("case", LN_CASES, ids=lambda c: c[0])
def test_resid_layernorm_nvfp4(fr, case):
    from parity import check_fp4
    name, T, H, dt, has_b, g, seed = case
    announce(f"resid_layernorm_nvfp4 {name} T={T} H={H} dtype={dt} g={g}")
    inp = workloads.resid_rmsnorm_inputs(T, H, dt, seed, outliers=True)
    rng = np.random.default_rng(seed + 1)
    bias = workloads.to16(0.1 * rng.standard_normal(H).astype(np.float32), dt) if has_b else None
    ro_g, q_g, s_g = _run_ln_nvfp4(fr, inp, bias, g, dt, 0xAA)
    ro_o, q_o, s_o = oracle.resid_layernorm_nvfp4(inp["x"], inp["residual"], inp["weight"],
                                                  bias, EPS, g, dt)
    check_exact(ro_g, ro_o, "residual_out")
    ident, frac = check_fp4(q_g, s_g, q_o, s_o, "resid_layernorm_nvfp4", block=16)
    announce(f"  codes identical {ident:.6f}, block scales differing {frac:.2e}")
    if name == "saturated_scales":
        assert np.mean(s_o == 0x7E) > 0.99
    if name == "zero_scales":
        assert np.any(s_o == 0) and np.any(s_o > 0)
    if T <= 64:                                        # every byte written: a second poison
        again = _run_ln_nvfp4(fr, inp, bias, g, dt, 0x55)
        for a, b_ in zip((ro_g, q_g, s_g), again):
            assert np.array_equal(a, b_)
