"""GPU parity of the Q/K norm + RoPE variants (fr_qk_norm_rope) against the
oracle: LayerNorm per head (Chameleon), RMSNorm over the full width with 3D
RoPE (Wan), and the other combinations, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import POISON16, announce, check16, check_exact, to_dev, to_host

pytestmark = pytest.mark.gpu
F16, BF16 = workloads.F16, workloads.BF16
EPS = 1e-6


@pytest.fixture(scope="module")
def fr():
    import memory_bound_amd
    return memory_bound_amd


CASES = [
    # (name, T, Hq, Hkv, D, dtype, kind, full, rope3, sections, style, theta, q_scale, seed)
    ("chameleon_layer_head", 128, 32, 32, 128, BF16, 2, False, False, None, 0, 1e4, 1.0, 601),
    ("wan_rms_full_3d", 256, 40, 40, 128, BF16, 1, True, True, (22, 21, 21), 1, 1e4, 1.0, 602),
    ("layer_full_3d_half", 33, 6, 2, 64, F16, 2, True, True, (12, 10, 10), 0, 1e4, 0.5, 603),
    ("rms_head_1d_gqa", 64, 32, 8, 128, BF16, 1, False, False, None, 0, 1e6, 128 ** -0.5, 604),
    ("none_d96_interleaved", 17, 5, 1, 96, F16, 0, False, False, None, 1, 1e4, 0.125, 605),
    ("d256_layer_head", 10, 8, 1, 256, F16, 2, False, False, None, 0, 1e4, 1.0, 606),
    ("d16_rms_full", 9, 3, 3, 16, BF16, 1, True, False, None, 1, 1e4, 1.0, 607),
    ("wan_bench_8192", 8192, 40, 40, 128, BF16, 1, True, True, (22, 21, 21), 1, 1e4, 1.0, 608),
    ("chameleon_bench_8192", 8192, 32, 32, 128, BF16, 2, False, False, None, 0, 1e4, 1.0, 609),
    # per-head norm over four full passes of heads (one workgroup per pass),
    # 3D RoPE, interleaved pairs
    ("rms_head_3d_four_passes", 50, 64, 32, 128, BF16, 1, False, True, (22, 21, 21), 1, 1e4, 0.5, 614),
    ("layer_head_f16_three_passes", 33, 32, 32, 128, F16, 2, False, False, None, 1, 1e4, 1.0, 615),
]


def run(fr, inp, case):
    name, T, Hq, Hkv, D, dt, kind, full, r3, sec, style, theta, qs, seed = case
    q = torch.full((T, Hq, D), POISON16, dtype=torch.int16, device="cuda")
    k = torch.full((T, Hkv, D), POISON16, dtype=torch.int16, device="cuda")
    v = torch.full((T, Hkv, D), POISON16, dtype=torch.int16, device="cuda")
    ws = [None if inp[n] is None else to_dev(inp[n])
          for n in ("q_norm_w", "q_norm_b", "k_norm_w", "k_norm_b")]
    fr.fr_qk_norm_rope(to_dev(inp["qkv"]), kind, int(full), *ws, EPS,
                       to_dev(inp["positions"]), 3 if r3 else 1, sec, theta, style,
                       qs, q, k, v, T, Hq, Hkv, D, dt)
    torch.cuda.synchronize()
    return to_host(q, np.uint16), to_host(k, np.uint16), to_host(v, np.uint16)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_qk_norm_rope(fr, case):
    name, T, Hq, Hkv, D, dt, kind, full, r3, sec, style, theta, qs, seed = case
    announce(f"qk_norm_rope {name} T={T} Hq={Hq} Hkv={Hkv} D={D} kind={kind} full={full} 3d={r3}")
    inp = workloads.qk_norm_rope_inputs(T, Hq, Hkv, D, dt, seed, scope_full=full, rope3=r3)
    qg, kg, vg = run(fr, inp, case)
    qo, ko, vo = oracle.qk_norm_rope(
        inp["qkv"], kind, int(full), inp["q_norm_w"], inp["q_norm_b"], inp["k_norm_w"],
        inp["k_norm_b"], EPS, inp["positions"], 3 if r3 else 1, sec, theta, style, qs,
        Hq, Hkv, D, dt)
    sq = check16(qg, qo, dt, "q_out")
    sk = check16(kg, ko, dt, "k_out")
    check_exact(vg, vo, "v_out")
    announce(f"  bit-identical q {sq:.6f} k {sk:.6f}")


ABSENT_CASES = [
    # (case, which optional inputs are absent): weights read as 1, biases as 0
    (("rms_head_noweight", 20, 8, 2, 128, BF16, 1, False, False, None, 0, 1e4, 1.0, 611), "wb"),
    (("layer_full_nobias", 12, 4, 4, 64, F16, 2, True, False, None, 1, 1e4, 0.5, 612), "b"),
    (("layer_head_noweight", 9, 6, 3, 128, BF16, 2, False, True, (22, 21, 21), 0, 1e4, 1.0, 613), "w"),
]


@pytest.mark.parametrize("case,absent", ABSENT_CASES, ids=lambda c: c[0] if isinstance(c, tuple) else c)
def test_qk_norm_rope_absent_weights(fr, case, absent):
    name, T, Hq, Hkv, D, dt, kind, full, r3, sec, style, theta, qs, seed = case
    announce(f"qk_norm_rope {name}: absent {absent}")
    inp = workloads.qk_norm_rope_inputs(T, Hq, Hkv, D, dt, seed, scope_full=full, rope3=r3)
    for n in ("q_norm_w", "k_norm_w") if "w" in absent else ():
        inp[n] = None
    for n in ("q_norm_b", "k_norm_b") if "b" in absent else ():
        inp[n] = None
    qg, kg, vg = run(fr, inp, case)
    qo, ko, vo = oracle.qk_norm_rope(
        inp["qkv"], kind, int(full), inp["q_norm_w"], inp["q_norm_b"], inp["k_norm_w"],
        inp["k_norm_b"], EPS, inp["positions"], 3 if r3 else 1, sec, theta, style, qs,
        Hq, Hkv, D, dt)
    check16(qg, qo, dt, "q_out")
    check16(kg, ko, dt, "k_out")
    check_exact(vg, vo, "v_out")
