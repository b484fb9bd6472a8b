"""Pins for the oracle of the FP8 block-scaled gate_up GEMM fused with the
gated activation and block-128 FP8 output (CPU only)."""
import math

import numpy as np
import pytest

import oracle
import workloads


def brute_acc(a, a_s, w, w_s):
    """Triple loop over decoded codes with explicit block-scale indexing."""
    tab = oracle.e4m3_table()
    M, K = a.shape
    N = w.shape[0]
    acc = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += (tab[a[m, k]] * a_s[m, k // 128]) * (tab[w[n, k]] * w_s[n // 128, k // 128])
            acc[m, n] = s
    return acc


def test_gemm_accumulator_matches_brute_force_with_block_scales():
    inp = workloads.gemm_inputs(2, 256, 128, seed=30)
    # make every scale block distinct so a transposed or shifted index fails
    inp["a_scales"] = np.array([[0.5, 2.0], [0.25, 4.0]], dtype=np.float32)
    inp["w_scales"] = np.array([[1.0, 3.0], [0.125, 8.0]], dtype=np.float32)
    _, _, acc = oracle.gemm_gated_act_fp8(inp["a"], inp["a_scales"], inp["w"],
                                          inp["w_scales"], oracle.ACT_SWIGLU)
    ref = brute_acc(inp["a"], inp["a_scales"], inp["w"], inp["w_scales"])
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-12)


def test_gemm_worked_example_interleave_and_codes():
    # A = all ones; W gate rows pick g = 1, up rows give u_j = 1, 2, 4, 8
    K, I = 128, 128
    a = np.full((1, K), 0x38, dtype=np.uint8)              # 1.0
    w = np.zeros((2 * I, K), dtype=np.uint8)
    w[0::2, 0] = 0x38                                      # gate row j: g = 1
    for j in range(I):
        w[2 * j + 1, : [1, 2, 4, 8][j % 4]] = 0x38         # up row j: u = 1,2,4,8
    a_s = np.ones((1, 1), np.float32)
    w_s = np.ones((2, 1), np.float32)
    q, s, acc = oracle.gemm_gated_act_fp8(a, a_s, w, w_s, oracle.ACT_SWIGLU)
    assert np.array_equal(acc[0, 0::2], np.ones(I))
    assert np.array_equal(acc[0, 1::2], np.tile([1.0, 2.0, 4.0, 8.0], I // 4))
    silu1 = 1.0 / (1.0 + math.exp(-1.0))
    assert s[0, 0] == np.float32(8.0 * silu1 / 448.0)
    # h/s = 56 u: 56, 112, 224, 448 -> exact e4m3 codes
    assert list(q[0, :4]) == [0x66, 0x6E, 0x76, 0x7E]
    # swapping gate and up would give silu(u) * 1 instead
    q2, _, _ = oracle.gemm_gated_act_fp8(a, a_s, w[np.arange(2 * I) ^ 1], w_s,
                                         oracle.ACT_SWIGLU)
    assert list(q2[0, :4]) != [0x66, 0x6E, 0x76, 0x7E]


def test_gemm_zero_up_rows_give_zero_codes():
    inp = workloads.gemm_inputs(3, 128, 256, seed=31)
    w = inp["w"].copy()
    w[1::2] = 0
    q, s, _ = oracle.gemm_gated_act_fp8(inp["a"], inp["a_scales"], w,
                                        inp["w_scales"], oracle.ACT_GEGLU_TANH)
    assert not (q & 0x7F).any()
    assert np.all(s == np.float32(np.float32(1e-10) / 448.0))


def test_gated_act_f64_agrees_with_16bit_entry():
    inp = workloads.gated_act_inputs(4, 256, workloads.BF16, 32)
    q1, s1 = oracle.gated_act_fp8(inp["gate_up"], oracle.ACT_SWIGLU, oracle.BF16)
    gu = oracle.decode16(inp["gate_up"], oracle.BF16)
    q2, s2 = oracle.gated_act_fp8_f64(gu, oracle.ACT_SWIGLU)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
