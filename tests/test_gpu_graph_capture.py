"""Every entry point under HIP graph capture (the decode path of the pages
runs its launches from a captured graph).  Each op is called once eagerly on
a stream, then captured on the same stream and replayed several times; before
each replay the outputs are overwritten by eager work on that stream, and
after it every output must equal the eager call's bit for bit (the kernels
are deterministic).  The captured graph must hold one kernel node per call
and no other node: no entry point records a memset, a copy or an allocation."""
import numpy as np
import pytest
import torch

import workloads
from parity import announce, to_dev

pytestmark = pytest.mark.gpu
EPS = 1e-6
REPLAYS = 3


@pytest.fixture(scope="module")
def fr():
    import memory_bound_amd
    return memory_bound_amd


def _empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


def _norm_in(T, H, dt, seed):
    inp = workloads.resid_rmsnorm_inputs(T, H, dt, seed, outliers=True)
    bias = workloads.to16(0.1 * np.random.default_rng(seed).standard_normal(H).astype(np.float32), dt)
    return {k: to_dev(v) for k, v in inp.items()}, to_dev(bias)


def case_resid_rmsnorm_fp8(fr):
    T, H = 40, 2048
    d, _ = _norm_in(T, H, fr.BF16, 801)
    ro, q, s = _empty((T, H), torch.int16), _empty((T, H), torch.uint8), _empty((T,), torch.float32)
    def call(st):
        fr.fr_resid_rmsnorm_fp8(d["x"], d["residual"], ro, d["weight"], fr.W_MUL, EPS, q,
                                fr.Q_TOKEN, 0.0, s, T, H, fr.BF16, stream=st)
    return call, [ro, q, s]


def case_adarms(fr):
    T, H = 10, 1024
    inp = {k: to_dev(v) for k, v in workloads.adarms_inputs(T, H, fr.F16, 802).items()}
    ro, q = _empty((T, H), torch.int16), _empty((T, H), torch.uint8)
    def call(st):
        fr.fr_adarms_gate_res_fp8(inp["x"], inp["gate"], inp["residual"], ro, inp["ada_scale"],
                                  inp["ada_shift"], EPS, q, fr.Q_STATIC, 56.0, None, T, H,
                                  fr.F16, stream=st)
    return call, [ro, q]


def case_qkv(fr):
    T, Hq, Hkv, D, P, pages = 10, 8, 1, 256, 16, 64
    inp = workloads.qkv_inputs(T, Hq, Hkv, D, fr.F16, 803, page_size=P, num_pages=pages,
                               positions=np.arange(300, 310))
    d = {k: (to_dev(v) if v is not None else None) for k, v in inp.items()}
    qo = _empty((T, Hq, D), torch.int16)
    def call(st):
        fr.fr_qkv_normrope_kvwrite(d["qkv"], d["q_norm_w"], d["k_norm_w"], EPS, d["positions"],
                                   1e4, fr.ROPE_HALF, qo, d["k_cache"], d["v_cache"],
                                   d["page_table"], pages, P, pages, None, T, Hq, Hkv, D,
                                   fr.F16, stream=st)
    return call, [qo], [d["k_cache"], d["v_cache"]]     # caches: only some slots written


def case_gated_act_fp8(fr):
    T, I = 24, 6144
    gu = to_dev(workloads.gated_act_inputs(T, I, fr.BF16, 804)["gate_up"])
    q, s = _empty((T, I), torch.uint8), _empty((T, I // 128), torch.float32)
    def call(st):
        fr.fr_gated_act_fp8(gu, fr.ACT_SWIGLU, q, s, T, I, fr.BF16, stream=st)
    return call, [q, s]


def case_gemm(fr):
    M, K, I = 96, 1024, 1024
    inp = workloads.gemm_inputs(M, K, I, 805)
    a, a_s, w_s = to_dev(inp["a"]), to_dev(inp["a_scales"]), to_dev(inp["w_scales"])
    wp = _empty((2 * I * K,), torch.uint8)
    fr.fr_gemm_pack_weights(to_dev(inp["w"]), wp, 2 * I, K)
    torch.cuda.synchronize()
    q, s = _empty((M, I), torch.uint8), _empty((M, I // 128), torch.float32)
    def call(st):
        fr.fr_gemm_gated_act_fp8(a, a_s, wp, w_s, fr.ACT_SWIGLU, q, s, M, K, I, stream=st)
    return call, [q, s]


def case_fp4_norms(fr):
    T, H = 17, 1024
    d, b = _norm_in(T, H, fr.BF16, 806)
    outs = [_empty((T, H), torch.int16), _empty((T, H // 2), torch.uint8),
            _empty((T, H // 32), torch.uint8),
            _empty((T, H), torch.int16), _empty((T, H // 2), torch.uint8),
            _empty((T, H // 16), torch.uint8),
            _empty((T, H), torch.int16), _empty((T, H // 2), torch.uint8),
            _empty((T, H // 16), torch.uint8)]
    def call(st):
        fr.fr_resid_rmsnorm_mxfp4(d["x"], d["residual"], outs[0], d["weight"], fr.W_MUL, EPS,
                                  outs[1], outs[2], T, H, fr.BF16, stream=st)
        fr.fr_resid_rmsnorm_nvfp4(d["x"], d["residual"], outs[3], d["weight"], fr.W_MUL, EPS,
                                  3.7e-2, outs[4], outs[5], T, H, fr.BF16, stream=st)
        fr.fr_resid_layernorm_nvfp4(d["x"], d["residual"], outs[6], d["weight"], b, EPS,
                                    3.7e-2, outs[7], outs[8], T, H, fr.BF16, stream=st)
    return call, outs


def case_layernorm(fr):
    T, H, H2 = 9, 1056, 1024
    d, b = _norm_in(T, H, fr.F16, 807)
    d2, b2 = _norm_in(T, H2, fr.F16, 810)
    ro1, q1, s1 = _empty((T, H), torch.int16), _empty((T, H), torch.uint8), _empty((T,), torch.float32)
    ro2, q2, s2 = (_empty((T, H2), torch.int16), _empty((T, H2 // 2), torch.uint8),
                   _empty((T, H2 // 32), torch.uint8))
    def call(st):
        fr.fr_resid_layernorm_fp8(d["x"], d["residual"], ro1, d["weight"], b, EPS, q1,
                                  fr.Q_TOKEN, 0.0, s1, T, H, fr.F16, stream=st)
        fr.fr_resid_layernorm_mxfp4(d2["x"], d2["residual"], ro2, d2["weight"], b2, EPS, q2, s2,
                                    T, H2, fr.F16, stream=st)
    return call, [ro1, q1, s1, ro2, q2, s2]


def case_gated_act_mxfp4(fr):
    T, I = 12, 2048
    gu = to_dev(workloads.gated_act_inputs(T, I, fr.BF16, 808)["gate_up"])
    q, s = _empty((T, I // 2), torch.uint8), _empty((T, I // 32), torch.uint8)
    def call(st):
        fr.fr_gated_act_mxfp4(gu, fr.ACT_GEGLU_TANH, q, s, T, I, fr.BF16, stream=st)
    return call, [q, s]


def case_qk_norm_rope(fr):
    T, Hq, Hkv, D = 24, 8, 2, 128
    inp = workloads.qk_norm_rope_inputs(T, Hq, Hkv, D, fr.BF16, 809)
    d = {k: to_dev(v) for k, v in inp.items()}
    q, k, v = (_empty((T, Hq, D), torch.int16), _empty((T, Hkv, D), torch.int16),
               _empty((T, Hkv, D), torch.int16))
    def call(st):
        fr.fr_qk_norm_rope(d["qkv"], fr.NORM_LAYER, fr.SCOPE_HEAD, d["q_norm_w"], d["q_norm_b"],
                           d["k_norm_w"], d["k_norm_b"], EPS, d["positions"], 1, None, 1e6,
                           fr.ROPE_HALF, 1.0, q, k, v, T, Hq, Hkv, D, fr.BF16, stream=st)
    return call, [q, k, v]


def case_pack_weights(fr):
    N, K = 512, 1024
    w = to_dev(np.random.default_rng(811).integers(0, 256, (N, K), dtype=np.uint8))
    wp = _empty((N * K,), torch.uint8)
    torch.cuda.synchronize()
    def call(st):
        fr.fr_gemm_pack_weights(w, wp, N, K, stream=st)
    return call, [wp]


def case_chain_persistent(fr):
    L, S, T, H, Hq, Hkv, D, P, pages = 2, 2, 10, 1024, 8, 1, 256, 1024, 1
    N = L * S
    rng = np.random.default_rng(812)
    f16 = lambda *shape, sd=1.0: to_dev(workloads.to16(
        sd * rng.standard_normal(shape, dtype=np.float32), fr.F16))
    x, gate, sc, sh = f16(L, T, H), f16(N, T, H, sd=0.1), f16(N, T, H, sd=0.1), f16(N, T, H, sd=0.1)
    qkv = f16(L, T, (Hq + 2 * Hkv) * D)
    res = _empty((N + 1, T, H), torch.int16)
    res[0] = f16(T, H)
    q8, qo = _empty((N, T, H), torch.uint8), _empty((L, T, Hq, D), torch.int16)
    kc = torch.full((L, pages, P, Hkv, D), workloads.SENTINEL, dtype=torch.int16, device="cuda")
    vc = kc.clone()
    pos = to_dev(np.arange(790, 800, dtype=np.int32))
    table = to_dev(np.zeros(1, np.int32))
    torch.cuda.synchronize()                            # the fills ran on torch's stream
    def call(st):
        fr.fr_decode_chain_persistent(x, gate, sc, sh, res, q8, EPS, 56.0, qkv, pos, 1e4,
                                      fr.ROPE_HALF, qo, kc, vc, table, pages, P, pages, None,
                                      L, S, T, H, Hq, Hkv, D, fr.F16, stream=st)
    return call, [res[1:], q8, qo], [kc, vc]          # res[0] is the chain's input


CASES = [("resid_rmsnorm_fp8", case_resid_rmsnorm_fp8, 1), ("adarms", case_adarms, 1),
         ("qkv", case_qkv, 1), ("gated_act_fp8", case_gated_act_fp8, 1),
         ("gemm_gated_act_fp8", case_gemm, 1), ("fp4_norm_producers", case_fp4_norms, 3),
         ("layernorm_fp8_mxfp4", case_layernorm, 2), ("gated_act_mxfp4", case_gated_act_mxfp4, 1),
         ("qk_norm_rope", case_qk_norm_rope, 1), ("gemm_pack_weights", case_pack_weights, 1),
         ("decode_chain_persistent", case_chain_persistent, 1)]


def _bits(t):
    return t.view(torch.uint8).cpu().numpy().copy()


@pytest.mark.parametrize("name,make,launches", CASES, ids=[c[0] for c in CASES])
def test_entry_point_under_graph_capture(fr, name, make, launches):
    from memory_bound_amd.hipgraph import HipGraph
    announce(f"graph capture: {name}")
    stream = torch.cuda.Stream()
    made = make(fr)
    call, outs = made[0], made[1]
    kept = made[2] if len(made) > 2 else []            # checked, not overwritten
    with torch.cuda.stream(stream):
        call(stream)
    torch.cuda.synchronize()
    want = [_bits(o) for o in outs]
    want_kept = [_bits(o) for o in kept]
    g = HipGraph(stream, lambda: call(stream))
    assert g.kernel_node_count() == launches
    assert len(g.nodes()) == launches                  # nothing but the kernels
    for rep in range(REPLAYS):
        with torch.cuda.stream(stream):                # eager work between replays
            for o in outs:
                o.view(torch.uint8).fill_(0x5A + rep)
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        for o, w in zip(outs + kept, want + want_kept):
            assert np.array_equal(_bits(o), w), f"{name}: replay {rep} differs from the eager call"
