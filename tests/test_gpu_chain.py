"""The decoder-step chain under a HIP graph: 10 flow steps x 18 layers x
(gate + residual + AdaRMSNorm + FP8, then QKV split + RoPE + KV write) at 10
tokens, captured once and replayed, against the oracle running the same 360
calls in the same order."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import announce, check16, check_exact, check_fp8, to_dev, to_host

pytestmark = pytest.mark.gpu

F16 = 0
EPS = 1e-6
THETA = 1e4


def oracle_chain(ci):
    d = ci["dims"]
    L, S, T, H = d["layers"], d["steps"], d["T"], d["H"]
    Hq, Hkv, D, P = d["Hq"], d["Hkv"], d["D"], d["page_size"]
    res = np.empty((L * S + 1, T, H), np.uint16)
    res[0] = ci["r0"]
    q8 = np.empty((L * S, T, H), np.uint8)
    q_out = np.empty((L, T, Hq, D), np.uint16)
    kc, vc = ci["k_cache"].copy(), ci["v_cache"].copy()
    n = 0
    for s in range(S):
        for l in range(L):
            res[n + 1], q8[n], _ = oracle.adarms_gate_res_fp8(
                ci["x"][l], ci["gate"][n], res[n], ci["ada_scale"][n],
                ci["ada_shift"][n], EPS, oracle.Q_STATIC, 56.0, F16)
            q_out[l], err = oracle.qkv_normrope_kvwrite(
                ci["qkv"][l], None, None, EPS, ci["positions"], THETA,
                oracle.ROPE_HALF, kc[l], vc[l], ci["page_table"], P, Hq, Hkv,
                D, F16)
            assert err == 0
            n += 1
    return res, q8, q_out, kc, vc


class DeviceChain:
    def __init__(self, fr, ci, stream):
        self.fr, self.ci, self.stream = fr, ci, stream
        d = ci["dims"]
        self.d = d
        L, S, T, H = d["layers"], d["steps"], d["T"], d["H"]
        self.x = to_dev(ci["x"])
        self.qkv = to_dev(ci["qkv"])
        self.gate = to_dev(ci["gate"])
        self.sc = to_dev(ci["ada_scale"])
        self.sh = to_dev(ci["ada_shift"])
        self.res = torch.empty((L * S + 1, T, H), dtype=torch.int16, device="cuda")
        self.res[0] = to_dev(ci["r0"])
        self.q8 = torch.empty((L * S, T, H), dtype=torch.uint8, device="cuda")
        self.q_out = torch.empty((L, T, d["Hq"], d["D"]), dtype=torch.int16,
                                 device="cuda")
        self.kc = to_dev(ci["k_cache"])
        self.vc = to_dev(ci["v_cache"])
        self.pos = to_dev(ci["positions"])
        self.table = to_dev(ci["page_table"])

    def poison(self):
        self.res[1:].fill_(0x7E01)
        self.q8.fill_(0x7F)
        self.q_out.fill_(0x7E01)

    def run(self):
        fr, d, s = self.fr, self.d, self.stream
        L, S, T, H = d["layers"], d["steps"], d["T"], d["H"]
        n = 0
        for _ in range(S):
            for l in range(L):
                fr.fr_adarms_gate_res_fp8(
                    self.x[l], self.gate[n], self.res[n], self.res[n + 1],
                    self.sc[n], self.sh[n], EPS, self.q8[n], fr.Q_STATIC, 56.0,
                    None, T, H, fr.F16, stream=s)
                fr.fr_qkv_normrope_kvwrite(
                    self.qkv[l], None, None, EPS, self.pos, THETA, fr.ROPE_HALF,
                    self.q_out[l], self.kc[l], self.vc[l], self.table, 1,
                    d["page_size"], 1, None, T, d["Hq"], d["Hkv"], d["D"],
                    fr.F16, stream=s)
                n += 1

    def host(self):
        return (to_host(self.res, np.uint16), to_host(self.q8, np.uint8),
                to_host(self.q_out, np.uint16), to_host(self.kc, np.uint16),
                to_host(self.vc, np.uint16))


def compare(got, want):
    res_g, q8_g, q_g, kc_g, vc_g = got
    res_o, q8_o, q_o, kc_o, vc_o = want
    check_exact(res_g, res_o, "residual chain")
    check_fp8(q8_g, q8_o, "fp8 outputs")
    check16(q_g, q_o, F16, "q_out")
    written = kc_o != workloads.SENTINEL
    check_exact(kc_g[~written], kc_o[~written], "k_cache untouched")
    check16(kc_g[written], kc_o[written], F16, "k_cache")
    check_exact(vc_g, vc_o, "v_cache")


def test_decode_chain_eager_and_graph():
    import memory_bound_amd as fr
    from memory_bound_amd.hipgraph import HipGraph
    announce("decode chain: 18 layers x 10 steps, eager then hipGraph")
    ci = workloads.chain_inputs()
    want = oracle_chain(ci)
    stream = torch.cuda.Stream()
    chain = DeviceChain(fr, ci, stream)
    chain.poison()
    chain.run()                                  # eager (also loads kernels)
    stream.synchronize()
    compare(chain.host(), want)

    graph = HipGraph(stream, chain.run)
    assert graph.kernel_node_count() == 360
    for _ in range(3):
        chain.poison()                           # eager work between replays
        torch.cuda.synchronize()
        graph.launch()
        stream.synchronize()
        compare(chain.host(), want)


def test_decode_chain_persistent_kernel():
    """The same 360 ops in one persistent launch, against the oracle; run
    twice with poisoned outputs in between (the second run must match too)."""
    import memory_bound_amd as fr
    announce("decode chain: persistent kernel")
    ci = workloads.chain_inputs()
    want = oracle_chain(ci)
    stream = torch.cuda.Stream()
    ch = DeviceChain(fr, ci, stream)
    d = ch.d
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        ch.poison()
        ch.kc.copy_(to_dev(ci["k_cache"]))
        ch.vc.copy_(to_dev(ci["v_cache"]))
        fr.fr_decode_chain_persistent(
            ch.x, ch.gate, ch.sc, ch.sh, ch.res, ch.q8, EPS, 56.0, ch.qkv,
            ch.pos, THETA, fr.ROPE_HALF, ch.q_out, ch.kc, ch.vc, ch.table, 1,
            d["page_size"], 1, err, d["layers"], d["steps"], d["T"], d["H"],
            d["Hq"], d["Hkv"], d["D"], fr.F16, stream=stream)
        stream.synchronize()
        compare(ch.host(), want)
        assert int(err.item()) == 0


SMALL_CHAINS = [
    # (name, L, S, T, H, Hq, Hkv, D, P, pages, dtype, style, theta, mult, seed)
    ("bf16_interleaved_T17_H512", 3, 2, 17, 512, 4, 3, 64, 8, 4, 1, 1, 5e5, 40.0, 909),
    # rows that do not fill every lane's chunks (the guarded kernel form).
    # Rows over 512 values are split over four waves of 4-value chunks: 768
    # (the fourth wave idle), 528 (the third wave 4 chunks, the fourth idle),
    # 1008 (the fourth wave 60 of 64 lanes); 256 is one wave of 8-value
    # chunks with half the lanes idle
    ("f16_H768_T10", 2, 3, 10, 768, 8, 1, 256, 1024, 1, 0, 0, 1e4, 56.0, 910),
    ("bf16_H256_T5", 2, 2, 5, 256, 2, 2, 128, 4, 3, 1, 0, 1e6, 56.0, 911),
    ("f16_H528_T3", 2, 2, 3, 528, 2, 1, 64, 16, 1, 0, 1, 1e4, 56.0, 912),
    ("f16_H1008_T1", 1, 3, 1, 1008, 1, 1, 256, 1024, 1, 0, 0, 1e4, 56.0, 914),
    # the most tokens a chain takes (64), full 1024-value rows
    ("bf16_H1024_T64", 2, 2, 64, 1024, 8, 2, 128, 16, 8, 1, 0, 1e6, 40.0, 913),
]


@pytest.mark.parametrize("case", SMALL_CHAINS, ids=lambda c: c[0])
def test_decode_chain_persistent_small(case):
    """Smaller chains through the persistent kernel against the oracle
    replaying the same calls: bf16 / interleaved RoPE / 3 KV heads / 17
    tokens (two rows per wave for some waves) / a paged table, and widths
    that do not fill whole 512-value lane rows."""
    import memory_bound_amd as fr
    name, L, S, T, H, Hq, Hkv, D, P, pages, BF, style, theta, mult, seed = case
    announce(f"decode chain persistent: {name}")
    rng = np.random.default_rng(seed)
    N = L * S
    x = workloads.to16(rng.standard_normal((L, T, H), dtype=np.float32), BF)
    gate = workloads.to16(0.1 * rng.standard_normal((N, T, H), dtype=np.float32), BF)
    sc = workloads.to16(0.1 * rng.standard_normal((N, T, H), dtype=np.float32), BF)
    sh = workloads.to16(0.1 * rng.standard_normal((N, T, H), dtype=np.float32), BF)
    r0 = workloads.to16(rng.standard_normal((T, H), dtype=np.float32), BF)
    qkv = workloads.to16(rng.standard_normal((L, T, (Hq + 2 * Hkv) * D), dtype=np.float32), BF)
    pos = np.arange(5, 5 + T, dtype=np.int32)
    table = rng.permutation(pages).astype(np.int32)
    kc0 = np.full((L, pages, P, Hkv, D), workloads.SENTINEL, np.uint16)
    vc0 = kc0.copy()
    # oracle
    res = np.empty((N + 1, T, H), np.uint16)
    res[0] = r0
    q8 = np.empty((N, T, H), np.uint8)
    qo = np.empty((L, T, Hq, D), np.uint16)
    kc, vc = kc0.copy(), vc0.copy()
    n = 0
    for s in range(S):
        for l in range(L):
            res[n + 1], q8[n], _ = oracle.adarms_gate_res_fp8(
                x[l], gate[n], res[n], sc[n], sh[n], EPS, oracle.Q_STATIC, mult, BF)
            qo[l], err = oracle.qkv_normrope_kvwrite(
                qkv[l], None, None, EPS, pos, theta, style, kc[l], vc[l], table, P, Hq,
                Hkv, D, BF)
            assert err == 0
            n += 1
    # device
    dres = torch.full((N + 1, T, H), 0x7E01, dtype=torch.int16, device="cuda")
    dres[0] = to_dev(r0)
    dq8 = torch.full((N, T, H), 0x7F, dtype=torch.uint8, device="cuda")
    dqo = torch.full((L, T, Hq, D), 0x7E01, dtype=torch.int16, device="cuda")
    dkc, dvc = to_dev(kc0), to_dev(vc0)
    fr.fr_decode_chain_persistent(
        to_dev(x), to_dev(gate), to_dev(sc), to_dev(sh), dres, dq8, EPS, mult,
        to_dev(qkv), to_dev(pos), theta, style, dqo, dkc, dvc,
        to_dev(table), pages, P, pages, None, L, S, T, H, Hq, Hkv, D, BF)
    torch.cuda.synchronize()
    check_exact(to_host(dres, np.uint16), res, "residual chain")
    check_fp8(to_host(dq8, np.uint8), q8, "fp8 outputs")
    check16(to_host(dqo, np.uint16), qo, BF, "q_out")
    kg = to_host(dkc, np.uint16)
    written = kc != workloads.SENTINEL
    check_exact(kg[~written], kc[~written], "k_cache untouched")
    check16(kg[written], kc[written], BF, "k_cache")
    check_exact(to_host(dvc, np.uint16), vc, "v_cache")
