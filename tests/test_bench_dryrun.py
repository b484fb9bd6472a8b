"""CPU dry run of bench.py: every call it makes into the HIP library and the
measurement support library is intercepted, and the byte extent each pointer
argument needs (from the C-ABI definitions in include/fr.h and
tests/gpu_support.hip) is checked against the allocation the pointer falls
in.  Device tensors are replaced by host tensors and nothing runs on a GPU.

Regression test for a benchmark bug that launched the Qwen3 prefill QKV op
with T = 1024 on buffers sized for 128 tokens (a closure read its token
count at call time, after a later loop had re-bound it)."""
import contextlib
import ctypes
import importlib
import sys
import types

import numpy as np
import pytest
import torch


class _Allocs:
    def __init__(self):
        self.spans = []

    def track(self, t):
        st = t.untyped_storage()
        self.spans.append((st.data_ptr(), st.data_ptr() + st.nbytes()))
        return t

    def need(self, op, p, nbytes, what):
        if p is None:
            raise AssertionError(f"{op}: {what} is NULL")
        a = p if isinstance(p, int) else p.data_ptr()
        for s, e in reversed(self.spans):          # the latest allocation at an address
            if s <= a < e:
                assert a + nbytes <= e, (f"{op}: {what} needs {nbytes} bytes at offset "
                                         f"{a - s} of a {e - s}-byte allocation")
                return
        raise AssertionError(f"{op}: {what} is not inside any allocation")


def _fake_library(al, calls):
    fr = types.ModuleType("memory_bound_amd")
    for name, val in dict(F16=0, BF16=1, W_NONE=0, W_MUL=1, W_ONE_PLUS=2, Q_STATIC=0,
                          Q_TOKEN=1, ACT_SWIGLU=0, ACT_GEGLU_TANH=1, ACT_SQRELU=2,
                          ROPE_HALF=0, ROPE_INTERLEAVED=1, NORM_NONE=0, NORM_RMS=1,
                          NORM_LAYER=2).items():
        setattr(fr, name, val)
    need = al.need

    def resid(x, r, ro, w, wmode, eps, q, qmode, s, sc, T, H, dt, stream=None):
        calls.append("resid")
        for p, n in ((x, "x"), (r, "residual"), (ro, "residual_out")):
            need("resid", p, T * H * 2, n)
        if wmode != 0:
            need("resid", w, H * 2, "weight")
        need("resid", q, T * H, "out_fp8")
        if qmode == 1:
            need("resid", sc, T * 4, "out_scales")

    def ada(x, g, r, ro, scl, sh, eps, q, qmode, s, sc, T, H, dt, stream=None):
        calls.append("ada")
        for p, n in ((x, "x"), (g, "gate"), (r, "residual"), (ro, "residual_out"),
                     (scl, "ada_scale"), (sh, "ada_shift")):
            need("ada", p, T * H * 2, n)
        need("ada", q, T * H, "out_fp8")
        if qmode == 1:
            need("ada", sc, T * 4, "out_scales")

    def qkv(qkv_, qw, kw, eps, pos, theta, style, qo, kc, vc, tab, tl, P, npg, err, T, Hq,
            Hkv, D, dt, stream=None, q_scale=1.0):
        calls.append("qkv")
        need("qkv", qkv_, T * (Hq + 2 * Hkv) * D * 2, "qkv")
        for w, n in ((qw, "q_norm_w"), (kw, "k_norm_w")):
            if w is not None:
                need("qkv", w, D * 2, n)
        need("qkv", pos, T * 4, "positions")
        need("qkv", qo, T * Hq * D * 2, "q_out")
        need("qkv", kc, npg * P * Hkv * D * 2, "k_cache")
        need("qkv", vc, npg * P * Hkv * D * 2, "v_cache")
        need("qkv", tab, tl * 4, "page_table")
        if err is not None:
            need("qkv", err, 4, "err_flag")
        # every position maps to a slot inside the caches
        pa = np.ctypeslib.as_array((ctypes.c_int32 * T).from_address(pos.data_ptr()))
        ta = np.ctypeslib.as_array((ctypes.c_int32 * tl).from_address(tab.data_ptr()))
        assert np.all((pa >= 0) & (pa // P < tl)), "position outside the page table"
        assert np.all((ta[pa // P] >= 0) & (ta[pa // P] < npg)), "page outside the pool"

    def act(gu, a, q, sc, T, I, dt, stream=None):
        calls.append("act")
        need("act", gu, T * 2 * I * 2, "gate_up")
        need("act", q, T * I, "out_fp8")
        need("act", sc, T * (I // 128) * 4, "out_scales")

    def gemm(a, a_s, wp, ws, act_, q, sc, M, K, I, stream=None):
        calls.append("gemm")
        need("gemm", a, M * K, "a")
        need("gemm", a_s, M * (K // 128) * 4, "a_scales")
        need("gemm", wp, 2 * I * K, "w_packed")
        need("gemm", ws, (2 * I // 128) * (K // 128) * 4, "w_scales")
        need("gemm", q, M * I, "out_fp8")
        need("gemm", sc, M * (I // 128) * 4, "out_scales")

    def pack(w, wp, N, K, stream=None):
        need("pack", w, N * K, "w")
        need("pack", wp, N * K, "w_packed")

    def mx_norm(x, r, ro, w, wmode, eps, q, s, T, H, dt, stream=None):
        calls.append("mx_norm")
        for p, n in ((x, "x"), (r, "residual"), (ro, "residual_out")):
            need("mx_norm", p, T * H * 2, n)
        need("mx_norm", q, T * H // 2, "out_fp4")
        need("mx_norm", s, T * H // 32, "out_scales")

    def nv_norm(x, r, ro, w, wmode, eps, g, q, s, T, H, dt, stream=None):
        calls.append("nv_norm")
        assert g > 0
        for p, n in ((x, "x"), (r, "residual"), (ro, "residual_out")):
            need("nv_norm", p, T * H * 2, n)
        need("nv_norm", q, T * H // 2, "out_fp4")
        need("nv_norm", s, T * H // 16, "out_scales")

    def mx_act(gu, a, q, s, T, I, dt, stream=None):
        calls.append("mx_act")
        need("mx_act", gu, T * 2 * I * 2, "gate_up")
        need("mx_act", q, T * I // 2, "out_fp4")
        need("mx_act", s, T * I // 32, "out_scales")

    def ln_mx(x, r, ro, w, b, eps, q, s, T, H, dt, stream=None):
        calls.append("ln_mx")
        for p, n in ((x, "x"), (r, "residual"), (ro, "residual_out")):
            need("ln_mx", p, T * H * 2, n)
        need("ln_mx", q, T * H // 2, "out_fp4")
        need("ln_mx", s, T * H // 32, "out_scales")

    def ln_nv(x, r, ro, w, b, eps, g, q, s, T, H, dt, stream=None):
        calls.append("ln_nv")
        assert g > 0
        for p, n in ((x, "x"), (r, "residual"), (ro, "residual_out")):
            need("ln_nv", p, T * H * 2, n)
        need("ln_nv", w, H * 2, "weight")
        need("ln_nv", q, T * H // 2, "out_fp4")
        need("ln_nv", s, T * H // 16, "out_scales")

    def qknr(qkv_, kind, full, qw, qb, kw, kb, eps, pos, rd, sec, theta, style, qs, qo, ko,
             vo, T, Hq, Hkv, D, dt, stream=None):
        calls.append("qknr")
        need("qknr", qkv_, T * (Hq + 2 * Hkv) * D * 2, "qkv")
        need("qknr", pos, T * 4 * (3 if rd == 3 else 1), "positions")
        need("qknr", qo, T * Hq * D * 2, "q_out")
        need("qknr", ko, T * Hkv * D * 2, "k_out")
        need("qknr", vo, T * Hkv * D * 2, "v_out")

    def chain(x, gate, scl, sh, res, q8, eps, s, qkv_, pos, theta, style, qo, kc, vc, tab,
              tl, P, npg, err, L, S, T, H, Hq, Hkv, D, dt, stream=None):
        calls.append("chain")
        N = L * S
        need("chain", x, L * T * H * 2, "x")
        for p, n in ((gate, "gate"), (scl, "ada_scale"), (sh, "ada_shift")):
            need("chain", p, N * T * H * 2, n)
        need("chain", res, (N + 1) * T * H * 2, "residual")
        need("chain", q8, N * T * H, "out_fp8")
        need("chain", qkv_, L * T * (Hq + 2 * Hkv) * D * 2, "qkv")
        need("chain", qo, L * T * Hq * D * 2, "q_out")
        need("chain", kc, L * npg * P * Hkv * D * 2, "k_cache")
        need("chain", vc, L * npg * P * Hkv * D * 2, "v_cache")

    for name, fn in (("fr_resid_rmsnorm_fp8", resid), ("fr_adarms_gate_res_fp8", ada),
                     ("fr_qkv_normrope_kvwrite", qkv), ("fr_gated_act_fp8", act),
                     ("fr_gemm_gated_act_fp8", gemm), ("fr_gemm_pack_weights", pack),
                     ("fr_resid_rmsnorm_mxfp4", mx_norm), ("fr_gated_act_mxfp4", mx_act),
                     ("fr_resid_rmsnorm_nvfp4", nv_norm),
                     ("fr_resid_layernorm_mxfp4", ln_mx), ("fr_resid_layernorm_nvfp4", ln_nv),
                     ("fr_qk_norm_rope", qknr),
                     ("fr_decode_chain_persistent", chain)):
        setattr(fr, name, fn)
    hg = types.ModuleType("memory_bound_amd.hipgraph")

    class HipGraph:
        def __init__(self, stream, fn):
            fn()

        def kernel_node_count(self):
            return 360

        def launch(self):
            pass
    hg.HipGraph = HipGraph
    return fr, hg


class _Support:
    def __init__(self, al, calls):
        self.al, self.calls = al, calls

    def stream_copy(self, src, dst, n16, nt, stream):
        self.calls.append("copy")
        self.al.need("stream_copy", src, n16 * 16, "src")
        self.al.need("stream_copy", dst, n16 * 16, "dst")
        return 0


class _Event:
    def __init__(self, **kw):
        pass

    def record(self, *a):
        pass

    def elapsed_time(self, other):
        return 0.01


class _Stream:
    cuda_stream = 0

    def synchronize(self):
        pass


def test_bench_calls_stay_inside_their_buffers(monkeypatch):
    al, calls = _Allocs(), []

    def host(fn):
        def f(*a, **k):
            k.pop("device", None)
            return al.track(fn(*a, **k))
        return f
    for name in ("empty", "zeros", "full", "empty_like", "zeros_like", "full_like"):
        monkeypatch.setattr(torch, name, host(getattr(torch, name)))
    clone = torch.Tensor.clone
    monkeypatch.setattr(torch.Tensor, "clone", lambda self, *a, **k: al.track(clone(self, *a, **k)))
    monkeypatch.setattr(torch.Tensor, "cuda", lambda self, *a, **k: al.track(clone(self)))
    monkeypatch.setattr(torch.cuda, "Stream", lambda *a, **k: _Stream())
    monkeypatch.setattr(torch.cuda, "stream", lambda s: contextlib.nullcontext())
    monkeypatch.setattr(torch.cuda, "Event", _Event)
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a: None)
    monkeypatch.setattr(torch.cuda, "init", lambda: None)
    fr, hg = _fake_library(al, calls)
    monkeypatch.setitem(sys.modules, "memory_bound_amd", fr)
    monkeypatch.setitem(sys.modules, "memory_bound_amd.hipgraph", hg)
    bench = importlib.import_module("bench")
    monkeypatch.setattr(bench, "load_support", lambda: _Support(al, calls))
    monkeypatch.setattr(bench, "_LEAD", {})
    monkeypatch.setattr(bench, "_COPY_BUFS", {})
    # small rotations, lead-ins and reference copies: the same call sequence
    # and shapes with less host memory
    monkeypatch.setattr(bench, "LEAD_COPIES", 1)
    monkeypatch.setattr(bench, "LEAD_BYTES", 1 << 20)
    monkeypatch.setattr(bench, "ROTATION_BYTES", 1 << 20)
    monkeypatch.setattr(bench, "WEIGHT_ROTATION_BYTES", 1 << 20)
    monkeypatch.setattr(bench, "COPY_BYTES", 512 << 20)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "4", "--warmup", "1",
                                      "--no-cpu-baseline", "--chain-replays", "2"])
    bench.main()
    for op in ("resid", "ada", "qkv", "act", "gemm", "mx_norm", "nv_norm", "mx_act", "ln_mx", "ln_nv", "qknr",
               "chain", "copy"):
        assert op in calls, f"bench made no {op} call"
