"""Benchmark of the fused layer-boundary kernels on one MI355X.

One step = one pass of the whole hot path over one batch of 8192 tokens:
  (a)  residual add + RMSNorm(w) + per-token FP8, hidden 4096, bf16
  (a') gate + residual + AdaRMSNorm + static FP8, hidden 1024, fp16
  (b)  packed QKV split + Q/K RMSNorm + RoPE + paged KV write, 32/8 heads x 128,
       bf16, 16-token pages
  (c)  SwiGLU on interleaved gate/up + block-128 FP8, inter 12288, bf16
Inputs are seeded synthetic tensors resident in HBM before timing starts.
`value` is the step's algorithmic bytes over its time (GB/s).  The line also
carries per-op microseconds, the roofline of the dominant kernel (measured
with HIP events on the launch stream), a sweep of every op over 10 ... 8192
tokens with a plain streaming copy of the same traffic beside it, the
Qwen3-style prefill QKV and gated-activation configurations, the 10-token
decoder chain (18 layers x 10 steps x 2 ops) replayed as one HIP graph and as
one persistent kernel, the fused gate_up GEMM, the FP4 producers, and the
CPU oracle timed on a bounded sample of the same workload (one thread and
all threads).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBS = 8000.0
T_BIG = 8192
# Lead-in before every timed region: ~35 ms of HBM-bound device copies on the
# timed stream.  It gives the host a head start (the launches of the timed
# region are enqueued while the copies run) and brings the GPU to its
# sustained-load clocks.  Measured on MI355X: after an idle spin kernel the
# first ~25 ms of memory-bound work run 6-15% slower than in steady state
# (the activation kernel 86-94 us instead of 80-81 us), so an idle spin as
# head start would time the clock ramp instead of the kernels.
LEAD_COPIES = 100            # 1 GiB device copies (~0.33 ms each)
LEAD_BYTES = 1 << 30
# Buffer rotation: every op's launches cycle through at least this many bytes
# of distinct buffers (the last-level cache holds 256 MB), the GEMM's weight
# copies through WEIGHT_ROTATION_BYTES; copies for the achievable figures
# move COPY_BYTES each way.
ROTATION_BYTES = 512 << 20
WEIGHT_ROTATION_BYTES = 400 << 20
COPY_BYTES = 1 << 30
_LEAD = {}


def progress(msg):
    """One line per benchmark leg on stderr, before its GPU work starts."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def lead_in(torch, stream):
    if "src" not in _LEAD:
        _LEAD["src"] = torch.zeros(LEAD_BYTES, dtype=torch.uint8, device="cuda")
        _LEAD["dst"] = torch.empty_like(_LEAD["src"])
    with torch.cuda.stream(stream):
        for _ in range(LEAD_COPIES):
            _LEAD["dst"].copy_(_LEAD["src"])


GROUP_REPEATS = 3
EPS = 1e-6


def op_bytes(T=T_BIG):
    """Algorithmic HBM bytes per call at T tokens (each input read once, each
    output written once; 16-bit values 2 B, FP8 1 B, fp32 scales 4 B, int32
    4 B; page-table entries: one per 16-token page touched)."""
    H_a, H_ada = 4096, 1024
    Hq, Hkv, D, P = 32, 8, 128, 16
    I = 12288
    return {
        # x, residual in; residual_out, fp8 out; weight; per-token scales
        "resid_rmsnorm_fp8": T * H_a * (2 + 2 + 2 + 1) + 2 * H_a + 4 * T,
        # x, gate, residual, scale, shift in; residual_out, fp8 out
        "adarms_gate_res_fp8": T * H_ada * (5 * 2 + 2 + 1),
        # qkv in; q_out + k + v out; positions; page-table entries; 2 norm weights
        "qkv_normrope_kvwrite": 2 * T * (Hq + 2 * Hkv) * D * 2 + 4 * T
        + 4 * (-(-T // P)) + 2 * D * 2,
        # gate_up in; fp8 out; block scales
        "gated_act_fp8": T * 2 * I * 2 + T * I + 4 * T * (I // 128),
    }


def kernel_source_hash(name):
    from bench_profile import code_hash
    return code_hash(os.path.join(HERE, "memory_bound_amd", "csrc", name))


def load_traffic(kernel_file, per_launch_bytes_key):
    """HBM traffic of the dominant kernel from the committed rocprofv3 PMC
    summary, only if it was taken on the current kernel source."""
    path = os.path.join(HERE, "profiles", "gated_act_fp8_T8192_I12288_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("code_sha256_16") != kernel_source_hash(kernel_file):
        return None
    return d.get(per_launch_bytes_key)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--chain-replays", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--pmc-pass", action="store_true",
                    help="only run each 8192-token op 3 times plus a 1 GiB "
                         "device copy (for rocprofv3 counter collection)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the fused ops are row-independent "
              "and run on one GPU's share of tokens; multi-GPU runs are not "
              "part of this benchmark (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import memory_bound_amd as fr
    from memory_bound_amd.hipgraph import HipGraph

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda()
        return torch.from_numpy(a).cuda()

    torch.cuda.init()
    stream = torch.cuda.Stream()
    T = T_BIG
    t0 = time.time()

    # ---- inputs (seeded, synthetic, resident in HBM) ----------------------
    # Every op gets several device copies of its buffers, used in rotation,
    # so that repeated launches of one op never find their data in the
    # 256 MB last-level cache (each op's rotation spans >= 512 MB).
    def sets(d, nbytes_op):
        if args.pmc_pass:
            return [d]
        r = max(2, -(-ROTATION_BYTES // nbytes_op))
        out = [d]
        for _ in range(r - 1):
            out.append({k: (v.clone() if v is not None else None) for k, v in d.items()})
        return out

    progress("inputs")
    nbytes = op_bytes()
    ri = workloads.resid_rmsnorm_inputs(T, 4096, workloads.BF16, 105, outliers=True)
    A = {k: dev(v) for k, v in ri.items()}
    A["ro"] = torch.empty_like(A["x"])
    A["q"] = torch.empty((T, 4096), dtype=torch.uint8, device="cuda")
    A["sc"] = torch.empty((T,), dtype=torch.float32, device="cuda")
    A = sets(A, nbytes["resid_rmsnorm_fp8"])

    ai = workloads.adarms_inputs(T, 1024, workloads.F16, 102)
    Ad = {k: dev(v) for k, v in ai.items()}
    Ad["ro"] = torch.empty_like(Ad["x"])
    Ad["q"] = torch.empty((T, 1024), dtype=torch.uint8, device="cuda")
    Ad = sets(Ad, nbytes["adarms_gate_res_fp8"])

    qi = workloads.qkv_inputs(T, 32, 8, 128, workloads.BF16, 103, page_size=16,
                              num_pages=512)
    B = {k: dev(v) for k, v in qi.items()}
    B["q_out"] = torch.empty((T, 32, 128), dtype=torch.int16, device="cuda")
    B["err"] = torch.zeros(1, dtype=torch.int32, device="cuda")
    B = sets(B, nbytes["qkv_normrope_kvwrite"])

    gi = workloads.gated_act_inputs(T, 12288, workloads.BF16, 105, outliers=True)
    C = {"gu": dev(gi["gate_up"])}
    C["q"] = torch.empty((T, 12288), dtype=torch.uint8, device="cuda")
    C["sc"] = torch.empty((T, 96), dtype=torch.float32, device="cuda")
    C = sets(C, nbytes["gated_act_fp8"])
    del ri, ai, qi, gi
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    # Each op takes (launch index i, tokens n).  Below 8192 tokens a launch
    # uses one block of n rows of one buffer set, rotating over every (set,
    # block) pair, so the rotation spans the same >= 512 MB at every n.
    def pick(sets_, i, n):
        stride = -(-n // 16) * 16            # blocks start at multiples of 16 rows (aligned)
        nb = max(1, T // stride)
        k = i % (len(sets_) * nb)
        return sets_[k % len(sets_)], (k // len(sets_)) % nb * stride

    def op_a(i, n=T):
        d, r = pick(A, i, n)
        fr.fr_resid_rmsnorm_fp8(d["x"][r:], d["residual"][r:], d["ro"][r:], d["weight"],
                                fr.W_MUL, EPS, d["q"][r:], fr.Q_TOKEN, 0.0, d["sc"][r:],
                                n, 4096, fr.BF16, stream=stream)

    def op_ada(i, n=T):
        d, r = pick(Ad, i, n)
        fr.fr_adarms_gate_res_fp8(d["x"][r:], d["gate"][r:], d["residual"][r:], d["ro"][r:],
                                  d["ada_scale"][r:], d["ada_shift"][r:], EPS, d["q"][r:],
                                  fr.Q_STATIC, 56.0, None, n, 1024, fr.F16,
                                  stream=stream)

    def op_b(i, n=T):
        d, r = pick(B, i, n)
        fr.fr_qkv_normrope_kvwrite(d["qkv"][r:], d["q_norm_w"], d["k_norm_w"], EPS,
                                   d["positions"][r:], 1e6, fr.ROPE_HALF, d["q_out"][r:],
                                   d["k_cache"], d["v_cache"], d["page_table"],
                                   512, 16, 512, d["err"], n, 32, 8, 128,
                                   fr.BF16, stream=stream)

    def op_c(i, n=T):
        d, r = pick(C, i, n)
        fr.fr_gated_act_fp8(d["gu"][r:], fr.ACT_SWIGLU, d["q"][r:], d["sc"][r:], n, 12288,
                            fr.BF16, stream=stream)

    ops = [("resid_rmsnorm_fp8", op_a), ("adarms_gate_res_fp8", op_ada),
           ("qkv_normrope_kvwrite", op_b), ("gated_act_fp8", op_c)]
    step_bytes = sum(nbytes.values())

    if args.pmc_pass:
        # calibration copy of known size (1 GiB read + 1 GiB written), then
        # each op three times
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(3):
                dst.copy_(src)
            for i in range(3):
                for _, f in ops:
                    f(i)
        torch.cuda.synchronize()
        run_mxfp4(torch, fr, workloads, dev, stream, 3, timed=False)
        run_qknorm(torch, fr, workloads, dev, stream, 3, timed=False, only="wan")
        run_gemm_act(torch, fr, workloads, dev, stream, reps=3, timed=False,
                     shapes=((128, 2048, 6144),))
        print(json.dumps({"pmc_pass": True, "copy_bytes_each_way": COPY_BYTES,
                          "op_bytes": nbytes}), flush=True)
        return

    def ev():
        return torch.cuda.Event(enable_timing=True)

    progress("timed step region")
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            for _, f in ops:
                f(i)
        stream.synchronize()

        # ---- timed region 1: K steps in layer order ----------------------
        # Events only at the ends (an event record between kernels costs a
        # few microseconds on this runtime).  The lead-in copies first let
        # the host enqueue the whole region ahead of the GPU, so host-side
        # launch cost opens no gaps, and bring the clocks to sustained load
        # (the lead-in is before the start event).
        start, end = ev(), ev()
        torch.cuda.synchronize()
        lead_in(torch, stream)
        start.record(stream)
        for k in range(args.steps):
            for _, f in ops:
                f(k)
        end.record(stream)
        torch.cuda.synchronize()
        ms_per_step = start.elapsed_time(end) / args.steps

        # ---- timed region 2: each op K times back to back ----------------
        # (buffer rotation keeps every launch reading from HBM); the average
        # launch duration of each op is its group's event time / K.  The
        # region is run GROUP_REPEATS times and the median is reported
        # (launch-to-launch variation on these GPUs is a few percent).
        per_op = {}
        reps = {name: [] for name, _ in ops}
        grouped = []
        for _ in range(GROUP_REPEATS):
            lead_in(torch, stream)
            marks = [ev() for _ in range(len(ops) + 1)]
            marks[0].record(stream)
            for j, (_, f) in enumerate(ops):
                for k in range(args.steps):
                    f(k)
                marks[j + 1].record(stream)
            torch.cuda.synchronize()
            for j, (name, _) in enumerate(ops):
                reps[name].append(marks[j].elapsed_time(marks[j + 1]) * 1e3 / args.steps)
            grouped.append(marks[0].elapsed_time(marks[-1]) / args.steps)
        for name, _ in ops:
            us = float(np.median(reps[name]))
            per_op[name] = {
                "bytes": nbytes[name],
                "us_per_launch": round(us, 3),
                "us_per_launch_repeats": [round(v, 2) for v in reps[name]],
                "GBps": round(nbytes[name] / (us * 1e-6) / 1e9, 1),
                "frac_of_peak": round(nbytes[name] / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                "buffer_sets": len({"resid_rmsnorm_fp8": A, "adarms_gate_res_fp8": Ad,
                                    "qkv_normrope_kvwrite": B, "gated_act_fp8": C}[name]),
            }
        ms_grouped = float(np.median(grouped))
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    dom = "gated_act_fp8"
    dom_us = per_op[dom]["us_per_launch"]
    achieved = nbytes[dom] / (dom_us * 1e-6) / 1e9
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_HBM_GBS, 4),
        "traffic": load_traffic("fr_act.hip", "hbm_bytes_per_launch"),
        "algorithmic_bytes_per_launch": nbytes[dom],
        "avg_launch_us": dom_us,
    }

    progress("decoder chain (graph + persistent)")
    # ---- 10-token decoder chain: 18 layers x 10 steps, one HIP graph -----
    chain = run_chain(torch, fr, workloads, HipGraph, dev, stream,
                      args.chain_replays)

    progress("10-token standalone calls")
    # ---- standalone 10-token decode-boundary calls (median of 50) --------
    small = run_small(torch, fr, workloads, dev, stream)

    progress("fused gate_up GEMM")
    # ---- gate_up FP8 GEMM fused with SwiGLU + block-128 FP8 --------------
    gemm = run_gemm_act(torch, fr, workloads, dev, stream)

    progress("FP4 producers (MX and NV)")
    # ---- MX FP4 producers at 8192 tokens ---------------------------------
    mxfp4 = run_mxfp4(torch, fr, workloads, dev, stream, args.steps)

    progress("Q/K norm + RoPE variants")
    # ---- Q/K norm + RoPE variants at 8192 tokens -------------------------
    qknorm = run_qknorm(torch, fr, workloads, dev, stream, args.steps)

    progress("T sweep")
    # ---- T sweep of the four ops, with the plain-copy reference ---------
    support = load_support()
    sweep = run_t_sweep(torch, stream, dict(ops), support, args.steps)

    progress("configurations")
    # ---- the pages' other configurations (Qwen3 prefill QKV, gated act) --
    configs = run_configs(torch, fr, workloads, dev, stream)

    progress("achievable copies")
    # ---- achievable: plain copies of COPY_BYTES each way ------------------
    achievable = run_achievable(torch, stream, support)

    progress("CPU oracle baseline")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_seconds)

    line = {
        "metric": "achieved HBM GB/s (% of peak) per fused op; us/call at T=10 and T=8192",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "ms_per_step_op_grouped": round(ms_grouped, 4),
        "config": {
            "workload": "layer-boundary pass at 8192 tokens: resid+RMSNorm+FP8 "
                        "(H=4096 bf16), AdaRMSNorm+gate+FP8 (H=1024 fp16), "
                        "QKV norm+RoPE+paged KV (32/8x128 bf16), SwiGLU+block-128 "
                        "FP8 (I=12288 bf16)",
            "tokens": T,
            "step_bytes": step_bytes,
            "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        },
        "per_op": per_op,
        "roofline": roofline,
        "chain": chain,
        "decode_t10": small,
        "gemm_gated_act_fp8": gemm,
        "fp4_producers": mxfp4,
        "qk_norm_rope_variants": qknorm,
        "t_sweep": sweep,
        "configs": configs,
        "achievable": achievable,
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(line), flush=True)


T_SWEEP = (10, 128, 1024, 4096, 8192)
SWEEP_GROUPS = 7


def load_support():
    """The measurement support library (tests/gpu_support.hip, built by
    __graft_entry__.build()): its plain streaming copy is the reference for
    what a kernel moving the same bytes reaches on this GPU."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_gpu_support", os.path.join(HERE, "tests", "gpu_support.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.load()


def pct(v, q):
    return round(float(np.percentile(v, q)), 3)


def time_groups(torch, stream, f, launches, groups, lead=True):
    """Per-launch microseconds of `groups` groups of `launches` back-to-back
    launches f(i), each group after the lead-in, events at the group ends."""
    out = []
    for _ in range(groups):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        if lead:
            lead_in(torch, stream)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(launches):
                f(i)
            e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / launches)
    return out


def time_standalone(torch, stream, f, calls=50):
    """Per-call microseconds of single launches, each bracketed by events and
    synchronised (launch latency included)."""
    ts = []
    for i in range(calls + 5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        f(i)
        e1.record(stream)
        stream.synchronize()
        if i >= 5:
            ts.append(e0.elapsed_time(e1) * 1e3)
    return ts


_COPY_BUFS = {}


def copy_reference(torch, stream, support, nbytes, groups=SWEEP_GROUPS, launches=20):
    """The plain streaming copy moving `nbytes` of traffic (nbytes / 2 read,
    nbytes / 2 written), non-temporal and cacheable, buffers rotated through
    >= 512 MB; returns the faster one's median per-launch microseconds."""
    half = (nbytes // 2) // 16 * 16
    if "buf" not in _COPY_BUFS:
        _COPY_BUFS["buf"] = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    buf = _COPY_BUFS["buf"]
    buf_bytes = buf.numel()
    assert 2 * half <= buf_bytes, "copy reference larger than its buffer"
    nset = max(1, min(buf_bytes // (2 * max(half, 1)), 64))   # source / dest pairs
    base = buf.data_ptr()
    best = None
    for nt in (1, 0):
        def f(i, nt=nt):
            k = i % nset
            rc = support.stream_copy(base + 2 * k * half, base + (2 * k + 1) * half,
                                     half // 16, nt, stream.cuda_stream)
            assert rc == 0, rc
        f(0)
        us = float(np.median(time_groups(torch, stream, f, launches, max(3, groups // 2))))
        best = us if best is None else min(best, us)
    return best


def run_t_sweep(torch, stream, ops, support, steps):
    """Each op at T in {10, 128, 1024, 4096, 8192}: p10/p50/p90 over groups of
    back-to-back launches (per-launch average; each group after the lead-in,
    so the host has enqueued the group before the GPU reaches it),
    algorithmic GB/s, fraction of the 8 TB/s peak, and for T >= 1024 the
    plain streaming copy of the same traffic as the achievable reference.
    At T <= 128 the time is launch and latency, reported in microseconds
    (and single calls' medians, which include the host's launch cost)."""
    out = {}
    for name, f in ops.items():
        out[name] = {}
        for n in T_SWEEP:
            progress(f"  {name} T={n}")
            nb = op_bytes(n)[name]
            g = lambda i, n=n, f=f: f(i, n)
            g(0)
            us = time_groups(torch, stream, g, steps, SWEEP_GROUPS)
            p50 = float(np.median(us))
            e = {"bytes": nb, "us_p10": pct(us, 10), "us_p50": pct(us, 50),
                 "us_p90": pct(us, 90),
                 "GBps": round(nb / (p50 * 1e-6) / 1e9, 1),
                 "frac_of_peak": round(nb / (p50 * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            if n >= 1024:
                cu = copy_reference(torch, stream, support, nb)
                e["copy_same_bytes_us"] = round(cu, 3)
                e["copy_same_bytes_frac_of_peak"] = round(nb / (cu * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
                e["frac_of_copy"] = round(cu / p50, 4)
            else:
                st = time_standalone(torch, stream, g)
                e["standalone_us_p50"] = pct(st, 50)
            out[name][f"T{n}"] = e
    return out


def run_configs(torch, fr, workloads, dev, stream):
    """The Qwen3-style prefill QKV post-processing (S = 128, 32/8 heads x
    128 bf16, theta 1e6, 16-token pages, 512 pages, permuted table) and the
    gated activation with block-128 FP8 on [S, 2 x 6144] bf16 for S in
    {128, 192, 1024}, SwiGLU and GeGLU: per-call microseconds (single calls,
    p10/p50/p90 of 50) and back-to-back per-launch microseconds (p10/p50/p90
    over 7 groups), with algorithmic GB/s."""
    out = {}
    # every closure below binds its sizes and buffers as default arguments
    # (a free variable would be read at call time)
    Sq = 128
    qi = workloads.qkv_inputs(Sq, 32, 8, 128, workloads.BF16, 103, page_size=16,
                              num_pages=512)
    dq = {k: dev(v) for k, v in qi.items()}
    dq["q_out"] = torch.empty((Sq, 32, 128), dtype=torch.int16, device="cuda")
    dq["err"] = torch.zeros(1, dtype=torch.int32, device="cuda")

    def qkv(i, d=dq, n=Sq):
        fr.fr_qkv_normrope_kvwrite(d["qkv"], d["q_norm_w"], d["k_norm_w"], EPS,
                                   d["positions"], 1e6, fr.ROPE_HALF, d["q_out"],
                                   d["k_cache"], d["v_cache"], d["page_table"], 512,
                                   16, 512, d["err"], n, 32, 8, 128, fr.BF16,
                                   stream=stream)

    cases = [("qwen3_prefill_qkv_S128_32x8x128_bf16", qkv,
              2 * Sq * 48 * 128 * 2 + 4 * Sq + 4 * (Sq // 16) + 2 * 128 * 2)]
    I = 6144
    for Sa in (128, 192, 1024):
        gi = workloads.gated_act_inputs(Sa, I, workloads.BF16, 104)
        gu = dev(gi["gate_up"])
        q = torch.empty((Sa, I), dtype=torch.uint8, device="cuda")
        sc = torch.empty((Sa, I // 128), dtype=torch.float32, device="cuda")
        for act, an in ((fr.ACT_SWIGLU, "swiglu"), (fr.ACT_GEGLU_TANH, "geglu")):
            def f(i, gu=gu, q=q, sc=sc, n=Sa, act=act):
                fr.fr_gated_act_fp8(gu, act, q, sc, n, I, fr.BF16, stream=stream)
            cases.append((f"gated_act_{an}_S{Sa}_I{I}_bf16", f,
                          Sa * 2 * I * 2 + Sa * I + 4 * Sa * (I // 128)))
    for name, f, nb in cases:
        progress(f"  {name}")
        f(0)
        torch.cuda.synchronize()
        st = time_standalone(torch, stream, f)
        bb = time_groups(torch, stream, f, 50, SWEEP_GROUPS)
        out[name] = {"bytes": nb,
                     "standalone_us_p10": pct(st, 10), "standalone_us_p50": pct(st, 50),
                     "standalone_us_p90": pct(st, 90),
                     "back_to_back_us_p10": pct(bb, 10), "back_to_back_us_p50": pct(bb, 50),
                     "back_to_back_us_p90": pct(bb, 90),
                     "GBps_back_to_back": round(nb / (float(np.median(bb)) * 1e-6) / 1e9, 1)}
    return out


def run_achievable(torch, stream, support):
    """Plain copies of 1 GiB each way: the runtime's device-to-device copy
    (hipMemcpyAsync, through torch) and the streaming copy kernel."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)

    def d2d(i):
        dst.copy_(src)

    def sc(i, nt):
        assert support.stream_copy(src.data_ptr(), dst.data_ptr(), COPY_BYTES // 16, nt,
                                   stream.cuda_stream) == 0
    res = {}
    for name, f in (("hip_memcpy_d2d", d2d), ("stream_copy_nontemporal", lambda i: sc(i, 1)),
                    ("stream_copy_cacheable", lambda i: sc(i, 0))):
        f(0)
        us = float(np.median(time_groups(torch, stream, f, 5, 3)))
        res[name + "_GBps"] = round(2 * COPY_BYTES / (us * 1e-6) / 1e9, 1)
    res["note"] = ("1 GiB read + 1 GiB written per copy; the T sweep gives the "
                   "streaming copy at each op's own traffic")
    del src, dst
    return res


def run_chain(torch, fr, workloads, HipGraph, dev, stream, replays):
    ci = workloads.chain_inputs()
    d = ci["dims"]
    L, S, T, H = d["layers"], d["steps"], d["T"], d["H"]
    x, qkv = dev(ci["x"]), dev(ci["qkv"])
    gate, sc, sh = dev(ci["gate"]), dev(ci["ada_scale"]), dev(ci["ada_shift"])
    res = torch.empty((L * S + 1, T, H), dtype=torch.int16, device="cuda")
    res[0] = dev(ci["r0"])
    q8 = torch.empty((L * S, T, H), dtype=torch.uint8, device="cuda")
    q_out = torch.empty((L, T, d["Hq"], d["D"]), dtype=torch.int16, device="cuda")
    kc, vc = dev(ci["k_cache"]), dev(ci["v_cache"])
    pos, table = dev(ci["positions"]), dev(ci["page_table"])

    def run():
        n = 0
        for _ in range(S):
            for l in range(L):
                fr.fr_adarms_gate_res_fp8(x[l], gate[n], res[n], res[n + 1],
                                          sc[n], sh[n], EPS, q8[n], fr.Q_STATIC,
                                          56.0, None, T, H, fr.F16, stream=stream)
                fr.fr_qkv_normrope_kvwrite(qkv[l], None, None, EPS, pos, 1e4,
                                           fr.ROPE_HALF, q_out[l], kc[l], vc[l],
                                           table, 1, d["page_size"], 1, None, T,
                                           d["Hq"], d["Hkv"], d["D"], fr.F16,
                                           stream=stream)
                n += 1

    run()
    stream.synchronize()
    # eager launches (host-bound reference)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / 3

    graph = HipGraph(stream, run)
    nodes = graph.kernel_node_count()
    for _ in range(5):
        graph.launch()
    stream.synchronize()
    times = []
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        graph.launch()
        b.record(stream)
        stream.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    t = np.array(times)

    # the same 360 ops as one persistent kernel launch
    def persistent():
        fr.fr_decode_chain_persistent(x, gate, sc, sh, res, q8, EPS, 56.0, qkv,
                                      pos, 1e4, fr.ROPE_HALF, q_out, kc, vc,
                                      table, 1, d["page_size"], 1, None, L, S, T,
                                      H, d["Hq"], d["Hkv"], d["D"], fr.F16,
                                      stream=stream)
    for _ in range(5):
        persistent()
    stream.synchronize()
    pt = []
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        persistent()
        b.record(stream)
        stream.synchronize()
        pt.append(a.elapsed_time(b) * 1e3)
    pt = np.array(pt)
    return {
        "kernel_nodes": nodes,
        "replay_us_p10": round(float(np.percentile(t, 10)), 1),
        "replay_us_p50": round(float(np.percentile(t, 50)), 1),
        "replay_us_p90": round(float(np.percentile(t, 90)), 1),
        "us_per_op_p50": round(float(np.percentile(t, 50)) / nodes, 3),
        "eager_us_per_op": round(eager_us / nodes, 3),
        "persistent_us_p50": round(float(np.percentile(pt, 50)), 1),
        "persistent_us_per_op_p50": round(float(np.percentile(pt, 50)) / nodes, 3),
    }


PEAK_FP8_TFLOPS = 5000.0


GEMM_SHAPES = ((128, 2048, 6144), (192, 2048, 6144), (1024, 2048, 6144),
               (128, 4096, 12288), (4096, 4096, 12288))


def run_gemm_act(torch, fr, workloads, dev, stream, reps=20, timed=True,
                 shapes=GEMM_SHAPES):
    """The gate_up projection of the prefill FFN fused with SwiGLU and the
    block-128 FP8 output, at the Qwen3-VL 2B (hidden 2048, inter 6144) and 8B
    (hidden 4096, inter 12288) shapes.  Weights are packed once (outside the
    timing) and rotate through >= 400 MB of copies so every launch streams
    them from HBM."""
    out = {}
    for (M, K, I) in shapes:
        progress(f"  gemm M={M} K={K} I={I}")
        inp = workloads.gemm_inputs(M, K, I, 800 + M)
        a, a_s = dev(inp["a"]), dev(inp["a_scales"])
        w_raw, w_s = dev(inp["w"]), dev(inp["w_scales"])
        w0 = torch.empty_like(w_raw)
        fr.fr_gemm_pack_weights(w_raw, w0, 2 * I, K, stream=stream)
        torch.cuda.synchronize()
        del w_raw
        nw = max(2, -(-WEIGHT_ROTATION_BYTES // w0.numel())) if timed else 1
        ws = [w0] + [w0.clone() for _ in range(nw - 1)]
        q = torch.empty((M, I), dtype=torch.uint8, device="cuda")
        sc = torch.empty((M, I // 128), dtype=torch.float32, device="cuda")

        def f(i):
            fr.fr_gemm_gated_act_fp8(a, a_s, ws[i % nw], w_s, fr.ACT_SWIGLU, q, sc,
                                     M, K, I, stream=stream)
        for i in range(3):
            f(i)
        torch.cuda.synchronize()
        if not timed:
            del ws, w0
            continue
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):                  # lead-in on the same stream
            lead_in(torch, stream)
            e0.record(stream)
            for i in range(reps):
                f(i)
            e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        flops = 2.0 * M * K * 2 * I
        nbytes = 2 * I * K + M * K + 4 * M * K // 128 + 4 * (2 * I // 128) * (K // 128) \
            + M * I + 4 * M * I // 128
        out[f"M{M}_K{K}_I{I}"] = {
            "us": round(us, 2),
            "TFLOPs": round(flops / (us * 1e-6) / 1e12, 1),
            "frac_of_fp8_peak": round(flops / (us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "bound": "mfma" if flops / (PEAK_FP8_TFLOPS * 1e12) > nbytes / (PEAK_HBM_GBS * 1e9) else "hbm",
        }
        del ws, w0
    return out


NVFP4_SCALE = 3.7e-2        # tensor dequant scale of the NVFP4 producer (amax ~ 100 / (6 * 448))


def run_mxfp4(torch, fr, workloads, dev, stream, reps, timed=True):
    """The FP4 producers at the bandwidth shapes (8192 tokens: RMSNorm
    H=4096 bf16 with weight -> MXFP4 and -> NVFP4, add + LayerNorm ->
    MXFP4 and -> NVFP4, SwiGLU I=12288 bf16 -> MXFP4), buffers rotated
    through >= 512 MB;
    reps launches back to back, events at the ends."""
    T, H, I = T_BIG, 4096, 12288
    e = 2
    nb_norm = T * H * 3 * e + H * e + T * H // 2 + T * H // 32
    nb_nv = T * H * 3 * e + H * e + T * H // 2 + T * H // 16
    nb_act = T * 2 * I * e + T * I // 2 + T * I // 32
    ri = workloads.resid_rmsnorm_inputs(T, H, workloads.BF16, 105, outliers=True)
    gi = workloads.gated_act_inputs(T, I, workloads.BF16, 104, outliers=True)
    N = [{k: dev(v) for k, v in ri.items()}]
    G = [{"gu": dev(gi["gate_up"])}]
    for lst, nb in ((N, nb_norm), (G, nb_act)):
        for _ in range(max(2, -(-ROTATION_BYTES // nb)) - 1 if timed else 0):
            lst.append({k: v.clone() for k, v in lst[0].items()})
    for d in N:
        d["ro"] = torch.empty_like(d["x"])
        d["q"] = torch.empty((T, H // 2), dtype=torch.uint8, device="cuda")
        d["s"] = torch.empty((T, H // 32), dtype=torch.uint8, device="cuda")
        d["s16"] = torch.empty((T, H // 16), dtype=torch.uint8, device="cuda")
    for d in G:
        d["q"] = torch.empty((T, I // 2), dtype=torch.uint8, device="cuda")
        d["s"] = torch.empty((T, I // 32), dtype=torch.uint8, device="cuda")

    def norm(i):
        d = N[i % len(N)]
        fr.fr_resid_rmsnorm_mxfp4(d["x"], d["residual"], d["ro"], d["weight"],
                                  fr.W_MUL, EPS, d["q"], d["s"], T, H,
                                  fr.BF16, stream=stream)

    def nv(i):
        d = N[i % len(N)]
        fr.fr_resid_rmsnorm_nvfp4(d["x"], d["residual"], d["ro"], d["weight"],
                                  fr.W_MUL, EPS, NVFP4_SCALE, d["q"], d["s16"], T, H,
                                  fr.BF16, stream=stream)

    def act(i):
        d = G[i % len(G)]
        fr.fr_gated_act_mxfp4(d["gu"], fr.ACT_SWIGLU, d["q"], d["s"], T, I,
                              fr.BF16, stream=stream)

    # the add + LayerNorm producer (ViT style): weight and bias, same rows
    bias = dev(workloads.to16(np.full(H, 0.01, np.float32), workloads.BF16))
    nb_ln = nb_norm + H * 2

    def ln(i):
        d = N[i % len(N)]
        fr.fr_resid_layernorm_mxfp4(d["x"], d["residual"], d["ro"], d["weight"], bias,
                                    EPS, d["q"], d["s"], T, H, fr.BF16, stream=stream)

    def ln_nv(i):
        d = N[i % len(N)]
        fr.fr_resid_layernorm_nvfp4(d["x"], d["residual"], d["ro"], d["weight"], bias,
                                    EPS, NVFP4_SCALE, d["q"], d["s16"], T, H, fr.BF16,
                                    stream=stream)

    out = {}
    for name, f, nb in (("resid_rmsnorm_mxfp4_T8192_H4096", norm, nb_norm),
                        ("resid_rmsnorm_nvfp4_T8192_H4096", nv, nb_nv),
                        ("gated_act_mxfp4_T8192_I12288", act, nb_act),
                        ("resid_layernorm_mxfp4_T8192_H4096", ln, nb_ln),
                        ("resid_layernorm_nvfp4_T8192_H4096", ln_nv, nb_nv + H * 2)):
        for i in range(3):
            f(i)
        torch.cuda.synchronize()
        if not timed:
            continue
        runs = []
        with torch.cuda.stream(stream):                  # lead-in on the same stream
            for _ in range(GROUP_REPEATS):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                lead_in(torch, stream)
                e0.record(stream)
                for i in range(reps):
                    f(i)
                e1.record(stream)
                torch.cuda.synchronize()
                runs.append(e0.elapsed_time(e1) * 1e3 / reps)
        us = float(np.median(runs))
        out[name] = {"bytes": nb, "us_per_launch": round(us, 3),
                     "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    return out


def run_qknorm(torch, fr, workloads, dev, stream, reps, timed=True, only=None):
    """fr_qk_norm_rope at 8192 tokens: the Wan-style full-width RMSNorm + 3D
    RoPE (40/40 heads x 128 bf16) and the Chameleon-style LayerNorm per head
    + RoPE (32/32 heads x 128 bf16); buffers rotated through >= 512 MB."""
    T, D = T_BIG, 128
    out = {}
    for name, Hq, Hkv, kind, full, r3, sec, style in (
            ("wan_rms_full_3d_T8192_40x128", 40, 40, fr.NORM_RMS, True, True, (22, 21, 21), 1),
            ("chameleon_layer_head_T8192_32x128", 32, 32, fr.NORM_LAYER, False, False, None, 0)):
        if only is not None and not name.startswith(only):
            continue
        NH = Hq + 2 * Hkv
        nb = 2 * T * NH * D * 2 + 4 * T * (3 if r3 else 1)
        inp = workloads.qk_norm_rope_inputs(T, Hq, Hkv, D, workloads.BF16, 610,
                                            scope_full=full, rope3=r3, grid=(8, 32, 32))
        w = {k: dev(inp[k]) for k in ("q_norm_w", "q_norm_b", "k_norm_w", "k_norm_b", "positions")}
        sets = []
        for _ in range(max(2, -(-ROTATION_BYTES // nb)) if timed else 1):
            sets.append({"qkv": dev(inp["qkv"]),
                         "q": torch.empty((T, Hq, D), dtype=torch.int16, device="cuda"),
                         "k": torch.empty((T, Hkv, D), dtype=torch.int16, device="cuda"),
                         "v": torch.empty((T, Hkv, D), dtype=torch.int16, device="cuda")})

        def f(i):
            d = sets[i % len(sets)]
            fr.fr_qk_norm_rope(d["qkv"], kind, int(full), w["q_norm_w"], w["q_norm_b"],
                               w["k_norm_w"], w["k_norm_b"], EPS, w["positions"],
                               3 if r3 else 1, sec, 1e4, style, 1.0, d["q"], d["k"],
                               d["v"], T, Hq, Hkv, D, fr.BF16, stream=stream)
        for i in range(3):
            f(i)
        torch.cuda.synchronize()
        if not timed:
            continue
        runs = []
        with torch.cuda.stream(stream):                  # lead-in on the same stream
            for _ in range(GROUP_REPEATS):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                lead_in(torch, stream)
                e0.record(stream)
                for i in range(reps):
                    f(i)
                e1.record(stream)
                torch.cuda.synchronize()
                runs.append(e0.elapsed_time(e1) * 1e3 / reps)
        us = float(np.median(runs))
        out[name] = {"bytes": nb, "us_per_launch": round(us, 3),
                     "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        del sets
    return out


def run_small(torch, fr, workloads, dev, stream):
    """Standalone (outside any graph) hipEvent medians at 10 tokens."""
    out = {}
    ri = workloads.resid_rmsnorm_inputs(10, 1024, workloads.F16, 101)
    x, r, w = dev(ri["x"]), dev(ri["residual"]), dev(ri["weight"])
    ro = torch.empty_like(x)
    q = torch.empty((10, 1024), dtype=torch.uint8, device="cuda")

    def a():
        fr.fr_resid_rmsnorm_fp8(x, r, ro, w, fr.W_NONE, EPS, q, fr.Q_STATIC,
                                56.0, None, 10, 1024, fr.F16, stream=stream)

    gi = workloads.gated_act_inputs(10, 6144, workloads.BF16, 104)
    gu = dev(gi["gate_up"])
    gq = torch.empty((10, 6144), dtype=torch.uint8, device="cuda")
    gs = torch.empty((10, 48), dtype=torch.float32, device="cuda")

    def c():
        fr.fr_gated_act_fp8(gu, fr.ACT_SWIGLU, gq, gs, 10, 6144, fr.BF16,
                            stream=stream)

    ai = workloads.adarms_inputs(10, 1024, workloads.F16, 102)
    ad = {k: dev(v) for k, v in ai.items()}
    aro = torch.empty_like(ad["x"])
    aq = torch.empty((10, 1024), dtype=torch.uint8, device="cuda")

    def ada():
        fr.fr_adarms_gate_res_fp8(ad["x"], ad["gate"], ad["residual"], aro,
                                  ad["ada_scale"], ad["ada_shift"], EPS, aq,
                                  fr.Q_STATIC, 56.0, None, 10, 1024, fr.F16,
                                  stream=stream)

    qi = workloads.qkv_inputs(10, 8, 1, 256, workloads.F16, 102, page_size=1024,
                              num_pages=1, positions=np.arange(790, 800),
                              norm=False, random_pages=False)
    qd = {k: (dev(v) if v is not None else None) for k, v in qi.items()}
    qo = torch.empty((10, 8, 256), dtype=torch.int16, device="cuda")

    def qkv():
        fr.fr_qkv_normrope_kvwrite(qd["qkv"], None, None, EPS, qd["positions"],
                                   1e4, fr.ROPE_HALF, qo, qd["k_cache"],
                                   qd["v_cache"], qd["page_table"], 1, 1024, 1,
                                   None, 10, 8, 1, 256, fr.F16, stream=stream)

    for name, f in (("resid_rmsnorm_fp8_T10_H1024", a),
                    ("adarms_gate_res_fp8_T10_H1024", ada),
                    ("qkv_normrope_kvwrite_T10_8x1x256", qkv),
                    ("gated_act_fp8_T10_I6144", c)):
        for _ in range(5):
            f()
        ts = []
        for _ in range(50):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            f()
            e1.record(stream)
            stream.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        out[name + "_us_p50"] = round(float(np.median(ts)), 2)
    return out


def cpu_threads():
    """Host threads this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS when that is set (the share of the host given to it)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s):
    """The oracle (plain C, double precision, as written) on row samples of
    the same four ops, in two settings: one thread, and the rows split over
    every host thread this process may use (the ops are row-independent, so
    the split is a harness split, not an oracle change; ctypes releases the
    GIL during each C call).  Only the C calls are timed (inputs and outputs
    are allocated before).  Reported in the same unit (algorithmic GB/s),
    with per-op milliseconds and their extrapolation to the 8192-token call."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    import workloads
    L = oracle.lib()
    nthr = cpu_threads()
    rows1 = {"resid_rmsnorm_fp8": 64, "adarms_gate_res_fp8": 256,
             "qkv_normrope_kvwrite": 32, "gated_act_fp8": 16}
    R = {k: v * nthr for k, v in rows1.items()}
    ri = workloads.resid_rmsnorm_inputs(R["resid_rmsnorm_fp8"], 4096, workloads.BF16, 105,
                                        outliers=True)
    ai = workloads.adarms_inputs(R["adarms_gate_res_fp8"], 1024, workloads.F16, 102)
    qi = workloads.qkv_inputs(R["qkv_normrope_kvwrite"], 32, 8, 128, workloads.BF16, 103,
                              page_size=16, num_pages=512)
    gi = workloads.gated_act_inputs(R["gated_act_fp8"], 12288, workloads.BF16, 105,
                                    outliers=True)
    ra = {"ro": np.empty_like(ri["x"]), "q": np.empty(ri["x"].shape, np.uint8),
          "sc": np.empty(ri["x"].shape[0], np.float32)}
    aa = {"ro": np.empty_like(ai["x"]), "q": np.empty(ai["x"].shape, np.uint8)}
    qa = {"q_out": np.empty((R["qkv_normrope_kvwrite"], 32, 128), np.uint16),
          "err": np.zeros(nthr, np.int32)}
    ga = {"q": np.empty((R["gated_act_fp8"], 12288), np.uint8),
          "sc": np.empty((R["gated_act_fp8"], 96), np.float32)}
    P = lambda a, off=0: a.ctypes.data + off

    def run(op, r0, r1, w):
        n = r1 - r0
        if op == "resid_rmsnorm_fp8":
            rb = r0 * 4096 * 2
            rc = L.oracle_resid_rmsnorm_fp8(
                P(ri["x"], rb), P(ri["residual"], rb), P(ra["ro"], rb), P(ri["weight"]),
                oracle.W_MUL, EPS, P(ra["q"], r0 * 4096), oracle.Q_TOKEN, 0.0,
                P(ra["sc"], r0 * 4), n, 4096, oracle.BF16)
        elif op == "adarms_gate_res_fp8":
            rb = r0 * 1024 * 2
            rc = L.oracle_adarms_gate_res_fp8(
                P(ai["x"], rb), P(ai["gate"], rb), P(ai["residual"], rb), P(aa["ro"], rb),
                P(ai["ada_scale"], rb), P(ai["ada_shift"], rb), EPS, P(aa["q"], r0 * 1024),
                oracle.Q_STATIC, 56.0, None, n, 1024, oracle.F16)
        elif op == "qkv_normrope_kvwrite":
            rc = L.oracle_qkv_normrope_kvwrite(
                P(qi["qkv"], r0 * 48 * 128 * 2), P(qi["q_norm_w"]), P(qi["k_norm_w"]), EPS,
                P(qi["positions"], r0 * 4), 1e6, oracle.ROPE_HALF, 1.0,
                P(qa["q_out"], r0 * 32 * 128 * 2), P(qi["k_cache"]), P(qi["v_cache"]),
                P(qi["page_table"]), 512, 16, 512, P(qa["err"], w * 4), n, 32, 8, 128,
                oracle.BF16)
        else:
            rc = L.oracle_gated_act_fp8(
                P(gi["gate_up"], r0 * 2 * 12288 * 2), oracle.ACT_SWIGLU,
                P(ga["q"], r0 * 12288), P(ga["sc"], r0 * 96 * 4), n, 12288, oracle.BF16)
        assert rc == 0, (op, rc)

    nb = op_bytes()
    ops = list(rows1)

    def setting(nt, seconds):
        pool = ThreadPoolExecutor(nt) if nt > 1 else None
        rows = {k: rows1[k] * nt for k in ops}
        per_op = {k: 0.0 for k in ops}
        passes = 0
        t_end = time.perf_counter() + seconds
        while passes < 1 or time.perf_counter() < t_end:
            for op in ops:
                chunk = rows[op] // nt
                t0 = time.perf_counter()
                if pool is None:
                    run(op, 0, rows[op], 0)
                else:
                    list(pool.map(lambda w, op=op: run(op, w * chunk, (w + 1) * chunk, w),
                                  range(nt)))
                per_op[op] += time.perf_counter() - t0
            passes += 1
        if pool is not None:
            pool.shutdown()
        secs = sum(per_op.values()) / passes
        sample_bytes = sum(nb[k] * rows[k] / T_BIG for k in ops)
        return {
            "threads": nt,
            "GBps": round(sample_bytes / secs / 1e9, 4),
            "passes": passes,
            "rows": rows,
            "ms_per_op_sample": {k: round(v / passes * 1e3, 3) for k, v in per_op.items()},
            "ms_per_8192_token_call": {k: round(v / passes * 1e3 * T_BIG / rows[k], 1)
                                       for k, v in per_op.items()},
        }

    one = setting(1, budget_s / 2)
    allt = setting(nthr, budget_s / 2) if nthr > 1 else one
    return {
        "value": allt["GBps"],
        "unit": "GB/s",
        "cores": allt["threads"],
        "kind": "oracle",
        "sample": (f"rows of the 8192-token step's four ops ({allt['rows']}), split over "
                   f"{allt['threads']} threads, {allt['passes']} passes; only the C calls "
                   f"timed"),
        "cpu_model": cpu_model(),
        "all_threads": allt,
        "single_thread": one,
    }


if __name__ == "__main__":
    main()
