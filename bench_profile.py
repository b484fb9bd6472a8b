"""Summarise rocprofv3 output of the benchmark into profiles/.

Kernel durations (per-kernel launch count, average, median, min):
    rocprofv3 --kernel-trace --stats -d <dir> -o bench -- python3 bench.py --steps 10 --no-cpu-baseline
    python3 bench_profile.py trace <dir>/bench_results.db

LDS counters (one pass):
    rocprofv3 --pmc SQ_LDS_BANK_CONFLICT ... -d <dir> -o lds --output-format csv -- python3 bench.py --pmc-pass
    python3 bench_profile.py lds <dir>/lds_counter_collection.csv

HBM byte counters of the 8192-token ops:
    rocprofv3 --pmc FETCH_SIZE -d <dir_f> -o fetch -- python3 bench.py --pmc-pass
    rocprofv3 --pmc WRITE_SIZE -d <dir_w> -o write -- python3 bench.py --pmc-pass
    python3 bench_profile.py pmc <dir_f>/fetch_results.db <dir_w>/write_results.db

The --pmc-pass run first copies 1 GiB device-to-device three times (the HIP
runtime's copyBuffer kernel, known traffic: 1 GiB read + 1 GiB written).
Each counter is scaled by known bytes / counted bytes of that copy, then
reported per launch for every fused-op kernel next to its algorithmic bytes.
Writes profiles/hbm_traffic_T8192.txt and, for the dominant kernel,
profiles/gated_act_fp8_T8192_I12288_pmc.json (with the hash of the kernel
source it was taken on; bench.py uses the traffic only while it matches).
"""
import collections
import hashlib
import json
import os
import re
import sqlite3
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
GIB = 1 << 30

ACT_FP8 = "void fr::k_act<1, 0, 4, true, false, false>"
KERNELS = {  # kernel name prefix -> (op, algorithmic read bytes, write bytes)
    "void fr::k_norm<1, 2, 1, true, true, false, false>": (
        "resid_rmsnorm_fp8 T=8192 H=4096 bf16 MUL TOKEN",
        8192 * 4096 * 4 + 4096 * 2, 8192 * 4096 * 3 + 8192 * 4),
    "void fr::k_norm<0, 2, 3, true, false, false, false>": (
        "adarms_gate_res_fp8 T=8192 H=1024 f16 STATIC",
        8192 * 1024 * 10, 8192 * 1024 * 3),
    "void fr::k_qkv<1, 8, true": (
        "qkv_normrope_kvwrite T=8192 32/8x128 bf16",
        8192 * 48 * 128 * 2 + 8192 * 4 + 512 * 4 + 512, 8192 * 48 * 128 * 2),
    ACT_FP8: (
        "gated_act_fp8 T=8192 I=12288 bf16 SwiGLU",
        8192 * 24576 * 2, 8192 * 12288 + 8192 * 96 * 4),
    "void fr::k_norm<1, 2, 1, true, true, true, false>": (
        "resid_rmsnorm_mxfp4 T=8192 H=4096 bf16 MUL",
        8192 * 4096 * 4 + 4096 * 2, 8192 * 4096 * 2 + 8192 * 2048 + 8192 * 128),
    "void fr::k_norm<1, 2, 1, true, true, false, true>": (
        "resid_rmsnorm_nvfp4 T=8192 H=4096 bf16 MUL",
        8192 * 4096 * 4 + 4096 * 2, 8192 * 4096 * 2 + 8192 * 2048 + 8192 * 256),
    "void fr::k_act<1, 0, 4, true, false, true>": (
        "gated_act_mxfp4 T=8192 I=12288 bf16 SwiGLU",
        8192 * 24576 * 2, 8192 * 6144 + 8192 * 384),
    "void fr::k_norm<1, 2, 4, true, true, true, false>": (
        "resid_layernorm_mxfp4 T=8192 H=4096 bf16",
        8192 * 4096 * 4 + 4096 * 4, 8192 * 4096 * 2 + 8192 * 2048 + 8192 * 128),
    "void fr::k_norm<1, 2, 4, true, true, false, true>": (
        "resid_layernorm_nvfp4 T=8192 H=4096 bf16",
        8192 * 4096 * 4 + 4096 * 4, 8192 * 4096 * 2 + 8192 * 2048 + 8192 * 256),
    "void fr::k_qknr<1, 8, 4>": (
        "qk_norm_rope T=8192 40/40x128 bf16 RMS full 3D (Wan)",
        8192 * 120 * 128 * 2 + 8192 * 12 + 2 * 5120 * 2 * 2, 8192 * 120 * 128 * 2),
    "void fr::k_gemm_act<0, 1, 2>": (
        "gemm_gated_act_fp8 M=128 K=2048 I=6144 (weight, A, scales)",
        12288 * 2048 + 128 * 2048 + 128 * 16 * 4 + 96 * 16 * 4,
        128 * 6144 + 128 * 48 * 4),
}


def code_hash(path):
    """sha256 (16 hex digits) of a C++ source with its comments and blank
    space removed: a counter record stays valid across comment edits and
    becomes stale on any change to the code itself."""
    with open(path) as fh:
        src = fh.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def per_kernel(db):
    c = sqlite3.connect(db)
    vals = collections.defaultdict(list)
    for name, val, grid in c.execute(
            "select kernel_name, value, grid_size from counters_collection order by dispatch_id"):
        vals[(name, grid)].append(val * 1024.0)          # KiB -> bytes
    return vals


def trace(db, out_name="kernel_trace_bench_T8192_and_T10_chain.txt"):
    c = sqlite3.connect(db)
    groups = collections.defaultdict(list)
    for name, dur, grid, wg in c.execute(
            "select name, duration, grid_x, workgroup_x from kernels"):
        groups[(name, grid, wg)].append(dur / 1000.0)
    lines = [
        "Kernel durations from rocprofv3 --kernel-trace (MI355X, gfx950), microseconds",
        "commands:",
        "  rocprofv3 --kernel-trace --stats -d gpurun_out/prof -o bench -- python3 -u bench.py --steps 10 --no-cpu-baseline --chain-replays 5",
        "  python3 bench_profile.py trace gpurun_out/prof/bench_results.db",
        "grid = work-items; the 8192-token ops are the large grids, the 10-token",
        "chain ops (2 x 180 per graph replay) the small ones.",
        "",
        f"{'calls':>6s} {'avg':>10s} {'median':>10s} {'min':>10s} {'grid':>9s} {'wg':>5s}  kernel",
    ]
    for (name, grid, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        d = sorted(d)
        lines.append(f"{len(d):6d} {sum(d) / len(d):10.3f} {d[len(d) // 2]:10.3f} "
                     f"{d[0]:10.3f} {grid:9d} {wg:5d}  {name[:90]}")
    with open(os.path.join(HERE, "profiles", out_name), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def pmc(fetch_db, write_db):
    f, w = per_kernel(fetch_db), per_kernel(write_db)
    # the three 1 GiB copies: copyBuffer launches with the largest grid
    cal = [k for k in f if k[0].startswith("__amd_rocclr_copyBuffer")]
    big = max(cal, key=lambda k: k[1])
    f_scale = GIB / (sum(f[big]) / len(f[big]))
    w_scale = GIB / (sum(w[big]) / len(w[big]))
    lines = [
        "HBM traffic per launch, rocprofv3 PMC counters (MI355X, gfx950)",
        "commands:",
        "  rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o fetch -- python3 -u bench.py --pmc-pass",
        "  rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_write -o write -- python3 -u bench.py --pmc-pass",
        "  python3 bench_profile.py pmc gpurun_out/pmc_fetch/fetch_results.db gpurun_out/pmc_write/write_results.db",
        f"calibration: 1 GiB device copy ({big[0]}, grid {big[1]}):",
        f"  FETCH_SIZE counted {sum(f[big]) / len(f[big]) / 1e6:.2f} MB -> scale {f_scale:.4f}",
        f"  WRITE_SIZE counted {sum(w[big]) / len(w[big]) / 1e6:.2f} MB -> scale {w_scale:.4f}",
        "",
        f"{'kernel / op':58s} {'read MB':>9s} {'alg':>9s} {'write MB':>9s} {'alg':>9s} {'total/alg':>9s}",
    ]
    out = {}
    for (name, grid), fv in sorted(f.items()):
        for prefix, (op, alg_r, alg_w) in KERNELS.items():
            if name.startswith(prefix) and (name, grid) in w:
                rd = sum(fv) / len(fv) * f_scale
                wr = sum(w[(name, grid)]) / len(w[(name, grid)]) * w_scale
                ratio = (rd + wr) / (alg_r + alg_w)
                lines.append(f"{op:58s} {rd / 1e6:9.2f} {alg_r / 1e6:9.2f} "
                             f"{wr / 1e6:9.2f} {alg_w / 1e6:9.2f} {ratio:9.4f}")
                out[prefix] = {"op": op, "read_bytes": rd, "write_bytes": wr,
                               "alg_read_bytes": alg_r, "alg_write_bytes": alg_w,
                               "launches": len(fv)}
    os.makedirs(os.path.join(HERE, "profiles"), exist_ok=True)
    with open(os.path.join(HERE, "profiles", "hbm_traffic_T8192.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    dom = out.get(ACT_FP8)
    if dom:
        sha = code_hash(os.path.join(HERE, "memory_bound_amd", "csrc", "fr_act.hip"))
        rec = {"kernel": "fr::k_act<bf16, SwiGLU>", "workload": "T=8192 I=12288 bf16",
               "code_sha256_16": sha,
               "hbm_bytes_per_launch": round(dom["read_bytes"] + dom["write_bytes"]),
               "read_bytes_per_launch": round(dom["read_bytes"]),
               "write_bytes_per_launch": round(dom["write_bytes"]),
               "fetch_scale": f_scale, "write_scale": w_scale}
        with open(os.path.join(HERE, "profiles", "gated_act_fp8_T8192_I12288_pmc.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")


LDS_COUNTERS = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS",
                "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES")


def lds(csv_path):
    """LDS counters per kernel from one rocprofv3 --pmc pass written as CSV
    (mean over the kernel's dispatches)."""
    import csv
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(csv_path) as fh:
        for row in csv.DictReader(fh):
            name = re.sub(r"^void ", "", row["Kernel_Name"]).split("(")[0]
            acc[name][row["Counter_Name"]].append(float(row["Counter_Value"]))
    lines = [
        "LDS counters per kernel, rocprofv3 PMC (MI355X, gfx950)",
        "command (one pass; the bench's PMC workload: each op a few times at its bench shape):",
        "  rocprofv3 --pmc " + " ".join(LDS_COUNTERS) + " \\",
        "    -d gpurun_out/pmclds -o lds --output-format csv -- python3 -u bench.py --pmc-pass",
        "  python3 bench_profile.py lds gpurun_out/pmclds/lds_counter_collection.csv",
        "values: mean over the kernel's dispatches; conflict% = SQ_LDS_BANK_CONFLICT / "
        "SQ_LDS_IDX_ACTIVE; lds-issue wait% = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES",
        "",
        f"{'kernel':62s} {'LDS insts':>10s} {'active':>10s} {'conflict':>10s} "
        f"{'conflict%':>9s} {'wait%':>6s}",
    ]
    for name, cs in sorted(acc.items()):
        m = {k: (sum(v) / len(v) if v else 0.0) for k, v in cs.items()}
        if not m.get("SQ_INSTS_LDS"):
            continue
        act = m.get("SQ_LDS_IDX_ACTIVE", 0.0)
        conf = m.get("SQ_LDS_BANK_CONFLICT", 0.0)
        cyc = m.get("SQ_WAVE_CYCLES", 0.0)
        lines.append(f"{name[:62]:62s} {m['SQ_INSTS_LDS']:10.3g} {act:10.3g} {conf:10.3g} "
                     f"{(100 * conf / act if act else 0):8.1f}% "
                     f"{(100 * m.get('SQ_WAIT_INST_LDS', 0.0) / cyc if cyc else 0):5.1f}%")
    with open(os.path.join(HERE, "profiles", "lds_bank_conflicts_bench_T8192.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    os.makedirs(os.path.join(HERE, "profiles"), exist_ok=True)
    if sys.argv[1] == "trace":
        trace(sys.argv[2])
    elif sys.argv[1] == "pmc":
        pmc(sys.argv[2], sys.argv[3])
    elif sys.argv[1] == "lds":
        lds(sys.argv[2])
    else:
        sys.exit("usage: bench_profile.py trace <db> | pmc <fetch_db> <write_db> | lds <csv>")
