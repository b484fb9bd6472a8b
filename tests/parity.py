"""Comparison rules and device plumbing shared by the GPU parity tests.

Acceptance rules (fixed before any kernel was written):
  * 16-bit outputs: |g - o| <= max(2e-3 |o|, ulp_dtype(o)) + 1e-5 elementwise,
    o the oracle's stored value.  (One bf16 ulp is above 2e-3 relative, so
    two independently rounded bf16 values may differ by one ulp.)
  * bit-exact: op (a)'s new residual (the sum of two 16-bit values is exact
    in fp32, and rounding it again to 16 bits is then a single rounding), the
    V cache copy, every cache slot no token maps to.
  * FP8 codes: >= 99.9% identical and every code within one step of the
    oracle's on the sign-magnitude order (+0 and -0 identified).
  * fp32 scales: |s_g - s_o| <= 1e-6 s_o.
  * MX FP4 (E2M1 codes + E8M0 block scales): where the kernel takes the
    oracle's decisions exactly (the residual-RMSNorm producer) codes and
    scales are bit-exact.  Otherwise (the activation and LayerNorm
    producers, fp32 vs float64 values) a scale may differ by one step only
    where the block maximum sits at a power of two, in at most 0.1% of
    blocks; in blocks with equal scales every code is within one E2M1 step
    and >= 99.9% are identical.
  * NVFP4 (E2M1 codes + E4M3 block scales, blocks of 16): bit-exact where
    the kernel takes the oracle's decisions exactly (the residual-RMSNorm
    producer); the LayerNorm producer (fp32 values) is held to the MX rule
    above with E4M3 steps (a scale code may differ by one where the block
    maximum / (6 g) sits at an E4M3 rounding boundary).
"""
import sys

import numpy as np
import torch

import oracle

F16, BF16 = 0, 1


def announce(msg):
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def to_host(t, dtype):
    return t.cpu().numpy().view(dtype)


def ulp16(o, dtype):
    a = np.abs(o)
    p, emin = (11, -14) if dtype == F16 else (8, -126)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.exp2(e - (p - 1))


def check16(got, want, dtype, what=""):
    """Tolerance rule for 16-bit outputs; returns the bit-identical fraction."""
    g = oracle.decode16(got, dtype)
    o = oracle.decode16(want, dtype)
    tol = np.maximum(2e-3 * np.abs(o), ulp16(o, dtype)) + 1e-5
    bad = ~(np.abs(g - o) <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} values out of tolerance; first "
            + ", ".join(f"{tuple(i)} got {g[tuple(i)]!r} want {o[tuple(i)]!r}"
                        for i in idx))
    return float(np.mean(got == want))


def check_exact(got, want, what=""):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at "
                             f"{[tuple(i) for i in bad[:5]]}")


def _ord(c):
    c = c.astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def check_fp8(got, want, what="", min_identical=0.999):
    """Returns the identical fraction (+0/-0 identified)."""
    got = np.asarray(got, dtype=np.uint8)
    want = np.asarray(want, dtype=np.uint8)
    nan = ((got & 0x7F) == 0x7F)
    assert not nan.any(), f"{what}: {nan.sum()} NaN / unwritten codes"
    step = np.abs(_ord(got) - _ord(want))
    if (step > 1).any():
        idx = np.argwhere(step > 1)[:5]
        raise AssertionError(
            f"{what}: {int((step > 1).sum())} codes more than one step off; first "
            + ", ".join(f"{tuple(i)} got {got[tuple(i)]:#04x} want "
                        f"{want[tuple(i)]:#04x}" for i in idx))
    ident = float(np.mean(step == 0))
    assert ident >= min_identical, f"{what}: only {ident:.6f} identical"
    return ident


def check_scales(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite / unwritten scales"
    rel = np.abs(got - want) / want
    assert np.all(rel <= 1e-6), f"{what}: max rel error {rel.max():.3e}"
    return float(rel.max())


def _ord4(c):
    c = c.astype(np.int32)
    return np.where(c & 8, -(c & 7), c & 7)


def check_fp4(q_g, s_g, q_o, s_o, what="", min_identical=0.999,
              max_scale_diff=1e-3, block=32):
    """q_*: packed E2M1 bytes [..., n/2]; s_*: block scale codes [..., n/block]
    (E8M0 for MX, blocks of 32; non-negative E4M3 for NVFP4, blocks of 16:
    both ordered like their values, so one step is a code difference of 1).
    Returns (identical code fraction, fraction of blocks with other scales)."""
    s_g = np.asarray(s_g, dtype=np.int32)
    s_o = np.asarray(s_o, dtype=np.int32)
    assert not (s_g == 255).any(), f"{what}: unwritten (poisoned) scales"
    ds = np.abs(s_g - s_o)
    assert ds.max(initial=0) <= 1, f"{what}: a scale differs by {ds.max()} steps"
    frac = float(np.mean(ds != 0))
    assert frac <= max_scale_diff, f"{what}: {frac:.5f} of block scales differ"
    cg = oracle.unpack_fp4(q_g).reshape(-1, block)
    co = oracle.unpack_fp4(q_o).reshape(-1, block)
    same_blk = (ds.reshape(-1) == 0)
    step = np.abs(_ord4(cg) - _ord4(co))[same_blk]
    if (step > 1).any():
        raise AssertionError(f"{what}: {int((step > 1).sum())} codes more than one step off")
    ident = float(np.mean(step == 0)) if step.size else 1.0
    assert ident >= min_identical, f"{what}: only {ident:.6f} identical"
    return ident, frac


# ---- device runners: allocate, poison outputs, call the library ------------

POISON16 = 0x7E01      # a 16-bit NaN pattern (float16) / huge value (bfloat16)


def run_resid_rmsnorm(fr, inp, wmode, eps, qmode, static_scale, dtype,
                      inplace=False, stream=None):
    T, H = inp["x"].shape
    x, r, w = to_dev(inp["x"]), to_dev(inp["residual"]), to_dev(inp["weight"])
    ro = r if inplace else torch.full((T, H), POISON16, dtype=torch.int16,
                                      device="cuda")
    q = torch.full((T, H), 0x7F, dtype=torch.uint8, device="cuda")
    sc = torch.full((max(T, 1),), float("nan"), dtype=torch.float32,
                    device="cuda")
    fr.fr_resid_rmsnorm_fp8(x, r, ro, w, wmode, eps, q, qmode, static_scale,
                            sc, T, H, dtype, stream=stream)
    torch.cuda.synchronize()
    return (to_host(ro, np.uint16), to_host(q, np.uint8),
            to_host(sc, np.float32)[:T] if qmode == 1 else None)


def run_adarms(fr, inp, eps, qmode, static_scale, dtype, inplace=False):
    T, H = inp["x"].shape
    d = {k: to_dev(inp[k]) for k in ("x", "gate", "residual", "ada_scale",
                                      "ada_shift")}
    ro = d["residual"] if inplace else torch.full(
        (T, H), POISON16, dtype=torch.int16, device="cuda")
    q = torch.full((T, H), 0x7F, dtype=torch.uint8, device="cuda")
    sc = torch.full((max(T, 1),), float("nan"), dtype=torch.float32,
                    device="cuda")
    fr.fr_adarms_gate_res_fp8(d["x"], d["gate"], d["residual"], ro,
                              d["ada_scale"], d["ada_shift"], eps, q, qmode,
                              static_scale, sc, T, H, dtype)
    torch.cuda.synchronize()
    return (to_host(ro, np.uint16), to_host(q, np.uint8),
            to_host(sc, np.float32)[:T] if qmode == 1 else None)


def run_qkv(fr, inp, eps, theta, style, Hq, Hkv, D, page_size, dtype,
            err=True, q_scale=1.0):
    T = inp["qkv"].shape[0]
    kc, vc = to_dev(inp["k_cache"]), to_dev(inp["v_cache"])
    q_out = torch.full((T, Hq, D), POISON16, dtype=torch.int16, device="cuda")
    ef = torch.zeros(1, dtype=torch.int32, device="cuda") if err else None
    qw = to_dev(inp["q_norm_w"]) if inp["q_norm_w"] is not None else None
    kw = to_dev(inp["k_norm_w"]) if inp["k_norm_w"] is not None else None
    pos = to_dev(inp["positions"])
    table = to_dev(inp["page_table"])
    fr.fr_qkv_normrope_kvwrite(to_dev(inp["qkv"]), qw, kw, eps, pos, theta,
                               style, q_out, kc, vc, table,
                               inp["page_table"].size, page_size,
                               inp["k_cache"].shape[0], ef, T, Hq, Hkv, D,
                               dtype, q_scale=q_scale)
    torch.cuda.synchronize()
    return (to_host(q_out, np.uint16), to_host(kc, np.uint16),
            to_host(vc, np.uint16), int(ef.item()) if err else None)


def run_gated_act(fr, inp, act, dtype):
    T, I2 = inp["gate_up"].shape
    I = I2 // 2
    q = torch.full((T, I), 0x7F, dtype=torch.uint8, device="cuda")
    sc = torch.full((T, I // 128), float("nan"), dtype=torch.float32,
                    device="cuda")
    fr.fr_gated_act_fp8(to_dev(inp["gate_up"]), act, q, sc, T, I, dtype)
    torch.cuda.synchronize()
    return to_host(q, np.uint8), to_host(sc, np.float32)


def run_resid_rmsnorm_mxfp4(fr, inp, wmode, eps, dtype, inplace=False,
                            poison=0xAA):
    T, H = inp["x"].shape
    x, r, w = to_dev(inp["x"]), to_dev(inp["residual"]), to_dev(inp["weight"])
    ro = r if inplace else torch.full((T, H), POISON16, dtype=torch.int16,
                                      device="cuda")
    q = torch.full((T, H // 2), poison, dtype=torch.uint8, device="cuda")
    sc = torch.full((T, H // 32), 0xFF, dtype=torch.uint8, device="cuda")
    fr.fr_resid_rmsnorm_mxfp4(x, r, ro, w, wmode, eps, q, sc, T, H, dtype)
    torch.cuda.synchronize()
    return to_host(ro, np.uint16), to_host(q, np.uint8), to_host(sc, np.uint8)


def run_resid_rmsnorm_nvfp4(fr, inp, wmode, eps, gscale, dtype, inplace=False,
                            poison=0xAA):
    T, H = inp["x"].shape
    x, r, w = to_dev(inp["x"]), to_dev(inp["residual"]), to_dev(inp["weight"])
    ro = r if inplace else torch.full((T, H), POISON16, dtype=torch.int16,
                                      device="cuda")
    q = torch.full((T, H // 2), poison, dtype=torch.uint8, device="cuda")
    sc = torch.full((T, H // 16), 0xFF, dtype=torch.uint8, device="cuda")
    fr.fr_resid_rmsnorm_nvfp4(x, r, ro, w, wmode, eps, gscale, q, sc, T, H, dtype)
    torch.cuda.synchronize()
    return to_host(ro, np.uint16), to_host(q, np.uint8), to_host(sc, np.uint8)


def run_gated_act_mxfp4(fr, inp, act, dtype, poison=0xAA):
    T, I2 = inp["gate_up"].shape
    I = I2 // 2
    q = torch.full((T, I // 2), poison, dtype=torch.uint8, device="cuda")
    sc = torch.full((T, I // 32), 0xFF, dtype=torch.uint8, device="cuda")
    fr.fr_gated_act_mxfp4(to_dev(inp["gate_up"]), act, q, sc, T, I, dtype)
    torch.cuda.synchronize()
    return to_host(q, np.uint8), to_host(sc, np.uint8)
