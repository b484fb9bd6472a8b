"""Seeded synthetic inputs for the fused layer-boundary ops.

This module only draws random numbers and lays them out; it holds none of
the ops' arithmetic.  Both sides of every parity check (the HIP library and
the CPU oracle) consume the same host arrays produced here, so neither side
re-implements the random generator.

Values are drawn with numpy's PCG64 (``default_rng(seed)``) in float32 and
stored as 16-bit bit patterns (uint16): float16 through numpy's cast, bfloat16
through torch's CPU cast, both round-to-nearest-even.

Shapes follow the workloads the pages measure on:
  * Pi0.5 decoder boundary: 10 action tokens, hidden 1024, 8 query heads /
    1 KV head of dim 256, 18 layers x 10 flow steps ("FlashRT cross-layer
    fusion" article, sections 一 to 三);
  * Qwen3-style prefill QKV post-processing: 32/8 heads of dim 128, paged
    cache of 16-token pages (same article, 2.2; Falcon article, paged cache);
  * gated activation at inter 6144 / 12288 with per-token block-128 FP8
    ("sm89 prefill FFN megakernel" issue, Phase 0 and Phase 2);
  * the bandwidth regime at 8192 tokens (hidden 4096, inter 12288).
"""
import numpy as np
import torch

F16, BF16 = 0, 1


def to16(a, dtype):
    """float32 array -> uint16 bit patterns of float16 / bfloat16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == F16:
        return a.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(a).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal(rng, shape, std=1.0, mean=0.0):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
            + np.float32(mean))


def with_outliers(rng, a, prob=0.001, factor=20.0):
    """Multiply each element by `factor` with probability `prob` (seeded
    Bernoulli draw)."""
    mask = rng.random(a.shape, dtype=np.float32) < prob
    out = a.copy()
    out[mask] *= np.float32(factor)
    return out


# ---------------------------------------------------------------------------
# residual add + RMSNorm + FP8
# ---------------------------------------------------------------------------

def resid_rmsnorm_inputs(T, H, dtype, seed, outliers=False, weight_std=0.05):
    """x, residual ~ N(0,1) [T,H]; weight ~ 1 + N(0, weight_std^2) [H]."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (T, H))
    r = normal(rng, (T, H))
    if outliers:
        x = with_outliers(rng, x)
        r = with_outliers(rng, r)
    w = normal(rng, (H,), std=weight_std, mean=1.0)
    return {"x": to16(x, dtype), "residual": to16(r, dtype),
            "weight": to16(w, dtype)}


# ---------------------------------------------------------------------------
# gate + residual + AdaRMSNorm + FP8
# ---------------------------------------------------------------------------

def adarms_inputs(T, H, dtype, seed, mod_std=0.1):
    """x, residual ~ N(0,1); gate, ada_scale, ada_shift ~ N(0, mod_std^2),
    all [T,H] (one modulation vector per token)."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (T, H))
    r = normal(rng, (T, H))
    gate = normal(rng, (T, H), std=mod_std)
    scale = normal(rng, (T, H), std=mod_std)
    shift = normal(rng, (T, H), std=mod_std)
    return {"x": to16(x, dtype), "residual": to16(r, dtype),
            "gate": to16(gate, dtype), "ada_scale": to16(scale, dtype),
            "ada_shift": to16(shift, dtype)}


# ---------------------------------------------------------------------------
# packed QKV + norm + RoPE + paged KV write
# ---------------------------------------------------------------------------

SENTINEL = 0x7C01   # a float16/bfloat16 NaN pattern never produced by the ops


def qkv_inputs(T, Hq, Hkv, D, dtype, seed, page_size, num_pages,
               positions=None, norm=True, random_pages=True, norm_std=0.05):
    """qkv ~ N(0,1) [T, (Hq+2Hkv)*D]; q/k norm weights ~ 1 + N(0, norm_std^2)
    [D] (None when norm is False); positions default to 0..T-1; page table =
    seeded permutation of the pages (identity when random_pages is False);
    caches [num_pages, page_size, Hkv, D] filled with a sentinel pattern."""
    rng = np.random.default_rng(seed)
    qkv = normal(rng, (T, (Hq + 2 * Hkv) * D))
    qw = normal(rng, (D,), std=norm_std, mean=1.0)
    kw = normal(rng, (D,), std=norm_std, mean=1.0)
    if positions is None:
        positions = np.arange(T, dtype=np.int32)
    if random_pages:
        table = rng.permutation(num_pages).astype(np.int32)
    else:
        table = np.arange(num_pages, dtype=np.int32)
    cache_shape = (num_pages, page_size, Hkv, D)
    return {"qkv": to16(qkv, dtype),
            "q_norm_w": to16(qw, dtype) if norm else None,
            "k_norm_w": to16(kw, dtype) if norm else None,
            "positions": np.asarray(positions, dtype=np.int32),
            "page_table": table,
            "k_cache": np.full(cache_shape, SENTINEL, dtype=np.uint16),
            "v_cache": np.full(cache_shape, SENTINEL, dtype=np.uint16)}


# ---------------------------------------------------------------------------
# gated activation + block-128 FP8
# ---------------------------------------------------------------------------

def gated_act_inputs(T, I, dtype, seed, outliers=False):
    """gate_up [T, 2I] ~ N(0,1), interleaved g0,u0,g1,u1,..."""
    rng = np.random.default_rng(seed)
    gu = normal(rng, (T, 2 * I))
    if outliers:
        gu = with_outliers(rng, gu)
    return {"gate_up": to16(gu, dtype)}


# ---------------------------------------------------------------------------
# decoder-step chain (Pi0.5 action decoder: 18 layers x 10 flow steps)
# ---------------------------------------------------------------------------

def chain_inputs(seed=102, layers=18, steps=10, T=10, H=1024, Hq=8, Hkv=1,
                 D=256, page_size=1024, prefix=790, mod_std=0.1):
    """Per layer: x_l [T,H] and qkv_l [T,(Hq+2Hkv)D] ~ N(0,1); per (layer,
    step): gate, ada_scale, ada_shift [T,H] ~ N(0, mod_std^2); residual chain
    seed r0 [T,H] ~ N(0,1); per-layer K/V caches [1, page_size, Hkv, D] with
    slots below `prefix` ~ N(0,1) and the rest sentinel; positions
    prefix..prefix+T-1; page table [0].  All float16."""
    rng = np.random.default_rng(seed)
    dt = F16
    n = layers * steps
    out = {
        "x": to16(normal(rng, (layers, T, H)), dt),
        "qkv": to16(normal(rng, (layers, T, (Hq + 2 * Hkv) * D)), dt),
        "gate": to16(normal(rng, (n, T, H), std=mod_std), dt),
        "ada_scale": to16(normal(rng, (n, T, H), std=mod_std), dt),
        "ada_shift": to16(normal(rng, (n, T, H), std=mod_std), dt),
        "r0": to16(normal(rng, (T, H)), dt),
        "positions": np.arange(prefix, prefix + T, dtype=np.int32),
        "page_table": np.zeros(1, dtype=np.int32),
    }
    kc = np.full((layers, 1, page_size, Hkv, D), SENTINEL, dtype=np.uint16)
    vc = np.full((layers, 1, page_size, Hkv, D), SENTINEL, dtype=np.uint16)
    kc[:, 0, :prefix] = to16(normal(rng, (layers, prefix, Hkv, D)), dt)
    vc[:, 0, :prefix] = to16(normal(rng, (layers, prefix, Hkv, D)), dt)
    out["k_cache"] = kc
    out["v_cache"] = vc
    out["dims"] = dict(layers=layers, steps=steps, T=T, H=H, Hq=Hq, Hkv=Hkv,
                       D=D, page_size=page_size)
    return out


# ---------------------------------------------------------------------------
# FP8 GEMM fused with the gated activation (gate_up projection)
# ---------------------------------------------------------------------------

def e4m3_codes(x):
    """float32 array -> OCP e4m3 codes through torch's float8_e4m3fn cast
    (values must be within +-448)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def gemm_inputs(M, K, I, seed, scale_lo=0.5, scale_hi=2.0):
    """A [M, K] and W [2I, K] as e4m3 codes of N(0,1) draws (x 32, well
    inside the e4m3 range), with positive uniform block dequant scales:
    a_scales [M, K/128] and w_scales [2I/128, K/128], each U(lo, hi) / 32 /
    sqrt(K).  W rows interleave gate (2j) and up (2j+1) rows."""
    rng = np.random.default_rng(seed)
    a = e4m3_codes(normal(rng, (M, K)) * np.float32(32.0))
    w = e4m3_codes(normal(rng, (2 * I, K)) * np.float32(32.0))
    unit = np.float32(1.0 / 32.0 / np.sqrt(K))
    a_s = rng.uniform(scale_lo, scale_hi, (M, K // 128)).astype(np.float32) * unit
    w_s = rng.uniform(scale_lo, scale_hi, (2 * I // 128, K // 128)).astype(np.float32) * np.float32(1.0 / 32.0)
    return {"a": a, "a_scales": a_s, "w": w, "w_scales": w_s}


# ---------------------------------------------------------------------------
# Q/K norm + RoPE variants (Chameleon LayerNorm per head, Wan full-width
# RMSNorm + 3D RoPE)
# ---------------------------------------------------------------------------

def qk_norm_rope_inputs(T, Hq, Hkv, D, dtype, seed, scope_full=False, rope3=False,
                        grid=(4, 8, 8), norm_std=0.05):
    """qkv ~ N(0,1) [T, (Hq+2Hkv)D]; norm weights 1 + N(0, norm_std^2) and
    biases N(0, norm_std^2), [D] per head or [Hq D] / [Hkv D] full width;
    positions 0..T-1, or for 3D the (time, height, width) coordinates of
    token t on a frames x height x width grid in raster order."""
    rng = np.random.default_rng(seed)
    qkv = normal(rng, (T, (Hq + 2 * Hkv) * D))
    nq, nk = (Hq * D, Hkv * D) if scope_full else (D, D)
    out = {"qkv": to16(qkv, dtype),
           "q_norm_w": to16(normal(rng, (nq,), std=norm_std, mean=1.0), dtype),
           "q_norm_b": to16(normal(rng, (nq,), std=norm_std), dtype),
           "k_norm_w": to16(normal(rng, (nk,), std=norm_std, mean=1.0), dtype),
           "k_norm_b": to16(normal(rng, (nk,), std=norm_std), dtype)}
    if rope3:
        f, h, w = grid
        t = np.arange(T)
        out["positions"] = np.stack([t // (h * w), (t // w) % h, t % w], axis=1).astype(np.int32)
    else:
        out["positions"] = np.arange(T, dtype=np.int32)
    return out
