"""Plain CPU oracle for the fused layer-boundary ops (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
library never links, loads or calls it, and it shares no code with the HIP
path: its own C source (``oracle.c``) implements every number format and
every step in double precision.

All tensors are numpy arrays on the host: 16-bit storage types as uint16 bit
patterns, FP8 codes as uint8, scales as float32.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

F16, BF16 = 0, 1
W_NONE, W_MUL, W_ONE_PLUS = 0, 1, 2
Q_STATIC, Q_TOKEN = 0, 1
ACT_SWIGLU, ACT_GEGLU_TANH, ACT_SQRELU = 0, 1, 2
ROPE_HALF, ROPE_INTERLEAVED = 0, 1


def build():
    """Compile liboracle.so with gcc (strict IEEE: no fast-math, no FMA
    contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-shared", "-fPIC", _SRC, "-o", LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_INT = ctypes.c_int
_F = ctypes.c_float
_D = ctypes.c_double


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        L.or_f16_decode.argtypes = [ctypes.c_uint16]
        L.or_f16_decode.restype = _D
        L.or_bf16_decode.argtypes = [ctypes.c_uint16]
        L.or_bf16_decode.restype = _D
        L.or_f16_encode.argtypes = [_D]
        L.or_f16_encode.restype = ctypes.c_uint16
        L.or_bf16_encode.argtypes = [_D]
        L.or_bf16_encode.restype = ctypes.c_uint16
        L.or_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.or_e4m3_decode.restype = _D
        L.or_e4m3_encode.argtypes = [_D]
        L.or_e4m3_encode.restype = ctypes.c_uint8
        L.or_f32_round.argtypes = [_D]
        L.or_f32_round.restype = _F
        for f in ("or_e4m3_encode_n", "or_f16_encode_n", "or_bf16_encode_n"):
            getattr(L, f).argtypes = [_P, _I64, _P]
            getattr(L, f).restype = None
        L.or_rms_rstd.argtypes = [_P, _I64, _D]
        L.or_rms_rstd.restype = _D
        L.or_rmsnorm.argtypes = [_P, _P, _INT, _I64, _D, _P]
        L.or_rmsnorm.restype = None
        L.or_adarms.argtypes = [_P, _P, _P, _I64, _D, _P]
        L.or_adarms.restype = None
        L.or_rope.argtypes = [_P, _I64, _I64, _D, _INT]
        L.or_rope.restype = None
        L.or_act.argtypes = [_D, _INT]
        L.or_act.restype = _D
        L.or_quant_static.argtypes = [_P, _I64, _D, _P]
        L.or_quant_static.restype = None
        L.or_quant_dynamic.argtypes = [_P, _I64, _P]
        L.or_quant_dynamic.restype = _F
        L.or_kv_slot.argtypes = [_I64, _P, _I32, _I32, _I32]
        L.or_kv_slot.restype = _I64
        L.or_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.or_e2m1_decode.restype = _D
        L.or_e2m1_encode.argtypes = [_D]
        L.or_e2m1_encode.restype = ctypes.c_uint8
        L.or_mx_scale_code.argtypes = [_D]
        L.or_mx_scale_code.restype = _INT
        L.or_quant_mxfp4.argtypes = [_P, _I64, _P, _P]
        L.or_quant_mxfp4.restype = None
        L.or_quant_nvfp4.argtypes = [_P, _I64, _D, _P, _P]
        L.or_quant_nvfp4.restype = None
        L.oracle_resid_rmsnorm_nvfp4.argtypes = [
            _P, _P, _P, _P, _INT, _F, _F, _P, _P, _I64, _I64, _INT]
        L.oracle_resid_rmsnorm_nvfp4.restype = _INT
        L.oracle_resid_rmsnorm_mxfp4.argtypes = [
            _P, _P, _P, _P, _INT, _F, _P, _P, _I64, _I64, _INT]
        L.oracle_resid_rmsnorm_mxfp4.restype = _INT
        L.oracle_gated_act_mxfp4.argtypes = [_P, _INT, _P, _P, _I64, _I64, _INT]
        L.oracle_gated_act_mxfp4.restype = _INT
        L.oracle_resid_layernorm.argtypes = [
            _P, _P, _P, _P, _P, _F, _INT, _P, _INT, _F, _P, _P, _I64, _I64, _INT]
        L.oracle_resid_layernorm.restype = _INT
        L.oracle_resid_layernorm_nvfp4.argtypes = [
            _P, _P, _P, _P, _P, _F, _F, _P, _P, _I64, _I64, _INT]
        L.oracle_resid_layernorm_nvfp4.restype = _INT
        L.or_layernorm.argtypes = [_P, _P, _P, _I64, _D, _P]
        L.or_layernorm.restype = None
        L.or_rope3d.argtypes = [_P, _I64, _P, _P, _D, _INT]
        L.or_rope3d.restype = None
        L.oracle_qk_norm_rope.argtypes = [
            _P, _INT, _INT, _P, _P, _P, _P, _F, _P, _INT, _P, _F, _INT, _F,
            _P, _P, _P, _I64, _I32, _I32, _I32, _INT]
        L.oracle_qk_norm_rope.restype = _INT
        L.oracle_resid_rmsnorm_fp8.argtypes = [
            _P, _P, _P, _P, _INT, _F, _P, _INT, _F, _P, _I64, _I64, _INT]
        L.oracle_adarms_gate_res_fp8.argtypes = [
            _P, _P, _P, _P, _P, _P, _F, _P, _INT, _F, _P, _I64, _I64, _INT]
        L.oracle_qkv_normrope_kvwrite.argtypes = [
            _P, _P, _P, _F, _P, _F, _INT, _F, _P, _P, _P, _P, _I32, _I32, _I32,
            _P, _I64, _I32, _I32, _I32, _INT]
        L.oracle_gated_act_fp8.argtypes = [_P, _INT, _P, _P, _I64, _I64, _INT]
        L.oracle_gated_act_fp8_f64.argtypes = [_P, _INT, _P, _P, _I64, _I64]
        L.oracle_gated_act_fp8_f64.restype = _INT
        for f in ("oracle_resid_rmsnorm_fp8", "oracle_adarms_gate_res_fp8",
                  "oracle_qkv_normrope_kvwrite", "oracle_gated_act_fp8"):
            getattr(L, f).restype = _INT
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dt)


# ---- number formats -------------------------------------------------------

def f16_decode(b):
    return lib().or_f16_decode(int(b))


def bf16_decode(b):
    return lib().or_bf16_decode(int(b))


def f16_encode(v):
    return lib().or_f16_encode(float(v))


def bf16_encode(v):
    return lib().or_bf16_encode(float(v))


def e4m3_decode(c):
    return lib().or_e4m3_decode(int(c))


def e4m3_encode(v):
    return lib().or_e4m3_encode(float(v))


_dec_cache = {}


def decode16(bits, dtype):
    """Vector decode of uint16 bit patterns to float64 (through a table
    filled from the oracle's scalar decoder)."""
    table = _dec_cache.get(dtype)
    if table is None:
        f = f16_decode if dtype == F16 else bf16_decode
        table = np.array([f(i) for i in range(65536)], dtype=np.float64)
        _dec_cache[dtype] = table
    return table[np.asarray(bits, dtype=np.uint16)]


def e4m3_encode_n(v):
    v = _c(np.ravel(v), np.float64)
    out = np.empty(v.size, dtype=np.uint8)
    lib().or_e4m3_encode_n(_ptr(v), v.size, _ptr(out))
    return out


def encode16_n(v, dtype):
    v = _c(np.ravel(v), np.float64)
    out = np.empty(v.size, dtype=np.uint16)
    f = lib().or_f16_encode_n if dtype == F16 else lib().or_bf16_encode_n
    f(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_table():
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e2m1_decode(c):
    return lib().or_e2m1_decode(int(c))


def e2m1_encode(v):
    return lib().or_e2m1_encode(float(v))


def mx_scale_code(amax):
    return lib().or_mx_scale_code(float(amax))


def quant_mxfp4(y):
    """y: float64 [n], n % 32 == 0 -> (packed uint8 [n/2], scales uint8 [n/32])."""
    y = _c(np.ravel(y), np.float64)
    assert y.size % 32 == 0
    packed = np.empty(y.size // 2, dtype=np.uint8)
    scales = np.empty(y.size // 32, dtype=np.uint8)
    lib().or_quant_mxfp4(_ptr(y), y.size, _ptr(packed), _ptr(scales))
    return packed, scales


def quant_nvfp4(y, global_scale):
    """y: float64 [n], n % 16 == 0 -> (packed uint8 [n/2], E4M3 block scale
    codes uint8 [n/16])."""
    y = _c(np.ravel(y), np.float64)
    assert y.size % 16 == 0
    packed = np.empty(y.size // 2, dtype=np.uint8)
    scales = np.empty(y.size // 16, dtype=np.uint8)
    lib().or_quant_nvfp4(_ptr(y), y.size, float(global_scale), _ptr(packed), _ptr(scales))
    return packed, scales


def unpack_fp4(packed):
    """uint8 [..., n/2] -> 4-bit codes uint8 [..., n] (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ---- building blocks --------------------------------------------------------

def rms_rstd(v, eps):
    v = _c(v, np.float64)
    return lib().or_rms_rstd(_ptr(v), v.size, float(eps))


def rmsnorm(v, w, wmode, eps):
    v = _c(v, np.float64)
    w = _c(w, np.float64) if w is not None else np.zeros_like(v)
    y = np.empty_like(v)
    lib().or_rmsnorm(_ptr(v), _ptr(w), wmode, v.size, float(eps), _ptr(y))
    return y


def adarms(h, scale, shift, eps):
    h = _c(h, np.float64)
    scale = _c(scale, np.float64)
    shift = _c(shift, np.float64)
    y = np.empty_like(h)
    lib().or_adarms(_ptr(h), _ptr(scale), _ptr(shift), h.size, float(eps),
                    _ptr(y))
    return y


def rope(v, pos, theta, style=ROPE_HALF):
    v = np.array(v, dtype=np.float64, copy=True)
    lib().or_rope(_ptr(v), v.size, int(pos), float(theta), style)
    return v


def act(g, kind):
    return lib().or_act(float(g), kind)


def quant_static(y, mult):
    y = _c(y, np.float64)
    q = np.empty(y.size, dtype=np.uint8)
    lib().or_quant_static(_ptr(y), y.size, float(mult), _ptr(q))
    return q


def quant_dynamic(y):
    y = _c(y, np.float64)
    q = np.empty(y.size, dtype=np.uint8)
    s = lib().or_quant_dynamic(_ptr(y), y.size, _ptr(q))
    return q, np.float32(s)


def kv_slot(pos, page_table, page_size, num_pages):
    pt = _c(page_table, np.int32)
    return lib().or_kv_slot(int(pos), _ptr(pt), pt.size, page_size, num_pages)


# ---- fused ops ----------------------------------------------------------------

def resid_rmsnorm_fp8(x, residual, weight, wmode, eps, qmode, static_scale,
                      dtype):
    """Returns (residual_out uint16 [T,H], out_fp8 uint8 [T,H],
    out_scales float32 [T] or None)."""
    x = _c(x, np.uint16)
    residual = _c(residual, np.uint16)
    T, H = x.shape
    weight = _c(weight, np.uint16)
    ro = np.empty_like(x)
    q = np.empty((T, H), dtype=np.uint8)
    sc = np.empty(T, dtype=np.float32) if qmode == Q_TOKEN else None
    rc = lib().oracle_resid_rmsnorm_fp8(
        _ptr(x), _ptr(residual), _ptr(ro), _ptr(weight), wmode, eps, _ptr(q),
        qmode, static_scale, _ptr(sc), T, H, dtype)
    assert rc == 0
    return ro, q, sc


def adarms_gate_res_fp8(x, gate, residual, ada_scale, ada_shift, eps, qmode,
                        static_scale, dtype):
    x, gate, residual, ada_scale, ada_shift = (
        _c(a, np.uint16) for a in (x, gate, residual, ada_scale, ada_shift))
    T, H = x.shape
    ro = np.empty_like(x)
    q = np.empty((T, H), dtype=np.uint8)
    sc = np.empty(T, dtype=np.float32) if qmode == Q_TOKEN else None
    rc = lib().oracle_adarms_gate_res_fp8(
        _ptr(x), _ptr(gate), _ptr(residual), _ptr(ro), _ptr(ada_scale),
        _ptr(ada_shift), eps, _ptr(q), qmode, static_scale, _ptr(sc), T, H,
        dtype)
    assert rc == 0
    return ro, q, sc


def qkv_normrope_kvwrite(qkv, q_norm_w, k_norm_w, eps, positions, rope_theta,
                         rope_style, k_cache, v_cache, page_table, page_size,
                         Hq, Hkv, D, dtype, q_scale=1.0):
    """k_cache / v_cache are updated in place (uint16 [pages, P, Hkv, D]).
    q_scale multiplies Q after RoPE (attention's pre-scale; 1 = none).
    Returns (q_out uint16 [T,Hq,D], err_flag int)."""
    qkv = _c(qkv, np.uint16)
    T = qkv.shape[0]
    q_norm_w = _c(q_norm_w, np.uint16)
    k_norm_w = _c(k_norm_w, np.uint16)
    positions = _c(positions, np.int32)
    page_table = _c(page_table, np.int32)
    assert k_cache.dtype == np.uint16 and k_cache.flags.c_contiguous
    assert v_cache.dtype == np.uint16 and v_cache.flags.c_contiguous
    num_pages = k_cache.shape[0]
    q_out = np.empty((T, Hq, D), dtype=np.uint16)
    err = np.zeros(1, dtype=np.int32)
    rc = lib().oracle_qkv_normrope_kvwrite(
        _ptr(qkv), _ptr(q_norm_w), _ptr(k_norm_w), eps, _ptr(positions),
        rope_theta, rope_style, q_scale, _ptr(q_out), _ptr(k_cache),
        _ptr(v_cache), _ptr(page_table), page_table.size, page_size, num_pages,
        _ptr(err), T, Hq, Hkv, D, dtype)
    assert rc == 0
    return q_out, int(err[0])


def gated_act_fp8(gate_up, act_kind, dtype):
    """Returns (out_fp8 uint8 [T,I], out_scales float32 [T, I/128])."""
    gate_up = _c(gate_up, np.uint16)
    T, I2 = gate_up.shape
    I = I2 // 2
    q = np.empty((T, I), dtype=np.uint8)
    sc = np.empty((T, I // 128), dtype=np.float32)
    rc = lib().oracle_gated_act_fp8(_ptr(gate_up), act_kind, _ptr(q), _ptr(sc),
                                    T, I, dtype)
    assert rc == 0
    return q, sc


def resid_rmsnorm_mxfp4(x, residual, weight, wmode, eps, dtype):
    """Returns (residual_out uint16 [T,H], out_fp4 uint8 [T,H/2],
    out_scales uint8 [T,H/32] E8M0 codes)."""
    x = _c(x, np.uint16)
    residual = _c(residual, np.uint16)
    T, H = x.shape
    weight = _c(weight, np.uint16)
    ro = np.empty_like(x)
    q = np.empty((T, H // 2), dtype=np.uint8)
    sc = np.empty((T, H // 32), dtype=np.uint8)
    rc = lib().oracle_resid_rmsnorm_mxfp4(
        _ptr(x), _ptr(residual), _ptr(ro), _ptr(weight), wmode, eps, _ptr(q),
        _ptr(sc), T, H, dtype)
    assert rc == 0
    return ro, q, sc


def resid_rmsnorm_nvfp4(x, residual, weight, wmode, eps, global_scale, dtype):
    """Returns (residual_out uint16 [T,H], out_fp4 uint8 [T,H/2],
    out_scales uint8 [T,H/16] E4M3 block scale codes)."""
    x = _c(x, np.uint16)
    residual = _c(residual, np.uint16)
    T, H = x.shape
    weight = _c(weight, np.uint16)
    ro = np.empty_like(x)
    q = np.empty((T, H // 2), dtype=np.uint8)
    sc = np.empty((T, H // 16), dtype=np.uint8)
    rc = lib().oracle_resid_rmsnorm_nvfp4(
        _ptr(x), _ptr(residual), _ptr(ro), _ptr(weight), wmode, eps, global_scale,
        _ptr(q), _ptr(sc), T, H, dtype)
    assert rc == 0
    return ro, q, sc


def gated_act_mxfp4(gate_up, act_kind, dtype):
    """Returns (out_fp4 uint8 [T,I/2], out_scales uint8 [T,I/32])."""
    gate_up = _c(gate_up, np.uint16)
    T, I2 = gate_up.shape
    I = I2 // 2
    q = np.empty((T, I // 2), dtype=np.uint8)
    sc = np.empty((T, I // 32), dtype=np.uint8)
    rc = lib().oracle_gated_act_mxfp4(_ptr(gate_up), act_kind, _ptr(q),
                                      _ptr(sc), T, I, dtype)
    assert rc == 0
    return q, sc


NORM_NONE, NORM_RMS, NORM_LAYER = 0, 1, 2
SCOPE_HEAD, SCOPE_FULL = 0, 1


def layernorm(v, w=None, b=None, eps=1e-6):
    v = _c(v, np.float64)
    w = _c(w, np.float64) if w is not None else None
    b = _c(b, np.float64) if b is not None else None
    y = np.empty_like(v)
    lib().or_layernorm(_ptr(v), _ptr(w), _ptr(b), v.size, float(eps), _ptr(y))
    return y


def rope3d(v, pos3, sections, theta, style=ROPE_HALF):
    v = _c(v, np.float64).copy()
    p = np.ascontiguousarray(pos3, dtype=np.int32)
    sec = np.ascontiguousarray(sections, dtype=np.int32)
    lib().or_rope3d(_ptr(v), v.size, _ptr(p), _ptr(sec), float(theta), style)
    return v


def resid_layernorm(x, residual, weight, bias, eps, out_kind, qmode, static_scale,
                    dtype):
    """out_kind 0 (FP8): returns (residual_out, codes [T,H], scales [T] or None);
    out_kind 1 (MXFP4): returns (residual_out, packed [T,H/2], e8m0 [T,H/32])."""
    x = _c(x, np.uint16)
    residual = _c(residual, np.uint16)
    T, H = x.shape
    weight = _c(weight, np.uint16)
    bias = _c(bias, np.uint16)
    ro = np.empty_like(x)
    if out_kind == 1:
        q = np.empty((T, H // 2), np.uint8)
        sc8 = np.empty((T, H // 32), np.uint8)
        scf = None
    else:
        q = np.empty((T, H), np.uint8)
        sc8 = None
        scf = np.empty(T, np.float32) if qmode == Q_TOKEN else None
    rc = lib().oracle_resid_layernorm(
        _ptr(x), _ptr(residual), _ptr(ro), _ptr(weight), _ptr(bias), eps, out_kind,
        _ptr(q), qmode, static_scale, _ptr(scf), _ptr(sc8), T, H, dtype)
    assert rc == 0
    return ro, q, (sc8 if out_kind == 1 else scf)


def resid_layernorm_nvfp4(x, residual, weight, bias, eps, global_scale, dtype):
    """Returns (residual_out uint16 [T,H], out_fp4 uint8 [T,H/2],
    out_scales uint8 [T,H/16] E4M3 block scale codes)."""
    x = _c(x, np.uint16)
    residual = _c(residual, np.uint16)
    T, H = x.shape
    weight = _c(weight, np.uint16)
    bias = None if bias is None else _c(bias, np.uint16)
    ro = np.empty_like(x)
    q = np.empty((T, H // 2), np.uint8)
    sc = np.empty((T, H // 16), np.uint8)
    rc = lib().oracle_resid_layernorm_nvfp4(
        _ptr(x), _ptr(residual), _ptr(ro), _ptr(weight), _ptr(bias), eps, global_scale,
        _ptr(q), _ptr(sc), T, H, dtype)
    assert rc == 0
    return ro, q, sc


def qk_norm_rope(qkv, norm_kind, norm_scope, q_norm_w, q_norm_b, k_norm_w,
                 k_norm_b, eps, positions, rope_dims, sections, rope_theta,
                 rope_style, q_scale, Hq, Hkv, D, dtype):
    """Returns (q_out [T,Hq,D], k_out [T,Hkv,D], v_out [T,Hkv,D]) uint16."""
    qkv = _c(qkv, np.uint16)
    T = qkv.shape[0]
    ws = [_c(a, np.uint16) for a in (q_norm_w, q_norm_b, k_norm_w, k_norm_b)]
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    sec = np.ascontiguousarray(sections, dtype=np.int32) if sections is not None else None
    q = np.empty((T, Hq, D), np.uint16)
    k = np.empty((T, Hkv, D), np.uint16)
    v = np.empty((T, Hkv, D), np.uint16)
    rc = lib().oracle_qk_norm_rope(
        _ptr(qkv), norm_kind, norm_scope, *[_ptr(a) for a in ws], eps, _ptr(pos),
        rope_dims, _ptr(sec), rope_theta, rope_style, q_scale, _ptr(q), _ptr(k),
        _ptr(v), T, Hq, Hkv, D, dtype)
    assert rc == 0
    return q, k, v


def gated_act_fp8_f64(gate_up, act_kind):
    """Same as gated_act_fp8 on float64 gate/up values [T, 2I]."""
    gate_up = _c(gate_up, np.float64)
    T, I2 = gate_up.shape
    I = I2 // 2
    q = np.empty((T, I), dtype=np.uint8)
    sc = np.empty((T, I // 128), dtype=np.float32)
    rc = lib().oracle_gated_act_fp8_f64(_ptr(gate_up), act_kind, _ptr(q),
                                        _ptr(sc), T, I)
    assert rc == 0
    return q, sc


def dequant_blocks(codes, scales, rows_per_scale):
    """e4m3 codes [R, K] times block dequant scales: scales[r // rows_per_scale,
    k // 128] (rows_per_scale = 1 for per-token activation scales, 128 for
    128 x 128 weight blocks).  Returns float64 [R, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, K = codes.shape
    v = e4m3_table()[codes]
    s = np.asarray(scales, dtype=np.float64)
    s_full = np.repeat(np.repeat(s, rows_per_scale, axis=0)[:R], 128, axis=1)[:, :K]
    return v * s_full


def gemm_gated_act_fp8(a, a_scales, w, w_scales, act_kind):
    """FP8 block-scaled GEMM fused with the gated activation and block-128
    FP8 output [SM89 Phase 2]:
      A [M, K] e4m3 with per-token block-128 dequant scales a_scales [M, K/128]
      W [2I, K] e4m3, rows interleaved (gate row j at 2j, up row j at 2j+1),
        with 128 x 128 block dequant scales w_scales [2I/128, K/128]
      acc = dequant(A) @ dequant(W)^T in float64 (numpy matmul)
      then act(acc[:, 2j]) * acc[:, 2j+1] and block-128 quantisation.
    Returns (codes uint8 [M, I], scales float32 [M, I/128], acc float64)."""
    A = dequant_blocks(a, a_scales, 1)
    W = dequant_blocks(w, w_scales, 128)
    acc = A @ W.T
    q, sc = gated_act_fp8_f64(acc, act_kind)
    return q, sc, acc
