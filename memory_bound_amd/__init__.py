"""Python binding of libfrhip.so, the fused layer-boundary kernels for
MI355X (gfx950).

Argument marshalling only: every function here has the name and the argument
order of the C entry point in include/fr.h, converts tensors to device
pointers, and calls the library once.  Tensor arguments may be torch device
tensors, raw integer device addresses, or None (NULL).  ``stream`` defaults
to torch's current stream.  A nonzero status raises FrError.

Importing this package loads the HIP library; a missing library is an error
(there is no fallback implementation).
"""
import ctypes
import os

# torch first: its bundled HIP runtime (SONAME libamdhip64.so.7) must be the
# one this library binds to, so that torch's streams and allocations and the
# library's launches share one runtime.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfrhip.so")

F16, BF16 = 0, 1
W_NONE, W_MUL, W_ONE_PLUS = 0, 1, 2
Q_STATIC, Q_TOKEN = 0, 1
ACT_SWIGLU, ACT_GEGLU_TANH, ACT_SQRELU = 0, 1, 2
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
NORM_NONE, NORM_RMS, NORM_LAYER = 0, 1, 2
SCOPE_HEAD, SCOPE_FULL = 0, 1

FR_OK, FR_ERR_NULL, FR_ERR_SHAPE, FR_ERR_DTYPE, FR_ERR_ALIGN, FR_ERR_MODE, \
    FR_ERR_UNSUPPORTED, FR_ERR_LAUNCH = range(8)


class FrError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_INT = ctypes.c_int
_F = ctypes.c_float

_SIGS = {
    "fr_resid_rmsnorm_fp8": [_P, _P, _P, _P, _INT, _F, _P, _INT, _F, _P, _I64,
                             _I64, _INT, _P],
    "fr_adarms_gate_res_fp8": [_P, _P, _P, _P, _P, _P, _F, _P, _INT, _F, _P,
                               _I64, _I64, _INT, _P],
    "fr_qkv_normrope_kvwrite": [_P, _P, _P, _F, _P, _F, _INT, _F, _P, _P, _P,
                                _P, _I32, _I32, _I32, _P, _I64, _I32, _I32,
                                _I32, _INT, _P],
    "fr_gated_act_fp8": [_P, _INT, _P, _P, _I64, _I64, _INT, _P],
    "fr_gemm_gated_act_fp8": [_P, _P, _P, _P, _INT, _P, _P, _I64, _I64, _I64,
                              _P],
    "fr_gemm_pack_weights": [_P, _P, _I64, _I64, _P],
    "fr_resid_rmsnorm_mxfp4": [_P, _P, _P, _P, _INT, _F, _P, _P, _I64, _I64,
                               _INT, _P],
    "fr_resid_rmsnorm_nvfp4": [_P, _P, _P, _P, _INT, _F, _F, _P, _P, _I64, _I64,
                               _INT, _P],
    "fr_gated_act_mxfp4": [_P, _INT, _P, _P, _I64, _I64, _INT, _P],
    "fr_resid_layernorm_fp8": [_P, _P, _P, _P, _P, _F, _P, _INT, _F, _P, _I64,
                               _I64, _INT, _P],
    "fr_resid_layernorm_mxfp4": [_P, _P, _P, _P, _P, _F, _P, _P, _I64, _I64,
                                 _INT, _P],
    "fr_resid_layernorm_nvfp4": [_P, _P, _P, _P, _P, _F, _F, _P, _P, _I64, _I64,
                                 _INT, _P],
    "fr_qk_norm_rope": [_P, _INT, _INT, _P, _P, _P, _P, _F, _P, _INT, _I32,
                        _I32, _I32, _F, _INT, _F, _P, _P, _P, _I64, _I32, _I32,
                        _I32, _INT, _P],
    "fr_decode_chain_persistent": [_P, _P, _P, _P, _P, _P, _F, _F, _P, _P, _F,
                                   _INT, _P, _P, _P, _P, _I32, _I32, _I32, _P,
                                   _I32, _I32, _I64, _I64, _I32, _I32, _I32,
                                   _INT, _P],
}


def hip_runtimes():
    """Paths of the HIP runtime libraries mapped into this process."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6 and "libamdhip64" in parts[-1]:
                paths.add(parts[-1])
    return sorted(paths)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built: run `python -m memory_bound_amd.build` "
            "(the kernels have no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, argtypes in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = _INT
    lib.fr_status_string.argtypes = [_INT]
    lib.fr_status_string.restype = ctypes.c_char_p
    lib.fr_abi_version.argtypes = []
    lib.fr_abi_version.restype = _INT
    rt = hip_runtimes()
    if len(rt) != 1:
        raise ImportError(f"expected one HIP runtime in the process, found {rt}")
    return lib


lib = _load()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status):
    if status != FR_OK:
        raise FrError(status, lib.fr_status_string(status).decode())


def status_string(status):
    return lib.fr_status_string(status).decode()


def abi_version():
    return lib.fr_abi_version()


def fr_resid_rmsnorm_fp8(x, residual, residual_out, weight, wmode, eps, out_fp8,
                         qmode, static_scale, out_scales, T, H, dtype,
                         stream=None):
    _check(lib.fr_resid_rmsnorm_fp8(
        _ptr(x), _ptr(residual), _ptr(residual_out), _ptr(weight), wmode, eps,
        _ptr(out_fp8), qmode, static_scale, _ptr(out_scales), T, H, dtype,
        _stream(stream)))


def fr_adarms_gate_res_fp8(x, gate, residual, residual_out, ada_scale,
                           ada_shift, eps, out_fp8, qmode, static_scale,
                           out_scales, T, H, dtype, stream=None):
    _check(lib.fr_adarms_gate_res_fp8(
        _ptr(x), _ptr(gate), _ptr(residual), _ptr(residual_out),
        _ptr(ada_scale), _ptr(ada_shift), eps, _ptr(out_fp8), qmode,
        static_scale, _ptr(out_scales), T, H, dtype, _stream(stream)))


def fr_qkv_normrope_kvwrite(qkv, q_norm_w, k_norm_w, eps, positions,
                            rope_theta, rope_style, q_out, k_cache, v_cache,
                            page_table, page_table_len, page_size, num_pages,
                            err_flag, T, Hq, Hkv, D, dtype, stream=None,
                            q_scale=1.0):
    _check(lib.fr_qkv_normrope_kvwrite(
        _ptr(qkv), _ptr(q_norm_w), _ptr(k_norm_w), eps, _ptr(positions),
        rope_theta, rope_style, q_scale, _ptr(q_out), _ptr(k_cache), _ptr(v_cache),
        _ptr(page_table), page_table_len, page_size, num_pages, _ptr(err_flag),
        T, Hq, Hkv, D, dtype, _stream(stream)))


def fr_gated_act_fp8(gate_up, act, out_fp8, out_scales, T, I, dtype,
                     stream=None):
    _check(lib.fr_gated_act_fp8(
        _ptr(gate_up), act, _ptr(out_fp8), _ptr(out_scales), T, I, dtype,
        _stream(stream)))


def fr_resid_rmsnorm_mxfp4(x, residual, residual_out, weight, wmode, eps,
                           out_fp4, out_scales, T, H, dtype, stream=None):
    _check(lib.fr_resid_rmsnorm_mxfp4(
        _ptr(x), _ptr(residual), _ptr(residual_out), _ptr(weight), wmode, eps,
        _ptr(out_fp4), _ptr(out_scales), T, H, dtype, _stream(stream)))


def fr_resid_rmsnorm_nvfp4(x, residual, residual_out, weight, wmode, eps,
                           global_scale, out_fp4, out_scales, T, H, dtype,
                           stream=None):
    _check(lib.fr_resid_rmsnorm_nvfp4(
        _ptr(x), _ptr(residual), _ptr(residual_out), _ptr(weight), wmode, eps,
        global_scale, _ptr(out_fp4), _ptr(out_scales), T, H, dtype,
        _stream(stream)))


def fr_gated_act_mxfp4(gate_up, act, out_fp4, out_scales, T, I, dtype,
                       stream=None):
    _check(lib.fr_gated_act_mxfp4(
        _ptr(gate_up), act, _ptr(out_fp4), _ptr(out_scales), T, I, dtype,
        _stream(stream)))


def fr_decode_chain_persistent(x, gate, ada_scale, ada_shift, residual,
                               out_fp8, eps, static_scale, qkv, positions,
                               rope_theta, rope_style, q_out, k_cache, v_cache,
                               page_table, page_table_len, page_size, num_pages,
                               err_flag, layers, steps, T, H, Hq, Hkv, D, dtype,
                               stream=None):
    _check(lib.fr_decode_chain_persistent(
        _ptr(x), _ptr(gate), _ptr(ada_scale), _ptr(ada_shift), _ptr(residual),
        _ptr(out_fp8), eps, static_scale, _ptr(qkv), _ptr(positions),
        rope_theta, rope_style, _ptr(q_out), _ptr(k_cache), _ptr(v_cache),
        _ptr(page_table), page_table_len, page_size, num_pages, _ptr(err_flag),
        layers, steps, T, H, Hq, Hkv, D, dtype, _stream(stream)))


def fr_resid_layernorm_fp8(x, residual, residual_out, weight, bias, eps,
                           out_fp8, qmode, static_scale, out_scales, T, H,
                           dtype, stream=None):
    _check(lib.fr_resid_layernorm_fp8(
        _ptr(x), _ptr(residual), _ptr(residual_out), _ptr(weight), _ptr(bias),
        eps, _ptr(out_fp8), qmode, static_scale, _ptr(out_scales), T, H, dtype,
        _stream(stream)))


def fr_resid_layernorm_mxfp4(x, residual, residual_out, weight, bias, eps,
                             out_fp4, out_scales, T, H, dtype, stream=None):
    _check(lib.fr_resid_layernorm_mxfp4(
        _ptr(x), _ptr(residual), _ptr(residual_out), _ptr(weight), _ptr(bias),
        eps, _ptr(out_fp4), _ptr(out_scales), T, H, dtype, _stream(stream)))


def fr_resid_layernorm_nvfp4(x, residual, residual_out, weight, bias, eps,
                             global_scale, out_fp4, out_scales, T, H, dtype,
                             stream=None):
    _check(lib.fr_resid_layernorm_nvfp4(
        _ptr(x), _ptr(residual), _ptr(residual_out), _ptr(weight), _ptr(bias),
        eps, global_scale, _ptr(out_fp4), _ptr(out_scales), T, H, dtype,
        _stream(stream)))


def fr_qk_norm_rope(qkv, norm_kind, norm_scope, q_norm_w, q_norm_b, k_norm_w,
                    k_norm_b, eps, positions, rope_dims, sections, rope_theta,
                    rope_style, q_scale, q_out, k_out, v_out, T, Hq, Hkv, D,
                    dtype, stream=None):
    sec = tuple(sections) if sections is not None else (0, 0, 0)
    _check(lib.fr_qk_norm_rope(
        _ptr(qkv), norm_kind, norm_scope, _ptr(q_norm_w), _ptr(q_norm_b),
        _ptr(k_norm_w), _ptr(k_norm_b), eps, _ptr(positions), rope_dims, *sec,
        rope_theta, rope_style, q_scale, _ptr(q_out), _ptr(k_out), _ptr(v_out),
        T, Hq, Hkv, D, dtype, _stream(stream)))


def fr_gemm_gated_act_fp8(a, a_scales, w_packed, w_scales, act, out_fp8,
                          out_scales, M, K, I, stream=None):
    _check(lib.fr_gemm_gated_act_fp8(
        _ptr(a), _ptr(a_scales), _ptr(w_packed), _ptr(w_scales), act,
        _ptr(out_fp8), _ptr(out_scales), M, K, I, _stream(stream)))


def fr_gemm_pack_weights(w, w_packed, N, K, stream=None):
    _check(lib.fr_gemm_pack_weights(_ptr(w), _ptr(w_packed), N, K,
                                    _stream(stream)))
