// fr_api.hip -- the C ABI declared in include/fr.h: host-side validation,
// then exactly one kernel launch on the caller's stream.  No allocation, no
// copies, no synchronisation, no state.
#include <math.h>
#include <stdint.h>

#include "fr.h"
#include "fr_launch.h"

#define FR_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool finite_nonneg(float v) { return isfinite(v) && v >= 0.0f; }

int launch_status(hipError_t e) { return e == hipSuccess ? FR_OK : FR_ERR_LAUNCH; }

// Shared checks of ops (a) and (a').
int check_norm_common(float eps, const uint8_t* out_fp8, int qmode,
                      float static_scale, const float* out_scales, int64_t T,
                      int64_t H, int dtype) {
    if (dtype != FR_F16 && dtype != FR_BF16) return FR_ERR_DTYPE;
    if (T < 0 || H <= 0 || H % 16 != 0) return FR_ERR_SHAPE;
    if (H > 32768) return FR_ERR_UNSUPPORTED;
    if (T > 0x7fffffffLL) return FR_ERR_UNSUPPORTED;          // grid limit
    if (qmode != FR_Q_STATIC && qmode != FR_Q_TOKEN) return FR_ERR_MODE;
    if (!finite_nonneg(eps)) return FR_ERR_MODE;
    if (out_fp8 == nullptr) return FR_ERR_NULL;
    if (!aligned16(out_fp8)) return FR_ERR_ALIGN;
    if (qmode == FR_Q_STATIC) {
        if (!(isfinite(static_scale) && static_scale > 0.0f)) return FR_ERR_MODE;
    } else {
        if (out_scales == nullptr) return FR_ERR_NULL;
        if (!aligned16(out_scales)) return FR_ERR_ALIGN;
    }
    return FR_OK;
}

}  // namespace

FR_EXPORT int fr_resid_rmsnorm_fp8(const void* x, const void* residual,
                                   void* residual_out, const void* weight,
                                   int wmode, float eps, uint8_t* out_fp8,
                                   int qmode, float static_scale,
                                   float* out_scales, int64_t T, int64_t H,
                                   int dtype, void* stream) {
    int st = check_norm_common(eps, out_fp8, qmode, static_scale, out_scales, T, H, dtype);
    if (st != FR_OK) return st;
    if (wmode != FR_W_NONE && wmode != FR_W_MUL && wmode != FR_W_ONE_PLUS) return FR_ERR_MODE;
    if (!x || !residual || !residual_out) return FR_ERR_NULL;
    if (wmode != FR_W_NONE && !weight) return FR_ERR_NULL;
    if (!aligned16(x) || !aligned16(residual) || !aligned16(residual_out)) return FR_ERR_ALIGN;
    if (wmode != FR_W_NONE && !aligned16(weight)) return FR_ERR_ALIGN;
    if (T == 0) return FR_OK;

    fr::NormArgs a{};
    a.x = x;
    a.res = residual;
    a.res_out = residual_out;
    a.w = weight;
    a.out = out_fp8;
    a.scales = out_scales;
    a.T = T;
    a.H = (int)H;
    a.wmode = wmode;
    a.qmode = qmode;
    a.eps = eps;
    a.static_scale = static_scale;
    return launch_status(fr::launch_norm(a, dtype, fr::NORM_FP8, (hipStream_t)stream));
}

FR_EXPORT int fr_adarms_gate_res_fp8(const void* x, const void* gate,
                                     const void* residual, void* residual_out,
                                     const void* ada_scale, const void* ada_shift,
                                     float eps, uint8_t* out_fp8, int qmode,
                                     float static_scale, float* out_scales,
                                     int64_t T, int64_t H, int dtype,
                                     void* stream) {
    int st = check_norm_common(eps, out_fp8, qmode, static_scale, out_scales, T, H, dtype);
    if (st != FR_OK) return st;
    if (!x || !gate || !residual || !residual_out || !ada_scale || !ada_shift)
        return FR_ERR_NULL;
    if (!aligned16(x) || !aligned16(gate) || !aligned16(residual) ||
        !aligned16(residual_out) || !aligned16(ada_scale) || !aligned16(ada_shift))
        return FR_ERR_ALIGN;
    if (T == 0) return FR_OK;

    fr::NormArgs a{};
    a.x = x;
    a.gate = gate;
    a.res = residual;
    a.res_out = residual_out;
    a.ada_scale = ada_scale;
    a.ada_shift = ada_shift;
    a.out = out_fp8;
    a.scales = out_scales;
    a.T = T;
    a.H = (int)H;
    a.qmode = qmode;
    a.eps = eps;
    a.static_scale = static_scale;
    return launch_status(fr::launch_norm(a, dtype, fr::NORM_ADA_FP8, (hipStream_t)stream));
}

FR_EXPORT int fr_qkv_normrope_kvwrite(const void* qkv, const void* q_norm_w,
                                      const void* k_norm_w, float eps,
                                      const int32_t* positions, float rope_theta,
                                      int rope_style, float q_scale, void* q_out,
                                      void* k_cache,
                                      void* v_cache, const int32_t* page_table,
                                      int32_t page_table_len, int32_t page_size,
                                      int32_t num_pages, int32_t* err_flag,
                                      int64_t T, int32_t Hq, int32_t Hkv,
                                      int32_t D, int dtype, void* stream) {
    if (dtype != FR_F16 && dtype != FR_BF16) return FR_ERR_DTYPE;
    if (T < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || D % 16 != 0) return FR_ERR_SHAPE;
    if (page_table_len <= 0 || page_size <= 0 || num_pages <= 0) return FR_ERR_SHAPE;
    if (D > 256) return FR_ERR_UNSUPPORTED;
    if ((int64_t)Hq + 2 * (int64_t)Hkv > 65536) return FR_ERR_UNSUPPORTED;
    if (rope_style != FR_ROPE_HALF && rope_style != FR_ROPE_INTERLEAVED) return FR_ERR_MODE;
    if (!finite_nonneg(eps)) return FR_ERR_MODE;
    if (!(isfinite(rope_theta) && rope_theta > 1.0f)) return FR_ERR_MODE;
    if (!(isfinite(q_scale) && q_scale > 0.0f)) return FR_ERR_MODE;
    if (!qkv || !positions || !q_out || !k_cache || !v_cache || !page_table)
        return FR_ERR_NULL;
    if (!aligned16(qkv) || !aligned16(q_out) || !aligned16(k_cache) || !aligned16(v_cache))
        return FR_ERR_ALIGN;
    if ((q_norm_w && !aligned16(q_norm_w)) || (k_norm_w && !aligned16(k_norm_w)))
        return FR_ERR_ALIGN;
    if (!aligned4(positions) || !aligned4(page_table) || (err_flag && !aligned4(err_flag)))
        return FR_ERR_ALIGN;
    if (T == 0) return FR_OK;

    fr::QkvArgs a{};
    a.qkv = qkv;
    a.qw = q_norm_w;
    a.kw = k_norm_w;
    a.pos = positions;
    a.table = page_table;
    a.q_out = q_out;
    a.kc = k_cache;
    a.vc = v_cache;
    a.err = err_flag;
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.table_len = page_table_len;
    a.page_size = page_size;
    a.num_pages = num_pages;
    a.style = rope_style;
    a.eps = eps;
    a.theta = rope_theta;
    a.q_scale = q_scale;
    // one wave per (token, head group); the grid must fit in 32 bits
    if ((T * (int64_t)(Hq + 2 * Hkv)) / 4 + 1 > 0x7fffffffLL) return FR_ERR_UNSUPPORTED;
    return launch_status(fr::launch_qkv(a, dtype, (hipStream_t)stream));
}

FR_EXPORT int fr_gated_act_fp8(const void* gate_up, int act, uint8_t* out_fp8,
                               float* out_scales, int64_t T, int64_t I,
                               int dtype, void* stream) {
    if (dtype != FR_F16 && dtype != FR_BF16) return FR_ERR_DTYPE;
    if (T < 0 || I <= 0 || I % 128 != 0) return FR_ERR_SHAPE;
    if (I > (1 << 24)) return FR_ERR_UNSUPPORTED;
    if (act != FR_ACT_SWIGLU && act != FR_ACT_GEGLU_TANH && act != FR_ACT_SQRELU)
        return FR_ERR_MODE;
    if (!gate_up || !out_fp8 || !out_scales) return FR_ERR_NULL;
    if (!aligned16(gate_up) || !aligned16(out_fp8) || !aligned16(out_scales))
        return FR_ERR_ALIGN;
    if (T == 0) return FR_OK;
    // waves = T * ceil(I/1024); the grid (waves/4 blocks) must fit in 32 bits
    if (T * ((I + 1023) / 1024) / 4 + 1 > 0x7fffffffLL) return FR_ERR_UNSUPPORTED;

    fr::ActArgs a{};
    a.gu = gate_up;
    a.out = out_fp8;
    a.scales = out_scales;
    a.T = T;
    a.I = (int)I;
    return launch_status(fr::launch_act(a, dtype, act, false, (hipStream_t)stream));
}

FR_EXPORT int fr_resid_rmsnorm_mxfp4(const void* x, const void* residual,
                                     void* residual_out, const void* weight,
                                     int wmode, float eps, uint8_t* out_fp4,
                                     uint8_t* out_scales, int64_t T, int64_t H,
                                     int dtype, void* stream) {
    if (dtype != FR_F16 && dtype != FR_BF16) return FR_ERR_DTYPE;
    if (T < 0 || H <= 0 || H % 32 != 0) return FR_ERR_SHAPE;
    if (H > 32768) return FR_ERR_UNSUPPORTED;
    if (T > 0x7fffffffLL) return FR_ERR_UNSUPPORTED;          // grid limit
    if (wmode != FR_W_NONE && wmode != FR_W_MUL && wmode != FR_W_ONE_PLUS) return FR_ERR_MODE;
    if (!finite_nonneg(eps)) return FR_ERR_MODE;
    if (!x || !residual || !residual_out || !out_fp4 || !out_scales) return FR_ERR_NULL;
    if (wmode != FR_W_NONE && !weight) return FR_ERR_NULL;
    if (!aligned16(x) || !aligned16(residual) || !aligned16(residual_out) ||
        !aligned16(out_fp4))
        return FR_ERR_ALIGN;
    if (wmode != FR_W_NONE && !aligned16(weight)) return FR_ERR_ALIGN;
    if (T == 0) return FR_OK;

    fr::NormArgs a{};
    a.x = x;
    a.res = residual;
    a.res_out = residual_out;
    a.w = weight;
    a.out = out_fp4;
    a.mx_scales = out_scales;
    a.T = T;
    a.H = (int)H;
    a.wmode = wmode;
    a.eps = eps;
    a.static_scale = 1.0f;
    return launch_status(fr::launch_norm(a, dtype, fr::NORM_MXFP4, (hipStream_t)stream));
}

FR_EXPORT int fr_resid_rmsnorm_nvfp4(const void* x, const void* residual,
                                     void* residual_out, const void* weight,
                                     int wmode, float eps, float global_scale,
                                     uint8_t* out_fp4, uint8_t* out_scales, int64_t T,
                                     int64_t H, int dtype, void* stream) {
    if (dtype != FR_F16 && dtype != FR_BF16) return FR_ERR_DTYPE;
    if (T < 0 || H <= 0 || H % 16 != 0) return FR_ERR_SHAPE;
    if (H > 32768) return FR_ERR_UNSUPPORTED;
    if (T > 0x7fffffffLL) return FR_ERR_UNSUPPORTED;          // grid limit
    if (wmode != FR_W_NONE && wmode != FR_W_MUL && wmode != FR_W_ONE_PLUS) return FR_ERR_MODE;
    if (!finite_nonneg(eps)) return FR_ERR_MODE;
    if (!(isfinite(global_scale) && global_scale > 0.0f)) return FR_ERR_MODE;
    if (!x || !residual || !residual_out || !out_fp4 || !out_scales) return FR_ERR_NULL;
    if (wmode != FR_W_NONE && !weight) return FR_ERR_NULL;
    if (!aligned16(x) || !aligned16(residual) || !aligned16(residual_out) ||
        !aligned16(out_fp4))
        return FR_ERR_ALIGN;
    if (wmode != FR_W_NONE && !aligned16(weight)) return FR_ERR_ALIGN;
    if (T == 0) return FR_OK;

    fr::NormArgs a{};
    a.x = x;
    a.res = residual;
    a.res_out = residual_out;
    a.w = weight;
    a.out = out_fp4;
    a.mx_scales = out_scales;
    a.T = T;
    a.H = (int)H;
    a.wmode = wmode;
    a.eps = eps;
    a.static_scale = 1.0f;
    a.gscale = global_scale;
    return launch_status(fr::launch_norm(a, dtype, fr::NORM_NVFP4, (hipStream_t)stream));
}

FR_EXPORT int fr_resid_layernorm_fp8(const void* x, const void* residual,
                                     void* residual_out, const void* weight,
                                     const void* bias, float eps, uint8_t* out_fp8,
                                     int qmode, float static_scale, float* out_scales,
                                     int64_t T, int64_t H, int dtype, void* stream) {
    int st = check_norm_common(eps, out_fp8, qmode, static_scale, out_scales, T, H, dtype);
    if (st != FR_OK) return st;
    if (!x || !residual || !residual_out || !weight) return FR_ERR_NULL;
    if (!aligned16(x) || !aligned16(residual) || !aligned16(residual_out) || !aligned16(weight))
        return FR_ERR_ALIGN;
    if (bias && !aligned16(bias)) return FR_ERR_ALIGN;
    if (T == 0) return FR_OK;
    fr::NormArgs a{};
    a.x = x;
    a.res = residual;
    a.res_out = residual_out;
    a.w = weight;
    a.b = bias;
    a.out = out_fp8;
    a.scales = out_scales;
    a.T = T;
    a.H = (int)H;
    a.qmode = qmode;
    a.eps = eps;
    a.static_scale = static_scale;
    return launch_status(fr::launch_norm(a, dtype, fr::NORM_LAYER_FP8, (hipStream_t)stream));
}

FR_EXPORT int fr_resid_layernorm_mxfp4(const void* x, const void* residual,
                                       void* residual_out, const void* weight,
                                       const void* bias, float eps, uint8_t* out_fp4,
                                       uint8_t* out_scales, int64_t T, int64_t H,
                                       int dtype, void* stream) {
    if (dtype != FR_F16 && dtype != FR_BF16) return FR_ERR_DTYPE;
    if (T < 0 || H <= 0 || H % 32 != 0) return FR_ERR_SHAPE;
    if (H > 32768 || T > 0x7fffffffLL) return FR_ERR_UNSUPPORTED;
    if (!finite_nonneg(eps)) return FR_ERR_MODE;
    if (!x || !residual || !residual_out || !weight || !out_fp4 || !out_scales) return FR_ERR_NULL;
    if (!aligned16(x) || !aligned16(residual) || !aligned16(residual_out) ||
        !aligned16(weight) || !aligned16(out_fp4))
        return FR_ERR_ALIGN;
    if (bias && !aligned16(bias)) return FR_ERR_ALIGN;
    if (T == 0) return FR_OK;
    fr::NormArgs a{};
    a.x = x;
    a.res = residual;
    a.res_out = residual_out;
    a.w = weight;
    a.b = bias;
    a.out = out_fp4;
    a.mx_scales = out_scales;
    a.T = T;
    a.H = (int)H;
    a.eps = eps;
    a.static_scale = 1.0f;
    return launch_status(fr::launch_norm(a, dtype, fr::NORM_LAYER_MXFP4, (hipStream_t)stream));
}

FR_EXPORT int fr_resid_layernorm_nvfp4(const void* x, const void* residual,
                                       void* residual_out, const void* weight,
                                       const void* bias, float eps, float global_scale,
                                       uint8_t* out_fp4, uint8_t* out_scales, int64_t T,
                                       int64_t H, int dtype, void* stream) {
    if (dtype != FR_F16 && dtype != FR_BF16) return FR_ERR_DTYPE;
    if (T < 0 || H <= 0 || H % 16 != 0) return FR_ERR_SHAPE;
    if (H > 32768 || T > 0x7fffffffLL) return FR_ERR_UNSUPPORTED;
    if (!finite_nonneg(eps)) return FR_ERR_MODE;
    if (!(isfinite(global_scale) && global_scale > 0.0f)) return FR_ERR_MODE;
    if (!x || !residual || !residual_out || !weight || !out_fp4 || !out_scales) return FR_ERR_NULL;
    if (!aligned16(x) || !aligned16(residual) || !aligned16(residual_out) ||
        !aligned16(weight) || !aligned16(out_fp4))
        return FR_ERR_ALIGN;
    if (bias && !aligned16(bias)) return FR_ERR_ALIGN;
    if (T == 0) return FR_OK;
    fr::NormArgs a{};
    a.x = x;
    a.res = residual;
    a.res_out = residual_out;
    a.w = weight;
    a.b = bias;
    a.out = out_fp4;
    a.mx_scales = out_scales;
    a.T = T;
    a.H = (int)H;
    a.eps = eps;
    a.static_scale = 1.0f;
    a.gscale = global_scale;
    return launch_status(fr::launch_norm(a, dtype, fr::NORM_LAYER_NVFP4, (hipStream_t)stream));
}

FR_EXPORT int fr_gated_act_mxfp4(const void* gate_up, int act, uint8_t* out_fp4,
                                 uint8_t* out_scales, int64_t T, int64_t I,
                                 int dtype, void* stream) {
    if (dtype != FR_F16 && dtype != FR_BF16) return FR_ERR_DTYPE;
    if (T < 0 || I <= 0 || I % 128 != 0) return FR_ERR_SHAPE;
    if (I > (1 << 24)) return FR_ERR_UNSUPPORTED;
    if (act != FR_ACT_SWIGLU && act != FR_ACT_GEGLU_TANH && act != FR_ACT_SQRELU)
        return FR_ERR_MODE;
    if (!gate_up || !out_fp4 || !out_scales) return FR_ERR_NULL;
    // the kernel writes the E8M0 codes of 4 blocks as one 4-byte store
    if (!aligned16(gate_up) || !aligned16(out_fp4) || !aligned4(out_scales)) return FR_ERR_ALIGN;
    if (T == 0) return FR_OK;
    if (T * ((I + 1023) / 1024) / 4 + 1 > 0x7fffffffLL) return FR_ERR_UNSUPPORTED;

    fr::ActArgs a{};
    a.gu = gate_up;
    a.out = out_fp4;
    a.mx_scales = out_scales;
    a.T = T;
    a.I = (int)I;
    return launch_status(fr::launch_act(a, dtype, act, true, (hipStream_t)stream));
}

FR_EXPORT int fr_gemm_gated_act_fp8(const uint8_t* a, const float* a_scales,
                                    const uint8_t* w_packed, const float* w_scales,
                                    int act, uint8_t* out_fp8, float* out_scales,
                                    int64_t M, int64_t K, int64_t I, void* stream) {
    if (M < 0 || K <= 0 || K % 128 != 0 || I <= 0 || I % 128 != 0) return FR_ERR_SHAPE;
    if (K > 16384 || I > (1 << 20) || M > (1LL << 26)) return FR_ERR_UNSUPPORTED;
    if (act != FR_ACT_SWIGLU && act != FR_ACT_GEGLU_TANH && act != FR_ACT_SQRELU)
        return FR_ERR_MODE;
    if (!a || !a_scales || !w_packed || !w_scales || !out_fp8 || !out_scales) return FR_ERR_NULL;
    if (!aligned16(a) || !aligned16(w_packed) || !aligned16(out_fp8)) return FR_ERR_ALIGN;
    if (!aligned4(a_scales) || !aligned4(w_scales) || !aligned4(out_scales)) return FR_ERR_ALIGN;
    if (M == 0) return FR_OK;
    if (((M + 31) / 32) * (I / 128) > 0x7ffffff0LL) return FR_ERR_UNSUPPORTED;   // grid
    fr::GemmActArgs g{};
    g.A = a;
    g.a_scales = a_scales;
    g.B = w_packed;
    g.b_scales = w_scales;
    g.out = out_fp8;
    g.out_scales = out_scales;
    g.M = (int)M;
    g.K = (int)K;
    g.I = (int)I;
    return launch_status(fr::launch_gemm_act(g, act, (hipStream_t)stream));
}

FR_EXPORT int fr_gemm_pack_weights(const uint8_t* w, uint8_t* w_packed, int64_t N,
                                   int64_t K, void* stream) {
    if (N < 0 || N % 32 != 0 || K <= 0 || K % 128 != 0) return FR_ERR_SHAPE;
    if (K > 16384 || N > (1LL << 22)) return FR_ERR_UNSUPPORTED;
    if (!w || !w_packed) return FR_ERR_NULL;
    if (!aligned16(w) || !aligned16(w_packed)) return FR_ERR_ALIGN;
    if (N == 0) return FR_OK;
    fr::PackArgs p{};
    p.w = w;
    p.wp = w_packed;
    p.N = N;
    p.K = K;
    return launch_status(fr::launch_pack_w(p, (hipStream_t)stream));
}

FR_EXPORT int fr_decode_chain_persistent(
    const void* x, const void* gate, const void* ada_scale, const void* ada_shift,
    void* residual, uint8_t* out_fp8, float eps, float static_scale,
    const void* qkv, const int32_t* positions, float rope_theta, int rope_style,
    void* q_out, void* k_cache, void* v_cache, const int32_t* page_table,
    int32_t page_table_len, int32_t page_size, int32_t num_pages,
    int32_t* err_flag, int32_t layers, int32_t steps, int64_t T, int64_t H,
    int32_t Hq, int32_t Hkv, int32_t D, int dtype, void* stream) {
    if (dtype != FR_F16 && dtype != FR_BF16) return FR_ERR_DTYPE;
    if (layers <= 0 || steps <= 0 || T < 0 || H <= 0 || H % 16 != 0) return FR_ERR_SHAPE;
    if (Hq <= 0 || Hkv <= 0 || D <= 0 || D % 16 != 0) return FR_ERR_SHAPE;
    if (page_table_len <= 0 || page_size <= 0 || num_pages <= 0) return FR_ERR_SHAPE;
    if (T > fr::kChainMaxT || H > fr::kChainMaxH || D > 256) return FR_ERR_UNSUPPORTED;
    if ((int64_t)layers * steps > (1LL << 24)) return FR_ERR_UNSUPPORTED;
    if ((int64_t)Hq + 2 * (int64_t)Hkv > 65536) return FR_ERR_UNSUPPORTED;
    if (rope_style != FR_ROPE_HALF && rope_style != FR_ROPE_INTERLEAVED) return FR_ERR_MODE;
    if (!finite_nonneg(eps)) return FR_ERR_MODE;
    if (!(isfinite(static_scale) && static_scale > 0.0f)) return FR_ERR_MODE;
    if (!(isfinite(rope_theta) && rope_theta > 1.0f)) return FR_ERR_MODE;
    if (!x || !gate || !ada_scale || !ada_shift || !residual || !out_fp8 || !qkv ||
        !positions || !q_out || !k_cache || !v_cache || !page_table)
        return FR_ERR_NULL;
    if (!aligned16(x) || !aligned16(gate) || !aligned16(ada_scale) || !aligned16(ada_shift) ||
        !aligned16(residual) || !aligned16(out_fp8) || !aligned16(qkv) || !aligned16(q_out) ||
        !aligned16(k_cache) || !aligned16(v_cache))
        return FR_ERR_ALIGN;
    if (!aligned4(positions) || !aligned4(page_table) || (err_flag && !aligned4(err_flag)))
        return FR_ERR_ALIGN;
    if (T == 0) return FR_OK;
    fr::ChainArgs a{};
    a.x = x;
    a.gate = gate;
    a.ada_scale = ada_scale;
    a.ada_shift = ada_shift;
    a.res = residual;
    a.out = out_fp8;
    a.qkv = qkv;
    a.pos = positions;
    a.table = page_table;
    a.q_out = q_out;
    a.kc = k_cache;
    a.vc = v_cache;
    a.err = err_flag;
    a.layers = layers;
    a.steps = steps;
    a.T = (int)T;
    a.H = (int)H;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.table_len = page_table_len;
    a.page_size = page_size;
    a.num_pages = num_pages;
    a.style = rope_style;
    a.eps = eps;
    a.static_scale = static_scale;
    a.theta = rope_theta;
    return launch_status(fr::launch_chain(a, dtype, (hipStream_t)stream));
}

FR_EXPORT int fr_qk_norm_rope(const void* qkv, int norm_kind, int norm_scope,
                              const void* q_norm_w, const void* q_norm_b,
                              const void* k_norm_w, const void* k_norm_b, float eps,
                              const int32_t* positions, int rope_dims,
                              int32_t sec_t, int32_t sec_h, int32_t sec_w,
                              float rope_theta, int rope_style, float q_scale,
                              void* q_out, void* k_out, void* v_out, int64_t T,
                              int32_t Hq, int32_t Hkv, int32_t D, int dtype,
                              void* stream) {
    if (dtype != FR_F16 && dtype != FR_BF16) return FR_ERR_DTYPE;
    if (T < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || D % 16 != 0) return FR_ERR_SHAPE;
    if (D > 256 || T > 0x7fffffffLL) return FR_ERR_UNSUPPORTED;
    int lp = 1;
    while (lp < D / 16) lp *= 2;
    if (((int64_t)Hq + 2 * (int64_t)Hkv) * lp > 1024) return FR_ERR_UNSUPPORTED;
    if (norm_kind != FR_NORM_NONE && norm_kind != FR_NORM_RMS && norm_kind != FR_NORM_LAYER)
        return FR_ERR_MODE;
    if (norm_scope != FR_SCOPE_HEAD && norm_scope != FR_SCOPE_FULL) return FR_ERR_MODE;
    if (rope_dims != 1 && rope_dims != 3) return FR_ERR_MODE;
    if (rope_dims == 3 && (sec_t < 1 || sec_h < 1 || sec_w < 1 || sec_t + sec_h + sec_w != D / 2))
        return FR_ERR_SHAPE;
    if (rope_style != FR_ROPE_HALF && rope_style != FR_ROPE_INTERLEAVED) return FR_ERR_MODE;
    if (!finite_nonneg(eps)) return FR_ERR_MODE;
    if (!(isfinite(rope_theta) && rope_theta > 1.0f)) return FR_ERR_MODE;
    if (!(isfinite(q_scale) && q_scale > 0.0f)) return FR_ERR_MODE;
    if (!qkv || !positions || !q_out || !k_out || !v_out) return FR_ERR_NULL;
    if (!aligned16(qkv) || !aligned16(q_out) || !aligned16(k_out) || !aligned16(v_out))
        return FR_ERR_ALIGN;
    const void* ws[4] = {q_norm_w, q_norm_b, k_norm_w, k_norm_b};
    for (const void* w : ws)
        if (w && !aligned16(w)) return FR_ERR_ALIGN;
    if (!aligned4(positions)) return FR_ERR_ALIGN;
    if (T == 0) return FR_OK;
    fr::QkNormArgs a{};
    a.qkv = qkv;
    a.qw = q_norm_w;
    a.qb = q_norm_b;
    a.kw = k_norm_w;
    a.kb = k_norm_b;
    a.pos = positions;
    a.q_out = q_out;
    a.k_out = k_out;
    a.v_out = v_out;
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.norm_kind = norm_kind;
    a.full = norm_scope == FR_SCOPE_FULL;
    a.rope3 = rope_dims == 3;
    a.sec[0] = sec_t;
    a.sec[1] = sec_h;
    a.sec[2] = sec_w;
    a.style = rope_style;
    a.eps = eps;
    a.theta = rope_theta;
    a.q_scale = q_scale;
    return launch_status(fr::launch_qknr(a, dtype, (hipStream_t)stream));
}

FR_EXPORT const char* fr_status_string(int status) {
    switch (status) {
    case FR_OK: return "FR_OK";
    case FR_ERR_NULL: return "FR_ERR_NULL: a required pointer is NULL";
    case FR_ERR_SHAPE: return "FR_ERR_SHAPE: invalid size";
    case FR_ERR_DTYPE: return "FR_ERR_DTYPE: dtype must be FR_F16 or FR_BF16";
    case FR_ERR_ALIGN: return "FR_ERR_ALIGN: pointer misaligned";
    case FR_ERR_MODE: return "FR_ERR_MODE: invalid mode or scalar argument";
    case FR_ERR_UNSUPPORTED: return "FR_ERR_UNSUPPORTED: size beyond the kernel's range";
    case FR_ERR_LAUNCH: return "FR_ERR_LAUNCH: kernel launch failed";
    default: return "unknown fr_status";
    }
}

FR_EXPORT int fr_abi_version(void) { return FR_ABI_VERSION; }
