/*
 * oracle.h -- plain, slow CPU oracle for the fused layer-boundary ops.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header, table or constant with
 * the HIP path.
 *
 * Every function works on host memory.  Floating-point work is done in
 * IEEE double; a value is rounded only when the op writes it to memory
 * (fp16 / bf16 round-to-nearest-even, e4m3 per or_e4m3_encode, fp32 scales
 * round-to-nearest-even).  A value that the op writes and also consumes is
 * consumed in its stored, rounded form.
 *
 * Sources (web pages; cited by title and section):
 *   [FR]  "FlashRT cross-layer fusion" article (xdnf.cn): section 二 (the
 *         per-layer fused-kernel table, 2.1, 2.2) and section 三 (adaptive
 *         RMSNorm kernel, weight pre-fold).
 *   [SM89] "sm89 prefill FFN megakernel" issue: Phase 2 (gated activation +
 *         per-token block-128 FP8) and its correctness notes.
 *   [FP]  "Falcon-Perception inference engine" article: the third technique
 *         (fused squared-ReLU gate on interleaved gate/up).
 */
#ifndef MB_ORACLE_H
#define MB_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage types of 16-bit tensors */
enum { OR_F16 = 0, OR_BF16 = 1 };
/* RMSNorm weight handling: none ("_noweight"), y*w, y*(1+w) */
enum { OR_W_NONE = 0, OR_W_MUL = 1, OR_W_ONE_PLUS = 2 };
/* FP8 quantisation: static multiplier, or per-token dynamic scale */
enum { OR_Q_STATIC = 0, OR_Q_TOKEN = 1 };
/* gated activations */
enum { OR_ACT_SWIGLU = 0, OR_ACT_GEGLU_TANH = 1, OR_ACT_SQRELU = 2 };
/* RoPE pairing */
enum { OR_ROPE_HALF = 0, OR_ROPE_INTERLEAVED = 1 };
enum { OR_NORM_NONE = 0, OR_NORM_RMS = 1, OR_NORM_LAYER = 2 };
enum { OR_SCOPE_HEAD = 0, OR_SCOPE_FULL = 1 };

/* ---- number formats ---- */
double   or_f16_decode(uint16_t bits);
double   or_bf16_decode(uint16_t bits);
uint16_t or_f16_encode(double v);           /* RNE, overflow -> inf */
uint16_t or_bf16_encode(double v);          /* RNE, overflow -> inf */
double   or_e4m3_decode(uint8_t code);
uint8_t  or_e4m3_encode(double v);          /* clamp to +-448, RNE, NaN -> 0x7F */
float    or_f32_round(double v);            /* RNE to binary32 */
void     or_e4m3_encode_n(const double* v, int64_t n, uint8_t* out);
void     or_f16_encode_n(const double* v, int64_t n, uint16_t* out);
void     or_bf16_encode_n(const double* v, int64_t n, uint16_t* out);

/* ---- building blocks in double ---- */
double or_rms_rstd(const double* v, int64_t n, double eps);
void   or_rmsnorm(const double* v, const double* w, int wmode, int64_t n,
                  double eps, double* y);
void   or_adarms(const double* h, const double* scale, const double* shift,
                 int64_t n, double eps, double* y);
void   or_rope(double* v, int64_t D, int64_t pos, double theta, int style);
void   or_layernorm(const double* v, const double* w, const double* b,
                    int64_t n, double eps, double* y);   /* w, b may be NULL */
void   or_rope3d(double* v, int64_t D, const int32_t* pos3, const int32_t* sec,
                 double theta, int style);
double or_act(double g, int act);
void   or_quant_static(const double* y, int64_t n, double mult, uint8_t* q);
float  or_quant_dynamic(const double* y, int64_t n, uint8_t* q);
double  or_e2m1_decode(uint8_t code);        /* 4-bit code, sign in bit 3 */
uint8_t or_e2m1_encode(double v);            /* RNE, |v| >= 6 -> 6, sign kept */
int     or_mx_scale_code(double amax);       /* E8M0 code of the MX block scale */
void    or_quant_mxfp4(const double* y, int64_t n, uint8_t* packed,
                       uint8_t* scales);     /* n % 32 == 0 */
void    or_quant_nvfp4(const double* y, int64_t n, double global_scale,
                       uint8_t* packed, uint8_t* scales);  /* n % 16 == 0 */
int64_t or_kv_slot(int64_t pos, const int32_t* page_table, int32_t table_len,
                   int32_t page_size, int32_t num_pages);

/* ---- the fused ops (same argument order as the device library) ---- */
int oracle_resid_rmsnorm_fp8(const uint16_t* x, const uint16_t* residual,
                             uint16_t* residual_out, const uint16_t* weight,
                             int wmode, float eps, uint8_t* out_fp8, int qmode,
                             float static_scale, float* out_scales,
                             int64_t T, int64_t H, int dtype);

int oracle_adarms_gate_res_fp8(const uint16_t* x, const uint16_t* gate,
                               const uint16_t* residual, uint16_t* residual_out,
                               const uint16_t* ada_scale, const uint16_t* ada_shift,
                               float eps, uint8_t* out_fp8, int qmode,
                               float static_scale, float* out_scales,
                               int64_t T, int64_t H, int dtype);

int oracle_qkv_normrope_kvwrite(const uint16_t* qkv, const uint16_t* q_norm_w,
                                const uint16_t* k_norm_w, float eps,
                                const int32_t* positions, float rope_theta,
                                int rope_style, float q_scale, uint16_t* q_out,
                                uint16_t* k_cache, uint16_t* v_cache,
                                const int32_t* page_table, int32_t page_table_len,
                                int32_t page_size, int32_t num_pages,
                                int32_t* err_flag, int64_t T, int32_t Hq,
                                int32_t Hkv, int32_t D, int dtype);

int oracle_gated_act_fp8(const uint16_t* gate_up, int act, uint8_t* out_fp8,
                         float* out_scales, int64_t T, int64_t I, int dtype);
int oracle_resid_rmsnorm_mxfp4(const uint16_t* x, const uint16_t* residual,
                               uint16_t* residual_out, const uint16_t* weight,
                               int wmode, float eps, uint8_t* out_fp4,
                               uint8_t* out_scales, int64_t T, int64_t H,
                               int dtype);
int oracle_resid_rmsnorm_nvfp4(const uint16_t* x, const uint16_t* residual,
                               uint16_t* residual_out, const uint16_t* weight,
                               int wmode, float eps, float global_scale,
                               uint8_t* out_fp4, uint8_t* out_scales, int64_t T,
                               int64_t H, int dtype);
int oracle_resid_layernorm(const uint16_t* x, const uint16_t* residual,
                           uint16_t* residual_out, const uint16_t* weight,
                           const uint16_t* bias, float eps, int out_kind,
                           uint8_t* out_codes, int qmode, float static_scale,
                           float* out_scales_f32, uint8_t* out_scales_e8m0,
                           int64_t T, int64_t H, int dtype);
int oracle_resid_layernorm_nvfp4(const uint16_t* x, const uint16_t* residual,
                                 uint16_t* residual_out, const uint16_t* weight,
                                 const uint16_t* bias, float eps, float global_scale,
                                 uint8_t* out_fp4, uint8_t* out_scales, int64_t T,
                                 int64_t H, int dtype);
int oracle_gated_act_mxfp4(const uint16_t* gate_up, int act, uint8_t* out_fp4,
                           uint8_t* out_scales, int64_t T, int64_t I, int dtype);
int oracle_qk_norm_rope(const uint16_t* qkv, int norm_kind, int norm_scope,
                        const uint16_t* q_norm_w, const uint16_t* q_norm_b,
                        const uint16_t* k_norm_w, const uint16_t* k_norm_b,
                        float eps, const int32_t* positions, int rope_dims,
                        const int32_t* sections, float rope_theta, int rope_style,
                        float q_scale, uint16_t* q_out, uint16_t* k_out,
                        uint16_t* v_out, int64_t T, int32_t Hq, int32_t Hkv,
                        int32_t D, int dtype);
int oracle_gated_act_fp8_f64(const double* gate_up, int act, uint8_t* out_fp8,
                             float* out_scales, int64_t T, int64_t I);

#ifdef __cplusplus
}
#endif
#endif
