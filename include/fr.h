/*
 * fr.h -- C ABI of the fused, memory-bound layer-boundary kernels for
 * small-batch transformer inference on MI355X (gfx950).
 *
 * Library: memory_bound_amd/libfrhip.so (HIP, gfx950 only).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees, copies or synchronises; it keeps no state.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *  - Arguments are validated on the host before any HIP call.  On error the
 *    call returns a nonzero fr_status and launches nothing.
 *  - On success each call enqueues exactly ONE kernel on `stream`, so it
 *    captures into a hipGraph as one node.  T == 0 returns FR_OK and
 *    launches nothing.
 *  - A launch failure is returned as FR_ERR_LAUNCH (no synchronisation, so
 *    faults inside the kernel surface at the caller's next sync).
 *  - Tensors are contiguous and row-major; every pointer must be 16-byte
 *    aligned (4-byte for the int32 arrays).
 *  - 16-bit tensors are float16 or bfloat16 bit patterns (`dtype`); FP8
 *    outputs are OCP E4M3 ("e4m3fn") codes: 1 sign, 4 exponent bits (bias
 *    7), 3 mantissa bits, subnormals, largest finite value 448 (0x7E/0xFE),
 *    no infinities.  A torch float8_e4m3fn tensor viewed as uint8 matches.
 *    Values are clamped to +-448 before rounding (saturating), rounding is
 *    to nearest, ties to even.
 *  - Arithmetic is fp32, except where an entry point says otherwise: the
 *    row sums of the residual norms (RMSNorm sum of squares; LayerNorm mean
 *    and variance) are accumulated in fp64, while the per-head Q/K norms of
 *    the QKV ops sum their D values in fp32.  A value that an op stores and
 *    also consumes (the new residual) is consumed in its stored, rounded
 *    form; every other intermediate stays in fp32 until its single store.
 *  - Results are deterministic: no atomics in value paths; repeated calls
 *    on the same inputs give bit-identical outputs.
 *
 * The operations are defined on these web pages (cited by title/section):
 *   [FR]   "FlashRT cross-layer fusion" article: section 二 (per-layer
 *          fused-kernel table; 2.1 naming "_fp8", "_noweight"; 2.2 QKV
 *          post-processing), section 三 (gate/residual/AdaRMSNorm/FP8 kernel;
 *          (1+weight) pre-fold), section 六 ("_merged", "_static").
 *   [SM89] "sm89 prefill FFN megakernel" issue: Phase 2 (gated activation +
 *          per-token block-128 FP8 with no intermediate bf16 rounding) and
 *          the correctness notes (every scale row must be written).
 *   [FP]   "Falcon-Perception inference engine" article: third technique
 *          (gated activation read from interleaved [g0,u0,g1,u1,...]) and
 *          the paged KV cache behind its CUDA-graph decode.
 */
#ifndef FR_H
#define FR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FR_ABI_VERSION 3   /* 2: fr_resid_rmsnorm_nvfp4; 3: fr_resid_layernorm_nvfp4 */

typedef enum {
    FR_OK = 0,
    FR_ERR_NULL = 1,         /* a required pointer is NULL */
    FR_ERR_SHAPE = 2,        /* negative/zero/non-multiple size */
    FR_ERR_DTYPE = 3,        /* dtype not FR_F16 / FR_BF16 */
    FR_ERR_ALIGN = 4,        /* pointer not 16-byte (int32 arrays: 4-byte) aligned */
    FR_ERR_MODE = 5,         /* unknown enum value, or bad scalar (eps, scale, theta) */
    FR_ERR_UNSUPPORTED = 6,  /* width above what one kernel row handles */
    FR_ERR_LAUNCH = 7        /* the HIP launch returned an error */
} fr_status;

typedef enum { FR_F16 = 0, FR_BF16 = 1 } fr_dtype;

/* RMSNorm weight: none ("_noweight": weight pre-folded into the next GEMM,
 * [FR 2.1, 三]), y*w, or y*(1+w). */
typedef enum { FR_W_NONE = 0, FR_W_MUL = 1, FR_W_ONE_PLUS = 2 } fr_wmode;

/* FP8 quantisation: static multiplier ("_static", [FR 六]) or per-token
 * dynamic dequant scale. */
typedef enum { FR_Q_STATIC = 0, FR_Q_TOKEN = 1 } fr_qmode;

/* Gate activation: SiLU (SwiGLU), GELU tanh approximation (GeGLU), ReLU^2. */
typedef enum { FR_ACT_SWIGLU = 0, FR_ACT_GEGLU_TANH = 1, FR_ACT_SQRELU = 2 } fr_act;

/* RoPE pairing: element i with i+D/2 ("rotate_half", [FR 2.2]), or
 * element 2i with 2i+1. */
typedef enum { FR_ROPE_HALF = 0, FR_ROPE_INTERLEAVED = 1 } fr_rope;

/* Q/K norm of fr_qk_norm_rope: kind and scope ([FR 2.2]). */
typedef enum { FR_NORM_NONE = 0, FR_NORM_RMS = 1, FR_NORM_LAYER = 2 } fr_norm_kind;
typedef enum { FR_SCOPE_HEAD = 0, FR_SCOPE_FULL = 1 } fr_norm_scope;

/*
 * (a) Residual add + RMSNorm + FP8 quantisation  [FR 二 table step 1, 2.1]
 *
 *   residual_out[t,j] = round_dtype(x[t,j] + residual[t,j])
 *   rstd_t  = 1 / sqrt(mean_j(residual_out[t,j]^2) + eps)
 *   y[t,j]  = residual_out[t,j] * rstd_t * W_j,  W_j = 1 | w_j | 1 + w_j
 *   FR_Q_STATIC: out_fp8[t,j] = E4M3(y[t,j] * static_scale)
 *   FR_Q_TOKEN:  out_scales[t] = max(max_j |y[t,j]|, 1e-10) / 448 (fp32),
 *                out_fp8[t,j] = E4M3(y[t,j] / out_scales[t])
 *
 *   x, residual, residual_out: [T,H] dtype.  residual_out may alias
 *     residual (in place); no other overlap is allowed.
 *   weight: [H] dtype; ignored (may be NULL) for FR_W_NONE.
 *   out_fp8: [T,H] uint8.  out_scales: [T] fp32 dequant scales, required
 *     for FR_Q_TOKEN, ignored for FR_Q_STATIC.
 *   static_scale: the quantisation MULTIPLIER (e.g. 448/8 = 56); the
 *     matching dequant scale is 1/static_scale.  Must be finite and > 0.
 *   eps >= 0 and finite.  H % 16 == 0, 16 <= H <= 32768.
 */
int fr_resid_rmsnorm_fp8(const void* x, const void* residual, void* residual_out,
                         const void* weight, int wmode, float eps,
                         uint8_t* out_fp8, int qmode, float static_scale,
                         float* out_scales, int64_t T, int64_t H, int dtype,
                         void* stream);

/*
 * (a') Gate multiply + residual + adaptive RMSNorm + FP8  [FR 三]
 *
 *   residual_out[t,j] = round_dtype(residual[t,j] + gate[t,j] * x[t,j]),
 *     the exact value rounded once
 *   y[t,j] = residual_out[t,j] * rstd_t * (1 + ada_scale[t,j]) + ada_shift[t,j]
 *   quantised as in (a).
 *
 *   x, gate, residual, residual_out, ada_scale, ada_shift: [T,H] dtype
 *   (one modulation vector per token).  residual_out may alias residual.
 *   Other arguments as in (a).
 */
int fr_adarms_gate_res_fp8(const void* x, const void* gate, const void* residual,
                           void* residual_out, const void* ada_scale,
                           const void* ada_shift, float eps, uint8_t* out_fp8,
                           int qmode, float static_scale, float* out_scales,
                           int64_t T, int64_t H, int dtype, void* stream);

/*
 * (b) Packed-QKV split + per-head Q/K RMSNorm + RoPE + paged KV write
 *     [FR 二 table step 3, 2.2; FP paged cache; HY 04 step 10 (the
 *     attention's Q preparation folded into RoPE)]
 *
 *   qkv row t = [Q heads: Hq*D | K heads: Hkv*D | V heads: Hkv*D], each head
 *     D-contiguous.
 *   For a Q or K head v (D values): if its norm weight is non-NULL,
 *     v = v * rstd(v) * w with rstd over the D values and one weight [D]
 *     shared by all heads; then RoPE at p = positions[t]: pair i
 *     (0 <= i < D/2) turns by p * rope_theta^(-2i/D); a Q head is then
 *     multiplied by q_scale (the attention's pre-scale, e.g. 1/sqrt(D);
 *     1 = none); then one rounding.
 *   q_out[t,h,:] = Q head h;   k_cache[slot,g,:] = K head g;
 *   v_cache[slot,g,:] = V head g copied bit for bit (V is never normed or
 *   rotated).
 *   slot = page_table[p / page_size] * page_size + p % page_size.
 *   If p < 0, p / page_size >= page_table_len, or the page id is outside
 *   [0, num_pages), the token's K/V writes are skipped and, when err_flag
 *   is non-NULL, bit 0 of *err_flag is set (atomic OR); q_out is still
 *   written.  Cache slots no token maps to are never touched.  Two tokens
 *   of one call that map to the same slot leave one of the two writes
 *   (which one is unspecified).
 *
 *   qkv: [T,(Hq+2Hkv)*D] dtype.  q_norm_w, k_norm_w: [D] dtype or NULL.
 *   positions: [T] int32 (device).  page_table: [page_table_len] int32.
 *   q_out: [T,Hq,D].  k_cache, v_cache: [num_pages, page_size, Hkv, D].
 *   positions and page_table are read on the device, so a captured graph
 *   can be replayed with new positions.
 *   D % 16 == 0, 16 <= D <= 256; Hq, Hkv >= 1; rope_theta > 1 and finite;
 *   q_scale > 0 and finite.
 */
int fr_qkv_normrope_kvwrite(const void* qkv, const void* q_norm_w,
                            const void* k_norm_w, float eps,
                            const int32_t* positions, float rope_theta,
                            int rope_style, float q_scale, void* q_out, void* k_cache,
                            void* v_cache, const int32_t* page_table,
                            int32_t page_table_len, int32_t page_size,
                            int32_t num_pages, int32_t* err_flag, int64_t T,
                            int32_t Hq, int32_t Hkv, int32_t D, int dtype,
                            void* stream);

/*
 * (c) Gated activation on interleaved gate/up + per-token block-128 FP8
 *     [SM89 Phase 2; FP third technique; FR 二 table steps 8-10]
 *
 *   gate_up row t = [g0, u0, g1, u1, ...] (2I values).
 *   h[t,j] = act(g_j) * u_j in fp32, not rounded in between;
 *     SiLU(g) = g / (1 + e^-g); GELU_tanh(g) = 0.5 g (1 + tanh(sqrt(2/pi)
 *     (g + 0.044715 g^3))); ReLU^2(g) = max(g, 0)^2.
 *   For each block b of 128 consecutive outputs of a row:
 *     out_scales[t,b] = max(max |h|, 1e-10) / 448 (fp32 dequant scale),
 *     out_fp8[t,j] = E4M3(h[t,j] / out_scales[t,b]).
 *   Every scale entry is written.
 *
 *   gate_up: [T,2I] dtype.  out_fp8: [T,I] uint8.  out_scales: [T, I/128]
 *   fp32, row-major.  I % 128 == 0, I >= 128.
 */
int fr_gated_act_fp8(const void* gate_up, int act, uint8_t* out_fp8,
                     float* out_scales, int64_t T, int64_t I, int dtype,
                     void* stream);

/*
 * MX FP4 producers [HY 04 steps 5 and 9, 06 census: the residual-RMSNorm
 *     and SwiGLU FP4 producers that feed FP4 GEMMs].  Format (OCP
 *     Microscaling MXFP4): blocks of 32 consecutive values of a row share
 *     one E8M0 scale code c (scale 2^(c - 127)); each value is an E2M1 code
 *     (sign in bit 3; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte,
 *     the even-indexed value in bits 3..0.
 *   c = clamp(floor(log2 amax) - 2 + 127, 0, 254) with amax the block's
 *     largest magnitude (c = 0 for an all-zero block); element =
 *     E2M1(v / 2^(c - 127)) rounded to nearest even, magnitudes >= 6
 *     saturate to 6, the sign kept also when the value rounds to zero.
 *
 * (a-fp4) residual add + RMSNorm + MXFP4: residual_out and the normalised
 *   value y exactly as fr_resid_rmsnorm_fp8 (wmode FR_W_NONE / MUL /
 *   ONE_PLUS); y is quantised in blocks of 32 along H.  The codes and scales
 *   are those of the exact y (the kernel takes every rounding decision on
 *   the exact value).  out_fp4: [T, H/2] bytes (16-byte aligned);
 *   out_scales: [T, H/32] bytes.  H % 32 == 0, H <= 32768.  x, residual,
 *   residual_out (may equal residual), weight: as fr_resid_rmsnorm_fp8.
 */
int fr_resid_rmsnorm_mxfp4(const void* x, const void* residual,
                           void* residual_out, const void* weight, int wmode,
                           float eps, uint8_t* out_fp4, uint8_t* out_scales,
                           int64_t T, int64_t H, int dtype, void* stream);

/*
 * (a-nvfp4) residual add + RMSNorm + NVFP4 [HY 04 step 5 and 06 census:
 *   residual_add_rms_norm_to_nvfp4, the residual-RMSNorm producer of the FP4
 *   GEMM inputs].  The pages name the format only; this follows its
 *   published definition: blocks of 16 consecutive values of a row share an
 *   E4M3 scale code (encoded as the FP8 outputs above), the whole tensor a
 *   caller-given fp32 dequantisation scale g; each value is an E2M1 code as
 *   in the MX producers, and decodes as e2m1(code) * e4m3(block code) * g.
 *   block code = E4M3(amax / (6 g)), amax the block's largest magnitude
 *     (nearest, ties to even, saturating at 448), so the block maximum maps
 *     to 6; element = E2M1(y / S), S = e4m3(block code) * g (nearest even,
 *     saturating at 6, sign kept); a block whose code decodes to 0 gets zero
 *     codes with the values' signs.
 *   residual_out and y exactly as fr_resid_rmsnorm_fp8 (wmode FR_W_NONE /
 *   MUL / ONE_PLUS).  Both decisions are taken on the exact y (the block
 *   scale on a double-precision value of amax / (6 g)).
 *   global_scale: g > 0, finite (FR_ERR_MODE otherwise), e.g. a calibrated
 *   tensor amax / (6 * 448).  out_fp4: [T, H/2] bytes (16-byte aligned), two
 *   codes per byte, the even-indexed value in bits 3..0; out_scales:
 *   [T, H/16] E4M3 codes (any alignment).  H % 16 == 0, H <= 32768.  x,
 *   residual, residual_out (may equal residual), weight: as
 *   fr_resid_rmsnorm_fp8.
 */
int fr_resid_rmsnorm_nvfp4(const void* x, const void* residual,
                           void* residual_out, const void* weight, int wmode,
                           float eps, float global_scale, uint8_t* out_fp4,
                           uint8_t* out_scales, int64_t T, int64_t H, int dtype,
                           void* stream);

/*
 * (a-ln) residual add + LayerNorm + FP8, MXFP4 or NVFP4 [HY 06 census: the
 *   ViT add + LayerNorm FP4 producer (add_layer_norm_to_nvfp4); FR 二 table
 *   step 1 for the fused FP8 form]
 *
 *   residual_out = round_dtype(x + residual) (bit-exact, as op (a));
 *   y = (residual_out - mean) / sqrt(var + eps) * weight + bias, mean and
 *   biased variance over the row (fp64 sums of the stored values), y in
 *   fp32; bias may be NULL (0).
 *   _fp8: quantised as fr_resid_rmsnorm_fp8 (FR_Q_STATIC multiplier or
 *   FR_Q_TOKEN scale); out_fp8 [T,H], out_scales [T] (token mode).
 *   _mxfp4: MXFP4 as fr_resid_rmsnorm_mxfp4; out_fp4 [T,H/2], out_scales
 *   [T,H/32]; H % 32 == 0.
 *   _nvfp4: NVFP4 as fr_resid_rmsnorm_nvfp4 (blocks of 16, E4M3 block
 *   codes, caller's tensor scale global_scale > 0 and finite, FR_ERR_MODE
 *   otherwise), taken on the fp32 y (the block code on a double-precision
 *   amax / (6 g)); out_fp4 [T,H/2], out_scales [T,H/16] E4M3 codes (any
 *   alignment); H % 16 == 0.
 *   weight: [H] required; all tensors 16-byte aligned (except _nvfp4's
 *   out_scales).
 */
int fr_resid_layernorm_fp8(const void* x, const void* residual,
                           void* residual_out, const void* weight,
                           const void* bias, float eps, uint8_t* out_fp8,
                           int qmode, float static_scale, float* out_scales,
                           int64_t T, int64_t H, int dtype, void* stream);
int fr_resid_layernorm_mxfp4(const void* x, const void* residual,
                             void* residual_out, const void* weight,
                             const void* bias, float eps, uint8_t* out_fp4,
                             uint8_t* out_scales, int64_t T, int64_t H,
                             int dtype, void* stream);
int fr_resid_layernorm_nvfp4(const void* x, const void* residual,
                             void* residual_out, const void* weight,
                             const void* bias, float eps, float global_scale,
                             uint8_t* out_fp4, uint8_t* out_scales, int64_t T,
                             int64_t H, int dtype, void* stream);

/*
 * (c-fp4) gated activation + MXFP4: h = act(g) * u as fr_gated_act_fp8 (fp32
 *   activation), quantised in blocks of 32 outputs.  out_fp4: [T, I/2]
 *   bytes (16-byte aligned); out_scales: [T, I/32] bytes (4-byte aligned:
 *   the codes of 4 blocks leave as one 4-byte store).  I % 128 == 0.
 */
int fr_gated_act_mxfp4(const void* gate_up, int act, uint8_t* out_fp4,
                       uint8_t* out_scales, int64_t T, int64_t I, int dtype,
                       void* stream);

/*
 * (c') FP8 gate_up GEMM fused with the gated activation and block-128 FP8
 *      [SM89 Phase 2 (gate_up GEMM + silu*up + per-token block-128 FP8 in
 *      one launch, no [S, 2*inter] bf16 intermediate); FP third technique
 *      (gate/up weight rows interleaved so one GEMM emits [g, u] pairs)]
 *
 *   acc[m,n] = sum_k dec(a[m,k]) a_scales[m,k/128] * dec(w[n,k]) w_scales[n/128,k/128]
 *   h[m,j]   = act(acc[m,2j]) * acc[m,2j+1]     (fp32, not rounded in between)
 *   out_scales[m,b] = max(max_j |h[m,j]| over block b of 128, 1e-10) / 448,
 *   out_fp8[m,j] = E4M3(h[m,j] / out_scales[m, j/128])
 *
 *   a: [M,K] e4m3 codes, row-major; a_scales: [M, K/128] fp32 dequant scales
 *     (the per-token block-128 format the FP8 producers write).
 *   w_packed: the [2I,K] e4m3 weight (row 2j = gate row j, row 2j+1 = up
 *     row j) in the layout fr_gemm_pack_weights writes (packed once, at
 *     load time); w_scales: [2I/128, K/128] fp32 dequant scales of 128 x 128
 *     blocks of the unpacked weight.
 *   out_fp8: [M,I]; out_scales: [M, I/128].
 *   Products are exact; sums are fp32 (matrix-core accumulation within a
 *   128-wide K block, then scaled and added in fp32).
 *   K % 128 == 0 (K <= 16384), I % 128 == 0; a, w_packed, out_fp8 16-byte
 *   aligned, scale arrays 4-byte aligned.  M == 0 launches nothing.
 */
int fr_gemm_gated_act_fp8(const uint8_t* a, const float* a_scales,
                          const uint8_t* w_packed, const float* w_scales, int act,
                          uint8_t* out_fp8, float* out_scales, int64_t M,
                          int64_t K, int64_t I, void* stream);

/*
 * Weight packing for fr_gemm_gated_act_fp8 (a byte permutation, no
 * arithmetic).  w: [N,K] e4m3 codes, row-major; w_packed: N*K bytes, must
 * not overlap w.  Unit u (16 bytes at w_packed + 16u) holds, with
 *   lane = u % 64, c = (u / 64) % 4, kb = (u / 256) % (K/128),
 *   G = u / (256 * K/128), row = 32 G + lane % 32,
 *   off = 64 (c / 2) + 32 (lane / 32) + 16 (c % 2),
 * the bytes w[row, 128 kb + off .. 128 kb + off + 15]: the operand
 * fragments of one 32-row group and one 128-wide K block form 4 KB of
 * consecutive bytes, so every fragment load of the GEMM reads whole cache
 * lines.  N % 32 == 0, K % 128 == 0 (K <= 16384); both pointers 16-byte
 * aligned.  N == 0 launches nothing.
 */
int fr_gemm_pack_weights(const uint8_t* w, uint8_t* w_packed, int64_t N,
                         int64_t K, void* stream);

/*
 * The small-batch decoder-step chain in one persistent kernel
 *   [FF abstract: one long-lived kernel for the forward pass at low batch;
 *   FR 一, 三: 18 layers x 10 flow steps of gate + residual + AdaRMSNorm +
 *   FP8, with QKV post-processing per layer, at 10 tokens]
 *
 *   for s in [0, steps), l in [0, layers), n = s * layers + l:
 *     op (a'): fr_adarms_gate_res_fp8(x[l], gate[n], residual[n] ->
 *              residual[n+1], ada_scale[n], ada_shift[n], eps, out_fp8[n],
 *              FR_Q_STATIC, static_scale)
 *     op (b):  fr_qkv_normrope_kvwrite(qkv[l], no q/k norm, positions,
 *              rope_theta, rope_style, q_scale 1, q_out[l], k_cache[l],
 *              v_cache[l], page_table, ...)
 *   with exactly the arithmetic of those two entry points, in this order.
 *   One launch; no host involvement and no synchronisation between the
 *   ops (each output location is owned by one wave for the whole chain).
 *
 *   x: [layers, T, H]; gate, ada_scale, ada_shift: [N, T, H]; residual:
 *   [N+1, T, H] (slice 0 is read, slices 1..N written); out_fp8: [N, T, H]
 *   (N = layers * steps).  qkv: [layers, T, (Hq+2Hkv)*D]; q_out:
 *   [layers, T, Hq, D]; k_cache, v_cache: [layers, num_pages, page_size,
 *   Hkv, D].  positions and page_table as in fr_qkv_normrope_kvwrite; an
 *   out-of-range slot skips the token's K/V writes and sets bit 0 of
 *   *err_flag.  T <= 64, H % 16 == 0 and H <= 1024, D % 16 == 0 and
 *   D <= 256.  All tensors 16-byte aligned (positions, page_table,
 *   err_flag 4-byte).
 */
int fr_decode_chain_persistent(
    const void* x, const void* gate, const void* ada_scale, const void* ada_shift,
    void* residual, uint8_t* out_fp8, float eps, float static_scale,
    const void* qkv, const int32_t* positions, float rope_theta, int rope_style,
    void* q_out, void* k_cache, void* v_cache, const int32_t* page_table,
    int32_t page_table_len, int32_t page_size, int32_t num_pages,
    int32_t* err_flag, int32_t layers, int32_t steps, int64_t T, int64_t H,
    int32_t Hq, int32_t Hkv, int32_t D, int dtype, void* stream);

/*
 * (b-var) Packed-QKV split + Q/K norm + RoPE into separate Q, K, V outputs:
 *     the variants of op (b)'s contract [FR 2.2: Q and K normalised, then
 *     rotated, V passed through; the Chameleon prefill path uses LayerNorm
 *     per head with rotate-half RoPE; the Wan video path normalises over the
 *     full width and applies a 3D RoPE; HY 04 step 10 for q_scale]
 *
 *   norm_kind: FR_NORM_NONE, FR_NORM_RMS (v * rstd * w), FR_NORM_LAYER
 *     ((v - mean) * rstd * w + b, biased variance); rstd = 1/sqrt(. + eps).
 *   norm_scope: FR_SCOPE_HEAD (per head over D; w, b: [D] shared by all
 *     heads) or FR_SCOPE_FULL (over all Hq*D Q values, and separately all
 *     Hkv*D K values; w, b: [Hq*D] and [Hkv*D]).  NULL weight = 1, NULL
 *     bias = 0; RMSNorm ignores the bias.
 *   rope_dims 1: pair i (0 <= i < D/2) turns by positions[t] *
 *     rope_theta^(-2i/D).  rope_dims 3: positions is [T,3] (time, height,
 *     width); the pairs split into ranges of sec_t, sec_h, sec_w pairs
 *     (each >= 1, sum D/2); pair k of range a turns by positions[t,a] *
 *     rope_theta^(-k / sec_a).  rope_style: FR_ROPE_HALF pairs (i, i+D/2),
 *     FR_ROPE_INTERLEAVED (2i, 2i+1).
 *   Q is multiplied by q_scale after RoPE; one rounding per output value.
 *   qkv: [T,(Hq+2Hkv)*D]; q_out: [T,Hq,D]; k_out, v_out: [T,Hkv,D] (V copied
 *   bit for bit).  D % 16 == 0, D <= 256, (Hq+2Hkv) * p <= 1024 with p the
 *   power of two >= D/16.  Tensors 16-byte aligned, positions 4-byte.
 */
int fr_qk_norm_rope(const void* qkv, int norm_kind, int norm_scope,
                    const void* q_norm_w, const void* q_norm_b,
                    const void* k_norm_w, const void* k_norm_b, float eps,
                    const int32_t* positions, int rope_dims, int32_t sec_t,
                    int32_t sec_h, int32_t sec_w, float rope_theta,
                    int rope_style, float q_scale, void* q_out, void* k_out,
                    void* v_out, int64_t T, int32_t Hq, int32_t Hkv, int32_t D,
                    int dtype, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* fr_status_string(int status);

/* FR_ABI_VERSION of the built library. */
int fr_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FR_H */
