/*
 * oracle.c -- plain, slow CPU oracle for the fused layer-boundary ops.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Written for a reader checking it
 * against the pages by eye: one loop per definition, double precision, no
 * blocking, no fusion, no reordering beyond what each definition states.
 *
 * Parity pins: every function here is pinned by the CPU tests (closed forms,
 * invariants, brute force and library routines); none is "parity unpinned".
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* Round v to a binary format with p significand bits (hidden bit
 * included) whose smallest normal exponent is emin, ties to even.  Below
 * 2^emin the quantum stays 2^(emin-p+1) (gradual underflow).  No overflow
 * handling here; the callers decide what happens above the format's max. */
static double round_to_format(double v, int p, int emin)
{
    if (v == 0.0 || !isfinite(v))
        return v;
    int e;
    frexp(fabs(v), &e);             /* |v| = f * 2^e, f in [0.5, 1) */
    int lead = e - 1;               /* exponent of the leading bit */
    if (lead < emin)
        lead = emin;
    double quantum = ldexp(1.0, lead - (p - 1));
    /* v / quantum is exact (power-of-two scaling); nearbyint rounds to
     * nearest with ties to even under the default rounding mode. */
    return nearbyint(v / quantum) * quantum;
}

/* Bits of an already-rounded finite value r in a format with the given
 * significand bits p, exponent bias and smallest normal exponent emin. */
static uint32_t pack_bits(double r, int p, int bias, int emin, int ebits)
{
    uint32_t sign = signbit(r) ? 1u : 0u;
    double a = fabs(r);
    uint32_t E, M;
    if (a < ldexp(1.0, emin)) {                 /* subnormal or zero */
        E = 0;
        M = (uint32_t)(a / ldexp(1.0, emin - (p - 1)));
    } else {
        int e;
        frexp(a, &e);
        int lead = e - 1;
        E = (uint32_t)(lead + bias);
        M = (uint32_t)(ldexp(a, (p - 1) - lead) - ldexp(1.0, p - 1));
    }
    return (sign << (ebits + p - 1)) | (E << (p - 1)) | M;
}

double or_f16_decode(uint16_t bits)
{
    int s = bits >> 15, e = (bits >> 10) & 0x1F, m = bits & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

double or_bf16_decode(uint16_t bits)
{
    int s = bits >> 15, e = (bits >> 7) & 0xFF, m = bits & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134);
    return s ? -v : v;
}

uint16_t or_f16_encode(double v)
{
    if (isnan(v))
        return 0x7E00;
    double r = round_to_format(v, 11, -14);
    if (fabs(r) > 65504.0)
        return (uint16_t)((signbit(r) ? 0x8000 : 0) | 0x7C00);
    return (uint16_t)pack_bits(r, 11, 15, -14, 5);
}

uint16_t or_bf16_encode(double v)
{
    if (isnan(v))
        return 0x7FC0;
    double r = round_to_format(v, 8, -126);
    if (fabs(r) > ldexp(255.0, 120))            /* (2 - 2^-7) * 2^127 */
        return (uint16_t)((signbit(r) ? 0x8000 : 0) | 0x7F80);
    return (uint16_t)pack_bits(r, 8, 127, -126, 8);
}

/* OCP 8-bit E4M3 ("fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
 * subnormals m * 2^-9, no infinities, S.1111.111 is NaN, largest finite
 * value 448 (S.1111.110). */
double or_e4m3_decode(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Saturating encoder: NaN -> 0x7F, otherwise clamp to [-448, 448] and round
 * to nearest, ties to even.  The sign is kept, so a negative value that
 * rounds to zero gives 0x80. */
uint8_t or_e4m3_encode(double v)
{
    if (isnan(v))
        return 0x7F;
    if (v > 448.0)
        v = 448.0;
    if (v < -448.0)
        v = -448.0;
    double r = round_to_format(v, 4, -6);
    return (uint8_t)pack_bits(r, 4, 7, -6, 4);
}

float or_f32_round(double v)
{
    return (float)v;                 /* C conversion: round to nearest even */
}

/* Array forms of the encoders (used by the tests to sweep many values). */
void or_e4m3_encode_n(const double* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_e4m3_encode(v[i]);
}

void or_f16_encode_n(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_f16_encode(v[i]);
}

void or_bf16_encode_n(const double* v, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_bf16_encode(v[i]);
}

static double dec16(uint16_t bits, int dtype)
{
    return dtype == OR_BF16 ? or_bf16_decode(bits) : or_f16_decode(bits);
}

static uint16_t enc16(double v, int dtype)
{
    return dtype == OR_BF16 ? or_bf16_encode(v) : or_f16_encode(v);
}

/* ------------------------------------------------------------------ */
/* Building blocks                                                     */
/* ------------------------------------------------------------------ */

/* RMSNorm scale [FR section 二, step 1]: rstd = 1 / sqrt(mean(v^2) + eps),
 * eps inside the square root, mean over the n normalised elements. */
double or_rms_rstd(const double* v, int64_t n, double eps)
{
    double ss = 0.0;
    for (int64_t j = 0; j < n; ++j)
        ss += v[j] * v[j];
    return 1.0 / sqrt(ss / (double)n + eps);
}

/* RMSNorm with the three weight conventions [FR section 二 2.1 and section
 * 三]: none (the "_noweight" kernel, weight already folded into the next
 * GEMM), y*w, or y*(1+w). */
void or_rmsnorm(const double* v, const double* w, int wmode, int64_t n,
                double eps, double* y)
{
    double rstd = or_rms_rstd(v, n, eps);
    for (int64_t j = 0; j < n; ++j) {
        double W = 1.0;
        if (wmode == OR_W_MUL)
            W = w[j];
        else if (wmode == OR_W_ONE_PLUS)
            W = 1.0 + w[j];
        y[j] = v[j] * rstd * W;
    }
}

/* Adaptive RMSNorm modulation [FR section 三]: normalise, then scale by
 * (1 + scale) and add shift; no learned weight. */
void or_adarms(const double* h, const double* scale, const double* shift,
               int64_t n, double eps, double* y)
{
    double rstd = or_rms_rstd(h, n, eps);
    for (int64_t j = 0; j < n; ++j)
        y[j] = h[j] * rstd * (1.0 + scale[j]) + shift[j];
}

/* Rotary position embedding, in place on one head of D elements [FR
 * section 二 2.2].  Pair i (0 <= i < D/2) turns by pos * theta^(-2i/D).
 * ROPE_HALF pairs element i with element i + D/2; ROPE_INTERLEAVED pairs
 * element 2i with element 2i+1.  In each pair (a, b) -> (a cos - b sin,
 * b cos + a sin). */
void or_rope(double* v, int64_t D, int64_t pos, double theta, int style)
{
    int64_t half = D / 2;
    for (int64_t i = 0; i < half; ++i) {
        double inv_freq = pow(theta, -(2.0 * (double)i) / (double)D);
        double ang = (double)pos * inv_freq;
        double c = cos(ang), s = sin(ang);
        int64_t ia = style == OR_ROPE_INTERLEAVED ? 2 * i : i;
        int64_t ib = style == OR_ROPE_INTERLEAVED ? 2 * i + 1 : i + half;
        double a = v[ia], b = v[ib];
        v[ia] = a * c - b * s;
        v[ib] = b * c + a * s;
    }
}

/* LayerNorm [FR section 2.2: the Chameleon prefill path normalises Q and K
 * with LayerNorm]: y = (v - mean) / sqrt(var + eps) * w + b with the mean
 * and the (biased) variance over the n values; w = 1 and b = 0 when NULL. */
void or_layernorm(const double* v, const double* w, const double* b,
                  int64_t n, double eps, double* y)
{
    double mean = 0.0;
    for (int64_t j = 0; j < n; ++j)
        mean += v[j];
    mean /= (double)n;
    double var = 0.0;
    for (int64_t j = 0; j < n; ++j)
        var += (v[j] - mean) * (v[j] - mean);
    var /= (double)n;
    double rstd = 1.0 / sqrt(var + eps);
    for (int64_t j = 0; j < n; ++j)
        y[j] = (v[j] - mean) * rstd * (w ? w[j] : 1.0) + (b ? b[j] : 0.0);
}

/* 3D RoPE [FR section 2.2: the Wan video path rotates Q and K with a 3D
 * RoPE].  The D/2 rotary pairs are split into three consecutive ranges of
 * sec[0], sec[1], sec[2] pairs (time, height, width; the sum is D/2); pair
 * i of range a, at local index k, turns by pos3[a] * theta^(-k / sec[a]),
 * i.e. each range is a 1D RoPE of width 2 sec[a] on its own axis.  Pairs
 * are (i, i + D/2) or (2i, 2i+1) as in or_rope. */
void or_rope3d(double* v, int64_t D, const int32_t* pos3, const int32_t* sec,
               double theta, int style)
{
    int64_t half = D / 2;
    for (int64_t i = 0; i < half; ++i) {
        int a = i < sec[0] ? 0 : (i < sec[0] + sec[1] ? 1 : 2);
        int64_t k = i - (a > 0 ? sec[0] : 0) - (a > 1 ? sec[1] : 0);
        double inv_freq = pow(theta, -(double)k / (double)sec[a]);
        double ang = (double)pos3[a] * inv_freq;
        double c = cos(ang), s = sin(ang);
        int64_t ia = style == OR_ROPE_INTERLEAVED ? 2 * i : i;
        int64_t ib = style == OR_ROPE_INTERLEAVED ? 2 * i + 1 : i + half;
        double x0 = v[ia], x1 = v[ib];
        v[ia] = x0 * c - x1 * s;
        v[ib] = x1 * c + x0 * s;
    }
}

/* Gate activations: SiLU (SwiGLU) [SM89 Phase 2], GELU with the tanh
 * approximation (GeGLU) [FR section 二 table, steps 8-10] and squared ReLU
 * [FP, third technique]. */
double or_act(double g, int act)
{
    switch (act) {
    case OR_ACT_SWIGLU:
        return g / (1.0 + exp(-g));
    case OR_ACT_GEGLU_TANH: {
        const double k = sqrt(2.0 / acos(-1.0));   /* sqrt(2/pi) */
        return 0.5 * g * (1.0 + tanh(k * (g + 0.044715 * g * g * g)));
    }
    case OR_ACT_SQRELU:
        return g > 0.0 ? g * g : 0.0;
    default:
        return NAN;
    }
}

/* Static quantisation ("_static": the activation scale is a fixed
 * constant, [FR section 六]): code = E(y * mult). */
void or_quant_static(const double* y, int64_t n, double mult, uint8_t* q)
{
    for (int64_t j = 0; j < n; ++j)
        q[j] = or_e4m3_encode(y[j] * mult);
}

/* Dynamic quantisation of one group (a token row, or one block of 128
 * outputs of a row) [SM89 Phase 2]: the dequant scale is the group's
 * largest magnitude over 448 (floored so that an all-zero group stays
 * finite), stored as fp32; code = E(y / scale). */
float or_quant_dynamic(const double* y, int64_t n, uint8_t* q)
{
    const double floor_amax = (double)1e-10f;
    double amax = 0.0;
    for (int64_t j = 0; j < n; ++j)
        if (fabs(y[j]) > amax)
            amax = fabs(y[j]);
    if (amax < floor_amax)
        amax = floor_amax;
    float s = or_f32_round(amax / 448.0);
    for (int64_t j = 0; j < n; ++j)
        q[j] = or_e4m3_encode(y[j] / (double)s);
    return s;
}

/* ---- MX FP4 [HY 04 steps 5 and 9, 06 census: the residual-RMSNorm and
 * SwiGLU producers that feed FP4 GEMMs].  The pages name the producers but
 * not the format; the reading taken is the OCP Microscaling format MXFP4:
 * E2M1 elements (sign, 2 exponent bits with bias 1, 1 mantissa bit; the
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) in blocks of 32 sharing one
 * power-of-two scale stored as E8M0 (2^(code - 127)). ---- */

double or_e2m1_decode(uint8_t code)
{
    int s = (code >> 3) & 1, E = (code >> 1) & 3, M = code & 1;
    double a = (E == 0) ? 0.5 * M : ldexp(1.0 + 0.5 * M, E - 1);
    return s ? -a : a;
}

/* Round to nearest on the E2M1 grid, ties to the even code (the even
 * mantissa), magnitudes at or above 6 saturate to 6; the sign bit is the
 * input's sign, also when the value rounds to zero. */
uint8_t or_e2m1_encode(double v)
{
    uint8_t s = signbit(v) ? 8 : 0;
    double a = fabs(v);
    if (!(a < 6.0))                             /* also inf and NaN */
        return s | 7;
    double r = round_to_format(a, 2, 0);        /* 2 significant bits, emin 0 */
    return s | (uint8_t)pack_bits(r, 2, 1, 0, 2);
}

/* The block scale is 2^(floor(log2 amax) - 2): 2 is the exponent of the
 * largest E2M1 value, so the block maximum lands in [4, 8) before
 * rounding.  Clamped to the E8M0 range [2^-127, 2^127]; an all-zero
 * block gets the smallest scale. */
int or_mx_scale_code(double amax)
{
    if (!(amax > 0.0))
        return 0;
    int e;
    frexp(amax, &e);                            /* amax = f 2^e, f in [0.5, 1) */
    int x = (e - 1) - 2;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
    return x + 127;
}

/* Blocks of 32 consecutive values: scales[b] = E8M0 code, and element i
 * of the block is E2M1(y_i / 2^(code - 127)); two elements per byte,
 * element 2k in bits 3..0 and 2k+1 in bits 7..4. */
void or_quant_mxfp4(const double* y, int64_t n, uint8_t* packed, uint8_t* scales)
{
    for (int64_t b = 0; b < n / 32; ++b) {
        const double* yb = y + b * 32;
        double amax = 0.0;
        for (int i = 0; i < 32; ++i)
            if (fabs(yb[i]) > amax)
                amax = fabs(yb[i]);
        int code = or_mx_scale_code(amax);
        scales[b] = (uint8_t)code;
        double X = ldexp(1.0, code - 127);
        for (int i = 0; i < 32; i += 2) {
            uint8_t lo = or_e2m1_encode(yb[i] / X);
            uint8_t hi = or_e2m1_encode(yb[i + 1] / X);
            packed[(b * 32 + i) / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

/* ---- NVFP4 [HY 04 step 5 and 06 census: residual_add_rms_norm_to_nvfp4,
 * the producer of the FP4 GEMM inputs on that GPU].  The pages name the
 * format only; the reading taken is its published definition: E2M1
 * elements (the grid above) in blocks of 16 consecutive values, each block
 * with a scale stored as an E4M3 code, and one fp32 scale for the whole
 * tensor, so a value decodes as e2m1(code) * e4m3(block code) * g.  The
 * block scale maps the block's largest magnitude to 6, the largest E2M1
 * value: block code = E4M3(amax / (6 g)) (nearest, ties to even,
 * saturating at 448); element code = E2M1(y / S) with S = e4m3(block
 * code) * g (nearest, ties to even, saturating at 6, the sign kept).  A
 * block whose scale code decodes to 0 stores zero codes with the elements'
 * signs.  g, the dequantisation scale of the tensor, is an input (a
 * calibrated constant, like the static FP8 multiplier). ---- */

/* Blocks of 16 consecutive values: scales[b] = E4M3 code, two elements per
 * byte, element 2k in bits 3..0 and 2k+1 in bits 7..4. */
void or_quant_nvfp4(const double* y, int64_t n, double g, uint8_t* packed,
                    uint8_t* scales)
{
    for (int64_t b = 0; b < n / 16; ++b) {
        const double* yb = y + b * 16;
        double amax = 0.0;
        for (int i = 0; i < 16; ++i)
            if (fabs(yb[i]) > amax)
                amax = fabs(yb[i]);
        uint8_t sc = or_e4m3_encode(amax / (6.0 * g));
        scales[b] = sc;
        double S = or_e4m3_decode(sc) * g;      /* exact: 4 x 24 significant bits */
        for (int i = 0; i < 16; i += 2) {
            uint8_t lo = S > 0.0 ? or_e2m1_encode(yb[i] / S) : (signbit(yb[i]) ? 8 : 0);
            uint8_t hi = S > 0.0 ? or_e2m1_encode(yb[i + 1] / S) : (signbit(yb[i + 1]) ? 8 : 0);
            packed[(b * 16 + i) / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

/* Paged KV-cache slot of a token position [FP, paged cache]: page
 * page_table[pos / page_size], offset pos % page_size.  -1 when the
 * position, the table entry or the page is out of range. */
int64_t or_kv_slot(int64_t pos, const int32_t* page_table, int32_t table_len,
                   int32_t page_size, int32_t num_pages)
{
    if (pos < 0)
        return -1;
    int64_t idx = pos / page_size;
    if (idx >= table_len)
        return -1;
    int64_t page = page_table[idx];
    if (page < 0 || page >= num_pages)
        return -1;
    return page * page_size + pos % page_size;
}

/* ------------------------------------------------------------------ */
/* Fused ops                                                           */
/* ------------------------------------------------------------------ */

/* Residual add + RMSNorm + FP8 [FR section 二 table step 1, 2.1]:
 *   residual_out = round(x + residual)
 *   y = RMSNorm(residual_out) with the chosen weight convention
 *   STATIC: code = E(y * static_scale);
 *   TOKEN:  scale_t = amax_t / 448, code = E(y / scale_t). */
int oracle_resid_rmsnorm_fp8(const uint16_t* x, const uint16_t* residual,
                             uint16_t* residual_out, const uint16_t* weight,
                             int wmode, float eps, uint8_t* out_fp8, int qmode,
                             float static_scale, float* out_scales,
                             int64_t T, int64_t H, int dtype)
{
    double* ro = malloc(sizeof(double) * (size_t)H);
    double* w = malloc(sizeof(double) * (size_t)H);
    double* y = malloc(sizeof(double) * (size_t)H);
    if (!ro || !w || !y) {
        free(ro); free(w); free(y);
        return -1;
    }
    for (int64_t j = 0; j < H; ++j)
        w[j] = (wmode != OR_W_NONE) ? dec16(weight[j], dtype) : 0.0;
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* xr = x + t * H;
        const uint16_t* rr = residual + t * H;
        uint16_t* orow = residual_out + t * H;
        for (int64_t j = 0; j < H; ++j) {
            uint16_t b = enc16(dec16(xr[j], dtype) + dec16(rr[j], dtype), dtype);
            orow[j] = b;
            ro[j] = dec16(b, dtype);        /* the norm reads the stored value */
        }
        or_rmsnorm(ro, w, wmode, H, (double)eps, y);
        if (qmode == OR_Q_STATIC)
            or_quant_static(y, H, (double)static_scale, out_fp8 + t * H);
        else
            out_scales[t] = or_quant_dynamic(y, H, out_fp8 + t * H);
    }
    free(ro); free(w); free(y);
    return 0;
}

/* Residual add + RMSNorm + MX FP4 [HY 04 step 5, 06 census: the residual
 * RMSNorm FP4 producer]: residual_out and y as in the op above; y is
 * quantised to MXFP4 in blocks of 32 along the row (out_fp4 [T, H/2],
 * out_scales [T, H/32] E8M0 codes). */
int oracle_resid_rmsnorm_mxfp4(const uint16_t* x, const uint16_t* residual,
                               uint16_t* residual_out, const uint16_t* weight,
                               int wmode, float eps, uint8_t* out_fp4,
                               uint8_t* out_scales, int64_t T, int64_t H,
                               int dtype)
{
    if (H % 32 != 0)
        return -2;
    double* ro = malloc(sizeof(double) * (size_t)H);
    double* w = malloc(sizeof(double) * (size_t)H);
    double* y = malloc(sizeof(double) * (size_t)H);
    if (!ro || !w || !y) {
        free(ro); free(w); free(y);
        return -1;
    }
    for (int64_t j = 0; j < H; ++j)
        w[j] = (wmode != OR_W_NONE) ? dec16(weight[j], dtype) : 0.0;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < H; ++j) {
            uint16_t b = enc16(dec16(x[t * H + j], dtype) + dec16(residual[t * H + j], dtype),
                               dtype);
            residual_out[t * H + j] = b;
            ro[j] = dec16(b, dtype);
        }
        or_rmsnorm(ro, w, wmode, H, (double)eps, y);
        or_quant_mxfp4(y, H, out_fp4 + t * (H / 2), out_scales + t * (H / 32));
    }
    free(ro); free(w); free(y);
    return 0;
}

/* Residual add + RMSNorm + NVFP4 [HY 04 step 5, 06 census:
 * residual_add_rms_norm_to_nvfp4]: residual_out and y as in the FP8 op; y
 * is quantised to NVFP4 with the tensor scale global_scale (out_fp4
 * [T, H/2], out_scales [T, H/16] E4M3 codes). */
int oracle_resid_rmsnorm_nvfp4(const uint16_t* x, const uint16_t* residual,
                               uint16_t* residual_out, const uint16_t* weight,
                               int wmode, float eps, float global_scale,
                               uint8_t* out_fp4, uint8_t* out_scales, int64_t T,
                               int64_t H, int dtype)
{
    if (H % 16 != 0 || !(global_scale > 0.0f))
        return -2;
    double* ro = malloc(sizeof(double) * (size_t)H);
    double* w = malloc(sizeof(double) * (size_t)H);
    double* y = malloc(sizeof(double) * (size_t)H);
    if (!ro || !w || !y) {
        free(ro); free(w); free(y);
        return -1;
    }
    for (int64_t j = 0; j < H; ++j)
        w[j] = (wmode != OR_W_NONE) ? dec16(weight[j], dtype) : 0.0;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < H; ++j) {
            uint16_t b = enc16(dec16(x[t * H + j], dtype) + dec16(residual[t * H + j], dtype),
                               dtype);
            residual_out[t * H + j] = b;
            ro[j] = dec16(b, dtype);
        }
        or_rmsnorm(ro, w, wmode, H, (double)eps, y);
        or_quant_nvfp4(y, H, (double)global_scale, out_fp4 + t * (H / 2),
                       out_scales + t * (H / 16));
    }
    free(ro); free(w); free(y);
    return 0;
}

/* Residual add + LayerNorm + FP8 or MX FP4 [HY 06 census: the ViT
 * add-LayerNorm FP4 producer; the FP8 output as in the RMSNorm op]:
 *   residual_out = round(x + residual); y = LayerNorm(residual_out) with
 *   weight and bias (bias may be NULL);
 *   out_kind 0: FP8, static (code = E(y * static_scale)) or per token
 *   (qmode 1: scale = amax / 448 into out_scales_f32);
 *   out_kind 1: MXFP4 blocks of 32 (out_codes [T, H/2], out_scales_e8m0
 *   [T, H/32]). */
int oracle_resid_layernorm(const uint16_t* x, const uint16_t* residual,
                           uint16_t* residual_out, const uint16_t* weight,
                           const uint16_t* bias, float eps, int out_kind,
                           uint8_t* out_codes, int qmode, float static_scale,
                           float* out_scales_f32, uint8_t* out_scales_e8m0,
                           int64_t T, int64_t H, int dtype)
{
    if (out_kind == 1 && H % 32 != 0)
        return -2;
    double* ro = malloc(sizeof(double) * (size_t)H);
    double* w = malloc(sizeof(double) * (size_t)H);
    double* b = malloc(sizeof(double) * (size_t)H);
    double* y = malloc(sizeof(double) * (size_t)H);
    if (!ro || !w || !b || !y) {
        free(ro); free(w); free(b); free(y);
        return -1;
    }
    for (int64_t j = 0; j < H; ++j) {
        w[j] = dec16(weight[j], dtype);
        b[j] = bias ? dec16(bias[j], dtype) : 0.0;
    }
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < H; ++j) {
            uint16_t c = enc16(dec16(x[t * H + j], dtype) + dec16(residual[t * H + j], dtype),
                               dtype);
            residual_out[t * H + j] = c;
            ro[j] = dec16(c, dtype);
        }
        or_layernorm(ro, w, b, H, (double)eps, y);
        if (out_kind == 1)
            or_quant_mxfp4(y, H, out_codes + t * (H / 2), out_scales_e8m0 + t * (H / 32));
        else if (qmode == OR_Q_STATIC)
            or_quant_static(y, H, (double)static_scale, out_codes + t * H);
        else
            out_scales_f32[t] = or_quant_dynamic(y, H, out_codes + t * H);
    }
    free(ro); free(w); free(b); free(y);
    return 0;
}

/* Residual add + LayerNorm + NVFP4 [HY 06 census: the ViT add + LayerNorm
 * producer to NVFP4 (add_layer_norm_to_nvfp4)]: the new residual and the
 * LayerNorm output y of the op above, then or_quant_nvfp4 of each row with
 * the caller's fp32 tensor scale.  H % 16 == 0. */
int oracle_resid_layernorm_nvfp4(const uint16_t* x, const uint16_t* residual,
                                 uint16_t* residual_out, const uint16_t* weight,
                                 const uint16_t* bias, float eps, float global_scale,
                                 uint8_t* out_fp4, uint8_t* out_scales, int64_t T,
                                 int64_t H, int dtype)
{
    if (H % 16 != 0)
        return -2;
    double* ro = malloc(sizeof(double) * (size_t)H);
    double* w = malloc(sizeof(double) * (size_t)H);
    double* b = malloc(sizeof(double) * (size_t)H);
    double* y = malloc(sizeof(double) * (size_t)H);
    if (!ro || !w || !b || !y) {
        free(ro); free(w); free(b); free(y);
        return -1;
    }
    for (int64_t j = 0; j < H; ++j) {
        w[j] = dec16(weight[j], dtype);
        b[j] = bias ? dec16(bias[j], dtype) : 0.0;
    }
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < H; ++j) {
            uint16_t c = enc16(dec16(x[t * H + j], dtype) + dec16(residual[t * H + j], dtype),
                               dtype);
            residual_out[t * H + j] = c;
            ro[j] = dec16(c, dtype);
        }
        or_layernorm(ro, w, b, H, (double)eps, y);
        or_quant_nvfp4(y, H, (double)global_scale, out_fp4 + t * (H / 2),
                       out_scales + t * (H / 16));
    }
    free(ro); free(w); free(b); free(y);
    return 0;
}

/* Gate multiply + residual + adaptive RMSNorm + FP8 [FR section 三]:
 *   residual_out = round(residual + gate * x)
 *   y = RMSNorm(residual_out) * (1 + ada_scale) + ada_shift
 *   quantised as in the op above. */
int oracle_adarms_gate_res_fp8(const uint16_t* x, const uint16_t* gate,
                               const uint16_t* residual, uint16_t* residual_out,
                               const uint16_t* ada_scale, const uint16_t* ada_shift,
                               float eps, uint8_t* out_fp8, int qmode,
                               float static_scale, float* out_scales,
                               int64_t T, int64_t H, int dtype)
{
    double* ro = malloc(sizeof(double) * (size_t)H);
    double* sc = malloc(sizeof(double) * (size_t)H);
    double* sh = malloc(sizeof(double) * (size_t)H);
    double* y = malloc(sizeof(double) * (size_t)H);
    if (!ro || !sc || !sh || !y) {
        free(ro); free(sc); free(sh); free(y);
        return -1;
    }
    for (int64_t t = 0; t < T; ++t) {
        int64_t o = t * H;
        for (int64_t j = 0; j < H; ++j) {
            double h = dec16(residual[o + j], dtype)
                     + dec16(gate[o + j], dtype) * dec16(x[o + j], dtype);
            uint16_t b = enc16(h, dtype);
            residual_out[o + j] = b;
            ro[j] = dec16(b, dtype);
            sc[j] = dec16(ada_scale[o + j], dtype);
            sh[j] = dec16(ada_shift[o + j], dtype);
        }
        or_adarms(ro, sc, sh, H, (double)eps, y);
        if (qmode == OR_Q_STATIC)
            or_quant_static(y, H, (double)static_scale, out_fp8 + o);
        else
            out_scales[t] = or_quant_dynamic(y, H, out_fp8 + o);
    }
    free(ro); free(sc); free(sh); free(y);
    return 0;
}

/* Packed QKV split + per-head Q/K RMSNorm + RoPE + KV-cache write [FR
 * section 二 table step 3 and 2.2; FP paged cache; HY 04, step 10: the
 * attention's Q preparation folded into RoPE]:
 *   row t of qkv = [Q heads (Hq*D) | K heads (Hkv*D) | V heads (Hkv*D)]
 *   Q, K heads: optional RMSNorm over D with a weight shared by all heads
 *   (skipped when the weight pointer is NULL), then RoPE at positions[t];
 *   Q is then multiplied by q_scale (1 = none); then one rounding to the
 *   storage type.  Q goes to q_out[t, h, :]; K to
 *   k_cache[slot, g, :]; V is copied bit for bit to v_cache[slot, g, :].
 *   An out-of-range slot skips that token's K/V writes and sets bit 0 of
 *   *err_flag (when err_flag is given). */
int oracle_qkv_normrope_kvwrite(const uint16_t* qkv, const uint16_t* q_norm_w,
                                const uint16_t* k_norm_w, float eps,
                                const int32_t* positions, float rope_theta,
                                int rope_style, float q_scale, uint16_t* q_out,
                                uint16_t* k_cache, uint16_t* v_cache,
                                const int32_t* page_table, int32_t page_table_len,
                                int32_t page_size, int32_t num_pages,
                                int32_t* err_flag, int64_t T, int32_t Hq,
                                int32_t Hkv, int32_t D, int dtype)
{
    int64_t row = (int64_t)(Hq + 2 * Hkv) * D;
    double* v = malloc(sizeof(double) * (size_t)D);
    double* y = malloc(sizeof(double) * (size_t)D);
    double* qw = malloc(sizeof(double) * (size_t)D);
    double* kw = malloc(sizeof(double) * (size_t)D);
    if (!v || !y || !qw || !kw) {
        free(v); free(y); free(qw); free(kw);
        return -1;
    }
    for (int32_t d = 0; d < D; ++d) {
        qw[d] = q_norm_w ? dec16(q_norm_w[d], dtype) : 1.0;
        kw[d] = k_norm_w ? dec16(k_norm_w[d], dtype) : 1.0;
    }
    for (int64_t t = 0; t < T; ++t) {
        int64_t pos = positions[t];
        int64_t slot = or_kv_slot(pos, page_table, page_table_len, page_size,
                                  num_pages);
        if (slot < 0 && err_flag)
            *err_flag |= 1;
        for (int32_t h = 0; h < Hq + 2 * Hkv; ++h) {
            const uint16_t* src = qkv + t * row + (int64_t)h * D;
            if (h >= Hq + Hkv) {                      /* V: pass-through */
                int32_t g = h - Hq - Hkv;
                if (slot >= 0)
                    memcpy(v_cache + (slot * Hkv + g) * D, src,
                           sizeof(uint16_t) * (size_t)D);
                continue;
            }
            int is_q = h < Hq;
            const uint16_t* nw = is_q ? q_norm_w : k_norm_w;
            for (int32_t d = 0; d < D; ++d)
                v[d] = dec16(src[d], dtype);
            if (nw) {
                or_rmsnorm(v, is_q ? qw : kw, OR_W_MUL, D, (double)eps, y);
                memcpy(v, y, sizeof(double) * (size_t)D);
            }
            or_rope(v, D, pos, (double)rope_theta, rope_style);
            uint16_t* dst;
            if (is_q) {
                for (int32_t d = 0; d < D; ++d)   /* attention's Q pre-scale */
                    v[d] *= (double)q_scale;
                dst = q_out + (t * Hq + h) * D;
            } else {
                if (slot < 0)
                    continue;
                dst = k_cache + (slot * Hkv + (h - Hq)) * D;
            }
            for (int32_t d = 0; d < D; ++d)
                dst[d] = enc16(v[d], dtype);
        }
    }
    free(v); free(y); free(qw); free(kw);
    return 0;
}

/* Gated activation on interleaved gate/up + per-token block-128 FP8 [SM89
 * Phase 2; FP third technique]:
 *   gate_up row t = [g0, u0, g1, u1, ...] (2I values)
 *   h_j = act(g_j) * u_j, kept unrounded
 *   for each block b of 128 consecutive outputs: scale[t, b] = amax/448,
 *   code = E(h / scale).
 * The _f64 form takes the gate/up values in double (the GEMM-fused op feeds
 * it the exact product of the dequantised operands). */
int oracle_gated_act_fp8_f64(const double* gate_up, int act, uint8_t* out_fp8,
                             float* out_scales, int64_t T, int64_t I)
{
    const int64_t B = 128;
    double h[128];
    for (int64_t t = 0; t < T; ++t) {
        const double* gu = gate_up + t * 2 * I;
        for (int64_t b = 0; b < I / B; ++b) {
            for (int64_t k = 0; k < B; ++k) {
                int64_t j = b * B + k;
                h[k] = or_act(gu[2 * j], act) * gu[2 * j + 1];
            }
            out_scales[t * (I / B) + b] =
                or_quant_dynamic(h, B, out_fp8 + t * I + b * B);
        }
    }
    return 0;
}

/* Packed QKV split + Q/K norm + RoPE, the common contract of the Q/K
 * post-processing variants [FR section 2.2: one kernel normalises Q and K
 * and rotates them, V passes through; the variants differ in the norm
 * (RMSNorm, or LayerNorm on the Chameleon path), its scope (per head, or
 * the full width of all Q and all K heads on the Wan path) and the RoPE
 * layout (1D, or 3D on the Wan path)].
 *   row t of qkv = [Q heads | K heads | V heads], each head D-contiguous.
 *   norm (Q and K separately): per head over D with weight / bias [D], or
 *   over all Hq*D (Hkv*D) values with weight / bias [Hq*D] ([Hkv*D]);
 *   NULL weight = 1, NULL bias = 0; RMSNorm takes no bias.
 *   RoPE per head at positions[t] (1D) or positions[3t..3t+2] (3D, with
 *   sections[3] pairs per axis); Q times q_scale; one rounding.
 *   q_out [T,Hq,D], k_out [T,Hkv,D], v_out [T,Hkv,D] (V copied bit for bit). */
int oracle_qk_norm_rope(const uint16_t* qkv, int norm_kind, int norm_scope,
                        const uint16_t* q_norm_w, const uint16_t* q_norm_b,
                        const uint16_t* k_norm_w, const uint16_t* k_norm_b,
                        float eps, const int32_t* positions, int rope_dims,
                        const int32_t* sections, float rope_theta, int rope_style,
                        float q_scale, uint16_t* q_out, uint16_t* k_out,
                        uint16_t* v_out, int64_t T, int32_t Hq, int32_t Hkv,
                        int32_t D, int dtype)
{
    int64_t NH = Hq + 2 * Hkv, row = NH * D;
    int64_t nq = (int64_t)Hq * D, nk = (int64_t)Hkv * D;
    int64_t wq = norm_scope == OR_SCOPE_FULL ? nq : D;
    int64_t wk = norm_scope == OR_SCOPE_FULL ? nk : D;
    double* v = malloc(sizeof(double) * (size_t)row);
    double* y = malloc(sizeof(double) * (size_t)row);
    double* w4 = malloc(sizeof(double) * (size_t)(2 * (wq + wk)));
    if (!v || !y || !w4) {
        free(v); free(y); free(w4);
        return -1;
    }
    double* qw = w4;
    double* qb = w4 + wq;
    double* kw = w4 + 2 * wq;
    double* kb = w4 + 2 * wq + wk;
    for (int64_t j = 0; j < wq; ++j) {
        qw[j] = q_norm_w ? dec16(q_norm_w[j], dtype) : 1.0;
        qb[j] = q_norm_b ? dec16(q_norm_b[j], dtype) : 0.0;
    }
    for (int64_t j = 0; j < wk; ++j) {
        kw[j] = k_norm_w ? dec16(k_norm_w[j], dtype) : 1.0;
        kb[j] = k_norm_b ? dec16(k_norm_b[j], dtype) : 0.0;
    }
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < row; ++j)
            v[j] = dec16(qkv[t * row + j], dtype);
        memcpy(y, v, sizeof(double) * (size_t)row);
        /* norm of Q (values [0, nq)) and of K ([nq, nq + nk)) */
        for (int part = 0; part < 2; ++part) {
            int64_t base = part == 0 ? 0 : nq;
            int64_t len = part == 0 ? nq : nk;
            int64_t span = norm_scope == OR_SCOPE_FULL ? len : D;
            const double* w = part == 0 ? qw : kw;
            const double* b = part == 0 ? qb : kb;
            if (norm_kind == OR_NORM_NONE)
                continue;
            for (int64_t o = 0; o < len; o += span) {
                if (norm_kind == OR_NORM_RMS)
                    or_rmsnorm(v + base + o, w, OR_W_MUL, span, (double)eps, y + base + o);
                else
                    or_layernorm(v + base + o, w, b, span, (double)eps, y + base + o);
            }
        }
        /* RoPE per Q / K head, Q pre-scale, one rounding */
        for (int64_t h = 0; h < Hq + Hkv; ++h) {
            double* yh = y + h * D;
            if (rope_dims == 3)
                or_rope3d(yh, D, positions + 3 * t, sections, (double)rope_theta, rope_style);
            else
                or_rope(yh, D, positions[t], (double)rope_theta, rope_style);
            uint16_t* dst = h < Hq ? q_out + (t * Hq + h) * D : k_out + (t * Hkv + (h - Hq)) * D;
            for (int64_t d = 0; d < D; ++d)
                dst[d] = enc16(h < Hq ? yh[d] * (double)q_scale : yh[d], dtype);
        }
        memcpy(v_out + t * nk, qkv + t * row + nq + nk, sizeof(uint16_t) * (size_t)nk);
    }
    free(v); free(y); free(w4);
    return 0;
}

/* Gated activation + MX FP4 [HY 04 step 9, 06 census: the SwiGLU FP4
 * producer]: h = act(g) * u in double, quantised to MXFP4 in blocks of 32
 * outputs (out_fp4 [T, I/2], out_scales [T, I/32] E8M0 codes). */
int oracle_gated_act_mxfp4(const uint16_t* gate_up, int act, uint8_t* out_fp4,
                           uint8_t* out_scales, int64_t T, int64_t I, int dtype)
{
    if (I % 32 != 0)
        return -2;
    double* h = malloc(sizeof(double) * (size_t)I);
    if (!h)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* gu = gate_up + t * 2 * I;
        for (int64_t j = 0; j < I; ++j)
            h[j] = or_act(dec16(gu[2 * j], dtype), act) * dec16(gu[2 * j + 1], dtype);
        or_quant_mxfp4(h, I, out_fp4 + t * (I / 2), out_scales + t * (I / 32));
    }
    free(h);
    return 0;
}

int oracle_gated_act_fp8(const uint16_t* gate_up, int act, uint8_t* out_fp8,
                         float* out_scales, int64_t T, int64_t I, int dtype)
{
    double* gu = malloc(sizeof(double) * (size_t)(2 * I));
    if (!gu)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < 2 * I; ++j)
            gu[j] = dec16(gate_up[t * 2 * I + j], dtype);
        oracle_gated_act_fp8_f64(gu, act, out_fp8 + t * I,
                                 out_scales + t * (I / 128), 1, I);
    }
    free(gu);
    return 0;
}
