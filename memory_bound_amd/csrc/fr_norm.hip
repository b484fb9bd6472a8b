// fr_norm.hip -- residual add + RMSNorm + FP8 (op a) and gate + residual +
// adaptive RMSNorm + FP8 (op a'), one kernel template for both.
//
// Definitions: "FlashRT cross-layer fusion" article, section 二 (fused-kernel
// table step 1: residual add + RMSNorm + FP8 in one kernel; 2.1: "_noweight"
// means the norm weight is folded into the next GEMM) and section 三 (gate
// multiply + residual + AdaRMSNorm modulation + FP8 in one kernel).  The new
// residual is the correctly rounded exact sum in both ops: x + residual of two
// 16-bit values needs no care (fp32 is wide enough for the double rounding to
// be harmless), residual + gate*x is summed with round-to-odd.
//
// Mapping: one workgroup of `nw` wave64s per token row.  The row is cut into
// 16-byte chunks (8 values); lane l of wave w owns chunks
// k*64*nw + w*64 + l (k < CPL), so every load and store instruction of a
// wave touches one contiguous 1 KB span.  All input chunks are loaded before
// any arithmetic (a ragged row re-loads its last chunk instead of branching).
// The new residual is rounded to the storage type, written, and kept packed
// in registers; its sum of squares is accumulated in fp64 (squares of 16-bit
// values are exact in fp32, and the fp64 sum is exact for any realistic row,
// so rstd does not depend on the summation order).  The row sum is a DPP +
// permlane wave reduction, with LDS only for the cross-wave step.
//
// FP8 decision of op (a): the code of element j is E(y_j * K) with
// y_j = ro_j * rstd * W_j and K the static multiplier or 1/scale.  The kernel
// forms t_j = ro_j * W_j (exact in fp32 for 16-bit operands) and the
// per-row factor rstd * K in fp64, split into two fp32 halves; the product is
// evaluated as a float pair and rounded to odd, so the e4m3 rounding that
// follows is the rounding of the exact value to within ~2^-46.  Without this,
// rows where rstd cancels against the per-token scale (no weight) put many
// values exactly on e4m3 rounding midpoints and fp32 noise picks the side.
//
// MX FP4 output (plain modes; Hy-Embodied report, 04 step 5 and 06: the
// residual RMSNorm FP4 producer): the same rounded-to-odd products y_j, in
// blocks of 32 values = 4 consecutive lanes; the block maximum is a DPP
// quad reduction, its fp32 exponent gives the E8M0 code, and the elements
// are converted by the hardware E2M1 conversion after an exact power-of-two
// scaling.  Round-to-odd keeps both decisions exact: the exponent of the
// maximum (a value rounded to odd never lands on a power of two it did not
// equal) and the E2M1 rounding (24 bits rounded to odd, then to 2).
//
// NVFP4 output (plain modes; same report, 04 step 5 and 06: the residual
// RMSNorm producer writes NVFP4 there): blocks of 16 values = 2 lanes with
// an E4M3 scale mapping the block maximum to 6 and an fp32 tensor scale g
// given by the caller; both decisions are taken on exact or double values
// (details at the code).
#include "fr_device.h"
#include "fr_launch.h"

namespace fr {

enum { M_NONE = 0, M_MUL = 1, M_ONE_PLUS = 2, M_ADA = 3, M_LAYER = 4 };

template <bool NT>
__device__ __forceinline__ u32x4 ld_in(const void* p) {
    if constexpr (NT) return ld128_stream(p); else return ld128(p);
}
template <bool NT>
__device__ __forceinline__ void st_out(void* p, u32x4 v) {
    if constexpr (NT) st128_stream(p, v); else st128(p, v);
}
template <bool NT>
__device__ __forceinline__ void st_out(void* p, u32x2 v) {
    if constexpr (NT) st64_stream(p, v); else st64(p, v);
}

// NTL / NTS: non-temporal loads of the streamed inputs / stores of the
// outputs (the norm weight is re-read by every row and stays cached).
// MX / NV: MX FP4 or NVFP4 output instead of FP8 (plain modes and
// LayerNorm).
template <int DT, int CPL, int MODE, bool NTL, bool NTS = NTL, bool MX = false, bool NV = false>
__global__ __launch_bounds__(512) void k_norm(NormArgs a) {
    constexpr bool ADA = MODE == M_ADA;
    constexpr bool LAYER = MODE == M_LAYER;
    constexpr bool HAS_W = MODE == M_MUL || MODE == M_ONE_PLUS || LAYER;
    __shared__ double red_ss[8];
    __shared__ double red_ss2[8];
    __shared__ float red_max[8];

    const int lane = threadIdx.x & 63;
    // Wave in the workgroup and row in the workgroup, made uniform
    // (readfirstlane), so the row arithmetic runs on the scalar unit, the
    // loads use scalar-base addressing and the division is skipped for the
    // launch shapes (one row per workgroup, or one wave per row).  That takes
    // ~80 vector instructions off op (a)'s ~580 per wave (1.4% faster at
    // 8192 x 4096), and brings the adaptive op from 70 to 57 registers, so
    // 8 instead of 7 waves fit per SIMD (8192 x 1024 fp16: one round of
    // 8192 waves instead of 1.14; 2% faster at 4096 tokens, 0-1% at 8192).
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int rw = a.nw == 1 ? wave : (a.rpb == 1 ? 0 : wave / a.nw);
    const int ww = wave - rw * a.nw;                     // wave in the row
    const int64_t t_row = (int64_t)blockIdx.x * a.rpb + rw;
    const bool row_ok = t_row < a.T;
    const int64_t t = row_ok ? t_row : a.T - 1;          // in-bounds duplicate
    const int C = a.H >> 3;
    const int stride = a.nw * 64;
    const int64_t rb = t * (int64_t)a.H * 2;   // row offset in bytes

    const char* xr = (const char*)a.x + rb;
    const char* rr = (const char*)a.res + rb;
    char* ror = (char*)a.res_out + rb;

    u32x4 xv[CPL], rv[CPL], gv[CPL], sv[CPL], hv[CPL], wv[CPL], bv[CPL];
    bool ok[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = k * stride + ww * 64 + lane;
        ok[k] = c < C;
        const int cl = ok[k] ? c : C - 1;            // in-bounds duplicate
        xv[k] = ld_in<NTL>(xr + cl * 16);
        rv[k] = ld_in<NTL>(rr + cl * 16);
        if constexpr (ADA) {
            gv[k] = ld_in<NTL>((const char*)a.gate + rb + cl * 16);
            sv[k] = ld_in<NTL>((const char*)a.ada_scale + rb + cl * 16);
            hv[k] = ld_in<NTL>((const char*)a.ada_shift + rb + cl * 16);
        }
        if constexpr (HAS_W) wv[k] = ld128((const char*)a.w + cl * 16);
        if constexpr (LAYER) bv[k] = a.b ? ld128((const char*)a.b + cl * 16) : (u32x4){0, 0, 0, 0};
    }

    // Pass 1: new residual, rounded once; sum of squares of the stored value.
    double ss0 = 0.0, ss1 = 0.0;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        double c0 = 0.0, c1 = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float h0, h1;
            if constexpr (ADA) {
                // gate * x is exact in fp32 for 16-bit inputs; the sum is
                // rounded to odd so that the 16-bit rounding below is the
                // single correct rounding of residual + gate * x.
                h0 = add_round_odd(lo16<DT>(rv[k][e]), lo16<DT>(gv[k][e]) * lo16<DT>(xv[k][e]));
                h1 = add_round_odd(hi16<DT>(rv[k][e]), hi16<DT>(gv[k][e]) * hi16<DT>(xv[k][e]));
            } else {
                h0 = lo16<DT>(xv[k][e]) + lo16<DT>(rv[k][e]);
                h1 = hi16<DT>(xv[k][e]) + hi16<DT>(rv[k][e]);
            }
            const u32 b = pack16<DT>(h0, h1);
            rv[k][e] = b;
            const double r0 = (double)lo16<DT>(b), r1 = (double)hi16<DT>(b);
            c0 = fma(r0, r0, c0);
            c1 = fma(r1, r1, c1);
        }
        if (ok[k]) {                                 // skip duplicated chunks
            ss0 += c0;
            ss1 += c1;
            if (row_ok) st_out<NTS>(ror + (k * stride + ww * 64 + lane) * 16, rv[k]);
        }
    }

    uint8_t* orow = a.out + t * (int64_t)a.H;
    if constexpr (LAYER) {
        // LayerNorm: mean, then the variance about it, both as fp64 row sums
        // of the stored values (exact for realistic rows, so independent of
        // the order); y = (ro - mean) * rstd * w + b in fp32.
        auto row_sum = [&](double v, double* slots) {
            v = wave_sum_d(v);
            if (a.nw > 1) {
                if (lane == 0) slots[wave] = v;
                __syncthreads();
                v = slots[rw * a.nw];
                for (int w = 1; w < a.nw; ++w) v += slots[rw * a.nw + w];
            }
            return v;
        };
        double s1 = 0.0;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            if (!ok[k]) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                s1 += (double)lo16<DT>(rv[k][e]) + (double)hi16<DT>(rv[k][e]);
        }
        const double mean_d = row_sum(s1, red_ss) * a.inv_h;
        double s2 = 0.0;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            if (!ok[k]) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double d0 = (double)lo16<DT>(rv[k][e]) - mean_d;
                const double d1 = (double)hi16<DT>(rv[k][e]) - mean_d;
                s2 = fma(d0, d0, fma(d1, d1, s2));
            }
        }
        const double var_d = row_sum(s2, red_ss2) * a.inv_h;
        const float rstd = (float)rsqrt_d(var_d + (double)a.eps);
        const float mean = (float)mean_d;
        float y[CPL][8];
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y[k][2 * e] = fmaf((lo16<DT>(rv[k][e]) - mean) * rstd, lo16<DT>(wv[k][e]),
                                   lo16<DT>(bv[k][e]));
                y[k][2 * e + 1] = fmaf((hi16<DT>(rv[k][e]) - mean) * rstd, hi16<DT>(wv[k][e]),
                                       hi16<DT>(bv[k][e]));
                if (ok[k]) amax = fmaxf(amax, fmaxf(fabsf(y[k][2 * e]), fabsf(y[k][2 * e + 1])));
            }
        }
        if constexpr (NV) {
            // NVFP4: a block of 16 values is a lane pair.  The block scale
            // code is E4M3(amax / (6 g)) of the fp32 y: amax / (6 g) in
            // double, rounded to odd into fp32 so the saturating conversion
            // rounds the double value; the elements are E2M1(y * K) with
            // K = 1 / S in fp32, S = e4m3(code) * g (y itself is fp32, so a
            // wider product would not bring the codes closer to the exact
            // ones; K is clamped to the fp32 range for tiny scales, where
            // every nonzero y saturates either way).
            uint8_t* orow4 = a.out + t * (int64_t)(a.H >> 1);
            uint8_t* srow = a.mx_scales + t * (int64_t)(a.H >> 4);
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                float m = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(y[k][e]));
                m = group_reduce<2>(m, OpMaxMag());      // the block's other lane
                const double sd = (double)m * a.inv6g;
                const float sh = (float)sd;
                const float sf = round_odd(sh, (float)(sd - (double)sh));
                const int code = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(sf), 0.0f, 0, false) & 0xFF;
                const double S = (double)__builtin_amdgcn_cvt_f32_fp8(code, 0) * (double)a.gscale;
                const float K = S > 0.0 ? (float)fmin(rcp_d(S), 3.4028234663852886e38) : 0.0f;
                const u32 pk = pack_e2m1x8(y[k], K);
                if (ok[k] && row_ok) {
                    const int c = k * stride + ww * 64 + lane;
                    u32* dst = (u32*)(orow4 + c * 4);
                    if constexpr (NTS) __builtin_nontemporal_store(pk, dst); else *dst = pk;
                    if ((lane & 1) == 0) srow[c >> 1] = (uint8_t)code;
                }
            }
            return;
        }
        if constexpr (MX) {
            uint8_t* orow4 = a.out + t * (int64_t)(a.H >> 1);
            uint8_t* srow = a.mx_scales + t * (int64_t)(a.H >> 5);
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                float m = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(y[k][e]));
                m = group_reduce<4>(m, OpMaxMag());      // a block of 32 = 4 lanes
                const int code = mx_code(m);
                const u32 p = pack_e2m1x8(y[k], mx_mult(code));
                if (ok[k] && row_ok) {
                    const int c = k * stride + ww * 64 + lane;
                    u32* dst = (u32*)(orow4 + c * 4);
                    if constexpr (NTS) __builtin_nontemporal_store(p, dst); else *dst = p;
                    if ((lane & 3) == 0) srow[c >> 2] = (uint8_t)code;
                }
            }
            return;
        }
        float mult = a.static_scale;
        if (a.qmode == 1) {
            amax = wave_reduce(amax, OpMaxMag());
            if (a.nw > 1) {
                if (lane == 0) red_max[wave] = amax;
                __syncthreads();
                amax = red_max[rw * a.nw];
                for (int w = 1; w < a.nw; ++w) amax = OpMaxMag()(amax, red_max[rw * a.nw + w]);
            }
            const float s = div448(fmaxf(amax, 1e-10f));     // correctly rounded
            mult = 1.0f / s;
            if (row_ok && ww == 0 && lane == 0) a.scales[t] = s;
        }
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            if (!ok[k] || !row_ok) continue;
            u32x2 q;
            q.x = pack_e4m3x4(y[k][0] * mult, y[k][1] * mult, y[k][2] * mult, y[k][3] * mult);
            q.y = pack_e4m3x4(y[k][4] * mult, y[k][5] * mult, y[k][6] * mult, y[k][7] * mult);
            st_out<NTS>(orow + (k * stride + ww * 64 + lane) * 8, q);
        }
        return;
    }

    // Pass 2 of the plain modes, before the row reduction: t = ro * W
    // (a float pair for the (1+w) case) and max |t|, which does not depend
    // on rstd, so the per-token amax travels with the sum of squares and the
    // row needs one cross-wave step, not two.
    float th[CPL][8], tl[CPL][8];
    float tmax = 0.0f;
    if constexpr (!ADA) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            float cmax = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const u32 rw = rv[k][e >> 1];
                const float ro = (e & 1) ? hi16<DT>(rw) : lo16<DT>(rw);
                float hi = ro, lo = 0.0f;
                if constexpr (MODE == M_MUL) {
                    const u32 ww = wv[k][e >> 1];
                    hi = ro * ((e & 1) ? hi16<DT>(ww) : lo16<DT>(ww));     // exact
                } else if constexpr (MODE == M_ONE_PLUS) {
                    const u32 ww = wv[k][e >> 1];
                    const float c = 1.0f + ((e & 1) ? hi16<DT>(ww) : lo16<DT>(ww));
                    hi = ro * c;
                    lo = fmaf(ro, c, -hi);                                  // exact remainder
                }
                th[k][e] = hi;
                tl[k][e] = lo;
                cmax = fmaxf(cmax, fabsf(hi));
            }
            if (ok[k]) tmax = fmaxf(tmax, cmax);         // one select per chunk
        }
    }
    const bool token_max = !ADA && !MX && !NV && a.qmode == 1;
    double ss = wave_sum_d(ss0 + ss1);
    if (token_max) tmax = wave_reduce(tmax, OpMaxMag());
    if (a.nw > 1) {
        if (lane == 0) {
            red_ss[wave] = ss;
            red_max[wave] = tmax;
        }
        __syncthreads();
        ss = red_ss[rw * a.nw];
        for (int w = 1; w < a.nw; ++w) ss += red_ss[rw * a.nw + w];
        if (token_max) {
            tmax = red_max[rw * a.nw];
            for (int w = 1; w < a.nw; ++w) tmax = OpMaxMag()(tmax, red_max[rw * a.nw + w]);
        }
    }
    const double rstd_d = rsqrt_d(ss * a.inv_h + (double)a.eps);

    if constexpr (ADA) {
        // Pass 2 (adaptive): y = n * (1 + scale) + shift in fp32.
        const float rstd = (float)rstd_d;
        float y[CPL][8];
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float n0 = lo16<DT>(rv[k][e]) * rstd;
                const float n1 = hi16<DT>(rv[k][e]) * rstd;
                const float y0 = fmaf(n0, 1.0f + lo16<DT>(sv[k][e]), lo16<DT>(hv[k][e]));
                const float y1 = fmaf(n1, 1.0f + hi16<DT>(sv[k][e]), hi16<DT>(hv[k][e]));
                y[k][2 * e] = y0;
                y[k][2 * e + 1] = y1;
                if (ok[k]) amax = fmaxf(amax, fmaxf(fabsf(y0), fabsf(y1)));
            }
        }
        float mult = a.static_scale;
        if (a.qmode == 1) {
            amax = wave_reduce(amax, OpMax());
            if (a.nw > 1) {
                if (lane == 0) red_max[wave] = amax;
                __syncthreads();
                amax = red_max[rw * a.nw];
                for (int w = 1; w < a.nw; ++w) amax = fmaxf(amax, red_max[rw * a.nw + w]);
            }
            const float s = div448(fmaxf(amax, 1e-10f));     // correctly rounded
            mult = 1.0f / s;
            if (row_ok && ww == 0 && lane == 0) a.scales[t] = s;
        }
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            if (!ok[k] || !row_ok) continue;
            u32x2 q;
            q.x = pack_e4m3x4(y[k][0] * mult, y[k][1] * mult, y[k][2] * mult, y[k][3] * mult);
            q.y = pack_e4m3x4(y[k][4] * mult, y[k][5] * mult, y[k][6] * mult, y[k][7] * mult);
            st_out<NTS>(orow + (k * stride + ww * 64 + lane) * 8, q);
        }
    } else {
        // Pass 3 (plain): the FP8 / FP4 codes of t * rstd * K.
        if constexpr (NV) {
            // NVFP4: a block of 16 values is a lane pair.  The block scale
            // code is E4M3(amax / (6 g)), decided on the double value
            // max|t| * rstd / (6 g) (|t| exact: hi + lo in double), rounded
            // to odd into fp32 before the saturating conversion, so the
            // conversion rounds the double value.  The elements are the
            // E2M1 codes of t * (rstd / S), S = e4m3(code) * g exact in
            // fp64, formed as round-to-odd products like the FP8 path.
            uint8_t* orow4 = a.out + t * (int64_t)(a.H >> 1);
            uint8_t* srow = a.mx_scales + t * (int64_t)(a.H >> 4);
            const double c6 = rstd_d * a.inv6g;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                double m;
                if constexpr (MODE == M_ONE_PLUS) {          // |t| = |hi + lo| needs fp64
                    m = 0.0;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        m = fmax(m, fabs((double)th[k][e] + (double)tl[k][e]));
                    m = fmax(m, dpp_d<DPP_PAIR>(m));     // the block's other lane
                } else {                                     // t is exact in fp32
                    float mf = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) mf = fmaxf(mf, fabsf(th[k][e]));
                    mf = group_reduce<2>(mf, OpMaxMag());    // the block's other lane
                    m = (double)mf;
                }
                const double sd = m * c6;
                const float sh = (float)sd;
                const float sf = round_odd(sh, (float)(sd - (double)sh));
                const int code = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(sf), 0.0f, 0, false) & 0xFF;
                const double S = (double)__builtin_amdgcn_cvt_f32_fp8(code, 0) * (double)a.gscale;
                const double Kd = S > 0.0 ? rstd_d * rcp_d(S) : 0.0;
                const float Kh = (float)Kd;
                const float Kl = (float)(Kd - (double)Kh);
                float q[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = th[k][e] * Kh;
                    float r = fmaf(th[k][e], Kh, -p);
                    r = fmaf(th[k][e], Kl, r);
                    if constexpr (MODE == M_ONE_PLUS) r = fmaf(tl[k][e], Kh, r);
                    q[e] = round_odd(p, r);
                }
                const u32 pk = pack_e2m1x8(q, 1.0f);
                if (ok[k] && row_ok) {
                    const int c = k * stride + ww * 64 + lane;
                    u32* dst = (u32*)(orow4 + c * 4);
                    if constexpr (NTS) __builtin_nontemporal_store(pk, dst); else *dst = pk;
                    if ((lane & 1) == 0) srow[c >> 1] = (uint8_t)code;
                }
            }
            return;
        }
        if constexpr (MX) {
            const float Kh = (float)rstd_d;
            const float Kl = (float)(rstd_d - (double)Kh);
            uint8_t* orow4 = a.out + t * (int64_t)(a.H >> 1);
            uint8_t* srow = a.mx_scales + t * (int64_t)(a.H >> 5);
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                float q[8];
                float m = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = th[k][e] * Kh;
                    float r = fmaf(th[k][e], Kh, -p);
                    r = fmaf(th[k][e], Kl, r);
                    if constexpr (MODE == M_ONE_PLUS) r = fmaf(tl[k][e], Kh, r);
                    q[e] = round_odd(p, r);
                    m = fmaxf(m, fabsf(q[e]));
                }
                // a block (4 lanes) is either wholly inside the row or not
                m = group_reduce<4>(m, OpMaxMag());
                const int code = mx_code(m);
                const u32 p = pack_e2m1x8(q, mx_mult(code));
                if (ok[k] && row_ok) {
                    const int c = k * stride + ww * 64 + lane;
                    u32* dst = (u32*)(orow4 + c * 4);
                    if constexpr (NTS) __builtin_nontemporal_store(p, dst); else *dst = p;
                    if ((lane & 3) == 0) srow[c >> 2] = (uint8_t)code;
                }
            }
            return;
        }
        double K = rstd_d * (double)a.static_scale;
        if (a.qmode == 1) {
            const double amax = fmax((double)tmax * rstd_d, (double)1e-10f);
            const float s = (float)div448_d(amax);
            K = rstd_d * rcp_d((double)s);
            if (row_ok && ww == 0 && lane == 0) a.scales[t] = s;
        }
        const float Kh = (float)K;
        const float Kl = (float)(K - (double)Kh);
        // Per-token scales bound every |t K| by amax / s <= 448 (1 + 2^-23),
        // inside the conversion's exact range, so that path needs no clamp.
        auto codes = [&](auto pack) {
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                if (!ok[k] || !row_ok) continue;
                float q[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = th[k][e] * Kh;
                    float r = fmaf(th[k][e], Kh, -p);
                    r = fmaf(th[k][e], Kl, r);
                    if constexpr (MODE == M_ONE_PLUS) r = fmaf(tl[k][e], Kh, r);
                    q[e] = round_odd(p, r);
                }
                u32x2 o;
                o.x = pack(q[0], q[1], q[2], q[3]);
                o.y = pack(q[4], q[5], q[6], q[7]);
                st_out<NTS>(orow + (k * stride + ww * 64 + lane) * 8, o);
            }
        };
        if (a.qmode == 1)
            codes([](float x0, float x1, float x2, float x3) { return pack_e4m3x4_in_range(x0, x1, x2, x3); });
        else
            codes([](float x0, float x1, float x2, float x3) { return pack_e4m3x4(x0, x1, x2, x3); });
    }
}

template <int DT, int MODE, bool NT, bool MX, bool NV = false>
static hipError_t launch_norm_mode(const NormArgs& a, int cpl, hipStream_t s) {
    // the adaptive op's outputs are stored cacheable even when streaming
    // (measured 2-3% faster at 8192 x 1024 fp16)
    constexpr bool NTS = NT && MODE != M_ADA;
    const void* fn;
    switch (cpl) {
    case 1: fn = (const void*)k_norm<DT, 1, MODE, NT, NTS, MX, NV>; break;
    case 2: fn = (const void*)k_norm<DT, 2, MODE, NT, NTS, MX, NV>; break;
    case 4: fn = (const void*)k_norm<DT, 4, MODE, NT, NTS, MX, NV>; break;
    default: fn = (const void*)k_norm<DT, 8, MODE, NT, NTS, MX, NV>; break;
    }
    NormArgs copy = a;
    void* args[] = {&copy};
    const unsigned blocks = (unsigned)((a.T + a.rpb - 1) / a.rpb);
    return hipLaunchKernel(fn, dim3(blocks), dim3(64 * a.nw * a.rpb), args, 0, s);
}

template <int DT, bool NT>
static hipError_t launch_norm_dt(const NormArgs& a, int mode, bool mx, bool nv, int cpl,
                                 hipStream_t s) {
    if (nv) {
        switch (mode) {
        case M_NONE: return launch_norm_mode<DT, M_NONE, NT, false, true>(a, cpl, s);
        case M_MUL: return launch_norm_mode<DT, M_MUL, NT, false, true>(a, cpl, s);
        case M_LAYER: return launch_norm_mode<DT, M_LAYER, NT, false, true>(a, cpl, s);
        default: return launch_norm_mode<DT, M_ONE_PLUS, NT, false, true>(a, cpl, s);
        }
    }
    if (mx) {
        switch (mode) {
        case M_NONE: return launch_norm_mode<DT, M_NONE, NT, true>(a, cpl, s);
        case M_MUL: return launch_norm_mode<DT, M_MUL, NT, true>(a, cpl, s);
        case M_LAYER: return launch_norm_mode<DT, M_LAYER, NT, true>(a, cpl, s);
        default: return launch_norm_mode<DT, M_ONE_PLUS, NT, true>(a, cpl, s);
        }
    }
    switch (mode) {
    case M_NONE: return launch_norm_mode<DT, M_NONE, NT, false>(a, cpl, s);
    case M_MUL: return launch_norm_mode<DT, M_MUL, NT, false>(a, cpl, s);
    case M_ONE_PLUS: return launch_norm_mode<DT, M_ONE_PLUS, NT, false>(a, cpl, s);
    case M_LAYER: return launch_norm_mode<DT, M_LAYER, NT, false>(a, cpl, s);
    default: return launch_norm_mode<DT, M_ADA, NT, false>(a, cpl, s);
    }
}

struct NormShape {
    int cpl, nw, rpb;
    bool nt;
};

// Launch shape: at most two 16-byte chunks per lane, so a row spreads over
// up to 8 wavefronts (more chunks per lane only for rows wider than 8192
// values), and in the bandwidth regime (T >= 2048) two single-wave rows per
// workgroup and non-temporal streaming.  Measured on MI355X at T = 8192 in
// steady state: H = 4096 bf16 at ~73% of 8 TB/s with 4 waves x 2 chunks per
// row (re-measured after the instruction trimming: 2 rows of 4 waves per
// workgroup 72%, 2 waves x 4 chunks 69-70%, 1 wave x 8 chunks 66%, 8 waves x
// 1 chunk 65%; before it, cacheable stores: 64%); H = 1024 fp16 adaptive at
// ~69% with 2 rows per workgroup (1 or 4 rows: 65-67%).  Small batches keep
// the outputs cacheable for the next op.
static NormShape pick_norm_shape(int64_t T, int H, bool adaptive) {
    (void)adaptive;
    const int C = H / 8;
    const bool big = T >= 2048;
    int c = 1;
    while (c < 2 && c * 64 < C) c *= 2;
    int w = (C + 64 * c - 1) / (64 * c);
    while (w > 8) {
        c *= 2;
        w = (C + 64 * c - 1) / (64 * c);
    }
    const int rpb = (big && w == 1) ? 2 : 1;
    return {c, w, rpb, big};
}

hipError_t launch_norm(const NormArgs& in, int dtype, int kind, hipStream_t s) {
    NormArgs a = in;
    const bool adaptive = kind == NORM_ADA_FP8;
    const bool layer = kind == NORM_LAYER_FP8 || kind == NORM_LAYER_MXFP4 || kind == NORM_LAYER_NVFP4;
    const bool mx = kind == NORM_MXFP4 || kind == NORM_LAYER_MXFP4;
    const bool nv = kind == NORM_NVFP4 || kind == NORM_LAYER_NVFP4;
    const NormShape sh = pick_norm_shape(a.T, a.H, adaptive);
    a.inv_h = 1.0 / (double)a.H;
    if (nv) a.inv6g = 1.0 / (6.0 * (double)a.gscale);
    a.nw = sh.nw;
    a.rpb = sh.rpb;
    const int mode = adaptive ? M_ADA : (layer ? M_LAYER : a.wmode);
    if (dtype == DT_BF16)
        return sh.nt ? launch_norm_dt<DT_BF16, true>(a, mode, mx, nv, sh.cpl, s)
                     : launch_norm_dt<DT_BF16, false>(a, mode, mx, nv, sh.cpl, s);
    return sh.nt ? launch_norm_dt<DT_F16, true>(a, mode, mx, nv, sh.cpl, s)
                 : launch_norm_dt<DT_F16, false>(a, mode, mx, nv, sh.cpl, s);
}

}  // namespace fr
