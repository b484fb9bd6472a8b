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
// any arithmetic.  The new residual is rounded to the storage type, written,
// and kept packed in registers; its sum of squares is accumulated in fp64
// (squares of 16-bit values are exact in fp32; the fp64 sum makes rstd
// independent of the summation order).  The row sum is a DPP + permlane wave
// reduction, with LDS only for the cross-wave step.  FP8 codes are packed
// with v_cvt_pk_fp8_f32 after a +-448 clamp and written 8 bytes per chunk.
#include "fr_device.h"
#include "fr_launch.h"

namespace fr {

template <int DT, int CPL, bool ADA>
__global__ __launch_bounds__(512) void k_norm(NormArgs a) {
    __shared__ double red_ss[8];
    __shared__ float red_max[8];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t t = blockIdx.x;
    const int C = a.H >> 3;
    const int stride = a.nw * 64;
    const int64_t rb = t * (int64_t)a.H * 2;   // row offset in bytes

    const char* xr = (const char*)a.x + rb;
    const char* rr = (const char*)a.res + rb;
    char* ror = (char*)a.res_out + rb;

    u32x4 xv[CPL], rv[CPL], gv[CPL], sv[CPL], hv[CPL], wv[CPL];
    bool ok[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = k * stride + wave * 64 + lane;
        ok[k] = c < C;
        xv[k] = rv[k] = gv[k] = sv[k] = hv[k] = wv[k] = (u32x4){0, 0, 0, 0};
        if (ok[k]) {
            xv[k] = ld128(xr + c * 16);
            rv[k] = ld128(rr + c * 16);
            if constexpr (ADA) {
                gv[k] = ld128((const char*)a.gate + rb + c * 16);
                sv[k] = ld128((const char*)a.ada_scale + rb + c * 16);
                hv[k] = ld128((const char*)a.ada_shift + rb + c * 16);
            } else {
                if (a.wmode != 0) wv[k] = ld128((const char*)a.w + c * 16);
            }
        }
    }

    // Pass 1: new residual, rounded once; sum of squares of the stored value.
    double ss0 = 0.0, ss1 = 0.0;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
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
            const u32 b = ok[k] ? pack16<DT>(h0, h1) : 0u;
            rv[k][e] = b;
            const double r0 = (double)lo16<DT>(b), r1 = (double)hi16<DT>(b);
            ss0 = fma(r0, r0, ss0);
            ss1 = fma(r1, r1, ss1);
        }
        if (ok[k]) st128(ror + (k * stride + wave * 64 + lane) * 16, rv[k]);
    }

    double ss = wave_sum_d(ss0 + ss1);
    if (a.nw > 1) {
        if (lane == 0) red_ss[wave] = ss;
        __syncthreads();
        ss = red_ss[0];
        for (int w = 1; w < a.nw; ++w) ss += red_ss[w];
    }
    const float rstd = (float)(1.0 / sqrt(ss / (double)a.H + (double)a.eps));

    // Pass 2: normalised (and modulated) values.
    float y[CPL][8];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float n0 = lo16<DT>(rv[k][e]) * rstd;
            const float n1 = hi16<DT>(rv[k][e]) * rstd;
            float y0, y1;
            if constexpr (ADA) {
                y0 = fmaf(n0, 1.0f + lo16<DT>(sv[k][e]), lo16<DT>(hv[k][e]));
                y1 = fmaf(n1, 1.0f + hi16<DT>(sv[k][e]), hi16<DT>(hv[k][e]));
            } else {
                y0 = n0;
                y1 = n1;
                if (a.wmode == 1) {
                    y0 *= lo16<DT>(wv[k][e]);
                    y1 *= hi16<DT>(wv[k][e]);
                } else if (a.wmode == 2) {
                    y0 *= 1.0f + lo16<DT>(wv[k][e]);
                    y1 *= 1.0f + hi16<DT>(wv[k][e]);
                }
            }
            y[k][2 * e] = y0;
            y[k][2 * e + 1] = y1;
            amax = fmaxf(amax, fmaxf(fabsf(y0), fabsf(y1)));
        }
    }

    float mult = a.static_scale;
    if (a.qmode == 1) {
        amax = wave_reduce(amax, OpMax());
        if (a.nw > 1) {
            if (lane == 0) red_max[wave] = amax;
            __syncthreads();
            amax = red_max[0];
            for (int w = 1; w < a.nw; ++w) amax = fmaxf(amax, red_max[w]);
        }
        const float s = fmaxf(amax, 1e-10f) / 448.0f;   // IEEE division
        mult = 1.0f / s;
        if (wave == 0 && lane == 0) a.scales[t] = s;
    }

    uint8_t* orow = a.out + t * (int64_t)a.H;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue;
        u32x2 q;
        q.x = pack_e4m3x4(y[k][0] * mult, y[k][1] * mult, y[k][2] * mult, y[k][3] * mult);
        q.y = pack_e4m3x4(y[k][4] * mult, y[k][5] * mult, y[k][6] * mult, y[k][7] * mult);
        st64(orow + (k * stride + wave * 64 + lane) * 8, q);
    }
}

template <int DT, bool ADA>
static hipError_t launch_norm_dt(const NormArgs& a, int cpl, hipStream_t s) {
    const void* fn;
    switch (cpl) {
    case 1: fn = (const void*)k_norm<DT, 1, ADA>; break;
    case 2: fn = (const void*)k_norm<DT, 2, ADA>; break;
    case 4: fn = (const void*)k_norm<DT, 4, ADA>; break;
    default: fn = (const void*)k_norm<DT, 8, ADA>; break;
    }
    NormArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel(fn, dim3((unsigned)a.T), dim3(64 * a.nw), args, 0, s);
}

// Chunks per lane and wavefronts per row.  Large batches (bandwidth regime)
// use few wavefronts per row with many chunks per lane, which keeps the whole
// row's loads in flight per wave without any LDS step; small batches
// (latency regime) spread each row over more wavefronts so that each lane has
// at most two chunks of serial work.
static void pick_norm_shape(int64_t T, int H, bool adaptive, int* cpl, int* nw) {
    const int C = H / 8;
    int target = T >= 2048 ? (adaptive ? 4 : 8) : 2;
    int c = 1;
    while (c < target && c * 64 < C) c *= 2;
    int w = (C + 64 * c - 1) / (64 * c);
    while (w > 8) {
        c *= 2;
        w = (C + 64 * c - 1) / (64 * c);
    }
    *cpl = c;
    *nw = w;
}

hipError_t launch_norm(const NormArgs& in, int dtype, bool adaptive, hipStream_t s) {
    NormArgs a = in;
    int cpl, nw;
    pick_norm_shape(a.T, a.H, adaptive, &cpl, &nw);
    a.nw = nw;
    if (dtype == DT_BF16)
        return adaptive ? launch_norm_dt<DT_BF16, true>(a, cpl, s)
                        : launch_norm_dt<DT_BF16, false>(a, cpl, s);
    return adaptive ? launch_norm_dt<DT_F16, true>(a, cpl, s)
                    : launch_norm_dt<DT_F16, false>(a, cpl, s);
}

}  // namespace fr
