// fr_qkv.hip -- packed QKV split + per-head Q/K RMSNorm + RoPE + paged
// KV-cache write (op b), one kernel.
//
// Definitions: "FlashRT cross-layer fusion" article, section 二 (table step 3:
// QKV split + RoPE + KV-cache write in one kernel; 2.2: q_norm -> RoPE -> Q,
// k_norm -> RoPE -> KV cache in one kernel, V passed through, RoPE pairs kept
// in one lane so no cross-lane shuffle is needed) and the "Falcon-Perception
// inference engine" article (paged KV cache written by the decode step).
//
// Mapping: a wave64 handles one token and a group of 64/LP heads; LP lanes
// (a power of two >= D/16) serve one head.  Lane j of a head holds the
// 16-byte chunk j of the first half of the head and chunk j of the second
// half, so each rotate-half pair (i, i+D/2) -- and each interleaved pair
// (2i, 2i+1) -- sits in one lane's registers.  The per-head sum of squares is
// a DPP reduction over the LP lanes.  Rotation angles are formed in fp64
// (pos * theta^(-2i/D), reduced modulo pi/2 by a two-constant Cody-Waite
// step with fma) and their sine/cosine come from Taylor polynomials on
// [-pi/4, pi/4], so the angle stays exact to ~1e-16 for any int32 position.
#include "fr_device.h"
#include "fr_launch.h"

namespace fr {

// sin and cos of x (radians).  k = nearest integer to x/(pi/2), r = x - k*pi/2
// with pi/2 split into a head (the double nearest pi/2) and its tail; fma
// keeps k*head exact.  Taylor series to r^11 / r^12 (truncation < 1e-11 on
// |r| <= pi/4), then the quadrant of k picks and signs the two.
__device__ __forceinline__ void sincos_pos(double x, float* s_out, float* c_out) {
    const double two_over_pi = 0.63661977236758134308;
    const double pio2_hi = 1.5707963267948966;          // nearest double to pi/2
    const double pio2_lo = 6.123233995736766e-17;       // pi/2 - pio2_hi
    const double k = rint(x * two_over_pi);
    double r = fma(-k, pio2_hi, x);
    r = fma(-k, pio2_lo, r);
    const double r2 = r * r;
    // 1/n! coefficients
    double sp = 2.505210838544172e-08;                  // 1/11!
    sp = fma(sp, r2, -2.7557319223985893e-06);          // 1/9!
    sp = fma(sp, r2, 1.984126984126984e-04);            // 1/7!
    sp = fma(sp, r2, -8.333333333333333e-03);           // 1/5!
    sp = fma(sp, r2, 1.6666666666666666e-01);           // 1/3!
    const double sn = fma(-r * r2, sp, r);
    double cp = 2.08767569878681e-09;                   // 1/12!
    cp = fma(cp, r2, -2.755731922398589e-07);           // 1/10!
    cp = fma(cp, r2, 2.48015873015873e-05);             // 1/8!
    cp = fma(cp, r2, -1.388888888888889e-03);           // 1/6!
    cp = fma(cp, r2, 4.1666666666666664e-02);           // 1/4!
    cp = fma(cp, r2, -0.5);                             // 1/2!
    const double cs = fma(cp, r2, 1.0);
    const int q = (int)((long long)k & 3);
    double s, c;
    if (q == 0) { s = sn; c = cs; }
    else if (q == 1) { s = cs; c = -sn; }
    else if (q == 2) { s = -sn; c = -cs; }
    else { s = -cs; c = sn; }
    *s_out = (float)s;
    *c_out = (float)c;
}

template <int DT, int LP>
__global__ __launch_bounds__(256) void k_qkv(QkvArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t task = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (task >= a.tasks) return;                        // whole wave exits
    const int64_t t = task / a.groups;
    const int hg = (int)(task - t * a.groups);

    constexpr int HPW = 64 / LP;
    const int NH = a.Hq + 2 * a.Hkv;
    const int D = a.D;
    const int L = D >> 4;                               // lanes with data per head
    const int head = hg * HPW + lane / LP;
    const int j = lane & (LP - 1);
    const bool active = (j < L) && (head < NH);
    const bool is_q = head < a.Hq;
    const bool is_v = head >= a.Hq + a.Hkv;

    // Token metadata (uniform across the wave).
    const int pos = a.pos[t];
    int64_t slot = -1;
    if (pos >= 0) {
        const int idx = pos / a.page_size;
        if (idx < a.table_len) {
            const int page = a.table[idx];
            if (page >= 0 && page < a.num_pages)
                slot = (int64_t)page * a.page_size + pos % a.page_size;
        }
    }
    if (slot < 0 && hg == 0 && lane == 0 && a.err != nullptr)
        __hip_atomic_fetch_or(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    const int64_t row_bytes = (int64_t)NH * D * 2;
    const char* src = (const char*)a.qkv + t * row_bytes + (int64_t)head * D * 2;
    const int off0 = j * 16;                 // bytes of chunk j, first half
    const int off1 = D + j * 16;             // bytes of chunk j, second half

    u32x4 c0 = {0, 0, 0, 0}, c1 = {0, 0, 0, 0}, w0 = {0, 0, 0, 0}, w1 = {0, 0, 0, 0};
    const void* nwp = is_q ? a.qw : a.kw;
    const bool has_norm = !is_v && nwp != nullptr;
    if (active) {
        c0 = ld128(src + off0);
        c1 = ld128(src + off1);
        if (has_norm) {
            w0 = ld128((const char*)nwp + off0);
            w1 = ld128((const char*)nwp + off1);
        }
    }

    if (is_v) {
        if (active && slot >= 0) {
            char* dst = (char*)a.vc + (slot * a.Hkv + (head - a.Hq - a.Hkv)) * (int64_t)D * 2;
            st128(dst + off0, c0);
            st128(dst + off1, c1);
        }
    }

    float v[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = lo16<DT>(c0[e]);
        v[2 * e + 1] = hi16<DT>(c0[e]);
        v[8 + 2 * e] = lo16<DT>(c1[e]);
        v[8 + 2 * e + 1] = hi16<DT>(c1[e]);
    }

    // Per-head RMSNorm over D (all lanes take part in the reduction; lanes
    // without data contribute zero).
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ss = fmaf(v[e], v[e], ss);
    ss = group_reduce<LP>(ss, OpSum());
    if (has_norm) {
        const float rstd = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = v[2 * e] * rstd * lo16<DT>(w0[e]);
            v[2 * e + 1] = v[2 * e + 1] * rstd * hi16<DT>(w0[e]);
            v[8 + 2 * e] = v[8 + 2 * e] * rstd * lo16<DT>(w1[e]);
            v[8 + 2 * e + 1] = v[8 + 2 * e + 1] * rstd * hi16<DT>(w1[e]);
        }
    }

    if (!active || is_v) return;

    // RoPE.  Frequency index of each pair held by this lane:
    //   rotate-half: pair e (e < 8) = elements (8j+e, D/2+8j+e), i = 8j+e
    //   interleaved: pair m of chunk 0 = (8j+2m, 8j+2m+1), i = 4j+m;
    //                pair m of chunk 1 = (D/2+8j+2m, ...),  i = D/4+4j+m.
    const double l2t = log2((double)a.theta);
    const double step = exp2(-2.0 / (double)D * l2t);          // theta^(-2/D)
    const double p = (double)pos;
    float sn[8], cs[8];
    if (a.style == 0) {
        double f = exp2(-(double)(2 * 8 * j) / (double)D * l2t);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sincos_pos(p * f, &sn[e], &cs[e]);
            f *= step;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x0 = v[e], x1 = v[8 + e];
            v[e] = fmaf(x0, cs[e], -x1 * sn[e]);
            v[8 + e] = fmaf(x1, cs[e], x0 * sn[e]);
        }
    } else {
        double f0 = exp2(-(double)(2 * 4 * j) / (double)D * l2t);
        double f1 = exp2(-(double)(2 * (D / 4 + 4 * j)) / (double)D * l2t);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            sincos_pos(p * f0, &sn[m], &cs[m]);
            sincos_pos(p * f1, &sn[4 + m], &cs[4 + m]);
            f0 *= step;
            f1 *= step;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float x0 = v[2 * m], x1 = v[2 * m + 1];
            v[2 * m] = fmaf(x0, cs[m], -x1 * sn[m]);
            v[2 * m + 1] = fmaf(x1, cs[m], x0 * sn[m]);
            x0 = v[8 + 2 * m];
            x1 = v[8 + 2 * m + 1];
            v[8 + 2 * m] = fmaf(x0, cs[4 + m], -x1 * sn[4 + m]);
            v[8 + 2 * m + 1] = fmaf(x1, cs[4 + m], x0 * sn[4 + m]);
        }
    }

    u32x4 o0, o1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        o0[e] = pack16<DT>(v[2 * e], v[2 * e + 1]);
        o1[e] = pack16<DT>(v[8 + 2 * e], v[8 + 2 * e + 1]);
    }
    char* dst;
    if (is_q) {
        dst = (char*)a.q_out + ((t * a.Hq + head) * (int64_t)D) * 2;
    } else {
        if (slot < 0) return;
        dst = (char*)a.kc + (slot * a.Hkv + (head - a.Hq)) * (int64_t)D * 2;
    }
    st128(dst + off0, o0);
    st128(dst + off1, o1);
}

template <int DT>
static hipError_t launch_qkv_dt(const QkvArgs& a, int lp, hipStream_t s) {
    const void* fn;
    switch (lp) {
    case 1: fn = (const void*)k_qkv<DT, 1>; break;
    case 2: fn = (const void*)k_qkv<DT, 2>; break;
    case 4: fn = (const void*)k_qkv<DT, 4>; break;
    case 8: fn = (const void*)k_qkv<DT, 8>; break;
    default: fn = (const void*)k_qkv<DT, 16>; break;
    }
    QkvArgs copy = a;
    void* args[] = {&copy};
    const unsigned blocks = (unsigned)((a.tasks + 3) / 4);
    return hipLaunchKernel(fn, dim3(blocks), dim3(256), args, 0, s);
}

hipError_t launch_qkv(const QkvArgs& in, int dtype, hipStream_t s) {
    QkvArgs a = in;
    const int L = a.D / 16;
    int lp = 1;
    while (lp < L) lp *= 2;
    const int hpw = 64 / lp;
    const int NH = a.Hq + 2 * a.Hkv;
    a.groups = (NH + hpw - 1) / hpw;
    a.tasks = a.T * a.groups;
    return dtype == DT_BF16 ? launch_qkv_dt<DT_BF16>(a, lp, s)
                            : launch_qkv_dt<DT_F16>(a, lp, s);
}

}  // namespace fr
