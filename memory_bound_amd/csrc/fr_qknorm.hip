// fr_qknorm.hip -- packed QKV split + Q/K norm + RoPE, the variants of the
// Q/K post-processing contract, one kernel.
//
// Definitions: "FlashRT cross-layer fusion" article, section 2.2 (one
// kernel normalises Q and K and rotates them, V passes through; the
// Chameleon prefill path uses LayerNorm per head with rotate-half RoPE and
// keeps each RoPE pair in one lane; the Wan video path splits the packed
// row three ways, RMS-normalises Q and K over their full width and applies a
// 3D RoPE, in one streaming read).
//
// Mapping: one workgroup (4 waves) per token.  LP lanes (a power of two >=
// D/16) serve one head; lane j of a head holds the 16-byte chunk j of the
// first half of the head and chunk j of the second half, so every RoPE
// pair -- rotate-half (i, i + D/2) or interleaved (2i, 2i+1) -- sits in one
// lane.  The token's heads are covered in U passes of 256/LP heads, all
// loaded before any arithmetic and kept in registers, so a full-width norm
// needs no second read: each thread sums its 16 values per head in fp32,
// then a wave reduction and one LDS step add the partial sums in fp64 (so
// the total barely depends on the order).  A per-head norm is a DPP
// reduction over the head's lanes.  LayerNorm subtracts the mean first
// (two reductions).  The token's D/2 rotation angles are computed once per
// workgroup (one per thread, fp64 as in op b) into LDS and serve every
// head; 3D RoPE splits the pairs into time / height / width ranges, each
// turned by its own position.  Heads stay in registers as raw 16-bit pairs
// and are widened on use (one shift or convert each), each pass widening
// afresh, which keeps four passes of heads within 96 registers: five
// workgroups (five tokens) per CU in flight.
#include "fr_device.h"
#include "fr_launch.h"

namespace fr {

template <int DT, int LP, int U>
__global__ __launch_bounds__(256) void k_qknr(QkNormArgs a) {
    __shared__ double red[4][4];
    __shared__ float tab[2][128];                        // cos / sin of the token

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int64_t t = blockIdx.x / a.split;              // token
    const int p0 = (int)(blockIdx.x - t * a.split);      // first pass of this workgroup
    constexpr int HPB = 256 / LP;                        // heads per pass
    const int D = a.D, L16 = D >> 4;
    const int NH = a.Hq + 2 * a.Hkv;
    const int j = tid & (LP - 1);
    const int off0 = j * 16, off1 = D + j * 16;          // byte offsets in a head
    const bool lane_ok = j < L16;

    // ---- loads: every head of the token, U passes ----
    const char* rowp = (const char*)a.qkv + t * (int64_t)NH * D * 2;
    u32x4 c0[U], c1[U];
    int head[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        head[u] = (p0 + u) * HPB + tid / LP;
        c0[u] = c1[u] = (u32x4){0, 0, 0, 0};
        if (lane_ok && head[u] < NH) {
            const char* src = rowp + (int64_t)head[u] * D * 2;
            c0[u] = ld128_stream(src + off0);
            c1[u] = ld128_stream(src + off1);
        }
    }
    // the token's D/2 angles, one per thread, while the loads are in flight
    if (tid < (D >> 1)) {
        const double l2t = log2((double)a.theta);
        const int* pp = a.pos + (a.rope3 ? 3 * t : t);
        double ang;
        if (a.rope3) {
            const int i = tid;
            const int ax = i < a.sec[0] ? 0 : (i < a.sec[0] + a.sec[1] ? 1 : 2);
            const int k = i - (ax > 0 ? a.sec[0] : 0) - (ax > 1 ? a.sec[1] : 0);
            ang = (double)pp[ax] * exp2(-(double)k / (double)a.sec[ax] * l2t);
        } else {
            ang = (double)pp[0] * exp2(-(double)(2 * tid) / (double)D * l2t);
        }
        sincos_pos(ang, &tab[1][tid], &tab[0][tid]);
    }
    // value e of unit u (0..7: chunk j of the first half, 8..15: second half)
    auto val = [&](int u, int e) -> float {
        const u32 w = e < 8 ? c0[u][(e & 7) >> 1] : c1[u][(e & 7) >> 1];
        return (e & 1) ? hi16<DT>(w) : lo16<DT>(w);
    };
    auto part = [&](int h) { return h < a.Hq ? 0 : (h < a.Hq + a.Hkv ? 1 : 2); };  // Q, K, V
    // Between passes over the heads the raw registers are marked as changed,
    // so each pass widens its values afresh instead of keeping all of them
    // widened (four times the registers) from the previous pass.
    auto fence_raw = [&]() {
#pragma unroll
        for (int u = 0; u < U; ++u) asm volatile("" : "+v"(c0[u]), "+v"(c1[u]));
    };

    // ---- norm statistics (per unit: mean[u], rstd[u]) ----
    float mean[U], rstd[U];
#pragma unroll
    for (int u = 0; u < U; ++u) { mean[u] = 0.0f; rstd[u] = 1.0f; }
    if (a.norm_kind != 0) {
        const bool layer = a.norm_kind == 2;
        if (a.full) {
            // sums over all Q values and over all K values of the token
            double sq = 0.0, sk = 0.0;
            double mq = 0.0, mk = 0.0;
            if (layer) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float su = 0.0f;                     // 16 values: fp32 is ample
#pragma unroll
                    for (int e = 0; e < 16; ++e) su += val(u, e);
                    const double s = (double)su;
                    const int p = part(head[u]);
                    if (p == 0) sq += s; else if (p == 1) sk += s;
                }
                fence_raw();
                sq = wave_sum_d(sq);
                sk = wave_sum_d(sk);
                if (lane == 0) { red[wv][0] = sq; red[wv][1] = sk; }
                __syncthreads();
                mq = (red[0][0] + red[1][0] + red[2][0] + red[3][0]) * a.inv_nq;
                mk = (red[0][1] + red[1][1] + red[2][1] + red[3][1]) * a.inv_nk;
                sq = sk = 0.0;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = part(head[u]);
                const float m = (float)(p == 0 ? mq : mk);
                float su = 0.0f;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float d = val(u, e) - m;
                    su = fmaf(d, d, su);
                }
                const double s = lane_ok ? (double)su : 0.0;
                if (p == 0) sq += s; else if (p == 1) sk += s;
            }
            sq = wave_sum_d(sq);
            sk = wave_sum_d(sk);
            if (lane == 0) { red[wv][2] = sq; red[wv][3] = sk; }
            __syncthreads();
            const double vq = (red[0][2] + red[1][2] + red[2][2] + red[3][2]) * a.inv_nq;
            const double vk = (red[0][3] + red[1][3] + red[2][3] + red[3][3]) * a.inv_nk;
            const float rq = 1.0f / sqrtf((float)vq + a.eps);
            const float rk = 1.0f / sqrtf((float)vk + a.eps);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int p = part(head[u]);
                mean[u] = (float)(p == 0 ? mq : mk);
                rstd[u] = p == 0 ? rq : rk;
            }
        } else {
            // per head, over the head's LP lanes
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float m = 0.0f;
                if (layer) {
                    float s = 0.0f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) s += val(u, e);
                    m = group_reduce<LP>(s, OpSum()) / (float)D;
                }
                float ss = 0.0f;
                if (lane_ok) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float d = val(u, e) - m;
                        ss = fmaf(d, d, ss);
                    }
                }
                ss = group_reduce<LP>(ss, OpSum());
                mean[u] = m;
                rstd[u] = 1.0f / sqrtf(ss / (float)D + a.eps);
            }
        }
    }

    fence_raw();
    __syncthreads();                                     // angle table complete

    // ---- apply, rotate, store ----
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int h = head[u];
        if (!lane_ok || h >= NH) continue;
        const int p = part(h);
        char* dst;
        if (p == 2) {                                    // V: bit copy
            dst = (char*)a.v_out + (t * a.Hkv + (h - a.Hq - a.Hkv)) * (int64_t)D * 2;
            st128_stream(dst + off0, c0[u]);
            st128_stream(dst + off1, c1[u]);
            continue;
        }
        const int hl = p == 0 ? h : h - a.Hq;            // head within Q or K
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = val(u, e);
        if (a.norm_kind != 0) {
            // weights [D] shared by the heads, or this head's slice of the
            // full-width weights (cache-resident either way)
            const void* w = p == 0 ? a.qw : a.kw;
            const void* b = a.norm_kind == 2 ? (p == 0 ? a.qb : a.kb) : nullptr;
            const int64_t o = a.full ? (int64_t)hl * D * 2 : 0;
            // absent weights read as a pair of 16-bit ones, absent biases as
            // zeros, so the element loop has no selects
            const u32 one2 = DT == DT_BF16 ? 0x3F803F80u : 0x3C003C00u;
            u32x4 w0 = {one2, one2, one2, one2}, w1 = w0;
            u32x4 b0 = {0, 0, 0, 0}, b1 = b0;
            if (w) { w0 = ld128((const char*)w + o + off0); w1 = ld128((const char*)w + o + off1); }
            if (b) { b0 = ld128((const char*)b + o + off0); b1 = ld128((const char*)b + o + off1); }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const u32 ww = e < 4 ? w0[e] : w1[e - 4];
                const u32 bb = e < 4 ? b0[e] : b1[e - 4];
                const int ia = e < 4 ? 2 * e : 8 + 2 * (e - 4);
                v[ia] = fmaf((v[ia] - mean[u]) * rstd[u], lo16<DT>(ww), lo16<DT>(bb));
                v[ia + 1] = fmaf((v[ia + 1] - mean[u]) * rstd[u], hi16<DT>(ww), hi16<DT>(bb));
            }
        }
        // rotate-half: pair e = (8j+e, D/2+8j+e); interleaved: pair m of
        // chunk 0 = angle 4j+m, of chunk 1 = angle D/4+4j+m
        if (a.style == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float cs = tab[0][8 * j + e], sn = tab[1][8 * j + e];
                const float x0 = v[e], x1 = v[8 + e];
                v[e] = fmaf(x0, cs, -x1 * sn);
                v[8 + e] = fmaf(x1, cs, x0 * sn);
            }
        } else {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int i = m < 4 ? 4 * j + m : (D >> 2) + 4 * j + (m - 4);
                const int b = m < 4 ? 2 * m : 8 + 2 * (m - 4);
                const float cs = tab[0][i], sn = tab[1][i];
                const float x0 = v[b], x1 = v[b + 1];
                v[b] = fmaf(x0, cs, -x1 * sn);
                v[b + 1] = fmaf(x1, cs, x0 * sn);
            }
        }
        if (a.q_scale != 1.0f) {                         // uniform; 1 is the common case
            const float qs = p == 0 ? a.q_scale : 1.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] *= qs;
        }
        u32x4 o0, o1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o0[e] = pack16<DT>(v[2 * e], v[2 * e + 1]);
            o1[e] = pack16<DT>(v[8 + 2 * e], v[8 + 2 * e + 1]);
        }
        dst = p == 0 ? (char*)a.q_out + (t * a.Hq + hl) * (int64_t)D * 2
                     : (char*)a.k_out + (t * a.Hkv + hl) * (int64_t)D * 2;
        st128_stream(dst + off0, o0);
        st128_stream(dst + off1, o1);
        __builtin_amdgcn_sched_barrier(0);               // one unit's temporaries at a time
    }
}

template <int DT, int LP>
static hipError_t launch_qknr_lp(const QkNormArgs& a, int u, hipStream_t s) {
    const void* fn = u == 1 ? (const void*)k_qknr<DT, LP, 1>
                   : u == 2 ? (const void*)k_qknr<DT, LP, 2>
                   : u == 3 ? (const void*)k_qknr<DT, LP, 3> : (const void*)k_qknr<DT, LP, 4>;
    QkNormArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel(fn, dim3((unsigned)(a.T * a.split)), dim3(256), args, 0, s);
}

template <int DT>
static hipError_t launch_qknr_dt(const QkNormArgs& a, int lp, int u, hipStream_t s) {
    switch (lp) {
    case 1: return launch_qknr_lp<DT, 1>(a, u, s);
    case 2: return launch_qknr_lp<DT, 2>(a, u, s);
    case 4: return launch_qknr_lp<DT, 4>(a, u, s);
    case 8: return launch_qknr_lp<DT, 8>(a, u, s);
    default: return launch_qknr_lp<DT, 16>(a, u, s);
    }
}

// U: passes of 256/LP heads per workgroup; the caller guarantees NH * LP <=
// 4 * 256.  A full-width norm needs every head of the token in one
// workgroup.  A per-head norm over three or four full passes takes one pass
// of one token per workgroup instead (the angle table is then computed once
// per pass): fewer registers per wave, so more waves per SIMD.  Measured on
// MI355X, same-box A/B, outputs identical: Chameleon style (LayerNorm per
// head, 32/32 x 128 bf16, 3 passes) 69.8 -> 67.6 us and 69.4 -> 68.4 us at
// 8192 tokens on two boxes, 37.2 -> 36.3 us at 4096; with 32/8 x 128 (1.5
// passes) the split was slower, 36.2 -> 41.4 us (a half-empty second
// workgroup per token).
hipError_t launch_qknr(const QkNormArgs& in, int dtype, hipStream_t s) {
    QkNormArgs a = in;
    a.inv_nq = 1.0 / ((double)a.Hq * a.D);
    a.inv_nk = 1.0 / ((double)a.Hkv * a.D);
    int lp = 1;
    while (lp < a.D / 16) lp *= 2;
    const int NH = a.Hq + 2 * a.Hkv;
    const int passes = (NH * lp + 255) / 256;
    a.split = 1;
    int u = passes < 4 ? passes : 4;
    if (!a.full && passes >= 3 && NH * lp % 256 == 0 && a.T * passes <= 0x7fffffffLL) {
        a.split = passes;
        u = 1;
    }
    return dtype == DT_BF16 ? launch_qknr_dt<DT_BF16>(a, lp, u, s)
                            : launch_qknr_dt<DT_F16>(a, lp, u, s);
}

}  // namespace fr
