// fr_chain.hip -- the small-batch decoder-step chain as one persistent kernel.
//
// Definitions: "FlashFormer: Whole-Model Kernels for Efficient Low-Batch
// Inference", abstract (one long-lived kernel for the whole forward pass to
// remove launch overhead at low batch); "FlashRT cross-layer fusion" article,
// sections 一 and 三 (at 10 tokens the decoder runs 18 layers x 10 flow steps
// of gate + residual + AdaRMSNorm + FP8, with QKV post-processing per layer,
// and launch count dominates).
//
// One workgroup of 16 waves walks the chain in order: for flow step s and
// layer l (op n = s L + l), op (a') on every token row, then op (b) on every
// (token, head) pair.  Work is assigned so that every output location
// belongs to one wave for the whole chain: row t is always handled by wave
// t % 16 and head unit u by one fixed wave.  The only value one op hands to
// the next is the residual row, and it stays in the registers of the wave
// that owns the row (it is still stored, as each op's output).  So program
// order within each wave is the whole ordering the chain needs: no barrier
// and no grid-wide synchronisation (nothing can deadlock), and waves run
// ahead into the next op while others finish.  One CU's bandwidth is enough
// for this launch- and latency-bound chain.  The rotation angles and KV
// slots of every token are computed once into LDS (positions are fixed for
// the chain).  The arithmetic of each op is the one of its own kernel:
// round-to-odd residual, fp64 sum of squares, fp32 modulation, e4m3 with a
// static multiplier; fp64 angles, RoPE in fp32, one rounding.
#include "fr_device.h"
#include "fr_launch.h"

namespace fr {

template <int DT, int CPL, int LP>
__global__ __launch_bounds__(1024) void k_chain(ChainArgs a) {
    __shared__ float tab[kChainMaxT][2][128];            // cos / sin per token
    __shared__ long long slot_of[kChainMaxT];

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int T = a.T, H = a.H, D = a.D;
    const int C = H >> 3;                                // 16-byte chunks per row
    const int half = D >> 1;

    // Angles i < D/2 of every token: pos * theta^(-2i/D), in fp64.
    {
        const double l2t = log2((double)a.theta);
        for (int i = threadIdx.x; i < T * half; i += 1024) {
            const int t = i / half, k = i - t * half;
            const double f = exp2(-(double)(2 * k) / (double)D * l2t);
            float sv, cv;
            sincos_pos((double)a.pos[t] * f, &sv, &cv);
            tab[t][0][k] = cv;
            tab[t][1][k] = sv;
        }
        for (int t = threadIdx.x; t < T; t += 1024) {
            const int p = a.pos[t];
            long long slot = -1;
            if (p >= 0) {
                const int idx = p / a.page_size;
                if (idx < a.table_len) {
                    const int page = a.table[idx];
                    if (page >= 0 && page < a.num_pages)
                        slot = (long long)page * a.page_size + p % a.page_size;
                }
            }
            slot_of[t] = slot;
            if (slot < 0 && a.err != nullptr)
                __hip_atomic_fetch_or(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();                                 // the only barrier
    }

    // Residual rows owned by this wave (rows w and w + 16), in registers.
    const int64_t rowb = (int64_t)H * 2;                 // bytes per 16-bit row
    u32x4 rres[2][CPL];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int t = w + 16 * r;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int c = min(k * 64 + lane, C - 1);
            rres[r][k] = (u32x4){0, 0, 0, 0};
            if (t < T) rres[r][k] = ld128((const char*)a.res + t * rowb + c * 16);
        }
    }

    constexpr int HPW = 64 / LP;                         // head units per wave pass
    const int NH = a.Hq + 2 * a.Hkv;
    const int units = T * NH;
    const int L16 = D >> 4;                              // lanes with data per head
    const int j = lane & (LP - 1);
    const int64_t step_rows = (int64_t)T * rowb;         // one op's [T,H] in bytes
    const int64_t qkv_row = (int64_t)NH * D * 2;
    const int64_t cache_l = (int64_t)a.num_pages * a.page_size * a.Hkv * D * 2;

    for (int s = 0; s < a.steps; ++s) {
        for (int l = 0; l < a.layers; ++l) {
            const int64_t n = (int64_t)s * a.layers + l;

            // ---- (a') gate + residual + AdaRMSNorm + FP8 (static) ----
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int t = w + 16 * r;
                if (t >= T) continue;                    // uniform in the wave
                const char* xr = (const char*)a.x + l * step_rows + t * rowb;
                const int64_t nr = n * step_rows + t * rowb;
                u32x4 xv[CPL], gv[CPL], sv[CPL], hv[CPL];
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    const int c = min(k * 64 + lane, C - 1);
                    xv[k] = ld128(xr + c * 16);
                    gv[k] = ld128((const char*)a.gate + nr + c * 16);
                    sv[k] = ld128((const char*)a.ada_scale + nr + c * 16);
                    hv[k] = ld128((const char*)a.ada_shift + nr + c * 16);
                }
                double ss = 0.0;
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    double c0 = 0.0, c1 = 0.0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float h0 = add_round_odd(lo16<DT>(rres[r][k][e]),
                                                       lo16<DT>(gv[k][e]) * lo16<DT>(xv[k][e]));
                        const float h1 = add_round_odd(hi16<DT>(rres[r][k][e]),
                                                       hi16<DT>(gv[k][e]) * hi16<DT>(xv[k][e]));
                        const u32 b = pack16<DT>(h0, h1);
                        rres[r][k][e] = b;
                        const double r0 = (double)lo16<DT>(b), r1 = (double)hi16<DT>(b);
                        c0 = fma(r0, r0, c0);
                        c1 = fma(r1, r1, c1);
                    }
                    const int c = k * 64 + lane;
                    if (c < C) {
                        ss += c0 + c1;
                        st128((char*)a.res + nr + step_rows + c * 16, rres[r][k]);
                    }
                }
                ss = wave_sum_d(ss);
                const float rstd = (float)(1.0 / sqrt(ss / (double)H + (double)a.eps));
                const float mult = a.static_scale;
                uint8_t* orow = a.out + n * (int64_t)T * H + (int64_t)t * H;
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    float y[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float n0 = lo16<DT>(rres[r][k][e]) * rstd;
                        const float n1 = hi16<DT>(rres[r][k][e]) * rstd;
                        y[2 * e] = fmaf(n0, 1.0f + lo16<DT>(sv[k][e]), lo16<DT>(hv[k][e]));
                        y[2 * e + 1] = fmaf(n1, 1.0f + hi16<DT>(sv[k][e]), hi16<DT>(hv[k][e]));
                    }
                    const int c = k * 64 + lane;
                    if (c < C) {
                        u32x2 q;
                        q.x = pack_e4m3x4(y[0] * mult, y[1] * mult, y[2] * mult, y[3] * mult);
                        q.y = pack_e4m3x4(y[4] * mult, y[5] * mult, y[6] * mult, y[7] * mult);
                        st64(orow + c * 8, q);
                    }
                }
            }

            // ---- (b) QKV split + RoPE + paged KV write (no q/k norm) ----
            const char* qkvl = (const char*)a.qkv + l * (int64_t)T * qkv_row;
            char* qo = (char*)a.q_out + l * (int64_t)T * a.Hq * D * 2;
            char* kc = (char*)a.kc + l * cache_l;
            char* vc = (char*)a.vc + l * cache_l;
            for (int u0 = w * HPW; u0 < units; u0 += kChainWaves * HPW) {
                const int u = u0 + lane / LP;
                const bool active = u < units && j < L16;
                const int uc = min(u, units - 1);
                const int t = uc / NH, head = uc - t * NH;
                const int off0 = j * 16, off1 = D + j * 16;
                u32x4 c0 = {0, 0, 0, 0}, c1 = c0;
                if (active) {
                    const char* src = qkvl + t * qkv_row + (int64_t)head * D * 2;
                    c0 = ld128(src + off0);
                    c1 = ld128(src + off1);
                }
                if (!active) continue;
                const long long slot = slot_of[t];
                if (head >= a.Hq + a.Hkv) {              // V: pass-through
                    if (slot >= 0) {
                        char* dst = vc + (slot * a.Hkv + (head - a.Hq - a.Hkv)) * (int64_t)D * 2;
                        st128(dst + off0, c0);
                        st128(dst + off1, c1);
                    }
                    continue;
                }
                float v[16];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = lo16<DT>(c0[e]);
                    v[2 * e + 1] = hi16<DT>(c0[e]);
                    v[8 + 2 * e] = lo16<DT>(c1[e]);
                    v[8 + 2 * e + 1] = hi16<DT>(c1[e]);
                }
                if (a.style == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float cs = tab[t][0][8 * j + e], sn = tab[t][1][8 * j + e];
                        const float x0 = v[e], x1 = v[8 + e];
                        v[e] = fmaf(x0, cs, -x1 * sn);
                        v[8 + e] = fmaf(x1, cs, x0 * sn);
                    }
                } else {
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        const int i = m < 4 ? 4 * j + m : (D >> 2) + 4 * j + (m - 4);
                        const int b = m < 4 ? 2 * m : 8 + 2 * (m - 4);
                        const float cs = tab[t][0][i], sn = tab[t][1][i];
                        const float x0 = v[b], x1 = v[b + 1];
                        v[b] = fmaf(x0, cs, -x1 * sn);
                        v[b + 1] = fmaf(x1, cs, x0 * sn);
                    }
                }
                u32x4 o0, o1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o0[e] = pack16<DT>(v[2 * e], v[2 * e + 1]);
                    o1[e] = pack16<DT>(v[8 + 2 * e], v[8 + 2 * e + 1]);
                }
                char* dst;
                if (head < a.Hq) {
                    dst = qo + ((int64_t)t * a.Hq + head) * D * 2;
                } else {
                    if (slot < 0) continue;
                    dst = kc + (slot * a.Hkv + (head - a.Hq)) * (int64_t)D * 2;
                }
                st128(dst + off0, o0);
                st128(dst + off1, o1);
            }
        }
    }
}

template <int DT, int CPL>
static hipError_t launch_chain_cpl(const ChainArgs& a, int lp, hipStream_t s) {
    const void* fn;
    switch (lp) {
    case 1: fn = (const void*)k_chain<DT, CPL, 1>; break;
    case 2: fn = (const void*)k_chain<DT, CPL, 2>; break;
    case 4: fn = (const void*)k_chain<DT, CPL, 4>; break;
    case 8: fn = (const void*)k_chain<DT, CPL, 8>; break;
    default: fn = (const void*)k_chain<DT, CPL, 16>; break;
    }
    ChainArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel(fn, dim3(1), dim3(64 * kChainWaves), args, 0, s);
}

template <int DT>
static hipError_t launch_chain_dt(const ChainArgs& a, int cpl, int lp, hipStream_t s) {
    return cpl == 1 ? launch_chain_cpl<DT, 1>(a, lp, s) : launch_chain_cpl<DT, 2>(a, lp, s);
}

hipError_t launch_chain(const ChainArgs& a, int dtype, hipStream_t s) {
    const int C = a.H / 8;
    const int cpl = C <= 64 ? 1 : 2;                     // H <= kChainMaxH
    int lp = 1;
    while (lp < a.D / 16) lp *= 2;
    return dtype == DT_BF16 ? launch_chain_dt<DT_BF16>(a, cpl, lp, s)
                            : launch_chain_dt<DT_F16>(a, cpl, lp, s);
}

}  // namespace fr
