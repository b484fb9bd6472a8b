// fr_chain.hip -- the small-batch decoder-step chain as one persistent kernel.
//
// Definitions: "FlashFormer: Whole-Model Kernels for Efficient Low-Batch
// Inference", abstract (one long-lived kernel for the whole forward pass to
// remove launch overhead at low batch); "FlashRT cross-layer fusion" article,
// sections 一 and 三 (at 10 tokens the decoder runs 18 layers x 10 flow steps
// of gate + residual + AdaRMSNorm + FP8, with QKV post-processing per layer,
// and launch count dominates).
//
// Every output location of the chain belongs to one wave (or, for rows
// wider than 512 values, one group of four waves) for the whole chain: row
// t's waves run op (a') on token row t for every op n = s L + l in order;
// each further wave owns a fixed set of (token, head) units and runs op (b)
// on them for every op in order.  The only value one op hands to the next
// is the residual row, and it stays in the registers of its row waves (it is
// still stored, as each op's output).  So program order within each wave is all
// the ordering the chain needs, apart from the sum of squares that a row's
// waves exchange per op inside their own workgroup: no grid-wide
// synchronisation (nothing can deadlock).  What remains serial is the
// residual hand-off of each row; every input load is independent of it, so
// each wave keeps the inputs of its next few ops in flight in a register
// ring and the chain runs at the speed of the arithmetic rather than of
// memory latency.  Rotation angles and KV slots are fixed for the chain and
// computed once per lane.  The arithmetic of each op is the one of its own
// kernel: round-to-odd residual, fp64 sum of squares, fp32 modulation, e4m3
// with a static multiplier; fp64 angles, RoPE in fp32, one rounding.
#include "fr_device.h"
#include "fr_launch.h"

namespace fr {

// Row waves: the inputs of op (a') for the next PA ops sit in a register
// ring (slot d holds op n with n % PA == d), refilled as each op retires, so
// only the residual hand-off is serial.  Unit waves: likewise PB ops deep.
// FULL: every lane's chunks are inside the row (H = 512 for one wave of
// 8-value chunks, 1024 for four waves of 4-value chunks), so the stores
// need no guard and consecutive ops form one basic block the compiler can
// interleave.
//
// NWR > 1: a row is split over NWR waves (wave part p takes the 64-chunk
// blocks NWR k + p), which divides each wave's work per op, the serial part
// of the chain.  The row's waves add their fp64 partial sums through LDS
// behind a barrier, so row waves get workgroups of their own (4 / NWR rows
// each; spare rows' waves run the same ops on a duplicate row and store
// nothing, so every barrier is reached by all four waves), and the unit
// waves follow in further workgroups.
// CW: 32-bit words per lane chunk (4: 8 values, 16-byte loads; 2: 4 values,
// 8-byte loads, for rows split over four waves).
template <int W> struct ChunkT;
template <> struct ChunkT<4> {
    typedef u32x4 type;
    static __device__ __forceinline__ type ld(const void* p) { return ld128(p); }
    static __device__ __forceinline__ void st(void* p, type v) { st128(p, v); }
};
template <> struct ChunkT<2> {
    typedef u32x2 type;
    static __device__ __forceinline__ type ld(const void* p) {
        return *reinterpret_cast<const u32x2*>(p);
    }
    static __device__ __forceinline__ void st(void* p, type v) { st64(p, v); }
};

template <int DT, int CPL, int LP, int PA, int PB, bool FULL, int NWR, int CW = 4>
__global__ __launch_bounds__(256) void k_chain(ChainArgs a) {
    constexpr int WGW = 4;                               // waves per workgroup
    typedef ChunkT<CW> Ch;
    typedef typename Ch::type chunk;
    constexpr int RPW = WGW / NWR;                       // rows per row workgroup
    __shared__ double red[2][WGW];                       // [op parity][wave]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int T = a.T, H = a.H, D = a.D;
    const int N = a.layers * a.steps;
    const int64_t rowb = (int64_t)H * 2;                 // bytes per 16-bit row
    const int64_t step_rows = (int64_t)T * rowb;         // one op's [T,H] in bytes
    const int row_wgs = NWR == 1 ? 0 : (T + RPW - 1) / RPW;   // workgroups of row waves
    const bool row_wave = NWR == 1 ? blockIdx.x * WGW + wave < T : (int)blockIdx.x < row_wgs;
    // unit-wave index (op (b) waves are numbered after the row waves)
    const int ug = NWR == 1 ? blockIdx.x * WGW + wave - T
                            : ((int)blockIdx.x - row_wgs) * WGW + wave;

    if (row_wave) {
        // ---------------- row wave: op (a') for row t, every op ----------
        const int t_raw = NWR == 1 ? blockIdx.x * WGW + wave : blockIdx.x * RPW + wave / NWR;
        const bool row_ok = t_raw < T;
        const int t = row_ok ? t_raw : T - 1;            // in-bounds duplicate
        const int part = NWR == 1 ? 0 : wave % NWR;      // this wave's share of the row
        const int C = H / (2 * CW);                      // chunks per row
        int cc[CPL];
        bool ok[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int c = (k * NWR + part) * 64 + lane;
            ok[k] = FULL || c < C;
            cc[k] = min(c, C - 1) * (4 * CW);            // byte offset of the chunk
        }
        chunk rres[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) rres[k] = Ch::ld((const char*)a.res + t * rowb + cc[k]);

        chunk xv[PA][CPL], gv[PA][CPL], sv[PA][CPL], hv[PA][CPL];
        auto fetch = [&](int d, int n) {
            const int l = n % a.layers;
            const char* xr = (const char*)a.x + l * step_rows + t * rowb;
            const int64_t nr = (int64_t)n * step_rows + t * rowb;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                xv[d][k] = Ch::ld(xr + cc[k]);
                gv[d][k] = Ch::ld((const char*)a.gate + nr + cc[k]);
                sv[d][k] = Ch::ld((const char*)a.ada_scale + nr + cc[k]);
                hv[d][k] = Ch::ld((const char*)a.ada_shift + nr + cc[k]);
            }
        };
        auto op = [&](int d, int n) {
            const int64_t nr = (int64_t)n * step_rows + t * rowb;
            double ss = 0.0;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                double c0 = 0.0, c1 = 0.0;
#pragma unroll
                for (int e = 0; e < CW; ++e) {
                    const float h0 = add_round_odd(lo16<DT>(rres[k][e]),
                                                   lo16<DT>(gv[d][k][e]) * lo16<DT>(xv[d][k][e]));
                    const float h1 = add_round_odd(hi16<DT>(rres[k][e]),
                                                   hi16<DT>(gv[d][k][e]) * hi16<DT>(xv[d][k][e]));
                    const u32 b = pack16<DT>(h0, h1);
                    rres[k][e] = b;
                    const double r0 = (double)lo16<DT>(b), r1 = (double)hi16<DT>(b);
                    c0 = fma(r0, r0, c0);
                    c1 = fma(r1, r1, c1);
                }
                if (ok[k]) {
                    ss += c0 + c1;
                    if (row_ok) Ch::st((char*)a.res + nr + step_rows + cc[k], rres[k]);
                }
            }
            ss = wave_sum_d(ss);
            if constexpr (NWR > 1) {
                // the rest of the row; every wave of the row adds the
                // partials in the same order, so all get the same rstd
                if (lane == 0) red[n & 1][wave] = ss;
                __syncthreads();
                const int base = wave & ~(NWR - 1);
                ss = red[n & 1][base];
#pragma unroll
                for (int w = 1; w < NWR; ++w) ss += red[n & 1][base + w];
            }
            const float rstd = (float)rsqrt_d(ss * (1.0 / (double)H) + (double)a.eps);
            const float mult = a.static_scale;
            uint8_t* orow = a.out + (int64_t)n * T * H + (int64_t)t * H;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                float y[2 * CW];
#pragma unroll
                for (int e = 0; e < CW; ++e) {
                    const float n0 = lo16<DT>(rres[k][e]) * rstd;
                    const float n1 = hi16<DT>(rres[k][e]) * rstd;
                    y[2 * e] = fmaf(n0, 1.0f + lo16<DT>(sv[d][k][e]), lo16<DT>(hv[d][k][e]));
                    y[2 * e + 1] = fmaf(n1, 1.0f + hi16<DT>(sv[d][k][e]), hi16<DT>(hv[d][k][e]));
                }
                if (ok[k] && row_ok) {
                    if constexpr (CW == 4) {
                        u32x2 q;
                        q.x = pack_e4m3x4(y[0] * mult, y[1] * mult, y[2] * mult, y[3] * mult);
                        q.y = pack_e4m3x4(y[4] * mult, y[5] * mult, y[6] * mult, y[7] * mult);
                        st64(orow + cc[k] / 2, q);
                    } else {
                        *reinterpret_cast<u32*>(orow + cc[k] / 2) =
                            pack_e4m3x4(y[0] * mult, y[1] * mult, y[2] * mult, y[3] * mult);
                    }
                }
            }
        };
#pragma unroll
        for (int d = 0; d < PA; ++d) fetch(d, min(d, N - 1));
        const int M = N - N % PA;                        // ops of the main loop
        for (int n0 = 0; n0 < M; n0 += PA) {
#pragma unroll
            for (int d = 0; d < PA; ++d) {
                op(d, n0 + d);
                fetch(d, min(n0 + d + PA, N - 1));       // past the end: unused
            }
        }
#pragma unroll
        for (int d = 0; d < PA; ++d)                     // the last N % PA ops
            if (d < N - M) op(d, M + d);
        return;
    }

    // ---------------- unit wave: op (b) for HPW fixed (token, head) units ---
    constexpr int HPW = 64 / LP;
    const int NH = a.Hq + 2 * a.Hkv;
    const int u = ug * HPW + lane / LP;
    const int j = lane & (LP - 1);
    if (u >= T * NH || j >= (D >> 4)) return;            // lanes without work
    const int t = u / NH, head = u - t * NH;
    const bool is_q = head < a.Hq, is_v = head >= a.Hq + a.Hkv;
    const int off0 = j * 16, off1 = D + j * 16;

    // KV slot of the token
    long long slot = -1;
    {
        const int p = a.pos[t];
        if (p >= 0) {
            const int idx = p / a.page_size;
            if (idx < a.table_len) {
                const int page = a.table[idx];
                if (page >= 0 && page < a.num_pages)
                    slot = (long long)page * a.page_size + p % a.page_size;
            }
        }
        if (slot < 0 && head == 0 && j == 0 && a.err != nullptr)
            __hip_atomic_fetch_or(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!is_q && slot < 0) return;                       // nothing to write

    // this lane's 8 rotation angles (rotate-half: pairs 8j+e; interleaved:
    // pairs 4j+m and D/4+4j+m), in fp64 once for the whole chain
    float cs[8], sn[8];
    if (!is_v) {
        const double l2t = log2((double)a.theta);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = a.style == 0 ? 8 * j + e : (e < 4 ? 4 * j + e : (D >> 2) + 4 * j + (e - 4));
            const double f = exp2(-(double)(2 * i) / (double)D * l2t);
            sincos_pos((double)a.pos[t] * f, &sn[e], &cs[e]);
        }
    }

    const int64_t qkv_row = (int64_t)NH * D * 2;
    const int64_t qkv_l = (int64_t)T * qkv_row;
    const int64_t cache_l = (int64_t)a.num_pages * a.page_size * a.Hkv * D * 2;
    const char* src0 = (const char*)a.qkv + t * qkv_row + (int64_t)head * D * 2;
    char* dst0;
    int64_t dst_l;
    if (is_q) {
        dst0 = (char*)a.q_out + ((int64_t)t * a.Hq + head) * D * 2;
        dst_l = (int64_t)T * a.Hq * D * 2;
    } else if (is_v) {
        dst0 = (char*)a.vc + (slot * a.Hkv + (head - a.Hq - a.Hkv)) * (int64_t)D * 2;
        dst_l = cache_l;
    } else {
        dst0 = (char*)a.kc + (slot * a.Hkv + (head - a.Hq)) * (int64_t)D * 2;
        dst_l = cache_l;
    }

    u32x4 c0[PB], c1[PB];
    auto fetch = [&](int d, int n) {
        const char* src = src0 + (n % a.layers) * qkv_l;
        c0[d] = ld128(src + off0);
        c1[d] = ld128(src + off1);
    };
    auto op = [&](int d, int n) {
        char* dst = dst0 + (n % a.layers) * dst_l;
        if (is_v) {
            st128(dst + off0, c0[d]);
            st128(dst + off1, c1[d]);
            return;
        }
        float v[16];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = lo16<DT>(c0[d][e]);
            v[2 * e + 1] = hi16<DT>(c0[d][e]);
            v[8 + 2 * e] = lo16<DT>(c1[d][e]);
            v[8 + 2 * e + 1] = hi16<DT>(c1[d][e]);
        }
        if (a.style == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x0 = v[e], x1 = v[8 + e];
                v[e] = fmaf(x0, cs[e], -x1 * sn[e]);
                v[8 + e] = fmaf(x1, cs[e], x0 * sn[e]);
            }
        } else {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int b = m < 4 ? 2 * m : 8 + 2 * (m - 4);
                const float x0 = v[b], x1 = v[b + 1];
                v[b] = fmaf(x0, cs[m], -x1 * sn[m]);
                v[b + 1] = fmaf(x1, cs[m], x0 * sn[m]);
            }
        }
        u32x4 o0, o1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o0[e] = pack16<DT>(v[2 * e], v[2 * e + 1]);
            o1[e] = pack16<DT>(v[8 + 2 * e], v[8 + 2 * e + 1]);
        }
        st128(dst + off0, o0);
        st128(dst + off1, o1);
    };
#pragma unroll
    for (int d = 0; d < PB; ++d) fetch(d, min(d, N - 1));
    const int M = N - N % PB;
    for (int n0 = 0; n0 < M; n0 += PB) {
#pragma unroll
        for (int d = 0; d < PB; ++d) {
            op(d, n0 + d);
            fetch(d, min(n0 + d + PB, N - 1));
        }
    }
#pragma unroll
    for (int d = 0; d < PB; ++d)
        if (d < N - M) op(d, M + d);
}

constexpr int kChainPA = 4;      // op (a') inputs in flight per row wave
constexpr int kChainPB = 8;      // op (b) inputs in flight per unit wave

template <int DT, int CPL, bool FULL, int NWR, int CW>
static hipError_t launch_chain_cpl(const ChainArgs& a, int lp, hipStream_t s) {
    const void* fn;
    switch (lp) {
    case 1: fn = (const void*)k_chain<DT, CPL, 1, kChainPA, kChainPB, FULL, NWR, CW>; break;
    case 2: fn = (const void*)k_chain<DT, CPL, 2, kChainPA, kChainPB, FULL, NWR, CW>; break;
    case 4: fn = (const void*)k_chain<DT, CPL, 4, kChainPA, kChainPB, FULL, NWR, CW>; break;
    case 8: fn = (const void*)k_chain<DT, CPL, 8, kChainPA, kChainPB, FULL, NWR, CW>; break;
    default: fn = (const void*)k_chain<DT, CPL, 16, kChainPA, kChainPB, FULL, NWR, CW>; break;
    }
    const int units = a.T * (a.Hq + 2 * a.Hkv);
    const int hpw = 64 / lp;
    const int unit_waves = (units + hpw - 1) / hpw;
    // row waves, then unit waves; with several waves per row the rows fill
    // workgroups of their own (4 / NWR rows each)
    constexpr int RPW = 4 / NWR;
    const int blocks = NWR == 1 ? (a.T + unit_waves + 3) / 4
                                : (a.T + RPW - 1) / RPW + (unit_waves + 3) / 4;
    ChainArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, s);
}

// Rows of up to 512 values take one wave each (one 16-byte chunk per lane);
// wider rows (up to 1024) are split over the four waves of a workgroup (one
// 8-byte chunk per lane each), which quarters the serial work per op on the
// row's path.  Measured at 10 tokens, H = 1024 / 768, the 360-op chain:
// one wave per row 173 / 193 us, two 130 / 133 us, four 97 / 99 us, eight
// (512-thread workgroups, 4-byte chunks) 98 / 99 us: past four waves the
// reduction, barrier and the fp64 rsqrt chain of each op set its time.
template <int DT>
static hipError_t launch_chain_dt(const ChainArgs& a, int lp, hipStream_t s) {
    if (a.H <= 512)
        return a.H == 512 ? launch_chain_cpl<DT, 1, true, 1, 4>(a, lp, s)
                          : launch_chain_cpl<DT, 1, false, 1, 4>(a, lp, s);
    return a.H == 1024 ? launch_chain_cpl<DT, 1, true, 4, 2>(a, lp, s)
                       : launch_chain_cpl<DT, 1, false, 4, 2>(a, lp, s);
}

hipError_t launch_chain(const ChainArgs& a, int dtype, hipStream_t s) {
    int lp = 1;                                          // H <= kChainMaxH = 1024
    while (lp < a.D / 16) lp *= 2;
    return dtype == DT_BF16 ? launch_chain_dt<DT_BF16>(a, lp, s)
                            : launch_chain_dt<DT_F16>(a, lp, s);
}

}  // namespace fr
