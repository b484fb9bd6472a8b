// fr_qkv.hip -- packed QKV split + per-head Q/K RMSNorm + RoPE + paged
// KV-cache write (op b), one kernel.
//
// Definitions: "FlashRT cross-layer fusion" article, section 二 (table step 3:
// QKV split + RoPE + KV-cache write in one kernel; 2.2: q_norm -> RoPE -> Q,
// k_norm -> RoPE -> KV cache in one kernel, V passed through, RoPE pairs kept
// in one lane so no cross-lane shuffle is needed) and the "Falcon-Perception
// inference engine" article (paged KV cache written by the decode step).
//
// Mapping: a wave64 handles one token and `gpw` groups of 64/LP heads; LP
// lanes (a power of two >= D/16) serve one head.  Lane j of a head holds the
// 16-byte chunk j of the first half of the head and chunk j of the second
// half, so each rotate-half pair (i, i+D/2) -- and each interleaved pair
// (2i, 2i+1) -- sits in one lane's registers.  Each group's loads are issued
// while the previous group is processed.  The wave index is uniform
// (readfirstlane), so the token's position and page-table entry are scalar
// loads (through the scalar cache, after the first row loads, so their
// dependent chain does not queue behind them), and the row arithmetic runs
// on the scalar unit.  The per-head sum of squares is a DPP reduction over
// the LP lanes, and rstd the hardware reciprocal square root.  The D/2
// rotation angles of the token are shared by every head: the wave computes
// each of them once (one or two per lane) into a per-wave LDS table, then
// every lane reads the cos/sin of its own pairs.  Angles are formed in fp64:
// theta^(-2i/D) = 2^(i * step) with step = -2 log2(theta) / D computed on
// the host, times the position, reduced modulo pi/2 by a two-constant
// Cody-Waite step with fma; sine and cosine come from Taylor polynomials on
// [-pi/4, pi/4], so the angle stays exact to ~1e-15 for any int32 position.
// The RoPE layout is a template parameter.
#include "fr_device.h"
#include "fr_launch.h"

namespace fr {

constexpr int kQkvMaxGroups = 8;   // head groups one wave may take

// NT: non-temporal loads of the packed rows and stores of Q, K and V (used
// in the bandwidth regime, where nothing is re-read soon).
template <int DT, int LP, bool NT, int STYLE, bool NTS = NT>
__global__ __launch_bounds__(256) void k_qkv(QkvArgs a) {
    __shared__ float tab[4][2][128];                     // per-wave cos / sin

    // Every kernel argument the kernel reads, consumed here so that they are
    // fetched in one batch of scalar loads (one memory trip) rather than in
    // dependent batches as each is first needed; the arguments span three
    // scalar-cache lines, and at a handful of tokens each trip is a visible
    // share of the kernel's time.
    asm volatile("" ::"s"(a.qkv), "s"(a.qw), "s"(a.kw), "s"(a.pos), "s"(a.table),
                 "s"(a.q_out), "s"(a.kc), "s"(a.vc), "s"(a.err), "s"(a.tasks), "s"(a.Hq),
                 "s"(a.Hkv), "s"(a.D), "s"(a.groups), "s"(a.gpw), "s"(a.wpt),
                 "s"(a.table_len), "s"(a.page_size), "s"(a.num_pages), "s"(a.eps),
                 "s"(a.q_scale), "s"(a.l2t), "s"(a.inv_d));

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t task = (int64_t)blockIdx.x * 4 + wv;
    if (task >= a.tasks) return;                         // whole wave exits
    const int64_t t = task / a.wpt;                      // token
    const int g0 = (int)(task - t * a.wpt) * a.gpw;      // first head group
    const int ng = min(a.gpw, a.groups - g0);            // groups of this wave

    constexpr int HPW = 64 / LP;
    const int NH = a.Hq + 2 * a.Hkv;
    const int D = a.D;
    const int L = D >> 4;                                // lanes with data per head
    const int j = lane & (LP - 1);
    const int hl = lane / LP;                            // head within a group

    // Head group g of this wave: its chunks are loaded one group ahead of
    // the group being processed.  Every lane loads (lanes past the row's
    // heads or past D/16 re-read a valid chunk and store nothing): a load
    // that some waves skip makes the compiler wait for every outstanding
    // load, the prefetch included, before each group.
    const char* rowp = (const char*)a.qkv + t * (int64_t)NH * D * 2;
    const int off0 = j * 16;                 // bytes of chunk j, first half
    const int off1 = D + j * 16;             // bytes of chunk j, second half
    const int jc = min(j, L - 1);
    auto load_group = [&](int g, u32x4& x0, u32x4& x1) {          // g < ng
        const int head = min((g0 + g) * HPW + hl, NH - 1);
        const char* src = rowp + (int64_t)head * D * 2 + jc * 16;
        x0 = NT ? ld128_stream(src) : ld128(src);
        x1 = NT ? ld128_stream(src + D) : ld128(src + D);
    };
    // Token metadata.  Small batches (latency: each wave's chain of memory
    // trips is its time) issue it before the row as vector loads, which
    // complete in order, so waiting for them does not wait for the row and
    // a wait for a kernel argument does not wait for them: the position
    // (the same word in every lane) and the first 64 page-table entries
    // (entry i in lane i; the table holds at least one), so that for tables
    // of up to 64 entries the slot needs no second trip once the position is
    // known.  Large batches (bandwidth) read the position and then its page
    // entry through the scalar cache, which adds no vector loads per wave.
    typedef const __attribute__((address_space(4))) int32_t* cptr;
    int posv = 0, tv = 0;
    if constexpr (!NT) {
        int z;                                           // 0, opaque to the compiler,
        asm volatile("v_mov_b32 %0, 0" : "=v"(z));       // so the load stays a vector load
        posv = a.pos[t + z];
        tv = a.table[min(lane, a.table_len - 1)];
    }

    u32x4 n0, n1;
    load_group(0, n0, n1);
    u32x4 qw0 = {0, 0, 0, 0}, qw1 = qw0, kw0 = qw0, kw1 = qw0;
    if (j < L) {
        if (a.qw) { qw0 = ld128((const char*)a.qw + off0); qw1 = ld128((const char*)a.qw + off1); }
        if (a.kw) { kw0 = ld128((const char*)a.kw + off0); kw1 = ld128((const char*)a.kw + off1); }
    }

    int pos;
    int64_t slot = -1;
    auto page_slot = [&](int page) {
        if (page >= 0 && page < a.num_pages) slot = (int64_t)page * a.page_size + pos % a.page_size;
    };
    float* cs_tab = tab[wv][0];
    float* sn_tab = tab[wv][1];
    if constexpr (NT) {
        pos = *((cptr)(uintptr_t)a.pos + t);
        if (pos >= 0) {
            const int idx = pos / a.page_size;
            if (idx < a.table_len) page_slot(*((cptr)(uintptr_t)a.table + idx));
        }
        // cos/sin table of the token: angle i = pos * theta^(-2i/D), i < D/2.
        for (int i = lane; i < (D >> 1); i += 64) {
            const double f = exp2((double)i * a.l2t);
            float sv, cv;
            sincos_pos((double)pos * f, &sv, &cv);
            cs_tab[i] = cv;
            sn_tab[i] = sv;
        }
    } else {
        // Rotation frequencies theta^(-2i/D) of this lane's angles i = lane
        // and lane + 64 (D/2 <= 128): they do not depend on the token, so
        // they are computed while its position is in flight; then both
        // angles at once (two independent fp64 chains), then the stores.
        double fq[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) fq[k] = exp2((double)(lane + 64 * k) * a.l2t);
        asm volatile("" ::"v"(fq[0]), "v"(fq[1]));      // computed here, not sunk
        pos = __builtin_amdgcn_readfirstlane(posv);
        float sv[2], cv[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) sincos_pos((double)pos * fq[k], &sv[k], &cv[k]);
        asm volatile("" ::"v"(sv[0]), "v"(sv[1]), "v"(cv[0]), "v"(cv[1]));
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int i = lane + 64 * k;
            if (i < (D >> 1)) {
                cs_tab[i] = cv[k];
                sn_tab[i] = sv[k];
            }
        }
        if (pos >= 0) {
            const int idx = pos / a.page_size;
            if (idx < a.table_len)
                page_slot(idx < 64 ? __builtin_amdgcn_readlane(tv, idx)
                                   : *((cptr)(uintptr_t)a.table + idx));
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (slot < 0 && g0 == 0 && lane == 0 && a.err != nullptr)
        __hip_atomic_fetch_or(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // This lane's pairs: rotate-half pair e = (8j+e, D/2+8j+e) turns by
    // angle 8j+e; interleaved pair m of chunk 0 = (8j+2m, 8j+2m+1) by angle
    // 4j+m, pair m of chunk 1 by angle D/4+4j+m.
    float cs[8], sn[8];
    if (j < L) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int i = STYLE == 0 ? 8 * j + e
                                       : (e < 4 ? 4 * j + e : (D >> 2) + 4 * j + (e - 4));
            cs[e] = cs_tab[i];
            sn[e] = sn_tab[i];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] = sn[e] = 0.0f;
    }

    auto process = [&](int g, const u32x4 c0, const u32x4 c1) {
        const int head = (g0 + g) * HPW + hl;
        const bool active = (j < L) && (head < NH);
        const bool is_q = head < a.Hq;
        const bool is_v = head >= a.Hq + a.Hkv;

        if (is_v) {
            if (active && slot >= 0) {
                char* dst = (char*)a.vc + (slot * a.Hkv + (head - a.Hq - a.Hkv)) * (int64_t)D * 2;
                if constexpr (NTS) {
                    st128_stream(dst + off0, c0);
                    st128_stream(dst + off1, c1);
                } else {
                    st128(dst + off0, c0);
                    st128(dst + off1, c1);
                }
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

        // Per-head RMSNorm over D (every lane takes part in the reduction;
        // lanes without data contribute zero).
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) ss = fmaf(v[e], v[e], ss);
        if (j >= L) ss = 0.0f;                           // padding lanes hold a re-read chunk
        ss = group_reduce<LP>(ss, OpSum());
        const bool has_norm = !is_v && (is_q ? a.qw : a.kw) != nullptr;
        if (has_norm) {
            const u32x4 w0 = is_q ? qw0 : kw0, w1 = is_q ? qw1 : kw1;
            const float rstd = __builtin_amdgcn_rsqf(fmaf(ss, a.inv_d, a.eps));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = v[2 * e] * rstd * lo16<DT>(w0[e]);
                v[2 * e + 1] = v[2 * e + 1] * rstd * hi16<DT>(w0[e]);
                v[8 + 2 * e] = v[8 + 2 * e] * rstd * lo16<DT>(w1[e]);
                v[8 + 2 * e + 1] = v[8 + 2 * e + 1] * rstd * hi16<DT>(w1[e]);
            }
        }
        if (!active || is_v) return;

        if constexpr (STYLE == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x0 = v[e], x1 = v[8 + e];
                v[e] = fmaf(x0, cs[e], -x1 * sn[e]);
                v[8 + e] = fmaf(x1, cs[e], x0 * sn[e]);
            }
        } else {
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

        // attention's Q pre-scale (exact for K: a multiply by 1)
        if (a.q_scale != 1.0f) {                         // uniform
            const float qs = is_q ? a.q_scale : 1.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] *= qs;
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
        if constexpr (NTS) {
            st128_stream(dst + off0, o0);
            st128_stream(dst + off1, o1);
        } else {
            st128(dst + off0, o0);
            st128(dst + off1, o1);
        }
    };

#pragma unroll 1
    for (int g = 0; g + 1 < ng; ++g) {                   // uniform trip count
        const u32x4 c0 = n0, c1 = n1;
        load_group(g + 1, n0, n1);
        process(g, c0, c1);
    }
    process(ng - 1, n0, n1);
}

template <int DT, bool NT, int STYLE>
static const void* pick_qkv(int lp) {
    switch (lp) {
    case 1: return (const void*)k_qkv<DT, 1, NT, STYLE>;
    case 2: return (const void*)k_qkv<DT, 2, NT, STYLE>;
    case 4: return (const void*)k_qkv<DT, 4, NT, STYLE>;
    case 8: return (const void*)k_qkv<DT, 8, NT, STYLE>;
    default: return (const void*)k_qkv<DT, 16, NT, STYLE>;
    }
}

template <int DT, bool NT>
static hipError_t launch_qkv_dt(const QkvArgs& a, int lp, hipStream_t s) {
    const void* fn = a.style == 0 ? pick_qkv<DT, NT, 0>(lp) : pick_qkv<DT, NT, 1>(lp);
    QkvArgs copy = a;
    void* args[] = {&copy};
    const unsigned blocks = (unsigned)((a.tasks + 3) / 4);
    return hipLaunchKernel(fn, dim3(blocks), dim3(256), args, 0, s);
}

// Head groups per wave.  In the bandwidth regime (T >= 2048) a token's groups
// are split over two waves, so each wave's angles serve several groups and
// consecutive groups' loads overlap, with non-temporal streaming; measured
// on MI355X at T = 8192 (32/8 heads x 128, 6 groups): 3 groups per wave
// 68-69% of 8 TB/s, 2 per wave 66%, 1 or 6 per wave 60%; cacheable stores
// 63%.  A kernel with this op's loads and stores and no arithmetic reaches
// 72.5% at 8192 tokens and 67% at 4096 (the same bytes as one plain copy
// stream: 77% and 71%).  Small batches give each group its own wave,
// trading repeated angle work for parallelism, and keep outputs cacheable.
hipError_t launch_qkv(const QkvArgs& in, int dtype, hipStream_t s) {
    QkvArgs a = in;
    a.l2t = -2.0 * log2((double)a.theta) / (double)a.D;   // exponent step per pair
    a.inv_d = 1.0f / (float)a.D;
    const int L = a.D / 16;
    int lp = 1;
    while (lp < L) lp *= 2;
    const int hpw = 64 / lp;
    const int NH = a.Hq + 2 * a.Hkv;
    const bool big = a.T >= 2048;
    a.groups = (NH + hpw - 1) / hpw;
    if (big) {
        a.gpw = (a.groups + 1) / 2;
        if (a.gpw > kQkvMaxGroups) a.gpw = kQkvMaxGroups;
    } else {
        a.gpw = 1;
    }
    a.wpt = (a.groups + a.gpw - 1) / a.gpw;
    a.tasks = a.T * a.wpt;
    if (dtype == DT_BF16)
        return big ? launch_qkv_dt<DT_BF16, true>(a, lp, s) : launch_qkv_dt<DT_BF16, false>(a, lp, s);
    return big ? launch_qkv_dt<DT_F16, true>(a, lp, s) : launch_qkv_dt<DT_F16, false>(a, lp, s);
}

}  // namespace fr
