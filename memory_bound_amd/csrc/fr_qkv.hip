// fr_qkv.hip -- packed QKV split + per-head Q/K RMSNorm + RoPE + paged
// KV-cache write (op b), one kernel.
//
// Definitions: "FlashRT cross-layer fusion" article, section 二 (table step 3:
// QKV split + RoPE + KV-cache write in one kernel; 2.2: q_norm -> RoPE -> Q,
// k_norm -> RoPE -> KV cache in one kernel, V passed through, RoPE pairs kept
// in one lane so no cross-lane shuffle is needed) and the "Falcon-Perception
// inference engine" article (paged KV cache written by the decode step).
//
// Mapping: a wave64 handles one group of 64/LP heads of one token; LP lanes
// (a power of two >= D/16) serve one head.  Lane j of a head holds the
// 16-byte chunk j of the first half of the head and chunk j of the second
// half, so each rotate-half pair (i, i+D/2) -- and each interleaved pair
// (2i, 2i+1) -- sits in one lane's registers.  The wave index is uniform
// (readfirstlane), so the token's position and page-table entry are scalar
// loads (through the scalar cache, after the first row loads, so their
// dependent chain does not queue behind them), and the row arithmetic runs
// on the scalar unit.  The per-head sum of squares is a DPP reduction over
// the LP lanes, and rstd the hardware reciprocal square root.  The D/2
// rotation angles of the token are shared by every head: the wave computes
// each of them once (one or two per lane) into a per-wave LDS table, and
// every lane reads the cos/sin of its own pairs from it where they are used
// (held in registers they would cost a wave slot per SIMD).  Each lane loads
// only its own head's norm weight (Q or K).  Angles are formed in fp64:
// theta^(-2i/D) = 2^(i * step) with step = -2 log2(theta) / D computed on
// the host, times the position, reduced modulo pi/2 by a two-constant
// Cody-Waite step with fma; sine and cosine come from Taylor polynomials on
// [-pi/4, pi/4], so the angle stays exact to ~1e-15 for any int32 position.
// The RoPE layout is a template parameter.
#include "fr_device.h"
#include "fr_launch.h"

namespace fr {

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
                 "s"(a.Hkv), "s"(a.D), "s"(a.groups),
                 "s"(a.table_len), "s"(a.page_size), "s"(a.num_pages), "s"(a.eps),
                 "s"(a.q_scale), "s"(a.l2t), "s"(a.inv_d));

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t task = (int64_t)blockIdx.x * 4 + wv;
    if (task >= a.tasks) return;                         // whole wave exits
    const int64_t t = task / a.groups;                   // token
    const int g0 = (int)(task - t * a.groups);           // this wave's head group

    constexpr int HPW = 64 / LP;
    const int NH = a.Hq + 2 * a.Hkv;
    const int D = a.D;
    const int L = D >> 4;                                // lanes with data per head
    const int j = lane & (LP - 1);
    const int hl = lane / LP;                            // head within a group

    // This lane's head and chunks.  Every lane loads (lanes past the row's
    // heads or past D/16 re-read a valid chunk and store nothing), so the
    // compiler's waits cover exactly the loads in use.
    const char* rowp = (const char*)a.qkv + t * (int64_t)NH * D * 2;
    const int off0 = j * 16;                 // bytes of chunk j, first half
    const int off1 = D + j * 16;             // bytes of chunk j, second half
    const int jc = min(j, L - 1);
    const int head = g0 * HPW + hl;
    const int head_c = min(head, NH - 1);
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

    u32x4 c0, c1;
    {
        const char* src = rowp + (int64_t)head_c * D * 2 + jc * 16;
        c0 = NT ? ld128_stream(src) : ld128(src);
        c1 = NT ? ld128_stream(src + D) : ld128(src + D);
    }
    u32x4 w0, w1;                                        // the head's norm weight
    {
        const char* wp = head_c < a.Hq ? (const char*)a.qw : (const char*)a.kw;
        if (wp == nullptr) wp = rowp;                    // unused (no norm)
        w0 = ld128(wp + jc * 16);
        w1 = ld128(wp + D + jc * 16);
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
    // this lane's pairs: rotate-half pair e = (8j+e, D/2+8j+e) turns by
    // angle 8j+e; interleaved pair m of chunk 0 = (8j+2m, 8j+2m+1) by
    // angle 4j+m, pair m of chunk 1 by angle D/4+4j+m
    float cs[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int i = STYLE == 0 ? 8 * j + e
                                   : (e < 4 ? 4 * j + e : (D >> 2) + 4 * j + (e - 4));
        cs[e] = cs_tab[i];
        sn[e] = sn_tab[i];
    }

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

// One head group per wave at every batch size.  In the bandwidth regime
// (T >= 2048) loads and stores are non-temporal.  Measured on MI355X at
// T = 8192, 32/8 heads x 128 bf16 (6 groups), same-box A/B, outputs
// identical: a token's groups split over 2 waves (a prefetch loop over 3
// groups each, 78 registers) 36.7 us; over 3 waves 34.5 us; one group per
// wave with the same registers 34.4 us; as here (the norm weight of the
// lane's own head only, cos/sin read from LDS where used: 68 registers, 7
// waves per SIMD instead of 6) 33.8 us.  At 4096 tokens 20.0 -> 18.3 us;
// 64/8 heads at 8192 tokens 60.0 -> 53.7 us.
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
    a.tasks = a.T * a.groups;
    if (dtype == DT_BF16)
        return big ? launch_qkv_dt<DT_BF16, true>(a, lp, s) : launch_qkv_dt<DT_BF16, false>(a, lp, s);
    return big ? launch_qkv_dt<DT_F16, true>(a, lp, s) : launch_qkv_dt<DT_F16, false>(a, lp, s);
}

}  // namespace fr
