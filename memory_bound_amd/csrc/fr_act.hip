// fr_act.hip -- gated activation on interleaved gate/up + per-token block-128
// FP8 quantisation (op c), one kernel.
//
// Definitions: "sm89 prefill FFN megakernel" issue, Phase 2 (silu(g)*u with
// per-token block-128 FP8 output, no intermediate bf16 rounding) and its
// correctness notes (every scale entry must be written); "Falcon-Perception
// inference engine" article, third technique (the gate kernel reads
// interleaved [g0, u0, g1, u1, ...] in one pass); "FlashRT cross-layer
// fusion" article, section 二 table steps 8-10 (GELU * up + FP8 fused).
//
// Mapping: each 32-bit word of a bf16/fp16 row holds one (g, u) pair, so one
// 16-byte chunk yields 4 outputs and a block of 128 outputs is 32 chunks:
// the lower or upper 32 lanes of one 128-bit wave load, so every load
// instruction of a wave reads one contiguous 1 KB span.  A wave walks STEPS
// consecutive block pairs of one row with every load issued before any
// arithmetic; the input is read once, so its loads are non-temporal in the
// bandwidth regime.  The block maximum is a DPP row reduction plus one
// permlane16 swap, taken as an integer maximum (the operands are magnitudes,
// never NaN, so their bit patterns order like the values and the DPP move
// folds into v_max_u32; 1% faster than the float maximum, whose operands
// need NaN canonicalisation).  The scale is the correctly rounded amax / 448
// (fma-corrected quotient); |h / scale| <= 448 (1 + 3 ulp) < 464, so the
// e4m3 conversion never sees a value that would overflow and needs no
// clamp.  The wave's codes form one contiguous span (STEPS * 256 bytes);
// they are gathered in LDS and leave as 16-byte stores (4-byte stores straight
// from each step: 3% slower); its block scales are gathered in LDS too (one
// write per block, 0.4% faster than collecting them in lanes with readlane
// and selects).  (Measured on MI355X at 8192 x 12288: this
// layout with 4 waves per workgroup is 5-15% faster than 2 or 8 waves per
// workgroup or 32-byte lane-contiguous chunks.)
//
// MX FP4 output (Hy-Embodied report, 04 step 9 and 06: the SwiGLU FP4
// producer): the same loads and activation; a block of 32 outputs is 8
// consecutive lanes, its maximum a DPP reduction over 8 lanes, whose fp32
// exponent gives the E8M0 code; the 4 outputs of a lane become 16 bits of
// E2M1 codes after an exact power-of-two scaling; codes and E8M0 scales are
// gathered in LDS like the FP8 codes.
#include "fr_device.h"
#include "fr_launch.h"

namespace fr {

constexpr int kActSteps = 4;   // block pairs per wave (bandwidth regime)

// STEPS: block pairs per wave; NTL / NTS: non-temporal loads / stores;
// MX: MX FP4 output instead of block-128 FP8.
template <int DT, int ACT, int STEPS = kActSteps, bool NTL = true, bool NTS = true,
          bool MX = false>
__global__ __launch_bounds__(256) void k_act(ActArgs a) {
    // the wave's codes (STEPS block pairs = one contiguous span: FP8 STEPS *
    // 256 bytes; MX FP4 STEPS * 128 bytes, then its STEPS * 8 E8M0 codes),
    // gathered so they leave as 16-byte stores
    constexpr int SPAN = MX ? STEPS * 136 : STEPS * 256;
    __shared__ __attribute__((aligned(16))) uint8_t obuf[4][SPAN];
    __shared__ float sbuf[4][2 * STEPS];                 // the wave's block scales
    // (the wave index is left in vector form: made uniform, its 64-bit
    // division by the waves per row moves to the scalar unit and delays the
    // first loads; measured 1% slower)
    const int wv = (int)(threadIdx.x >> 6);
    uint8_t* ob = obuf[wv];
    float* sb = sbuf[wv];
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * 4 + wv;
    if (wid >= a.waves) return;                          // whole wave exits
    const int64_t t = wid / a.wpr;
    const int wc = (int)(wid - t * a.wpr);
    const int half = lane >> 5;
    const int cb = lane & 31;                            // chunk within block

    const char* row = (const char*)a.gu + t * (int64_t)a.I * 4;
    uint8_t* orow = a.out + t * (int64_t)a.I;
    float* srow = a.scales + t * (int64_t)a.nb;

    u32x4 in[STEPS];                                     // all loads first
#pragma unroll
    for (int k = 0; k < STEPS; ++k) {
        const int b = (wc * STEPS + k) * 2 + half;
        const unsigned off = (unsigned)(b < a.nb ? b : a.nb - 1) * 512u + (unsigned)cb * 16u;
        in[k] = NTL ? ld128_stream(row + off) : ld128(row + off);
    }

#pragma unroll
    for (int k = 0; k < STEPS; ++k) {
        float h[4];
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = gate_act<ACT>(lo16<DT>(in[k][e])) * hi16<DT>(in[k][e]);
            m = fmaxf(m, fabsf(h[e]));
        }
        if constexpr (MX) {
            m = group_reduce<8>(m, OpMaxMag());          // block of 32 outputs
            const int code = mx_code(m);
            const u32 p = pack_e2m1x4(h[0], h[1], h[2], h[3], mx_mult(code));
            *reinterpret_cast<uint16_t*>(ob + (2 * k + half) * 64 + cb * 2) = (uint16_t)p;
            if ((cb & 7) == 0) ob[STEPS * 128 + (2 * k + half) * 4 + (cb >> 3)] = (uint8_t)code;
            continue;
        }
        // Block maximum over 32 lanes (all 64 lanes take part); m is a
        // maximum of magnitudes (never NaN), so the integer maximum applies.
        m = group_reduce<16>(m, OpMaxMag());
        m = rows_pair(m, OpMaxMag());
        const float s = div448(fmaxf(m, 1e-10f));        // correctly rounded
        const float inv = __builtin_amdgcn_rcpf(s);
        {
            int q = __builtin_amdgcn_cvt_pk_fp8_f32(h[0] * inv, h[1] * inv, 0, false);
            q = __builtin_amdgcn_cvt_pk_fp8_f32(h[2] * inv, h[3] * inv, q, true);
            *reinterpret_cast<u32*>(ob + (2 * k + half) * 128 + cb * 4) = (u32)q;
        }
        if (cb == 0) sb[2 * k + half] = s;               // block 2k + half
    }
    const int b0 = wc * STEPS * 2;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if constexpr (MX) {
        // codes: 16-byte chunk c is in block b0 + c / 4; E8M0 codes: 4 per block
        uint8_t* o4 = a.out + t * (int64_t)(a.I >> 1) + (int64_t)b0 * 64;
#pragma unroll
        for (int c = lane; c < STEPS * 8; c += 64) {
            if (b0 + (c >> 2) < a.nb) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(ob + c * 16);
                if constexpr (NTS) st128_stream(o4 + c * 16, v); else st128(o4 + c * 16, v);
            }
        }
        if (lane < 2 * STEPS && b0 + lane < a.nb) {
            const u32 e = *reinterpret_cast<const u32*>(ob + STEPS * 128 + lane * 4);
            u32* dst = reinterpret_cast<u32*>(a.mx_scales + t * (int64_t)(a.I >> 5) + (b0 + lane) * 4);
            if constexpr (NTS) __builtin_nontemporal_store(e, dst); else *dst = e;
        }
        return;
    }
    // the codes: 16-byte chunk c of the wave's span is block b0 + c / 8
#pragma unroll
    for (int c = lane; c < STEPS * 16; c += 64) {
        if (b0 + (c >> 3) < a.nb) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(ob + c * 16);
            if constexpr (NTS) st128_stream(orow + (int64_t)b0 * 128 + c * 16, v);
            else st128(orow + (int64_t)b0 * 128 + c * 16, v);
        }
    }
    // one contiguous store of the wave's 2 * STEPS block scales
    if (lane < 2 * STEPS && b0 + lane < a.nb) {
        const float sc = sb[lane];
        if constexpr (NTS) __builtin_nontemporal_store(sc, srow + b0 + lane); else srow[b0 + lane] = sc;
    }
}

template <int DT, int STEPS, bool NTL, bool NTS, bool MX>
static hipError_t launch_act_cfg(const ActArgs& in, int act, hipStream_t s) {
    ActArgs a = in;
    const int per_wave = 2 * STEPS;                      // blocks per wave
    a.wpr = (a.nb + per_wave - 1) / per_wave;
    a.waves = a.T * a.wpr;
    const void* fn;
    switch (act) {
    case ACT_SWIGLU: fn = (const void*)k_act<DT, ACT_SWIGLU, STEPS, NTL, NTS, MX>; break;
    case ACT_GEGLU_TANH: fn = (const void*)k_act<DT, ACT_GEGLU_TANH, STEPS, NTL, NTS, MX>; break;
    default: fn = (const void*)k_act<DT, ACT_SQRELU, STEPS, NTL, NTS, MX>; break;
    }
    void* args[] = {&a};
    const unsigned blocks = (unsigned)((a.waves + 3) / 4);
    return hipLaunchKernel(fn, dim3(blocks), dim3(256), args, 0, s);
}

// Bandwidth regime (T >= 2048): 4 block pairs per wave, non-temporal loads,
// cacheable stores.  Measured back to back on MI355X at 8192 x 12288 bf16
// (~6.4 TB/s): 8 pairs 1.5% slower (MX FP4 output: 2.8%), 16 pairs 5%, 2
// pairs 11%, 1 pair 36% slower; non-temporal stores ~5% slower, cacheable
// loads ~15% slower.  (Before the block maximum and the scale gather were
// trimmed, 8 pairs were the fastest.)  Small batches: 2 block pairs per wave
// for more parallel waves, everything cacheable for the next op.
template <bool MX>
static hipError_t launch_act_fmt(const ActArgs& a, int dtype, int act, hipStream_t s) {
    const bool big = a.T >= 2048;
    if (dtype == DT_BF16)
        return big ? launch_act_cfg<DT_BF16, kActSteps, true, false, MX>(a, act, s)
                   : launch_act_cfg<DT_BF16, 2, false, false, MX>(a, act, s);
    return big ? launch_act_cfg<DT_F16, kActSteps, true, false, MX>(a, act, s)
               : launch_act_cfg<DT_F16, 2, false, false, MX>(a, act, s);
}

hipError_t launch_act(const ActArgs& in, int dtype, int act, bool mx, hipStream_t s) {
    ActArgs a = in;
    a.nb = a.I / 128;
    return mx ? launch_act_fmt<true>(a, dtype, act, s) : launch_act_fmt<false>(a, dtype, act, s);
}

}  // namespace fr
