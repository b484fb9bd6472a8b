// fr_gemm.hip -- FP8 block-scaled gate_up GEMM fused with the gated
// activation and per-token block-128 FP8 output, on the gfx950 matrix cores.
//
// Definitions: "sm89 prefill FFN megakernel" issue, Phase 2 (gate_up GEMM +
// silu * up + per-token block-128 FP8 quantisation in one launch, removing
// the [S, 2 * inter] bf16 intermediate; the fused path has one bf16 rounding
// fewer) and its correctness notes (every scale row must be written);
// "Falcon-Perception inference engine" article, third technique (gate and up
// weights interleaved so one GEMM emits [g, u] pairs).
//
// C[m, n] = sum_k A[m, k] a_s[m, k/128] * W[n, k] w_s[n/128, k/128] with A,
// W e4m3 and fp32 dequant scales; n = 2j is gate output j, n = 2j+1 its up
// partner.  Each workgroup (4 waves) owns a tile of 32 rows x 256 columns,
// i.e. exactly one 128-output block of the result, so the block maximum
// never leaves the workgroup.  Wave w computes columns [64w, 64w+64) as two
// 32x32 tiles with v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unit MX
// scales): per 128-wide K block it runs 2 x 2 MFMAs into a fresh fp32
// partial, then folds the partial into the accumulator times
// a_s(row) * w_s, with the activation scale panel of the tile in LDS.  The
// instruction's own sum of 64 products is not exact (about 15 bits relative
// to the sum of magnitudes on MI355X), so partials are promoted to fp32 at
// every 128-wide K block.  Operand fragments come straight from global
// memory (lane l: row l % 32, 32 consecutive K bytes at 32 * (l / 32)),
// DEPTH K blocks ahead of the MFMAs.
// Epilogue: the fp32 tile goes through LDS, then each wave takes 8 rows:
// every lane reads (g, u, g, u) for two outputs, applies the activation,
// and the wave reduces the block maximum and writes 128 codes and a scale.
// Tiles are ordered so that each XCD (which serves blocks b with b % 8
// fixed) walks a contiguous range of tiles, and the 32-row tiles of one
// 256-column weight panel run together on one XCD and share its L2.
#include "fr_device.h"
#include "fr_launch.h"

namespace fr {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kGemmMaxKB = 128;   // K <= 16384
constexpr int kGemmDepth = 2;      // K blocks in flight per wave

__device__ __forceinline__ i32x8 ld256(const uint8_t* p) {
    const u32x4 lo = ld128(p), hi = ld128(p + 16);
    i32x8 r;
    r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
    return r;
}

// 32x32x64 e4m3 x e4m3 -> fp32 with unit (2^0) MX scales
__device__ __forceinline__ f32x16 mma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// DEPTH: K blocks whose operand fragments are in flight per wave (a ring of
// registers; the loop is unrolled by DEPTH so every slot index is static).
// The loop body is one basic block that issues no global load other than
// the ring refills, so the wait for slot d never covers the loads of later
// slots.  K is padded to a multiple of DEPTH with blocks whose scales are
// zero (their operands re-read the last real block, so they stay finite).
template <int ACT, int DEPTH>
__global__ __launch_bounds__(256) void k_gemm_act(GemmActArgs a) {
    static_assert(kGemmMaxKB % DEPTH == 0 && 2 * kGemmMaxKB == 256, "padding");
    __shared__ float tile[32 * 256];
    __shared__ float4 asc4[kGemmMaxKB * 8];              // [kb][row / 4], 4 rows
    __shared__ float bsc[2 * kGemmMaxKB];                // [128-col block][kb]

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int L = (int)(blockIdx.x & 7) * a.per_xcd + (int)(blockIdx.x >> 3);
    if (L >= a.tiles) return;                            // whole workgroup exits
    const int n_tile = L / a.mt;
    const int m_tile = L - n_tile * a.mt;
    const int m0 = m_tile * 32;
    const int n0 = n_tile * 256;
    const int KB = a.K >> 7;
    const int KBp = (KB + DEPTH - 1) / DEPTH * DEPTH;

    // Scale panels of the tile: activation scales of its 32 rows (rows past
    // M repeat row M-1), stored transposed so that one 16-byte LDS read gives
    // the 4 consecutive rows that accumulator registers 4q..4q+3 of a lane
    // hold; weight scales of its two 128-column blocks.  Padding blocks get
    // zero.  Loaded to registers first so that the LDS stores below wait
    // only for these loads, not for the operand ring issued after them.
    float sv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {                       // 16 * 256 = 32 * kGemmMaxKB
        const int i = threadIdx.x + 256 * j;             // = kb * 32 + row
        const int kb = i >> 5;
        const int m = min(m0 + (i & 31), a.M - 1);
        sv[j] = a.a_scales[(int64_t)m * KB + min(kb, KB - 1)];
    }
    float bv;
    {
        const int t = min((int)threadIdx.x, 2 * KBp - 1);
        const int j = t / KBp, kb = t - j * KBp;
        bv = a.b_scales[(int64_t)((n0 >> 7) + j) * KB + min(kb, KB - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);                   // scale loads first

    const int rl = lane & 31;                            // fragment row / column
    const int kh = lane >> 5;                            // K half of a 64-wide step
    const uint8_t* ap = a.A + (int64_t)min(m0 + rl, a.M - 1) * a.K + kh * 32;
    const uint8_t* bp0 = a.B + (int64_t)(n0 + 64 * w + rl) * a.K + kh * 32;
    const uint8_t* bp1 = bp0 + (int64_t)32 * a.K;

    // operand ring: slot d holds K block kb with kb % DEPTH == d
    i32x8 ra0[DEPTH], ra1[DEPTH], rb00[DEPTH], rb01[DEPTH], rb10[DEPTH], rb11[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        const int o = min(d, KB - 1) * 128;
        ra0[d] = ld256(ap + o);
        ra1[d] = ld256(ap + o + 64);
        rb00[d] = ld256(bp0 + o);
        rb01[d] = ld256(bp0 + o + 64);
        rb10[d] = ld256(bp1 + o);
        rb11[d] = ld256(bp1 + o + 64);
    }

    float* ascf = reinterpret_cast<float*>(asc4);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int i = threadIdx.x + 256 * j;
        ascf[i] = (i >> 5) < KB ? sv[j] : 0.0f;
    }
    {
        const int t = min((int)threadIdx.x, 2 * KBp - 1);
        bsc[threadIdx.x] = t - t / KBp * KBp < KB ? bv : 0.0f;   // >= 2 KBp: unused
    }
    __syncthreads();
    const float* bs = bsc + (w >> 1) * KBp;

    f32x16 acc0 = {}, acc1 = {};
    for (int kb0 = 0; kb0 < KBp; kb0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int kb = kb0 + d;
            float4 sa[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) sa[q] = asc4[kb * 8 + 2 * q + kh];
            const float bk = bs[kb];
            f32x16 p0 = {}, p1 = {};
            p0 = mma_e4m3(ra0[d], rb00[d], p0);
            p1 = mma_e4m3(ra0[d], rb10[d], p1);
            p0 = mma_e4m3(ra1[d], rb01[d], p0);
            p1 = mma_e4m3(ra1[d], rb11[d], p1);
            // refill the slot (past the end: re-read the last block, a cache
            // hit, so the loop body stays free of branches)
            const int o = min(kb + DEPTH, KB - 1) * 128;
            ra0[d] = ld256(ap + o);
            ra1[d] = ld256(ap + o + 64);
            rb00[d] = ld256(bp0 + o);
            rb01[d] = ld256(bp0 + o + 64);
            rb10[d] = ld256(bp1 + o);
            rb11[d] = ld256(bp1 + o + 64);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float f[4] = {sa[q].x * bk, sa[q].y * bk, sa[q].z * bk, sa[q].w * bk};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc0[4 * q + e] = fmaf(p0[4 * q + e], f[e], acc0[4 * q + e]);
                    acc1[4 * q + e] = fmaf(p1[4 * q + e], f[e], acc1[4 * q + e]);
                }
            }
        }
    }

    // epilogue: tile to LDS, then one row per step per wave
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * kh + (r & 3);
        tile[row * 256 + 64 * w + rl] = acc0[r];
        tile[row * 256 + 64 * w + 32 + rl] = acc1[r];
    }
    __syncthreads();
#pragma unroll 1
    for (int i = 0; i < 8; ++i) {
        const int row = w * 8 + i;
        const int m = m0 + row;
        const float4 v = *reinterpret_cast<const float4*>(&tile[row * 256 + 4 * lane]);
        const float h0 = gate_act<ACT>(v.x) * v.y;
        const float h1 = gate_act<ACT>(v.z) * v.w;
        const float mx = wave_reduce(fmaxf(fabsf(h0), fabsf(h1)), OpMax());
        const float s = div448(fmaxf(mx, 1e-10f));
        const float inv = __builtin_amdgcn_rcpf(s);
        if (m < a.M) {
            // |h * inv| <= 448 (1 + 3 ulp) < 464: no clamp needed
            const int q = __builtin_amdgcn_cvt_pk_fp8_f32(h0 * inv, h1 * inv, 0, false);
            *reinterpret_cast<uint16_t*>(a.out + (int64_t)m * a.I + n_tile * 128 + 2 * lane) =
                (uint16_t)q;
            if (lane == 0) a.out_scales[(int64_t)m * (a.I >> 7) + n_tile] = s;
        }
    }
}

template <int DEPTH>
static hipError_t launch_gemm_depth(const GemmActArgs& in, int act, hipStream_t s) {
    GemmActArgs a = in;
    a.mt = (a.M + 31) / 32;
    a.tiles = a.mt * (a.I / 128);
    a.per_xcd = (a.tiles + 7) / 8;
    const void* fn;
    switch (act) {
    case ACT_SWIGLU: fn = (const void*)k_gemm_act<ACT_SWIGLU, DEPTH>; break;
    case ACT_GEGLU_TANH: fn = (const void*)k_gemm_act<ACT_GEGLU_TANH, DEPTH>; break;
    default: fn = (const void*)k_gemm_act<ACT_SQRELU, DEPTH>; break;
    }
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3((unsigned)(8 * a.per_xcd)), dim3(256), args, 0, s);
}

hipError_t launch_gemm_act(const GemmActArgs& in, int act, hipStream_t s) {
    return launch_gemm_depth<kGemmDepth>(in, act, s);
}

}  // namespace fr
