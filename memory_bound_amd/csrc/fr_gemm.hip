// fr_gemm.hip -- FP8 block-scaled gate_up GEMM fused with the gated
// activation and per-token block-128 FP8 output, on the gfx950 matrix cores,
// and the one-time weight packing it reads.
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
// partner.  Each workgroup (4 waves) owns a tile of 32 RG rows x 256
// columns, i.e. exactly one 128-output block of the result per row, so the
// block maximum never leaves the workgroup (large batches use a 128-row,
// 8-wave variant, k_gemm_act_big, below).  Wave w computes columns
// [64w, 64w+64) of all the tile's rows as 2 RG tiles of 32x32 with
// v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unit MX scales), in
// transposed form (weight fragment first; see the kernel): per 128-wide K
// block it runs two MFMAs per tile into a fresh fp32 partial, then folds
// the partial into the accumulator times a_s(row) * w_s.  The
// instruction's own sum of 64 products is not exact (about 15 bits relative
// to the sum of magnitudes on MI355X), so partials are promoted to fp32 at
// every 128-wide K block.
//
// Operand traffic.  An MFMA fragment puts row (l % 32) in lane l, so a
// fragment loaded straight from a row-major matrix touches 32 cache lines
// per instruction.  The weights are therefore packed once
// (fr_gemm_pack_weights) so that every fragment load of a wave reads 1 KB
// of consecutive bytes, DEPTH K blocks ahead of the MFMAs, into registers.
// The activation tile is shared by the 4 waves: each wave fetches one
// quarter of every K block (DEPTH blocks ahead, in registers) and writes it
// to a double-buffered LDS stage laid out in fragment order, so the
// fragment reads are conflict-free; one barrier per K block.  (Direct
// global->LDS loads would save the register hop, but the compiler then
// waits for every outstanding load before each LDS read.)  The scale
// panels of the tile are staged in LDS before the loop.  Measured on
// MI355X, this layout runs 1.5x (128 tokens) to 3x (4096 tokens) faster
// than fragments loaded straight from the row-major weight.
//
// Epilogue: a lane holds one activation row and, for each of its 16 weight
// columns per 32-column group, gate and up partner in adjacent registers,
// so act(g) * u needs no lane exchange.  Row maxima are reduced over the
// lane's values, the other lane half and the 4 waves (LDS); the codes go
// through LDS so each output row leaves as 128 contiguous bytes (8-byte
// stores into a row-swizzled tile, free of bank conflicts: 4-9% faster
// than one 2-byte store per output pair, whose 32 rows shared one bank),
// and the row scales are gathered in LDS and leave as one store.  Lanes that hold
// the same value all write it, so the epilogue has no per-row branches (it
// was ~20% of the kernel at 128 tokens with them).  Tiles are ordered so
// that each XCD (which serves blocks b with b % 8 fixed) walks a contiguous
// range of tiles: the row tiles of one 256-column weight panel run together
// on one XCD and share its L2.
#include "fr_device.h"
#include "fr_launch.h"

namespace fr {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kGemmMaxKB = 128;     // K <= 16384
constexpr int kGemmPanel = 4096;    // rows x K blocks of the staged a_s panel
constexpr int kCUs = 256;           // compute units of an MI355X

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
    i32x8 r;
    r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
    return r;
}

// 32x32x64 e4m3 x e4m3 -> fp32 with unit (2^0) MX scales
__device__ __forceinline__ f32x16 mma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ u32x4 lds128(const uint8_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Byte offset, within a 128-wide K block, of the 16 bytes that chunk c
// (0..3) gives lane half kh: chunks 2h and 2h+1 form the 32-byte fragment
// of the h-th 64-wide MFMA step.
__device__ __forceinline__ int chunk_koff(int c, int kh) {
    return 64 * (c >> 1) + 32 * kh + 16 * (c & 1);
}

// Output tile in LDS: [row][128] codes, the 16-byte chunk c of a row kept at
// chunk c ^ (row % 8), so that the 32 rows of one store (rows 128 bytes
// apart) spread over the banks.
__device__ __forceinline__ int otile_off(int row, int chunk) {
    return row * 128 + ((chunk ^ (row & 7)) << 4);
}

// Store one row's codes of a 32-output quarter q (two 16-output tiles t).
// c[t][i] holds the codes of outputs 16 t + 4 i + 2 kh + {0, 1}, so each
// lane half has two of every four bytes; one permlane32 swap per tile hands
// each lane the partner's half of the dwords it writes (lane half 0 the
// first 8 bytes of the tile, half 1 the last 8), one 8-byte store each.
__device__ __forceinline__ void store_codes(uint8_t* otile, int row, int q, int kh,
                                            const u32 (&c)[2][4]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const u32 send = kh ? (c[t][0] | c[t][1] << 16) : (c[t][2] | c[t][3] << 16);
        const auto pr = __builtin_amdgcn_permlane32_swap(send, send, false, false);
        const u32 recv = kh ? (u32)pr[0] : (u32)pr[1];
        const u32 lo0 = kh ? (recv & 0xFFFFu) : c[t][0];
        const u32 hi0 = kh ? c[t][2] : (recv & 0xFFFFu);
        const u32 lo1 = kh ? (recv >> 16) : c[t][1];
        const u32 hi1 = kh ? c[t][3] : (recv >> 16);
        u32x2 v;
        v.x = lo0 | hi0 << 16;
        v.y = lo1 | hi1 << 16;
        *reinterpret_cast<u32x2*>(otile + otile_off(row, 2 * q + t) + 8 * kh) = v;
    }
}

// Every kernel argument consumed at once (an empty asm statement that reads
// them), so that the compiler fetches the two scalar-cache lines they span
// in one batch of scalar loads rather than in dependent batches as each is
// first needed (one memory trip fewer at the start of a launch).
__device__ __forceinline__ void fetch_args(const GemmActArgs& a) {
    asm volatile("" ::"s"(a.A), "s"(a.a_scales), "s"(a.B), "s"(a.b_scales), "s"(a.out),
                 "s"(a.out_scales), "s"(a.M), "s"(a.K), "s"(a.I), "s"(a.mt), "s"(a.tiles),
                 "s"(a.per_xcd));
}

// RG: 32-row groups per tile (32 RG x K/128 <= kGemmPanel); DEPTH: K blocks
// in flight per wave (even, so the LDS stage of a block is static).
//
// The matrix cores compute the transposed tile, C^T = W A^T: the weight
// fragment is the first operand and the activation fragment the second (the
// two operands have the same lane layout, so this is only an argument swap).
// A lane then holds one activation row (row 32 g + lane % 32) and 16 weight
// columns of each 32-column group, so
//  - the fold factor a_s(row, kb) * w_s(block, kb) is one value per lane and
//    row group (one LDS read, where the direct product needs the scales of
//    the lane's 16 rows);
//  - a gate column and its up partner (columns 2j, 2j + 1) sit in registers
//    2i and 2i + 1 of the same lane, so act(g) * u needs no lane exchange;
//  - a row's block maximum is 16 values in the lane, the other lane half
//    (one permlane32 swap) and the other 3 waves (LDS).
// Measured against the direct product (same outputs, bit for bit): 1-4%
// faster at 128 / 1024 / 4096 tokens, 4% slower at 192 tokens.
template <int ACT, int RG, int DEPTH>
__global__ __launch_bounds__(256) void k_gemm_act(GemmActArgs a) {
    constexpr int ROWS = 32 * RG;
    static_assert(DEPTH % 2 == 0, "stage parity must be static");
    __shared__ __attribute__((aligned(16))) uint8_t stage[2 * RG * 4096];
    __shared__ __attribute__((aligned(16))) float asp[kGemmPanel];          // [kb][row]
    __shared__ __attribute__((aligned(16))) float bsp[2 * kGemmMaxKB];     // [block][kb]
    __shared__ __attribute__((aligned(16))) float red[ROWS * 4];           // [row][wave]
    __shared__ __attribute__((aligned(16))) float osc[ROWS];               // row scales

    fetch_args(a);
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;                      // column quarter
    const int L = (int)(blockIdx.x & 7) * a.per_xcd + (int)(blockIdx.x >> 3);
    if (L >= a.tiles) return;                            // whole workgroup exits
    const int n_tile = L / a.mt;
    const int m_tile = L - n_tile * a.mt;
    const int m0 = m_tile * ROWS;
    const int KB = a.K >> 7;
    const int KBp = (KB + DEPTH - 1) / DEPTH * DEPTH;    // padded: factor 0
    const int rl = lane & 31;
    const int kh = lane >> 5;

    // Scale panels, loaded to registers before the operand loads so that
    // their LDS stores below wait for these loads only: a_s of the tile's
    // rows (rows past M repeat row M-1) as [kb][row], read back as one value
    // per lane (each row's K/128 scales are contiguous in memory, so the
    // panel load reads whole lines; per-lane loads of a_s in the loop would
    // gather 32 lines per instruction and measured 15% slower); w_s of the
    // two 128-column blocks (2 consecutive rows of w_s).
    constexpr int PJ = kGemmPanel / 256;
    float sv[PJ];
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
        const int e = min((int)threadIdx.x + 256 * j, ROWS * KB - 1);
        const int kb = e / ROWS, row = e - kb * ROWS;
        sv[j] = a.a_scales[(int64_t)min(m0 + row, a.M - 1) * KB + kb];
    }
    const int tb = min((int)threadIdx.x, 2 * KB - 1);
    const float bv = a.b_scales[(int64_t)(2 * n_tile) * KB + tb];
    __builtin_amdgcn_sched_barrier(0);

    // Activation chunk of this wave: chunk w of every row group.
    const uint8_t* ag[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g)
        ag[g] = a.A + (int64_t)min(m0 + 32 * g + rl, a.M - 1) * a.K + chunk_koff(w, kh);
    // Packed weights: the wave's two 32-column groups, 4 KB per K block each.
    const uint8_t* bq0 = a.B + (int64_t)(8 * n_tile + 2 * w) * KB * 4096 + lane * 16;
    const uint8_t* bq1 = bq0 + (int64_t)KB * 4096;

    u32x4 ra[DEPTH][RG];
    i32x8 rb00[DEPTH], rb01[DEPTH], rb10[DEPTH], rb11[DEPTH];   // [group][step]
    auto issue = [&](int d, int kb) {
        const int o = kb * 4096;
        rb00[d] = join(ld128(bq0 + o), ld128(bq0 + o + 1024));
        rb01[d] = join(ld128(bq0 + o + 2048), ld128(bq0 + o + 3072));
        rb10[d] = join(ld128(bq1 + o), ld128(bq1 + o + 1024));
        rb11[d] = join(ld128(bq1 + o + 2048), ld128(bq1 + o + 3072));
#pragma unroll
        for (int g = 0; g < RG; ++g) ra[d][g] = ld128(ag[g] + kb * 128);
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d, min(d, KB - 1));
    __builtin_amdgcn_sched_barrier(0);                   // operand loads before the stores

#pragma unroll
    for (int j = 0; j < PJ; ++j) asp[threadIdx.x + 256 * j] = sv[j];
    bsp[threadIdx.x] = bv;                               // entries >= 2 KB unused

    f32x16 acc[RG][2];
#pragma unroll
    for (int g = 0; g < RG; ++g) acc[g][0] = acc[g][1] = f32x16{};
    const float* bsw = bsp + (w >> 1) * KB;
    for (int kb0 = 0; kb0 < KBp; kb0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int kb = kb0 + d;
            uint8_t* st = stage + (d & 1) * RG * 4096 + lane * 16;
#pragma unroll
            for (int g = 0; g < RG; ++g)
                *reinterpret_cast<u32x4*>(st + (g * 4 + w) * 1024) = ra[d][g];
            __syncthreads();                             // stage (and panels) complete
            i32x8 fa[RG][2];
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                fa[g][0] = join(lds128(st + (g * 4 + 0) * 1024), lds128(st + (g * 4 + 1) * 1024));
                fa[g][1] = join(lds128(st + (g * 4 + 2) * 1024), lds128(st + (g * 4 + 3) * 1024));
            }
            const int kbc = min(kb, KB - 1);
            const float bk = kb < KB ? bsw[kbc] : 0.0f;  // padding blocks add 0
            float f[RG];                                 // a_s(row, kb) * w_s(block, kb)
#pragma unroll
            for (int g = 0; g < RG; ++g) f[g] = asp[kbc * ROWS + 32 * g + rl] * bk;
            f32x16 p[RG][2];
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                p[g][0] = mma_e4m3(rb00[d], fa[g][0], f32x16{});
                p[g][1] = mma_e4m3(rb10[d], fa[g][0], f32x16{});
                p[g][0] = mma_e4m3(rb01[d], fa[g][1], p[g][0]);
                p[g][1] = mma_e4m3(rb11[d], fa[g][1], p[g][1]);
            }
            // refill the slot (past the end: re-read the last block, never used)
            issue(d, min(kb + DEPTH, KB - 1));
#pragma unroll
            for (int g = 0; g < RG; ++g) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    acc[g][0][r] = fmaf(p[g][0][r], f[g], acc[g][0][r]);
                    acc[g][1][r] = fmaf(p[g][1][r], f[g], acc[g][1][r]);
                }
            }
            // Keep K blocks in order: block kb's MFMAs and fold must not
            // drift behind the barrier of the next block (that would halve
            // the prefetch distance).  An empty volatile asm that takes the
            // accumulators pins the fold here.
#pragma unroll
            for (int g = 0; g < RG; ++g) asm volatile("" : "+v"(acc[g][0]), "+v"(acc[g][1]));
        }
    }

    // Epilogue.  Register r of tile t holds weight column
    // 64 w + 32 t + 8 (r / 4) + 4 kh + r % 4 of the tile for activation row
    // 32 g + rl; r = 2i is gate and r = 2i + 1 its up partner of output
    // j = 32 w + 16 t + 4 (i / 2) + 2 kh + i % 2 of the block.
    float h[RG][2][8];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                h[g][t][i] = gate_act<ACT>(acc[g][t][2 * i]) * acc[g][t][2 * i + 1];
                m = fmaxf(m, fabsf(h[g][t][i]));
            }
        }
        // the other lane half holds the rest of this wave's 32 outputs;
        // magnitudes, never NaN: integer maximum
        m = halves(m, OpMaxMag());
        red[(32 * g + rl) * 4 + w] = m;                  // both halves write it
    }
    __syncthreads();                                     // stages are reused below
    uint8_t* otile = stage;                              // [row][128] codes
    const int nbo = a.I >> 7;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int row = 32 * g + rl;
        const float4 mm = *reinterpret_cast<const float4*>(red + row * 4);
        const float mx = fmaxf(fmaxf(mm.x, mm.y), fmaxf(mm.z, mm.w));
        const float s = div448(fmaxf(mx, 1e-10f));       // correctly rounded
        const float inv = __builtin_amdgcn_rcpf(s);
        // |h * inv| <= 448 (1 + 3 ulp) < 464: no clamp needed
        u32 c[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2)
                c[t][i2] = (u32)__builtin_amdgcn_cvt_pk_fp8_f32(h[g][t][2 * i2] * inv,
                                                               h[g][t][2 * i2 + 1] * inv, 0, false);
        }
        store_codes(otile, row, w, kh, c);
        osc[row] = s;                                    // equal values from every writer
    }
    __syncthreads();
    if (threadIdx.x < ROWS && m0 + (int)threadIdx.x < a.M)   // one store per row
        a.out_scales[(int64_t)(m0 + threadIdx.x) * nbo + n_tile] = osc[threadIdx.x];
    {
#pragma unroll
        for (int i = 0; i < RG; ++i) {
            const int row = (w + 4 * i) * 8 + (lane >> 3);
            if (m0 + row < a.M)
                st128(a.out + (int64_t)(m0 + row) * a.I + n_tile * 128 + (lane & 7) * 16,
                      lds128(otile + otile_off(row, lane & 7)));
        }
    }
}

// Large-batch tile: 128 rows x 256 columns per workgroup of 8 waves, both
// operands staged through LDS.  Wave w computes rows [64 (w / 4), +64) x
// columns [64 (w % 4), +64) in the transposed form above.  Per K block the
// workgroup fetches 16 KB of activation and 32 KB of weight fragments once
// (each wave one 4 KB packed column group and two 1 KB activation chunks,
// DEPTH blocks ahead in registers) and every wave reads its fragments from
// the double-buffered stage; the weight bytes per output are half those of
// the 64-row tile, whose waves load their own weight fragments.
constexpr int kBigPanel = 4096;     // rows x K blocks of the staged a_s panel (128 x 32)

template <int ACT, int DEPTH>
__global__ __launch_bounds__(512) void k_gemm_act_big(GemmActArgs a) {
    constexpr int ROWS = 128;
    static_assert(DEPTH % 2 == 0, "stage parity must be static");
    __shared__ __attribute__((aligned(16))) uint8_t astage[2][16384];      // [rg][chunk][lane]
    __shared__ __attribute__((aligned(16))) uint8_t wstage[2][32768];      // [cg][chunk][lane]
    __shared__ __attribute__((aligned(16))) float asp[kBigPanel];          // [kb][row]
    __shared__ __attribute__((aligned(16))) float bsp[2 * kGemmMaxKB];     // [block][kb]
    __shared__ __attribute__((aligned(16))) float red[ROWS * 4];           // [row][col quarter]
    __shared__ __attribute__((aligned(16))) float osc[ROWS];

    fetch_args(a);
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;                      // 0..7
    const int wr = w >> 2, wc = w & 3;                   // row half, column quarter
    const int L = (int)(blockIdx.x & 7) * a.per_xcd + (int)(blockIdx.x >> 3);
    if (L >= a.tiles) return;                            // whole workgroup exits
    const int n_tile = L / a.mt;
    const int m_tile = L - n_tile * a.mt;
    const int m0 = m_tile * ROWS;
    const int KB = a.K >> 7;
    const int KBp = (KB + DEPTH - 1) / DEPTH * DEPTH;
    const int rl = lane & 31;
    const int kh = lane >> 5;

    // scale panels (see k_gemm_act)
    constexpr int PJ = kBigPanel / 512;
    float sv[PJ];
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
        const int e = min((int)threadIdx.x + 512 * j, ROWS * KB - 1);
        const int kb = e / ROWS, row = e - kb * ROWS;
        sv[j] = a.a_scales[(int64_t)min(m0 + row, a.M - 1) * KB + kb];
    }
    const int tb = min((int)threadIdx.x, 2 * KB - 1);
    const float bv = a.b_scales[(int64_t)(2 * n_tile) * KB + tb];
    __builtin_amdgcn_sched_barrier(0);

    // This wave's global fetch per K block: activation chunks c0 = w and
    // c1 = w + 8 of the 16 (row group c / 4, chunk c % 4), and packed weight
    // column group w (4 chunks).
    const uint8_t* ag0 = a.A + (int64_t)min(m0 + 32 * (w >> 2) + rl, a.M - 1) * a.K
                         + chunk_koff(w & 3, kh);
    const uint8_t* ag1 = a.A + (int64_t)min(m0 + 32 * (2 + (w >> 2)) + rl, a.M - 1) * a.K
                         + chunk_koff(w & 3, kh);
    const uint8_t* bq = a.B + (int64_t)(8 * n_tile + w) * KB * 4096 + lane * 16;

    u32x4 ra0[DEPTH], ra1[DEPTH], rw[DEPTH][4];
    auto issue = [&](int d, int kb) {
        const int o = kb * 4096;
#pragma unroll
        for (int c = 0; c < 4; ++c) rw[d][c] = ld128(bq + o + c * 1024);
        ra0[d] = ld128(ag0 + kb * 128);
        ra1[d] = ld128(ag1 + kb * 128);
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) issue(d, min(d, KB - 1));
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int j = 0; j < PJ; ++j) asp[threadIdx.x + 512 * j] = sv[j];
    if (threadIdx.x < 2 * kGemmMaxKB) bsp[threadIdx.x] = bv;

    f32x16 acc[2][2];                                    // [row group][column group]
#pragma unroll
    for (int g = 0; g < 2; ++g) acc[g][0] = acc[g][1] = f32x16{};
    const float* bsw = bsp + (wc >> 1) * KB;
    for (int kb0 = 0; kb0 < KBp; kb0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int kb = kb0 + d;
            uint8_t* as = astage[d & 1] + lane * 16;
            uint8_t* ws = wstage[d & 1] + lane * 16;
            *reinterpret_cast<u32x4*>(as + w * 1024) = ra0[d];
            *reinterpret_cast<u32x4*>(as + (w + 8) * 1024) = ra1[d];
#pragma unroll
            for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(ws + (w * 4 + c) * 1024) = rw[d][c];
            __syncthreads();                             // stage (and panels) complete
            i32x8 fa[2][2], fb[2][2];                    // [group][K step]
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int rg = 2 * wr + g, cg = 2 * wc + g;
                fa[g][0] = join(lds128(as + (rg * 4 + 0) * 1024), lds128(as + (rg * 4 + 1) * 1024));
                fa[g][1] = join(lds128(as + (rg * 4 + 2) * 1024), lds128(as + (rg * 4 + 3) * 1024));
                fb[g][0] = join(lds128(ws + (cg * 4 + 0) * 1024), lds128(ws + (cg * 4 + 1) * 1024));
                fb[g][1] = join(lds128(ws + (cg * 4 + 2) * 1024), lds128(ws + (cg * 4 + 3) * 1024));
            }
            const int kbc = min(kb, KB - 1);
            const float bk = kb < KB ? bsw[kbc] : 0.0f;
            float f[2];
#pragma unroll
            for (int g = 0; g < 2; ++g) f[g] = asp[kbc * ROWS + 32 * (2 * wr + g) + rl] * bk;
            f32x16 p[2][2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    p[g][t] = mma_e4m3(fb[t][0], fa[g][0], f32x16{});
                    p[g][t] = mma_e4m3(fb[t][1], fa[g][1], p[g][t]);
                }
            }
            issue(d, min(kb + DEPTH, KB - 1));
#pragma unroll
            for (int g = 0; g < 2; ++g) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    acc[g][0][r] = fmaf(p[g][0][r], f[g], acc[g][0][r]);
                    acc[g][1][r] = fmaf(p[g][1][r], f[g], acc[g][1][r]);
                }
            }
#pragma unroll
            for (int g = 0; g < 2; ++g) asm volatile("" : "+v"(acc[g][0]), "+v"(acc[g][1]));
        }
    }

    // Epilogue as in k_gemm_act; this wave's outputs of the block are
    // j = 32 wc + 16 t + 4 (i / 2) + 2 kh + i % 2 for rows 64 wr + 32 g + rl.
    float h[2][2][8];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                h[g][t][i] = gate_act<ACT>(acc[g][t][2 * i]) * acc[g][t][2 * i + 1];
                m = fmaxf(m, fabsf(h[g][t][i]));
            }
        }
        m = halves(m, OpMaxMag());
        red[(64 * wr + 32 * g + rl) * 4 + wc] = m;
    }
    __syncthreads();                                     // stages are reused below
    uint8_t* otile = astage[0];                          // [row][128] codes (16 KB)
    const int nbo = a.I >> 7;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int row = 64 * wr + 32 * g + rl;
        const float4 mm = *reinterpret_cast<const float4*>(red + row * 4);
        const float mx = fmaxf(fmaxf(mm.x, mm.y), fmaxf(mm.z, mm.w));
        const float s = div448(fmaxf(mx, 1e-10f));
        const float inv = __builtin_amdgcn_rcpf(s);
        u32 c[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2)
                c[t][i2] = (u32)__builtin_amdgcn_cvt_pk_fp8_f32(h[g][t][2 * i2] * inv,
                                                               h[g][t][2 * i2 + 1] * inv, 0, false);
        }
        store_codes(otile, row, wc, kh, c);
        osc[row] = s;
    }
    __syncthreads();
    if (threadIdx.x < ROWS && m0 + (int)threadIdx.x < a.M)
        a.out_scales[(int64_t)(m0 + threadIdx.x) * nbo + n_tile] = osc[threadIdx.x];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = (w + 8 * i) * 8 + (lane >> 3);
        if (m0 + row < a.M)
            st128(a.out + (int64_t)(m0 + row) * a.I + n_tile * 128 + (lane & 7) * 16,
                  lds128(otile + otile_off(row, lane & 7)));
    }
}

template <int DEPTH>
static hipError_t launch_gemm_big(const GemmActArgs& in, int act, hipStream_t s) {
    GemmActArgs a = in;
    a.mt = (a.M + 127) / 128;
    a.tiles = a.mt * (a.I / 128);
    a.per_xcd = (a.tiles + 7) / 8;
    const void* fn;
    switch (act) {
    case ACT_SWIGLU: fn = (const void*)k_gemm_act_big<ACT_SWIGLU, DEPTH>; break;
    case ACT_GEGLU_TANH: fn = (const void*)k_gemm_act_big<ACT_GEGLU_TANH, DEPTH>; break;
    default: fn = (const void*)k_gemm_act_big<ACT_SQRELU, DEPTH>; break;
    }
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3((unsigned)(8 * a.per_xcd)), dim3(512), args, 0, s);
}

template <int RG, int DEPTH>
static hipError_t launch_gemm_cfg(const GemmActArgs& in, int act, hipStream_t s) {
    GemmActArgs a = in;
    a.mt = (a.M + 32 * RG - 1) / (32 * RG);
    a.tiles = a.mt * (a.I / 128);
    a.per_xcd = (a.tiles + 7) / 8;
    const void* fn;
    switch (act) {
    case ACT_SWIGLU: fn = (const void*)k_gemm_act<ACT_SWIGLU, RG, DEPTH>; break;
    case ACT_GEGLU_TANH: fn = (const void*)k_gemm_act<ACT_GEGLU_TANH, RG, DEPTH>; break;
    default: fn = (const void*)k_gemm_act<ACT_SQRELU, RG, DEPTH>; break;
    }
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3((unsigned)(8 * a.per_xcd)), dim3(256), args, 0, s);
}

// Row groups per tile.  Measured on MI355X (hidden 2048 / 4096, inter 6144 /
// 12288, 128 to 4096 tokens): 64-row tiles win once they still give three
// quarters of the 256 CUs a tile (128 x 4096 x 12288: 192 tiles, 41.7 us vs
// 47.1 us with 32-row tiles), and also once 32-row tiles would need more
// than one workgroup on some CUs (192 x 2048 x 6144: 144 tiles of 64 rows
// 18.4 us vs 288 of 32 rows 19.9 us); 32-row tiles otherwise (128 x 2048 x
// 6144: 96 vs 192 tiles, 26.1 vs 19.1 us; 160 x 2048 x 6144: 144 vs 240
// tiles, 17.9 vs 15.5 us); 128-row tiles, 4 K blocks in flight, and waves
// loading their own activation fragments (no LDS stage) were never faster.
//
// Large batches take the 128-row, 8-wave tile once it gives at least three
// workgroups per CU (measured, outputs identical: 2048 x 2048 x 6144 88.0 ->
// 81.9 us, 2048 x 4096 x 12288 309 -> 286 us, 4096 x 4096 x 12288 596 -> 570
// us; with 1.5 rounds of workgroups it loses: 1024 x 2048 x 6144 46.6 ->
// 52.5 us, 512 x 4096 x 12288 82 -> 90 us), and also when its tiles fit in
// one round while 64-row tiles would not (512 x 2048 x 6144: 192 tiles
// 25.1 us vs 384 tiles of 64 rows 28.7 us; 384 x 2048 x 6144: 24.7 vs
// 25.2 us; with more than one round of its own it loses: 768 x 2048 x 6144
// 44.2 vs 39.8 us, 384 x 4096 x 12288 82.7 vs 73.8 us).
hipError_t launch_gemm_act(const GemmActArgs& in, int act, hipStream_t s) {
    const int64_t nt = in.I / 128;
    const int KB = in.K / 128;
    const int64_t t128 = ((int64_t)in.M + 127) / 128 * nt;
    const int64_t t64 = ((int64_t)in.M + 63) / 64 * nt;
    if (128 * KB <= kBigPanel && (t128 >= 768 || (t128 <= kCUs && t64 > kCUs)))
        return launch_gemm_big<2>(in, act, s);
    if (64 * KB <= kGemmPanel && (t64 >= 192 || ((int64_t)in.M + 31) / 32 * nt > kCUs))
        return launch_gemm_cfg<2, 2>(in, act, s);
    return launch_gemm_cfg<1, 2>(in, act, s);
}

// Weight packing: 16-byte unit i of the packed array is lane (i % 64) of
// chunk ((i / 64) % 4) of K block ((i / 256) % KB) of 32-row group
// (i / (256 KB)); it holds the bytes chunk_koff(c, lane / 32) .. +15 of K
// block kb of row 32 G + lane % 32.
__global__ __launch_bounds__(256) void k_pack_w(PackArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.units) return;
    const int lane = (int)(i & 63);
    const int c = (int)((i >> 6) & 3);
    const int64_t rest = i >> 8;
    const int64_t G = rest / a.KB;
    const int kb = (int)(rest - G * a.KB);
    const int64_t row = 32 * G + (lane & 31);
    const uint8_t* src = a.w + row * a.K + kb * 128 + chunk_koff(c, lane >> 5);
    st128(a.wp + i * 16, ld128(src));
}

hipError_t launch_pack_w(const PackArgs& in, hipStream_t s) {
    PackArgs a = in;
    a.KB = (int)(a.K >> 7);
    a.units = a.N * a.K / 16;
    void* args[] = {&a};
    return hipLaunchKernel((const void*)k_pack_w, dim3((unsigned)((a.units + 255) / 256)),
                           dim3(256), args, 0, s);
}

}  // namespace fr
