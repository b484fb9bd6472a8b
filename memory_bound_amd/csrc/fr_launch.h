// fr_launch.h -- host-side launch descriptors shared by the kernel files and
// the C-ABI layer.  Each launcher enqueues exactly one kernel on `stream` via
// hipLaunchKernel (which reports launch errors directly, without touching the
// thread's sticky error state) and returns its hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fr {

// Residual add + RMSNorm (+ optional adaptive modulation) + FP8.
struct NormArgs {
    const void* x;          // [T,H]
    const void* gate;       // [T,H]   (adaptive variant only)
    const void* res;        // [T,H]
    void* res_out;          // [T,H]
    const void* w;          // [H]     (plain variant, FR_W_MUL / FR_W_ONE_PLUS; LayerNorm)
    const void* b;          // [H]     (LayerNorm bias, may be NULL)
    const void* ada_scale;  // [T,H]   (adaptive variant only)
    const void* ada_shift;  // [T,H]   (adaptive variant only)
    uint8_t* out;           // [T,H] FP8, or [T,H/2] MX FP4
    float* scales;          // [T]     (FR_Q_TOKEN)
    uint8_t* mx_scales;     // [T,H/32] E8M0 (MX FP4 output) or [T,H/16] E4M3 (NVFP4)
    int64_t T;
    int H;
    int nw;                 // wavefronts per row
    int rpb;                // rows per workgroup (block = 64*nw*rpb threads)
    int wmode;
    int qmode;
    float eps;
    float static_scale;
    double inv_h;           // 1 / H: set by launch_norm
    float gscale;           // NVFP4 output: the tensor's fp32 dequantisation scale g
    double inv6g;           // NVFP4 output: 1 / (6 g), set by launch_norm
};

// Packed QKV split + per-head norm + RoPE + paged KV write.
struct QkvArgs {
    const void* qkv;
    const void* qw;
    const void* kw;
    const int32_t* pos;
    const int32_t* table;
    void* q_out;
    void* kc;
    void* vc;
    int32_t* err;
    int64_t T;
    int64_t tasks;          // T * groups wavefronts
    int Hq, Hkv, D;
    int groups;             // head groups (64/LP heads each) per token, one wave each
    int table_len, page_size, num_pages;
    int style;
    float eps;
    float theta;
    float q_scale;          // multiplies Q after RoPE
    double l2t;             // -2 log2(theta) / D: set by launch_qkv
    float inv_d;            // 1 / D: set by launch_qkv
};

// Gated activation on interleaved gate/up + block-128 FP8.
struct ActArgs {
    const void* gu;         // [T,2I]
    uint8_t* out;           // [T,I] FP8, or [T,I/2] MX FP4
    float* scales;          // [T,I/128]
    uint8_t* mx_scales;     // [T,I/32] E8M0 (MX FP4 output)
    int64_t T;
    int64_t waves;          // T * wpr
    int I;
    int nb;                 // I / 128
    int wpr;                // wavefronts per row
};

// FP8 block-scaled GEMM (gate_up projection) + gated activation + block-128 FP8.
struct GemmActArgs {
    const uint8_t* A;       // [M, K] e4m3
    const float* a_scales;  // [M, K/128]
    const uint8_t* B;       // [2I, K] e4m3, gate/up rows interleaved, packed
    const float* b_scales;  // [2I/128, K/128]
    uint8_t* out;           // [M, I]
    float* out_scales;      // [M, I/128]
    int M, K, I;
    int mt;                 // row tiles
    int tiles;              // mt * (I / 128)
    int per_xcd;            // ceil(tiles / 8)
};

// Weight packing for the GEMM above (a permutation of 16-byte units).
struct PackArgs {
    const uint8_t* w;       // [N, K] e4m3 row-major
    uint8_t* wp;            // packed, N * K bytes
    int64_t N, K;
    int KB;                 // K / 128
    int64_t units;          // N * K / 16
};

// The decoder-step chain (op a' then op b per layer and flow step) in one
// persistent launch: one wave (or four, for rows over 512 values) per token
// row, further waves per head units.
constexpr int kChainMaxT = 64;
constexpr int kChainMaxH = 4 * 64 * 4;          // one 4-value chunk per lane of four waves
struct ChainArgs {
    const void* x;          // [layers, T, H]
    const void* gate;       // [N, T, H]  (N = layers * steps)
    const void* ada_scale;  // [N, T, H]
    const void* ada_shift;  // [N, T, H]
    void* res;              // [N + 1, T, H]
    uint8_t* out;           // [N, T, H]
    const void* qkv;        // [layers, T, (Hq + 2 Hkv) D]
    const int32_t* pos;     // [T]
    const int32_t* table;
    void* q_out;            // [layers, T, Hq, D]
    void* kc;               // [layers, pages, page_size, Hkv, D]
    void* vc;
    int32_t* err;
    int layers, steps, T, H, Hq, Hkv, D;
    int table_len, page_size, num_pages;
    int style;
    float eps, static_scale, theta;
};
hipError_t launch_chain(const ChainArgs& a, int dtype, hipStream_t s);

// Packed QKV split + Q/K norm (RMS / Layer, per head / full width) + RoPE
// (1D / 3D) into separate Q, K, V outputs.
struct QkNormArgs {
    const void* qkv;        // [T, (Hq + 2 Hkv) D]
    const void* qw;         // [D] or [Hq D]
    const void* qb;
    const void* kw;         // [D] or [Hkv D]
    const void* kb;
    const int32_t* pos;     // [T] or [T, 3]
    void* q_out;            // [T, Hq, D]
    void* k_out;            // [T, Hkv, D]
    void* v_out;            // [T, Hkv, D]
    int64_t T;
    int Hq, Hkv, D;
    int norm_kind;          // 0 none, 1 RMS, 2 Layer
    int full;               // norm over the full Q (K) width
    int split;              // workgroups per token (each one pass of heads), or 1
    int rope3;              // 3D RoPE
    int sec[3];             // 3D RoPE pairs per axis
    int style;
    float eps, theta, q_scale;
    double inv_nq, inv_nk;  // 1 / (Hq D), 1 / (Hkv D): set by launch_qknr
};
hipError_t launch_qknr(const QkNormArgs& a, int dtype, hipStream_t s);

enum { NORM_FP8 = 0, NORM_ADA_FP8 = 1, NORM_MXFP4 = 2, NORM_LAYER_FP8 = 3, NORM_LAYER_MXFP4 = 4,
       NORM_NVFP4 = 5, NORM_LAYER_NVFP4 = 6 };
hipError_t launch_norm(const NormArgs& a, int dtype, int kind, hipStream_t s);
hipError_t launch_qkv(const QkvArgs& a, int dtype, hipStream_t s);
hipError_t launch_act(const ActArgs& a, int dtype, int act, bool mx, hipStream_t s);
hipError_t launch_gemm_act(const GemmActArgs& a, int act, hipStream_t s);
hipError_t launch_pack_w(const PackArgs& a, hipStream_t s);

}  // namespace fr
