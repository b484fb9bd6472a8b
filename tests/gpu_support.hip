// gpu_support.hip -- test and measurement support, not part of the library.
//
// 1. mfma_probe_e4m3: runs the gfx950 e4m3 matrix instruction that the fused
//    gate_up GEMM uses (v_mfma_scale_f32_32x32x64_f8f6f4, e4m3 x e4m3, unit MX
//    scales) on given operand tiles, so that a test can compare the
//    instruction's sums with the exact ones computed on the host.
//
//    Operands: x, y are n tiles of 32 rows x 128 bytes (e4m3 codes,
//    row-major, K contiguous).  For each tile the kernel starts from a zero
//    accumulator and issues `ninstr` (1 or 2) instructions over K = [0, 64)
//    and [64, 128), exactly as the GEMM forms one 128-wide K block's partial
//    sum, and writes out[tile][i][j] = sum_k x[tile][i][k] * y[tile][j][k] as
//    computed by the hardware (fp32, [n][32][32] row-major).
//
//    Fragment layout of the instruction (the same one the GEMM's packed
//    weight layout serves): lane l holds row l % 32 and the 32 bytes
//    K = [32 (l / 32), +32) of the instruction's 64; the result value r of
//    lane l is row 8 (r / 4) + 4 (l / 32) + r % 4 of x and row l % 32 of y.
//
// 2. stream_copy: a plain streaming copy (one 16-byte chunk per thread, a
//    one-shot grid, non-temporal or cacheable), the reference the benchmark
//    reports as the bandwidth a kernel can reach for a given traffic on this
//    GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(64) void k_mfma_probe(const uint8_t* x, const uint8_t* y,
                                                   float* out, int n, int ninstr) {
    const int tile = blockIdx.x;
    if (tile >= n) return;
    const int l = threadIdx.x;
    const int row = l & 31, kh = l >> 5;
    const uint8_t* xt = x + (size_t)tile * 32 * 128 + row * 128;
    const uint8_t* yt = y + (size_t)tile * 32 * 128 + row * 128;
    f32x16 c = {};
    for (int i = 0; i < ninstr; ++i) {
        const int k0 = 64 * i + 32 * kh;
        i32x8 xa, ya;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            xa[q] = *(const int*)(xt + k0 + 4 * q);
            ya[q] = *(const int*)(yt + k0 + 4 * q);
        }
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa, ya, c, 0, 0, 0, 127, 0, 127);
    }
    float* ot = out + (size_t)tile * 32 * 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) ot[(8 * (r >> 2) + 4 * kh + (r & 3)) * 32 + row] = c[r];
}

// Returns 0 on success, 2 on a bad argument (nothing launched), 7 if the
// launch failed.  x, y: device pointers to n * 4096 bytes each, 4-byte
// aligned; out: device pointer to n * 1024 floats.
extern "C" __attribute__((visibility("default")))
int mfma_probe_e4m3(const void* x, const void* y, void* out, int n, int ninstr, void* stream) {
    if (n < 0 || (ninstr != 1 && ninstr != 2) || x == nullptr || y == nullptr || out == nullptr)
        return 2;
    if ((((uintptr_t)x) | ((uintptr_t)y) | ((uintptr_t)out)) & 3u) return 2;
    if (n == 0) return 0;
    const uint8_t* xp = (const uint8_t*)x;
    const uint8_t* yp = (const uint8_t*)y;
    float* op = (float*)out;
    void* args[] = {&xp, &yp, &op, &n, &ninstr};
    return hipLaunchKernel((const void*)k_mfma_probe, dim3(n), dim3(64), args, 0,
                           (hipStream_t)stream) == hipSuccess ? 0 : 7;
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ __launch_bounds__(256) void k_stream_copy(const u32x4_t* src, u32x4_t* dst, long n16) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n16) return;
    if constexpr (NT) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
    else dst[i] = src[i];
}

// Copies n16 16-byte chunks from src to dst (device pointers, 16-byte
// aligned, not overlapping).  Returns 0, 2 on a bad argument (nothing
// launched) or 7 if the launch failed.
extern "C" __attribute__((visibility("default")))
int stream_copy(const void* src, void* dst, long n16, int nontemporal, void* stream) {
    if (n16 < 0 || src == nullptr || dst == nullptr) return 2;
    if ((((uintptr_t)src) | ((uintptr_t)dst)) & 15u) return 2;
    if (n16 == 0) return 0;
    if ((n16 + 255) / 256 > 0x7fffffffL) return 2;
    const u32x4_t* s = (const u32x4_t*)src;
    u32x4_t* d = (u32x4_t*)dst;
    void* args[] = {&s, &d, &n16};
    const void* fn = nontemporal ? (const void*)k_stream_copy<true> : (const void*)k_stream_copy<false>;
    return hipLaunchKernel(fn, dim3((unsigned)((n16 + 255) / 256)), dim3(256), args, 0,
                           (hipStream_t)stream) == hipSuccess ? 0 : 7;
}
