// fr_device.h -- gfx950 device helpers shared by the fused kernels:
// 16-bit storage conversions, saturating OCP E4M3 packing, and wave64
// cross-lane reductions built from DPP row operations and the gfx950
// permlane swaps (no LDS traffic inside a wavefront).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fr {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

enum { DT_F16 = 0, DT_BF16 = 1 };

// ---------------------------------------------------------------------------
// 16-bit storage types, two values per 32-bit word (element 2k in the low
// half, 2k+1 in the high half).
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float lo16(u32 w) {
    if constexpr (DT == DT_BF16)
        return __uint_as_float(w << 16);
    else
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}

template <int DT>
__device__ __forceinline__ float hi16(u32 w) {
    if constexpr (DT == DT_BF16)
        return __uint_as_float(w & 0xffff0000u);
    else
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Round two fp32 values to the storage type (nearest, ties to even) and pack.
template <int DT>
__device__ __forceinline__ u32 pack16(float a, float b) {
    if constexpr (DT == DT_BF16) {
        bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
        return __builtin_bit_cast(u32, v);
    } else {
        f16x2 v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(u32, v);
    }
}

// Round-to-odd of the exact value p + e, where p = fp32(p + e) and e is the
// (small) remainder: if e != 0 and p's last significand bit is even, step one
// ulp towards the exact value.  A later rounding of the result to a format
// with at least two fewer significand bits (e4m3 has 4) is then the correct
// rounding of p + e.
__device__ __forceinline__ float round_odd(float p, float e) {
    const u32 b = __float_as_uint(p);
    // +1 (away from zero) when e has the sign of p, else -1; only an even
    // significand moves
    const u32 dir = (u32)((int)(__float_as_uint(e) ^ b) >> 31) | 1u;
    const u32 even = (b & 1u) - 1u;                      // all ones if b is even
    return __uint_as_float(b + (e != 0.0f ? (dir & even) : 0u));
}

// r + p rounded to fp32 with round-to-odd: TwoSum gives s = fp32(r + p) and
// the exact error e of that sum, and round_odd moves an even s one ulp
// towards the exact value.  Rounding the result once more to a format with
// at most 22 bits of precision (fp16, bf16) gives the correctly rounded exact
// sum, because fp32 keeps at least two extra bits.  (s is 0 only when r + p
// is exactly 0: a sum of two fp32 values that rounds to 0 is representable,
// so e is 0 there and no step is taken.)
__device__ __forceinline__ float add_round_odd(float r, float p) {
    const float s = r + p;
    const float bb = s - r;
    const float e = (r - (s - bb)) + (p - bb);
    return round_odd(s, e);
}

// ---------------------------------------------------------------------------
// OCP E4M3 ("fn") packing.  v_cvt_pk_fp8_f32 rounds to nearest-even with
// subnormals but turns magnitudes above 464 into NaN, so values are clamped
// to +-448 first (med3), which makes the conversion saturating.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sat448(float v) {
    return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

__device__ __forceinline__ u32 pack_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
    return (u32)w;
}
// The same for values already known to lie within +-464 (the conversion is
// then exact RNE and saturates at 448 by itself): no clamp.
__device__ __forceinline__ u32 pack_e4m3x4_in_range(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (u32)w;
}

// ---------------------------------------------------------------------------
// Cross-lane reductions.  DPP row operations combine lanes inside a 16-lane
// row: quad_perm [1,0,3,2] (pairs), quad_perm [2,3,0,1] (quads),
// row_half_mirror (8 lanes), row_mirror (16 lanes).  After the first k steps
// every lane holds the result over its aligned group of 2^k lanes.  The
// gfx950 permlane16/32 swaps then combine rows.  Every lane ends with the
// same value, and the combination order is fixed (deterministic).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    u32x2 w = __builtin_bit_cast(u32x2, v);
    w.x = (u32)__builtin_amdgcn_update_dpp(0, (int)w.x, CTRL, 0xF, 0xF, true);
    w.y = (u32)__builtin_amdgcn_update_dpp(0, (int)w.y, CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(double, w);
}

enum { DPP_PAIR = 0xB1, DPP_QUAD = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140,
       DPP_ROR2 = 0x122, DPP_ROR4 = 0x124, DPP_ROR8 = 0x128 };   // rotations in a row

struct OpSum {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
    __device__ __forceinline__ double operator()(double a, double b) const { return a + b; }
};
struct OpMax {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
// Maximum of non-negative floats (magnitudes) as unsigned integers: the bit
// patterns of non-negative floats are ordered like the values, and the
// integer maximum needs no NaN canonicalisation of the operands.
struct OpMaxMag {
    __device__ __forceinline__ float operator()(float a, float b) const {
        return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b)));
    }
};

// Reduce over aligned groups of G lanes (G = 1, 2, 4, 8 or 16).
template <int G, class Op>
__device__ __forceinline__ float group_reduce(float v, Op op) {
    if constexpr (G >= 2) v = op(v, dpp_f<DPP_PAIR>(v));
    if constexpr (G >= 4) v = op(v, dpp_f<DPP_QUAD>(v));
    if constexpr (G >= 8) v = op(v, dpp_f<DPP_HALF_MIRROR>(v));
    if constexpr (G >= 16) v = op(v, dpp_f<DPP_MIRROR>(v));
    return v;
}

// Combine 16-lane rows pairwise (rows 0+1, rows 2+3).
template <class Op>
__device__ __forceinline__ float rows_pair(float v, Op op) {
    u32 u = __builtin_bit_cast(u32, v);
    auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return op(__builtin_bit_cast(float, (u32)p[0]), __builtin_bit_cast(float, (u32)p[1]));
}

// Combine the two 32-lane halves.
template <class Op>
__device__ __forceinline__ float halves(float v, Op op) {
    u32 u = __builtin_bit_cast(u32, v);
    auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return op(__builtin_bit_cast(float, (u32)p[0]), __builtin_bit_cast(float, (u32)p[1]));
}

template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
    v = group_reduce<16>(v, op);
    v = rows_pair(v, op);
    return halves(v, op);
}

__device__ __forceinline__ double swap16_sum(double v) {
    u32x2 w = __builtin_bit_cast(u32x2, v);
    auto px = __builtin_amdgcn_permlane16_swap(w.x, w.x, false, false);
    auto py = __builtin_amdgcn_permlane16_swap(w.y, w.y, false, false);
    u32x2 a = {(u32)px[0], (u32)py[0]}, b = {(u32)px[1], (u32)py[1]};
    return __builtin_bit_cast(double, a) + __builtin_bit_cast(double, b);
}

__device__ __forceinline__ double swap32_sum(double v) {
    u32x2 w = __builtin_bit_cast(u32x2, v);
    auto px = __builtin_amdgcn_permlane32_swap(w.x, w.x, false, false);
    auto py = __builtin_amdgcn_permlane32_swap(w.y, w.y, false, false);
    u32x2 a = {(u32)px[0], (u32)py[0]}, b = {(u32)px[1], (u32)py[1]};
    return __builtin_bit_cast(double, a) + __builtin_bit_cast(double, b);
}

__device__ __forceinline__ double wave_sum_d(double v) {
    v += dpp_d<DPP_PAIR>(v);
    v += dpp_d<DPP_QUAD>(v);
    v += dpp_d<DPP_HALF_MIRROR>(v);
    v += dpp_d<DPP_MIRROR>(v);
    v = swap16_sum(v);
    return swap32_sum(v);
}

// ---------------------------------------------------------------------------
// Gate activations (fp32): SiLU for SwiGLU, GELU with the tanh approximation
// for GeGLU, squared ReLU.  v_exp_f32 / v_rcp_f32 are ~1 ulp.
// ---------------------------------------------------------------------------
enum { ACT_SWIGLU = 0, ACT_GEGLU_TANH = 1, ACT_SQRELU = 2 };

template <int ACT>
__device__ __forceinline__ float gate_act(float g) {
    constexpr float kLog2e = 1.4426950408889634f;
    if constexpr (ACT == ACT_SWIGLU) {
        // g * sigmoid(g) = g / (1 + 2^(-g log2 e))
        const float e = __builtin_amdgcn_exp2f(-g * kLog2e);
        return g * __builtin_amdgcn_rcpf(1.0f + e);
    } else if constexpr (ACT == ACT_GEGLU_TANH) {
        // 0.5 g (1 + tanh z) = g * sigmoid(2z), z = sqrt(2/pi)(g + 0.044715 g^3);
        // the sigmoid form has no cancellation for negative z.
        constexpr float c1 = 2.0f * 0.7978845608028654f * kLog2e;
        constexpr float c3 = 2.0f * 0.7978845608028654f * 0.044715f * kLog2e;
        const float g2 = g * g;
        const float arg = g * fmaf(c3, g2, c1);            // 2z log2 e
        const float e = __builtin_amdgcn_exp2f(-arg);
        return g * __builtin_amdgcn_rcpf(1.0f + e);
    } else {
        const float r = fmaxf(g, 0.0f);
        return r * r;
    }
}

// fp64 row scalars without the runtime's division and square-root
// sequences: the hardware estimates refined by two Newton steps each
// (an estimate good to ~2^-22 becomes good to the last bits of fp64), and
// the quotient by 448 as a product with one remainder correction.
__device__ __forceinline__ double rsqrt_d(double x) {         // x > 0
    double y = __builtin_amdgcn_rsq(x);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const double e = fma(-(x * y), y, 1.0);               // 1 - x y^2
        y = fma(0.5 * y, e, y);
    }
    return y;
}
__device__ __forceinline__ double rcp_d(double x) {           // x > 0
    double r = __builtin_amdgcn_rcp(x);
#pragma unroll
    for (int i = 0; i < 2; ++i) r = fma(r, fma(-x, r, 1.0), r);
    return r;
}
__device__ __forceinline__ double div448_d(double v) {
    constexpr double kInv = 1.0 / 448.0;
    const double q0 = v * kInv;
    return fma(fma(-q0, 448.0, v), kInv, q0);
}

// Correctly rounded amax / 448: q0 = amax * (1/448), then one fma correction
// with the exact remainder amax - q0 * 448.
__device__ __forceinline__ float div448(float amax) {
    constexpr float kInv448 = 1.0f / 448.0f;
    const float q0 = amax * kInv448;
    return fmaf(fmaf(-q0, 448.0f, amax), kInv448, q0);
}

// ---------------------------------------------------------------------------
// Global memory access: 128-bit vector loads/stores.
// ---------------------------------------------------------------------------
// MX FP4 (OCP MXFP4: E2M1 elements, blocks of 32, E8M0 scale).  The block
// scale is 2^(floor(log2 amax) - 2), so the block maximum lands in [4, 8):
// with E the biased fp32 exponent of amax, the E8M0 code is E - 2 (0 for
// amax below 2^-124, zero included), and the elements are amax-relative
// values times 2^(127 - code), a power of two (exact).  The conversion
// v_cvt_scalef32_pk_fp4_f32 rounds to nearest even on the E2M1 grid,
// saturates at 6 and keeps the sign of values that round to zero (checked
// on MI355X); with scale 1 it converts the values as given.
__device__ __forceinline__ int mx_code(float amax) {
    const int E = (int)((__builtin_bit_cast(u32, amax) >> 23) & 0xFF);
    return E > 2 ? E - 2 : 0;
}
__device__ __forceinline__ float mx_mult(int code) {          // 2^(127 - code)
    return __builtin_bit_cast(float, (u32)(254 - code) << 23);
}
// 8 values -> 8 E2M1 codes, value 2i in the low nibble of byte i.
__device__ __forceinline__ u32 pack_e2m1x8(const float* v, float m) {
    u32 p = 0;
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[0] * m, v[1] * m, 1.0f, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[2] * m, v[3] * m, 1.0f, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[4] * m, v[5] * m, 1.0f, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[6] * m, v[7] * m, 1.0f, 3);
    return p;
}
// 4 values -> 4 E2M1 codes in the low 16 bits.
__device__ __forceinline__ u32 pack_e2m1x4(float a, float b, float c, float d, float m) {
    u32 p = 0;
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, a * m, b * m, 1.0f, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, c * m, d * m, 1.0f, 1);
    return p;
}

// sin and cos of x (radians).  k = nearest integer to x/(pi/2), r = x - k*pi/2
// with pi/2 split into a head (the double nearest pi/2) and its tail; fma
// keeps k*head exact.  Taylor series to r^11 / r^12 (truncation < 1e-11 on
// |r| <= pi/4), then the quadrant of k picks and signs the two.
__device__ __forceinline__ void sincos_pos(double x, float* s_out, float* c_out) {
    const double two_over_pi = 0.63661977236758134308;
    const double pio2_hi = 1.5707963267948966;          // nearest double to pi/2
    const double pio2_lo = 6.123233995736766e-17;       // pi/2 - pio2_hi
    const double k = rint(x * two_over_pi);
    double r = fma(-k, pio2_hi, x);
    r = fma(-k, pio2_lo, r);
    const double r2 = r * r;
    // 1/n! coefficients
    double sp = 2.505210838544172e-08;                  // 1/11!
    sp = fma(sp, r2, -2.7557319223985893e-06);          // 1/9!
    sp = fma(sp, r2, 1.984126984126984e-04);            // 1/7!
    sp = fma(sp, r2, -8.333333333333333e-03);           // 1/5!
    sp = fma(sp, r2, 1.6666666666666666e-01);           // 1/3!
    const double sn = fma(-r * r2, sp, r);
    double cp = 2.08767569878681e-09;                   // 1/12!
    cp = fma(cp, r2, -2.755731922398589e-07);           // 1/10!
    cp = fma(cp, r2, 2.48015873015873e-05);             // 1/8!
    cp = fma(cp, r2, -1.388888888888889e-03);           // 1/6!
    cp = fma(cp, r2, 4.1666666666666664e-02);           // 1/4!
    cp = fma(cp, r2, -0.5);                             // 1/2!
    const double cs = fma(cp, r2, 1.0);
    // quadrant q: (sin, cos) = (sn, cs), (cs, -sn), (-sn, -cs), (-cs, sn);
    // selects rather than branches (q differs between lanes)
    const int q = (int)((long long)k & 3);
    double s = (q & 1) ? cs : sn;
    double c = (q & 1) ? sn : cs;
    s = (q & 2) ? -s : s;
    c = ((q + 1) & 2) ? -c : c;
    *s_out = (float)s;
    *c_out = (float)c;
}

__device__ __forceinline__ u32x4 ld128(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld128_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st128(void* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ void st128_stream(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st64(void* p, u32x2 v) {
    *reinterpret_cast<u32x2*>(p) = v;
}
__device__ __forceinline__ void st64_stream(void* p, u32x2 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace fr
