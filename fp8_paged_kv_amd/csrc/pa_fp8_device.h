// Device helpers shared by the decode kernels (internal header).
//
// Operand conventions of the 16x16x32 bf16 MFMA used for both products:
// lane l = n + 16*g holds 8 bf16 values of row/column n = l % 16 for k-slots
// 8g..8g+7 (g = l / 16); the 16x16 f32 result gives lane l the elements
// [4g + i][l % 16], i = 0..3.  Any permutation of k applied identically to
// both operands leaves the product unchanged, which the kernels use to pick
// k orders that match how the data is loaded.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.807354922057604f;   // log2(448)
constexpr float kDropLog2 = 40.f;         // a tile 2^40 below the running max adds nothing (dropped)

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// 4x4 byte transpose: out[c] byte k = in[k] byte c.
__device__ __forceinline__ void transpose4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                           uint32_t& o0, uint32_t& o1, uint32_t& o2, uint32_t& o3) {
    const uint32_t e0 = perm(b, a, 0x06020400u);   // a0 b0 a2 b2
    const uint32_t e1 = perm(b, a, 0x07030501u);   // a1 b1 a3 b3
    const uint32_t f0 = perm(d, c, 0x06020400u);   // c0 d0 c2 d2
    const uint32_t f1 = perm(d, c, 0x07030501u);   // c1 d1 c3 d3
    o0 = perm(f0, e0, 0x05040100u);                // a0 b0 c0 d0
    o1 = perm(f1, e1, 0x05040100u);                // a1 b1 c1 d1
    o2 = perm(f0, e0, 0x07060302u);                // a2 b2 c2 d2
    o3 = perm(f1, e1, 0x07060302u);                // a3 b3 c3 d3
}

// Four FP32 values to four E4M3 codes (RNE, no clamp), byte i = value i.
__device__ __forceinline__ uint32_t cvt4_fp8(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Four E4M3 codes (bytes of w) -> four exact bf16 values in two dwords.
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    lo = __builtin_bit_cast(uint32_t, a);
    hi = __builtin_bit_cast(uint32_t, b);
}

// Eight E4M3 codes (two dwords) -> the bf16x8 operand of one MFMA.
__device__ __forceinline__ bf16x8 fp8x8_to_op(uint32_t w0, uint32_t w1) {
    uint32_t d0, d1, d2, d3;
    fp8x4_to_bf16(w0, d0, d1);
    fp8x4_to_bf16(w1, d2, d3);
    const i32x4 v = {(int)d0, (int)d1, (int)d2, (int)d3};
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// Two FP32 values -> two bf16 rounded to nearest even, low half = a: one
// v_cvt_pk_bf16_f32.  For every one of the 2^32 inputs it gives the bits of
// rounding the pattern by hand (add 0x7fff plus the kept lsb, keep the high
// half; a NaN keeps its sign and top payload bits and becomes quiet), checked
// on the device; subnormals are kept.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) { return (uint16_t)pack_bf16x2(x, 0.f); }

// Broadcast lane n of every 16-lane row to the whole row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + N, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_max_over_groups(float v) {
    // max over lanes {l, l^16, l^32, l^48}
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    return v;
}

__device__ __forceinline__ float wave_sum_over_groups(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// token of k-slot (lane group g, byte j) inside a 32-token chunk; equals the
// token held in element i of MFMA block k of the S^T accumulator (j = 4k + i)
__device__ __forceinline__ int chunk_token(int g, int j) {
    return (j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4);
}

// Step 1 of the decode for 16 bf16 query values of one row: code = E4M3(q / qs),
// the quotient rounded as an IEEE FP32 division (the codes are decided in FP32),
// saturated to +-448 (the gfx950 convert rounds to nearest even but does not
// clamp).  raw: 8 dwords = 16 bf16; out: 4 dwords of codes, byte i = value i.
//
// One division per row instead of one per value: with y = RN(1/qs) and the
// product q0 = RN(q y) (a faithful quotient), the residual q - qs q0 is exact
// in one FMA and q0 + residual * y rounds to RN(q / qs) (Markstein's
// correction, IBM J. Res. Dev. 34(1), 1990).  It needs the residual to stay
// normal: taken for qs in [2^-60, 2^60] and quotients below 2048 in magnitude
// (a larger one saturates to 448 from either value; a zero keeps its sign);
// for |q| < 2^-100 the residual may underflow and the quotient be one unit
// off, but it is then below 2^-40 and its code is zero either way.  Any other
// qs (0, negative, tiny, huge, NaN) divides value by value.
struct QRecip {
    float qs, y;
    bool fast;
};
__device__ __forceinline__ QRecip q_recip(float qs) {
    QRecip r;
    r.qs = qs;
    r.fast = qs >= 0x1p-60f && qs <= 0x1p60f;
    r.y = r.fast ? 1.f / qs : 0.f;
    return r;
}
__device__ __forceinline__ void quantise_q16(const uint32_t raw[8], const QRecip& d, uint32_t out[4]) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        x[2 * i] = bf16_to_f32((uint16_t)(raw[i] & 0xffffu));
        x[2 * i + 1] = bf16_to_f32((uint16_t)(raw[i] >> 16));
    }
    if (d.fast) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float q = x[i] * d.y;
            if (q != 0.f && fabsf(q) < 2048.f) q = __builtin_fmaf(__builtin_fmaf(-d.qs, q, x[i]), d.y, q);
            x[i] = q;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = (d.qs == 0.f) ? 0.f : x[i] / d.qs;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_fmed3f(x[i], -448.f, 448.f);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = cvt4_fp8(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
}

}  // namespace pa
