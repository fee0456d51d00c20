// KvCompressEpilog quant modes 0 and 1 on gfx950: quantise bf16 rows and write
// them, in place, into the paged cache rows their slots name.
//
// Web page "CANN ops-transformer aclnnKvCompressEpilog 算子详解": section 功能说明
// -- the last 64 columns of a row x[t, 0:d] are its rope part (kept bf16), the
// first d - 64 its nope part, quantised per group to FP8 E4M3 with
// scale = max|x_g| / 448 (section 计算公式); mode 0 stores the scale as bf16,
// mode 1 as an e8m0 power of two (rounded up when roundScale); slot -1 skips
// the token.  Section 约束说明 / the kvCacheCol walkthrough fix the row:
// [rope bf16, 128 B][nope codes, d - 64 B][one scale per 64 nope columns:
// 2 B (mode 0) or 1 B (mode 1)], at cache + block * block_stride +
// offset * head_dim.
//
// Arithmetic: the scale is an fp32 division, mode 0 rounds it to bf16 (RNE) and
// divides by the stored bf16 value, mode 1 by 2^k (as a product with the exact
// 2^-k, which rounds the same quotient once); quotients are fp32, clamped to
// +-448 and rounded to E4M3 (RNE) -- the codes are decided in fp32, as on the
// page's vector unit.
//
// Work: one wave per token.  Lane l handles 8 consecutive nope columns (one
// 16-byte load); the 8 lanes of a 64-column group reduce its maximum with
// lane shuffles.  Rows may start at any byte (head_dim 323 is the page's own
// example), so stores are 8-byte stores when the row is 8-byte aligned and
// byte stores otherwise.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_fp8_common.h"
#include "pa_fp8_device.h"

namespace pa {

__device__ __forceinline__ void store8(uint8_t* p, uint32_t lo, uint32_t hi, bool aligned) {
    if (aligned) {
        *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = (uint8_t)(lo >> (8 * i));
            p[4 + i] = (uint8_t)(hi >> (8 * i));
        }
    }
}

// One row: rope bytes, codes and scales of one token, whose first 512 nope
// columns and rope the caller has loaded (lane l: columns 8l .. 8l + 7).
template <int MODE>
__device__ __forceinline__ void write_row(const EpilogParams& a, const uint16_t* xr, uint8_t* row, uint2 rope,
                                          i32x4 raw0, int lane) {
    const bool al8 = (reinterpret_cast<uintptr_t>(row) & 7) == 0;
    const int nope = a.d - 64;
    if (lane < 16) store8(row + 8 * lane, rope.x, rope.y, al8);
    for (int base = 0; base < nope; base += 512) {
        const int c0 = base + 8 * lane;
        const bool act = c0 < nope;
        float v[8];
        i32x4 raw = raw0;
        if (base > 0) {
            raw = i32x4{0, 0, 0, 0};
            if (act) raw = *reinterpret_cast<const i32x4*>(xr + c0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float((uint32_t)raw[i] << 16);
            v[2 * i + 1] = __uint_as_float((uint32_t)raw[i] & 0xFFFF0000u);
        }
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        m = fmaxf(m, __shfl_xor(m, 4, 64));
        const float scale = m / 448.f;
        float used, inv = 0.f;
        uint32_t sbits;
        if (MODE == 0) {
            const __bf16 sb = (__bf16)scale;
            used = (float)sb;
            sbits = __builtin_bit_cast(uint16_t, sb);
        } else {
            int k = -127;
            if (scale > 0.f) {
                int e2;
                const float f = frexpf(scale, &e2);            // scale = f 2^e2, f in [0.5, 1)
                k = (a.round_scale && f != 0.5f) ? e2 : e2 - 1;
                k = k < -127 ? -127 : (k > 127 ? 127 : k);
            }
            used = scale > 0.f ? ldexpf(1.f, k) : 0.f;
            // k <= 120 (scale <= bf16 max / 448 < 2^120), so 2^-k is a normal float and
            // x * 2^-k is the same correctly rounded number as x / 2^k, without a division
            inv = scale > 0.f ? ldexpf(1.f, -k) : 0.f;
            sbits = (uint32_t)(k + 127);
        }
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float y = MODE == 0 ? (used > 0.f ? v[i] / used : 0.f) : v[i] * inv;
            q[i] = fminf(fmaxf(y, -448.f), 448.f);
        }
        const uint32_t lo = cvt4_fp8(q[0], q[1], q[2], q[3]);
        const uint32_t hi = cvt4_fp8(q[4], q[5], q[6], q[7]);
        if (act) {
            store8(row + 128 + c0, lo, hi, al8);
            if ((lane & 7) == 0) {
                const int g = c0 / 64;
                uint8_t* sp = row + 128 + nope;
                if (MODE == 0) {
                    sp[2 * g] = (uint8_t)(sbits & 0xFF);
                    sp[2 * g + 1] = (uint8_t)(sbits >> 8);
                } else {
                    sp[g] = (uint8_t)sbits;
                }
            }
        }
    }
}

// The row's columns are requested together with its slot, not after the slot
// test: the two memory round trips overlap (a skipped token's columns are read
// for nothing, which costs less than a serial slot -> column chain per row).
template <typename SlotT, int MODE>
__global__ __launch_bounds__(256) void kv_compress_epilog_kernel(EpilogParams a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= a.num_tokens) return;
    const int nope = a.d - 64;
    const uint16_t* xr = a.x + t * a.d;
    const int64_t s = (int64_t)static_cast<const SlotT*>(a.slots)[t];
    uint2 rope = make_uint2(0u, 0u);
    i32x4 raw = {0, 0, 0, 0};
    if (lane < 16) rope = *reinterpret_cast<const uint2*>(xr + nope + 4 * lane);
    if (8 * lane < nope) raw = *reinterpret_cast<const i32x4*>(xr + 8 * lane);
    if (s < 0 || s >= a.num_slots) return;
    const int64_t blk = s / a.block_size, off = s - blk * a.block_size;
    write_row<MODE>(a, xr, a.cache + blk * a.block_stride + off * a.head_dim, rope, raw, lane);
}

hipError_t launch_kv_compress_epilog(const EpilogParams& p, int slot_bits, hipStream_t st) {
    const int64_t grid = (p.num_tokens + 3) / 4;
    if (grid <= 0) return hipSuccess;
    const dim3 g((unsigned)grid), b(256);
    if (slot_bits == 32) {
        if (p.mode == 0) hipLaunchKernelGGL((kv_compress_epilog_kernel<int32_t, 0>), g, b, 0, st, p);
        else hipLaunchKernelGGL((kv_compress_epilog_kernel<int32_t, 1>), g, b, 0, st, p);
    } else {
        if (p.mode == 0) hipLaunchKernelGGL((kv_compress_epilog_kernel<int64_t, 0>), g, b, 0, st, p);
        else hipLaunchKernelGGL((kv_compress_epilog_kernel<int64_t, 1>), g, b, 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace pa
