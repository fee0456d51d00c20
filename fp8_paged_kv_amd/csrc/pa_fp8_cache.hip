// FP8 KV-cache writer on gfx950: the in-place slot scatter that fills the paged
// caches the decode reads.
//
// Web page on ops-transformer's scatter_pa_kv_cache_with_k_scale, section
// 功能说明与计算公式: for every token i and head j, block = slot[i] / block_size and
// offset = slot[i] % block_size; the token's FP8 key row, value row and FP32 key
// scale of head j are copied to that (block, head, offset) of the key cache,
// value cache and key-scale cache.  Sections 约束说明 and the SIMT kernel notes:
// a slot below 0 or above num_blocks * block_size - 1 is skipped; slots are
// distinct (a repeated slot is the caller's error).
//
// Two cache layouts: BSND [block, offset, head, d] with scales [block, offset,
// head] -- the layout of the GLM-4.5 paged-attention page's kernel signature,
// which the decode kernels read -- and BNBD [block, head, offset, d] with
// scales [block, head, offset], the writer page's documented default.
//
// HBM-bound copy.  One wave moves two tokens: both rows (key, value) of each, as
// 16-byte pieces, all four rows' loads issued before their stores.  In BSND a
// token's rows land contiguously (slot * num_head * head_size); in BNBD each
// head's piece goes to its own (block, head) plane.  Lanes below num_head copy
// the key scales.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_fp8_common.h"
#include "pa_fp8_device.h"

namespace pa {

template <typename SlotT, int LAYOUT>
__global__ __launch_bounds__(256) void scatter_kv_kernel(ScatterParams a) {
    constexpr int kTok = 2;                               // tokens per wave
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tok0 = wave * kTok;
    if (tok0 >= a.num_tokens) return;

    int64_t slot[kTok];
    bool ok[kTok];
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
        const int64_t tok = tok0 + t;
        const int64_t s = tok < a.num_tokens ? (int64_t)static_cast<const SlotT*>(a.slots)[tok] : -1;
        ok[t] = s >= 0 && s < a.num_slots;
        slot[t] = ok[t] ? s : 0;
    }
    const int H = a.num_head, bs = a.block_size;
    const int kp = H * a.k_head_size / 16, vp = H * a.v_head_size / 16;   // 16-byte pieces per row
    const int np = kp > vp ? kp : vp;
    for (int base = 0; base < np; base += 64) {
        const int i = base + lane;
        i32x4 x[2 * kTok];
#pragma unroll
        for (int u = 0; u < 2 * kTok; ++u) {
            const int t = u >> 1;
            const bool v = u & 1;
            if (ok[t] && i < (v ? vp : kp)) {
                const uint8_t* src = (v ? a.value : a.key) + (tok0 + t) * (v ? a.v_stride : a.k_stride) + 16 * i;
                x[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(src));
            }
        }
#pragma unroll
        for (int u = 0; u < 2 * kTok; ++u) {
            const int t = u >> 1;
            const bool v = u & 1;
            if (ok[t] && i < (v ? vp : kp)) {
                const int hs = v ? a.v_head_size : a.k_head_size;
                int64_t dst;
                if (LAYOUT == 0) {
                    dst = slot[t] * ((int64_t)H * hs) + 16 * i;
                } else {
                    const int64_t blk = slot[t] / bs, off = slot[t] - blk * bs;
                    const int h = (16 * i) / hs, d = 16 * i - h * hs;
                    dst = ((blk * H + h) * bs + off) * hs + d;
                }
                uint8_t* cache = v ? a.value_cache : a.key_cache;
                __builtin_nontemporal_store(x[u], reinterpret_cast<i32x4*>(cache + dst));
            }
        }
    }
    for (int h = lane; h < H; h += 64) {
#pragma unroll
        for (int t = 0; t < kTok; ++t) {
            if (!ok[t]) continue;
            const float s = a.key_scale[(tok0 + t) * a.ks_token_stride + (int64_t)h * a.ks_head_stride];
            int64_t dst;
            if (LAYOUT == 0) {
                dst = slot[t] * H + h;
            } else {
                const int64_t blk = slot[t] / bs, off = slot[t] - blk * bs;
                dst = (blk * H + h) * bs + off;
            }
            a.key_scale_cache[dst] = s;
        }
    }
}

hipError_t launch_scatter_kv(const ScatterParams& p, int slot_bits, int layout, hipStream_t st) {
    const int64_t waves = (p.num_tokens + 1) / 2;
    const int64_t grid = (waves + 3) / 4;
    if (grid <= 0) return hipSuccess;
    const dim3 g((unsigned)grid), b(256);
    if (slot_bits == 32) {
        if (layout == 0) hipLaunchKernelGGL((scatter_kv_kernel<int32_t, 0>), g, b, 0, st, p);
        else hipLaunchKernelGGL((scatter_kv_kernel<int32_t, 1>), g, b, 0, st, p);
    } else {
        if (layout == 0) hipLaunchKernelGGL((scatter_kv_kernel<int64_t, 0>), g, b, 0, st, p);
        else hipLaunchKernelGGL((scatter_kv_kernel<int64_t, 1>), g, b, 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace pa
