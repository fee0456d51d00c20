// Bandwidth probes for the paged FP8 decode's memory access pattern (a
// measurement tool beside the decode library, not part of its ABI).
//
// Each probe reads bytes and folds them into one XOR word per workgroup
// (written to `sink`), so the loads cannot be dropped; nothing else is
// computed.  They give the read rate the hardware sustains for:
//  * probe_paged_kernel: the bytes the decode must read, in the decode's cache
//    layout -- for every (batch, pair of KV heads, 128-token block) of the
//    valid blocks, the 256-byte K and V slices of the pair in each of the 128
//    token rows and the pair's two k_scale words per token -- one workgroup per
//    such block (blocks past a sequence exit at once), the hardware
//    dispatcher balancing the load;
//  * probe_contiguous_kernel: a plain contiguous read of a buffer with 16-byte
//    loads, grid-strided.
// Beside them: the FP8 MFMA against exact sums, the issue rate of the VALU
// instructions that dequantise FP8 codes, and the LDS read rate of lane address patterns.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold_wg(uint32_t x, uint32_t* red) {
    for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    uint32_t r = 0;
    if (threadIdx.x == 0)
        for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r ^= red[i];
    return r;
}

// grid = B * (nkv / NH) * max_blocks, 256 threads.  Workgroup (v, blk): batch
// v / NG, KV heads NH (v % NG) .. + NH - 1, block blk of the sequence: the NH
// heads' K and V slices (NH * 128 contiguous bytes of each token row) and their
// k_scale words, 16 loads in flight per thread.
template <int NH>
__global__ __launch_bounds__(256) void probe_paged_kernel(const uint8_t* k_cache, const float* k_scale,
                                                          const uint8_t* v_cache, const int32_t* table,
                                                          const int32_t* seqs, int nkv, int max_blocks,
                                                          int num_blocks, uint32_t* sink) {
    __shared__ uint32_t red[4];
    constexpr int PPT = NH * 8;                           // 16-byte pieces per token slice
    const int NG = nkv / NH;
    const int blk = blockIdx.x % max_blocks, v = blockIdx.x / max_blocks;
    const int b = v / NG, h0 = NH * (v % NG);
    const int seq = seqs[b];
    if (blk * 128 >= seq) return;
    int id = table[(int64_t)b * max_blocks + blk];
    id = (id < 0 || id >= num_blocks) ? 0 : id;
    const int64_t tok_stride = (int64_t)nkv * 128;
    const uint8_t* kb = k_cache + (int64_t)id * 128 * tok_stride + h0 * 128;
    const uint8_t* vb = v_cache + (int64_t)id * 128 * tok_stride + h0 * 128;
    uint32_t x = 0;
#pragma unroll
    for (int r0 = 0; r0 < NH / 2; ++r0) {                // rounds of 8 K + 8 V pieces per thread
        u32x4 kv[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int piece = (r0 * 8 + i) * 256 + threadIdx.x;
            const int t = piece / PPT, o = (piece % PPT) * 16;
            kv[i] = *reinterpret_cast<const u32x4*>(kb + t * tok_stride + o);
            kv[8 + i] = *reinterpret_cast<const u32x4*>(vb + t * tok_stride + o);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) x ^= kv[i][0] ^ kv[i][1] ^ kv[i][2] ^ kv[i][3];
    }
#pragma unroll
    for (int j = 0; j < NH / 2; ++j) {
        const int w = j * 256 + threadIdx.x;              // k_scale word: token w / NH, head w % NH
        x ^= __float_as_uint(k_scale[((int64_t)id * 128 + w / NH) * nkv + h0 + w % NH]);
    }
    const uint32_t r = fold_wg(x, red);
    if (threadIdx.x == 0) sink[blockIdx.x] = r;
}

// U 16-byte loads in flight per thread
template <int U>
__global__ __launch_bounds__(256) void probe_contiguous_kernel(const u32x4* p, int64_t n16, uint32_t* sink) {
    __shared__ uint32_t red[4];
    uint32_t x = 0;
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    for (int64_t i = (int64_t)blockIdx.x * 256 * U + threadIdx.x; i < n16; i += stride) {
        u32x4 a[U];
#pragma unroll
        for (int j = 0; j < U; ++j) a[j] = (i + j * 256 < n16) ? p[i + j * 256] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < U; ++j) x ^= a[j][0] ^ a[j][1] ^ a[j][2] ^ a[j][3];
    }
    const uint32_t r = fold_wg(x, red);
    if (threadIdx.x == 0) sink[blockIdx.x] = r;
}

// Persistent form of probe_paged_kernel: `gridDim.x` workgroups walk the
// (batch, KV-head pair, block) items with a stride, the next item's loads issued
// before the current one is folded.
__global__ __launch_bounds__(256) void probe_paged_persistent_kernel(const uint8_t* k_cache, const float* k_scale,
                                                                     const uint8_t* v_cache, const int32_t* table,
                                                                     const int32_t* seqs, int nkv, int max_blocks,
                                                                     int num_blocks, int items, uint32_t* sink) {
    __shared__ uint32_t red[4];
    const int NG = nkv / 2;
    const int64_t tok_stride = (int64_t)nkv * 128;
    uint32_t x = 0;
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int blk = it % max_blocks, v = it / max_blocks;
        const int b = v / NG, h0 = 2 * (v % NG);
        if (blk * 128 >= seqs[b]) continue;
        int id = table[(int64_t)b * max_blocks + blk];
        id = (id < 0 || id >= num_blocks) ? 0 : id;
        const uint8_t* kb = k_cache + (int64_t)id * 128 * tok_stride + h0 * 128;
        const uint8_t* vb = v_cache + (int64_t)id * 128 * tok_stride + h0 * 128;
        u32x4 kv[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int piece = i * 256 + threadIdx.x;
            const int t = piece >> 4, o = (piece & 15) * 16;
            kv[i] = *reinterpret_cast<const u32x4*>(kb + t * tok_stride + o);
            kv[8 + i] = *reinterpret_cast<const u32x4*>(vb + t * tok_stride + o);
        }
        const float ks = k_scale[((int64_t)id * 128 + (threadIdx.x >> 1)) * nkv + h0 + (threadIdx.x & 1)];
#pragma unroll
        for (int i = 0; i < 16; ++i) x ^= kv[i][0] ^ kv[i][1] ^ kv[i][2] ^ kv[i][3];
        x ^= __float_as_uint(ks);
    }
    const uint32_t r = fold_wg(x, red);
    if (threadIdx.x == 0) sink[blockIdx.x] = r;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// One 16x16x32 product per workgroup (one wave) on E4M3 codes: a [16 rows][32 k]
// and b [16 columns][32 k] bytes; c [16][16] fp32 from the FP8 MFMA
// (v_mfma_f32_16x16x32_fp8_fp8) and c_ref [16][16] from the bf16 MFMA on the
// codes decoded exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8 with scale 1).
// Lane l holds k = 8 (l / 16) .. + 8 of row / column l % 16; the result gives
// lane l the elements [4 (l / 16) + i][l % 16].
__global__ __launch_bounds__(64) void probe_fp8_mfma_kernel(const uint8_t* a, const uint8_t* b, float* c,
                                                            float* c_ref) {
    const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;
    const uint8_t* ap = a + (int64_t)blockIdx.x * 512 + n * 32 + 8 * g;
    const uint8_t* bp = b + (int64_t)blockIdx.x * 512 + n * 32 + 8 * g;
    const uint2 av = *reinterpret_cast<const uint2*>(ap);
    const uint2 bv = *reinterpret_cast<const uint2*>(bp);
    const long a64 = (long)(((uint64_t)av.y << 32) | av.x), b64 = (long)(((uint64_t)bv.y << 32) | bv.x);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4 r = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a64, b64, zero, 0, 0, 0);
    auto dec = [](uint32_t w0, uint32_t w1) {
        const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
        const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
        const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
        const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
        bf16x8 v = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        return v;
    };
    const f32x4 rr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dec(av.x, av.y), dec(bv.x, bv.y), zero, 0, 0, 0);
    float* cp = c + (int64_t)blockIdx.x * 256;
    float* crp = c_ref + (int64_t)blockIdx.x * 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        cp[(4 * g + i) * 16 + n] = r[i];
        crp[(4 * g + i) * 16 + n] = rr[i];
    }
}

// Issue rate of one VALU instruction: every wave runs `iters` rounds of eight
// independent instances (eight dependency chains), so with several waves per SIMD
// the SIMD's issue rate, not latency, sets the time.  OP: 0 v_mul_f32,
// 1 v_cvt_pk_f32_fp8, 2 v_cvt_pk_bf16_f32, 3 v_cvt_scalef32_pk_bf16_fp8,
// 4 v_perm_b32, 5 v_fma_f32.  sink: one word per thread.
template <int OP>
__global__ void probe_valu_rate_kernel(int iters, float* sink) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    float f[8];
    uint32_t u[8];
    for (int i = 0; i < 8; ++i) {
        f[i] = 1.0f + 0.001f * (float)(threadIdx.x + i);
        u[i] = 0x38403840u + 0x01010101u * (uint32_t)i + threadIdx.x;
    }
    const float sc = 1.0009765625f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (OP == 0) {
                asm volatile("v_mul_f32 %0, %0, %1" : "+v"(f[i]) : "v"(sc));
            } else if (OP == 1) {
                f32x2 r;
                asm volatile("v_cvt_pk_f32_fp8 %0, %1" : "=v"(r) : "v"(u[i]));
                u[i] ^= __builtin_bit_cast(uint32_t, r.x) >> 16;
            } else if (OP == 2) {
                uint32_t r;
                asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(f[i]), "v"(sc));
                f[i] = __builtin_bit_cast(float, (r & 0x007fffffu) | 0x3f800000u);
            } else if (OP == 3) {
                uint32_t r;
                asm volatile("v_cvt_scalef32_pk_bf16_fp8 %0, %1, %2" : "=v"(r) : "v"(u[i]), "v"(sc));
                u[i] ^= r >> 16;
            } else if (OP == 4) {
                asm volatile("v_perm_b32 %0, %0, %1, %2" : "+v"(u[i]) : "v"(u[(i + 1) & 7]), "v"(0x05010400u));
            } else {
                asm volatile("v_fma_f32 %0, %0, %1, %1" : "+v"(f[i]) : "v"(sc));
            }
        }
    }
    float acc = 0.f;
    for (int i = 0; i < 8; ++i) acc += f[i] + (float)(u[i] & 0xffu);
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// LDS read-rate probe: each lane reads WIDTH bytes (ds_read_b128 or ds_read_b64) at byte
// address base(lane) + 4096 u + 256 (it % 16) of a 64 KB LDS buffer, u = 0..7 per iteration
// (offsets that are multiples of 256 bytes keep every lane in the same bank).  base(lane),
// lane = 16 g + r: pattern 0: WIDTH lane (contiguous); 1: r stride + WIDTH g (sixteen rows,
// four pieces each: an MFMA operand read from a row-major tile); 2: (lane / 4) stride +
// WIDTH (lane % 4); 3: lane stride.  The host keeps base(lane) <= 32768 - WIDTH.
template <int WIDTH>
__global__ __launch_bounds__(512) void probe_lds_kernel(int pattern, int stride, int iters, uint32_t* sink) {
    __shared__ __attribute__((aligned(16))) uint32_t buf[16384];
    for (int i = threadIdx.x; i < 16384; i += blockDim.x) buf[i] = (uint32_t)i * 2654435761u;
    __syncthreads();
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    int base;
    if (pattern == 0) base = WIDTH * lane;
    else if (pattern == 1) base = r * stride + WIDTH * g;
    else if (pattern == 2) base = (lane >> 2) * stride + WIDTH * (lane & 3);
    else base = lane * stride;
    const uint8_t* p = reinterpret_cast<const uint8_t*>(buf) + base;
    uint32_t acc = 0;
    for (int it = 0; it < iters; ++it) {
        const uint8_t* q = p + 256 * (it & 15);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (WIDTH == 16) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(q + 4096 * u);
                acc ^= v[0] ^ v[3];
            } else {
                typedef int i32x2 __attribute__((ext_vector_type(2)));
                const i32x2 v = *reinterpret_cast<const i32x2*>(q + 4096 * u);
                acc ^= (uint32_t)(v[0] ^ v[1]);
            }
        }
    }
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// LDS read-pattern probe (see probe_lds_kernel): `grid` workgroups of 512 threads, width 8
// or 16 bytes per lane.  sink: grid * 512 words.  Returns 0 or a hipError_t (invalid value
// when a lane's address would leave the buffer).
int pa_probe_lds_pattern(int pattern, int stride, int width, int grid, int iters, uint32_t* sink, void* stream) {
    if (grid <= 0 || iters <= 0 || pattern < 0 || pattern > 3 || stride < 0 || (width != 8 && width != 16))
        return (int)hipErrorInvalidValue;
    const int64_t top = pattern == 0 ? (int64_t)width * 63
                      : pattern == 1 ? (int64_t)15 * stride + width * 3
                      : pattern == 2 ? (int64_t)15 * stride + width * 3
                      : (int64_t)63 * stride;
    if (top > 32768 - width || (stride % 8) != 0) return (int)hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (width == 16)
        hipLaunchKernelGGL(probe_lds_kernel<16>, dim3(grid), dim3(512), 0, st, pattern, stride, iters, sink);
    else
        hipLaunchKernelGGL(probe_lds_kernel<8>, dim3(grid), dim3(512), 0, st, pattern, stride, iters, sink);
    return (int)hipGetLastError();
}

// VALU issue-rate probe: `grid` workgroups of `threads` threads (a multiple of 64, at
// most 1024), each wave running iters x 8 instructions of kind `op` (see
// probe_valu_rate_kernel).  sink: grid * threads floats.  Returns 0 or a hipError_t.
int pa_probe_valu_rate(int op, int grid, int threads, int iters, float* sink, void* stream) {
    if (grid <= 0 || threads <= 0 || threads > 1024 || threads % 64 || iters <= 0 || op < 0 || op > 5)
        return (int)hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (op) {
        case 0: hipLaunchKernelGGL(probe_valu_rate_kernel<0>, dim3(grid), dim3(threads), 0, st, iters, sink); break;
        case 1: hipLaunchKernelGGL(probe_valu_rate_kernel<1>, dim3(grid), dim3(threads), 0, st, iters, sink); break;
        case 2: hipLaunchKernelGGL(probe_valu_rate_kernel<2>, dim3(grid), dim3(threads), 0, st, iters, sink); break;
        case 3: hipLaunchKernelGGL(probe_valu_rate_kernel<3>, dim3(grid), dim3(threads), 0, st, iters, sink); break;
        case 4: hipLaunchKernelGGL(probe_valu_rate_kernel<4>, dim3(grid), dim3(threads), 0, st, iters, sink); break;
        default: hipLaunchKernelGGL(probe_valu_rate_kernel<5>, dim3(grid), dim3(threads), 0, st, iters, sink); break;
    }
    return (int)hipGetLastError();
}

// FP8 MFMA probe: `count` independent 16x16x32 products (a, b: count * 512 code
// bytes; c, c_ref: count * 256 floats).  Returns 0 or a hipError_t.
int pa_probe_fp8_mfma(const uint8_t* a, const uint8_t* b, float* c, float* c_ref, int count, void* stream) {
    if (count <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_fp8_mfma_kernel, dim3(count), dim3(64), 0, static_cast<hipStream_t>(stream), a, b, c,
                       c_ref);
    return (int)hipGetLastError();
}

// Paged-pattern read probe.  persistent_grid == 0: one workgroup per item of
// heads_per_item (2, 4 or 8) KV heads (sink: B * (nkv / heads_per_item) *
// max_blocks words); else (heads_per_item 2) that many workgroups walk the items
// (sink: persistent_grid words).  nkv a multiple of heads_per_item.  Returns 0 or
// a hipError_t.
int pa_probe_paged_read(const uint8_t* k_cache, const float* k_scale, const uint8_t* v_cache, const int32_t* table,
                        const int32_t* seqs, int B, int nkv, int max_blocks, int num_blocks, int persistent_grid,
                        int heads_per_item, uint32_t* sink, void* stream) {
    const int nh = heads_per_item;
    if (B <= 0 || nkv <= 0 || max_blocks <= 0 || num_blocks <= 0 || persistent_grid < 0 ||
        (nh != 2 && nh != 4 && nh != 8) || nkv % nh || (persistent_grid > 0 && nh != 2))
        return (int)hipErrorInvalidValue;
    const int64_t items = (int64_t)B * (nkv / nh) * max_blocks;
    if (items > 0x7fffffff) return (int)hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (persistent_grid == 0 && nh == 2)
        hipLaunchKernelGGL(probe_paged_kernel<2>, dim3((unsigned)items), dim3(256), 0, st, k_cache, k_scale, v_cache,
                           table, seqs, nkv, max_blocks, num_blocks, sink);
    else if (persistent_grid == 0 && nh == 4)
        hipLaunchKernelGGL(probe_paged_kernel<4>, dim3((unsigned)items), dim3(256), 0, st, k_cache, k_scale, v_cache,
                           table, seqs, nkv, max_blocks, num_blocks, sink);
    else if (persistent_grid == 0)
        hipLaunchKernelGGL(probe_paged_kernel<8>, dim3((unsigned)items), dim3(256), 0, st, k_cache, k_scale, v_cache,
                           table, seqs, nkv, max_blocks, num_blocks, sink);
    else
        hipLaunchKernelGGL(probe_paged_persistent_kernel, dim3(persistent_grid), dim3(256), 0,
                           static_cast<hipStream_t>(stream), k_cache, k_scale, v_cache, table, seqs, nkv, max_blocks,
                           num_blocks, (int)items, sink);
    return (int)hipGetLastError();
}

// Contiguous read probe of n16 16-byte words with `grid` workgroups and `unroll`
// (4 or 8) loads in flight per thread; sink: grid words.
int pa_probe_contiguous_read(const void* p, int64_t n16, int grid, int unroll, uint32_t* sink, void* stream) {
    if (n16 <= 0 || grid <= 0 || (unroll != 4 && unroll != 8)) return (int)hipErrorInvalidValue;
    if (unroll == 4)
        hipLaunchKernelGGL(probe_contiguous_kernel<4>, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                           static_cast<const u32x4*>(p), n16, sink);
    else
        hipLaunchKernelGGL(probe_contiguous_kernel<8>, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                           static_cast<const u32x4*>(p), n16, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
