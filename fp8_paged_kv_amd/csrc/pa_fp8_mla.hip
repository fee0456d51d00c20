// MLA-style sparse attention decode with an FP8 latent cache (MI355X / gfx950).
//
// Web page "PyPTO-Gym 算子实战DeepSeek V32 MLA 的 Sparse Attention FP8 反量化算子":
// a cache row is 672 bytes -- 512 E4M3 "nope" values, 64 BF16 "rope" values
// (bytes 512..639) and four FP32 scales, one per 128-value group (bytes
// 640..655) -- section 核心参数与 KV Cache 布局.  Per query token, the first
// n = clamp(seq - s1 + 1 + s, 0, topk) top-k indices name logical tokens; each
// is mapped through the block table to a row (section 关键实现细节), dequantised
// to BF16 (value x group scale in FP32, then BF16), K = [nope | rope] and
// V = nope (section 计算流程).  Per tile of s2_tile indices: S = [qn | qr] . K
// x softmax_scale, m = tile max, P = exp(S - m) in BF16 feeds P.V while the
// unquantised P feeds the running sum; tiles are merged online and the result
// divided by the sum (section 在线反量化与 Online Softmax).
//
// Work: one workgroup per (query token, tile, block of 32 query heads); eight
// waves (four for 128-index tiles), two per SIMD.  Q of the 32 heads sits in
// LDS, already in MFMA B-operand order.  Wave w computes the scores of its
// T/8 rows of the tile for the 32
// heads, 16 rows at a time, gathering and dequantising K straight into MFMA
// operands (16x16x32 bf16, products exact, FP32 accumulation); the K rows of
// the next groups are requested before the current one is multiplied.  The
// waves exchange row maxima and sums through LDS and publish BF16 P in LDS;
// then wave w computes P.V for its 64 output channels over all
// rows of the tile, dequantising V rows on the fly (an 8x8 byte transpose
// turns row-major codes into MFMA operands), again with the next blocks'
// rows in flight.  Each (token, head, tile) leaves an (O, m, l) partial;
// mla_merge_kernel combines the tiles of each (token, head).
//
// The rows are addressed as three planes (nope codes, rope values, group
// scales), each with its own base and row stride: the packed 672-byte row is
// the three planes at offsets 0 / 512 / 640 with stride 672, and the page's
// kv_split sister operator keeps them as three tensors (section 相关算子对比).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_fp8_common.h"
#include "pa_fp8_device.h"

// Phase timing, built only into the phase-stamp variant of the library (PA_FP8_PHASES;
// the results are those of the plain build): eight 64-bit words per workgroup, times
// from s_memrealtime (100 MHz) -- 0 entry, 1 rows and queries staged, 2 score pass
// done, 3 tile maxima exchanged, 4 P staged, 5 P.V pass done, 6 exit.
#ifdef PA_FP8_PHASES
static __device__ unsigned long long g_mla_phases[4096 * 8];
extern "C" unsigned long long* pa_fp8_phases_mla() {
    void* p = nullptr;
    return hipGetSymbolAddress(&p, HIP_SYMBOL(g_mla_phases)) == hipSuccess ? (unsigned long long*)p : nullptr;
}
#define PH_STAMP(k) do { if (threadIdx.x == 0 && blockIdx.x < 4096) g_mla_phases[blockIdx.x * 8 + (k)] = __builtin_amdgcn_s_memrealtime(); } while (0)
#else
#define PH_STAMP(k) do { } while (0)
#endif

namespace pa {

constexpr int kMlaNope = 512, kMlaRope = 64, kMlaHeads = 32;

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Eight E4M3 codes (two dwords, byte i = value i), each times its own FP32
// scale, rounded to BF16 (the dequantised key of the page: FP32 product, BF16).
__device__ __forceinline__ bf16x8 dequant8(uint32_t w0, uint32_t w1, const float* sc) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
    const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
    const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
    bf16x8 r;
    r[0] = (__bf16)(a[0] * sc[0]);
    r[1] = (__bf16)(a[1] * sc[1]);
    r[2] = (__bf16)(b[0] * sc[2]);
    r[3] = (__bf16)(b[1] * sc[3]);
    r[4] = (__bf16)(c[0] * sc[4]);
    r[5] = (__bf16)(c[1] * sc[5]);
    r[6] = (__bf16)(d[0] * sc[6]);
    r[7] = (__bf16)(d[1] * sc[7]);
    return r;
}

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Direct global -> LDS load of 16 bytes per lane: lane i's bytes land at dst + 16 i.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_to_lds(const void* src, lds_ptr dst) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "s"(m) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) (gfx9 encoding, lgkmcnt and expcnt left at their maxima): this
// wave's vector memory operations complete in issue order.  The scheduling barriers
// keep the compiler from moving the work of the previous block below the wait.
template <int N>
__device__ __forceinline__ void mla_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    __builtin_amdgcn_sched_barrier(0);
}

// gfx950 transposing LDS read of 8-bit data.  In each group of 16 lanes, lanes
// 2j + h (j = 0..7, h = 0..1) name 8-byte chunks; lane 8h + c receives byte c of
// each of the 8 chunks named by lanes 2j + h, byte j from lane 2j + h.
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}

// Workgroup barrier that is also a compiler memory barrier, without the release
// fence of __syncthreads (which would wait for every load in flight).
__device__ __forceinline__ void barrier_nofence_mla() { asm volatile("s_barrier" ::: "memory"); }

template <int T, int NWV>
__global__ __launch_bounds__(NWV * 64) void mla_decode_kernel(MlaParams a) {
    constexpr int RW = T / NWV;           // rows of the tile whose scores a wave computes
    constexpr int NCH = RW / 32;          // 32-row chunks per wave
    constexpr int NB = T / 32;            // 32-row blocks of the tile
    constexpr int CPW = kMlaNope / NWV;   // output channels per wave in P.V
    constexpr int CL = CPW / 16;          // of them per lane (one MFMA each)
    static_assert(NCH >= 1 && (CL == 8 || CL == 4), "tile of at least 32 rows per wave");

    __shared__ int s_row[T];                                   // cache row of each tile position, -1 = past n
    // byte offsets of that row (row 0 for -1) in the three planes, formed once per position:
    // the gathers would otherwise redo a 64-bit multiply for every row they touch
    __shared__ int64_t s_noff[T], s_roff[T], s_soff[T];
    __shared__ __attribute__((aligned(16))) uint8_t s_p[NB][2][64 * 16];   // BF16 P, MFMA A-operand layout
    __shared__ float s_max[NWV][kMlaHeads], s_sum[NWV][kMlaHeads];
    __shared__ __attribute__((aligned(16))) uint8_t s_qop[2][18][64 * 16];  // Q as MFMA B operands, per lane
    // ring of 32-row V blocks (nope codes, 512 bytes a row), filled by DMA; 16-byte piece p of
    // row r sits in slot p ^ (r & 15) so that the transposing reads of one 16-channel column
    // spread over the banks
    constexpr int NBUF = 3;
    static_assert(NBUF >= 2 && NBUF <= 4, "ring depth");
    constexpr int DPW = 16 / NWV;         // DMA instructions (two rows each) per wave per block
    __shared__ __attribute__((aligned(16))) uint8_t s_v[NBUF][32 * 512];
    __shared__ __attribute__((aligned(16))) float s_sc[4][T];   // group scales by row, 0 past n

    PH_STAMP(0);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int nhb = a.nq / kMlaHeads;
    const int nbt = (int)gridDim.x / nhb;                      // (token, tile) pairs
    int hb, rest;
    if (nbt % 8 == 0) {
        // workgroups are dealt round-robin to the 8 XCDs: keep the head blocks of one
        // (token, tile) on one XCD so its L2 serves the rows they all gather
        const int x = (int)blockIdx.x % 8, k = (int)blockIdx.x / 8;
        hb = k % nhb;
        rest = x + 8 * (k / nhb);
    } else {
        hb = (int)blockIdx.x % nhb;
        rest = (int)blockIdx.x / nhb;
    }
    const int t = rest % a.ntiles_max, bs = rest / a.ntiles_max;
    const int b = bs / a.s1, s = bs - b * a.s1;
    const int kvh = hb * kMlaHeads / (a.nq / a.nkv);         // the KV head (top-k slice) of these heads

    int seq = a.seqs[b];
    seq = seq < 0 ? 0 : (seq > a.capacity ? a.capacity : seq);
    int n = seq - a.s1 + 1 + s;
    n = n < 0 ? 0 : (n > a.topk ? a.topk : n);
    if (t * T >= n) return;                                    // no such tile for this token

    // ---- cache rows of the tile's positions -----------------------------------------------
    for (int i = threadIdx.x; i < T; i += NWV * 64) {
        const int j = t * T + i;
        int row = -1;
        if (j < n) {
            int pos = a.topk_idx[((int64_t)bs * a.nkv + kvh) * a.topk + j];
            pos = pos < 0 ? 0 : (pos >= seq ? seq - 1 : pos);
            int id = a.block_table[(int64_t)b * a.max_blocks + pos / kBlock];
            id = (id < 0 || id >= a.num_blocks) ? 0 : id;
            row = id * kBlock + pos % kBlock;
        }
        s_row[i] = row;
        const int64_t r = row < 0 ? 0 : row;
        s_noff[i] = r * a.nope_stride;
        s_roff[i] = r * a.rope_stride;
        s_soff[i] = r * a.scale_stride;
        const f32x4 g = *reinterpret_cast<const f32x4*>(a.scales + r * a.scale_stride);
#pragma unroll
        for (int k = 0; k < 4; ++k) s_sc[k][i] = row < 0 ? 0.f : g[k];
    }

    // ---- query operands: heads h0 + 16 hh + lr; k-slot order shared with K ----------------
    // MFMA ks (0..15) takes nope channels 64 (ks / 2) + 16 g + 8 (ks % 2) + [0, 8);
    // ks 16, 17 take rope channels 16 g + 8 (ks - 16) + [0, 8).
    const int h0 = hb * kMlaHeads;
    for (int pq = w; pq < 36; pq += NWV) {                     // (head half, k-slot) pairs over the waves
        const int hh = pq / 18, ks = pq - 18 * (pq / 18);
        const int64_t qrow = (int64_t)bs * a.nq + h0 + 16 * hh + lr;
        const uint16_t* src = ks < 16 ? a.q_nope + qrow * kMlaNope + 64 * (ks >> 1) + 16 * lg + 8 * (ks & 1)
                                      : a.q_rope + qrow * kMlaRope + 16 * lg + 8 * (ks - 16);
        *reinterpret_cast<i32x4*>(&s_qop[hh][ks][16 * lane]) = *reinterpret_cast<const i32x4*>(src);
    }
    __syncthreads();
    PH_STAMP(1);
    auto qop = [&](int hh, int ks) { return *reinterpret_cast<const bf16x8*>(&s_qop[hh][ks][16 * lane]); };

    // V block bi (rows 32 bi .. 32 bi + 31 of the tile) into ring slot bi % NBUF: this wave's
    // DMA instructions cover rows 2 i and 2 i + 1 for i in [DPW w, DPW w + DPW)
    auto issue_vblock = [&](int bi) {
#pragma unroll
        for (int d = 0; d < DPW; ++d) {
            const int i = DPW * w + d;
            const int r = 2 * i + (lane >> 5);
            const int piece = (lane & 31) ^ (r & 15);
            dma16_to_lds(a.nope + s_noff[32 * bi + r] + 16 * piece, (lds_ptr)&s_v[bi % NBUF][1024 * i]);
        }
    };
    constexpr int NBV = T / 32;
#pragma unroll
    for (int bi = 0; bi < NBUF - 1; ++bi)
        if (bi < NBV) issue_vblock(bi);

    // ---- scores of this wave's rows: S^T (rows x heads), log2 units ------------------------
    const float coef = a.softmax_scale * kLog2e;
    float sv[2][NCH][8];
    float rmax[2] = {-INFINITY, -INFINITY};
    // K rows of 16-row group gq + 3 are requested while group gq is multiplied
    constexpr int NGQ = 2 * NCH;                          // 16-row groups of this wave
    struct KRows { f32x4 gs; i32x4 x[8]; i32x4 r0, r1; };
    KRows kq[3];
    auto issue_k = [&](int gq, KRows& kr) {
        const int idx = w * RW + 16 * gq + lr;            // this lane's K row (A operand row lr)
        const uint8_t* rp = a.nope + s_noff[idx];
        const uint8_t* rrp = a.rope + s_roff[idx];
        kr.gs = *reinterpret_cast<const f32x4*>(a.scales + s_soff[idx]);
#pragma unroll
        for (int pr = 0; pr < 8; ++pr) kr.x[pr] = *reinterpret_cast<const i32x4*>(rp + 64 * pr + 16 * lg);
        kr.r0 = *reinterpret_cast<const i32x4*>(rrp + 32 * lg);
        kr.r1 = *reinterpret_cast<const i32x4*>(rrp + 32 * lg + 16);
    };
#pragma unroll
    for (int i = 0; i < 3; ++i)
        if (i < NGQ) issue_k(i, kq[i]);
#pragma unroll
    for (int gq = 0; gq < NGQ; ++gq) {
        const int c = gq >> 1, k = gq & 1;
        KRows& kr = kq[gq % 3];
        f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int pr = 0; pr < 8; ++pr) {
            const float g = kr.gs[pr >> 1];
            const float sc[8] = {g, g, g, g, g, g, g, g};
            const bf16x8 k0 = dequant8((uint32_t)kr.x[pr][0], (uint32_t)kr.x[pr][1], sc);
            const bf16x8 k1 = dequant8((uint32_t)kr.x[pr][2], (uint32_t)kr.x[pr][3], sc);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                acc[hh] = mfma_bf16(k0, qop(hh, 2 * pr), acc[hh]);
                acc[hh] = mfma_bf16(k1, qop(hh, 2 * pr + 1), acc[hh]);
            }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            acc[hh] = mfma_bf16(__builtin_bit_cast(bf16x8, kr.r0), qop(hh, 16), acc[hh]);
            acc[hh] = mfma_bf16(__builtin_bit_cast(bf16x8, kr.r1), qop(hh, 17), acc[hh]);
        }
        if (gq + 3 < NGQ) issue_k(gq + 3, kr);
        // lane (head lr, group lg) holds rows 16 k + 4 lg + i of this 32-row chunk
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = s_row[w * RW + 32 * c + 16 * k + 4 * lg + i] >= 0;
                const float x = ok ? acc[hh][i] * coef : -INFINITY;
                sv[hh][c][4 * k + i] = x;
                rmax[hh] = fmaxf(rmax[hh], x);
            }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const float m = wave_max_over_groups(rmax[hh]);
        if (lg == 0) s_max[w][16 * hh + lr] = m;
    }
    PH_STAMP(2);
    __syncthreads();
    PH_STAMP(3);

    // ---- tile max, P = exp2(S - m) in BF16 to LDS, unquantised sums -------------------------
    float mt[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int hc = 16 * hh + lr;
        mt[hh] = s_max[0][hc];
#pragma unroll
        for (int i = 1; i < NWV; ++i) mt[hh] = fmaxf(mt[hh], s_max[i][hc]);
        float l = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            bf16x8 pb;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float pv = __builtin_amdgcn_exp2f(sv[hh][c][j] - mt[hh]);
                l += pv;
                pb[j] = (__bf16)pv;
            }
            *reinterpret_cast<bf16x8*>(&s_p[w * NCH + c][hh][16 * lane]) = pb;
        }
        l = wave_sum_over_groups(l);
        if (lg == 0) s_sum[w][hc] = l;
    }
    __syncthreads();

    PH_STAMP(4);
    // ---- P.V for channels [CPW w, CPW w + CPW): O[head][channel] -------------------------
    // MFMA c takes channels CPW w + 16 c + [0, 16); lane (n, g) holds channel n of rows
    // chunk_token(g, j), j = 0..7, the rows of the P operand's k-slots.
    f32x4 O[2][CL];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int c = 0; c < CL; ++c) O[hh][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int grp = CPW * w / 128;                            // the channels' scale group
    // transposing reads: lane 2 j + h of each 16-lane group names row chunk_token(g, j),
    // bytes 8 h .. 8 h + 7 of the 16-channel column
    const int tr_r = chunk_token(lg, (lane & 15) >> 1);
    int tr_off[CL];
#pragma unroll
    for (int c = 0; c < CL; ++c) tr_off[c] = tr_r * 512 + 16 * ((CPW * w / 16 + c) ^ (tr_r & 15)) + 8 * (lane & 1);
    const int nvalid = n - t * T;                             // valid rows of this tile (> 0)
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
        // this wave's DMA of block bi has landed once only the younger blocks' remain
        {
            const int younger = (NB - 1 - bi < NBUF - 2) ? NB - 1 - bi : NBUF - 2;
            if (younger >= 2) mla_wait_vm<2 * DPW>();
            else if (younger == 1) mla_wait_vm<DPW>();
            else mla_wait_vm<0>();
        }
        if (32 * bi + 32 > nvalid) {
            // rows past n read row 0, whose codes may be NaN: zero the rows this wave loaded
#pragma unroll
            for (int d = 0; d < DPW; ++d)
#pragma unroll
                for (int hr = 0; hr < 2; ++hr) {
                    const int r = 2 * (DPW * w + d) + hr;
                    if (32 * bi + r >= nvalid)
                        *reinterpret_cast<uint2*>(&s_v[bi % NBUF][r * 512 + 8 * lane]) = uint2{0u, 0u};
                }
        }
        barrier_nofence_mla();
        if (bi + NBUF - 1 < NB) issue_vblock(bi + NBUF - 1);   // into the slot block bi - 1 used
        bf16x8 pop[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) pop[hh] = *reinterpret_cast<const bf16x8*>(&s_p[bi][hh][16 * lane]);
        const f32x4 sa = *reinterpret_cast<const f32x4*>(&s_sc[grp][32 * bi + 4 * lg]);
        const f32x4 sb = *reinterpret_cast<const f32x4*>(&s_sc[grp][32 * bi + 16 + 4 * lg]);
        const float scj[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
        const uint8_t* vb = &s_v[bi % NBUF][0];
#pragma unroll
        for (int c = 0; c < CL; ++c) {
            const i32x2 x = lds_read_tr8(vb + tr_off[c]);
            const bf16x8 vop = dequant8((uint32_t)x[0], (uint32_t)x[1], scj);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) O[hh][c] = mfma_bf16(pop[hh], vop, O[hh][c]);
        }
    }

    PH_STAMP(5);
    // ---- partial of this tile: O (relative to the tile max), m, l --------------------------
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int head = h0 + 16 * hh + 4 * lg + i;
            const int64_t slot = ((int64_t)bs * a.nq + head) * a.ntiles_max + t;
            float* po = a.part_o + slot * kMlaNope + CPW * w + lr;
#pragma unroll
            for (int c = 0; c < CL; ++c) po[16 * c] = O[hh][c][i];
        }
        if (w == 0 && lg == 0) {
            const int hc = 16 * hh + lr;
            const int64_t slot = ((int64_t)bs * a.nq + h0 + hc) * a.ntiles_max + t;
            float l = 0.f;
#pragma unroll
            for (int i = 0; i < NWV; ++i) l += s_sum[i][hc];
            a.part_ml[slot * 2] = mt[hh];
            a.part_ml[slot * 2 + 1] = l;
        }
    }
    PH_STAMP(6);
}

// Online merge of the tile partials of every (query token, head), in tile order;
// one wave per (token, head), eight channels per lane.  n == 0 gives zeros.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaParams a, int T) {
    const int lane = threadIdx.x & 63;
    const int64_t qh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);      // (token, head)
    if (qh >= (int64_t)a.B * a.s1 * a.nq) return;
    const int bs = (int)(qh / a.nq);
    const int b = bs / a.s1, s = bs - b * a.s1;
    int seq = a.seqs[b];
    seq = seq < 0 ? 0 : (seq > a.capacity ? a.capacity : seq);
    int n = seq - a.s1 + 1 + s;
    n = n < 0 ? 0 : (n > a.topk ? a.topk : n);
    const int nt = (n + T - 1) / T;
    float M = -INFINITY, L = 0.f;
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < nt; ++t) {
        const int64_t slot = qh * a.ntiles_max + t;
        const float m = a.part_ml[slot * 2], l = a.part_ml[slot * 2 + 1];
        const float* po = a.part_o + slot * kMlaNope + 8 * lane;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(po);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(po + 4);
        const float mn = fmaxf(M, m);
        const float fa = __builtin_amdgcn_exp2f(M - mn), fb = __builtin_amdgcn_exp2f(m - mn);
        L = L * fa + l * fb;
        o0 = o0 * fa + x0 * fb;
        o1 = o1 * fa + x1 * fb;
        M = mn;
    }
    const float inv = nt > 0 ? 1.f / L : 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float y0 = (c < 2 ? o0[2 * c] : o1[2 * c - 4]) * inv;
        const float y1 = (c < 2 ? o0[2 * c + 1] : o1[2 * c - 3]) * inv;
        pk[c] = pack_bf16x2(y0, y1);
    }
    *reinterpret_cast<i32x4*>(a.out + qh * kMlaNope + 8 * lane) = i32x4{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
}

template <int T>
static hipError_t launch_mla_t(const MlaParams& p, hipStream_t st) {
    constexpr int NWV = T >= 256 ? 8 : 4;                     // waves: at least 32 tile rows each
    const int64_t grid = (int64_t)p.B * p.s1 * p.ntiles_max * (p.nq / kMlaHeads);
    if (grid > 0) hipLaunchKernelGGL((mla_decode_kernel<T, NWV>), dim3((unsigned)grid), dim3(NWV * 64), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)p.B * p.s1 * p.nq;
    hipLaunchKernelGGL(mla_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, p, T);
    return hipGetLastError();
}

// query heads of one KV head come in whole blocks of 32 (a workgroup reads one top-k slice)
bool mla_supported(int nq, int nkv, int s2_tile) {
    return nkv >= 1 && nq % nkv == 0 && (nq / nkv) % kMlaHeads == 0 &&
           (s2_tile == 128 || s2_tile == 256 || s2_tile == 512);
}

hipError_t launch_mla(const MlaParams& p, hipStream_t st) {
    switch (p.s2_tile) {
        case 128: return launch_mla_t<128>(p, st);
        case 256: return launch_mla_t<256>(p, st);
        default: return launch_mla_t<512>(p, st);
    }
}

}  // namespace pa
