// FP8 paged GQA attention for many query rows per KV head: chunked prefill and long
// multi-token decode (MI355X / gfx950).
//
// The operation is that of the decode (web page "PyPTO 实现 GLM-4.5 Paged Attention FP8
// 量化算子…", section 计算流程 steps 1-10), with the causal limit of the MLA page
// ("PyPTO-Gym 算子实战DeepSeek V32 MLA…", section 关键实现细节) when asked for: row s of the
// s1 query positions sees the first seq - s1 + 1 + s tokens.  The decode kernels take a KV
// head's rows at most 32 at a time, so with hundreds of rows every block of 32 re-reads and
// re-converts the whole sequence's K and V.  Here:
//
//  * A workgroup owns (batch, KV head, 128 query rows) and walks all tiles of the sequence
//    itself (no split, no merge).  Wave w owns rows 16 w .. 16 w + 15, one 16-row MFMA block.
//  * Each 128-token block of K (then of V) is staged once in LDS by direct global->LDS loads
//    and converted once to BF16 (the codes are exact in BF16) by all 512 threads; the eight
//    waves then read their MFMA operands from the BF16 copy.  V is stored transposed, each
//    channel's tokens in the k-slot order of the P operand, through gfx950's transposing byte
//    read (lane 8 h + c of each 16-lane group receives byte c of the 8-byte chunks named by
//    lanes 2 j + h, in j order).
//  * A tile's scores (16 rows x s2_tile tokens per wave) stay in registers until the tile's
//    row maxima are known; P is quantised per row and tile as in the decode, and kept in
//    registers as the A operand of P.V.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_fp8_common.h"
#include "pa_fp8_device.h"

namespace pa {

namespace {

typedef __attribute__((address_space(3))) void* lds_ptr_p;
typedef int i32x2p __attribute__((ext_vector_type(2)));

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Direct global -> LDS loads: lane i's 16 (4) bytes from src_i land at dst + 16 i (4 i).
__device__ __forceinline__ void pf_dma16(const void* src, lds_ptr_p dst) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "s"(m) : "memory", "m0");
}
__device__ __forceinline__ void pf_dma4(const void* src, lds_ptr_p dst) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" :: "v"(src), "s"(m) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N), gfx9 encoding; the scheduling barriers keep other work on its side.
template <int N>
__device__ __forceinline__ void pf_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    __builtin_amdgcn_sched_barrier(0);
}

// the same with a run-time count (at most 15 here)
__device__ __forceinline__ void pf_wait_vm_n(int n) {
    switch (n) {
        case 0: pf_wait_vm<0>(); break;
        case 1: pf_wait_vm<1>(); break;
        case 2: pf_wait_vm<2>(); break;
        case 3: pf_wait_vm<3>(); break;
        case 4: pf_wait_vm<4>(); break;
        case 5: pf_wait_vm<5>(); break;
        case 6: pf_wait_vm<6>(); break;
        case 7: pf_wait_vm<7>(); break;
        case 8: pf_wait_vm<8>(); break;
        case 9: pf_wait_vm<9>(); break;
        case 10: pf_wait_vm<10>(); break;
        case 11: pf_wait_vm<11>(); break;
        default: pf_wait_vm<0>(); break;
    }
}

__device__ __forceinline__ void pf_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ i32x2p pf_read_tr8(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2p*)(p));
}

constexpr int kRowsPerWg = 128;              // query rows of a KV head per workgroup
// Row r of the BF16 copy (a K token or a V channel, 256 bytes) starts at byte
// 288 r + 16 ((r / 16) % 2).  gfx950 serves a 16-byte LDS read or write 32 lanes at a time over
// 128 four-byte banks: with this layout the MFMA operand reads (16 rows x 2 pieces) and the
// conversions' writes (32 rows x 1 piece) each cover all 128 banks once.  (With rows 272 bytes
// apart the operand reads took two passes.)
constexpr int kBf16Stride = 288;
__device__ __forceinline__ int pf_row(int r) { return kBf16Stride * r + 16 * ((r >> 4) & 1); }
constexpr int kOrderMax = 256;               // batches ordered by length (longest first) up to this count

// Staged FP8 rows are 128 bytes (eight 16-byte pieces), so every token row starts in the same
// LDS bank; piece p of token t is stored in slot p ^ pf_swz(t).  With this swizzle the
// conversions' reads (a token's pieces across the lanes of a K read, eight tokens' same piece
// across the lanes of a transposing V read) fall in distinct banks.
__device__ __forceinline__ int pf_swz(int t) { return (t ^ (t >> 1) ^ (t >> 2)) & 7; }

}  // namespace

template <int NBLK>
__global__ __launch_bounds__(512) void prefill_kernel(DecodeParams a) {
    constexpr int T = NBLK * kBlock;          // s2_tile
    constexpr int NQ = T / 32;                // 32-token chunks of a tile
    constexpr int NST = 2;                    // staging ring of FP8 blocks: one in flight (3, 4, 5 were slower)
    __shared__ __attribute__((aligned(16))) uint8_t s_stage[NST][kBlock * kHeadDim];
    __shared__ __attribute__((aligned(16))) float s_ks[NST][kBlock];
    // BF16 copies, double-buffered: K [token][dim] or V [channel][slot]; and the K block's scales
    __shared__ __attribute__((aligned(16))) uint8_t s_bf[2][kBlock * kBf16Stride];
    __shared__ __attribute__((aligned(16))) float s_ksb[2][kBlock];
    __shared__ int s_order[kOrderMax], s_len[kOrderMax];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int rows = a.s1 * a.G;
    const int rtiles = (rows + kRowsPerWg - 1) / kRowsPerWg;
    // workgroup -> (batch rank, KV head, row tile)
    const int rt = (int)blockIdx.x % rtiles;
    const int bh = (int)blockIdx.x / rtiles;
    const int bo = bh / a.nkv, h = bh - bo * a.nkv;
    // batches longest first (workgroups are dispatched in index order, so the long ones start
    // first and the short ones fill in behind them); identity past kOrderMax batches
    int b = bo;
    if (a.B <= kOrderMax) {
        for (int i = threadIdx.x; i < a.B; i += 512) s_len[i] = a.seqs[i];
        __syncthreads();
        for (int i = threadIdx.x; i < a.B; i += 512) {
            const int si = s_len[i];
            int rank = 0;
            for (int j = 0; j < a.B; ++j) {
                const int sj = s_len[j];
                rank += (sj > si) || (sj == si && j < i);
            }
            s_order[rank] = i;
        }
        __syncthreads();
        b = __builtin_amdgcn_readfirstlane(s_order[bo]);
    }
    int seq = a.seqs[b];
    seq = seq < 0 ? 0 : (seq > a.capacity ? a.capacity : seq);

    // ---- step 1: this lane's query row (S layout: row lr of the wave's block) -> BF16 operands
    const int ra = kRowsPerWg * rt + 16 * w + lr;            // row among the head's s1 G
    const bool row_ok = ra < rows;
    const int s_of = row_ok ? ra / a.G : 0;
    const int lim = row_ok ? seq - (a.causal ? a.s1 - 1 - s_of : 0) : 0;   // tokens this row sees
    // tokens every row of this wave sees: its first row's (limits grow with the row), 0 if the
    // wave holds rows past the end
    const int wave_lim = (kRowsPerWg * rt + 16 * w + 15 < rows) ? __builtin_amdgcn_readfirstlane(lim) : 0;
    // tokens any row of the workgroup sees (rows grow with s, so the last valid row sees most)
    const int ra_last = min(kRowsPerWg * rt + kRowsPerWg, rows) - 1;
    const int wg_lim = seq - (a.causal ? a.s1 - 1 - ra_last / a.G : 0);

    const int nblocks = wg_lim <= 0 ? 0 : (wg_lim + kBlock - 1) / kBlock;   // blocks any row needs
    const int ntiles = (nblocks + NBLK - 1) / NBLK;
    const int32_t* table = a.block_table + (int64_t)b * a.max_blocks;
    // staged step k: tile t's K blocks, then its V blocks; the last tile may hold fewer blocks
    const int nsteps = 2 * nblocks;
    const int nfull = nblocks / NBLK, nb_last = nblocks - nfull * NBLK;
    auto step_of = [&](int k, int& blk, bool& is_v) {
        if (k < 2 * NBLK * nfull) {
            const int t = k / (2 * NBLK), r = k - t * 2 * NBLK;
            is_v = r >= NBLK;
            blk = t * NBLK + (is_v ? r - NBLK : r);
        } else {
            const int r = k - 2 * NBLK * nfull;
            is_v = r >= nb_last;
            blk = nfull * NBLK + (is_v ? r - nb_last : r);
        }
    };
    // loads of step k into ring slot k % NST: two 1 KB loads per wave (eight tokens each),
    // and for a K block its 128 scales on waves 0 and 1
    auto issue = [&](int k) {
        int blk;
        bool is_v;
        step_of(k, blk, is_v);
        // a scalar load: a vector one would share vmcnt with the ring's loads and, waited for
        // before the addresses it feeds, drain every block in flight
        int id = ((const __attribute__((address_space(4))) int32_t*)table)[blk];
        id = (id < 0 || id >= a.num_blocks) ? 0 : id;
        const uint8_t* base = (is_v ? a.v_cache : a.k_cache) + ((int64_t)id * kBlock * a.nkv + h) * kHeadDim;
        uint8_t* st = s_stage[k % NST];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const int i = 2 * w + d;                          // tokens 8 i .. 8 i + 7
            const int tok = 8 * i + (lane >> 3);              // slot lane % 8 of its row
            pf_dma16(base + (int64_t)tok * a.nkv * kHeadDim + 16 * ((lane & 7) ^ pf_swz(tok)), (lds_ptr_p)(st + 1024 * i));
        }
        if (!is_v && w < 2) {
            const int tok = 64 * w + lane;
            pf_dma4(a.k_scale + ((int64_t)id * kBlock + tok) * a.nkv + h, (lds_ptr_p)&s_ks[k % NST][64 * w]);
        }
    };
    // this wave's loads of step k
    auto loads_of = [&](int k) {
        int blk;
        bool is_v;
        step_of(k, blk, is_v);
        return (!is_v && w < 2) ? 3 : 2;
    };
    // wait for this wave's loads of step k, those of steps k + 1 .. last_issued being younger
    auto wait_loads = [&](int k, int last_issued) {
        int n = 0;
        for (int j = k + 1; j <= last_issued && j < nsteps; ++j) n += loads_of(j);
        pf_wait_vm_n(n);
    };
    // FP8 block of step k (staged, every wave's loads landed) -> BF16 copy k % 2
    auto convert = [&](int k) {
        int blk;
        bool is_v;
        step_of(k, blk, is_v);
        const uint8_t* st = s_stage[k % NST];
        uint8_t* bf = s_bf[k & 1];
        if (!is_v) {
            // K codes -> BF16 [token][dim]: thread i takes token i % 128, dims 32 (i / 128) .. + 32
            // (pieces 2 (i / 128) and 2 (i / 128) + 1)
            const int tok = threadIdx.x & 127, qd = threadIdx.x >> 7, sw = pf_swz(tok);
            const i32x4 c0 = *reinterpret_cast<const i32x4*>(st + tok * kHeadDim + 16 * ((2 * qd) ^ sw));
            const i32x4 c1 = *reinterpret_cast<const i32x4*>(st + tok * kHeadDim + 16 * ((2 * qd + 1) ^ sw));
            uint8_t* dst = bf + pf_row(tok) + 64 * qd;
            *reinterpret_cast<bf16x8*>(dst) = fp8x8_to_op((uint32_t)c0[0], (uint32_t)c0[1]);
            *reinterpret_cast<bf16x8*>(dst + 16) = fp8x8_to_op((uint32_t)c0[2], (uint32_t)c0[3]);
            *reinterpret_cast<bf16x8*>(dst + 32) = fp8x8_to_op((uint32_t)c1[0], (uint32_t)c1[1]);
            *reinterpret_cast<bf16x8*>(dst + 48) = fp8x8_to_op((uint32_t)c1[2], (uint32_t)c1[3]);
            if (threadIdx.x < kBlock) s_ksb[k & 1][threadIdx.x] = s_ks[k % NST][threadIdx.x];
        } else {
            // V codes -> BF16 [channel][slot]: a 16-lane group takes 32-token chunk cq, slot group
            // sg (tokens chunk_token(sg, j)) and 16-channel column cb; lane 2 j + hh names token
            // chunk_token(sg, j), bytes 16 cb + 8 hh .. + 8
            const int p0blk = blk * kBlock;
            const int grp = 4 * w + lg;                       // 0..31
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int combo = 32 * it + grp;              // 0..127: (cq, sg, cb)
                const int cq = combo >> 5, sg = (combo >> 3) & 3, cb = combo & 7;
                const int jj = (lane & 15) >> 1, hh = lane & 1;
                const int tok = 32 * cq + chunk_token(sg, jj);
                const i32x2p x = pf_read_tr8(st + tok * kHeadDim + 16 * (cb ^ pf_swz(tok)) + 8 * hh);
                uint32_t x0 = (uint32_t)x[0], x1 = (uint32_t)x[1];
                if (p0blk + 32 * cq + 32 > seq) {
                    // tokens past the sequence (their codes may be NaN) contribute exact zeros
                    uint32_t m0 = 0, m1 = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        m0 |= (p0blk + 32 * cq + chunk_token(sg, j) < seq ? 0xffu : 0u) << (8 * j);
                        m1 |= (p0blk + 32 * cq + chunk_token(sg, j + 4) < seq ? 0xffu : 0u) << (8 * j);
                    }
                    x0 &= m0;
                    x1 &= m1;
                }
                const int ch = 16 * cb + (lane & 15);
                *reinterpret_cast<bf16x8*>(bf + pf_row(ch) + 2 * (32 * cq + 8 * sg)) = fp8x8_to_op(x0, x1);
            }
        }
    };
    // Step k: its BF16 copy was made during step k - 1.  Wait for the loads of step k + 1; the
    // barrier then also ends every wave's use of the BF16 copy (k + 1) % 2 and of ring slot
    // k % NST; refill that slot with step k + NST, multiply step k, then convert step k + 1.
    // (Half the waves converting before they multiply, so that each SIMD overlaps one wave's
    // conversion with the other's MFMAs, was 8 % slower once the LDS accesses were
    // conflict-free.)
    int gs = 0;
    auto step_begin = [&]() {
        if (gs + 1 < nsteps) wait_loads(gs + 1, gs + NST - 1);
        pf_barrier();
        if (gs + NST < nsteps) issue(gs + NST);
    };
    auto step_end = [&]() {
        if (gs + 1 < nsteps) convert(gs + 1);
        ++gs;
    };

    // the first blocks' loads go out before the query rows are staged, so that the two
    // latencies overlap
    for (int k = 0; k < NST && k < nsteps; ++k) issue(k);       // one step per ring slot
    bf16x8 qop[4];
    float qcoef = 0.f;
    {
        uint32_t wds[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
        if (row_ok) {
            const int64_t qrow = ((int64_t)b * a.s1 + s_of) * a.nq + h * a.G + (ra - s_of * a.G);
            const float qs = a.q_scale[qrow];
            qcoef = qs * a.softmax_scale * kLog2e;
            const QRecip d = q_recip(qs);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                // dims 32 ks + 8 lg + [0, 8) for ks = 2 half, 2 half + 1
                const uint16_t* qp = a.q + qrow * kHeadDim + 64 * half + 8 * lg;
                const i32x4 v0 = *reinterpret_cast<const i32x4*>(qp);
                const i32x4 v1 = *reinterpret_cast<const i32x4*>(qp + 32);
                const uint32_t raw[8] = {(uint32_t)v0[0], (uint32_t)v0[1], (uint32_t)v0[2], (uint32_t)v0[3],
                                         (uint32_t)v1[0], (uint32_t)v1[1], (uint32_t)v1[2], (uint32_t)v1[3]};
                quantise_q16(raw, d, wds[half]);
            }
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qop[ks] = fp8x8_to_op(wds[ks >> 1][2 * (ks & 1)], wds[ks >> 1][2 * (ks & 1) + 1]);
    }
    if (nsteps > 0) {
        wait_loads(0, NST - 1);
        pf_barrier();
        convert(0);
    }

    float M_s = -INFINITY, L_s = 0.f;          // running max / sum of row lr (S layout; this lane's tokens)
    float M_o[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};   // of rows 4 lg + i (O layout)
    f32x4 O[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) O[c] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int t = 0; t < ntiles; ++t) {
        const int nb = min(NBLK, nblocks - t * NBLK);
        float sv[NQ][8];
        float rmax = -INFINITY;
        // ---------------- K pass: S = q8 . k8 * scales, masked ----------------------------------
#pragma unroll
        for (int r = 0; r < NBLK; ++r) {
            if (r < nb) {
                step_begin();
                const uint8_t* bf = s_bf[gs & 1];
                const float* ksr = s_ksb[gs & 1];
                const int p0blk = (t * NBLK + r) * kBlock;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {                  // 32-token chunks of the block
                    const int q = 4 * r + cc;
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const int tb = 32 * cc + 16 * k;          // 16-token block
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks) {
                            const bf16x8 kop = *reinterpret_cast<const bf16x8*>(bf + pf_row(tb + lr) +
                                                                               2 * (32 * ks + 8 * lg));
                            acc = mfma_bf16(kop, qop[ks], acc);
                        }
                        const f32x4 kk = *reinterpret_cast<const f32x4*>(&ksr[tb + 4 * lg]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) sv[q][4 * k + i] = acc[i] * kk[i] * qcoef;
                    }
                }
                if (p0blk + kBlock > wave_lim) {                   // some row of the wave stops in this block
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            sv[4 * r + cc][j] = (p0blk + 32 * cc + chunk_token(lg, j) < lim) ? sv[4 * r + cc][j] : -INFINITY;
                }
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                    for (int j = 0; j < 8; ++j) rmax = fmaxf(rmax, sv[4 * r + cc][j]);
                step_end();
            } else {
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                    for (int j = 0; j < 8; ++j) sv[4 * r + cc][j] = -INFINITY;
            }
        }
        // ---------------- tile maximum, P' = 448 exp2(S - m) as FP8 codes, its sum -------------
        const float m = wave_max_over_groups(rmax);            // row lr over the tile
        const float poff = (m == -INFINITY || M_s - m > kDropLog2) ? -INFINITY : kLog2_448 - m;
        float lsum = 0.f;
        uint32_t p8[NQ][2];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float pv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                pv[j] = __builtin_amdgcn_exp2f(sv[q][j] + poff);
                lsum += pv[j];
            }
            p8[q][0] = cvt4_fp8(pv[0], pv[1], pv[2], pv[3]);
            p8[q][1] = cvt4_fp8(pv[4], pv[5], pv[6], pv[7]);
        }
        float mt_o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mo = __shfl(m, 4 * lg + i, 64);
            mt_o[i] = mo;
            const float d = M_o[i] - mo;
            const float sc = (mo == -INFINITY || d > kDropLog2) ? 1.f : __builtin_amdgcn_exp2f(d);
#pragma unroll
            for (int c = 0; c < 8; ++c) O[c][i] *= sc;
        }
        // ---------------- V pass: O += P8 . V8 ---------------------------------------------------
#pragma unroll
        for (int r = 0; r < NBLK; ++r) {
            if (r < nb) {
                step_begin();
                const uint8_t* bf = s_bf[gs & 1];
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    const int q = 4 * r + cc;
                    const bf16x8 pop = fp8x8_to_op(p8[q][0], p8[q][1]);
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const bf16x8 vop = *reinterpret_cast<const bf16x8*>(bf + pf_row(16 * c + lr) +
                                                                           2 * (32 * cc + 8 * lg));
                        O[c] = mfma_bf16(pop, vop, O[c]);
                    }
                }
                step_end();
            }
        }
        // ---------------- finish the rescale, update the running state ---------------------------
        if (m != -INFINITY) {
            const float mn = fmaxf(M_s, m);
            L_s = L_s * __builtin_amdgcn_exp2f(M_s - mn) + lsum * __builtin_amdgcn_exp2f(m - mn);
            M_s = mn;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mo = fmaxf(M_o[i], mt_o[i]);
            const float d = M_o[i] - mt_o[i];
            const float sc = (mt_o[i] == -INFINITY || d > kDropLog2) ? 1.f : __builtin_amdgcn_exp2f(mt_o[i] - mo);
            M_o[i] = mo;
#pragma unroll
            for (int c = 0; c < 8; ++c) O[c][i] *= sc;
        }
    }

    // ---- step 10: out = O * v_scale / L' (L' = 448 L), bf16; rows 4 lg + i, channels 16 c + lr
    const float* vsp = a.v_scale + ((int64_t)b * a.nkv + h) * kHeadDim;
    float vs[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) vs[c] = vsp[16 * c + lr];
    // each lane's L_s sums its own tokens (4 of every 16); the row's sum is over the four groups
    const float Lw = wave_sum_over_groups(L_s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float Lr = __shfl(Lw, 4 * lg + i, 64);
        const int rr = kRowsPerWg * rt + 16 * w + 4 * lg + i;
        if (rr >= rows) continue;
        const int s = rr / a.G, gq = rr - s * a.G;
        const int64_t qrow = ((int64_t)b * a.s1 + s) * a.nq + h * a.G + gq;
        const float inv = Lr > 0.f ? 1.f / Lr : 0.f;          // no token at all (causal): zeros
#pragma unroll
        for (int c = 0; c < 8; ++c) a.out[qrow * kHeadDim + 16 * c + lr] = f32_to_bf16_rne(O[c][i] * vs[c] * inv);
    }
}

int prefill_row_tiles(int rows) { return (rows + kRowsPerWg - 1) / kRowsPerWg; }

bool prefill_supported(int s2_tile) { return s2_tile == 128 || s2_tile == 256 || s2_tile == 512; }

hipError_t launch_prefill(const DecodeParams& p, hipStream_t st) {
    const int64_t grid = (int64_t)p.B * p.nkv * prefill_row_tiles(p.s1 * p.G);
    if (grid <= 0) return hipSuccess;
    switch (p.s2_tile) {
        case 128: hipLaunchKernelGGL(prefill_kernel<1>, dim3((unsigned)grid), dim3(512), 0, st, p); break;
        case 256: hipLaunchKernelGGL(prefill_kernel<2>, dim3((unsigned)grid), dim3(512), 0, st, p); break;
        default: hipLaunchKernelGGL(prefill_kernel<4>, dim3((unsigned)grid), dim3(512), 0, st, p); break;
    }
    return hipGetLastError();
}

}  // namespace pa
