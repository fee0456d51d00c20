// FP8 paged GQA decode, whole-row path (MI355X / gfx950).
//
// Same operation as the per-head path (web page "PyPTO 实现 GLM-4.5 Paged
// Attention FP8 量化算子…", section 计算流程 steps 1-10), organised for the
// memory system:
//
//  * One workgroup holds one wave per KV head (nkv <= 8) and reads whole
//    token rows of the cache ([token][all KV heads][128] bytes, contiguous)
//    with gfx950's direct global->LDS loads.  Every wave then takes its own
//    head's bytes from LDS.  Reading whole rows keeps DRAM pages fully used;
//    one workgroup per head reading 128 of every 1024 bytes measured ~17 %
//    slower on this pattern.
//  * The LDS ring holds NST stages of one 32-token chunk (K or V of all
//    heads, plus k_scale); loads for the next NST-1 chunks are always in
//    flight and cost no registers.  LDS-DMA completion is not tracked by the
//    compiler, so every step waits with an explicit vmcnt and a raw barrier.
//  * Work is balanced "stream-K" style: the (batch, tile, head) atoms of the
//    whole call, in that order, are split into equal contiguous ranges, one
//    per workgroup (one workgroup per CU).  A range may cover parts of
//    several sequences and only some heads of its first and last tile.  A
//    (batch, head) handled by one workgroup is finished in place; otherwise
//    each workgroup writes an (O, M, L) partial and a second small kernel
//    merges them in range order.
//  * Each wave keeps the whole tile's scores S (s2_tile x 16 rows, fp32) in
//    registers, since the FP8 quantisation of P needs the tile's row max
//    before any P of the tile is used.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_fp8_common.h"
#include "pa_fp8_device.h"

namespace pa {

typedef __attribute__((address_space(3))) void* lds_ptr;

// Direct global->LDS loads (lane i writes dst + size * i), issued from inline
// asm so that the compiler does not see them as LDS stores.  Otherwise it
// conservatively waits for every load in flight (vmcnt(0)) before any LDS read
// of the ring, which would serialise the prefetch.  Their completion is
// ordered by hand with wait_vm<N>() and a barrier.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_b128(const void* src, lds_ptr dst) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"((uint32_t)(uintptr_t)dst) : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const void* src, lds_ptr dst) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :: "v"(src), "s"((uint32_t)(uintptr_t)dst) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt left free), gfx9 encoding.  vmcnt counts
// this wave's vector memory operations, which complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that is also a compiler memory barrier, without the
// release fence of __syncthreads (which would wait for every DMA in flight).
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// Load of a wave-uniform int32 through the constant address space, i.e. as a
// scalar load.  A vector load would share the in-order vmcnt counter with the
// ring's loads, and waiting for its result would drain the whole ring.
__device__ __forceinline__ int ld_uniform(const int32_t* p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// Swizzle of 16-byte slots inside a staged chunk: slot (token t, piece p) is
// stored at t * 8HG + (p ^ f(t)).  K reads (16 tokens, one piece) and V
// reads (tokens t and t+4, eight pieces) then hit distinct LDS banks.
template <int HG>
__device__ __forceinline__ int swz(int t) {
    if (HG == 1) return (t >> 1) & 7;
    return (t & 15) ^ ((t & 4) << 1);
}

// One unit = one tile of one virtual sequence (batch b, heads h0 .. h0+HG-1);
// the workgroup works on heads [hlo, hhi) of the group in it.
struct RowsUnit {
    int v, b, h0, t, hlo, hhi, seq;
};

constexpr int kQRowsMax = 128;            // s1 * nq rows of one sequence staged in LDS
constexpr int kPrefixMax = 1024;          // batch size limit of this path

template <int NRB, int NCH, int HG, int NST, bool DBG>
__global__ __launch_bounds__(HG * 64) void decode_rows_kernel(DecodeParams a) {
    constexpr int T = NCH * 32;           // s2_tile
    constexpr int R = NRB * 16;
    constexpr int CHUNK = HG * 4096;      // bytes of one staged chunk (32 tokens, HG heads)
    constexpr int STEPS = 2 * NCH;        // per unit: NCH chunks of K, then NCH of V
    constexpr int AHEAD = NST - 1;        // chunks in flight
    constexpr int PER_STEP = 5;           // loads per wave and step: 4 chunk + 1 k_scale
    constexpr int TOK16 = 16 * 8 * HG * 16;   // LDS bytes of 16 staged tokens
    static_assert(AHEAD >= 1 && AHEAD < STEPS, "ring depth");
    // Per virtual sequence: Q rows of the batch (1 KB loads), q_scale (dword loads)
    // and v_scale of the group's heads (1 KB loads).  Every wave issues exactly QNW of
    // them (padded with loads of a hot line) so the wait counts are static.
    constexpr int QI = kQRowsMax * 256 / 1024, QSI = kQRowsMax / 64, VSI = (HG * kHeadDim * 4 + 1023) / 1024;
    constexpr int QNW = (QI + QSI + VSI + HG - 1) / HG;
    static_assert(PER_STEP * (AHEAD - 1) + QNW < 64, "vmcnt range");

    __shared__ __attribute__((aligned(16))) uint8_t s_ring[NST][CHUNK];
    __shared__ __attribute__((aligned(16))) float s_ks[NST][HG][64];
    __shared__ __attribute__((aligned(16))) uint8_t s_q[kQRowsMax * 256];
    __shared__ __attribute__((aligned(16))) float s_qs[kQRowsMax];
    __shared__ int s_pref[kPrefixMax + 1];
    // v_scale of the group's heads, double-buffered: the next sequence's is staged
    // before the current one's flush has read it.  Rows padded to whole 1 KB loads.
    __shared__ __attribute__((aligned(16))) float s_vs[2][VSI * 2][kHeadDim];
    __shared__ __attribute__((aligned(16))) float s_qpad[HG][64];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // head of the group
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int NG = a.nkv / HG;            // head groups per token row
    const int BV = a.B * NG;              // virtual sequences: (batch, head group)

    // ---- tiles per virtual sequence and their exclusive prefix (wave 0) -------------------
    if (w == 0) {
        const int strip = (BV + 63) / 64;
        const int v0 = lane * strip, v1 = min(v0 + strip, BV);
        int sum = 0;
        for (int v = v0; v < v1; ++v) {
            int s = a.seqs[v / NG];
            s = s < 0 ? 0 : (s > a.capacity ? a.capacity : s);
            sum += (s + T - 1) / T;
        }
        int incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int x = __shfl_up(incl, o, 64);
            if (lane >= o) incl += x;
        }
        int run = incl - sum;
        for (int v = v0; v < v1; ++v) {
            s_pref[v] = run;
            int s = a.seqs[v / NG];
            s = s < 0 ? 0 : (s > a.capacity ? a.capacity : s);
            run += (s + T - 1) / T;
        }
        if (lane == 63) s_pref[BV] = incl;
    }
    __syncthreads();
    const int U = __builtin_amdgcn_readfirstlane(s_pref[BV]);
    const int Geff = min((int)gridDim.x, U);
    const int g = blockIdx.x;

    if (g == 0) {
        // publish the partition for the merge kernel; zero the rows of empty sequences
        for (int i = threadIdx.x; i <= BV; i += HG * 64) a.rows_meta[i] = s_pref[i];
        if (threadIdx.x == 0) a.rows_meta[BV + 1] = Geff;
        for (int b = 0; b < a.B; ++b) {
            if (s_pref[b * NG + NG] != s_pref[b * NG]) continue;
            for (int e = threadIdx.x; e < a.s1 * a.nq * kHeadDim; e += HG * 64)
                a.out[(int64_t)b * a.s1 * a.nq * kHeadDim + e] = 0;
        }
    }
    if (g >= Geff) return;

    // Atoms (tile u, head w of the group) are numbered u * HG + w; this workgroup
    // owns [a0, a1).  Every range holds at least HG atoms (Geff <= U), so it
    // meets every head of the group.
    const int64_t A = (int64_t)U * HG;
    const int64_t a0 = (int64_t)g * A / Geff, a1 = (int64_t)(g + 1) * A / Geff;
    const int u_first = (int)(a0 / HG), u_end = (int)((a1 - 1) / HG) + 1;

    auto unit_info = [&](int u) -> RowsUnit {
        RowsUnit r;
        int lo = 0, hi = BV - 1;              // largest v with s_pref[v] <= u
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (__builtin_amdgcn_readfirstlane(s_pref[mid]) <= u) lo = mid; else hi = mid - 1;
        }
        r.v = lo;                             // s_pref[lo] <= u < s_pref[lo + 1]
        r.b = lo / NG;
        r.h0 = (lo - r.b * NG) * HG;
        r.t = u - __builtin_amdgcn_readfirstlane(s_pref[lo]);
        r.hlo = (int)max((int64_t)0, a0 - (int64_t)u * HG);
        r.hhi = (int)min((int64_t)HG, a1 - (int64_t)u * HG);
        const int s = ld_uniform(a.seqs, r.b);
        r.seq = s < 0 ? 0 : (s > a.capacity ? a.capacity : s);
        return r;
    };

    // ---- per-lane constants of the staged layout ----------------------------------------
    const int64_t tok_stride = (int64_t)a.nkv * kHeadDim;      // one token row, all heads
    // DMA: load i of wave w fills 16-byte slots [(4w + i) 64, +64); slot -> (token, piece)
    uint32_t dmaoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int s = (4 * w + i) * 64 + lane;
        const int t = s / (8 * HG);
        const int p = (s % (8 * HG)) ^ swz<HG>(t);
        dmaoff[i] = (uint32_t)(t * tok_stride + 16 * p);
    }
    // K operand reads: token lr (+16), pieces 8w + lg and 8w + 4 + lg.  V operand
    // reads: token chunk_token(lg, j), bytes [8lr, 8lr + 8) of head w.  Token t + 16
    // has the swizzle of t, so the second half is a constant offset.
    int kslot[2], vaddr[4];
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf) {
        const int t = lr, p = 8 * w + 4 * hlf + lg;
        kslot[hlf] = (t * 8 * HG + (p ^ swz<HG>(t))) * 16;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = chunk_token(lg, j), p = 8 * w + (lr >> 1);
        vaddr[j] = (t * 8 * HG + (p ^ swz<HG>(t))) * 16 + 8 * (lr & 1);
    }

    const int qrows_ = a.s1 * a.nq;
    const int qbytes_ = qrows_ * 256;
    const int lane_ = lane;

    // Physical first token row of each 128-token block of a unit's tile (scalar).
    constexpr int BPT = T / kBlock;
    struct UnitBlocks {
        int64_t row0[BPT];
    };
    auto unit_blocks = [&](const RowsUnit& ui, bool ok) -> UnitBlocks {
        UnitBlocks ub;
        // all entries are loaded (index clamped to the row) so the loads issue together
        int raw[BPT];
#pragma unroll
        for (int i = 0; i < BPT; ++i)
            raw[i] = ld_uniform(a.block_table, (int64_t)ui.b * a.max_blocks + min(ui.t * BPT + i, a.max_blocks - 1));
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int p = ui.t * T + i * kBlock;
            const int id = (ok && p < ui.seq && raw[i] >= 0 && raw[i] < a.num_blocks) ? raw[i] : 0;
            ub.row0[i] = (int64_t)id * kBlock;
        }
        return ub;
    };

    // Issue the loads of step `r` (static) of a unit into ring stage `st`:
    // 4 chunk loads and one k_scale load per wave (PER_STEP, always).
    auto issue = [&](int r, int st, const RowsUnit& ui, const UnitBlocks& ub, bool unit_ok) {
        const int c = r < NCH ? r : r - NCH;
        const bool isv = r >= NCH;
        const bool valid = unit_ok && ui.t * T + 32 * c < ui.seq;
        const bool full = ui.hlo == 0 && ui.hhi == HG;
        const int64_t slot0 = valid ? ub.row0[c / 4] + 32 * (c % 4) : 0;
        const uint8_t* cache = isv ? a.v_cache : a.k_cache;
        const uint8_t* base = cache + slot0 * tok_stride + ui.h0 * kHeadDim;
        int ln = lane_;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bool use = valid;
            if (!full) {
                // only the heads of this workgroup's atoms are read
                const int s = (4 * w + i) * 64 + ln;
                const int t = s / (8 * HG);
                const int head = ((s % (8 * HG)) ^ swz<HG>(t)) >> 3;
                use = use && head >= ui.hlo && head < ui.hhi;
            }
            const uint8_t* src = use ? base + dmaoff[i] : cache + 16 * ln;   // unused lanes: a hot line
            dma_b128(src, (lds_ptr)(&s_ring[st][(4 * w + i) * 1024]));
        }
        // k_scale of head w, tokens lane & 31 (lanes 32-63 repeat them)
        const bool kuse = valid && !isv && w >= ui.hlo && w < ui.hhi;
        const float* ksrc = kuse ? a.k_scale + (slot0 + (ln & 31)) * a.nkv + ui.h0 + w : a.k_scale + (ln & 31);
        dma_b32(ksrc, (lds_ptr)(&s_ks[st][w][0]));
    };

    // The QNW loads of this wave that stage Q and q_scale of batch b and v_scale of
    // heads h0 .. h0+HG-1.  Rare (once per virtual sequence), so the addresses are
    // recomputed on every call: the opaque copies keep the compiler from hoisting
    // them out of the loop.
    auto issue_q = [&](int b, int h0, int buf) {
        int lane = lane_, qbytes = qbytes_, qrows = qrows_;
        asm volatile("" : "+v"(lane));
        asm volatile("" : "+s"(qbytes), "+s"(qrows));
        const uint8_t* qb = reinterpret_cast<const uint8_t*>(a.q) + (int64_t)b * qbytes;
        const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.v_scale + ((int64_t)b * a.nkv + h0) * kHeadDim);
#pragma unroll
        for (int n = 0; n < QNW; ++n) {
            const int j = w + n * HG;
            if (j < QI) {
                const int off = j * 1024 + 16 * lane;
                const uint8_t* src = off < qbytes ? qb + off : qb;        // past the rows: a line of them
                dma_b128(src, (lds_ptr)(&s_q[j * 1024]));
            } else if (j < QI + QSI) {
                const int row = (j - QI) * 64 + lane;
                const float* src = a.q_scale + (int64_t)b * qrows + (row < qrows ? row : 0);
                dma_b32(src, (lds_ptr)(&s_qs[(j - QI) * 64]));
            } else if (j < QI + QSI + VSI) {
                const int off = (j - QI - QSI) * 1024 + 16 * lane;
                const uint8_t* src = off < HG * kHeadDim * 4 ? vb + off : vb;
                dma_b128(src, (lds_ptr)(reinterpret_cast<uint8_t*>(&s_vs[buf][0][0]) + (j - QI - QSI) * 1024));
            } else {
                // padding: reload the batch's first q_scale into this wave's own slot
                dma_b32(a.q_scale + (int64_t)b * qrows, (lds_ptr)(&s_qpad[w][0]));
            }
        }
    };

    // ---- running state of this wave's head ------------------------------------------------
    bf16x8 qop[NRB][4];
    float qcoef[NRB];
    float M_s[NRB], L_s[NRB], M_o[NRB][4];
    f32x4 O[NRB][8];
    bool has_state = false;

    // prologue: Q of the first virtual sequence, then the first AHEAD steps
    RowsUnit cur = unit_info(u_first);
    RowsUnit nxt = (u_first + 1 < u_end) ? unit_info(u_first + 1) : cur;
    UnitBlocks cub = unit_blocks(cur, true);
    UnitBlocks nub = unit_blocks(nxt, u_first + 1 < u_end);
    issue_q(cur.b, cur.h0, 0);
    int last_q_step = 0;                     // step whose loads included the latest Q staging
    int nseg_issued = 1;                     // sequences staged so far (segment i uses s_vs[i & 1])
    int vs_buf = 1;                          // s_vs buffer of the current segment
#pragma unroll
    for (int r = 0; r < AHEAD; ++r) issue(r, r % NST, cur, cub, true);
    int prev_v = -1;                         // virtual sequence of the previous unit
    int step0 = 0;                           // global step index of the unit's first step

    for (int u = u_first; u < u_end; ++u, step0 += STEPS) {
        const bool seg_start = (cur.v != prev_v);
        if (seg_start) vs_buf ^= 1;
        const bool next_ok = (u + 1 < u_end);
        const bool next_new_seg = next_ok && (nxt.v != cur.v);
        const bool active = (w >= cur.hlo && w < cur.hhi);
        const int h = cur.h0 + w;            // this wave's KV head in the unit
        float sv[NRB][NCH][8];
        uint32_t p8[NRB][NCH][2];             // FP8 codes of 448 P for the whole tile
        float rmax[NRB], mt_s[NRB], mt_o[NRB][4], lsum[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            rmax[rb] = -INFINITY;
            lsum[rb] = 0.f;
        }

#pragma unroll
        for (int r = 0; r < STEPS; ++r) {
            const int step = step0 + r;
            const int st = step % NST;
            // ---- wait for this step's chunk (own loads), then for every wave -----------
            // Loads complete in issue order; the ones issued after this step's are the
            // chunk loads of the next AHEAD-1 steps, plus QNW Q-staging loads if those
            // were issued with one of them.
            if (last_q_step > step && last_q_step <= step + AHEAD - 1)
                wait_vm<PER_STEP * (AHEAD - 1) + QNW>();
            else
                wait_vm<PER_STEP * (AHEAD - 1)>();
            barrier_nofence();
            // ---- keep AHEAD chunks in flight: issue step + AHEAD ------------------------
            {
                const int rn = r + AHEAD;
                if (rn < STEPS) {
                    issue(rn, (step + AHEAD) % NST, cur, cub, true);
                } else {
                    if (rn == STEPS && next_new_seg) {
                        issue_q(nxt.b, nxt.h0, nseg_issued & 1);   // staged with the next unit's first step
                        ++nseg_issued;
                        last_q_step = step + AHEAD;
                    }
                    issue(rn - STEPS, (step + AHEAD) % NST, nxt, nub, next_ok);
                }
            }
            const uint8_t* ring = s_ring[st];
            const int c = r < NCH ? r : r - NCH;
            const int p0 = cur.t * T + 32 * c;
            const bool valid = p0 < cur.seq;

            if (r == 0 && seg_start) {
                // ---- step 1: this head's query rows -> bf16 operands of exact FP8 codes
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb) {
                    const int rr = rb * 16 + lr;
                    uint32_t wds[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    qcoef[rb] = 0.f;
                    if (rr < a.rows) {
                        const int s = rr / a.G, gq = rr % a.G;
                        const int qi = s * a.nq + h * a.G + gq;        // row inside the staged block
                        const float qs = s_qs[qi];
                        qcoef[rb] = qs * a.softmax_scale * kLog2e;
#pragma unroll
                        for (int hlf = 0; hlf < 2; ++hlf) {
                            const uint8_t* qp = s_q + qi * 256 + (hlf * 64 + 16 * lg) * 2;
                            const i32x4 v0 = *reinterpret_cast<const i32x4*>(qp);
                            const i32x4 v1 = *reinterpret_cast<const i32x4*>(qp + 16);
                            const uint32_t raw[8] = {(uint32_t)v0[0], (uint32_t)v0[1], (uint32_t)v0[2], (uint32_t)v0[3],
                                                     (uint32_t)v1[0], (uint32_t)v1[1], (uint32_t)v1[2], (uint32_t)v1[3]};
                            quantise_q16(raw, qs, &wds[hlf * 4]);
                        }
                        if (DBG && a.dbg_q8) {
                            const int64_t qrow = ((int64_t)cur.b * a.s1 + s) * a.nq + h * a.G + gq;
                            uint8_t* dst = a.dbg_q8 + qrow * kHeadDim;
#pragma unroll
                            for (int hlf = 0; hlf < 2; ++hlf)
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    *reinterpret_cast<uint32_t*>(dst + hlf * 64 + 16 * lg + 4 * i) = wds[hlf * 4 + i];
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) qop[rb][i] = fp8x8_to_op(wds[2 * i], wds[2 * i + 1]);
                    M_s[rb] = -INFINITY;
                    L_s[rb] = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) M_o[rb][i] = -INFINITY;
#pragma unroll
                    for (int cc = 0; cc < 8; ++cc) O[rb][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                has_state = false;
            }

            if (r < NCH) {
                // ---- steps 2-4: S^T = K Q^T, dequantise, mask ----------------------------
                if (active && valid) {
                    if (DBG && a.dbg_rows && h == 0 && lg == 0) {
                        const int64_t s0 = cub.row0[c / 4] + 32 * (c % 4);
#pragma unroll
                        for (int k = 0; k < 2; ++k)
                            if (p0 + 16 * k + lr < cur.seq)
                                a.dbg_rows[(int64_t)cur.b * a.capacity + p0 + 16 * k + lr] = (int32_t)(s0 + 16 * k + lr);
                    }
                    float ks[8];
                    {
                        const f32x4 k0 = *reinterpret_cast<const f32x4*>(&s_ks[st][w][4 * lg]);
                        const f32x4 k1 = *reinterpret_cast<const f32x4*>(&s_ks[st][w][16 + 4 * lg]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            ks[i] = k0[i];
                            ks[4 + i] = k1[i];
                        }
                    }
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const i32x4 lo = *reinterpret_cast<const i32x4*>(ring + kslot[0] + k * TOK16);
                        const i32x4 hi = *reinterpret_cast<const i32x4*>(ring + kslot[1] + k * TOK16);
                        f32x4 acc[NRB];
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const bf16x8 kop = (i < 2) ? fp8x8_to_op((uint32_t)lo[2 * i], (uint32_t)lo[2 * i + 1])
                                                       : fp8x8_to_op((uint32_t)hi[2 * i - 4], (uint32_t)hi[2 * i - 3]);
#pragma unroll
                            for (int rb = 0; rb < NRB; ++rb) acc[rb] = mfma_bf16(kop, qop[rb][i], acc[rb]);
                        }
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) sv[rb][c][4 * k + i] = acc[rb][i] * ks[4 * k + i] * qcoef[rb];
                    }
                    if (p0 + 32 > cur.seq) {
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                            for (int j = 0; j < 8; ++j)
                                sv[rb][c][j] = (p0 + chunk_token(lg, j) < cur.seq) ? sv[rb][c][j] : -INFINITY;
                    }
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                        for (int j = 0; j < 8; ++j) rmax[rb] = fmaxf(rmax[rb], sv[rb][c][j]);
                } else {
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                        for (int j = 0; j < 8; ++j) sv[rb][c][j] = -INFINITY;
                }

                if (r == NCH - 1 && active) {
                    // ---- step 5a: tile max per row; O <- O * exp2(M_old - m_tile) ----------
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        const float m = wave_max_over_groups(rmax[rb]);
                        mt_s[rb] = m;
                        // P' = 448 exp2(S - m_tile) = exp2(S + off); a dropped row gets off = -inf
                        const float poff = (M_s[rb] - m > kDropLog2) ? -INFINITY : kLog2_448 - m;
                        // steps 5b-6 for the whole tile: the FP8 code of P' (the tile's max maps
                        // to 448) and the running sum of the unquantised P'
#pragma unroll
                        for (int cc = 0; cc < NCH; ++cc) {
                            float pv[8];
#pragma unroll
                            for (int j = 0; j < 8; ++j) {
                                pv[j] = __builtin_amdgcn_exp2f(sv[rb][cc][j] + poff);
                                lsum[rb] += pv[j];
                            }
                            p8[rb][cc][0] = cvt4_fp8(pv[0], pv[1], pv[2], pv[3]);
                            p8[rb][cc][1] = cvt4_fp8(pv[4], pv[5], pv[6], pv[7]);
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float mo = __shfl(m, 4 * lg + i, 64);
                            mt_o[rb][i] = mo;
                            const float d = M_o[rb][i] - mo;
                            const float sc = d > kDropLog2 ? 1.f : __builtin_amdgcn_exp2f(d);
#pragma unroll
                            for (int cc = 0; cc < 8; ++cc) O[rb][cc][i] *= sc;
                        }
                    }
                }
            } else {
                // ---- steps 5b-7: P, per-tile FP8 quantisation, P.V -------------------------
                if (active && valid) {
                    uint32_t xl[8], xh[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint2 x = *reinterpret_cast<const uint2*>(ring + vaddr[j & 3] + (j >> 2) * TOK16);
                        xl[j] = x.x;
                        xh[j] = x.y;
                    }
                    if (p0 + 32 > cur.seq) {
                        // tokens past the sequence: zero their V bytes (0 * NaN would poison P.V)
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const bool in = p0 + chunk_token(lg, j) < cur.seq;
                            xl[j] = in ? xl[j] : 0u;
                            xh[j] = in ? xh[j] : 0u;
                        }
                    }
                    uint32_t ylo[8], yhi[8];
                    transpose4(xl[0], xl[1], xl[2], xl[3], ylo[0], ylo[1], ylo[2], ylo[3]);
                    transpose4(xl[4], xl[5], xl[6], xl[7], yhi[0], yhi[1], yhi[2], yhi[3]);
                    transpose4(xh[0], xh[1], xh[2], xh[3], ylo[4], ylo[5], ylo[6], ylo[7]);
                    transpose4(xh[4], xh[5], xh[6], xh[7], yhi[4], yhi[5], yhi[6], yhi[7]);
                    bf16x8 pop[NRB];
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) pop[rb] = fp8x8_to_op(p8[rb][c][0], p8[rb][c][1]);
#pragma unroll
                    for (int cc = 0; cc < 8; ++cc) {
                        const bf16x8 vop = fp8x8_to_op(ylo[cc], yhi[cc]);
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb) O[rb][cc] = mfma_bf16(pop[rb], vop, O[rb][cc]);
                    }
                }

                if (r == STEPS - 1 && active) {
                    // ---- steps 8-9: finish the rescale, update the running state -----------
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        const float mn = fmaxf(M_s[rb], mt_s[rb]);
                        L_s[rb] = L_s[rb] * __builtin_amdgcn_exp2f(M_s[rb] - mn) +
                                  lsum[rb] * __builtin_amdgcn_exp2f(mt_s[rb] - mn);
                        M_s[rb] = mn;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float mo = fmaxf(M_o[rb][i], mt_o[rb][i]);
                            const float d = M_o[rb][i] - mt_o[rb][i];
                            const float sc = d > kDropLog2 ? 1.f : __builtin_amdgcn_exp2f(mt_o[rb][i] - mo);
                            M_o[rb][i] = mo;
#pragma unroll
                            for (int cc = 0; cc < 8; ++cc) O[rb][cc][i] *= sc;
                        }
                    }
                    has_state = true;
                }
            }
        }

        // ---- end of a (virtual sequence, head) segment: finish in place or write a partial --
        const bool seg_end = !next_ok || next_new_seg;
        if (seg_end && has_state) {
            const int b = cur.b;
            const int pv0 = __builtin_amdgcn_readfirstlane(s_pref[cur.v]);
            const int64_t nb = __builtin_amdgcn_readfirstlane(s_pref[cur.v + 1]) - pv0;
            const int64_t af = (int64_t)pv0 * HG + w, al = (pv0 + nb - 1) * HG + w;
            const int64_t gf = ((af + 1) * Geff - 1) / A, gl = ((al + 1) * Geff - 1) / A;
            const int count = (int)(gl - gf + 1);
            const int k = (int)(g - gf);
            float Lw[NRB];
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) Lw[rb] = wave_sum_over_groups(L_s[rb]);
            const f32x4 vs0 = *reinterpret_cast<const f32x4*>(&s_vs[vs_buf][w][8 * lr]);
            const f32x4 vs1 = *reinterpret_cast<const f32x4*>(&s_vs[vs_buf][w][8 * lr + 4]);
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = rb * 16 + 4 * lg + i;
                    const float Lr = __shfl(Lw[rb], 4 * lg + i, 64);
                    if (rr >= a.rows) continue;
                    const int s = rr / a.G, gq = rr % a.G;
                    const int64_t qrow = ((int64_t)b * a.s1 + s) * a.nq + h * a.G + gq;
                    if (count == 1) {
                        // step 10: out = O * v_scale / L' (L' = 448 L), bf16
                        const float inv = 1.f / Lr;
                        uint32_t pk[4];
#pragma unroll
                        for (int q2 = 0; q2 < 4; ++q2) {
                            const int c0 = 2 * q2, c1 = 2 * q2 + 1;
                            const float x0 = O[rb][c0][i] * (c0 < 4 ? vs0[c0] : vs1[c0 - 4]) * inv;
                            const float x1 = O[rb][c1][i] * (c1 < 4 ? vs0[c1] : vs1[c1 - 4]) * inv;
                            pk[q2] = (uint32_t)f32_to_bf16_rne(x0) | ((uint32_t)f32_to_bf16_rne(x1) << 16);
                        }
                        *reinterpret_cast<i32x4*>(a.out + qrow * kHeadDim + 8 * lr) =
                            i32x4{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
                    } else {
                        const int64_t slot = ((int64_t)b * a.nkv + h) * a.rows_kmax + k;
                        float* po = a.part_o + (slot * R + rr) * kHeadDim + 8 * lr;
                        *reinterpret_cast<f32x4*>(po) = f32x4{O[rb][0][i], O[rb][1][i], O[rb][2][i], O[rb][3][i]};
                        *reinterpret_cast<f32x4*>(po + 4) = f32x4{O[rb][4][i], O[rb][5][i], O[rb][6][i], O[rb][7][i]};
                        if (lr == 0) {
                            float* pm = a.part_ml + (slot * R + rr) * 2;
                            pm[0] = M_o[rb][i];
                            pm[1] = Lr;
                        }
                    }
                }
            }
            has_state = false;
        }

        prev_v = cur.v;
        cur = nxt;
        cub = nub;
        if (u + 2 < u_end) {
            nxt = unit_info(u + 2);
            nub = unit_blocks(nxt, true);
        }
    }
    // drain the ring before the workgroup retires (padding loads may still be in flight)
    wait_vm<0>();
}

// Merge the partials of every (batch, KV head) that several workgroups worked on,
// in workgroup order (deterministic).  One wave per output row.
__global__ __launch_bounds__(256) void merge_rows_kernel(DecodeParams a, int R, int HG) {
    const int lane = threadIdx.x & 63;
    const int64_t row_id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // over B * nkv * rows
    const int64_t total = (int64_t)a.B * a.nkv * a.rows;
    if (row_id >= total) return;
    const int rr = (int)(row_id % a.rows);
    const int bh = (int)(row_id / a.rows);
    const int b = bh / a.nkv, h = bh % a.nkv;
    const int NG = a.nkv / HG, BV = a.B * NG;
    const int v = b * NG + h / HG, hl = h % HG;
    const int* meta = a.rows_meta;
    const int U = meta[BV], Geff = meta[BV + 1];
    const int nb = meta[v + 1] - meta[v];
    if (nb == 0 || Geff <= 0) return;
    const int64_t A = (int64_t)U * HG;
    const int64_t af = (int64_t)meta[v] * HG + hl, al = ((int64_t)meta[v] + nb - 1) * HG + hl;
    const int64_t gf = ((af + 1) * Geff - 1) / A, gl = ((al + 1) * Geff - 1) / A;
    const int count = (int)(gl - gf + 1);
    if (count <= 1) return;
    const int64_t slot0 = ((int64_t)b * a.nkv + h) * a.rows_kmax;
    float Ms = -INFINITY;
    for (int k = 0; k < count; ++k) Ms = fmaxf(Ms, a.part_ml[((slot0 + k) * R + rr) * 2]);
    float L = 0.f, o0 = 0.f, o1 = 0.f;
    for (int k = 0; k < count; ++k) {
        const float* pm = a.part_ml + ((slot0 + k) * R + rr) * 2;
        const float f = __builtin_amdgcn_exp2f(pm[0] - Ms);
        L += pm[1] * f;
        const float2 o = *reinterpret_cast<const float2*>(a.part_o + ((slot0 + k) * R + rr) * kHeadDim + 2 * lane);
        o0 += o.x * f;
        o1 += o.y * f;
    }
    const int s = rr / a.G, gq = rr % a.G;
    const int64_t qrow = ((int64_t)b * a.s1 + s) * a.nq + h * a.G + gq;
    const float* vs = a.v_scale + ((int64_t)b * a.nkv + h) * kHeadDim;
    const uint16_t r0 = f32_to_bf16_rne(o0 * vs[2 * lane] / L);
    const uint16_t r1 = f32_to_bf16_rne(o1 * vs[2 * lane + 1] / L);
    *reinterpret_cast<uint32_t*>(a.out + qrow * kHeadDim + 2 * lane) = (uint32_t)r0 | ((uint32_t)r1 << 16);
}

// ------------------------------------------------------------------ dispatch

// Ring stages of the four-head kernel: 16 KB each; six keep 80 KB of loads in
// flight per CU within the 160 KB of LDS.
#ifndef PA_ROWS_NST4
#define PA_ROWS_NST4 6
#endif

// Heads per workgroup: one wave per head, at most four (one wave per SIMD, so
// each wave has the 256 VGPRs that a 512-token score tile needs).
int rows_group(int nkv) { return nkv >= 4 ? 4 : nkv; }

template <int NRB, int NCH, int HG, int NST>
static hipError_t launch_rows_t(const DecodeParams& p, int grid, hipStream_t st, bool dbg) {
    if (dbg)
        hipLaunchKernelGGL((decode_rows_kernel<NRB, NCH, HG, NST, true>), dim3(grid), dim3(HG * 64), 0, st, p);
    else
        hipLaunchKernelGGL((decode_rows_kernel<NRB, NCH, HG, NST, false>), dim3(grid), dim3(HG * 64), 0, st, p);
    return hipGetLastError();
}

// Shapes of the whole-row path: (s2_tile, padded rows) in {128, 256} x {16, 32}
// and 512 x 16.
template <int HG, int NST>
static hipError_t launch_rows_hg(const DecodeParams& p, int grid, hipStream_t st, bool dbg) {
    const int nrb = (p.rows + 15) / 16;
    switch (p.s2_tile) {
        case 128:
            if (nrb == 1) return launch_rows_t<1, 4, HG, NST>(p, grid, st, dbg);
            return launch_rows_t<2, 4, HG, NST>(p, grid, st, dbg);
        case 256:
            if (nrb == 1) return launch_rows_t<1, 8, HG, NST>(p, grid, st, dbg);
            return launch_rows_t<2, 8, HG, NST>(p, grid, st, dbg);
        default:
            return launch_rows_t<1, 16, HG, NST>(p, grid, st, dbg);
    }
}

bool rows_path_supported(int nkv, int s2_tile, int rows, int s1, int nq, int B) {
    const int rpad = (rows + 15) / 16 * 16;
    return (nkv == 1 || nkv == 2 || nkv == 4 || nkv == 8) && (s2_tile == 128 || s2_tile == 256 || s2_tile == 512) &&
           rpad <= 32 && s2_tile * rpad <= 8192 && s1 * nq <= kQRowsMax &&
           (int64_t)B * (nkv / rows_group(nkv)) <= kPrefixMax;
}

hipError_t launch_decode_rows(const DecodeParams& p, int cus, hipStream_t st, bool dbg) {
    hipError_t e;
    const int hg = rows_group(p.nkv);
    // one workgroup per CU for four heads (110 KB of LDS), else two
    const int grid = cus * (hg == 4 ? 1 : 2);
    switch (hg) {
        case 1: e = launch_rows_hg<1, 4>(p, grid, st, dbg); break;
        case 2: e = launch_rows_hg<2, 4>(p, grid, st, dbg); break;
        default: e = launch_rows_hg<4, PA_ROWS_NST4>(p, grid, st, dbg); break;
    }
    if (e != hipSuccess) return e;
    const int R = (p.rows + 15) / 16 * 16;
    const int64_t total = (int64_t)p.B * p.nkv * p.rows;
    hipLaunchKernelGGL(merge_rows_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, st, p, R, hg);
    return hipGetLastError();
}

}  // namespace pa
