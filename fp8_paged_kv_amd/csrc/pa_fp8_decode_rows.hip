// FP8 paged GQA decode, whole-row path (MI355X / gfx950).
//
// Same operation as the per-head path (web page "PyPTO 实现 GLM-4.5 Paged
// Attention FP8 量化算子…", section 计算流程 steps 1-10), organised for the
// memory system and for one wave per SIMD:
//
//  * A workgroup serves a group of HG <= 2 KV heads with 2*HG waves: wave
//    w = 2*hl + p owns head hl of the group and token half p of every
//    128-token cache block.  The two waves of a head exchange their row
//    maxima through LDS at the end of a tile's K pass, so both quantise P with
//    the maximum of the whole tile, exactly as one wave holding the tile would;
//    each then keeps only half of the tile's scores in registers.
//  * A step stages one cache block (128 tokens x the group's 128-byte head
//    slices, contiguous per token row) through an LDS ring filled by direct
//    global->LDS loads with a scalar base and 32-bit lane offsets.  Two steps
//    are always in flight.  The loads are issued from inline asm so the
//    compiler does not see them as LDS stores (it would otherwise drain them
//    before every LDS read); completion is ordered by hand with an explicit
//    vmcnt wait and a raw barrier at every step.
//  * Work unit = one tile of one (batch, head group).  The units of the whole
//    call, in (batch, group, tile) order, are split into contiguous ranges of
//    equal cost (2 steps per valid block, plus a charge for each sequence
//    start), one per workgroup; blocks past a sequence's end cost nothing and
//    are not visited.  A (batch, group) whose
//    tiles land in one workgroup is finished in place.  Otherwise every
//    workgroup writes an (O, M, L) partial and a second, small kernel merges
//    them (the kernel boundary orders the writes; no fences or atomics).
#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

#include "pa_fp8_common.h"
#include "pa_fp8_device.h"

// Phase timing, built only into the phase-stamp variant of the library (PA_FP8_PHASES;
// the results are those of the plain build): sixteen 64-bit words per workgroup --
// 0 entry, 1 start of the main loop, 2 exit, 3 summed query conversion, 4 summed
// segment ends (combine and stores), 5 steps, 6 segments, 7 first step's data,
// 8 lengths staged, 9 cost prefix done, 10 first unit found, 11 its table entries
// arrived -- times from s_memrealtime (100 MHz).
#ifdef PA_FP8_PHASES
static __device__ unsigned long long g_rows_phases[256 * 16];
extern "C" unsigned long long* pa_fp8_phases_rows() {
    void* p = nullptr;
    return hipGetSymbolAddress(&p, HIP_SYMBOL(g_rows_phases)) == hipSuccess ? (unsigned long long*)p : nullptr;
}
#define PH_NOW() __builtin_amdgcn_s_memrealtime()
#define PH_SET(k, v) do { if (threadIdx.x == 0) g_rows_phases[blockIdx.x * 16 + (k)] = (v); } while (0)
#else
#define PH_NOW() 0ull
#define PH_SET(k, v) do { } while (0)
#endif

namespace pa {

typedef __attribute__((address_space(3))) void* lds_ptr;

// A wave-uniform pointer, forced into scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// Direct global->LDS loads: lane i writes dst + size * i from sbase + voff_i.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, lds_ptr dst) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(uniform_ptr(sbase)), "s"((uint32_t)(uintptr_t)dst) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, lds_ptr dst) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(voff), "s"(uniform_ptr(sbase)), "s"((uint32_t)(uintptr_t)dst) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) lgkmcnt(0), gfx9 encoding.  vmcnt counts this wave's
// vector memory operations, which complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) only (vmcnt left at its maximum, 63).
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Workgroup barrier that is also a compiler memory barrier, without the
// release fence of __syncthreads (which would wait for every load in flight).
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// Load of a wave-uniform int32 through the constant address space, i.e. as a
// scalar load (a vector load would share vmcnt with the ring's loads).
__device__ __forceinline__ int ld_uniform(const int32_t* p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

__device__ __forceinline__ int lds_uniform(const int* p) { return __builtin_amdgcn_readfirstlane(*p); }

// Inclusive prefix sum over the 64 lanes of a wave: row shifts by 1, 2, 4 and 8 (a lane
// with no source in its 16-lane row adds 0), then lane 15 of rows 0 and 2 into rows 1
// and 3, and lane 31 into rows 2 and 3 (DPP row broadcasts).
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
    return x;
}

// floor(x / d) for 0 <= x and x + d < 2^22, given inv = 1.0f / d (IEEE): (x + 0.5) / d lies at
// least 0.5 / d from an integer and the two roundings move it by less than that.
__device__ __forceinline__ int small_div(int x, float inv) { return (int)(((float)x + 0.5f) * inv); }

// floor(num / den) for 0 <= num < 2^53, den > 0 and a quotient below 2^31, in double precision:
// a non-integer quotient is at least 1 / den from the next integer, far beyond the rounding.
__device__ __forceinline__ int floor_div64(int64_t num, int64_t den) { return (int)((double)num / (double)den); }

constexpr int kStepTok = 128;             // tokens per step = one cache block
constexpr int kPrefixMax = 1024;          // (batch, head group) pairs of one call
// Cost of starting a (batch, group) sequence in a workgroup (staging and converting its
// query rows, and finishing its output), in steps; the partition charges it to the
// sequence's first tile.  Measured at two to four steps; charges from 2 to 6 move the
// slowest range by a tile's rounding either way.
constexpr int kSegW = 4;

template <int NRB, int NBLK, int HG, bool DBG>
__global__ __launch_bounds__(2 * HG * 64) void decode_rows_kernel(DecodeParams a) {
    constexpr int NW = 2 * HG;            // waves: w = 2 * hl + p
    constexpr int NST = 3, AHEAD = 2;     // ring stages, steps in flight
    constexpr int T = NBLK * kStepTok;    // s2_tile
    constexpr int R = NRB * 16;           // padded query rows per head
    constexpr int NPC = 8 * HG;           // 16-byte pieces of a staged token (the group's heads)
    constexpr int TOKB = NPC * 16;        // LDS bytes of a staged token
    constexpr int STEP_BYTES = kStepTok * TOKB;
    constexpr int DPW = STEP_BYTES / 1024 / NW;   // 1 KB loads per wave and step
    constexpr int PER_STEP = DPW + 1;     // + the k_scale load
    constexpr int NQ = 2 * NBLK;          // 32-token chunks of a tile held by one wave
    constexpr int QROWS = 32 * HG;        // staged query rows (HG heads x <= 32 rows)
    constexpr int QI = QROWS * 256 / 1024, QNW = (QI + 2 + NW - 1) / NW;
    static_assert(DPW == 8, "eight 1 KB loads per wave and step");
    static_assert(PER_STEP * (AHEAD - 1) + QNW < 64, "vmcnt range");

    __shared__ __attribute__((aligned(16))) uint8_t s_ring[NST][STEP_BYTES];
    __shared__ __attribute__((aligned(16))) float s_ks[NST][NW][64];
    // query rows, q_scale and v_scale of the group, double-buffered by segment parity: the
    // next sequence's are staged while the current one may still be reading its own
    __shared__ __attribute__((aligned(16))) uint8_t s_q[2][QROWS * 256];
    __shared__ __attribute__((aligned(16))) float s_qs[2][64];
    __shared__ __attribute__((aligned(16))) float s_vs[2][256];
    // sequence ends: each token-half wave's outgoing four columns of O (4 rows x 64 lanes x
    // f32x4 per wave) and its 16 row sums, per head
    __shared__ __attribute__((aligned(16))) float s_comb[HG][2 * 1024 + 2 * 16];
    __shared__ __attribute__((aligned(16))) float s_max[NW][R];
    __shared__ __attribute__((aligned(16))) float s_qpad[NW][64];
    __shared__ int s_pref[kPrefixMax + 1];   // exclusive cost prefix over (batch, group), in steps
    __shared__ int s_seq[kPrefixMax];        // clamped length per batch
    __shared__ int s_units;

    const unsigned long long ph_t0 = PH_NOW();
    unsigned long long ph_q = 0, ph_end = 0, ph_t7 = 0;
    int ph_segs = 0;
    PH_SET(0, ph_t0);
    PH_SET(2, ph_t0);
    PH_SET(5, 0);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = w >> 1, p = w & 1;
    const int lr = lane & 15, lg = lane >> 4;
    // A unit of work is (batch, head group, row block): a KV head's query rows come in
    // blocks of 32 when there are more than 32 of them (a prefill chunk), each block a
    // sequence of its own here ("virtual batch" bv = b RBK + block), all reading the same
    // K and V; with at most 32 rows, RBK = 1 and bv = b.
    const int RBK = a.row_blocks, B = a.B * RBK, NG = a.nkv / HG, BV = B * NG;
    const int nkv = a.nkv;
    const float inv_ng = 1.0f / NG, inv_g = 1.0f / a.G, inv_rbk = 1.0f / RBK;

    // ---- lengths, cost prefix and unit count ------------------------------------------------
    for (int b = threadIdx.x; b < B; b += NW * 64) {
        const int s = a.seqs[RBK == 1 ? b : small_div(b, inv_rbk)];
        s_seq[b] = s < 0 ? 0 : (s > a.capacity ? a.capacity : s);
    }
    __syncthreads();
    PH_SET(8, PH_NOW());
    if (w == 0) {
        const int strip = (BV + 63) / 64;
        const int v0 = lane * strip, v1 = min(v0 + strip, BV);
        const int bs0 = small_div(v0, inv_ng), gs0 = v0 - bs0 * NG;   // batch and group of v0
        int cost = 0, units = 0;
        for (int v = v0, bb = bs0, gg = gs0; v < v1; ++v) {
            const int s = s_seq[bb];
            const int nb = (s + kStepTok - 1) / kStepTok;
            cost += 2 * nb + (nb > 0 ? kSegW : 0);
            units += (s + T - 1) / T;
            if (++gg == NG) {
                gg = 0;
                ++bb;
            }
        }
        const int incl = wave_incl_scan(cost);
        int run = incl - cost;
        for (int v = v0, bb = bs0, gg = gs0; v < v1; ++v) {
            s_pref[v] = run;
            const int nb = (s_seq[bb] + kStepTok - 1) / kStepTok;
            run += 2 * nb + (nb > 0 ? kSegW : 0);
            if (++gg == NG) {
                gg = 0;
                ++bb;
            }
        }
        if (lane == 63) s_pref[BV] = incl;
        units = wave_incl_scan(units);
        if (lane == 63) s_units = units;
    }
    __syncthreads();
    PH_SET(9, PH_NOW());
    const int64_t C = lds_uniform(&s_pref[BV]);
    const int U = lds_uniform(&s_units);
    const int Geff = min((int)gridDim.x, U);
    // workgroups are dispatched round-robin over the 8 XCDs: neighbouring ranges (usually
    // the head groups of one sequence, which read the same k_scale sectors and table row)
    // go to one XCD so that they share its L2
    const int G8 = (int)gridDim.x / 8;
    const int g = ((int)gridDim.x % 8 == 0) ? ((int)blockIdx.x % 8) * G8 + (int)blockIdx.x / 8 : (int)blockIdx.x;

    if (g == 0) {
        // the partition, for the merge kernel: cost prefix over (batch, group), then Geff
        for (int i = threadIdx.x; i <= BV; i += NW * 64) a.rows_meta[i] = s_pref[i];
        if (threadIdx.x == 0) a.rows_meta[BV + 1] = Geff;
    }
    // rows of empty sequences are zero: workgroup g clears batches g, g + grid, ...
    for (int b = g; b < a.B; b += gridDim.x) {
        if (lds_uniform(&s_seq[b * RBK]) != 0) continue;
        for (int e = threadIdx.x; e < a.s1 * a.nq * kHeadDim; e += NW * 64)
            a.out[(int64_t)b * a.s1 * a.nq * kHeadDim + e] = 0;
        if (DBG && a.dbg_q8) {
            // the query codes of step 1 for the dump, which no unit of this batch computes
            for (int e = threadIdx.x; e < a.s1 * a.nq * (kHeadDim / 16); e += NW * 64) {
                const int64_t qrow = (int64_t)b * a.s1 * a.nq + e / (kHeadDim / 16);
                const int d0 = 16 * (e % (kHeadDim / 16));
                const i32x4 v0 = *reinterpret_cast<const i32x4*>(a.q + qrow * kHeadDim + d0);
                const i32x4 v1 = *reinterpret_cast<const i32x4*>(a.q + qrow * kHeadDim + d0 + 8);
                const uint32_t raw[8] = {(uint32_t)v0[0], (uint32_t)v0[1], (uint32_t)v0[2], (uint32_t)v0[3],
                                         (uint32_t)v1[0], (uint32_t)v1[1], (uint32_t)v1[2], (uint32_t)v1[3]};
                uint32_t wds[4];
                quantise_q16(raw, q_recip(a.q_scale[qrow]), wds);
                *reinterpret_cast<i32x4*>(a.dbg_q8 + qrow * kHeadDim + d0) =
                    i32x4{(int)wds[0], (int)wds[1], (int)wds[2], (int)wds[3]};
            }
        }
    }
    if (g >= Geff) return;

    // Unit (v, t) spans cost [s_pref[v] + 2 NBLK t, + 2 nvs); its midpoint mid(v, t)
    // decides its workgroup: workgroup g owns the units whose midpoints lie in [lo, hi),
    // so a range is off its share by at most half a unit.
    const int lo = floor_div64((int64_t)g * C, Geff), hi = floor_div64((int64_t)(g + 1) * C, Geff);
    // A unit carries its sequence's batch, head group and length, so that stepping to the
    // next tile of the same sequence divides nothing.
    struct Unit {
        int v, b, h0, t, seq;                // b: the virtual batch
        int br, rk;                          // its batch and row block
        int nvs;                             // valid blocks (steps per pass); 0 = no unit
        int ids;                             // lane i < NBLK: physical block of block i of the tile
        int raw[NBLK];                       // the table entries as loaded (scalar), until finish_ids
    };
    auto nblocks = [&](int seq) { return (seq + kStepTok - 1) / kStepTok; };
    auto unit_mid = [&](const Unit& u, int t) -> int {
        return lds_uniform(&s_pref[u.v]) + (t == 0 ? kSegW / 2 : kSegW) + 2 * NBLK * t + min(NBLK, nblocks(u.seq) - t * NBLK);
    };
    // (v, b, h0, seq) name a sequence; t its tile; !ok = no unit
    auto make_unit = [&](int v, int b, int h0, int seq, int t, bool ok) -> Unit {
        Unit u;
        u.v = v;
        u.b = ok ? b : 0;
        u.h0 = ok ? h0 : 0;
        u.t = t;
        u.seq = ok ? seq : 0;
        u.br = RBK == 1 ? u.b : small_div(u.b, inv_rbk);
        u.rk = u.b - u.br * RBK;
        u.nvs = ok ? min(NBLK, nblocks(u.seq) - t * NBLK) : 0;
        // the scalar table loads are only issued here; finish_ids, called when the unit's
        // first step is about to be issued, waits for them (they then have long arrived)
#pragma unroll
        for (int i = 0; i < NBLK; ++i)
            u.raw[i] = ok ? ld_uniform(a.block_table, (int64_t)u.br * a.max_blocks + min(t * NBLK + i, a.max_blocks - 1)) : 0;
        u.ids = 0;
        return u;
    };
    // block ids into one VGPR (lane i = block i) to keep scalar registers free
    auto finish_ids = [&](Unit& u) {
        int ids = 0;
#pragma unroll
        for (int i = 0; i < NBLK; ++i)
            ids = (lane == i) ? ((i < u.nvs && u.raw[i] >= 0 && u.raw[i] < a.num_blocks) ? u.raw[i] : 0) : ids;
        u.ids = ids;
    };
    // the unit after u in this workgroup's range, or none
    auto next_unit = [&](const Unit& u) -> Unit {
        if (u.t + 1 < (u.seq + T - 1) / T) {
            const bool ok = unit_mid(u, u.t + 1) < hi;
            return make_unit(u.v, u.b, u.h0, u.seq, u.t + 1, ok);
        }
        // the next non-empty sequence: later groups of this batch, then later batches
        int v = u.v + 1, b = u.b, h0 = u.h0 + HG;
        if (h0 == nkv) {
            h0 = 0;
            ++b;
        }
        int seq = 0;
        while (v < BV && (seq = lds_uniform(&s_seq[b])) == 0) {
            v += (nkv - h0) / HG;
            ++b;
            h0 = 0;
        }
        if (v >= BV) return make_unit(0, 0, 0, 0, 0, false);
        const bool ok = lds_uniform(&s_pref[v]) + kSegW / 2 + min(NBLK, nblocks(seq)) < hi;   // tile 0's midpoint
        return make_unit(v, b, h0, seq, 0, ok);
    };

    // first unit: the first midpoint >= lo.  The largest v with s_pref[v] <= lo is found
    // with two rounds of 64 parallel LDS reads; it is a non-empty sequence (an empty one
    // would share its prefix with v + 1, and s_pref[BV] = C > lo).
    Unit cur;
    {
        const int stride = (BV + 63) / 64;
        const uint64_t m1 = __ballot(s_pref[min(lane * stride, BV - 1)] <= lo);
        const int base = min((__popcll(m1) - 1) * stride, BV - 1);
        const uint64_t m2 = __ballot(lane < stride && s_pref[min(base + lane, BV - 1)] <= lo);
        int v = __builtin_amdgcn_readfirstlane(min(base + __popcll(m2) - 1, BV - 1));
        int b = small_div(v, inv_ng), h0 = (v - b * NG) * HG;
        int seq = lds_uniform(&s_seq[b]);
        int pv = lds_uniform(&s_pref[v]);
        const int nbv = nblocks(seq), ntv = (seq + T - 1) / T;
        auto midv = [&](int t) { return pv + (t == 0 ? kSegW / 2 : kSegW) + 2 * NBLK * t + min(NBLK, nbv - t * NBLK); };
        const int d = lo - pv - kSegW - NBLK;       // mid of a full tile t > 0: pv + kSegW + NBLK (2t + 1)
        int t = d <= 0 ? 0 : min(ntv, (d + 2 * NBLK - 1) / (2 * NBLK));
        while (t > 0 && midv(t - 1) >= lo) --t;    // the last tile's midpoint is earlier
        while (t < ntv && midv(t) < lo) ++t;
        int mid;
        if (t < ntv) {
            mid = midv(t);
        } else {
            // every midpoint of v lies below lo: tile 0 of the next non-empty sequence
            t = 0;
            seq = 0;
            while (seq == 0) {
                ++v;
                h0 += HG;
                if (h0 == nkv) {
                    h0 = 0;
                    ++b;
                }
                if (v >= BV) {
                    if (threadIdx.x == 0) a.part_tag[2 * g] = a.part_tag[2 * g + 1] = -1;
                    return;
                }
                seq = lds_uniform(&s_seq[b]);
            }
            pv = lds_uniform(&s_pref[v]);
            mid = pv + kSegW / 2 + min(NBLK, nblocks(seq));
        }
        if (mid >= hi) {                            // no midpoint in this range: no work
            if (threadIdx.x == 0) a.part_tag[2 * g] = a.part_tag[2 * g + 1] = -1;
            return;
        }
        PH_SET(10, PH_NOW());
        cur = make_unit(v, b, h0, seq, t, true);   // its table loads overlap the Q staging below
    }
    const int first_v = cur.v;               // the range's first (batch, group)
    Unit nxt;
    bool nxt_ready = false;                  // finish_ids(nxt) done

    // ---- per-lane constants of the staged layout ----------------------------------------------
    // Slot (token t, physical piece pp) holds logical piece pp ^ (t mod NPC) of token t.
    const int64_t tok_stride = (int64_t)nkv * kHeadDim;        // bytes of one token row (all heads)
    uint32_t dmaoff[DPW];
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
        const int s = (DPW * w + i) * 64 + lane;
        const int t = s / NPC, pp = s % NPC;
        dmaoff[i] = (uint32_t)(t * tok_stride + 16 * (pp ^ (t & (NPC - 1))));
    }
    // K operand (token 16k + lr of a chunk; pieces 8hl + lg and 8hl + 4 + lg) and V operand
    // (token chunk_token(lg, j); bytes 8lr .. 8lr + 7 of head hl).  Tokens that differ by a
    // multiple of 16 share a swizzle, so chunk and half offsets are constants.
    int kslot[2], vaddr[4];
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf)
        kslot[hlf] = (lr * NPC + ((8 * hl + 4 * hlf + lg) ^ (lr & (NPC - 1)))) * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = chunk_token(lg, j), pc = 8 * hl + (lr >> 1);
        vaddr[j] = (t * NPC + (pc ^ (t & (NPC - 1)))) * 16 + 8 * (lr & 1);
    }
    const uint32_t ksoff = (uint32_t)(lane * nkv * 4);

    // Issue the loads of step `idx` of unit u (K pass: idx < nvs, then the V pass) into
    // stage st: DPW block loads and one k_scale load per wave, always PER_STEP.  Nothing is
    // issued past the last unit; the last step then waits for all loads.
    auto issue = [&](const Unit& u, int idx, int st) {
        const bool ok = u.nvs > 0;
        const bool isv = ok && idx >= u.nvs;
        const int blk = isv ? idx - u.nvs : (ok ? idx : 0);
        const int id = __builtin_amdgcn_readlane(u.ids, blk);
        const int64_t row0 = (int64_t)id * kStepTok;
        const uint8_t* base = (isv ? a.v_cache : a.k_cache) + row0 * tok_stride + u.h0 * kHeadDim;
#pragma unroll
        for (int i = 0; i < DPW; ++i) dma16(base, dmaoff[i], (lds_ptr)(&s_ring[st][(DPW * w + i) * 1024]));
        // k_scale of head h0 + hl, tokens 64p + lane of the block
        const float* ksb = a.k_scale + (row0 + 64 * p) * nkv + u.h0 + hl;
        dma4(ksb, ksoff, (lds_ptr)(&s_ks[st][w][0]));
    };

    // The QNW loads of this wave that stage the query rows and q_scale of the unit's heads
    // h0 .. h0+HG-1 and their v_scale.  Staged row sr = hs * qstride + rr (rr < the block's
    // rows) is query row ra = 32 rk + rr of head h0 + hs: b s1 nq + s nq + (h0 + hs) G + gq
    // with (s, gq) = divmod(ra, G).  Padding rows stage the batch's first row (unused).
    const int qstride = RBK == 1 ? a.rows : 32;   // staged rows per head
    const float inv_qstride = 1.0f / qstride;
    auto issue_q = [&](const Unit& u, int buf) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int rows_u = min(32, a.rows - 32 * u.rk);
        auto off_of = [&](int sr) {
            const int hs = small_div(sr, inv_qstride), rr = sr - hs * qstride;
            const int ra = 32 * u.rk + rr;
            const int s = small_div(ra, inv_g), gq = ra - s * a.G;
            return (sr < HG * qstride && rr < rows_u) ? s * a.nq + hs * a.G + gq : -1;
        };
        const int qrow0 = u.br * a.s1 * a.nq;                  // first query row of the batch
        const int qrowh = qrow0 + u.h0 * a.G;
#pragma unroll
        for (int n = 0; n < QNW; ++n) {
            const int j = w + n * NW;
            const int off = j < QI ? off_of(4 * j + (ln >> 4)) : (j == QI ? off_of(ln) : -1);
            const int row = off >= 0 ? qrowh + off : qrow0;
            if (j < QI) {
                dma16(a.q, (uint32_t)(row * 256 + 16 * (ln & 15)), (lds_ptr)(&s_q[buf][j * 1024]));
            } else if (j == QI) {
                dma4(a.q_scale, (uint32_t)(row * 4), (lds_ptr)(&s_qs[buf][0]));
            } else if (j == QI + 1) {
                const uint32_t vb = (uint32_t)((u.br * nkv + u.h0) * kHeadDim * 4);
                dma16(a.v_scale, vb + (16 * ln < HG * kHeadDim * 4 ? 16 * ln : 0), (lds_ptr)(&s_vs[buf][0]));
            } else {
                dma4(a.q_scale, (uint32_t)(qrow0 * 4), (lds_ptr)(&s_qpad[w][0]));
            }
        }
    };

    // ---- running state of this wave (head hl, token half p) -----------------------------------
    bf16x8 qop[NRB][4];
    float qcoef[NRB];
    int lim[NRB];                            // tokens this lane's query row attends to (causal: fewer)
    int mlim = 0;                            // the smallest of them over the rows
    float M_s[NRB], L_s[NRB], M_o[NRB][4];
    f32x4 O[NRB][8];

    // prologue: Q of the first sequence, then the first AHEAD steps (a unit has >= 2)
    issue_q(cur, 0);
    int last_q_step = 0;                     // step whose loads followed the latest Q staging
    int nseg_issued = 1;                     // sequences staged so far (segment i uses buffer i & 1)
    int vs_buf = 1;
    finish_ids(cur);
    PH_SET(11, PH_NOW());
    issue(cur, 0, 0);
    issue(cur, 1, 1);
    nxt = next_unit(cur);
    int gs = 0;                              // global step index (ring position)
    int prev_v = -1;

    // one step: wait for its loads, barrier, keep AHEAD steps in flight
    auto step_begin = [&](int idx) {
        if (idx + 1 >= 2 * cur.nvs && nxt.nvs == 0)
            wait_vm<0>();                        // the last step: nothing was issued behind it
        else if (last_q_step == gs + 1)
            wait_vm<PER_STEP * (AHEAD - 1) + QNW>();
        else
            wait_vm<PER_STEP * (AHEAD - 1)>();
        barrier_nofence();
        const int nidx = idx + AHEAD, st = (gs + AHEAD) % NST;
        if (nidx < 2 * cur.nvs) {
            issue(cur, nidx, st);
        } else {
            const int k = nidx - 2 * cur.nvs;   // 0 or 1; the next unit has >= 2 steps
            if (!nxt_ready) {
                finish_ids(nxt);
                nxt_ready = true;
            }
            if (k == 0 && nxt.nvs > 0 && nxt.v != cur.v) {
                issue_q(nxt, nseg_issued & 1);
                ++nseg_issued;
                last_q_step = gs + AHEAD;
            }
            if (nxt.nvs > 0) issue(nxt, k, st);
        }
    };

    PH_SET(1, PH_NOW());
    while (true) {
        const bool seg_start = cur.v != prev_v;
        const int cur_rows = min(32, a.rows - 32 * cur.rk);   // query rows of this unit's block
        if (seg_start) {
            vs_buf ^= 1;
        }
        const int h = cur.h0 + hl;
        float sv[NRB][NQ][8];
        uint32_t p8[NRB][NQ][2];
        float rmax[NRB], mt_s[NRB], mt_o[NRB][4], lsum[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            rmax[rb] = -INFINITY;
            lsum[rb] = 0.f;
        }

        // ---------------- K pass: steps 2-4, S = q8 . k8 * scales, masked -------------------------
#pragma unroll
        for (int r = 0; r < NBLK; ++r) {
            if (r < cur.nvs) {
                step_begin(r);
                if (gs == 0) ph_t7 = PH_NOW();
                const uint8_t* ring = s_ring[gs % NST];
                const float* ksr = s_ks[gs % NST][w];
                if (r == 0 && seg_start) {
                    const unsigned long long ph_a = PH_NOW();
                    ++ph_segs;
                    // step 1: this head's query rows -> bf16 operands of exact FP8 codes.  The two
                    // token-half waves of a head need the same operands: wave p converts the
                    // values of half p of each row (MFMA operands 2p, 2p + 1) and the halves are
                    // swapped through LDS (free here: the last sequence end is behind a barrier).
                    auto convert = [&](auto P) {
                        constexpr int PH = decltype(P)::value;
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb) {
                            const int rr = rb * 16 + lr;
                            uint32_t wds[4] = {0, 0, 0, 0};
                            qcoef[rb] = 0.f;
                            // causal decode: position s of s1 attends to the first seq - s1 + 1 + s tokens
                            const int ra = 32 * cur.rk + rr;       // the row among the head's s1 G
                            lim[rb] = cur.seq - (a.causal ? a.s1 - 1 - (rr < cur_rows ? small_div(ra, inv_g) : a.s1 - 1) : 0);
                            mlim = cur.seq - (a.causal ? a.s1 - 1 : 0);
                            if (rr < cur_rows) {
                                const int sr = hl * qstride + rr;
                                const float qs = s_qs[vs_buf][sr];
                                qcoef[rb] = qs * a.softmax_scale * kLog2e;
                                const uint8_t* qp = s_q[vs_buf] + sr * 256 + (PH * 64 + 16 * lg) * 2;
                                const i32x4 v0 = *reinterpret_cast<const i32x4*>(qp);
                                const i32x4 v1 = *reinterpret_cast<const i32x4*>(qp + 16);
                                const uint32_t raw[8] = {(uint32_t)v0[0], (uint32_t)v0[1], (uint32_t)v0[2], (uint32_t)v0[3],
                                                         (uint32_t)v1[0], (uint32_t)v1[1], (uint32_t)v1[2], (uint32_t)v1[3]};
                                quantise_q16(raw, q_recip(qs), wds);
                                if (DBG && a.dbg_q8) {
                                    const int s = small_div(ra, inv_g), gq = ra - s * a.G;
                                    const int64_t qrow = ((int64_t)cur.br * a.s1 + s) * a.nq + h * a.G + gq;
                                    uint8_t* dst = a.dbg_q8 + qrow * kHeadDim + PH * 64 + 16 * lg;
#pragma unroll
                                    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(dst + 4 * i) = wds[i];
                                }
                            }
#pragma unroll
                            for (int ii = 0; ii < 2; ++ii) {
                                qop[rb][2 * PH + ii] = fp8x8_to_op(wds[2 * ii], wds[2 * ii + 1]);
                                *reinterpret_cast<bf16x8*>(&s_comb[hl][PH * NRB * 512 + ((rb * 2 + ii) * 64 + lane) * 4]) =
                                    qop[rb][2 * PH + ii];
                            }
                        }
                        wait_lgkm();
                        barrier_nofence();
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                            for (int ii = 0; ii < 2; ++ii)
                                qop[rb][2 * (1 - PH) + ii] = *reinterpret_cast<const bf16x8*>(
                                    &s_comb[hl][(1 - PH) * NRB * 512 + ((rb * 2 + ii) * 64 + lane) * 4]);
                    };
                    if (p == 0) convert(std::integral_constant<int, 0>{});
                    else convert(std::integral_constant<int, 1>{});
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        M_s[rb] = -INFINITY;
                        L_s[rb] = 0.f;
#pragma unroll
                        for (int i = 0; i < 4; ++i) M_o[rb][i] = -INFINITY;
#pragma unroll
                        for (int cc = 0; cc < 8; ++cc) O[rb][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                    ph_q += PH_NOW() - ph_a;
                }
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const int q = 2 * r + cc;                      // chunk of this wave in the tile
                    const int tb = 64 * p + 32 * cc;               // first token of the chunk in the block
                    const int p0 = cur.t * T + r * kStepTok + tb;  // its logical position
                    if (DBG && a.dbg_rows && h == 0 && lg == 0) {
                        const int64_t s0 = (int64_t)__builtin_amdgcn_readlane(cur.ids, r) * kStepTok + tb;
#pragma unroll
                        for (int k = 0; k < 2; ++k)
                            if (p0 + 16 * k + lr < cur.seq)
                                a.dbg_rows[(int64_t)cur.br * a.capacity + p0 + 16 * k + lr] = (int32_t)(s0 + 16 * k + lr);
                    }
                    const f32x4 k0 = *reinterpret_cast<const f32x4*>(&ksr[32 * cc + 4 * lg]);
                    const f32x4 k1 = *reinterpret_cast<const f32x4*>(&ksr[32 * cc + 16 + 4 * lg]);
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const i32x4 klo = *reinterpret_cast<const i32x4*>(ring + kslot[0] + (tb + 16 * k) * TOKB);
                        const i32x4 khi = *reinterpret_cast<const i32x4*>(ring + kslot[1] + (tb + 16 * k) * TOKB);
                        f32x4 acc[NRB];
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const bf16x8 kop = (i < 2) ? fp8x8_to_op((uint32_t)klo[2 * i], (uint32_t)klo[2 * i + 1])
                                                       : fp8x8_to_op((uint32_t)khi[2 * i - 4], (uint32_t)khi[2 * i - 3]);
#pragma unroll
                            for (int rb = 0; rb < NRB; ++rb) acc[rb] = mfma_bf16(kop, qop[rb][i], acc[rb]);
                        }
                        const f32x4 kk = k ? k1 : k0;
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) sv[rb][q][4 * k + i] = acc[rb][i] * kk[i] * qcoef[rb];
                    }
                    if (p0 + 32 > mlim) {
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                            for (int j = 0; j < 8; ++j)
                                sv[rb][q][j] = (p0 + chunk_token(lg, j) < lim[rb]) ? sv[rb][q][j] : -INFINITY;
                    }
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                        for (int j = 0; j < 8; ++j) rmax[rb] = fmaxf(rmax[rb], sv[rb][q][j]);
                }
                ++gs;
            } else {
#pragma unroll
                for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                        for (int j = 0; j < 8; ++j) sv[rb][2 * r + cc][j] = -INFINITY;
            }
        }
        // this half's row maxima; the partner's arrive through LDS by the next barrier
        float mown[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            mown[rb] = wave_max_over_groups(rmax[rb]);
            if (lg == 0) s_max[w][rb * 16 + lr] = mown[rb];
        }

        // ---------------- V pass: steps 5-7, P, its per-tile FP8 codes, P.V -------------------------
#pragma unroll
        for (int r = 0; r < NBLK; ++r) {
            if (r < cur.nvs) {
                step_begin(cur.nvs + r);
                const uint8_t* ring = s_ring[gs % NST];
                if (r == 0) {
                    // step 5a: tile max per row; O <- O * exp2(M_old - m_tile)
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        const float m = fmaxf(mown[rb], s_max[w ^ 1][rb * 16 + lr]);
                        mt_s[rb] = m;
                        // P' = 448 exp2(S - m_tile) = exp2(S + off); a dropped row, or one with no
                        // token in this tile (causal), gets off = -inf
                        const float poff = (m == -INFINITY || M_s[rb] - m > kDropLog2) ? -INFINITY : kLog2_448 - m;
                        // steps 5b-6 for this half of the tile: the FP8 code of P' (the tile's
                        // max maps to 448) and the running sum of the unquantised P'
#pragma unroll
                        for (int q = 0; q < NQ; ++q) {
                            float pv[8];
#pragma unroll
                            for (int j = 0; j < 8; ++j) {
                                pv[j] = __builtin_amdgcn_exp2f(sv[rb][q][j] + poff);
                                lsum[rb] += pv[j];
                            }
                            p8[rb][q][0] = cvt4_fp8(pv[0], pv[1], pv[2], pv[3]);
                            p8[rb][q][1] = cvt4_fp8(pv[4], pv[5], pv[6], pv[7]);
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float mo = __shfl(m, 4 * lg + i, 64);
                            mt_o[rb][i] = mo;
                            const float d = M_o[rb][i] - mo;
                            const float sc = (mo == -INFINITY || d > kDropLog2) ? 1.f : __builtin_amdgcn_exp2f(d);
#pragma unroll
                            for (int cc = 0; cc < 8; ++cc) O[rb][cc][i] *= sc;
                        }
                    }
                }
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const int q = 2 * r + cc;
                    const int tb = 64 * p + 32 * cc;
                    const int p0 = cur.t * T + r * kStepTok + tb;
                    uint32_t xl[8], xh[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint2 x = *reinterpret_cast<const uint2*>(ring + vaddr[j & 3] + (tb + 16 * (j >> 2)) * TOKB);
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
                    for (int rb = 0; rb < NRB; ++rb) pop[rb] = fp8x8_to_op(p8[rb][q][0], p8[rb][q][1]);
#pragma unroll
                    for (int c8 = 0; c8 < 8; ++c8) {
                        const bf16x8 vop = fp8x8_to_op(ylo[c8], yhi[c8]);
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb) O[rb][c8] = mfma_bf16(pop[rb], vop, O[rb][c8]);
                    }
                }
                ++gs;
            }
        }
        // ---- steps 8-9: finish the rescale, update the running state --------------------------
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            // a row with no token in this tile (causal) keeps its state
            if (mt_s[rb] != -INFINITY) {
                const float mn = fmaxf(M_s[rb], mt_s[rb]);
                L_s[rb] = L_s[rb] * __builtin_amdgcn_exp2f(M_s[rb] - mn) + lsum[rb] * __builtin_amdgcn_exp2f(mt_s[rb] - mn);
                M_s[rb] = mn;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float mo = fmaxf(M_o[rb][i], mt_o[rb][i]);
                const float d = M_o[rb][i] - mt_o[rb][i];
                const float sc = (mt_o[rb][i] == -INFINITY || d > kDropLog2) ? 1.f : __builtin_amdgcn_exp2f(mt_o[rb][i] - mo);
                M_o[rb][i] = mo;
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) O[rb][cc][i] *= sc;
            }
        }

        // ---- end of a (batch, group) segment in this workgroup --------------------------------
        const bool seg_end = nxt.nvs == 0 || nxt.v != cur.v;
        const unsigned long long ph_b = seg_end ? PH_NOW() : 0ull;
        if (seg_end) {
            // finished here unless some tile of the sequence lies outside this range
            const bool split = unit_mid(cur, 0) < lo || unit_mid(cur, (cur.seq + T - 1) / T - 1) >= hi;
            // only a range's first and last segments can be split: a split first segment
            // leaves its partial in slot (g, 0), a split last one in (g, 1); the tags name
            // the (batch, group) of each slot (-1: none), written once per call
            const bool first_seg = cur.v == first_v, last_seg = nxt.nvs == 0;
            const int64_t slot_base = (int64_t)(2 * g + (first_seg ? 0 : 1)) * HG + hl;
            if (threadIdx.x == 0) {
                if (first_seg) a.part_tag[2 * g] = split ? cur.v : -1;
                if (last_seg) a.part_tag[2 * g + 1] = (split && !first_seg) ? cur.v : -1;
            }
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                // the two token halves of each head: wave p finishes output columns
                // 8 lr + [4p, 4p + 4) of every row and hands the other four columns of its O,
                // and its L, to its partner (wave p ^ 1) through LDS
                const float Lw = wave_sum_over_groups(L_s[rb]);
                auto handoff = [&](auto P) {
                    constexpr int PH = decltype(P)::value, OT = 4 * (1 - PH);
                    float* dst = &s_comb[hl][PH * 1024];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *reinterpret_cast<f32x4*>(dst + (i * 64 + lane) * 4) =
                            f32x4{O[rb][OT][i], O[rb][OT + 1][i], O[rb][OT + 2][i], O[rb][OT + 3][i]};
                    if (lg == 0) s_comb[hl][2048 + 16 * PH + lr] = Lw;
                };
                if (p == 0) handoff(std::integral_constant<int, 0>{});
                else handoff(std::integral_constant<int, 1>{});
                wait_lgkm();
                barrier_nofence();
                auto finish = [&](auto P) {
                    constexpr int PH = decltype(P)::value, MY = 4 * PH;
                    const float* src = &s_comb[hl][(1 - PH) * 1024];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const f32x4 o = *reinterpret_cast<const f32x4*>(src + (i * 64 + lane) * 4);
#pragma unroll
                        for (int cc = 0; cc < 4; ++cc) O[rb][MY + cc][i] += o[cc];
                    }
                    const float Lt = Lw + s_comb[hl][2048 + 16 * (1 - PH) + lr];
                    const f32x4 vs = *reinterpret_cast<const f32x4*>(&s_vs[vs_buf][hl * kHeadDim + 8 * lr + MY]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = rb * 16 + 4 * lg + i;
                        const float Lr = __shfl(Lt, 4 * lg + i, 64);
                        if (rr >= cur_rows) continue;
                        const int ra = 32 * cur.rk + rr;
                        const int s = small_div(ra, inv_g), gq = ra - s * a.G;
                        const int64_t qrow = ((int64_t)cur.br * a.s1 + s) * a.nq + h * a.G + gq;
                        if (!split) {
                            // step 10: out = O * v_scale / L' (L' = 448 L), bf16
                            const float inv = Lr > 0.f ? 1.f / Lr : 0.f;     // no token at all (causal): zeros
                            const uint32_t pk0 = pack_bf16x2(O[rb][MY][i] * vs[0] * inv, O[rb][MY + 1][i] * vs[1] * inv);
                            const uint32_t pk1 =
                                pack_bf16x2(O[rb][MY + 2][i] * vs[2] * inv, O[rb][MY + 3][i] * vs[3] * inv);
                            *reinterpret_cast<uint2*>(a.out + qrow * kHeadDim + 8 * lr + MY) = uint2{pk0, pk1};
                        } else {
                            float* po = a.part_o + (slot_base * R + rr) * kHeadDim + 8 * lr + MY;
                            *reinterpret_cast<f32x4*>(po) =
                                f32x4{O[rb][MY][i], O[rb][MY + 1][i], O[rb][MY + 2][i], O[rb][MY + 3][i]};
                            if (PH == 0 && lr == 0) {
                                float* pm = a.part_ml + (slot_base * R + rr) * 2;
                                pm[0] = M_o[rb][i];
                                pm[1] = Lr;
                            }
                        }
                    }
                };
                if (p == 0) finish(std::integral_constant<int, 0>{});
                else finish(std::integral_constant<int, 1>{});
                if (NRB > 1) {                        // s_comb is reused by the next row block
                    wait_lgkm();
                    barrier_nofence();
                }
            }
        }

        if (seg_end) ph_end += PH_NOW() - ph_b;
        prev_v = cur.v;
        if (nxt.nvs == 0) break;
        cur = nxt;
        nxt = next_unit(cur);
        nxt_ready = false;
    }
    // the workgroup retires with no load in flight (the last step waited for all of them)
    wait_vm<0>();
    PH_SET(2, PH_NOW());
    PH_SET(3, ph_q);
    PH_SET(4, ph_end);
    PH_SET(5, (unsigned long long)gs);
    PH_SET(6, (unsigned long long)ph_segs);
    PH_SET(7, ph_t7);
}

// Merge of the partials of split (batch, head) pairs: one workgroup per pair, 16
// threads per query row (8 columns each).  The partition is recomputed from what
// the decode kernel published (cost prefix and workgroup count): decode
// workgroup g owns the tiles whose cost midpoints lie in [g C / Geff,
// (g + 1) C / Geff), so the pair's tiles lie in the ranges of the owners g0..g1 of
// its first and last tiles, each holding one segment of it; the slot tags say
// which of a workgroup's two slots holds that segment.
template <int NBLK, int HG>
__global__ __launch_bounds__(512) void merge_rows_kernel(DecodeParams a, int R) {
    const int RBK = a.row_blocks, NG = a.nkv / HG, BV = a.B * RBK * NG;
    const int bh = blockIdx.x, bv = bh / a.nkv, h = bh - bv * a.nkv;   // (virtual batch, head)
    const int b = bv / RBK, rk = bv - b * RBK;
    const int v = bv * NG + h / HG, hl = h - (h / HG) * HG;
    const int* meta = a.rows_meta;
    // independent loads first
    const int64_t C = meta[BV];
    const int Geff = meta[BV + 1];
    const int64_t pv = meta[v];
    int seq = a.seqs[b];
    const int sub = threadIdx.x & 15, d0 = 8 * sub, rr = threadIdx.x >> 4;
    const float* vsp = a.v_scale + ((int64_t)b * a.nkv + h) * kHeadDim + d0;
    const f32x4 vs0 = *reinterpret_cast<const f32x4*>(vsp);
    const f32x4 vs1 = *reinterpret_cast<const f32x4*>(vsp + 4);
    if (C <= 0 || Geff <= 0) return;
    seq = seq < 0 ? 0 : (seq > a.capacity ? a.capacity : seq);
    constexpr int T = NBLK * kStepTok;
    const int nt = (seq + T - 1) / T, nb = (seq + kStepTok - 1) / kStepTok;
    if (nt == 0) return;
    auto mid_of = [&](int t) -> int64_t {
        return pv + (t == 0 ? kSegW / 2 : kSegW) + 2LL * NBLK * t + min(NBLK, nb - t * NBLK);
    };
    auto owner = [&](int64_t x) -> int { return floor_div64((x + 1) * Geff - 1, C); };
    const int g0 = owner(mid_of(0)), g1 = owner(mid_of(nt - 1));
    if (g0 == g1 || rr >= min(32, a.rows - 32 * rk)) return;   // finished in place by the decode kernel
    const int n = g1 - g0 + 1;                 // <= the decode grid (<= 256)
    float Mx = -INFINITY, L = 0.f;
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
    constexpr int SB = 4;                      // segments whose loads are issued together
    for (int i0 = 0; i0 < n; i0 += SB) {
        int k[SB];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int g = min(g0 + i0 + j, g1);
            const int t0 = a.part_tag[2 * g], t1 = a.part_tag[2 * g + 1];
            k[j] = (i0 + j >= n) ? -1 : (t0 == v ? 0 : (t1 == v ? 1 : -1));
        }
        float m[SB], l[SB];
        f32x4 x0[SB], x1[SB];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int g = min(g0 + i0 + j, g1);
            const int64_t slot = ((int64_t)(2 * g + (k[j] > 0 ? 1 : 0)) * HG + hl) * R + rr;
            const float* pm = a.part_ml + slot * 2;
            const float* po = a.part_o + slot * kHeadDim + d0;
            m[j] = k[j] >= 0 ? pm[0] : -INFINITY;
            l[j] = pm[1];
            x0[j] = *reinterpret_cast<const f32x4*>(po);
            x1[j] = *reinterpret_cast<const f32x4*>(po + 4);
        }
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            if (m[j] == -INFINITY) continue;
            // running merge in range order: rescale to the larger maximum
            const float mn = fmaxf(Mx, m[j]);
            const float fa = __builtin_amdgcn_exp2f(Mx - mn), fb = __builtin_amdgcn_exp2f(m[j] - mn);
            L = L * fa + l[j] * fb;
            o0 = o0 * fa + x0[j] * fb;
            o1 = o1 * fa + x1[j] * fb;
            Mx = mn;
        }
    }
    const int ra = 32 * rk + rr;                 // the row among the head's s1 G
    const int sq = small_div(ra, 1.0f / a.G), gq = ra - sq * a.G;
    const int64_t qrow = ((int64_t)b * a.s1 + sq) * a.nq + h * a.G + gq;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float y0 = (c < 2 ? o0[2 * c] : o1[2 * c - 4]) * (c < 2 ? vs0[2 * c] : vs1[2 * c - 4]) * inv;
        const float y1 = (c < 2 ? o0[2 * c + 1] : o1[2 * c - 3]) * (c < 2 ? vs0[2 * c + 1] : vs1[2 * c - 3]) * inv;
        pk[c] = pack_bf16x2(y0, y1);
    }
    *reinterpret_cast<i32x4*>(a.out + qrow * kHeadDim + d0) = i32x4{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
}

// ------------------------------------------------------------------ dispatch

// Heads per workgroup: two when nkv is even (four waves, one per SIMD), else one.
int rows_group(int nkv) { return nkv % 2 == 0 ? 2 : 1; }

template <int NRB, int NBLK, int HG>
static hipError_t launch_rows_t(const DecodeParams& p, int grid, hipStream_t st, bool dbg) {
    if (dbg)
        hipLaunchKernelGGL((decode_rows_kernel<NRB, NBLK, HG, true>), dim3(grid), dim3(2 * HG * 64), 0, st, p);
    else
        hipLaunchKernelGGL((decode_rows_kernel<NRB, NBLK, HG, false>), dim3(grid), dim3(2 * HG * 64), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one workgroup per (batch, head); 16 threads per query row
    hipLaunchKernelGGL((merge_rows_kernel<NBLK, HG>), dim3(p.B * p.row_blocks * p.nkv), dim3(NRB * 256), 0, st, p,
                       NRB * 16);
    return hipGetLastError();
}

template <int HG>
static hipError_t launch_rows_hg(const DecodeParams& p, int grid, hipStream_t st, bool dbg) {
    const bool two = p.row_block > 16;
    switch (p.s2_tile) {
        case 128: return two ? launch_rows_t<2, 1, HG>(p, grid, st, dbg) : launch_rows_t<1, 1, HG>(p, grid, st, dbg);
        case 256: return two ? launch_rows_t<2, 2, HG>(p, grid, st, dbg) : launch_rows_t<1, 2, HG>(p, grid, st, dbg);
        case 512: return two ? launch_rows_t<2, 4, HG>(p, grid, st, dbg) : launch_rows_t<1, 4, HG>(p, grid, st, dbg);
        default: return launch_rows_t<1, 8, HG>(p, grid, st, dbg);
    }
}

// Row blocks per KV head on the whole-row path: one for up to 32 query rows, else
// blocks of 32.
int rows_row_blocks(int rows) { return rows <= 32 ? 1 : (rows + 31) / 32; }

// Shapes of the whole-row path: any nkv; s2_tile 128-1024; up to 32 query rows per
// KV head (16 for s2_tile 1024), or more in blocks of 32 with s2_tile up to 512; at
// most kPrefixMax (batch, head group, row block) units.
bool rows_path_supported(int nkv, int s2_tile, int rows, int s1, int nq, int B) {
    (void)s1;
    (void)nq;
    const int rbk = rows_row_blocks(rows);
    const bool tile_ok = s2_tile == 128 || s2_tile == 256 || s2_tile == 512 ||
                         (s2_tile == 1024 && rows <= 16);
    return tile_ok && rows >= 1 && (int64_t)B * rbk * (nkv / rows_group(nkv)) <= kPrefixMax;
}

hipError_t launch_decode_rows(const DecodeParams& p, int cus, hipStream_t st, bool dbg) {
    // one workgroup per CU (163 KB of LDS with two heads, 87 KB with one): the ranges
    // have equal cost, so every workgroup must be resident at once
    // (at most 256: the merge kernel's table of one sequence's workgroups holds 256)
    const int grid = cus < kRowsMaxGrid ? cus : kRowsMaxGrid;
    if (rows_group(p.nkv) == 2) return launch_rows_hg<2>(p, grid, st, dbg);
    return launch_rows_hg<1>(p, grid, st, dbg);
}

}  // namespace pa
