// FP8 paged GQA decode for MI355X (gfx950, CDNA4, wave64).
//
// Operation: web page "PyPTO 实现 GLM-4.5 Paged Attention FP8 量化算子分页 KV Cache 与
// E4M3 混合精度 Kernel 实战解析" (m.nxbn.cn/news/52221), section 计算流程 steps 1-10,
// section 循环结构 (tiles of s2_tile over the actual length), section 注意事项
// (block table rules).  The page's own loop nest and tiling target another
// machine; this file keeps only the arithmetic.
//
// Work decomposition (one launch):
//   workgroup  = (batch b, split sp, KV head h); NW waves.  With several
//                splits holding work, each writes (O, M, L) partials and the
//                last one to finish (an arrival counter per (b, h) in the
//                workspace, left at zero again) merges them in split order.
//   split sp   = tiles [sp*tps, (sp+1)*tps) of the sequence (s2_tile aligned,
//                so every P-quantisation tile is processed whole).
//   wave w     = tokens [w*TW, (w+1)*TW) of every tile (TW = 64 or 128).
//   chunk      = 32 consecutive tokens (one MFMA K-step of P.V); a chunk never
//                straddles a 128-token block.
// Per tile each wave computes S^T = K . Q^T for its chunks (A = 16 tokens x
// 128 dims of K, loaded straight from HBM with 16-byte loads; B = the query
// rows kept in registers).  The S^T layout leaves every lane with 8 tokens of
// ONE query row, which is exactly the A-operand layout of the P.V product, so
// P never moves between lanes.  The tile's row max is exchanged through LDS
// (one barrier per tile), then P = exp2(S - m_tile) is quantised to FP8
// (448 * P) in registers and multiplied with V.  V rows are channel-contiguous,
// so each lane loads 8-byte pieces of 8 token rows and transposes the 8x8
// bytes in registers with v_perm_b32; the output column of MFMA c is d = 8n + c.
//
// Both products are FP8 x FP8 contractions, but they run on the bf16
// 16x16x32 MFMA with the E4M3 codes decoded exactly to bf16 (one
// v_cvt_scalef32_pk_bf16_fp8 per two codes).  On gfx950 the FP8 MFMAs add
// each group of 8 products in a ~14-bit window aligned to the group's largest
// product and truncate the rest, which biases S by percents when an outlier
// channel dominates a group; the bf16 MFMA accumulates the (exact) products
// in full FP32, matching the FP32-accumulated FP8 matmul of the page.
//
// Numerics: S is kept in the log2 domain (scaled by log2 e) so exp is
// v_exp_f32.  The P-quant scale of a tile is max P / 448 = exp(m_tile - M_new)
// / 448, so the FP8 weights are E4M3(448 * exp(S - m_tile)) and the tile adds
// exp(m_tile - M_new) / 448 * (P8 . V) to the accumulator; v_scale is a
// per-channel constant of (b, h) and is applied once at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_fp8_common.h"
#include "pa_fp8_device.h"

namespace pa {

// Workgroup placement.  Workgroups are dealt round-robin over the 8 XCDs
// (id x runs on XCD x % 8), each XCD with its own L2.  A work unit is a
// (batch b, split sp); its nkv heads get consecutive ids on ONE XCD, so the
// k_scale lines they share ([token][kv head] interleaved) are fetched from
// HBM once.  Units are spread over XCDs by (b + sp) % 8 so every die gets a
// mix of short and long sequences.  The id space is padded (splits to a
// multiple of 8, or batches to a multiple of 8 without splits); padded ids
// are empty.
struct Placement {
    int b, sp, h;
    bool empty;
};

__device__ __forceinline__ Placement place(int x, int B, int nsplit, int nsplit_pad, int nkv) {
    Placement r;
    const int xcd = x & 7, pos = x >> 3;
    r.h = pos % nkv;
    const int q = pos / nkv;
    if (nsplit_pad == 1) {
        r.b = q * 8 + xcd;
        r.sp = 0;
    } else {
        const int per = nsplit_pad >> 3;
        r.b = q / per;
        r.sp = 8 * (q % per) + ((xcd - r.b) & 7);
    }
    r.empty = r.b >= B || r.sp >= nsplit;
    return r;
}

// ------------------------------------------------------------------ kernel

// ------------------------------------------------------------------ kernel

constexpr int kRing = 4;                  // register ring of chunk buffers (3 in flight)

// One prefetched chunk: 16 dwords of K (two 16-token blocks x 32 bytes) or of
// V (8 tokens x 8 bytes), plus the lane's k_scale word for K chunks.
struct Chunk {
    uint32_t w[16];
    float ks;
};

template <int NRB, int NW, int CPW, bool DBG>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NRB == 1 ? 2 : 1)))
void decode_kernel(DecodeParams a) {
    constexpr int TW = CPW * 32;          // tokens per wave per tile
    constexpr int T = NW * TW;            // s2_tile
    constexpr int R = NRB * 16;           // padded query rows per KV head
    constexpr int STEPS = 2 * CPW;        // chunk steps per tile: CPW of K, then CPW of V
    static_assert(STEPS % kRing == 0, "ring must divide the steps of a tile");

    __shared__ float s_max[2][NW][R];     // per-wave row max of a tile (double-buffered by tile parity)
    __shared__ float s_acc[R][kHeadDim];  // cross-wave reduction of O (also the combine's staging)
    __shared__ float s_l[R];
    __shared__ float s_ms[R];
    __shared__ int s_last;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, made scalar
    const int lr = lane & 15;
    const int lg = lane >> 4;

    const Placement pl = place(blockIdx.x, a.B, a.nsplit, a.nsplit_pad, a.nkv);
    if (pl.empty) return;
    const int b = pl.b, sp = pl.sp, h = pl.h;
    // query rows [r0, rend) of KV head h: one block of R rows per blockIdx.y
    const int r0 = (int)blockIdx.y * R, rend = min(r0 + R, a.rows);

    int seq = a.seqs[b];
    seq = seq < 0 ? 0 : (seq > a.capacity ? a.capacity : seq);
    // tokens row r attends to: all of [0, seq), or with causal decode the first
    // seq - s1 + 1 + s of them (s = r / G, its query position)
    auto row_lim = [&](int r) -> int {
        if (!a.causal) return seq;
        const int n = seq - a.s1 + 1 + r / a.G;
        return n < 0 ? 0 : (n > seq ? seq : n);
    };
    const int seq_lo = row_lim(r0), seq_hi = row_lim(rend - 1);   // rows see nondecreasing prefixes
    const int ntiles = (seq_hi + T - 1) / T;
    const int t_begin = sp * a.tiles_per_split;
    const int t_end = min(t_begin + a.tiles_per_split, ntiles);

    if (seq_hi == 0) {
        // nothing to attend to: these rows are zero
        if (sp == 0) {
            for (int e = threadIdx.x; e < (rend - r0) * kHeadDim; e += NW * 64) {
                const int r = r0 + e / kHeadDim, d = e % kHeadDim;
                const int s = r / a.G, gq = r % a.G;
                const int64_t qrow = ((int64_t)b * a.s1 + s) * a.nq + h * a.G + gq;
                a.out[qrow * kHeadDim + d] = 0;
            }
        }
        if (!DBG || sp != 0) return;
    } else if (t_begin >= t_end) {
        return;                           // split beyond this sequence (uniform)
    }

    // ---- step 1: query rows of this KV head -> bf16 operands of exact FP8 values --------
    // lane (lr, lg) holds row rb*16+lr, dims [16lg, 16lg+16) and [64+16lg, 64+16lg+16).
    bf16x8 qop[NRB][4];                   // operand i: codes [8i, 8i+8) of the lane's 32
    float qcoef[NRB];                     // q_scale * softmax_scale * log2 e for row lr
    int lim[NRB];                         // tokens the lane's row attends to
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const int r = r0 + rb * 16 + lr;
        uint32_t wds[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        qcoef[rb] = 0.f;
        lim[rb] = r < rend ? row_lim(r) : 0;
        if (r < rend) {
            const int s = r / a.G, gq = r % a.G;
            const int64_t qrow = ((int64_t)b * a.s1 + s) * a.nq + h * a.G + gq;
            const float qs = a.q_scale[qrow];
            qcoef[rb] = qs * a.softmax_scale * kLog2e;
            const QRecip qd = q_recip(qs);
            const uint16_t* qp = a.q + qrow * kHeadDim;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int d0 = half * 64 + 16 * lg;
                const i32x4 v0 = *reinterpret_cast<const i32x4*>(qp + d0);
                const i32x4 v1 = *reinterpret_cast<const i32x4*>(qp + d0 + 8);
                const uint32_t raw[8] = {(uint32_t)v0[0], (uint32_t)v0[1], (uint32_t)v0[2], (uint32_t)v0[3],
                                         (uint32_t)v1[0], (uint32_t)v1[1], (uint32_t)v1[2], (uint32_t)v1[3]};
                quantise_q16(raw, qd, &wds[half * 4]);
            }
            if (DBG && sp == 0 && w == 0 && a.dbg_q8) {
                uint8_t* dst = a.dbg_q8 + qrow * kHeadDim;
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *reinterpret_cast<uint32_t*>(dst + half * 64 + 16 * lg + 4 * i) = wds[half * 4 + i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) qop[rb][i] = fp8x8_to_op(wds[2 * i], wds[2 * i + 1]);
    }
    if (seq_hi == 0) return;              // debug dump of Q only

    const int64_t tok_stride = (int64_t)a.nkv * kHeadDim;      // bytes between tokens of one head
    const uint8_t* kbase = a.k_cache + (int64_t)h * kHeadDim;
    const uint8_t* vbase = a.v_cache + (int64_t)h * kHeadDim;
    const int32_t* trow = a.block_table + (int64_t)b * a.max_blocks;

    // First physical token row of chunk c of tile t for this wave, or -1 when
    // the chunk holds no valid token.  A chunk never straddles a block.  All
    // of it is wave-uniform (scalar registers).
    auto chunk_slot = [&](int t, int c) -> int64_t {
        const int p0 = t * T + w * TW + 32 * c;
        if (t >= t_end || p0 >= seq_hi) return -1;
        int id = trow[p0 / kBlock];
        id = (id < 0 || id >= a.num_blocks) ? 0 : id;
        return (int64_t)id * kBlock + (p0 % kBlock);
    };
    // Per-lane byte offsets inside a chunk (constant over the loop): K rows
    // 16k + lr at bytes 16lg and 64 + 16lg; V rows chunk_token(lg, j) at byte
    // 8lr; the k_scale word of token chunk_token(lg, lr & 7).
    uint32_t koff[2], voff[8];
#pragma unroll
    for (int k = 0; k < 2; ++k) koff[k] = (uint32_t)((16 * k + lr) * tok_stride + 16 * lg);
#pragma unroll
    for (int j = 0; j < 8; ++j) voff[j] = (uint32_t)(chunk_token(lg, j) * tok_stride + 8 * lr);
    const uint32_t ksoff = (uint32_t)(chunk_token(lg, lr & 7) * a.nkv * 4);
    const uint8_t* ksbase = reinterpret_cast<const uint8_t*>(a.k_scale + h);

    // Issue the loads of step u (static) of tile t into ring slot `ch`.  Chunks
    // without valid tokens load block 0's first rows instead (always in
    // bounds, L2-resident, never used), which keeps the code straight-line.
    auto issue = [&](Chunk& ch, int t, int u) {
        const int c = u < CPW ? u : u - CPW;
        int64_t s0 = chunk_slot(t, c);
        s0 = s0 < 0 ? 0 : s0;
        if (u < CPW) {
            const uint8_t* kb = kbase + s0 * tok_stride;              // uniform base
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const i32x4 lo = *reinterpret_cast<const i32x4*>(kb + koff[k]);
                const i32x4 hi = *reinterpret_cast<const i32x4*>(kb + koff[k] + 64);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ch.w[8 * k + i] = (uint32_t)lo[i];
                    ch.w[8 * k + 4 + i] = (uint32_t)hi[i];
                }
            }
            ch.ks = *reinterpret_cast<const float*>(ksbase + s0 * a.nkv * 4 + ksoff);
        } else {
            const uint8_t* vb = vbase + s0 * tok_stride;              // uniform base
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint2 v = *reinterpret_cast<const uint2*>(vb + voff[j]);
                ch.w[2 * j] = v.x;
                ch.w[2 * j + 1] = v.y;
            }
        }
    };

    // running state; M in the S^T-row layout (row lr) and in the O layout (rows 4lg+i)
    float M_s[NRB], L_s[NRB];
    float M_o[NRB][4];
    f32x4 O[NRB][8];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        M_s[rb] = -INFINITY;
        L_s[rb] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) M_o[rb][i] = -INFINITY;
#pragma unroll
        for (int c = 0; c < 8; ++c) O[rb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    Chunk ring[kRing];
#pragma unroll
    for (int u = 0; u < kRing - 1; ++u) issue(ring[u], t_begin, u);

    for (int t = t_begin; t < t_end; ++t) {
        const int wlo = t * T + w * TW;
        float sv[NRB][CPW][8];
        float rmax[NRB];
        float mt_s[NRB], mt_o[NRB][4];
        float lsum[NRB];
        float poff[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            rmax[rb] = -INFINITY;
            lsum[rb] = 0.f;
        }

#pragma unroll
        for (int u = 0; u < STEPS; ++u) {
            // keep kRing-1 chunks in flight: load step u + kRing - 1 (maybe next tile)
            {
                const int un = u + kRing - 1;
                if (un < STEPS) issue(ring[un % kRing], t, un);
                else issue(ring[un % kRing], t + 1, un - STEPS);
            }
            Chunk& ch = ring[u % kRing];
            const int c = u < CPW ? u : u - CPW;
            const int p0 = wlo + 32 * c;
            const bool valid = p0 < seq_hi;

            if (u < CPW) {
                // ---- steps 2-4: S^T = K Q^T (exact products, FP32 sums), dequantise, mask
                if (valid) {
                    if (DBG && a.dbg_rows && h == 0 && lg == 0) {
                        const int64_t s0 = chunk_slot(t, c);
#pragma unroll
                        for (int k = 0; k < 2; ++k)
                            if (p0 + 16 * k + lr < seq)
                                a.dbg_rows[(int64_t)b * a.capacity + p0 + 16 * k + lr] = (int32_t)(s0 + 16 * k + lr);
                    }
                    float ks[8];
                    ks[0] = row_bcast<0>(ch.ks); ks[1] = row_bcast<1>(ch.ks);
                    ks[2] = row_bcast<2>(ch.ks); ks[3] = row_bcast<3>(ch.ks);
                    ks[4] = row_bcast<4>(ch.ks); ks[5] = row_bcast<5>(ch.ks);
                    ks[6] = row_bcast<6>(ch.ks); ks[7] = row_bcast<7>(ch.ks);
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        bf16x8 kop[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) kop[i] = fp8x8_to_op(ch.w[8 * k + 2 * i], ch.w[8 * k + 2 * i + 1]);
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb) {
                            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc = mfma_bf16(kop[i], qop[rb][i], acc);
#pragma unroll
                            for (int i = 0; i < 4; ++i) sv[rb][c][4 * k + i] = acc[i] * ks[4 * k + i] * qcoef[rb];
                        }
                    }
                    if (p0 + 32 > seq_lo) {
                        // some row's tokens end inside this chunk: mask the tokens past each row's end
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                            for (int j = 0; j < 8; ++j)
                                sv[rb][c][j] = (p0 + chunk_token(lg, j) < lim[rb]) ? sv[rb][c][j] : -INFINITY;
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

                if (u == CPW - 1) {
                    // ---- step 5a: tile max per row across lanes and waves ------------
                    const int par = t & 1;
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        const float m = wave_max_over_groups(rmax[rb]);
                        if (lg == 0) s_max[par][w][rb * 16 + lr] = m;
                    }
                    __syncthreads();
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        float m = -INFINITY;
                        float mo[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
                        for (int ww = 0; ww < NW; ++ww) {
                            m = fmaxf(m, s_max[par][ww][rb * 16 + lr]);
#pragma unroll
                            for (int i = 0; i < 4; ++i) mo[i] = fmaxf(mo[i], s_max[par][ww][rb * 16 + 4 * lg + i]);
                        }
                        mt_s[rb] = m;
                        // exp2 argument offset: P' = 448 * exp2(S - m_tile) = exp2(S + off);
                        // a dropped row, or one with no token in this tile (causal), gets
                        // off = -inf (P' = 0, nothing added)
                        poff[rb] = (m == -INFINITY || M_s[rb] - m > kDropLog2) ? -INFINITY : kLog2_448 - m;
                        // O <- O * exp2(M_old - m_tile): alpha if the tile raises the max,
                        // else 1/beta; the tile's P.V is then added and the sum scaled by beta.
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            mt_o[rb][i] = mo[i];
                            const float d = M_o[rb][i] - mo[i];
                            const float sc = (mo[i] == -INFINITY || d > kDropLog2) ? 1.f : __builtin_amdgcn_exp2f(d);
#pragma unroll
                            for (int cc = 0; cc < 8; ++cc) O[rb][cc][i] *= sc;
                        }
                    }
                }
            } else {
                // ---- steps 5b-7: P, per-tile FP8 quantisation, P.V ----------------------
                if (valid) {
                    uint32_t xl[8], xh[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        xl[j] = ch.w[2 * j];
                        xh[j] = ch.w[2 * j + 1];
                    }
                    if (p0 + 32 > seq_hi) {
                        // tokens past the rows' last one: zero their V bytes (0 * NaN would poison P.V)
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const bool in = p0 + chunk_token(lg, j) < seq_hi;
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
                    for (int rb = 0; rb < NRB; ++rb) {
                        float p[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            p[j] = __builtin_amdgcn_exp2f(sv[rb][c][j] + poff[rb]);
                            lsum[rb] += p[j];
                        }
                        // step 6: FP8 code of 448 * P (the tile's max P maps to 448), held as bf16
                        const uint32_t lo = cvt4_fp8(p[0], p[1], p[2], p[3]);
                        const uint32_t hi = cvt4_fp8(p[4], p[5], p[6], p[7]);
                        pop[rb] = fp8x8_to_op(lo, hi);
                    }
#pragma unroll
                    for (int cc = 0; cc < 8; ++cc) {
                        const bf16x8 vop = fp8x8_to_op(ylo[cc], yhi[cc]);
#pragma unroll
                        for (int rb = 0; rb < NRB; ++rb) O[rb][cc] = mfma_bf16(pop[rb], vop, O[rb][cc]);
                    }
                }

                if (u == STEPS - 1) {
                    // ---- steps 8-9: finish the rescale, update the running state --------
#pragma unroll
                    for (int rb = 0; rb < NRB; ++rb) {
                        // a row with no token in this tile (causal) keeps its state
                        if (mt_s[rb] != -INFINITY) {
                            const float mn = fmaxf(M_s[rb], mt_s[rb]);
                            L_s[rb] = L_s[rb] * __builtin_amdgcn_exp2f(M_s[rb] - mn) +
                                      lsum[rb] * __builtin_amdgcn_exp2f(mt_s[rb] - mn);
                            M_s[rb] = mn;
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float mo = fmaxf(M_o[rb][i], mt_o[rb][i]);
                            const float d = M_o[rb][i] - mt_o[rb][i];
                            const float sc = (mt_o[rb][i] == -INFINITY || d > kDropLog2)
                                                 ? 1.f : __builtin_amdgcn_exp2f(mt_o[rb][i] - mo);
                            M_o[rb][i] = mo;
#pragma unroll
                            for (int cc = 0; cc < 8; ++cc) O[rb][cc][i] *= sc;
                        }
                    }
                }
            }
        }
    }

    // ---- cross-wave reduction (fixed order w = 0, 1, ...) --------------------------------
    float Lw[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) Lw[rb] = wave_sum_over_groups(L_s[rb]);
    for (int ww = 0; ww < NW; ++ww) {
        if (w == ww) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float* dst = &s_acc[rb * 16 + 4 * lg + i][8 * lr];
#pragma unroll
                    for (int cc = 0; cc < 8; ++cc) dst[cc] = (ww == 0) ? O[rb][cc][i] : dst[cc] + O[rb][cc][i];
                }
                if (lg == 0) s_l[rb * 16 + lr] = (ww == 0) ? Lw[rb] : s_l[rb * 16 + lr] + Lw[rb];
            }
        }
        __syncthreads();
    }

    const float* vs = a.v_scale + ((int64_t)b * a.nkv + h) * kHeadDim;
    const int nact = (ntiles + a.tiles_per_split - 1) / a.tiles_per_split;   // splits with work
    const int nrow = rend - r0;
    if (nact == 1) {
        // ---- step 10: out = O * v_scale / L' (L' = 448 L: P' = 448 P is summed), bf16 ----
        // (a row that attends to no token at all, causal, is zero)
        for (int e = threadIdx.x; e < nrow * kHeadDim; e += NW * 64) {
            const int rl = e / kHeadDim, d = e % kHeadDim, r = r0 + rl;
            const int s = r / a.G, gq = r % a.G;
            const int64_t qrow = ((int64_t)b * a.s1 + s) * a.nq + h * a.G + gq;
            const float L = s_l[rl];
            a.out[qrow * kHeadDim + d] = L > 0.f ? f32_to_bf16_rne(s_acc[rl][d] * vs[d] / L) : (uint16_t)0;
        }
        return;
    }

    // ---- split partials, then the last split of the unit merges them -----------------------
    // unit = (b, h, row block); partial layout: [unit][split][R rows][128] for O,
    // [unit][split][R][2] for (M, L)
    const int64_t unit = ((int64_t)b * a.nkv + h) * a.row_blocks + blockIdx.y;
    float* po = a.part_o + (unit * a.nsplit + sp) * (R * kHeadDim);
    float* pml = a.part_ml + (unit * a.nsplit + sp) * (R * 2);
    for (int e = threadIdx.x; e < nrow * kHeadDim; e += NW * 64) po[e] = s_acc[e / kHeadDim][e % kHeadDim];
    if (w == 0 && lg == 0) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            const int r = rb * 16 + lr;
            if (r < nrow) {
                pml[2 * r] = M_s[rb];
                pml[2 * r + 1] = s_l[r];
            }
        }
    }
    __syncthreads();                      // every partial store of this workgroup is done
    if (threadIdx.x == 0) {
        // release our partials, count the arrival (agent scope: splits run on any XCD)
        const int prev = __hip_atomic_fetch_add(a.counters + unit, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == nact - 1);
        if (s_last) __hip_atomic_store(a.counters + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    __atomic_thread_fence(__ATOMIC_ACQUIRE);

    // log-sum-exp merge of the nact partials, in split order (deterministic)
    const float* po0 = a.part_o + (unit * a.nsplit) * (R * kHeadDim);
    const float* pml0 = a.part_ml + (unit * a.nsplit) * (R * 2);
    for (int r = threadIdx.x; r < nrow; r += NW * 64) {
        float Ms = -INFINITY;
        for (int i = 0; i < nact; ++i) Ms = fmaxf(Ms, pml0[i * R * 2 + 2 * r]);
        float L = 0.f;
        if (Ms != -INFINITY)              // a split where the row saw nothing has M = -inf, L = 0
            for (int i = 0; i < nact; ++i)
                L += pml0[i * R * 2 + 2 * r + 1] * __builtin_amdgcn_exp2f(pml0[i * R * 2 + 2 * r] - Ms);
        s_l[r] = L;
        s_ms[r] = Ms;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nrow * kHeadDim; e += NW * 64) {
        const int rl = e / kHeadDim, d = e % kHeadDim, r = r0 + rl;
        const float Ms = s_ms[rl];
        float o = 0.f;
        if (Ms != -INFINITY)
            for (int i = 0; i < nact; ++i)
                o += po0[(int64_t)i * R * kHeadDim + e] * __builtin_amdgcn_exp2f(pml0[i * R * 2 + 2 * rl] - Ms);
        const int s = r / a.G, gq = r % a.G;
        const int64_t qrow = ((int64_t)b * a.s1 + s) * a.nq + h * a.G + gq;
        const float L = s_l[rl];
        a.out[qrow * kHeadDim + d] = L > 0.f ? f32_to_bf16_rne(o * vs[d] / L) : (uint16_t)0;
    }
}

// Fill an int32 buffer (debug dump of gathered rows).
__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// ------------------------------------------------------------------ dispatch

template <int NRB, int NW, int CPW>
static hipError_t launch_nrb(const DecodeParams& p, int grid, hipStream_t st, bool dbg) {
    const dim3 g(grid, p.row_blocks);    // (batch, split, KV head) x blocks of query rows
    if (dbg)
        hipLaunchKernelGGL((decode_kernel<NRB, NW, CPW, true>), g, dim3(NW * 64), 0, st, p);
    else
        hipLaunchKernelGGL((decode_kernel<NRB, NW, CPW, false>), g, dim3(NW * 64), 0, st, p);
    return hipGetLastError();
}

template <int NW, int CPW>
static hipError_t launch_tile(const DecodeParams& p, int nrb, int grid, hipStream_t st, bool dbg) {
    switch (nrb) {
        case 1: return launch_nrb<1, NW, CPW>(p, grid, st, dbg);
        case 2: return launch_nrb<2, NW, CPW>(p, grid, st, dbg);
        case 3: return launch_nrb<3, NW, CPW>(p, grid, st, dbg);
        default: return launch_nrb<4, NW, CPW>(p, grid, st, dbg);
    }
}

hipError_t launch_fill_rows(const DecodeParams& p, hipStream_t st) {
    const int64_t n = (int64_t)p.B * p.capacity;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)), dim3(256),
                       0, st, p.dbg_rows, n, -1);
    return hipGetLastError();
}

int grid_size(const DecodeParams& p) {
    const int bpad = p.nsplit_pad == 1 ? (p.B + 7) / 8 * 8 : p.B;
    return bpad * p.nsplit_pad * p.nkv;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t st, bool dbg) {
    const int nrb = p.row_block / 16;
    const int grid = grid_size(p);
    hipError_t e;
    if (dbg && p.dbg_rows) {
        const int64_t n = (int64_t)p.B * p.capacity;
        hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)),
                           dim3(256), 0, st, p.dbg_rows, n, -1);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    switch (p.s2_tile) {
        case 128: e = launch_tile<2, 2>(p, nrb, grid, st, dbg); break;
        case 256: e = launch_tile<4, 2>(p, nrb, grid, st, dbg); break;
        case 512: e = launch_tile<4, 4>(p, nrb, grid, st, dbg); break;
        case 1024: e = launch_tile<8, 4>(p, nrb, grid, st, dbg); break;
        default: e = launch_tile<16, 4>(p, nrb, grid, st, dbg); break;
    }
    return e;
}

}  // namespace pa
