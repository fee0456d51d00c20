/*
 * CPU oracle for FP8 paged-attention decode — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct C.  Only the test-suite, the smoke check and
 * the benchmark's CPU-baseline leg load this library; the decode library never
 * does.  It shares no code, header, table or constant with the HIP path.
 *
 * Sources:
 * [P1] web page "PyPTO 实现 GLM-4.5 Paged Attention FP8 量化算子分页 KV Cache 与
 *      E4M3 混合精度 Kernel 实战解析" (m.nxbn.cn/news/52221).
 *      - section 计算流程 (computation flow, per batch / s1 / group): the ten
 *        steps Q tile, KV assembly, MM1, dequant, online softmax, P quant,
 *        MM2, dequant, accumulate, final divide + BF16 cast;
 *      - section 循环结构 (loop structure): tiles per sequence =
 *        (cur_seq + s2_tile - 1) // s2_tile; the KV assembly reads
 *        s2_tile / block_size table entries per tile, clamps -1 to 0 and
 *        keeps only the valid tokens of the tile (valid_shape);
 *      - section 量化策略 (quantisation strategy): per-token / per-channel
 *        scales from amax/448, cast to float8_e4m3fn, dequantise with the
 *        reciprocal;
 *      - section 关键特性 (key features): E4M3 range [-448, 448], FP32
 *        softmax state.
 * [P5] web page on ops-transformer's scatter_pa_kv_cache_with_k_scale
 *      (www.lmnt.cn/news/278797).
 *      - section 功能说明与计算公式: per token i and head j, block = slot / block_size,
 *        offset = slot % block_size; the key, value and key-scale rows of (i, j)
 *        go to that (block, head, offset) of the three caches, in place;
 *      - section 约束说明 and the SIMT kernel paragraph: slots below 0 or above
 *        num_blocks * block_size - 1 are skipped; repeated slots are the
 *        caller's error (no result is promised).
 * [P3] web page "CANN ops-transformer aclnnKvCompressEpilog 算子详解"
 *      (www.lmnt.cn/news/267091).
 *      - section 功能说明 (semantics): bf16 rows x [tokens, d] are quantised and
 *        written in place to the cache row of their slot; slot -1 skips the
 *        token; the last 64 columns are the rope part, the first d - 64 the
 *        nope part; quant modes 0 (FP8 groups, bf16 scale) and 1 (FP8 groups,
 *        e8m0 power-of-two scale, roundScale rounds the scale up to a power
 *        of two);
 *      - section 计算公式: scale_g = max|x_g| / 448, q = round(x / scale_g);
 *      - section 约束说明 and the kvCacheCol walkthrough: row layout
 *        [rope bf16, 128 B][nope e4m3, d - 64 B][one scale per 64 columns,
 *        2 B (mode 0) or 1 B (mode 1)]; the cache row must hold kvCacheCol
 *        bytes (mode 1: the written bytes; mode 0: rounded up to 32).
 * [P2] web page "PyPTO-Gym 算子实战DeepSeek V32 MLA 的 Sparse Attention FP8 反量化
 *      算子" (www.mhpn.cn/news/2272720).
 *      - section 核心参数与 KV Cache 布局: 672-byte row = 512 e4m3 nope,
 *        64 bf16 rope (bytes 512..639), 4 fp32 group scales (640..655);
 *      - section 计算流程 (5 层嵌套循环): gather via top-k + block_table,
 *        dequant per 128-group to bf16, K = [nope | rope], Q = [qn | qr],
 *        V = the dequantised nope, softmax, cast P to bf16, P·V;
 *      - section 关键实现细节: valid count
 *        clamp(cur_act_seq - s1 + 1 + s, 0, topk);
 *      - section 在线反量化与 Online Softmax: fp8 -> fp32, times the group
 *        scale, -> bf16; first tile assigns, later tiles rescale old state
 *        by exp(max_old - max_new) and new by exp(m_tile - max_new), the last
 *        divides by the sum.
 *
 * Precision: FP64 throughout, except where the pages fix the precision of a
 * step that decides an integer code: the value cast to FP8 is an FP32 value
 * (P1 dtype table "FP32 -> FP8 E4M3"), and the MLA dequantised key is the
 * FP32 product cast to BF16 (P2).  Those values are rounded to FP32 first.
 *
 * Readings where the pages are silent (each stated where it is used):
 *  R-q   Q arrives as bf16 with a given dequant scale qs; code = E4M3(fp32(q/qs)).
 *  R-sat E4M3 rounding is round-to-nearest-even; magnitudes above 448 saturate
 *        to 448; the sign of zero is kept; no NaN is ever produced from a
 *        finite input.
 *  R-0   qs == 0 (an all-zero query row) gives all-zero codes.
 *  R-ids table entries < 0 or >= num_blocks read physical block 0 (page: -1
 *        is clamped to 0); only table entries that cover [0, seq) are read.
 *  R-seq seq is clamped to [0, max_blocks_per_seq * block_size]; seq == 0
 *        gives an all-zero output row.
 *  R-p   P quant: a = max P over the tile's valid tokens, ps = a / 448,
 *        code = E4M3(fp32(P / ps)); the running sum uses unquantised P.
 *  R-g   query head qh = h * G + g serves KV head h (contiguous groups).
 *  R-s1  every one of the s1 query positions attends to all of [0, seq),
 *        unless the causal variant is asked for (R-causal).
 *  R-causal causal multi-token decode: query position s of s1 attends to the
 *        first n_s = clamp(seq - s1 + 1 + s, 0, seq) tokens -- [P2]'s valid
 *        count with the sequence in place of topk (section 关键实现细节) --
 *        with its own tiles over [0, n_s) (n_s = 0 gives a zero row).
 *  R-lay the cache writer serves two layouts: BSND [block, offset, head, d]
 *        with scales [block, offset, head] -- [P1]'s layout, the one the
 *        decode reads -- and BNBD [block, head, offset, d] with scales
 *        [block, head, offset] -- [P5]'s documented layout.
 *  R-dup with a repeated slot the later token wins here (tests never repeat).
 *  R-ep-grp  in modes 0 / 1 a group is 64 nope columns whatever quantGroupSize
 *        says ([P3]'s row-size formula counts ceil((d - 64) / 64) scales;
 *        quantGroupSize governs mode 2).
 *  R-ep-scale scale = fp32(amax / 448).  Mode 0 stores bf16(scale) (RNE) and
 *        divides by the stored bf16 value; mode 1 stores 2^k as e8m0 (code
 *        k + 127, k clamped to [-127, 127]) with k = ceil(log2 scale) when
 *        roundScale, else floor(log2 scale), and divides by 2^k.  The
 *        quotient is an fp32 division; codes are E4M3 RNE saturating at 448.
 *  R-ep-zero an all-zero group (or a stored mode-0 scale of 0) gives zero
 *        codes; its stored scale is bf16 0 (mode 0) or e8m0 code 0 (mode 1).
 *  R-ep-pad  bytes of a cache row past the written ones are left untouched.
 *  R-ep-slot slots < 0 or >= blockNum * blockSize are skipped.
 *  R-mla-nkv [P2]'s signature gives topk_indices the shape (t, n_kv*topk) and
 *        its loops run over KV heads, then the query group of each, while the
 *        latent cache has one row per token slot: KV head h reads the shared
 *        rows through its own slice [h*topk, (h+1)*topk), and query head hq
 *        belongs to KV head hq / (nq / n_kv).
 *  R-mla-pos a top-k position outside [0, seq) among the first n is clamped
 *        into it (the table rule applied to positions; the page promises
 *        in-range indices and says nothing of others).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_E4M3_MAX 448.0

/* ---------------------------------------------------------------- codecs */

/* OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities, S.1111.111 is NaN; subnormals m * 2^-9. */
double oracle_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* Round x to the nearest E4M3 value, ties to even, saturating at +-448.
 * x is finite.  Sign of zero kept. */
uint8_t oracle_e4m3_encode(double x)
{
    int s = signbit(x) ? 1 : 0;
    double a = fabs(x);
    int code;
    if (isnan(x))
        return 0x7F;
    if (a >= OR_E4M3_MAX) {
        code = 0x7E;                       /* 1.1111.110 = 448 */
    } else if (a < ldexp(1.0, -6)) {       /* subnormal range, quantum 2^-9 */
        double n = nearbyint(a * 512.0);   /* exact scaling, RNE */
        code = (int)n;                     /* n == 8 is the smallest normal, code 8 */
    } else {
        int e2;
        frexp(a, &e2);                     /* a = f * 2^e2, f in [0.5, 1) */
        int e = e2 - 1;                    /* a in [2^e, 2^(e+1)) */
        double n = nearbyint(ldexp(a, 3 - e));     /* in [8, 16] */
        code = (e + 7) * 8 + (int)n - 8;   /* n == 16 carries into the exponent */
        if (code > 0x7E)
            code = 0x7E;
    }
    return (uint8_t)(code | (s << 7));
}

double oracle_bf16_decode(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round to the nearest bf16, ties to even.  Done in two exact steps: x is
 * split at the bf16 quantum of its binade, like any RNE to p = 8 bits. */
uint16_t oracle_bf16_encode(double x)
{
    if (isnan(x))
        return 0x7FC0;
    int s = signbit(x) ? 1 : 0;
    double a = fabs(x);
    uint16_t r;
    if (a == 0.0) {
        r = 0;
    } else {
        int e2;
        frexp(a, &e2);
        int e = e2 - 1;                    /* a in [2^e, 2^(e+1)) */
        if (e < -126) e = -126;            /* bf16 subnormals share the min quantum */
        double n = nearbyint(ldexp(a, 7 - e));     /* mantissa with 7 fraction bits */
        double v = ldexp(n, e - 7);
        if (v >= ldexp(1.0, 128)) {
            r = 0x7F80;                    /* overflow to infinity */
        } else {
            float f = (float)v;            /* exact: v has <= 8 significant bits */
            uint32_t u;
            memcpy(&u, &f, 4);
            r = (uint16_t)(u >> 16);
        }
    }
    return (uint16_t)(r | (s << 15));
}

static double round_to_fp32(double x) { return (double)(float)x; }

/* ------------------------------------------------------ GQA paged decode */

static int clamp_seq(int seq, int cap)
{
    if (seq < 0) return 0;
    if (seq > cap) return cap;
    return seq;
}

/* Tokens query position s attends to (R-s1, R-causal). */
static int row_seq(int seq, int s1, int s, int causal)
{
    if (!causal) return seq;
    int n = seq - s1 + 1 + s;
    return n < 0 ? 0 : (n > seq ? seq : n);
}

/* Physical slot of logical token p of batch b ([P1] KV assembly, R-ids). */
static int64_t gqa_slot(const int32_t* block_table, int max_blocks, int block_size,
                        int num_blocks, int b, int p)
{
    int id = block_table[(int64_t)b * max_blocks + p / block_size];
    if (id < 0 || id >= num_blocks)
        id = 0;
    return (int64_t)id * block_size + p % block_size;
}

/*
 * One query row: batch b, query position s, KV head h, group member g.
 * Writes out_row[D] (FP64 O/L), and returns L and M through pointers.
 * Scratch: S, P sized >= s2_tile; q8 sized >= D; O, Oraw sized >= D.
 */
static void gqa_row(const uint16_t* q_bf16, const float* q_scale,
                    const uint8_t* k8, const float* k_scale,
                    const uint8_t* v8, const float* v_scale,
                    const int32_t* block_table,
                    int b, int s, int h, int g, int seq,
                    int s1, int nq, int nkv, int D, int block_size,
                    double softmax_scale, int s2_tile, int max_blocks, int num_blocks,
                    double* out_row, uint8_t* q8_row, double* M_out, double* L_out,
                    double* S, double* P, uint8_t* P8, double* O, double* Oraw)
{
    const int G = nq / nkv;
    const int qh = h * G + g;                                   /* R-g */
    const int64_t qrow = ((int64_t)b * s1 + s) * nq + qh;
    const double qs = (double)q_scale[qrow];
    int d;

    /* Step 1: Q tile in FP8 with its scale (R-q, R-0). */
    for (d = 0; d < D; ++d) {
        double q = oracle_bf16_decode(q_bf16[qrow * D + d]);
        if (qs == 0.0)
            q8_row[d] = 0;
        else
            q8_row[d] = oracle_e4m3_encode(round_to_fp32((double)((float)q / (float)qs)));
    }

    double M = -INFINITY, L = 0.0;
    for (d = 0; d < D; ++d) O[d] = 0.0;

    const int ntiles = (seq + s2_tile - 1) / s2_tile;          /* [P1] loop structure */
    for (int t = 0; t < ntiles; ++t) {
        const int lo = t * s2_tile;
        const int hi = (lo + s2_tile < seq) ? lo + s2_tile : seq;   /* valid_shape crop */
        const int n = hi - lo;

        /* Steps 2-4: assemble K rows through the table, MM1 (exact in FP64),
         * dequantise with q_scale * k_scale, then the softmax scale. */
        for (int i = 0; i < n; ++i) {
            int64_t slot = gqa_slot(block_table, max_blocks, block_size, num_blocks, b, lo + i);
            const uint8_t* krow = k8 + (slot * nkv + h) * D;
            double acc = 0.0;
            for (d = 0; d < D; ++d)
                acc += oracle_e4m3_decode(q8_row[d]) * oracle_e4m3_decode(krow[d]);
            S[i] = acc * qs * (double)k_scale[slot * nkv + h] * softmax_scale;
        }

        /* Step 5: online softmax update. */
        double m_t = -INFINITY;
        for (int i = 0; i < n; ++i)
            if (S[i] > m_t) m_t = S[i];
        const double M_new = (M > m_t) ? M : m_t;
        const double alpha = exp(M - M_new);                    /* exp(-inf) = 0 on the first tile */
        double sumP = 0.0;
        for (int i = 0; i < n; ++i) {
            P[i] = exp(S[i] - M_new);
            sumP += P[i];
        }
        L = L * alpha + sumP;

        /* Step 6: P quantised per row over this tile (R-p). */
        double a = 0.0;
        for (int i = 0; i < n; ++i)
            if (P[i] > a) a = P[i];
        const double ps = a / OR_E4M3_MAX;
        for (int i = 0; i < n; ++i)
            P8[i] = (ps == 0.0) ? 0 : oracle_e4m3_encode(round_to_fp32(P[i] / ps));

        /* Step 7: MM2 over the tile's V rows (exact in FP64). */
        for (d = 0; d < D; ++d) Oraw[d] = 0.0;
        for (int i = 0; i < n; ++i) {
            int64_t slot = gqa_slot(block_table, max_blocks, block_size, num_blocks, b, lo + i);
            const uint8_t* vrow = v8 + (slot * nkv + h) * D;
            double p = oracle_e4m3_decode(P8[i]);
            for (d = 0; d < D; ++d)
                Oraw[d] += p * oracle_e4m3_decode(vrow[d]);
        }

        /* Steps 8-9: dequantise with P_scale * V_scale, rescale and add. */
        const float* vs = v_scale + ((int64_t)b * nkv + h) * D;
        for (d = 0; d < D; ++d)
            O[d] = O[d] * alpha + Oraw[d] * ps * (double)vs[d];
        M = M_new;
    }

    /* Step 10: final divide (R-seq: an empty sequence gives zeros). */
    for (d = 0; d < D; ++d)
        out_row[d] = (seq == 0) ? 0.0 : O[d] / L;
    *M_out = M;
    *L_out = L;
}

/*
 * Decode batches [b_lo, b_hi) (causal != 0: R-causal).  Layouts (all dense, row-major):
 *   q_bf16      [B*s1, nq, D]              bf16 bit patterns
 *   q_scale     [B*s1, nq]
 *   k8, v8      [num_blocks, block_size, nkv, D]  E4M3 codes
 *   k_scale     [num_blocks, block_size, nkv]
 *   v_scale     [B, nkv, D]
 *   block_table [B, max_blocks]
 *   seqs        [B]
 * Outputs (rows of batches outside [b_lo, b_hi) untouched):
 *   out_f64     [B*s1, nq, D]  O / L in FP64
 *   out_bf16    [B*s1, nq, D]  bf16 RNE of out_f64            (may be NULL)
 *   q8_out      [B*s1, nq, D]  the FP8 query codes            (may be NULL)
 *   M_out,L_out [B*s1, nq]     final running max / sum        (may be NULL)
 *   rows_out    [B, max_blocks*block_size] physical slot read for each
 *               logical token p < seq, -1 for p >= seq       (may be NULL)
 * Returns 0, or -1 on an invalid shape.
 */
int oracle_pa_fp8_decode(const uint16_t* q_bf16, const float* q_scale,
                         const uint8_t* k8, const float* k_scale,
                         const uint8_t* v8, const float* v_scale,
                         const int32_t* block_table, const int32_t* seqs,
                         int B, int s1, int nq, int nkv, int D, int block_size,
                         double softmax_scale, int s2_tile, int max_blocks, int num_blocks,
                         int causal, int b_lo, int b_hi,
                         double* out_f64, uint16_t* out_bf16, uint8_t* q8_out,
                         double* M_out, double* L_out, int32_t* rows_out)
{
    if (B <= 0 || s1 <= 0 || nq <= 0 || nkv <= 0 || D <= 0 || block_size <= 0 ||
        s2_tile <= 0 || max_blocks <= 0 || num_blocks <= 0 || nq % nkv != 0 ||
        b_lo < 0 || b_hi > B || b_lo > b_hi)
        return -1;
    const int G = nq / nkv;
    double* S = malloc(sizeof(double) * s2_tile);
    double* P = malloc(sizeof(double) * s2_tile);
    uint8_t* P8 = malloc(s2_tile);
    double* O = malloc(sizeof(double) * D);
    double* Oraw = malloc(sizeof(double) * D);
    uint8_t* q8 = malloc(D);
    if (!S || !P || !P8 || !O || !Oraw || !q8) {
        free(S); free(P); free(P8); free(O); free(Oraw); free(q8);
        return -2;
    }
    for (int b = b_lo; b < b_hi; ++b) {
        const int seq = clamp_seq(seqs[b], max_blocks * block_size);
        if (rows_out) {
            for (int p = 0; p < max_blocks * block_size; ++p)
                rows_out[(int64_t)b * max_blocks * block_size + p] =
                    p < seq ? (int32_t)gqa_slot(block_table, max_blocks, block_size, num_blocks, b, p) : -1;
        }
        for (int s = 0; s < s1; ++s)
            for (int h = 0; h < nkv; ++h)
                for (int g = 0; g < G; ++g) {
                    const int64_t qrow = ((int64_t)b * s1 + s) * nq + h * G + g;
                    double M, L;
                    gqa_row(q_bf16, q_scale, k8, k_scale, v8, v_scale, block_table,
                            b, s, h, g, row_seq(seq, s1, s, causal), s1, nq, nkv, D, block_size, softmax_scale,
                            s2_tile, max_blocks, num_blocks,
                            out_f64 + qrow * D, q8, &M, &L, S, P, P8, O, Oraw);
                    if (q8_out) memcpy(q8_out + qrow * D, q8, D);
                    if (out_bf16)
                        for (int d = 0; d < D; ++d)
                            out_bf16[qrow * D + d] = oracle_bf16_encode(out_f64[qrow * D + d]);
                    if (M_out) M_out[qrow] = M;
                    if (L_out) L_out[qrow] = L;
                }
    }
    free(S); free(P); free(P8); free(O); free(Oraw); free(q8);
    return 0;
}

/*
 * Same as oracle_pa_fp8_decode but only for the listed query rows
 * (row = (b*s1 + s)*nq + qh); used to spot-check full-size workloads.
 * out_f64 / out_bf16 are [nrows, D] in list order; M_out/L_out [nrows].
 */
int oracle_pa_fp8_decode_rows(const uint16_t* q_bf16, const float* q_scale,
                              const uint8_t* k8, const float* k_scale,
                              const uint8_t* v8, const float* v_scale,
                              const int32_t* block_table, const int32_t* seqs,
                              int B, int s1, int nq, int nkv, int D, int block_size,
                              double softmax_scale, int s2_tile, int max_blocks, int num_blocks,
                              int causal, const int64_t* rows, int nrows,
                              double* out_f64, uint16_t* out_bf16, double* M_out, double* L_out)
{
    if (B <= 0 || s1 <= 0 || nq <= 0 || nkv <= 0 || D <= 0 || block_size <= 0 ||
        s2_tile <= 0 || max_blocks <= 0 || num_blocks <= 0 || nq % nkv != 0 || nrows < 0)
        return -1;
    const int G = nq / nkv;
    double* S = malloc(sizeof(double) * s2_tile);
    double* P = malloc(sizeof(double) * s2_tile);
    uint8_t* P8 = malloc(s2_tile);
    double* O = malloc(sizeof(double) * D);
    double* Oraw = malloc(sizeof(double) * D);
    uint8_t* q8 = malloc(D);
    if (!S || !P || !P8 || !O || !Oraw || !q8) {
        free(S); free(P); free(P8); free(O); free(Oraw); free(q8);
        return -2;
    }
    int rc = 0;
    for (int i = 0; i < nrows; ++i) {
        const int64_t r = rows[i];
        if (r < 0 || r >= (int64_t)B * s1 * nq) { rc = -1; break; }
        const int b = (int)(r / ((int64_t)s1 * nq));
        const int s = (int)((r / nq) % s1);
        const int qh = (int)(r % nq);
        const int seq = clamp_seq(seqs[b], max_blocks * block_size);
        double M, L;
        gqa_row(q_bf16, q_scale, k8, k_scale, v8, v_scale, block_table,
                b, s, qh / G, qh % G, row_seq(seq, s1, s, causal), s1, nq, nkv, D, block_size, softmax_scale,
                s2_tile, max_blocks, num_blocks,
                out_f64 + (int64_t)i * D, q8, &M, &L, S, P, P8, O, Oraw);
        if (out_bf16)
            for (int d = 0; d < D; ++d)
                out_bf16[(int64_t)i * D + d] = oracle_bf16_encode(out_f64[(int64_t)i * D + d]);
        if (M_out) M_out[i] = M;
        if (L_out) L_out[i] = L;
    }
    free(S); free(P); free(P8); free(O); free(Oraw); free(q8);
    return rc;
}

/* ------------------------------------------------ MLA sparse decode ([P2]) */

#define OR_MLA_ROW 672
#define OR_MLA_NOPE 512
#define OR_MLA_ROPE 64
#define OR_MLA_GROUP 128

/*
 * Dequantise one gathered cache row into K = [kn | kr] (576 values, each a
 * bf16 value held in a double).  kn[c] = bf16(fp32(dec(code[c]) * scale[c/128])).
 */
void oracle_mla_dequant_row(const uint8_t* row, double* kvec)
{
    float scale[4];
    memcpy(scale, row + 640, 16);
    for (int c = 0; c < OR_MLA_NOPE; ++c) {
        float prod = (float)oracle_e4m3_decode(row[c]) * scale[c / OR_MLA_GROUP];
        kvec[c] = oracle_bf16_decode(oracle_bf16_encode((double)prod));
    }
    for (int c = 0; c < OR_MLA_ROPE; ++c) {
        uint16_t hbits;
        memcpy(&hbits, row + OR_MLA_NOPE + 2 * c, 2);
        kvec[OR_MLA_NOPE + c] = oracle_bf16_decode(hbits);
    }
}

/*
 * Decode batches [b_lo, b_hi) of the MLA-style sparse attention.
 *   q_nope [B*s1*nq, 512] bf16, q_rope [B*s1*nq, 64] bf16
 *   cache  [num_blocks*block_size, 672] bytes
 *   topk   [B*s1, nkv*topk] logical token ids: KV head h's slice is
 *          [h*topk, (h+1)*topk) ([P2] API 签名: topk_indices (t, n_kv*topk));
 *          the first n of each slice are used
 *   block_table [B, max_blocks], seqs [B]
 * Outputs: out_f64 [B*s1*nq, 512], out_bf16 (may be NULL).
 * Per query position s of batch b: n = clamp(seq - s1 + 1 + s, 0, topk).
 * Query head hq belongs to KV head hq / (nq / nkv) ([P2] loops: KV head, then
 * the query group of that head); every KV head reads the same latent rows,
 * through its own top-k slice (reading R-mla-nkv).
 * Tiles of s2_tile index positions; P = exp(S - m_tile) cast to bf16 feeds
 * P.V, the unquantised P feeds the sum (readings stated in the header).
 */
int oracle_mla_sparse_decode(const uint16_t* q_nope, const uint16_t* q_rope,
                             const uint8_t* cache, const int32_t* topk_idx,
                             const int32_t* block_table, const int32_t* seqs,
                             int B, int s1, int nq, int nkv, int topk, int block_size,
                             int max_blocks, int num_blocks, double softmax_scale, int s2_tile,
                             int b_lo, int b_hi, double* out_f64, uint16_t* out_bf16)
{
    const int DK = OR_MLA_NOPE + OR_MLA_ROPE, DV = OR_MLA_NOPE;
    if (B <= 0 || s1 <= 0 || nq <= 0 || nkv <= 0 || nq % nkv != 0 || topk <= 0 || block_size <= 0 ||
        max_blocks <= 0 || num_blocks <= 0 || s2_tile <= 0 || b_lo < 0 || b_hi > B || b_lo > b_hi)
        return -1;
    const int G = nq / nkv;
    double* K = malloc(sizeof(double) * (size_t)topk * DK);
    double* S = malloc(sizeof(double) * s2_tile);
    double* P = malloc(sizeof(double) * s2_tile);
    double* O = malloc(sizeof(double) * DV);
    double* Ot = malloc(sizeof(double) * DV);
    double* qv = malloc(sizeof(double) * DK);
    if (!K || !S || !P || !O || !Ot || !qv) {
        free(K); free(S); free(P); free(O); free(Ot); free(qv);
        return -2;
    }
    for (int b = b_lo; b < b_hi; ++b) {
        int seq = clamp_seq(seqs[b], max_blocks * block_size);
        for (int s = 0; s < s1; ++s) {
            int n = seq - s1 + 1 + s;
            if (n < 0) n = 0;
            if (n > topk) n = topk;
            for (int h = 0; h < nkv; ++h) {
            const int32_t* idx = topk_idx + (((int64_t)b * s1 + s) * nkv + h) * topk;
            /* Gather + dequantise the n selected rows once per (query token, KV head). */
            for (int j = 0; j < n; ++j) {
                int p = idx[j];
                if (p < 0) p = 0;                              /* R-mla-pos */
                if (p >= seq) p = seq - 1;
                int id = block_table[(int64_t)b * max_blocks + p / block_size];
                if (id < 0 || id >= num_blocks) id = 0;
                const uint8_t* row = cache + ((int64_t)id * block_size + p % block_size) * OR_MLA_ROW;
                oracle_mla_dequant_row(row, K + (int64_t)j * DK);
            }
            for (int hq = h * G; hq < (h + 1) * G; ++hq) {
                const int64_t qrow = ((int64_t)b * s1 + s) * nq + hq;
                for (int c = 0; c < OR_MLA_NOPE; ++c) qv[c] = oracle_bf16_decode(q_nope[qrow * OR_MLA_NOPE + c]);
                for (int c = 0; c < OR_MLA_ROPE; ++c) qv[OR_MLA_NOPE + c] = oracle_bf16_decode(q_rope[qrow * OR_MLA_ROPE + c]);
                double M = -INFINITY, L = 0.0;
                for (int c = 0; c < DV; ++c) O[c] = 0.0;
                const int ntiles = (n + s2_tile - 1) / s2_tile;
                for (int t = 0; t < ntiles; ++t) {
                    const int lo = t * s2_tile, hi = (lo + s2_tile < n) ? lo + s2_tile : n;
                    double m_t = -INFINITY;
                    for (int j = lo; j < hi; ++j) {
                        double acc = 0.0;
                        for (int c = 0; c < DK; ++c) acc += qv[c] * K[(int64_t)j * DK + c];
                        S[j - lo] = acc * softmax_scale;
                        if (S[j - lo] > m_t) m_t = S[j - lo];
                    }
                    double l_t = 0.0;
                    for (int c = 0; c < DV; ++c) Ot[c] = 0.0;
                    for (int j = lo; j < hi; ++j) {
                        P[j - lo] = exp(S[j - lo] - m_t);
                        l_t += P[j - lo];
                        double pb = oracle_bf16_decode(oracle_bf16_encode(round_to_fp32(P[j - lo])));
                        for (int c = 0; c < DV; ++c) Ot[c] += pb * K[(int64_t)j * DK + c];
                    }
                    const double M_new = (M > m_t) ? M : m_t;
                    const double a_old = exp(M - M_new), a_new = exp(m_t - M_new);
                    for (int c = 0; c < DV; ++c) O[c] = O[c] * a_old + Ot[c] * a_new;
                    L = L * a_old + l_t * a_new;
                    M = M_new;
                }
                for (int c = 0; c < DV; ++c) {
                    double v = (n == 0) ? 0.0 : O[c] / L;
                    out_f64[qrow * DV + c] = v;
                    if (out_bf16) out_bf16[qrow * DV + c] = oracle_bf16_encode(v);
                }
            }
            }
        }
    }
    free(K); free(S); free(P); free(O); free(Ot); free(qv);
    return 0;
}

/* ------------------------------------------------- [P5] FP8 KV-cache writer */

/*
 * In-place scatter of one step's FP8 key / value rows and per-(token, head)
 * key scales into the paged caches ([P5] 功能说明与计算公式).
 *   key   token i, head j, byte d at key[i * key_token_stride + j * k_head_size + d]
 *   value likewise with value_token_stride and v_head_size
 *   key_scale (i, j) at key_scale[i * ks_token_stride + j * ks_head_stride]
 *   slots [num_tokens] (int64 here; the caller widens int32 slots)
 * layout 0 (BSND): key_cache[((block * block_size + offset) * num_head + j) * k_head_size + d],
 *                  key_scale_cache[(block * block_size + offset) * num_head + j];
 * layout 1 (BNBD): key_cache[((block * num_head + j) * block_size + offset) * k_head_size + d],
 *                  key_scale_cache[(block * num_head + j) * block_size + offset].
 * Tokens whose slot lies outside [0, num_blocks * block_size) are skipped.
 * Returns the number of tokens written, or -1 on a bad argument.
 */
int oracle_scatter_kv_cache(const uint8_t* key, const uint8_t* value,
                            uint8_t* key_cache, uint8_t* value_cache,
                            const int64_t* slots, const float* key_scale, float* key_scale_cache,
                            int num_tokens, int num_head, int k_head_size, int v_head_size,
                            int num_blocks, int block_size, int layout,
                            int64_t key_token_stride, int64_t value_token_stride,
                            int64_t ks_token_stride, int64_t ks_head_stride)
{
    if (num_tokens < 0 || num_head <= 0 || k_head_size <= 0 || v_head_size <= 0 ||
        num_blocks <= 0 || block_size <= 0 || (layout != 0 && layout != 1))
        return -1;
    const int64_t num_slots = (int64_t)num_blocks * block_size;
    int written = 0;
    for (int i = 0; i < num_tokens; ++i) {
        const int64_t slot = slots[i];
        if (slot < 0 || slot > num_slots - 1)
            continue;
        const int64_t block = slot / block_size, offset = slot % block_size;
        for (int j = 0; j < num_head; ++j) {
            int64_t kpos, vpos, spos;
            if (layout == 0) {
                kpos = ((block * block_size + offset) * num_head + j) * k_head_size;
                vpos = ((block * block_size + offset) * num_head + j) * v_head_size;
                spos = (block * block_size + offset) * num_head + j;
            } else {
                kpos = ((block * num_head + j) * block_size + offset) * k_head_size;
                vpos = ((block * num_head + j) * block_size + offset) * v_head_size;
                spos = (block * num_head + j) * block_size + offset;
            }
            for (int d = 0; d < k_head_size; ++d)
                key_cache[kpos + d] = key[(int64_t)i * key_token_stride + (int64_t)j * k_head_size + d];
            for (int d = 0; d < v_head_size; ++d)
                value_cache[vpos + d] = value[(int64_t)i * value_token_stride + (int64_t)j * v_head_size + d];
            key_scale_cache[spos] = key_scale[(int64_t)i * ks_token_stride + (int64_t)j * ks_head_stride];
        }
        ++written;
    }
    return written;
}

/* --------------------------------------------- [P3] KvCompressEpilog modes 0/1 */

/* Bytes written per token (the page's concatCol): rope 128 B, d - 64 FP8
 * codes, one scale per 64 nope columns (2 B in mode 0, 1 B in mode 1). */
int oracle_kv_compress_row_bytes(int d, int mode)
{
    if (d <= 64 || (mode != 0 && mode != 1))
        return -1;
    const int groups = (d - 64 + 63) / 64;
    return (d - 64) + 128 + groups * (mode == 0 ? 2 : 1);
}

/* Minimum cache row (kvCacheCol): mode 1 as written, mode 0 rounded up to 32. */
int oracle_kv_compress_cache_col(int d, int mode)
{
    int c = oracle_kv_compress_row_bytes(d, mode);
    if (c < 0)
        return -1;
    return mode == 1 ? c : (c + 31) / 32 * 32;
}

/*
 * In-place quantising scatter of bf16 rows x [num_tokens, d] (R-ep-*):
 * token t with slot s in [0, block_num * block_size) writes row
 * cache + (s / block_size) * block_stride + (s % block_size) * head_dim.
 * Returns the number of tokens written, or -1 on a bad argument.
 */
int oracle_kv_compress_epilog(uint8_t* cache, const uint16_t* x, const int64_t* slots, int num_tokens, int d,
                              int block_num, int block_size, int head_dim, int64_t block_stride, int mode,
                              int round_scale)
{
    const int row_bytes = oracle_kv_compress_row_bytes(d, mode);
    if (row_bytes < 0 || d % 64 != 0 || d > 8192 || num_tokens < 0 || block_num <= 0 || block_size <= 0 ||
        head_dim < oracle_kv_compress_cache_col(d, mode) || block_stride < (int64_t)block_size * head_dim)
        return -1;
    const int64_t num_slots = (int64_t)block_num * block_size;
    const int nope = d - 64, groups = nope / 64;
    int written = 0;
    for (int t = 0; t < num_tokens; ++t) {
        const int64_t slot = slots[t];
        if (slot < 0 || slot >= num_slots)
            continue;
        uint8_t* row = cache + (slot / block_size) * block_stride + (slot % block_size) * head_dim;
        const uint16_t* xr = x + (int64_t)t * d;
        for (int c = 0; c < 64; ++c) {                 /* rope: the last 64 columns, bf16 bytes */
            row[2 * c] = (uint8_t)(xr[nope + c] & 0xFF);
            row[2 * c + 1] = (uint8_t)(xr[nope + c] >> 8);
        }
        for (int g = 0; g < groups; ++g) {
            double amax = 0.0;
            for (int c = 0; c < 64; ++c) {
                double v = fabs(oracle_bf16_decode(xr[64 * g + c]));
                if (v > amax) amax = v;
            }
            const double scale = round_to_fp32(amax / OR_E4M3_MAX);
            double used;
            uint8_t* sp = row + 128 + nope;
            if (mode == 0) {
                uint16_t sb = oracle_bf16_encode(scale);
                sp[2 * g] = (uint8_t)(sb & 0xFF);
                sp[2 * g + 1] = (uint8_t)(sb >> 8);
                used = oracle_bf16_decode(sb);
            } else {
                int k = -127;
                if (scale > 0.0) {
                    int e2;
                    double f = frexp(scale, &e2);      /* scale = f * 2^e2, f in [0.5, 1) */
                    k = (round_scale && f != 0.5) ? e2 : e2 - 1;
                    if (k < -127) k = -127;
                    if (k > 127) k = 127;
                }
                sp[g] = (uint8_t)(k + 127);
                used = (scale > 0.0) ? ldexp(1.0, k) : 0.0;
            }
            for (int c = 0; c < 64; ++c) {
                double q = 0.0;
                if (used > 0.0)
                    q = round_to_fp32(oracle_bf16_decode(xr[64 * g + c]) / used);
                row[128 + 64 * g + c] = oracle_e4m3_encode(q);
            }
        }
        ++written;
    }
    return written;
}
