/*
 * Host sanitizer driver for the CPU oracle (test infrastructure only).
 *
 * Built with -fsanitize=address,undefined together with oracle/pa_oracle.c by
 * tests/test_sanitize_host.py and run as a subprocess: every oracle entry point
 * on small inputs with the edge cases the tests use (empty, clamped and
 * ragged sequences, -1 and out-of-range block ids, skipped slots, top-k
 * positions out of range, invalid shapes).  Any out-of-bounds access, use of
 * uninitialised heap memory through ASan's poisoning, or undefined behaviour
 * aborts the run; the process prints "ok" and exits 0 otherwise.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e4m3_decode(uint8_t c);
uint8_t oracle_e4m3_encode(double x);
double oracle_bf16_decode(uint16_t h);
uint16_t oracle_bf16_encode(double x);
void oracle_mla_dequant_row(const uint8_t* row, double* kvec);
int oracle_pa_fp8_decode(const uint16_t* q_bf16, const float* q_scale, const uint8_t* k8, const float* k_scale,
                         const uint8_t* v8, const float* v_scale, const int32_t* block_table, const int32_t* seqs,
                         int B, int s1, int nq, int nkv, int D, int block_size, double softmax_scale, int s2_tile,
                         int max_blocks, int num_blocks, int causal, int b_lo, int b_hi, double* out_f64,
                         uint16_t* out_bf16, uint8_t* q8_out, double* M_out, double* L_out, int32_t* rows_out);
int oracle_pa_fp8_decode_rows(const uint16_t* q_bf16, const float* q_scale, const uint8_t* k8, const float* k_scale,
                              const uint8_t* v8, const float* v_scale, const int32_t* block_table,
                              const int32_t* seqs, int B, int s1, int nq, int nkv, int D, int block_size,
                              double softmax_scale, int s2_tile, int max_blocks, int num_blocks, int causal,
                              const int64_t* rows, int nrows, double* out_f64, uint16_t* out_bf16, double* M_out,
                              double* L_out);
int oracle_mla_sparse_decode(const uint16_t* q_nope, const uint16_t* q_rope, const uint8_t* cache,
                             const int32_t* topk_idx, const int32_t* block_table, const int32_t* seqs, int B, int s1,
                             int nq, int nkv, int topk, int block_size, int max_blocks, int num_blocks,
                             double softmax_scale, int s2_tile, int b_lo, int b_hi, double* out_f64,
                             uint16_t* out_bf16);
int oracle_scatter_kv_cache(const uint8_t* key, const uint8_t* value, uint8_t* key_cache, uint8_t* value_cache,
                            const int64_t* slots, const float* key_scale, float* key_scale_cache, int num_tokens,
                            int num_head, int k_head_size, int v_head_size, int num_blocks, int block_size,
                            int layout, int64_t key_token_stride, int64_t value_token_stride,
                            int64_t ks_token_stride, int64_t ks_head_stride);
int oracle_kv_compress_epilog(uint8_t* cache, const uint16_t* x, const int64_t* slots, int num_tokens, int d,
                              int block_num, int block_size, int head_dim, int64_t block_stride, int mode,
                              int round_scale);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}
static double next_unit(void) { return (next_u32() & 0xffffff) / 16777216.0; }
static uint8_t finite_code(void) {
    uint8_t c = (uint8_t)(next_u32() & 0xff);
    return (c & 0x7f) == 0x7f ? (uint8_t)(c & 0xf0) : c;       /* never a NaN code */
}
static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "malloc\n"); exit(2); }
    return p;
}
#define CHECK(cond) do { if (!(cond)) { fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); exit(1); } } while (0)

static void codecs(void) {
    for (int c = 0; c < 256; ++c) {
        double v = oracle_e4m3_decode((uint8_t)c);
        if (!isnan(v)) CHECK(oracle_e4m3_encode(v) == c || v == 0.0);
    }
    const double xs[] = {0.0, -0.0, 1e-300, 3.5, 448.0, 464.0, 1e9, -1e9, NAN, INFINITY, 1e38, 3.4e38, 1e-40};
    for (size_t i = 0; i < sizeof(xs) / sizeof(xs[0]); ++i) {
        (void)oracle_e4m3_encode(xs[i]);
        (void)oracle_bf16_decode(oracle_bf16_encode(xs[i]));
    }
}

static void gqa(int causal) {
    const int B = 4, s1 = 3, nq = 8, nkv = 2, D = 128, bs = 128, tile = 256, mb = 5, nb = 12;
    const int64_t nrows = (int64_t)B * s1 * nq;
    uint16_t* q = xmalloc(sizeof(uint16_t) * nrows * D);
    float* qs = xmalloc(sizeof(float) * nrows);
    uint8_t* k = xmalloc((size_t)nb * bs * nkv * D);
    uint8_t* v = xmalloc((size_t)nb * bs * nkv * D);
    float* ks = xmalloc(sizeof(float) * nb * bs * nkv);
    float* vs = xmalloc(sizeof(float) * B * nkv * D);
    int32_t* table = xmalloc(sizeof(int32_t) * B * mb);
    int32_t seqs[4] = {0, 300, 1000000, 2};                  /* empty, ragged, clamped to 640, shorter than s1 */
    for (int64_t i = 0; i < nrows * D; ++i) q[i] = oracle_bf16_encode((next_unit() - 0.5) * 4.0);
    for (int64_t i = 0; i < nrows; ++i) qs[i] = (float)(0.001 + next_unit() * 0.01);
    qs[5] = 0.0f;                                            /* an all-zero query row's scale */
    for (size_t i = 0; i < (size_t)nb * bs * nkv * D; ++i) { k[i] = finite_code(); v[i] = finite_code(); }
    for (int i = 0; i < nb * bs * nkv; ++i) ks[i] = (float)(0.001 + next_unit() * 0.01);
    for (int i = 0; i < B * nkv * D; ++i) vs[i] = (float)(0.001 + next_unit() * 0.01);
    for (int i = 0; i < B * mb; ++i) table[i] = (int32_t)(next_u32() % nb);
    table[1 * mb + 1] = -1;                                  /* -1 inside the sequence: block 0 */
    table[2 * mb + 4] = 1000;                                /* out of range: block 0 */
    double* out = xmalloc(sizeof(double) * nrows * D);
    uint16_t* outb = xmalloc(sizeof(uint16_t) * nrows * D);
    uint8_t* q8 = xmalloc((size_t)nrows * D);
    double* M = xmalloc(sizeof(double) * nrows);
    double* L = xmalloc(sizeof(double) * nrows);
    int32_t* rows = xmalloc(sizeof(int32_t) * B * mb * bs);
    for (int t = 128; t <= 512; t *= 2)
        CHECK(oracle_pa_fp8_decode(q, qs, k, ks, v, vs, table, seqs, B, s1, nq, nkv, D, bs, 0.088, t, mb, nb,
                                   causal, 0, B, out, outb, q8, M, L, rows) == 0);
    for (int64_t i = 0; i < nrows * D; ++i) CHECK(!isnan(out[i]));
    int64_t list[5] = {0, 7, nrows - 1, 30, 50};
    double out2[5 * 128], M2[5], L2[5];
    uint16_t outb2[5 * 128];
    CHECK(oracle_pa_fp8_decode_rows(q, qs, k, ks, v, vs, table, seqs, B, s1, nq, nkv, D, bs, 0.088, tile, mb, nb,
                                    causal, list, 5, out2, outb2, M2, L2) == 0);
    int64_t bad[1] = {nrows};
    CHECK(oracle_pa_fp8_decode_rows(q, qs, k, ks, v, vs, table, seqs, B, s1, nq, nkv, D, bs, 0.088, tile, mb, nb,
                                    causal, bad, 1, out2, outb2, M2, L2) == -1);
    CHECK(oracle_pa_fp8_decode(q, qs, k, ks, v, vs, table, seqs, B, s1, 7, nkv, D, bs, 0.088, tile, mb, nb,
                               causal, 0, B, out, NULL, NULL, NULL, NULL, NULL) == -1);      /* nq % nkv != 0 */
    CHECK(oracle_pa_fp8_decode(q, qs, k, ks, v, vs, table, seqs, B, s1, nq, nkv, D, bs, 0.088, tile, mb, nb,
                               causal, 2, 5, out, NULL, NULL, NULL, NULL, NULL) == -1);      /* b_hi > B */
    free(q); free(qs); free(k); free(v); free(ks); free(vs); free(table);
    free(out); free(outb); free(q8); free(M); free(L); free(rows);
}

static void mla(void) {
    const int B = 2, s1 = 2, nkv = 2, nq = 4, K = 96, bs = 128, mb = 3, nb = 6;
    const int64_t nrows = (int64_t)B * s1 * nq;
    uint16_t* qn = xmalloc(sizeof(uint16_t) * nrows * 512);
    uint16_t* qr = xmalloc(sizeof(uint16_t) * nrows * 64);
    uint8_t* cache = xmalloc((size_t)nb * bs * 672);
    int32_t* topk = xmalloc(sizeof(int32_t) * B * s1 * nkv * K);
    int32_t table[2 * 3] = {4, -1, 2, 0, 5, 99};
    int32_t seqs[2] = {50, 300};
    for (int64_t i = 0; i < nrows * 512; ++i) qn[i] = oracle_bf16_encode(next_unit() - 0.5);
    for (int64_t i = 0; i < nrows * 64; ++i) qr[i] = oracle_bf16_encode(next_unit() - 0.5);
    for (int r = 0; r < nb * bs; ++r) {
        uint8_t* row = cache + (size_t)r * 672;
        for (int c = 0; c < 512; ++c) row[c] = finite_code();
        for (int c = 0; c < 64; ++c) { uint16_t h = oracle_bf16_encode(next_unit() - 0.5); memcpy(row + 512 + 2 * c, &h, 2); }
        for (int g = 0; g < 4; ++g) { float s = (float)(0.001 + next_unit() * 0.01); memcpy(row + 640 + 4 * g, &s, 4); }
        memset(row + 656, 0, 16);
    }
    for (int i = 0; i < B * s1 * nkv * K; ++i) topk[i] = (int32_t)(next_u32() % 400) - 50;   /* some < 0 or >= seq */
    double* out = xmalloc(sizeof(double) * nrows * 512);
    uint16_t* outb = xmalloc(sizeof(uint16_t) * nrows * 512);
    double kvec[576];
    oracle_mla_dequant_row(cache, kvec);
    for (int t = 32; t <= 4096; t *= 8)
        CHECK(oracle_mla_sparse_decode(qn, qr, cache, topk, table, seqs, B, s1, nq, nkv, K, bs, mb, nb, 0.04, t, 0, B,
                                       out, outb) == 0);
    CHECK(oracle_mla_sparse_decode(qn, qr, cache, topk, table, seqs, B, s1, nq, 3, K, bs, mb, nb, 0.04, 32, 0, B,
                                   out, outb) == -1);                                   /* nq % nkv != 0 */
    free(qn); free(qr); free(cache); free(topk); free(out); free(outb);
}

static void writers(void) {
    const int T = 6, H = 2, dk = 16, dv = 32, nb = 2, bs = 4;
    uint8_t key[6 * 2 * 16], value[6 * 2 * 32], kc[2 * 4 * 2 * 16], vc[2 * 4 * 2 * 32];
    float ks[6 * 2], ksc[2 * 4 * 2];
    int64_t slots[6] = {0, 7, -1, 8, 3, 100};                   /* skipped: -1, 8 (= nb*bs), 100 */
    for (size_t i = 0; i < sizeof(key); ++i) key[i] = finite_code();
    for (size_t i = 0; i < sizeof(value); ++i) value[i] = finite_code();
    for (int i = 0; i < 12; ++i) ks[i] = (float)next_unit();
    for (int layout = 0; layout < 2; ++layout) {
        memset(kc, 0, sizeof(kc)); memset(vc, 0, sizeof(vc)); memset(ksc, 0, sizeof(ksc));
        CHECK(oracle_scatter_kv_cache(key, value, kc, vc, slots, ks, ksc, T, H, dk, dv, nb, bs, layout, H * dk,
                                      H * dv, H, 1) == 3);
    }
    CHECK(oracle_scatter_kv_cache(key, value, kc, vc, slots, ks, ksc, T, H, dk, dv, nb, bs, 2, H * dk, H * dv, H,
                                  1) < 0);
    const int d = 256, tokens = 5, bn = 2, bsz = 4, hd = 323;
    uint16_t* x = xmalloc(sizeof(uint16_t) * tokens * d);
    for (int i = 0; i < tokens * d; ++i) x[i] = oracle_bf16_encode((next_unit() - 0.5) * ldexp(1.0, (int)(next_u32() % 60) - 30));
    for (int i = 0; i < d; ++i) x[2 * d + i] = 0;               /* an all-zero row */
    int64_t es[5] = {0, 7, -1, 3, 8};
    for (int mode = 0; mode < 2; ++mode)
        for (int rs = 0; rs < 2; ++rs) {
            const int col = mode == 1 ? hd : 352;
            uint8_t* cache = xmalloc((size_t)bn * bsz * col);
            memset(cache, 0xAB, (size_t)bn * bsz * col);
            CHECK(oracle_kv_compress_epilog(cache, x, es, tokens, d, bn, bsz, col, (int64_t)bsz * col, mode, rs) == 3);
            CHECK(oracle_kv_compress_epilog(cache, x, es, tokens, d, bn, bsz, col - 1, (int64_t)bsz * col, mode, rs) < 0);
            free(cache);
        }
    free(x);
}

int main(void) {
    codecs();
    gqa(0);
    gqa(1);
    mla();
    writers();
    printf("ok\n");
    return 0;
}
