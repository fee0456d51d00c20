/*
 * pa_fp8.h — C ABI of the MI355X (gfx950) FP8 paged-attention decode library.
 *
 * Sources (web pages; cited by title and section):
 * [P1] "PyPTO 实现 GLM-4.5 Paged Attention FP8 量化算子分页 KV Cache 与 E4M3 混合精度
 *      Kernel 实战解析" (m.nxbn.cn/news/52221) — the decode operation:
 *      section 计算流程 (the ten computation steps), section Kernel 签名
 *      (tensor shapes and dtypes), section 量化策略 (scale rules),
 *      section 注意事项 (block-table and sequence-length rules).
 * [P2] "PyPTO-Gym 算子实战DeepSeek V32 MLA 的 Sparse Attention FP8 反量化算子"
 *      (www.mhpn.cn/news/2272720) — the MLA sparse variant: section
 *      核心参数与 KV Cache 布局 (672-byte rows), section API 签名 (tensors),
 *      section 计算流程 (gather, dequant, attention).
 * [P3] "CANN ops-transformer aclnnKvCompressEpilog 算子详解" (www.lmnt.cn/news/267091)
 *      — the two-phase convention (query the workspace size, then run with
 *      a caller-owned workspace) and distinct null-pointer / invalid-argument
 *      status codes.
 *      Also the KvCompressEpilog operator itself (quant modes 0 and 1).
 * [P5] the ops-transformer scatter_pa_kv_cache_with_k_scale page
 *      (www.lmnt.cn/news/278797) — the FP8 KV-cache writer: section
 *      功能说明与计算公式 (slot -> block, offset), section 函数原型 and 约束说明
 *      (tensors, layouts, skipped slots).
 *
 * Conventions for every entry point:
 *  - Pointers named *_dev are device pointers (HBM of the current device);
 *    pointers named *_host are host pointers.  Tensors are dense row-major.
 *  - The caller owns every buffer.  The library allocates nothing, frees
 *    nothing and never synchronises the stream; work is enqueued on `stream`
 *    (a hipStream_t; NULL = the null stream) and returns immediately.
 *  - Inputs are read only.  Outputs are written completely.
 *  - Workspace (size from pa_fp8_decode_workspace_size): scratch for the
 *    partial results of split sequences.  With an explicit split count its
 *    first bytes hold one arrival counter per (batch, KV head), which must
 *    be zero before the first call that uses the buffer (allocate it
 *    zero-filled); every call leaves them zero again.
 *  - Arguments are validated on the host before anything is enqueued; on an
 *    error nothing is launched and a status != PA_OK is returned, with a
 *    message available from pa_fp8_last_error_string() (per host thread).
 *  - Scales are dequantisation multipliers (amax / 448): a value is
 *    code_value * scale.  [P1] stores 448 / amax and dequantises with its
 *    reciprocal; the two are the same scale.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef PA_FP8_H
#define PA_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int pa_status_t;
enum {
    PA_OK = 0,
    PA_ERR_NULLPTR = 1,      /* a required pointer is NULL                       */
    PA_ERR_INVALID = 2,      /* a shape or scalar violates the operation's rules */
    PA_ERR_UNSUPPORTED = 3,  /* legal in principle but not built (e.g. D != 128) */
    PA_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required          */
    PA_ERR_HIP = 5           /* the HIP runtime reported an error at launch      */
};

/* Paged-cache layouts of the cache writer. */
enum {
    PA_CACHE_BSND = 0,       /* [num_blocks, block_size, num_head, head_size] — the decode's layout ([P1]) */
    PA_CACHE_BNBD = 1        /* [num_blocks, num_head, block_size, head_size] — [P5]'s default          */
};

/*
 * Workspace bytes pa_fp8_decode needs for these sizes and split count
 * (num_splits 0 = the library's choice, the same one pa_fp8_decode makes).
 * Writes the size to *bytes_host (0 when no workspace is needed) and, when
 * splits_host is not NULL, the split count that will be used.
 */
pa_status_t pa_fp8_decode_workspace_size(int B, int s1, int nq, int nkv, int D, int block_size,
                                         int max_blocks_per_seq, int s2_tile, int num_splits,
                                         size_t* bytes_host, int* splits_host);

/*
 * FP8 paged GQA decode, [P1] section 计算流程 steps 1-10.  For every batch b,
 * query position s < s1 and query head qh (served by KV head h = qh / (nq/nkv),
 * contiguous groups):
 *   1  q8 = E4M3(q / q_scale) (round to nearest even, saturate at +-448);
 *   2  the tokens p < seq_b are read through block_table in tiles of s2_tile;
 *   3  S_raw = q8 . k8 (exact FP8 x FP8 products, FP32 accumulation);
 *   4  S = S_raw * q_scale * k_scale[p] * softmax_scale;
 *   5  running max M, running sum L += sum exp(S - M) (unquantised);
 *   6  per row and tile: P8 = E4M3(P * 448 / max_tile P);
 *   7  O_tile = P8 . v8 (exact products, FP32 accumulation);
 *   8-9 O = O * exp(M_old - M_new) + O_tile * (max_tile P / 448) * v_scale;
 *   10 out = bf16(O / L).
 * Layouts:
 *   q_dev            [B*s1, nq, D]                  bf16
 *   q_scale_dev      [B*s1, nq]                     fp32, per query token and head
 *   k_cache_dev      [num_blocks, block_size, nkv, D] OCP e4m3fn codes
 *   k_scale_dev      [num_blocks, block_size, nkv]  fp32, per token and KV head
 *   v_cache_dev      [num_blocks, block_size, nkv, D] OCP e4m3fn codes
 *   v_scale_dev      [B, nkv, D]                    fp32, per batch, KV head and channel
 *   block_table_dev  [B, max_blocks_per_seq]        int32 physical block ids
 *   kv_act_seqs_dev  [B]                            int32 valid tokens per batch
 *   out_dev          [B*s1, nq, D]                  bf16, written completely
 * Device-side rules ([P1] section 注意事项): only table entries that cover
 * tokens p < seq_b are read; an entry < 0 or >= num_blocks reads block 0
 * (the page clamps -1 to 0); seq_b is clamped to
 * [0, max_blocks_per_seq * block_size]; seq_b == 0 gives zero output rows;
 * bytes of tokens p >= seq_b are never used (their values may be NaN).
 * Supported: D == 128, block_size == 128, s2_tile in {128, 256, 512, 1024,
 * 2048}, s1 * nq / nkv <= 65535 * 32.  num_splits: 0 = the library's choice, else
 * the number of contiguous tile ranges each sequence is split into (>= 1).
 * Whenever pa_fp8_decode_workspace_size reports a nonzero size,
 * workspace_dev must hold at least that many bytes.
 * Three kernels serve the call (same results within the stated tolerance):
 *  - num_splits == 0, at least 128 query rows per KV head (s1 * nq / nkv),
 *    s2_tile 128, 256 or 512 and at least 64 (batch, KV head, 128-row tile)
 *    workgroups (a prefill chunk, a long multi-token step): one workgroup per
 *    such tile walks the whole sequence, staging each 128-token K or V block
 *    once for its 128 rows; no workspace is used (the debug entry point
 *    takes the whole-row path instead).
 *  - num_splits == 0 and the shape inside the whole-row path's limits: one
 *    workgroup per CU streams a cost-balanced range of (batch, KV-head pair,
 *    block of query rows, tile) units and a small second kernel merges split
 *    sequences.  A KV head's s1 * nq / nkv query rows form one block when
 *    there are at most 32 of them, else blocks of 32, each streaming the
 *    sequence's K and V.  Limits: s2_tile 128, 256 or 512 (1024 only with at
 *    most 16 query rows per KV head; 2048 is not served) and
 *    B * (row blocks) * ceil(nkv / 2) <= 1024 units (nkv odd: nkv in place of
 *    ceil(nkv / 2)).
 *  - otherwise (an explicit num_splits, or a shape outside those limits,
 *    e.g. B >= 257 at nkv = 8): one workgroup per (batch, KV head, block of
 *    query rows, split) -- all of a KV head's rows when they are at most 64,
 *    else blocks of 32 -- with the split count chosen from the table capacity
 *    (no split once there are 1024 or more such units).  It is the slower
 *    path; choose shapes inside the whole-row limits where speed matters.
 */
pa_status_t pa_fp8_decode(const void* q_dev, const float* q_scale_dev,
                          const uint8_t* k_cache_dev, const float* k_scale_dev,
                          const uint8_t* v_cache_dev, const float* v_scale_dev,
                          const int32_t* block_table_dev, const int32_t* kv_act_seqs_dev,
                          void* out_dev,
                          int B, int s1, int nq, int nkv, int D, int block_size,
                          float softmax_scale, int s2_tile, int max_blocks_per_seq, int num_blocks,
                          int num_splits, void* workspace_dev, size_t workspace_bytes,
                          void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * pa_fp8_decode without a workspace argument.  The partial results of split
 * sequences live in a static scratch array of the library,
 * PA_FP8_NOALLOC_SCRATCH_BYTES per device, held from the library's load
 * until the process ends; this call allocates and frees nothing.  A call
 * whose workspace (pa_fp8_decode_workspace_size, same arguments) exceeds
 * that size returns PA_ERR_WORKSPACE before anything is launched (the
 * whole-row path needs at most about 17 MB; the per-head path grows with
 * B * nkv * splits).  Every call on one device shares that device's array,
 * which keeps the last call's contents: calls that overlap in time on one
 * GPU (other streams, other host threads) race and give wrong results.
 * Same arguments (minus the workspace), rules, results and other status
 * codes as pa_fp8_decode.
 */
#define PA_FP8_NOALLOC_SCRATCH_BYTES (32u << 20)
pa_status_t pa_fp8_decode_noalloc(const void* q_dev, const float* q_scale_dev,
                                  const uint8_t* k_cache_dev, const float* k_scale_dev,
                                  const uint8_t* v_cache_dev, const float* v_scale_dev,
                                  const int32_t* block_table_dev, const int32_t* kv_act_seqs_dev,
                                  void* out_dev,
                                  int B, int s1, int nq, int nkv, int D, int block_size,
                                  float softmax_scale, int s2_tile, int max_blocks_per_seq, int num_blocks,
                                  int num_splits, void* stream);

/*
 * pa_fp8_decode plus two dumps taken from inside the kernel:
 *   rows_dev [B, max_blocks_per_seq * block_size] int32: for every logical
 *            token p < seq_b the physical token row (block_id * block_size +
 *            p % block_size) whose K was read; -1 for every other position.
 *   q8_dev   [B*s1, nq, D] uint8: the FP8 query codes of step 1.
 * Same arguments, rules and return codes as pa_fp8_decode.
 */
pa_status_t pa_fp8_decode_debug(const void* q_dev, const float* q_scale_dev,
                                const uint8_t* k_cache_dev, const float* k_scale_dev,
                                const uint8_t* v_cache_dev, const float* v_scale_dev,
                                const int32_t* block_table_dev, const int32_t* kv_act_seqs_dev,
                                void* out_dev,
                                int B, int s1, int nq, int nkv, int D, int block_size,
                                float softmax_scale, int s2_tile, int max_blocks_per_seq, int num_blocks,
                                int num_splits, void* workspace_dev, size_t workspace_bytes,
                                int32_t* rows_dev, uint8_t* q8_dev, void* stream);

/*
 * Causal multi-token decode and chunked prefill: pa_fp8_decode with query
 * position s of s1 attending to the first n_s = clamp(seq - s1 + 1 + s, 0, seq)
 * tokens only (the s1 new tokens are the sequence's last ones and each sees
 * itself and what precedes it) -- [P2]'s valid count (section 关键实现细节)
 * with the sequence in place of topk; [P2] section API 签名与 Decode / Prefill
 * 差异 gives decode and prefill one signature, and so does this entry: s1 may
 * be a prefill chunk (hundreds of positions).  Each position keeps its own
 * tiles over [0, n_s) (P quantised per row over the tile's tokens that row
 * sees); n_s = 0 gives a zero row.  Same arguments, workspace, split count
 * and paths as pa_fp8_decode: the prefill kernel for 128 or more query rows
 * per KV head under its conditions, the whole-row path (query rows in blocks
 * of 32 when there are more than 32) when num_splits == 0 and the shape is
 * inside its limits, else the per-head path, which takes any number of query
 * rows per KV head (blocks of 32 rows when there are more than 64).
 */
pa_status_t pa_fp8_decode_causal(const void* q_dev, const float* q_scale_dev, const uint8_t* k_cache_dev,
                                 const float* k_scale_dev, const uint8_t* v_cache_dev, const float* v_scale_dev,
                                 const int32_t* block_table_dev, const int32_t* kv_act_seqs_dev, void* out_dev,
                                 int B, int s1, int nq, int nkv, int D, int block_size, float softmax_scale,
                                 int s2_tile, int max_blocks_per_seq, int num_blocks, int num_splits,
                                 void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes pa_fp8_mla_sparse_decode needs for these sizes.
 */
pa_status_t pa_fp8_mla_workspace_size(int B, int s1, int nq, int topk, int s2_tile, size_t* bytes_host);

/*
 * MLA-style sparse attention decode over an FP8 latent cache, [P2] sections
 * 核心参数与 KV Cache 布局, API 签名, 计算流程, 关键实现细节 and 在线反量化与
 * Online Softmax.  nkv KV heads read the same latent rows, each through its
 * own top-k slice: query head qh uses KV head h = qh / (nq / nkv) and the
 * indices topk_dev[b*s1 + s, h*topk .. h*topk + topk) ([P2]'s
 * topk_indices (t, n_kv*topk)).  For batch b and query position s < s1, the
 * first n = clamp(seq_b - s1 + 1 + s, 0, topk) entries of a slice are
 * logical token positions (each clamped to [0, seq_b)); position p reads
 * cache row block_table[b, p / 128] * 128 + p % 128.
 *   kn[c] = bf16(fp32(e4m3(row[c]) * scale[c / 128]))   c < 512 (row bytes 0..511,
 *           scales = FP32 at bytes 640..655)
 *   kr    = the 64 BF16 values at row bytes 512..639;  K = [kn | kr], V = kn
 *   per tile of s2_tile positions: S = [qn | qr] . K * softmax_scale,
 *   m = max S, P = exp(S - m); bf16(P) . V and the unquantised sum of P are
 *   merged over tiles; out = bf16(O / L).  n == 0 gives zero rows.
 * Layouts:
 *   q_nope_dev   [B*s1*nq, 512] bf16      q_rope_dev [B*s1*nq, 64] bf16
 *   cache_dev    [num_blocks*128, 672] bytes (one row per token slot)
 *   topk_dev     [B*s1, nkv*topk] int32   block_table_dev [B, max_blocks_per_seq] int32
 *   kv_act_seqs_dev [B] int32             out_dev [B*s1*nq, 512] bf16 (written completely)
 * Device-side rules as for pa_fp8_decode (ids < 0 or >= num_blocks read block
 * 0; seq clamped to the table capacity); only the first n entries of a
 * slice are read, and bytes of rows they do not select are never used
 * (they may hold NaN codes and scales).  Host checks: NULL pointers
 * (PA_ERR_NULLPTR); sizes > 0, nq % nkv == 0, finite softmax_scale > 0
 * (PA_ERR_INVALID); block_size 128, nq / nkv a multiple of 32, s2_tile
 * 128 / 256 / 512, 16-byte aligned queries, cache planes and output
 * (PA_ERR_UNSUPPORTED).  The workspace (size from pa_fp8_mla_workspace_size)
 * holds per-tile partial results.
 */
pa_status_t pa_fp8_mla_sparse_decode(const void* q_nope_dev, const void* q_rope_dev, const uint8_t* cache_dev,
                                     const int32_t* topk_dev, const int32_t* block_table_dev,
                                     const int32_t* kv_act_seqs_dev, void* out_dev, int B, int s1, int nq,
                                     int nkv, int topk, int block_size, int max_blocks_per_seq, int num_blocks,
                                     float softmax_scale, int s2_tile, void* workspace_dev,
                                     size_t workspace_bytes, void* stream);

/*
 * pa_fp8_mla_sparse_decode with the cache as the three tensors of [P2]'s
 * kv_split sister operator (section 相关算子对比) instead of packed rows:
 *   kn_quant_dev  [num_blocks*128, 512] E4M3 codes (row stride 512 bytes)
 *   kr_dev        [num_blocks*128, 64]  bf16        (row stride 128 bytes)
 *   kn_scales_dev [num_blocks*128, 4]   fp32 group scales (row stride 16 bytes)
 * Same computation, same results bit for bit as the packed layout holding the
 * same values; same arguments, checks and workspace otherwise.  All three
 * planes (and q, out) must be 16-byte aligned (PA_ERR_UNSUPPORTED).
 */
pa_status_t pa_fp8_mla_sparse_decode_kv_split(const void* q_nope_dev, const void* q_rope_dev,
                                              const uint8_t* kn_quant_dev, const void* kr_dev,
                                              const float* kn_scales_dev, const int32_t* topk_dev,
                                              const int32_t* block_table_dev, const int32_t* kv_act_seqs_dev,
                                              void* out_dev, int B, int s1, int nq, int nkv, int topk,
                                              int block_size, int max_blocks_per_seq, int num_blocks,
                                              float softmax_scale, int s2_tile, void* workspace_dev,
                                              size_t workspace_bytes, void* stream);

/*
 * FP8 KV-cache writer, [P5] section 功能说明与计算公式: for every token i and
 * head j, with block = slot[i] / block_size and offset = slot[i] % block_size,
 * copy token i's key row and value row of head j and its key scale (i, j) to
 * (block, head j, offset) of key_cache_dev, value_cache_dev and
 * key_scale_cache_dev, in place.  Nothing else is written.
 *   key_dev     token i, head j, byte d at key_dev[i*key_token_stride + j*k_head_size + d]
 *               (E4M3 codes; the bytes are copied, never interpreted)
 *   value_dev   likewise with value_token_stride and v_head_size
 *   slot_mapping_dev [num_tokens] int32 (slot_bits 32) or int64 (slot_bits 64)
 *   key_scale_dev    FP32 (i, j) at key_scale_dev[i*key_scale_token_stride + j*key_scale_head_stride]
 *   layout PA_CACHE_BSND: key_cache  [num_blocks, block_size, num_head, k_head_size],
 *                         value_cache [num_blocks, block_size, num_head, v_head_size],
 *                         key_scale_cache [num_blocks, block_size, num_head]
 *                         (the layouts pa_fp8_decode reads as k_cache / v_cache / k_scale);
 *          PA_CACHE_BNBD: [num_blocks, num_head, block_size, head_size] and
 *                         key_scale_cache [num_blocks, num_head, block_size] ([P5]'s
 *                         [.., 1] shape, same bytes).
 * Tokens whose slot is < 0 or > num_blocks*block_size - 1 are skipped, as [P5]
 * prescribes.  Slots must be distinct (repeated slots: one of the tokens wins,
 * which one is unspecified).  Caller error, not checked: a stride or buffer
 * that does not cover its rows.  Host checks: every pointer non-NULL
 * (PA_ERR_NULLPTR); num_tokens >= 1 ([P5] accepts no empty tensor), positive
 * sizes, slot_bits 32 / 64, a known layout, token strides >= num_head *
 * head_size, scale strides >= 0 (PA_ERR_INVALID); head sizes and token
 * strides multiples of 16 bytes, rows and caches 16-byte aligned
 * (PA_ERR_UNSUPPORTED).  No workspace; asynchronous on `stream`.
 */
pa_status_t pa_fp8_scatter_kv_cache(const uint8_t* key_dev, const uint8_t* value_dev, uint8_t* key_cache_dev,
                                    uint8_t* value_cache_dev, const void* slot_mapping_dev,
                                    const float* key_scale_dev, float* key_scale_cache_dev, int num_tokens,
                                    int num_head, int k_head_size, int v_head_size, int num_blocks,
                                    int block_size, int slot_bits, int layout, int64_t key_token_stride,
                                    int64_t value_token_stride, int64_t key_scale_token_stride,
                                    int64_t key_scale_head_stride, void* stream);

/*
 * KvCompressEpilog, quant modes 0 and 1 ([P3] sections 功能说明, 计算公式,
 * 约束说明).  Two-phase like [P3]: the size query validates the shape and
 * reports the workspace (always 0 bytes here); workspace arguments of the run
 * call are ignored.
 *
 * For every token t whose slot s = slot_mapping[t] lies in
 * [0, block_num * block_size) (others, [P3]'s -1 included, are skipped), the
 * bf16 row x[t, 0:d] is written at
 *     row = cache_dev + (s / block_size) * block_stride + (s % block_size) * head_dim
 * as [rope: the last 64 values, bf16, 128 B][nope codes, d - 64 B][scales]:
 *   per group g of 64 nope columns, scale = fp32(max|x_g| / 448);
 *   mode 0: stored bf16(scale) (RNE, 2 B), code = E4M3(fp32(x / stored));
 *   mode 1: stored e8m0 2^k (1 B, code k + 127, k in [-127, 127]),
 *           k = ceil(log2 scale) when round_scale, else floor(log2 scale),
 *           code = E4M3(fp32(x / 2^k));
 *   codes round to nearest even and saturate at +-448; an all-zero group
 *   gives zero codes (stored scale 0 / e8m0 code 0).  Bytes of the row past
 *   the written ones are not touched; nothing outside the rows of valid
 *   slots is touched.
 *   cache_dev  [block_num] blocks of block_size rows of head_dim bytes, block
 *              starts block_stride bytes apart (>= block_size * head_dim)
 *   x_dev      [num_tokens, d] bf16, 16-byte aligned
 *   slot_mapping_dev [num_tokens] int32 (slot_bits 32) or int64 (64); slots
 *              must be distinct (repeats: unspecified).
 * Host checks: NULL pointers (PA_ERR_NULLPTR); num_tokens >= 1 ([P3] accepts
 * no empty tensor), d % 64 == 0 with 64 < d <= 8192, head_dim >= the row size
 * [P3] requires (mode 1: the written bytes, 323 for d = 256; mode 0: rounded
 * up to 32), block_stride, quant_mode in {0, 1, 2}, slot_bits (PA_ERR_INVALID);
 * quant_mode 2 (hifloat8 / FP4) and misaligned x (PA_ERR_UNSUPPORTED).
 * quant_group_size matters only for mode 2 (modes 0/1 use groups of 64, as
 * [P3]'s row-size formula does); x_scale only for mode 2.
 */
pa_status_t pa_fp8_kv_compress_epilog_workspace_size(int num_tokens, int d, int block_num, int block_size,
                                                     int head_dim, int64_t block_stride, int quant_group_size,
                                                     int quant_mode, size_t* bytes_host);
pa_status_t pa_fp8_kv_compress_epilog(uint8_t* cache_dev, const void* x_dev, const void* slot_mapping_dev,
                                      int num_tokens, int d, int block_num, int block_size, int head_dim,
                                      int64_t block_stride, int slot_bits, int quant_group_size, int quant_mode,
                                      int round_scale, float x_scale, void* workspace_dev, size_t workspace_bytes,
                                      void* stream);

/* Message of the last failed call on this host thread ("" if none); the
 * pointer stays valid until the thread's next call into the library. */
const char* pa_fp8_last_error_string(void);

/* The same message (earlier name, kept for existing callers). */
const char* pa_fp8_last_error(void);

/* Library version string, e.g. "pa_fp8 0.1 gfx950". */
const char* pa_fp8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_FP8_H */
