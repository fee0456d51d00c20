// Shared host/device definitions of the HIP decode library (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kHeadDim = 128;   // D of the GQA path
constexpr int kBlock = 128;     // tokens per cache block

// Everything a decode launch needs; filled and validated on the host.
struct DecodeParams {
    const uint16_t* q;          // [B*s1, nq, 128] bf16
    const float* q_scale;       // [B*s1, nq]
    const uint8_t* k_cache;     // [num_blocks, 128, nkv, 128]
    const float* k_scale;       // [num_blocks, 128, nkv]
    const uint8_t* v_cache;     // [num_blocks, 128, nkv, 128]
    const float* v_scale;       // [B, nkv, 128]
    const int32_t* block_table; // [B, max_blocks]
    const int32_t* seqs;        // [B]
    uint16_t* out;              // [B*s1, nq, 128] bf16
    int32_t* counters;          // per-head path: [B*nkv] arrival counters (zero between calls)
    int32_t* rows_meta;         // whole-row path: cost prefix over (batch, head group), workgroups used
    int32_t* part_tag;          // whole-row path: [256, 2] (batch, head group) of each partial slot, -1 = none
    float* part_o;              // per-head path: [B*nkv, nsplit, rows_pad, 128];
                                // whole-row path: [256, 2, HG, rows_pad, 128] (workgroup, first / last segment)
    float* part_ml;             // the same with 2 floats per row (M in log2 units, L)
    int32_t* dbg_rows;          // [B, capacity] or null
    uint8_t* dbg_q8;            // [B*s1, nq, 128] or null
    int B, s1, nq, nkv, G, rows;
    int s2_tile, max_blocks, num_blocks, capacity;
    int nsplit, nsplit_pad, tiles_per_split;
    int row_block, row_blocks;  // query rows per block (padded) and blocks per KV head: per-head path
                                // 16..64 per workgroup; whole-row path all rows (<= 32) or blocks of 32
    int causal;                 // position s of s1 sees the first seq - s1 + 1 + s tokens
    float softmax_scale;
};

// MLA-style sparse decode (one latent KV head, 672-byte cache rows).
struct MlaParams {
    const uint16_t* q_nope;     // [B*s1*nq, 512] bf16
    const uint16_t* q_rope;     // [B*s1*nq, 64] bf16
    const uint8_t* nope;        // row r: 512 E4M3 codes at nope + r * nope_stride
    const uint8_t* rope;        // row r: 64 bf16 at rope + r * rope_stride
    const uint8_t* scales;      // row r: 4 fp32 group scales at scales + r * scale_stride
    int64_t nope_stride, rope_stride, scale_stride;   // bytes
    const int32_t* topk_idx;    // [B*s1, nkv*topk] logical token positions, one slice per KV head
    const int32_t* block_table; // [B, max_blocks]
    const int32_t* seqs;        // [B]
    uint16_t* out;              // [B*s1*nq, 512] bf16
    float* part_o;              // [B*s1*nq, ntiles_max, 512]
    float* part_ml;             // [B*s1*nq, ntiles_max, 2]  (tile max in log2 units, sum)
    int B, s1, nq, nkv, topk, max_blocks, num_blocks, capacity, s2_tile, ntiles_max;
    float softmax_scale;
};

// FP8 KV-cache writer (slot scatter of key / value rows and key scales).
struct ScatterParams {
    const uint8_t* key;         // token i, head j at key + i * k_stride + j * k_head_size
    const uint8_t* value;       // likewise with v_stride, v_head_size
    uint8_t* key_cache;         // BSND [nb, bs, H, dk] or BNBD [nb, H, bs, dk]
    uint8_t* value_cache;       // same layout with dv
    const void* slots;          // [num_tokens] int32 or int64
    const float* key_scale;     // (i, j) at i * ks_token_stride + j * ks_head_stride
    float* key_scale_cache;     // BSND [nb, bs, H] or BNBD [nb, H, bs]
    int64_t num_tokens, num_slots;
    int num_head, k_head_size, v_head_size, block_size;
    int64_t k_stride, v_stride, ks_token_stride, ks_head_stride;
};

// KvCompressEpilog modes 0 / 1 (quantising slot scatter of bf16 rows).
struct EpilogParams {
    uint8_t* cache;             // row of slot s: cache + (s / block_size) * block_stride + (s % block_size) * head_dim
    const uint16_t* x;          // [num_tokens, d] bf16
    const void* slots;          // [num_tokens] int32 or int64
    int64_t num_tokens, num_slots, block_stride;
    int d, block_size, head_dim, mode, round_scale;
};

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream, bool debug);
hipError_t launch_kv_compress_epilog(const EpilogParams& p, int slot_bits, hipStream_t stream);
hipError_t launch_scatter_kv(const ScatterParams& p, int slot_bits, int layout, hipStream_t stream);
bool mla_supported(int nq, int nkv, int s2_tile);
hipError_t launch_mla(const MlaParams& p, hipStream_t stream);
int grid_size(const DecodeParams& p);
bool rows_path_supported(int nkv, int s2_tile, int rows, int s1, int nq, int B);
constexpr int kRowsMaxGrid = 256;   // whole-row path: at most one workgroup per CU, at most 256
int rows_group(int nkv);            // KV heads per whole-row workgroup
int rows_row_blocks(int rows);      // query-row blocks per KV head on the whole-row path
hipError_t launch_decode_rows(const DecodeParams& p, int cus, hipStream_t stream, bool debug);
// many query rows per KV head (chunked prefill): one workgroup per (batch, KV head, 128 rows)
int prefill_row_tiles(int rows);
bool prefill_supported(int s2_tile);
hipError_t launch_prefill(const DecodeParams& p, hipStream_t stream);
hipError_t launch_fill_rows(const DecodeParams& p, hipStream_t stream);

}  // namespace pa
