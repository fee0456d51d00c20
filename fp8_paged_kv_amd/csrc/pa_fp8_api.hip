// Host side of the C ABI declared in include/pa_fp8.h: argument validation,
// split planning, workspace sizing and launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <mutex>

#include "../../include/pa_fp8.h"
#include "pa_fp8_common.h"

// Device memory that pa_fp8_decode_noalloc uses in place of a caller's
// workspace: one array per device, held from the library's load until the
// process ends.  In host code `scratch` only names the symbol; its device
// address comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) uint8_t scratch[PA_FP8_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

pa_status_t fail(pa_status_t code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

bool tile_supported(int t) { return t == 128 || t == 256 || t == 512 || t == 1024 || t == 2048; }

// Shape rules shared by every GQA entry point.
pa_status_t check_shapes(int B, int s1, int nq, int nkv, int D, int block_size, int max_blocks,
                         int s2_tile, int num_splits) {
    if (B <= 0 || s1 <= 0 || nq <= 0 || nkv <= 0 || D <= 0 || block_size <= 0 || max_blocks <= 0 ||
        s2_tile <= 0)
        return fail(PA_ERR_INVALID, "sizes must be positive (B=%d s1=%d nq=%d nkv=%d D=%d block_size=%d "
                    "max_blocks_per_seq=%d s2_tile=%d)", B, s1, nq, nkv, D, block_size, max_blocks, s2_tile);
    if (nq % nkv != 0)
        return fail(PA_ERR_INVALID, "nq (%d) must be a multiple of nkv (%d)", nq, nkv);
    if (s2_tile % block_size != 0)
        return fail(PA_ERR_INVALID, "s2_tile (%d) must be a multiple of block_size (%d)", s2_tile, block_size);
    if (num_splits < 0)
        return fail(PA_ERR_INVALID, "num_splits (%d) must be >= 0", num_splits);
    if (D != pa::kHeadDim)
        return fail(PA_ERR_UNSUPPORTED, "head dim %d not built (only 128)", D);
    if (block_size != pa::kBlock)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d not built (only 128)", block_size);
    if (!tile_supported(s2_tile))
        return fail(PA_ERR_UNSUPPORTED, "s2_tile %d not built (128, 256, 512, 1024, 2048)", s2_tile);
    if ((int64_t)s1 * (nq / nkv) > (int64_t)65535 * 32)
        return fail(PA_ERR_UNSUPPORTED, "s1 * nq / nkv = %lld query rows per KV head exceeds 65535 * 32",
                    (long long)s1 * (nq / nkv));
    if ((int64_t)max_blocks * block_size > (int64_t)1 << 30)
        return fail(PA_ERR_UNSUPPORTED, "max_blocks_per_seq * block_size exceeds 2^30 tokens");
    if ((int64_t)B * s1 * nq > ((int64_t)1 << 31) / 128)
        return fail(PA_ERR_UNSUPPORTED, "B * s1 * nq too large");
    return PA_OK;
}

// Number of contiguous tile ranges per sequence.  The host never reads device
// memory, so the choice uses the capacity (table row length), not the actual
// lengths: splits beyond a sequence exit at once.  Aim for enough workgroups
// to keep every CU streaming; more than one split is rounded to a multiple of
// 8 (the placement spreads splits over the 8 XCDs).
int plan_splits(int B, int nkv, int row_blocks, int max_tiles, int requested) {
    if (requested > 0) return requested < max_tiles ? requested : max_tiles;
    const int64_t units = (int64_t)B * nkv * row_blocks;
    const int64_t target = 2048;                  // launched workgroups to aim for
    int64_t s = (target + units - 1) / units;
    if (s <= 1 || units >= 1024) return 1;        // four or more workgroups per CU already
    s = (s + 7) / 8 * 8;
    if (s > max_tiles) s = max_tiles;
    return (int)s;
}

int rows_pad(int s1, int nq, int nkv) { return (s1 * (nq / nkv) + 15) / 16 * 16; }

// Per-head path: query rows per workgroup -- all of a KV head's rows (padded to 16)
// up to 64, else blocks of 32 -- and the number of such blocks per KV head.
int head_row_block(int s1, int nq, int nkv) { const int rp = rows_pad(s1, nq, nkv); return rp <= 64 ? rp : 32; }
int head_row_blocks(int s1, int nq, int nkv) {
    const int rb = head_row_block(s1, nq, nkv);
    return (s1 * (nq / nkv) + rb - 1) / rb;
}

// CUs of the current device, queried once per device (the only state the library keeps).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// The whole-row path (one workgroup per CU, stream-K over (batch, tile, head))
// serves the shapes it was built for when the caller leaves the split count to
// the library; an explicit split count selects the per-head path.
bool use_rows_path(int B, int s1, int nq, int nkv, int s2_tile, int num_splits) {
    return num_splits == 0 && pa::rows_path_supported(nkv, s2_tile, s1 * (nq / nkv), s1, nq, B);
}

// Many query rows per KV head (a prefill chunk, a long multi-token step): the prefill
// kernel, one workgroup per (batch, KV head, 128 rows) sharing each staged K / V block among
// its rows, when there are enough such workgroups to occupy the device; not for the debug
// entry point (it has no dumps).
bool use_prefill_path(int B, int s1, int nq, int nkv, int s2_tile, int num_splits, bool debug) {
    const int rows = s1 * (nq / nkv);
    return num_splits == 0 && !debug && pa::prefill_supported(s2_tile) && rows >= 128 &&
           (int64_t)B * nkv * pa::prefill_row_tiles(rows) >= 64;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Zero n int32 words (the per-head path's arrival counters in the scratch array).
__global__ void zero_words_kernel(int32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// Device address of `scratch` on the current device, looked up once per device
// with that device current.
std::mutex g_scratch_mu;
void* g_scratch_addr[64];

pa_status_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(PA_ERR_UNSUPPORTED, "device %d: at most 64 devices", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                        hipGetErrorString(e));
        g_scratch_addr[dev] = ptr;
    }
    *out = g_scratch_addr[dev];
    return PA_OK;
}

struct WorkspaceLayout {
    size_t meta, tags, part_ml, part_o, total;   // meta: arrival counters (per-head path) or the partition
};

// Per-head path with splits: [U int32 counters | pad][U*nsplit*R*2 | pad][U*nsplit*R*128], U = B*nkv*row blocks
// Whole-row path:             [U int32, untouched | pad][U+2 int32 partition | pad]
//                             [256*2 int32 slot tags | pad][256*2*HG*R*2 | pad][256*2*HG*R*128]
// with U = B*nkv*row blocks, two partial slots per workgroup (its first and last segment,
// the only ones that can be split), HG KV heads per workgroup and R query rows per block
// (all of a KV head's rows padded to 16, or 32).  The whole-row path never writes the
// first U words, so the per-head path's arrival counters stay zero when one workspace
// serves calls of both paths.
WorkspaceLayout layout_for(int B, int s1, int nq, int nkv, int nsplit, bool rows) {
    WorkspaceLayout l = {0, 0, 0, 0, 0};
    if (rows) {
        const int rbk = pa::rows_row_blocks(s1 * (nq / nkv));
        const size_t units = (size_t)B * nkv * rbk, R = (size_t)(rbk > 1 ? 32 : rows_pad(s1, nq, nkv));
        const size_t slots = (size_t)pa::kRowsMaxGrid * 2 * pa::rows_group(nkv);
        l.meta = align256(units * sizeof(int32_t));
        l.tags = l.meta + align256((units + 2) * sizeof(int32_t));
        l.part_ml = l.tags + align256((size_t)pa::kRowsMaxGrid * 2 * sizeof(int32_t));
        l.part_o = l.part_ml + align256(slots * R * 2 * sizeof(float));
        l.total = l.part_o + slots * R * pa::kHeadDim * sizeof(float);
        return l;
    }
    if (nsplit <= 1) return l;
    const size_t units = (size_t)B * nkv * head_row_blocks(s1, nq, nkv), R = (size_t)head_row_block(s1, nq, nkv);
    l.meta = 0;
    l.part_ml = align256(units * sizeof(int32_t));
    l.part_o = l.part_ml + align256(units * nsplit * R * 2 * sizeof(float));
    l.total = l.part_o + units * nsplit * R * pa::kHeadDim * sizeof(float);
    return l;
}

pa_status_t run(const void* q, const float* q_scale, const uint8_t* k_cache, const float* k_scale,
                const uint8_t* v_cache, const float* v_scale, const int32_t* block_table,
                const int32_t* seqs, void* out, int B, int s1, int nq, int nkv, int D, int block_size,
                float softmax_scale, int s2_tile, int max_blocks, int num_blocks, int num_splits,
                void* workspace, size_t workspace_bytes, int32_t* rows_dev, uint8_t* q8_dev,
                bool debug, bool causal, void* stream, bool clear_counters = false) {
    g_err[0] = 0;
    if (!q || !q_scale || !k_cache || !k_scale || !v_cache || !v_scale || !block_table || !seqs || !out)
        return fail(PA_ERR_NULLPTR, "a required tensor pointer is NULL");
    if (debug && (!rows_dev || !q8_dev))
        return fail(PA_ERR_NULLPTR, "debug dump pointers must not be NULL");
    pa_status_t st = check_shapes(B, s1, nq, nkv, D, block_size, max_blocks, s2_tile, num_splits);
    if (st != PA_OK) return st;
    if (num_blocks <= 0) return fail(PA_ERR_INVALID, "num_blocks (%d) must be positive", num_blocks);
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
        return fail(PA_ERR_INVALID, "softmax_scale must be finite and > 0");

    const int capacity = max_blocks * block_size;
    const int max_tiles = (capacity + s2_tile - 1) / s2_tile;
    const bool rows = use_rows_path(B, s1, nq, nkv, s2_tile, num_splits);
    const int rblocks = rows ? pa::rows_row_blocks(s1 * (nq / nkv)) : head_row_blocks(s1, nq, nkv);
    const int nsplit = rows ? 1 : plan_splits(B, nkv, rblocks, max_tiles, num_splits);
    const int tps = (max_tiles + nsplit - 1) / nsplit;
    const WorkspaceLayout lay = layout_for(B, s1, nq, nkv, nsplit, rows);
    const size_t need = lay.total;
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed for %d splits (got %zu)", need, nsplit,
                    workspace ? workspace_bytes : (size_t)0);
    const int nsplit_pad = nsplit == 1 ? 1 : (nsplit + 7) / 8 * 8;
    if ((int64_t)((B + 7) / 8 * 8) * nsplit_pad * nkv > 0x7fffffff)
        return fail(PA_ERR_UNSUPPORTED, "grid too large");
    if ((int64_t)B * nkv * rblocks * nsplit > 0x7fffffff)
        return fail(PA_ERR_UNSUPPORTED, "too many (batch, KV head, row block, split) units");

    pa::DecodeParams p;
    std::memset(&p, 0, sizeof(p));
    p.q = static_cast<const uint16_t*>(q);
    p.q_scale = q_scale;
    p.k_cache = k_cache;
    p.k_scale = k_scale;
    p.v_cache = v_cache;
    p.v_scale = v_scale;
    p.block_table = block_table;
    p.seqs = seqs;
    p.out = static_cast<uint16_t*>(out);
    if (need > 0) {
        char* base = static_cast<char*>(workspace);
        if (rows) {
            p.rows_meta = reinterpret_cast<int32_t*>(base + lay.meta);
            p.part_tag = reinterpret_cast<int32_t*>(base + lay.tags);
        } else {
            p.counters = reinterpret_cast<int32_t*>(base + lay.meta);
        }
        p.part_ml = reinterpret_cast<float*>(base + lay.part_ml);
        p.part_o = reinterpret_cast<float*>(base + lay.part_o);
    }
    p.dbg_rows = debug ? rows_dev : nullptr;
    p.dbg_q8 = debug ? q8_dev : nullptr;
    p.B = B;
    p.s1 = s1;
    p.nq = nq;
    p.nkv = nkv;
    p.G = nq / nkv;
    p.rows = s1 * (nq / nkv);
    p.s2_tile = s2_tile;
    p.max_blocks = max_blocks;
    p.num_blocks = num_blocks;
    p.capacity = capacity;
    p.nsplit = nsplit;
    p.nsplit_pad = nsplit_pad;
    p.tiles_per_split = tps;
    p.row_block = rows ? (rblocks > 1 ? 32 : rows_pad(s1, nq, nkv)) : head_row_block(s1, nq, nkv);
    p.row_blocks = rblocks;
    p.softmax_scale = softmax_scale;
    p.causal = causal ? 1 : 0;

    hipError_t e;
    if (clear_counters && p.counters) {
        // a workspace the caller did not zero (the library's scratch): clear the arrival counters
        const int n = B * nkv * rblocks;
        hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                           p.counters, n);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(PA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
    }
    if (use_prefill_path(B, s1, nq, nkv, s2_tile, num_splits, debug)) {
        e = pa::launch_prefill(p, static_cast<hipStream_t>(stream));
    } else if (rows) {
        if (debug && p.dbg_rows) {
            e = pa::launch_fill_rows(p, static_cast<hipStream_t>(stream));
            if (e != hipSuccess) return fail(PA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
        }
        e = pa::launch_decode_rows(p, device_cus(), static_cast<hipStream_t>(stream), debug);
    } else {
        e = pa::launch_decode(p, static_cast<hipStream_t>(stream), debug);
    }
    if (e != hipSuccess) return fail(PA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

// MLA sparse decode over three row planes (packed rows: one buffer at offsets
// 0 / 512 / 640 with stride 672; kv_split: three tensors).
pa_status_t run_mla(const void* q_nope, const void* q_rope, const uint8_t* nope, const uint8_t* rope,
                    const uint8_t* scales, int64_t nope_stride, int64_t rope_stride, int64_t scale_stride,
                    const int32_t* topk_dev, const int32_t* block_table_dev, const int32_t* kv_act_seqs_dev,
                    void* out_dev, int B, int s1, int nq, int nkv, int topk, int block_size,
                    int max_blocks_per_seq, int num_blocks, float softmax_scale, int s2_tile, void* workspace_dev,
                    size_t workspace_bytes, void* stream) {
    if (!q_nope || !q_rope || !topk_dev || !block_table_dev || !kv_act_seqs_dev || !out_dev)
        return fail(PA_ERR_NULLPTR, "a required pointer is NULL");
    size_t need = 0;
    pa_status_t st = pa_fp8_mla_workspace_size(B, s1, nq, topk, s2_tile, &need);
    if (st != PA_OK) return st;
    if (nkv <= 0 || nq % nkv != 0)
        return fail(PA_ERR_INVALID, "nkv (%d) must be positive and divide nq (%d)", nkv, nq);
    if (!pa::mla_supported(nq, nkv, s2_tile))
        return fail(PA_ERR_UNSUPPORTED, "MLA decode built for nq / nkv a multiple of 32 (nq=%d nkv=%d)", nq, nkv);
    if ((int64_t)B * s1 * nkv * topk > ((int64_t)1 << 31) - 1)
        return fail(PA_ERR_UNSUPPORTED, "B * s1 * nkv * topk exceeds 2^31 - 1 indices");
    if (block_size != pa::kBlock)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d not built (only 128)", block_size);
    if (max_blocks_per_seq <= 0 || num_blocks <= 0)
        return fail(PA_ERR_INVALID, "max_blocks_per_seq (%d) and num_blocks (%d) must be positive",
                    max_blocks_per_seq, num_blocks);
    if ((int64_t)num_blocks * block_size > ((int64_t)1 << 31) - 1)
        return fail(PA_ERR_UNSUPPORTED, "num_blocks * block_size exceeds 2^31 - 1 rows");
    if ((int64_t)max_blocks_per_seq * block_size > (int64_t)1 << 30)
        return fail(PA_ERR_UNSUPPORTED, "max_blocks_per_seq * block_size exceeds 2^30 tokens");
    if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
        return fail(PA_ERR_INVALID, "softmax_scale must be finite and > 0");
    auto mis = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) != 0; };
    if (mis(q_nope) || mis(q_rope) || mis(nope) || mis(rope) || mis(scales) || mis(out_dev))
        return fail(PA_ERR_UNSUPPORTED, "queries, cache planes and output must be 16-byte aligned");
    if (!workspace_dev || workspace_bytes < need)
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                    workspace_dev ? workspace_bytes : (size_t)0);
    pa::MlaParams p;
    std::memset(&p, 0, sizeof(p));
    p.q_nope = static_cast<const uint16_t*>(q_nope);
    p.q_rope = static_cast<const uint16_t*>(q_rope);
    p.nope = nope;
    p.rope = rope;
    p.scales = scales;
    p.nope_stride = nope_stride;
    p.rope_stride = rope_stride;
    p.scale_stride = scale_stride;
    p.topk_idx = topk_dev;
    p.block_table = block_table_dev;
    p.seqs = kv_act_seqs_dev;
    p.out = static_cast<uint16_t*>(out_dev);
    const size_t rows = (size_t)B * s1 * nq;
    p.ntiles_max = (topk + s2_tile - 1) / s2_tile;
    char* base = static_cast<char*>(workspace_dev);
    p.part_ml = reinterpret_cast<float*>(base);
    p.part_o = reinterpret_cast<float*>(base + align256(rows * p.ntiles_max * 2 * sizeof(float)));
    p.B = B;
    p.s1 = s1;
    p.nq = nq;
    p.nkv = nkv;
    p.topk = topk;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    p.capacity = max_blocks_per_seq * block_size;
    p.s2_tile = s2_tile;
    p.softmax_scale = softmax_scale;
    hipError_t e = pa::launch_mla(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status_t pa_fp8_decode_workspace_size(int B, int s1, int nq, int nkv, int D, int block_size,
                                         int max_blocks_per_seq, int s2_tile, int num_splits,
                                         size_t* bytes_host, int* splits_host) {
    g_err[0] = 0;
    if (!bytes_host) return fail(PA_ERR_NULLPTR, "bytes_host is NULL");
    pa_status_t st = check_shapes(B, s1, nq, nkv, D, block_size, max_blocks_per_seq, s2_tile, num_splits);
    if (st != PA_OK) return st;
    const int capacity = max_blocks_per_seq * block_size;
    const int max_tiles = (capacity + s2_tile - 1) / s2_tile;
    const bool rows = use_rows_path(B, s1, nq, nkv, s2_tile, num_splits);
    const int nsplit = rows ? 1 : plan_splits(B, nkv, head_row_blocks(s1, nq, nkv), max_tiles, num_splits);
    *bytes_host = layout_for(B, s1, nq, nkv, nsplit, rows).total;
    if (splits_host) *splits_host = nsplit;
    return PA_OK;
}

pa_status_t pa_fp8_decode(const void* q_dev, const float* q_scale_dev, const uint8_t* k_cache_dev,
                          const float* k_scale_dev, const uint8_t* v_cache_dev, const float* v_scale_dev,
                          const int32_t* block_table_dev, const int32_t* kv_act_seqs_dev, void* out_dev, int B,
                          int s1, int nq, int nkv, int D, int block_size, float softmax_scale, int s2_tile,
                          int max_blocks_per_seq, int num_blocks, int num_splits, void* workspace_dev,
                          size_t workspace_bytes, void* stream) {
    return run(q_dev, q_scale_dev, k_cache_dev, k_scale_dev, v_cache_dev, v_scale_dev, block_table_dev,
               kv_act_seqs_dev, out_dev, B, s1, nq, nkv, D, block_size, softmax_scale, s2_tile,
               max_blocks_per_seq, num_blocks, num_splits, workspace_dev, workspace_bytes, nullptr, nullptr,
               false, false, stream);
}

pa_status_t pa_fp8_decode_noalloc(const void* q_dev, const float* q_scale_dev, const uint8_t* k_cache_dev,
                                  const float* k_scale_dev, const uint8_t* v_cache_dev, const float* v_scale_dev,
                                  const int32_t* block_table_dev, const int32_t* kv_act_seqs_dev, void* out_dev,
                                  int B, int s1, int nq, int nkv, int D, int block_size, float softmax_scale,
                                  int s2_tile, int max_blocks_per_seq, int num_blocks, int num_splits,
                                  void* stream) {
    g_err[0] = 0;
    if (!q_dev || !q_scale_dev || !k_cache_dev || !k_scale_dev || !v_cache_dev || !v_scale_dev ||
        !block_table_dev || !kv_act_seqs_dev || !out_dev)
        return fail(PA_ERR_NULLPTR, "a required tensor pointer is NULL");
    size_t need = 0;
    int nsplit = 0;
    pa_status_t st = pa_fp8_decode_workspace_size(B, s1, nq, nkv, D, block_size, max_blocks_per_seq, s2_tile,
                                                  num_splits, &need, &nsplit);
    if (st != PA_OK) return st;
    if (need > (size_t)PA_FP8_NOALLOC_SCRATCH_BYTES)
        return fail(PA_ERR_WORKSPACE, "this call needs %zu bytes of scratch (%d splits); the library holds %zu "
                    "per device: use pa_fp8_decode with a workspace", need, nsplit,
                    (size_t)PA_FP8_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != PA_OK) return st;
    return run(q_dev, q_scale_dev, k_cache_dev, k_scale_dev, v_cache_dev, v_scale_dev, block_table_dev,
               kv_act_seqs_dev, out_dev, B, s1, nq, nkv, D, block_size, softmax_scale, s2_tile,
               max_blocks_per_seq, num_blocks, num_splits, ws, (size_t)PA_FP8_NOALLOC_SCRATCH_BYTES, nullptr,
               nullptr, false, false, stream, true);
}

pa_status_t pa_fp8_decode_debug(const void* q_dev, const float* q_scale_dev, const uint8_t* k_cache_dev,
                                const float* k_scale_dev, const uint8_t* v_cache_dev, const float* v_scale_dev,
                                const int32_t* block_table_dev, const int32_t* kv_act_seqs_dev, void* out_dev,
                                int B, int s1, int nq, int nkv, int D, int block_size, float softmax_scale,
                                int s2_tile, int max_blocks_per_seq, int num_blocks, int num_splits,
                                void* workspace_dev, size_t workspace_bytes, int32_t* rows_dev, uint8_t* q8_dev,
                                void* stream) {
    return run(q_dev, q_scale_dev, k_cache_dev, k_scale_dev, v_cache_dev, v_scale_dev, block_table_dev,
               kv_act_seqs_dev, out_dev, B, s1, nq, nkv, D, block_size, softmax_scale, s2_tile,
               max_blocks_per_seq, num_blocks, num_splits, workspace_dev, workspace_bytes, rows_dev, q8_dev,
               true, false, stream);
}

pa_status_t pa_fp8_decode_causal(const void* q_dev, const float* q_scale_dev, const uint8_t* k_cache_dev,
                                 const float* k_scale_dev, const uint8_t* v_cache_dev, const float* v_scale_dev,
                                 const int32_t* block_table_dev, const int32_t* kv_act_seqs_dev, void* out_dev,
                                 int B, int s1, int nq, int nkv, int D, int block_size, float softmax_scale,
                                 int s2_tile, int max_blocks_per_seq, int num_blocks, int num_splits,
                                 void* workspace_dev, size_t workspace_bytes, void* stream) {
    return run(q_dev, q_scale_dev, k_cache_dev, k_scale_dev, v_cache_dev, v_scale_dev, block_table_dev,
               kv_act_seqs_dev, out_dev, B, s1, nq, nkv, D, block_size, softmax_scale, s2_tile,
               max_blocks_per_seq, num_blocks, num_splits, workspace_dev, workspace_bytes, nullptr, nullptr, false,
               true, stream);
}

pa_status_t pa_fp8_mla_workspace_size(int B, int s1, int nq, int topk, int s2_tile, size_t* bytes_host) {
    g_err[0] = 0;
    if (!bytes_host) return fail(PA_ERR_NULLPTR, "bytes_host is NULL");
    if (B <= 0 || s1 <= 0 || nq <= 0 || topk <= 0 || s2_tile <= 0)
        return fail(PA_ERR_INVALID, "sizes must be positive (B=%d s1=%d nq=%d topk=%d s2_tile=%d)", B, s1, nq,
                    topk, s2_tile);
    if (s2_tile != 128 && s2_tile != 256 && s2_tile != 512)
        return fail(PA_ERR_UNSUPPORTED, "MLA decode built for s2_tile 128/256/512 (s2_tile=%d)", s2_tile);
    const size_t rows = (size_t)B * s1 * nq, nt = (size_t)((topk + s2_tile - 1) / s2_tile);
    *bytes_host = align256(rows * nt * 2 * sizeof(float)) + rows * nt * 512 * sizeof(float);
    return PA_OK;
}

pa_status_t pa_fp8_mla_sparse_decode(const void* q_nope_dev, const void* q_rope_dev, const uint8_t* cache_dev,
                                     const int32_t* topk_dev, const int32_t* block_table_dev,
                                     const int32_t* kv_act_seqs_dev, void* out_dev, int B, int s1, int nq,
                                     int nkv, int topk, int block_size, int max_blocks_per_seq, int num_blocks,
                                     float softmax_scale, int s2_tile, void* workspace_dev,
                                     size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (!cache_dev) return fail(PA_ERR_NULLPTR, "a required pointer is NULL");
    return run_mla(q_nope_dev, q_rope_dev, cache_dev, cache_dev + 512, cache_dev + 640, 672, 672, 672, topk_dev,
                   block_table_dev, kv_act_seqs_dev, out_dev, B, s1, nq, nkv, topk, block_size, max_blocks_per_seq,
                   num_blocks, softmax_scale, s2_tile, workspace_dev, workspace_bytes, stream);
}

pa_status_t pa_fp8_mla_sparse_decode_kv_split(const void* q_nope_dev, const void* q_rope_dev,
                                              const uint8_t* kn_quant_dev, const void* kr_dev,
                                              const float* kn_scales_dev, const int32_t* topk_dev,
                                              const int32_t* block_table_dev, const int32_t* kv_act_seqs_dev,
                                              void* out_dev, int B, int s1, int nq, int nkv, int topk,
                                              int block_size, int max_blocks_per_seq, int num_blocks,
                                              float softmax_scale, int s2_tile, void* workspace_dev,
                                              size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    if (!kn_quant_dev || !kr_dev || !kn_scales_dev) return fail(PA_ERR_NULLPTR, "a required pointer is NULL");
    return run_mla(q_nope_dev, q_rope_dev, kn_quant_dev, static_cast<const uint8_t*>(kr_dev),
                   reinterpret_cast<const uint8_t*>(kn_scales_dev), 512, 128, 16, topk_dev, block_table_dev,
                   kv_act_seqs_dev, out_dev, B, s1, nq, nkv, topk, block_size, max_blocks_per_seq, num_blocks,
                   softmax_scale, s2_tile, workspace_dev, workspace_bytes, stream);
}

pa_status_t pa_fp8_scatter_kv_cache(const uint8_t* key_dev, const uint8_t* value_dev, uint8_t* key_cache_dev,
                                    uint8_t* value_cache_dev, const void* slot_mapping_dev,
                                    const float* key_scale_dev, float* key_scale_cache_dev, int num_tokens,
                                    int num_head, int k_head_size, int v_head_size, int num_blocks,
                                    int block_size, int slot_bits, int layout, int64_t key_token_stride,
                                    int64_t value_token_stride, int64_t key_scale_token_stride,
                                    int64_t key_scale_head_stride, void* stream) {
    g_err[0] = 0;
    if (!key_dev || !value_dev || !key_cache_dev || !value_cache_dev || !slot_mapping_dev || !key_scale_dev ||
        !key_scale_cache_dev)
        return fail(PA_ERR_NULLPTR, "a required pointer is NULL");
    if (num_tokens <= 0 || num_head <= 0 || k_head_size <= 0 || v_head_size <= 0 || num_blocks <= 0 ||
        block_size <= 0)
        return fail(PA_ERR_INVALID, "sizes must be positive (num_tokens=%d num_head=%d k_head_size=%d "
                    "v_head_size=%d num_blocks=%d block_size=%d)", num_tokens, num_head, k_head_size,
                    v_head_size, num_blocks, block_size);
    if (slot_bits != 32 && slot_bits != 64) return fail(PA_ERR_INVALID, "slot_bits must be 32 or 64 (got %d)", slot_bits);
    if (layout != PA_CACHE_BSND && layout != PA_CACHE_BNBD)
        return fail(PA_ERR_INVALID, "layout must be PA_CACHE_BSND or PA_CACHE_BNBD (got %d)", layout);
    if (key_token_stride < (int64_t)num_head * k_head_size || value_token_stride < (int64_t)num_head * v_head_size)
        return fail(PA_ERR_INVALID, "token strides must cover num_head * head_size bytes");
    if (key_scale_token_stride < 0 || key_scale_head_stride < 0)
        return fail(PA_ERR_INVALID, "key_scale strides must be >= 0");
    if (k_head_size % 16 || v_head_size % 16 || key_token_stride % 16 || value_token_stride % 16)
        return fail(PA_ERR_UNSUPPORTED, "head sizes and token strides must be multiples of 16 bytes");
    auto mis = [](const void* ptr, uintptr_t al) { return (reinterpret_cast<uintptr_t>(ptr) & (al - 1)) != 0; };
    if (mis(key_dev, 16) || mis(value_dev, 16) || mis(key_cache_dev, 16) || mis(value_cache_dev, 16) ||
        mis(key_scale_dev, 4) || mis(key_scale_cache_dev, 4) || mis(slot_mapping_dev, slot_bits / 8))
        return fail(PA_ERR_UNSUPPORTED, "rows and caches must be 16-byte aligned, scales 4-byte, slots "
                    "aligned to their width");
    pa::ScatterParams p;
    std::memset(&p, 0, sizeof(p));
    p.key = key_dev;
    p.value = value_dev;
    p.key_cache = key_cache_dev;
    p.value_cache = value_cache_dev;
    p.slots = slot_mapping_dev;
    p.key_scale = key_scale_dev;
    p.key_scale_cache = key_scale_cache_dev;
    p.num_tokens = num_tokens;
    p.num_slots = (int64_t)num_blocks * block_size;
    p.num_head = num_head;
    p.k_head_size = k_head_size;
    p.v_head_size = v_head_size;
    p.block_size = block_size;
    p.k_stride = key_token_stride;
    p.v_stride = value_token_stride;
    p.ks_token_stride = key_scale_token_stride;
    p.ks_head_stride = key_scale_head_stride;
    hipError_t e = pa::launch_scatter_kv(p, slot_bits, layout, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

pa_status_t pa_fp8_kv_compress_epilog_workspace_size(int num_tokens, int d, int block_num, int block_size,
                                                     int head_dim, int64_t block_stride, int quant_group_size,
                                                     int quant_mode, size_t* bytes_host) {
    g_err[0] = 0;
    if (!bytes_host) return fail(PA_ERR_NULLPTR, "bytes_host is NULL");
    if (num_tokens <= 0 || block_num <= 0 || block_size <= 0 || head_dim <= 0)
        return fail(PA_ERR_INVALID, "sizes must be positive (num_tokens=%d block_num=%d block_size=%d head_dim=%d)",
                    num_tokens, block_num, block_size, head_dim);
    if (d % 64 != 0 || d <= 64 || d > 8192)
        return fail(PA_ERR_INVALID, "d must be a multiple of 64 in (64, 8192] (got %d)", d);
    if (quant_mode < 0 || quant_mode > 2) return fail(PA_ERR_INVALID, "quant_mode must be 0, 1 or 2 (got %d)", quant_mode);
    if (quant_mode == 2) {
        if (quant_group_size != 16 && quant_group_size != 32 && quant_group_size != 64)
            return fail(PA_ERR_INVALID, "mode 2 takes quant_group_size 16, 32 or 64 (got %d)", quant_group_size);
        return fail(PA_ERR_UNSUPPORTED, "quant_mode 2 (hifloat8 rope, FP4 nope) is not built");
    }
    const int groups = (d - 64 + 63) / 64;
    const int written = (d - 64) + 128 + groups * (quant_mode == 0 ? 2 : 1);
    const int col = quant_mode == 1 ? written : (written + 31) / 32 * 32;
    if (head_dim < col)
        return fail(PA_ERR_INVALID, "head_dim %d below the %d bytes a row of mode %d needs", head_dim, col, quant_mode);
    if (block_stride < (int64_t)block_size * head_dim)
        return fail(PA_ERR_INVALID, "block_stride must be >= block_size * head_dim");
    *bytes_host = 0;
    return PA_OK;
}

pa_status_t pa_fp8_kv_compress_epilog(uint8_t* cache_dev, const void* x_dev, const void* slot_mapping_dev,
                                      int num_tokens, int d, int block_num, int block_size, int head_dim,
                                      int64_t block_stride, int slot_bits, int quant_group_size, int quant_mode,
                                      int round_scale, float x_scale, void* workspace_dev, size_t workspace_bytes,
                                      void* stream) {
    (void)x_scale;                     // used by mode 2 only
    (void)workspace_dev;
    (void)workspace_bytes;
    g_err[0] = 0;
    if (!cache_dev || !x_dev || !slot_mapping_dev) return fail(PA_ERR_NULLPTR, "a required pointer is NULL");
    size_t need = 0;
    pa_status_t st = pa_fp8_kv_compress_epilog_workspace_size(num_tokens, d, block_num, block_size, head_dim,
                                                              block_stride, quant_group_size, quant_mode, &need);
    if (st != PA_OK) return st;
    if (slot_bits != 32 && slot_bits != 64) return fail(PA_ERR_INVALID, "slot_bits must be 32 or 64 (got %d)", slot_bits);
    if ((reinterpret_cast<uintptr_t>(x_dev) & 15) || (reinterpret_cast<uintptr_t>(slot_mapping_dev) & (slot_bits / 8 - 1)))
        return fail(PA_ERR_UNSUPPORTED, "x must be 16-byte aligned and slots aligned to their width");
    pa::EpilogParams p;
    std::memset(&p, 0, sizeof(p));
    p.cache = cache_dev;
    p.x = static_cast<const uint16_t*>(x_dev);
    p.slots = slot_mapping_dev;
    p.num_tokens = num_tokens;
    p.num_slots = (int64_t)block_num * block_size;
    p.block_stride = block_stride;
    p.d = d;
    p.block_size = block_size;
    p.head_dim = head_dim;
    p.mode = quant_mode;
    p.round_scale = round_scale ? 1 : 0;
    hipError_t e = pa::launch_kv_compress_epilog(p, slot_bits, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
    return PA_OK;
}

const char* pa_fp8_last_error_string(void) { return g_err; }

const char* pa_fp8_last_error(void) { return g_err; }

const char* pa_fp8_version(void) { return "pa_fp8 0.1 gfx950"; }

}  // extern "C"
