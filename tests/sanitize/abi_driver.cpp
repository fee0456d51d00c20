// Host sanitizer driver for the library's argument validation (test
// infrastructure only).  Built by tests/test_sanitize_host.py from the HIP
// sources compiled for the host only, with -fsanitize=address,undefined on the
// host side, and run as a subprocess without a GPU: every entry point is called
// with arguments that fail validation (NULL pointers, bad shapes, missing or
// short workspaces, over-large scratch needs), and every size query with valid
// and invalid shapes.  No call reaches a kernel launch.  Prints "ok" and
// exits 0 when every status code is the expected one and no sanitizer fired.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "pa_fp8.h"

#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
            std::exit(1);                                                        \
        }                                                                        \
    } while (0)

static void* const F = reinterpret_cast<void*>(0x10000);    // never dereferenced
static const float* const FF = reinterpret_cast<const float*>(0x10000);
static const uint8_t* const FU = reinterpret_cast<const uint8_t*>(0x10000);
static const int32_t* const FI = reinterpret_cast<const int32_t*>(0x10000);

static int dec(const void* q, int B, int s1, int nq, int nkv, int D, int bs, float sc, int tile, int mb, int nb,
               int splits, void* ws, size_t wsb) {
    return pa_fp8_decode(q, FF, FU, FF, FU, FF, FI, FI, F, B, s1, nq, nkv, D, bs, sc, tile, mb, nb, splits, ws, wsb,
                         nullptr);
}

int main() {
    size_t n = 0;
    int sp = 0;
    CHECK(pa_fp8_decode_workspace_size(32, 1, 96, 8, 128, 128, 64, 512, 0, &n, &sp) == PA_OK && n > 0);
    CHECK(pa_fp8_decode_workspace_size(2, 256, 96, 8, 128, 128, 64, 512, 0, &n, &sp) == PA_OK);
    CHECK(pa_fp8_decode_workspace_size(2, 1, 8, 3, 128, 128, 6, 256, 1, &n, &sp) == PA_ERR_INVALID);
    CHECK(pa_fp8_decode_workspace_size(2, 1, 8, 2, 128, 128, 6, 256, 1, nullptr, &sp) == PA_ERR_NULLPTR);
    CHECK(std::strlen(pa_fp8_last_error_string()) > 0);

    CHECK(dec(nullptr, 2, 1, 8, 2, 128, 128, 0.088f, 256, 6, 8, 1, nullptr, 0) == PA_ERR_NULLPTR);
    CHECK(dec(F, 0, 1, 8, 2, 128, 128, 0.088f, 256, 6, 8, 1, nullptr, 0) == PA_ERR_INVALID);
    CHECK(dec(F, 2, 1, 8, 2, 128, 128, -1.f, 256, 6, 8, 1, nullptr, 0) == PA_ERR_INVALID);
    CHECK(dec(F, 2, 1, 8, 2, 128, 128, 0.088f, 200, 6, 8, 1, nullptr, 0) == PA_ERR_INVALID);
    CHECK(dec(F, 2, 1, 8, 2, 64, 128, 0.088f, 256, 6, 8, 1, nullptr, 0) == PA_ERR_UNSUPPORTED);
    CHECK(dec(F, 2, 1, 8, 2, 128, 128, 0.088f, 384, 6, 8, 1, nullptr, 0) == PA_ERR_UNSUPPORTED);
    CHECK(dec(F, 2, 1, 8, 2, 128, 128, 0.088f, 256, 6, 8, 2, nullptr, 0) == PA_ERR_WORKSPACE);
    CHECK(dec(F, 2, 1, 8, 2, 128, 128, 0.088f, 256, 6, 8, 2, F, 16) == PA_ERR_WORKSPACE);
    CHECK(dec(F, 4, 300, 96, 8, 128, 128, 0.088f, 512, 64, 512, 2, F, 64) == PA_ERR_WORKSPACE);

    CHECK(pa_fp8_decode_causal(F, FF, FU, FF, FU, FF, FI, FI, F, 2, 512, 96, 8, 128, 128, 0.088f, 512, 64, 128, 2,
                               F, 1024, nullptr) == PA_ERR_WORKSPACE);
    CHECK(pa_fp8_decode_causal(nullptr, FF, FU, FF, FU, FF, FI, FI, F, 2, 2, 8, 2, 128, 128, 0.088f, 256, 6, 8, 0,
                               nullptr, 0, nullptr) == PA_ERR_NULLPTR);
    int32_t* rows = reinterpret_cast<int32_t*>(0x20000);
    CHECK(pa_fp8_decode_debug(F, FF, FU, FF, FU, FF, FI, FI, F, 2, 1, 8, 2, 128, 128, 0.088f, 256, 6, 8, 0, nullptr,
                              0, rows, nullptr, nullptr) == PA_ERR_NULLPTR);
    CHECK(pa_fp8_decode_noalloc(F, FF, FU, FF, FU, FF, FI, FI, F, 64, 1, 64, 1, 128, 128, 0.088f, 256, 1024, 8, 64,
                                nullptr) == PA_ERR_WORKSPACE);
    CHECK(pa_fp8_decode_noalloc(F, nullptr, FU, FF, FU, FF, FI, FI, F, 2, 1, 8, 2, 128, 128, 0.088f, 256, 6, 8, 0,
                                nullptr) == PA_ERR_NULLPTR);

    CHECK(pa_fp8_mla_workspace_size(16, 1, 128, 2048, 512, &n) == PA_OK && n > 0);
    CHECK(pa_fp8_mla_workspace_size(16, 1, 128, 2048, 1024, &n) == PA_ERR_UNSUPPORTED);
    CHECK(pa_fp8_mla_sparse_decode(F, F, FU, FI, FI, FI, F, 2, 1, 64, 4, 512, 128, 8, 16, 0.04f, 512, F, 1u << 30,
                                   nullptr) == PA_ERR_UNSUPPORTED);
    CHECK(pa_fp8_mla_sparse_decode(F, F, FU, FI, FI, FI, F, 2, 1, 64, 3, 512, 128, 8, 16, 0.04f, 512, F, 1u << 30,
                                   nullptr) == PA_ERR_INVALID);
    CHECK(pa_fp8_mla_sparse_decode(F, F, FU, FI, FI, FI, F, 2, 1, 64, 2, 512, 128, 8, 16, 0.04f, 512, nullptr, 0,
                                   nullptr) == PA_ERR_WORKSPACE);
    CHECK(pa_fp8_mla_sparse_decode_kv_split(F, F, FU, F, nullptr, FI, FI, FI, F, 2, 1, 64, 2, 512, 128, 8, 16, 0.04f,
                                            512, F, 1u << 30, nullptr) == PA_ERR_NULLPTR);

    CHECK(pa_fp8_scatter_kv_cache(FU, FU, reinterpret_cast<uint8_t*>(F), reinterpret_cast<uint8_t*>(F), F, FF,
                                  reinterpret_cast<float*>(F), 0, 8, 128, 128, 2, 16, 32, 1, 1024, 1024, 8,
                                  1, nullptr) == PA_ERR_INVALID);
    CHECK(pa_fp8_scatter_kv_cache(FU, FU, reinterpret_cast<uint8_t*>(F), reinterpret_cast<uint8_t*>(F), F, FF,
                                  reinterpret_cast<float*>(F), 4, 8, 120, 128, 2, 16, 32, 1, 960, 1024, 8, 1,
                                  nullptr) == PA_ERR_UNSUPPORTED);
    CHECK(pa_fp8_kv_compress_epilog_workspace_size(4, 256, 2, 16, 323, 16 * 323, 64, 1, &n) == PA_OK && n == 0);
    CHECK(pa_fp8_kv_compress_epilog_workspace_size(4, 256, 2, 16, 322, 16 * 323, 64, 1, &n) == PA_ERR_INVALID);
    CHECK(pa_fp8_kv_compress_epilog(reinterpret_cast<uint8_t*>(F), F, F, 4, 256, 2, 16, 323, 16 * 323, 32, 64, 2, 1,
                                    1.f, nullptr, 0, nullptr) == PA_ERR_UNSUPPORTED);
    CHECK(std::strcmp(pa_fp8_last_error_string(), pa_fp8_last_error()) == 0);
    CHECK(std::strncmp(pa_fp8_version(), "pa_fp8", 6) == 0);
    std::printf("ok\n");
    return 0;
}
