// Host program that runs the C ABI's host-side validation and planning under AddressSanitizer
// and UndefinedBehaviorSanitizer, without a GPU: ca_workspace_size over valid shapes, limits and
// a pseudo-random sweep of in- and out-of-range parameters (sizes up to 2^40, where the size
// arithmetic would overflow if it were done carelessly), and every entry point's argument checks,
// which must fail before any HIP call. Exit status 0 when every status is one of the documented
// codes and the expected ones came back.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "condensate.h"

static int failures = 0;
#define CHECK(c)                                                               \
    do {                                                                       \
        if (!(c)) {                                                            \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                        \
        }                                                                      \
    } while (0)

static ca_params P(int32_t batch, int32_t heads, int32_t kv, int32_t d, int64_t n, int64_t nq,
                   int32_t W, int32_t topk, int32_t dtype, int32_t chunk) {
    ca_params p;
    p.batch = batch; p.heads = heads; p.kv_heads = kv; p.d = d; p.n = n; p.nq = nq;
    p.W = W; p.topk = topk; p.dtype = dtype; p.chunk = chunk;
    return p;
}

static bool documented(int rc) {
    return rc == CA_OK || rc == CA_ERR_INVALID_ARG || rc == CA_ERR_UNSUPPORTED ||
           rc == CA_ERR_WORKSPACE || rc == CA_ERR_HIP;
}

static uint64_t rng = 0x243F6A8885A308D3ull;
static uint64_t next() {
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return rng;
}
static int64_t pick(const int64_t *v, int n) { return v[next() % (uint64_t)n]; }

int main() {
    size_t bytes = 0;
    // Valid shapes of every path: decode, prefill (MFMA and chunked), fp32, 1M batch 4.
    const ca_params ok[] = {
        P(1, 32, 8, 128, 131072, 1, 256, 64, CA_BF16, 0),
        P(1, 32, 32, 128, 32768, 4096, 256, 64, CA_BF16, 0),
        P(1, 8, 8, 64, 131072, 131072, 64, 32, CA_BF16, 0),
        P(4, 32, 8, 128, 1048576, 1, 256, 128, CA_BF16, 0),
        P(1, 4, 1, 64, 1000, 1000, 16, 8, CA_F32, 0),
        P(1, 4, 1, 128, 8192, 1, 128, 32, CA_F32, 256),
        P(2, 8, 2, 64, 1, 1, 1, 0, CA_BF16, 0),
    };
    for (const ca_params &p : ok) {
        const int rc = ca_workspace_size(&p, &bytes);
        CHECK(rc == CA_OK);
    }
    // Argument errors.
    CHECK(ca_workspace_size(nullptr, &bytes) == CA_ERR_INVALID_ARG);
    CHECK(ca_workspace_size(&ok[0], nullptr) == CA_ERR_INVALID_ARG);
    const ca_params bad[] = {
        P(0, 32, 8, 128, 131072, 1, 256, 64, CA_BF16, 0),      // batch 0
        P(1, 30, 8, 128, 131072, 1, 256, 64, CA_BF16, 0),      // heads % kv_heads
        P(1, 32, 0, 128, 131072, 1, 256, 64, CA_BF16, 0),      // kv_heads 0
        P(1, 32, 8, 128, 0, 1, 256, 64, CA_BF16, 0),           // n 0
        P(1, 32, 8, 128, 100, 101, 16, 8, CA_BF16, 0),         // nq > n
        P(1, 32, 8, 128, 100, 0, 16, 8, CA_BF16, 0),           // nq 0
        P(1, 32, 8, 128, 100, 1, 0, 8, CA_BF16, 0),            // W 0
        P(1, 32, 8, 128, 100, 1, 16, -1, CA_BF16, 0),          // topk < 0
        P(1, 32, 8, 128, 100, 1, 16, 8, CA_BF16, 300),         // chunk
        P(-1, 32, 8, 128, 100, 1, 16, 8, CA_BF16, 0),          // batch < 0
        P(1, 32, 8, 128, -5, 1, 16, 8, CA_BF16, 0),            // n < 0
    };
    for (const ca_params &p : bad) CHECK(ca_workspace_size(&p, &bytes) == CA_ERR_INVALID_ARG);
    const ca_params unsupported[] = {
        P(1, 32, 8, 96, 100, 1, 16, 8, CA_BF16, 0),        // d 96
        P(1, 32, 8, 128, 100, 1, 16, 8, 7, 0),             // dtype 7
        P(1, 32, 8, 128, 10000, 1, 4000, 200, CA_BF16, 0), // 1 + W + topk > CA_MAX_SET
        P(1, 32, 8, 128, 10000, 1, 16, 600, CA_BF16, 0),   // topk > 512
    };
    for (const ca_params &p : unsupported) CHECK(ca_workspace_size(&p, &bytes) == CA_ERR_UNSUPPORTED);
    // Pseudo-random sweep, sizes up to 2^40: every status documented, no undefined behaviour.
    const int64_t ns[] = {1, 2, 255, 256, 257, 4096, 131072, 1048576, (int64_t)1 << 31,
                          ((int64_t)1 << 31) + 1, (int64_t)1 << 36, (int64_t)1 << 40, -1, 0};
    const int64_t hs[] = {1, 2, 4, 8, 32, 64, 128, 4096, 65536, 1 << 24, 0x7FFFFFFF, 0, -3};
    const int64_t ws[] = {1, 2, 63, 64, 256, 1024, 3000, 4095, 4096, 0x7FFFFFFF, 0, -1};
    const int64_t ks[] = {0, 1, 32, 64, 128, 129, 256, 257, 512, 513, 4096, 0x7FFFFFFF, -1};
    const int64_t ds[] = {64, 128, 32, 0, -64, 256};
    const int64_t dts[] = {CA_F32, CA_BF16, 2, -1};
    const int64_t cs[] = {0, 0, 0, 256, 512, 1024, 128, -1};
    int counts[5] = {0, 0, 0, 0, 0};
    for (int it = 0; it < 200000; ++it) {
        const int64_t n = pick(ns, 14);
        int64_t nq = next() % 3 == 0 ? n : pick(ns, 14);
        const int32_t kv = (int32_t)pick(hs, 13);
        const int32_t g = (int32_t)pick(hs, 6);
        const int32_t heads = next() % 5 == 0 ? (int32_t)pick(hs, 13) : (int32_t)((int64_t)kv * g);
        ca_params p = P((int32_t)pick(hs, 6), heads, kv, (int32_t)pick(ds, 6), n, nq, (int32_t)pick(ws, 12),
                        (int32_t)pick(ks, 13), (int32_t)pick(dts, 4), (int32_t)pick(cs, 8));
        const int rc = ca_workspace_size(&p, &bytes);
        CHECK(documented(rc));
        CHECK(rc != CA_ERR_HIP && rc != CA_ERR_WORKSPACE);
        counts[-rc] += 1;
    }
    std::printf("sweep: ok %d, invalid %d, unsupported %d\n", counts[0], counts[1], counts[2]);
    CHECK(counts[0] > 0 && counts[1] > 0 && counts[2] > 0);
    // Entry points: argument and workspace errors come back before any HIP call.
    const ca_params &p = ok[0];
    CHECK(ca_workspace_size(&p, &bytes) == CA_OK && bytes > 0);
    void *fake = reinterpret_cast<void *>(static_cast<uintptr_t>(256));  // never dereferenced
    float *fo = static_cast<float *>(fake);
    int32_t *fi = static_cast<int32_t *>(fake);
    CHECK(ca_condensate_attention_ex(&p, nullptr, fake, fake, fo, fi, fake, bytes, nullptr) == CA_ERR_INVALID_ARG);
    CHECK(ca_condensate_attention_ex(&p, fake, fake, fake, fo, nullptr, fake, bytes, nullptr) == CA_ERR_INVALID_ARG);
    CHECK(ca_condensate_attention_ex(&p, fake, fake, fake, fo, fi, fake, bytes - 1, nullptr) == CA_ERR_WORKSPACE);
    CHECK(ca_condensate_attention_ex(&p, fake, fake, fake, fo, fi, nullptr, bytes, nullptr) == CA_ERR_WORKSPACE);
    CHECK(ca_condensate_attention_ex(&bad[1], fake, fake, fake, fo, fi, fake, bytes, nullptr) == CA_ERR_INVALID_ARG);
    CHECK(ca_condensate_attention_mass_ex(&p, fake, fake, fake, fo, fi, nullptr, fake, bytes, nullptr) == CA_ERR_INVALID_ARG);
    CHECK(ca_condensate_attention_mass_ex(&p, fake, fake, fake, fo, fi, fo, fake, bytes - 1, nullptr) == CA_ERR_WORKSPACE);
    const ca_params no_candidates = P(1, 32, 8, 128, 131072, 1, 256, 0, CA_BF16, 256);  // topk = 0
    CHECK(ca_condensate_attention_mass_ex(&no_candidates, fake, fake, fake, fo, fi, fo, fake, (size_t)1 << 40, nullptr) == CA_ERR_UNSUPPORTED);
    CHECK(ca_condensate_select(&p, nullptr, fake, fi, fake, bytes, nullptr) == CA_ERR_INVALID_ARG);
    CHECK(ca_condensate_select(&p, fake, fake, fi, fake, bytes - 1, nullptr) == CA_ERR_WORKSPACE);
    CHECK(ca_attention_on_subset(&p, fake, fake, fake, nullptr, fo, nullptr) == CA_ERR_INVALID_ARG);
    CHECK(ca_attention_on_subset(&bad[0], fake, fake, fake, fi, fo, nullptr) == CA_ERR_INVALID_ARG);
    const ca_params f32 = P(1, 4, 1, 64, 1000, 1000, 16, 8, CA_F32, 0);
    CHECK(ca_dense_attention_ex(&f32, fake, fake, fake, fo, nullptr) == CA_ERR_UNSUPPORTED);
    CHECK(ca_dense_attention_ex(&p, nullptr, fake, fake, fo, nullptr) == CA_ERR_INVALID_ARG);
    const ca_params huge = P(4, 32, 8, 128, 1048576, 1, 256, 128, CA_BF16, 0);  // 528 MiB workspace
    CHECK(ca_condensate_attention_noscratch(&huge, fake, fake, fake, fo, fi, nullptr) == CA_ERR_UNSUPPORTED);
    CHECK(ca_condensate_attention_noscratch(&p, nullptr, fake, fake, fo, fi, nullptr) == CA_ERR_INVALID_ARG);
    CHECK(ca_condensate_attention(nullptr, fake, fake, 100, 64, 2, 1, 16, 8, fo, fi) == CA_ERR_INVALID_ARG);
    CHECK(ca_condensate_attention(fake, fake, fake, 100, 96, 2, 1, 16, 8, fo, fi) == CA_ERR_UNSUPPORTED);
    // Status strings and the last error are plain static / thread-local text.
    for (int s = 0; s >= -5; --s) CHECK(ca_status_string(s) != nullptr && std::strlen(ca_status_string(s)) > 0);
    CHECK(ca_last_error() != nullptr && std::strlen(ca_last_error()) > 0);
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("capi exercise: all checks passed\n");
    return 0;
}
