// C ABI of the condensate-attention library: host-side validation, work planning, workspace
// layout and launch sequencing. Every argument check runs on the host before any HIP call.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "ca_internal.h"
#include "condensate.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(CA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

constexpr int kMinChunk = 256, kMaxChunk = 4096;
constexpr int kKeyLdsBytes = 32 * 1024;  // LDS for one score-and-select workgroup's keys
constexpr int64_t kTargetBlocks = 1024;  // score-and-select workgroups to aim for (256 CUs)

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Validates p and fills the plan. Host only.
int make_plan(const ca_params *p, ca::Plan *pl) {
    if (!p) return fail(CA_ERR_INVALID_ARG, "params is NULL");
    if (p->batch < 1) return fail(CA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", p->batch);
    if (p->heads < 1 || p->kv_heads < 1)
        return fail(CA_ERR_INVALID_ARG, "heads and kv_heads must be >= 1 (got %d, %d)", p->heads, p->kv_heads);
    if (p->heads % p->kv_heads)
        return fail(CA_ERR_INVALID_ARG, "heads (%d) must be a multiple of kv_heads (%d)", p->heads, p->kv_heads);
    if (p->n < 1 || p->n > INT32_MAX)
        return fail(CA_ERR_INVALID_ARG, "n must be in [1, 2^31-1] (got %lld)", (long long)p->n);
    if (p->nq < 1 || p->nq > p->n)
        return fail(CA_ERR_INVALID_ARG, "nq must be in [1, n] (got %lld)", (long long)p->nq);
    if (p->W < 1) return fail(CA_ERR_INVALID_ARG, "W must be >= 1 (got %d)", p->W);
    if (p->topk < 0) return fail(CA_ERR_INVALID_ARG, "topk must be >= 0 (got %d)", p->topk);
    if (p->dtype != CA_F32 && p->dtype != CA_BF16)
        return fail(CA_ERR_UNSUPPORTED, "dtype %d is not supported (0 = float32, 1 = bfloat16)", p->dtype);
    if (p->d != 64 && p->d != 128)
        return fail(CA_ERR_UNSUPPORTED, "head dimension %d is not supported (64 or 128)", p->d);
    if ((int64_t)p->W + p->topk + 1 > CA_MAX_SET)
        return fail(CA_ERR_UNSUPPORTED, "1 + W + topk = %lld exceeds %d", (long long)p->W + p->topk + 1, CA_MAX_SET);
    if (p->chunk != 0 && (!is_pow2(p->chunk) || p->chunk < kMinChunk || p->chunk > kMaxChunk))
        return fail(CA_ERR_INVALID_ARG, "chunk must be 0 or a power of two in [%d, %d] (got %d)",
                    kMinChunk, kMaxChunk, p->chunk);

    ca::Plan &P = *pl;
    P.B = p->batch; P.Hq = p->heads; P.Hkv = p->kv_heads; P.g = p->heads / p->kv_heads;
    P.d = p->d; P.W = p->W; P.topk = p->topk; P.dtype = p->dtype; P.n = p->n; P.nq = p->nq;
    P.nqv = (int64_t)P.B * P.Hq * P.nq;
    P.cap = 1 + P.W + P.topk;
    P.rmax = (P.n - 1) - P.W;

    const int64_t nvec = (int64_t)P.g * P.nq;  // query vectors per KV head
    const int row_bytes = P.d * (P.dtype == CA_BF16 ? 2 : 4);
    const int gmax = row_bytes > 256 ? 2 : 4;  // register budget of the query slices
    P.G = nvec >= 4 ? 4 : (nvec >= 2 ? 2 : 1);
    if (P.G > gmax) P.G = gmax;
    P.groups = (nvec + P.G - 1) / P.G;

    P.chunk = 0;
    P.nchunks = 0;
    P.cand_bytes = 0;
    if (P.topk > 0 && P.rmax >= 1) {
        const int lds_cap = kKeyLdsBytes / (4 * P.G);
        int chunk = p->chunk;
        if (chunk == 0) {
            // Largest chunk that still gives about kTargetBlocks workgroups.
            const int64_t units = (int64_t)P.B * P.Hkv * P.groups;
            chunk = kMaxChunk;
            while (chunk > kMinChunk && units * ((P.rmax + chunk - 1) / chunk) < kTargetBlocks) chunk >>= 1;
        }
        if (chunk > lds_cap) chunk = lds_cap;
        P.chunk = chunk;
        P.nchunks = (P.rmax + chunk - 1) / chunk;
        const int64_t blocks = P.nchunks * P.groups * (int64_t)P.B * P.Hkv;
        if (blocks > (int64_t)UINT32_MAX / 256)
            return fail(CA_ERR_UNSUPPORTED, "problem too large for one launch (%lld workgroups)", (long long)blocks);
        const double bytes = (double)P.nqv * (double)P.nchunks * (double)P.topk * 8.0;
        if (bytes > 9.0e18) return fail(CA_ERR_UNSUPPORTED, "workspace size overflows");
        P.cand_bytes = (size_t)P.nqv * (size_t)P.nchunks * (size_t)P.topk * sizeof(uint64_t);
    }
    if (P.nqv > (int64_t)UINT32_MAX / 256)
        return fail(CA_ERR_UNSUPPORTED, "too many query vectors for one launch (%lld)", (long long)P.nqv);
    P.ws_bytes = P.cand_bytes;
    return CA_OK;
}

int check_ws(const ca::Plan &pl, void *ws, size_t ws_bytes) {
    if (ws_bytes < pl.ws_bytes)
        return fail(CA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, pl.ws_bytes);
    if (pl.ws_bytes > 0 && !ws) return fail(CA_ERR_WORKSPACE, "workspace pointer is NULL");
    return CA_OK;
}

// Stage 1: scores, chunk-local top-k, merge and set assembly into out_idx.
int run_select(const ca::Plan &pl, const void *q, const void *k, int32_t *out_idx, void *ws,
               hipStream_t s) {
    uint64_t *cand = static_cast<uint64_t *>(ws);
    hipError_t e;
    if (pl.nchunks > 0) {
        e = ca::launch_score_select(pl, q, k, cand, s);
        if (e != hipSuccess) return hip_fail(e, "score_select launch");
    }
    e = ca::launch_merge_assemble(pl, cand, out_idx, s);
    if (e != hipSuccess) return hip_fail(e, "merge_assemble launch");
    return CA_OK;
}

}  // namespace

extern "C" {

const char *ca_status_string(int status) {
    switch (status) {
        case CA_OK: return "CA_OK: success";
        case CA_ERR_INVALID_ARG: return "CA_ERR_INVALID_ARG: invalid argument";
        case CA_ERR_UNSUPPORTED: return "CA_ERR_UNSUPPORTED: valid but unsupported problem";
        case CA_ERR_WORKSPACE: return "CA_ERR_WORKSPACE: workspace missing or too small";
        case CA_ERR_HIP: return "CA_ERR_HIP: HIP runtime error";
        default: return "unknown status";
    }
}

const char *ca_last_error(void) { return g_last_error; }

int ca_workspace_size(const ca_params *p, size_t *bytes) {
    if (!bytes) return fail(CA_ERR_INVALID_ARG, "bytes is NULL");
    ca::Plan pl;
    int rc = make_plan(p, &pl);
    if (rc != CA_OK) return rc;
    *bytes = pl.ws_bytes;
    return CA_OK;
}

int ca_condensate_select(const ca_params *p, const void *q, const void *k, int32_t *out_idx,
                         void *ws, size_t ws_bytes, void *stream) {
    ca::Plan pl;
    int rc = make_plan(p, &pl);
    if (rc != CA_OK) return rc;
    if (!q || !k || !out_idx) return fail(CA_ERR_INVALID_ARG, "q, k and out_idx must be non-NULL");
    if ((rc = check_ws(pl, ws, ws_bytes)) != CA_OK) return rc;
    return run_select(pl, q, k, out_idx, ws, static_cast<hipStream_t>(stream));
}

int ca_attention_on_subset(const ca_params *p, const void *q, const void *k, const void *v,
                           const int32_t *idx, float *out, void *stream) {
    ca::Plan pl;
    int rc = make_plan(p, &pl);
    if (rc != CA_OK) return rc;
    if (!q || !k || !v || !idx || !out) return fail(CA_ERR_INVALID_ARG, "q, k, v, idx and out must be non-NULL");
    hipError_t e = ca::launch_gather_softmax_av(pl, q, k, v, idx, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "attend launch");
    return CA_OK;
}

int ca_condensate_attention_ex(const ca_params *p, const void *q, const void *k, const void *v,
                               float *out, int32_t *out_idx, void *ws, size_t ws_bytes,
                               void *stream) {
    ca::Plan pl;
    int rc = make_plan(p, &pl);
    if (rc != CA_OK) return rc;
    if (!q || !k || !v || !out || !out_idx)
        return fail(CA_ERR_INVALID_ARG, "q, k, v, out and out_idx must be non-NULL");
    if ((rc = check_ws(pl, ws, ws_bytes)) != CA_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = run_select(pl, q, k, out_idx, ws, s)) != CA_OK) return rc;
    hipError_t e = ca::launch_gather_softmax_av(pl, q, k, v, out_idx, out, s);
    if (e != hipSuccess) return hip_fail(e, "attend launch");
    return CA_OK;
}

int ca_condensate_attention(const void *q, const void *k, const void *v, int64_t n, int32_t d,
                            int32_t heads, int32_t kv_heads, int32_t W, int32_t topk, float *out,
                            int32_t *out_idx) {
    ca_params p;
    memset(&p, 0, sizeof p);
    p.batch = 1; p.heads = heads; p.kv_heads = kv_heads; p.d = d; p.n = n; p.nq = n;
    p.W = W; p.topk = topk; p.dtype = CA_F32; p.chunk = 0;
    ca::Plan pl;
    int rc = make_plan(&p, &pl);
    if (rc != CA_OK) return rc;
    if (!q || !k || !v || !out || !out_idx)
        return fail(CA_ERR_INVALID_ARG, "q, k, v, out and out_idx must be non-NULL");
    void *ws = nullptr;
    hipError_t e;
    if (pl.ws_bytes > 0) {
        e = hipMalloc(&ws, pl.ws_bytes);
        if (e != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
    }
    rc = ca_condensate_attention_ex(&p, q, k, v, out, out_idx, ws, pl.ws_bytes, nullptr);
    if (rc == CA_OK) {
        e = hipStreamSynchronize(nullptr);
        if (e != hipSuccess) rc = hip_fail(e, "hipStreamSynchronize");
    } else {
        (void)hipStreamSynchronize(nullptr);
    }
    if (ws) {
        e = hipFree(ws);
        if (e != hipSuccess && rc == CA_OK) rc = hip_fail(e, "hipFree(workspace)");
    }
    return rc;
}

}  // extern "C"
