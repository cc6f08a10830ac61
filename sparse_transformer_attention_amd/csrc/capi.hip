// C ABI of the condensate-attention library: host-side validation, work planning, workspace
// layout and launch sequencing. Every argument check runs on the host before any HIP call.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "ca_internal.h"
#include "condensate.h"

namespace {

// ---- measurement hooks: HIP events around each launch while profiling is on ----------------
enum { K_SCORE = 0, K_FINISH = 1, K_ATTEND = 2, K_BOUND = 3, K_CAND = 4, K_DSTREAM = 5, K_WINDOW = 6,
       K_DENSE = 7, K_DFINISH = 8, K_COUNT = 9 };
const char *const kKernelNames[K_COUNT] = {"score_select", "finish", "attend", "mfma_bound", "mfma_cand",
                                           "decode_stream", "mfma_window", "dense", "decode_finish"};

struct Profiler {
    std::mutex mu;
    bool on = false;
    std::vector<hipEvent_t> pool;
    struct Rec { int kernel; hipEvent_t start, stop; };
    std::vector<Rec> recs;

    hipEvent_t take() {
        if (pool.empty()) {
            hipEvent_t e = nullptr;
            if (hipEventCreate(&e) != hipSuccess) return nullptr;
            return e;
        }
        hipEvent_t e = pool.back();
        pool.pop_back();
        return e;
    }
};
Profiler g_prof;

// Brackets one launch with events when profiling is on.
// Set while ca_condensate_attention_noscratch runs on this thread: its launches are not
// bracketed (creating events on demand could allocate).
thread_local bool t_no_prof = false;

struct ProfScope {
    int kernel;
    hipStream_t s;
    hipEvent_t start = nullptr;
    ProfScope(int k, hipStream_t st) : kernel(k), s(st) {
        if (t_no_prof) return;
        std::lock_guard<std::mutex> lk(g_prof.mu);
        if (!g_prof.on) return;
        start = g_prof.take();
        if (start && hipEventRecord(start, s) != hipSuccess) {
            g_prof.pool.push_back(start);
            start = nullptr;
        }
    }
    void done() {
        if (!start) return;
        std::lock_guard<std::mutex> lk(g_prof.mu);
        hipEvent_t stop = g_prof.take();
        if (stop && hipEventRecord(stop, s) == hipSuccess) {
            g_prof.recs.push_back({kernel, start, stop});
        } else {
            g_prof.pool.push_back(start);
            if (stop) g_prof.pool.push_back(stop);
        }
        start = nullptr;
    }
};

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

constexpr int kMinChunk = 256, kMaxChunk = 1024, kDefaultChunk = 256;
constexpr int kMaxTopk = 512;            // running lists hold topk + chunk <= 1024 keys
constexpr int64_t kTargetBlocks = 1024;  // score_topk workgroups to aim for (4 per CU)
constexpr int kStreamBlockRows = 256;    // key rows per block record of the decode path
constexpr double kStreamKeysMax = 1024.0 * 1024 * 1024;  // key buffer budget (bytes)
constexpr int64_t kMfmaMinVectors = 64;  // query vectors per KV head for the MFMA passes
constexpr int kMfmaMaxTopk = 128;        // classes of the MFMA bound
constexpr int kDecodeMaxTopk = 256;      // selected rows per query the finish kernel holds in LDS

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
    if (p->topk > kMaxTopk)
        return fail(CA_ERR_UNSUPPORTED, "topk %d exceeds %d", p->topk, kMaxTopk);
    if (p->chunk != 0 && (!is_pow2(p->chunk) || p->chunk < kMinChunk || p->chunk > kMaxChunk))
        return fail(CA_ERR_INVALID_ARG, "chunk must be 0 or a power of two in [%d, %d] (got %d)",
                    kMinChunk, kMaxChunk, p->chunk);

    ca::Plan &P = *pl;
    P.B = p->batch; P.Hq = p->heads; P.Hkv = p->kv_heads; P.g = p->heads / p->kv_heads;
    P.d = p->d; P.W = p->W; P.topk = p->topk; P.dtype = p->dtype; P.n = p->n; P.nq = p->nq;
    P.nqv = (int64_t)P.B * P.Hq * P.nq;
    // (32-bit query-vector math in the kernels; grids of one workgroup per query vector.)
    if (P.nqv >= ((int64_t)1 << 31))
        return fail(CA_ERR_UNSUPPORTED, "batch * heads * nq = %lld query vectors exceeds 2^31 - 1",
                    (long long)P.nqv);
    P.cap = 1 + P.W + P.topk;
    P.rmax = (P.n - 1) - P.W;

    const int64_t nvec = (int64_t)P.g * P.nq;  // query vectors per KV head
    const int row_bytes = P.d * (P.dtype == CA_BF16 ? 2 : 4);
    const int gmax = row_bytes > 256 ? 2 : 4;  // register budget of the query slices
    P.G = nvec >= 4 ? 4 : (nvec >= 2 ? 2 : 1);
    if (P.G > gmax) P.G = gmax;
    P.groups = (nvec + P.G - 1) / P.G;
    P.units = (int64_t)P.B * P.Hkv * P.groups;
    P.candidates = P.topk > 0 && P.rmax >= 1;

    // Running-list capacity: 512, 768 or 1536 keys, the smallest that takes k plus one chunk
    // (topk <= 512 and chunk <= 1024, so 1536 always does); the list is cut back to k only when
    // another chunk might not fit. Halve the chunk while the selection buffers exceed 64 KiB of
    // LDS.
    int chunk = p->chunk ? p->chunk : kDefaultChunk;
    for (;;) {
        P.chunk = chunk;
        const int need = P.topk + chunk;
        P.rcap = need <= 512 ? 512 : need <= 768 ? 768 : 1536;
        if (ca::topk_lds_bytes(P) <= 64 * 1024 || chunk <= kMinChunk) break;
        chunk /= 2;
    }
    // Decode-shaped problems stream K once (decode_stream, block records; decode_finish reads
    // them) when the fallback's key buffer stays within kStreamKeysMax; others use the fused
    // score_topk kernel.
    P.stream = false;
    P.mfma = false;
    P.seg = 1;
    P.win_offset = 0;
    P.win_chunks = 0;
    P.zmass_offset = 0;
    // Many bf16 query vectors per KV head: the MFMA passes (bound, then candidate lists in the
    // segment layout of the chunked path: 4 segments of kMfmaSeg keys per query). They address
    // a KV head's key rows with 32-bit byte offsets.
    if (P.candidates && p->chunk == 0 && P.dtype == CA_BF16 && P.topk <= kMfmaMaxTopk &&
        nvec >= kMfmaMinVectors && nvec < ((int64_t)1 << 31) && P.nqv < ((int64_t)1 << 31) &&
        P.n * (int64_t)P.d * 2 <= ((int64_t)1 << 32)) {
        P.mfma = true;
        P.wpu = 4;
        P.seg = ca::kMfmaSeg;
        P.lmax = (int64_t)P.wpu * P.seg;
        P.nwg = 0;
        const size_t slot_bytes = ((size_t)(3 * P.nqv * P.wpu) * sizeof(uint32_t) + 255) & ~(size_t)255;
        P.slots_offset = 0;
        P.lists_offset = P.slots_offset + slot_bytes;
        P.win_offset = (P.lists_offset + (size_t)P.nqv * (size_t)P.lmax * sizeof(uint64_t) + 255) & ~(size_t)255;
        P.zmass_offset = (P.win_offset + (size_t)P.nqv * (size_t)(P.d + 2) * sizeof(float) + 255) & ~(size_t)255;
        P.ws_bytes = P.zmass_offset + (size_t)P.nqv * 2 * sizeof(float);
        return CA_OK;
    }
    if (P.candidates && p->chunk == 0) {
        // Blocks of 256 rows from row 0 cover rows 1..rmax.
        const int64_t nblk = (P.rmax + kStreamBlockRows) / kStreamBlockRows;
        const double kb = (double)P.units * (double)(nblk * kStreamBlockRows) * P.G * 4.0;
        // (Index math of the decode kernels in 32 bits.)
        const int64_t wpb = (nblk + 1) / 2;
        // decode_stream's grid: the key workgroups, then one per query vector and window chunk;
        // workgroups times 512 threads stay below 2^32.
        const int64_t nch = (P.W + 1 + ca::kWinChunkRows - 1) / ca::kWinChunkRows;
        const int64_t stream_wg = P.units * wpb + P.units * P.G * nch;
        if (kb <= kStreamKeysMax && P.units * nblk < ((int64_t)1 << 31) && nvec < ((int64_t)1 << 31) &&
            P.topk <= kDecodeMaxTopk && stream_wg < ((int64_t)1 << 23) &&
            P.units * P.G < ((int64_t)1 << 31)) {
            P.stream = true;
            P.nblk = (int)nblk;
            P.rstride = nblk * kStreamBlockRows;
            P.wpu = 1;
            P.nwg = P.units * wpb;
            P.lmax = 0;
            P.lists_offset = 0;
            auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
            const size_t rq = (size_t)P.units * P.G * (size_t)P.nblk;  // (unit, query, block) records
            P.summ_offset = 0;
            P.scratch_offset = up(P.summ_offset + rq * 2 * sizeof(uint4));
            P.ws_bytes = P.scratch_offset + (size_t)P.units * P.G * (size_t)P.rstride * sizeof(uint32_t);
            P.win_chunks = (int)nch;
            P.win_offset = up(P.ws_bytes);
            P.ws_bytes = P.win_offset + (size_t)P.nqv * P.win_chunks * (size_t)(P.d + 2) * sizeof(float);
            return CA_OK;
        }
    }
    const int64_t nchunks = P.rmax >= 1 ? (P.rmax + chunk - 1) / chunk : 0;
    if (P.units >= kTargetBlocks || nchunks <= 1) {
        P.wpu = 1;
    } else {
        int64_t w = (kTargetBlocks + P.units - 1) / P.units;
        P.wpu = (int)(w < nchunks ? w : nchunks);
    }
    P.nwg = P.wpu > 1 ? P.units * P.wpu : P.units;
    P.seg = P.topk > 0 ? P.topk : 1;
    P.lmax = (int64_t)P.wpu * P.seg;
    if (P.nwg > (int64_t)UINT32_MAX / 256)
        return fail(CA_ERR_UNSUPPORTED, "problem too large for one launch");
    const double list_bytes = (double)P.nqv * (double)P.lmax * 8.0;
    if (list_bytes > 9.0e18) return fail(CA_ERR_UNSUPPORTED, "workspace size overflows");
    const size_t slot_bytes = ((size_t)(3 * P.nqv * P.wpu) * sizeof(uint32_t) + 255) & ~(size_t)255;
    P.slots_offset = 0;
    P.lists_offset = P.slots_offset + slot_bytes;
    P.zmass_offset = (P.lists_offset + (size_t)P.nqv * (size_t)P.lmax * sizeof(uint64_t) + 255) & ~(size_t)255;
    P.ws_bytes = P.candidates ? P.zmass_offset + (size_t)P.nqv * (size_t)P.wpu * 2 * sizeof(float) : 0;
    if (ca::topk_lds_bytes(P) > 64 * 1024)
        return fail(CA_ERR_UNSUPPORTED, "selection buffers exceed the LDS budget");
    return CA_OK;
}

int check_ws(const ca::Plan &pl, void *ws, size_t ws_bytes) {
    if (ws_bytes < pl.ws_bytes)
        return fail(CA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, pl.ws_bytes);
    if (pl.ws_bytes > 0 && !ws) return fail(CA_ERR_WORKSPACE, "workspace pointer is NULL");
    return CA_OK;
}

// Scores and candidate lists, then the merge and set assembly into out_idx; with out != nullptr
// the restricted softmax times V runs in the same (finish) kernel.
int run_path(const ca::Plan &pl, const void *q, const void *k, const void *v, int32_t *out_idx,
             float *out, void *ws, hipStream_t s, float *mass = nullptr) {
    hipError_t e;
    if (pl.candidates && pl.mfma) {
        ProfScope pb(K_BOUND, s);
        e = ca::launch_mfma_select(pl, q, k, ws, s, 0, mass != nullptr);
        pb.done();
        if (e != hipSuccess) return hip_fail(e, "mfma_select (bound) launch");
        ProfScope pc(K_CAND, s);
        e = ca::launch_mfma_select(pl, q, k, ws, s, 1);
        pc.done();
        if (e != hipSuccess) return hip_fail(e, "mfma_select (candidates) launch");
        if (v) {
            ProfScope pw(K_WINDOW, s);
            e = ca::launch_mfma_window(pl, q, k, v, ws, s);
            pw.done();
            if (e != hipSuccess) return hip_fail(e, "mfma_window launch");
        }
    } else if (pl.candidates && pl.stream) {
        // Two kernels: the key stream with its block records, then per query vector the
        // selection, set assembly and attend.
        {
            ProfScope pd(K_DSTREAM, s);
            e = ca::launch_decode_stream(pl, q, k, v, ws, mass != nullptr, out != nullptr, s);
            pd.done();
            if (e != hipSuccess) return hip_fail(e, "decode_stream launch");
        }
        ProfScope pf(K_DFINISH, s);
        e = ca::launch_decode_finish(pl, q, k, v, ws, out_idx, out, mass, s);
        pf.done();
        if (e != hipSuccess) return hip_fail(e, "decode_finish launch");
        return CA_OK;
    } else if (pl.candidates) {
        ProfScope ps(K_SCORE, s);
        e = ca::launch_score_select(pl, q, k, ws, s, mass != nullptr);
        ps.done();
        if (e != hipSuccess) return hip_fail(e, "score_topk launch");
    }
    ProfScope pf(K_FINISH, s);
    e = ca::launch_finish(pl, pl.candidates ? ws : nullptr, q, k, v, out_idx, out, s, mass);
    pf.done();
    if (e != hipSuccess) return hip_fail(e, "finish launch");
    return CA_OK;
}

int run_attend(const ca::Plan &pl, const void *q, const void *k, const void *v,
               const int32_t *idx, float *out, hipStream_t s) {
    ProfScope pa(K_ATTEND, s);
    hipError_t e = ca::launch_gather_softmax_av(pl, q, k, v, idx, out, s);
    pa.done();
    if (e != hipSuccess) return hip_fail(e, "attend launch");
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
    return run_path(pl, q, k, nullptr, out_idx, nullptr, ws, static_cast<hipStream_t>(stream));
}

int ca_attention_on_subset(const ca_params *p, const void *q, const void *k, const void *v,
                           const int32_t *idx, float *out, void *stream) {
    ca::Plan pl;
    int rc = make_plan(p, &pl);
    if (rc != CA_OK) return rc;
    if (!q || !k || !v || !idx || !out) return fail(CA_ERR_INVALID_ARG, "q, k, v, idx and out must be non-NULL");
    return run_attend(pl, q, k, v, idx, out, static_cast<hipStream_t>(stream));
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
    return run_path(pl, q, k, v, out_idx, out, ws, static_cast<hipStream_t>(stream));
}

// ---- the entry point that allocates nothing: the workspace is a device array of this file ----
namespace {

// One copy per GPU, held until the process ends; every call on that GPU shares it.
static __device__ __align__(256) unsigned char scratch[CA_NOSCRATCH_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` per device (null: not yet)

// Device address of this device's copy of `scratch`, looked up on the first call on a device
// with that device current. In host code the array's name is a host-side stand-in, never a
// device address: only the looked-up pointer is passed to kernels.
int scratch_for_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(CA_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(CA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return CA_OK;
}

}  // namespace

int ca_condensate_attention_noscratch(const ca_params *p, const void *q, const void *k, const void *v,
                                      float *out, int32_t *out_idx, void *stream) {
    ca::Plan pl;
    int rc = make_plan(p, &pl);
    if (rc != CA_OK) return rc;
    if (!q || !k || !v || !out || !out_idx)
        return fail(CA_ERR_INVALID_ARG, "q, k, v, out and out_idx must be non-NULL");
    if (pl.ws_bytes > (size_t)CA_NOSCRATCH_MAX_BYTES)
        return fail(CA_ERR_UNSUPPORTED, "the problem needs %zu bytes of workspace, more than the %d of the "
                                        "library's device array", pl.ws_bytes, CA_NOSCRATCH_MAX_BYTES);
    void *ws = nullptr;
    if (pl.ws_bytes > 0 && (rc = scratch_for_current_device(&ws)) != CA_OK) return rc;
    t_no_prof = true;
    rc = run_path(pl, q, k, v, out_idx, out, ws, static_cast<hipStream_t>(stream));
    t_no_prof = false;
    return rc;
}

int ca_condensate_attention_mass_ex(const ca_params *p, const void *q, const void *k,
                                    const void *v, float *out, int32_t *out_idx, float *mass,
                                    void *ws, size_t ws_bytes, void *stream) {
    ca::Plan pl;
    int rc = make_plan(p, &pl);
    if (rc != CA_OK) return rc;
    if (!pl.candidates)
        return fail(CA_ERR_UNSUPPORTED, "the mass diagnostic needs a scoring pass: some query with candidates "
                                        "(topk > 0 and i > W)");
    if (!q || !k || !v || !out || !out_idx || !mass)
        return fail(CA_ERR_INVALID_ARG, "q, k, v, out, out_idx and mass must be non-NULL");
    if ((rc = check_ws(pl, ws, ws_bytes)) != CA_OK) return rc;
    return run_path(pl, q, k, v, out_idx, out, ws, static_cast<hipStream_t>(stream), mass);
}

int ca_dense_attention_ex(const ca_params *p, const void *q, const void *k, const void *v,
                          float *out, void *stream) {
    ca::Plan pl;
    int rc = make_plan(p, &pl);
    if (rc != CA_OK) return rc;
    if (pl.dtype != CA_BF16)
        return fail(CA_ERR_UNSUPPORTED, "dense attention runs on the matrix cores: bfloat16 inputs only");
    if (pl.n * (int64_t)pl.d * 2 > ((int64_t)1 << 32))
        return fail(CA_ERR_UNSUPPORTED, "dense attention addresses a KV head's rows in 32 bits: n * d * 2 bytes must be at most 4 GiB");
    if (!q || !k || !v || !out) return fail(CA_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    ProfScope pd(K_DENSE, s);
    hipError_t e = ca::launch_dense_attention(pl, q, k, v, out, s);
    pd.done();
    if (e != hipSuccess) return hip_fail(e, "dense attention launch");
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

int ca_profile_start(int32_t reserve_launches) {
    if (reserve_launches < 0) return fail(CA_ERR_INVALID_ARG, "reserve_launches must be >= 0");
    std::lock_guard<std::mutex> lk(g_prof.mu);
    for (auto &r : g_prof.recs) {
        g_prof.pool.push_back(r.start);
        g_prof.pool.push_back(r.stop);
    }
    g_prof.recs.clear();
    while ((int64_t)g_prof.pool.size() < 2 * (int64_t)reserve_launches) {
        hipEvent_t e = nullptr;
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return hip_fail(err, "hipEventCreate");
        g_prof.pool.push_back(e);
    }
    g_prof.recs.reserve(reserve_launches);
    g_prof.on = true;
    return CA_OK;
}

int ca_profile_stop(ca_kernel_time *out, int32_t capacity, int32_t *count) {
    if (!count || (capacity > 0 && !out)) return fail(CA_ERR_INVALID_ARG, "out/count must be non-NULL");
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.on = false;
    int64_t launches[K_COUNT] = {};
    double ms[K_COUNT] = {};
    int rc = CA_OK;
    for (auto &r : g_prof.recs) {
        if (rc == CA_OK) {
            hipError_t e = hipEventSynchronize(r.stop);
            float t = 0.f;
            if (e == hipSuccess) e = hipEventElapsedTime(&t, r.start, r.stop);
            if (e != hipSuccess) rc = hip_fail(e, "reading profile events");
            launches[r.kernel] += 1;
            ms[r.kernel] += t;
        }
        g_prof.pool.push_back(r.start);
        g_prof.pool.push_back(r.stop);
    }
    g_prof.recs.clear();
    int n = 0;
    for (int kid = 0; kid < K_COUNT; ++kid) {
        if (!launches[kid]) continue;
        if (n < capacity) out[n] = {kKernelNames[kid], launches[kid], ms[kid]};
        ++n;
    }
    *count = n;
    return rc;
}

}  // extern "C"
