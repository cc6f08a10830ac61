/*
 * condensate.h -- C ABI of the MI355X (gfx950) condensate-attention library.
 *
 * The operation (pages of "The Condensate Theorem: Transformers Are O(n), Not O(n^2)",
 * arXiv:2602.06317; section names are those of the metaphor-xennon blog page on it):
 *   for each causal query at position i, with scores S_ij = q_i . k_j / sqrt(d), j <= i
 *   (section 1.1 equation; section 2.1, S = QK^T/sqrt(d_k)),
 *     C_i = {0} u {i-W+1 .. i} u Top-k_i(S_i)         (section 2.1, Definition 1)
 *   where the top-k part ranks the positions R_i = {1 .. i-W} outside the anchor and the window
 *   (section 2.2.3; disjoint parts as counted in the section 4.2.1 table), takes all of R_i when
 *   |R_i| < k, and breaks equal scores toward the smaller position; then
 *     out_i = sum_{j in C_i} softmax_{C_i}(S_i)_j v_j  (section 2.3, Theorem 1's Attention_C)
 *   |C_i| = min(i+1, 1+W+k) <= 1+W+k                  (section 2.4, Corollary 2).
 * The two stages of the section 5.2.2 sketch, identify_condensate and
 * flash_attention_on_subset, are exported separately as well.
 *
 * Layouts (all contiguous, row-major; element type float32 or bfloat16, one type for q, k, v):
 *   q        [batch][heads][nq][d]       query rows are the LAST nq positions: row r sits at
 *                                        position i = n - nq + r
 *   k, v     [batch][kv_heads][n][d]     query head h reads KV head h / (heads / kv_heads)
 *   out      [batch][heads][nq][d]       float32 (fp32-accumulated result)
 *   out_idx  [batch][heads][nq][1+W+topk] int32, C_i in ascending order, padded with -1
 *
 * Ownership and errors:
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library never keeps one
 *     after a call returns and never frees caller memory.
 *   - Arguments are validated on the host before any HIP call; a bad argument returns
 *     CA_ERR_INVALID_ARG or CA_ERR_UNSUPPORTED and launches nothing. HIP failures return
 *     CA_ERR_HIP. ca_last_error() gives a thread-local message for the last failure.
 *   - The *_ex / select / subset entry points are asynchronous on the given stream (a
 *     hipStream_t passed as void*, NULL = the default stream); they return after enqueuing.
 *   - Nothing is thrown across this ABI. Calls on different streams may run concurrently as
 *     long as they do not share a workspace.
 *
 * Supported: d in {64, 128}; n < 2^31; batch * heads * nq < 2^31; heads % kv_heads == 0; W >= 1;
 * 0 <= topk <= 512; 1 + W + topk <= CA_MAX_SET.
 */
#ifndef CONDENSATE_H
#define CONDENSATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CA_MAX_SET 4096

typedef enum {
    CA_OK = 0,
    CA_ERR_INVALID_ARG = -1,  /* null pointer, size out of range, inconsistent heads */
    CA_ERR_UNSUPPORTED = -2,  /* valid but not implemented (d, dtype, set size) */
    CA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than ca_workspace_size() */
    CA_ERR_HIP = -4           /* a HIP runtime call or kernel launch failed */
} ca_status;

typedef enum { CA_F32 = 0, CA_BF16 = 1 } ca_dtype;

typedef struct {
    int32_t batch;     /* independent sequences, >= 1 */
    int32_t heads;     /* query heads */
    int32_t kv_heads;  /* key/value heads; heads % kv_heads == 0 (GQA when smaller) */
    int32_t d;         /* head dimension: 64 or 128 */
    int64_t n;         /* keys in the cache: positions 0..n-1 */
    int64_t nq;        /* queries: the last nq positions, 1 <= nq <= n (1 = decode step) */
    int32_t W;         /* local window length, >= 1 (the window includes position i) */
    int32_t topk;      /* dynamic top-k size, >= 0 */
    int32_t dtype;     /* ca_dtype of q, k, v */
    int32_t chunk;     /* scoring strategy. 0 = automatic: bf16 problems with many query
                          vectors per KV head take the matrix-core passes; decode-shaped
                          problems (topk <= 256 and a fallback key buffer of 4 bytes per query
                          vector and cache row within 1 GiB) take two kernels: one streams K
                          once and keeps a record of each block of 256 rows per query vector
                          (its four best rows and a bound on the rest), the other selects from
                          the records, assembles C_i and attends, one workgroup per query
                          vector; anything else the chunked select below with 256-row chunks.
                          256, 512 or 1024 = always the chunked select (one pass that keeps
                          running top-k lists per chunk of that many key rows; a hint: halved
                          while its buffers would exceed 64 KiB of LDS). Results do not depend
                          on it. */
} ca_params;

/* The one-call form, as the method is usually stated: float32 q/k/v, batch 1, every position
 * is a query (nq = n: causal self-attention over n tokens), default stream, synchronous.
 * Allocates and frees its own workspace. q: [heads][n][d]; k, v: [kv_heads][n][d];
 * out: [heads][n][d] float32; out_idx: [heads][n][1+W+topk] int32. */
int ca_condensate_attention(const void *q, const void *k, const void *v, int64_t n, int32_t d,
                            int32_t heads, int32_t kv_heads, int32_t W, int32_t topk,
                            float *out, int32_t *out_idx);

/* Bytes of device workspace that ca_condensate_attention_ex / ca_condensate_select /
 * ca_condensate_attention_mass_ex need for problem p (may be 0). Host only. The workspace needs
 * no initialisation and may serve any sequence of problems whose size it covers: each call
 * writes what it reads, or clears it, on the call's stream. Calls that share a workspace must
 * be ordered (same stream, or events).
 * Size: on decode-shaped problems 32 bytes per (query vector, block of 256 cache rows) for the
 * block records, plus 4 bytes per query vector and cache row for the exact fallback's keys
 * (written only when a query's candidates exceed what the kernel holds in LDS: exact ties at
 * the threshold, dense clusters of high scores): 16.5 MiB at 131,072 rows and 32 query vectors,
 * 528 MiB at 1,048,576 rows and 128 query vectors. */
int ca_workspace_size(const ca_params *p, size_t *bytes);

/* Full method, asynchronous on `stream`, caller-provided workspace (ws may be NULL only if
 * ca_workspace_size() reported 0). Writes out and out_idx. */
int ca_condensate_attention_ex(const ca_params *p, const void *q, const void *k, const void *v,
                               float *out, int32_t *out_idx, void *ws, size_t ws_bytes,
                               void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): ca_condensate_attention_ex without a workspace argument. The workspace
 * is a device array of the library (CA_NOSCRATCH_MAX_BYTES, one copy per GPU, held until the
 * process ends); the call allocates nothing and records no profiling events. Problems whose
 * ca_workspace_size() exceeds CA_NOSCRATCH_MAX_BYTES return CA_ERR_UNSUPPORTED before any HIP
 * call (the 131,072-row, 32-query-vector decode step needs 16.5 MiB). Every call on one GPU
 * shares that array and leaves its contents to the next: calls that overlap on one GPU (other
 * streams, other threads) race and must not be issued. Asynchronous on `stream`. */
#define CA_NOSCRATCH_MAX_BYTES (32 * 1024 * 1024)
int ca_condensate_attention_noscratch(const ca_params *p, const void *q, const void *k, const void *v,
                                      float *out, int32_t *out_idx, void *stream);

/* The full method plus the mass diagnostic of the pages (metaphor-xennon blog: section 3.2.2,
 * the weight the full causal softmax puts outside C_i; sections 2.2.1-2.2.3, the parts of C_i):
 * as ca_condensate_attention_ex, and mass[batch][heads][nq][4] float32 (device pointer, owned
 * by the caller) = {eps_i, anchor, window, top-k}: the full-softmax weight of the positions
 * outside C_i, of position 0, of the window positions other than 0, and of the top-k positions
 * (the four sum to 1; fp32 sums, so eps is resolved to about 1e-6 of the candidates' mass). The
 * candidates' part of the full normaliser is summed inside the pass that already scores every
 * candidate row (the decode path's streaming pass, the matrix-core prefill path's bound pass,
 * the chunked path's selection pass). Problems without any candidate row (topk = 0, or no
 * query with i > W) return CA_ERR_UNSUPPORTED before any HIP call. The set and the output are
 * those of ca_condensate_attention_ex, bit for bit. Same workspace. */
int ca_condensate_attention_mass_ex(const ca_params *p, const void *q, const void *k,
                                    const void *v, float *out, int32_t *out_idx, float *mass,
                                    void *ws, size_t ws_bytes, void *stream);

/* Dense causal attention, the baseline of the pages' speed comparison (section 5.1.2, against
 * full attention): for each query, softmax of q . k_j / sqrt(d) over every j <= i, times V, on
 * the matrix cores (bf16 products, fp32 accumulation; the weights enter the V product as bf16).
 * W and topk of p are validated but not used. bfloat16 only, with n * d * 2 bytes per KV head at
 * most 4 GiB (else CA_ERR_UNSUPPORTED); no workspace; asynchronous on `stream`. */
int ca_dense_attention_ex(const ca_params *p, const void *q, const void *k, const void *v,
                          float *out, void *stream);

/* Stage 1 (identify_condensate, section 5.2.2): scores every causal key and writes C_i to
 * out_idx only. Same workspace as the full method. */
int ca_condensate_select(const ca_params *p, const void *q, const void *k, int32_t *out_idx,
                         void *ws, size_t ws_bytes, void *stream);

/* Stage 2 (flash_attention_on_subset, section 5.2.2; the restricted softmax of Theorem 1):
 * for each query, softmax of q . k_j / sqrt(d) over the positions listed in its idx row,
 * times V. idx: [batch][heads][nq][1+W+topk] int32 in any order; entries outside 0..i are
 * treated as padding; a listed position must not repeat. A row with no valid entry gives a
 * zero output row. No workspace. */
int ca_attention_on_subset(const ca_params *p, const void *q, const void *k, const void *v,
                           const int32_t *idx, float *out, void *stream);

/* Measurement hooks (not part of the method). While profiling is on -- a process-wide switch --
 * every kernel this library enqueues is bracketed by two HIP events recorded on the stream it
 * is launched on, so the durations are the kernels' own. ca_profile_start pre-creates events
 * for `reserve_launches` launches (more are created on demand) and clears earlier records.
 * ca_profile_stop turns profiling off, waits for the recorded events, and writes one entry per
 * kernel name (launches, summed milliseconds) into out[0..capacity), setting *count to the
 * number of kernels seen. Not meant to be used from several threads at once. */
typedef struct {
    const char *kernel;  /* static name: "decode_stream", "decode_finish", "score_select",
                            "mfma_bound", "mfma_cand", "mfma_window", "finish", "attend" or
                            "dense" */
    int64_t launches;
    double total_ms;
} ca_kernel_time;

int ca_profile_start(int32_t reserve_launches);
int ca_profile_stop(ca_kernel_time *out, int32_t capacity, int32_t *count);

/* Static text for a status code. */
const char *ca_status_string(int status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char *ca_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CONDENSATE_H */
