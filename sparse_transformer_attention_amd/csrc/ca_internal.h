// Internal declarations shared by the host entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ca {

// Work plan of one call: problem sizes plus the decode-path decomposition.
//
// score_topk works on units = (batch, KV head, query group): up to G query vectors that read
// the same KV head (the g query heads of a GQA group and/or consecutive query rows, ordered
// t = r*g + (h - kvh*g)). A unit's candidate rows {1 .. max (i-W)} are cut into chunks of
// `chunk` rows; workgroup m of the unit's wpu workgroups takes chunks m, m + wpu, ...
//
// Workspace: [nqv][wpu] published k-th keys and [nqv][wpu] published best keys (cleared by the
// library at the start of every call), [nqv][wpu] segment lengths (32-bit words), then at
// lists_offset the segments, [nqv][wpu][topk] 64-bit ranking keys.
struct Plan {
    int B, Hq, Hkv, g, d, W, topk, dtype;
    int64_t n, nq;
    int64_t nqv;          // query vectors: B*Hq*nq
    int cap;              // 1 + W + topk (out_idx row length)
    int64_t rmax;         // last candidate row of the last query: (n-1) - W (may be < 1)
    int G;                // query vectors per unit
    int64_t groups;       // units per KV head: ceil(g*nq / G)
    int64_t units;        // B * Hkv * groups
    bool candidates;      // topk > 0 and some query has a non-empty R_i
    int chunk;            // key rows per chunk
    int rcap;             // running-list capacity per query: 512, 768 or 1536
    int wpu;              // workgroups per unit
    int64_t nwg;          // score_topk workgroups
    int64_t lmax;         // candidate slots per query (wpu * seg)
    int seg;              // keys per segment: topk (score_topk) or kMfmaSeg (MFMA passes)
    size_t slots_offset;  // byte offset of the per-query slot words
    size_t lists_offset;  // byte offset of the lists in the workspace
    size_t ws_bytes;      // total workspace
    // Decode path (decode_stream, then decode_finish reading its block records): blocks of 256
    // rows per unit (nblk, rstride = 256 nblk rows covered), the records [units][G][nblk] of 32
    // bytes at summ_offset and the fallback's scratch keys [units][G][rstride] at scratch_offset
    // (written only for a query whose candidates exceed what LDS holds).
    bool stream;
    // Prefill path with bf16 inputs (mfma_select bound + cand, then finish over the segments):
    // taus [nqv] in the first words of the workspace, the lengths and lists as above with
    // wpu = 4 segments of seg = kMfmaSeg keys per query.
    bool mfma;
    size_t win_offset;    // MFMA path: anchor-and-window partials [nqv][d + 2] floats
    size_t zmass_offset;  // mass diagnostic: [nqv] (MFMA path) or [nqv][wpu] (chunked path)
                          // (reference score, sum) over R_i
    int64_t rstride;
    int nblk;
    // Decode path: the anchor-and-window rows of a query in chunks of kWinChunkRows, one extra
    // decode_stream workgroup each; partials [nqv][win_chunks][d + 2] at win_offset.
    int win_chunks;
    size_t summ_offset, scratch_offset;
};


// Launchers (enqueue only; return the hipError_t of the last launch).
// mass: also each workgroup's softmax sum over its rows of R_i, per query ([nqv][wpu] at
// zmass_offset).
hipError_t launch_score_select(const Plan &pl, const void *q, const void *k, void *ws,
                               hipStream_t s, bool mass = false);
// Merge + set assembly (+ restricted softmax times V when out != nullptr), one workgroup per
// query vector (chunked and MFMA paths).
// mass != nullptr (MFMA path): also [nqv][4] = excluded mass, anchor, window, top-k.
hipError_t launch_finish(const Plan &pl, const void *ws, const void *q, const void *k,
                         const void *v, int32_t *out_idx, float *out, hipStream_t s,
                         float *mass = nullptr);
// Restricted softmax times V on caller-supplied index sets.
hipError_t launch_gather_softmax_av(const Plan &pl, const void *q, const void *k, const void *v,
                                    const int32_t *idx, float *out, hipStream_t s);
size_t topk_lds_bytes(const Plan &pl);
// Decode path, first kernel: every key row scored once; per block of 256 rows and query vector a
// record of its best rows (mass: also the block's softmax sums). With attend, extra workgroups
// at the end of the grid make the anchor-and-window partials.
hipError_t launch_decode_stream(const Plan &pl, const void *q, const void *k, const void *v, void *ws,
                                bool mass, bool attend, hipStream_t s);
// Decode path, second kernel: per query vector the exact top-k' from the records, out_idx and
// (out != nullptr) the restricted softmax times V (mass != nullptr: also the mass diagnostic).
hipError_t launch_decode_finish(const Plan &pl, const void *q, const void *k, const void *v, void *ws,
                                int32_t *out_idx, float *out, float *mass, hipStream_t s);
// Anchor-and-window rows per window workgroup of decode_stream. Small chunks run in the
// stream's tail, where CUs fall idle; decode_finish then only merges their partials.
constexpr int kWinChunkRows = 64;
// Query blocks of 16 per wavefront of the two MFMA passes (16 * QB * kMfmaWaves query vectors per
// workgroup).
// Bound pass, per d. Measured: 3 at d = 64 (more products per operand read, 2 wavefronts per
// SIMD instead of 3) gives 9.0 ms against 8.8 on the 131K prefill; at d = 128, 3 spills.
constexpr int kMfmaQBBound128 = 2;
constexpr int kMfmaQBBound64 = 2;
constexpr int kMfmaQBCand = 4;
// Wavefronts per workgroup of the MFMA passes (they share its LDS tiles). Measured: 8 (half the
// key-row traffic from L2) is slower, 131K prefill candidate pass 9.8 -> 13.0 ms.
constexpr int kMfmaWaves = 4;
// The candidate pass keeps four lists of kMfmaSeg keys per query (one per lane that holds it).
constexpr int kMfmaSeg = 64;
// pass 0: the bound of every query (mass: also its softmax sum over R_i); pass 1: its candidate
// list.
hipError_t launch_mfma_select(const Plan &pl, const void *q, const void *k, void *ws, hipStream_t s,
                              int pass, bool mass = false);
// Dense causal attention (bf16, matrix cores): the baseline the method is measured against.
hipError_t launch_dense_attention(const Plan &pl, const void *q, const void *k, const void *v,
                                  float *out, hipStream_t s);
// Anchor-and-window softmax partials of every query vector into the workspace (MFMA path).
hipError_t launch_mfma_window(const Plan &pl, const void *q, const void *k, const void *v, void *ws,
                              hipStream_t s);


}  // namespace ca
