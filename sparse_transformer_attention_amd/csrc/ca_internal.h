// Internal declarations shared by the host entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ca {

// Work plan of one call: problem sizes plus the decode-path decomposition.
//
// Score-and-select ("stage 1a") runs on a grid of (chunk, query group, batch*kv_head).
// A query group is up to G query vectors that read the same KV head: the g query heads of a
// GQA group and/or consecutive query rows, ordered t = r*g + (h - kvh*g). A chunk is `chunk`
// consecutive key rows of the candidate range {1 .. (n-1)-W} (the union of every query's R_i).
// Each (query, chunk) pair leaves min(topk, |chunk & R_i|) keys in the candidate workspace.
struct Plan {
    int B, Hq, Hkv, g, d, W, topk, dtype;
    int64_t n, nq;
    int64_t nqv;          // query vectors: B*Hq*nq
    int cap;              // 1 + W + topk (out_idx row length)
    int64_t rmax;         // last candidate row of the last query: (n-1) - W (may be < 1)
    int G;                // query vectors per score-and-select workgroup
    int64_t groups;       // query groups per KV head: ceil(g*nq / G)
    int chunk;            // key rows per chunk
    int64_t nchunks;      // chunks over rows 1..rmax (0 if rmax < 1)
    size_t cand_bytes;    // candidate keys: nqv * nchunks * topk * 8
    size_t ws_bytes;      // total workspace
};

// Launchers (enqueue only; return the hipError_t of the launch).
hipError_t launch_score_select(const Plan &pl, const void *q, const void *k, uint64_t *cand,
                               hipStream_t s);
hipError_t launch_merge_assemble(const Plan &pl, const uint64_t *cand, int32_t *out_idx,
                                 hipStream_t s);
hipError_t launch_gather_softmax_av(const Plan &pl, const void *q, const void *k, const void *v,
                                    const int32_t *idx, float *out, hipStream_t s);

}  // namespace ca
