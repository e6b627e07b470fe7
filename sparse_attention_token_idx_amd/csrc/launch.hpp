// Kernel launchers of libdsaidx (internal; the C-ABI in api.cpp validates and calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsaidx {

// Rows of the per-row candidate buffer used by the fused score + top-k kernel.
int candidate_capacity(int topk);

// ---- projections (project.hip)
hipError_t launch_project(const uint16_t *x, int64_t ldx, const uint16_t *c_q, int64_t ldc,
                          int64_t T, const uint16_t *W_q, const uint16_t *W_k,
                          const uint16_t *W_w, const uint16_t *gamma, const uint16_t *beta,
                          float eps, uint16_t *q, uint16_t *k_base, const int64_t *k_slot,
                          uint16_t *w, hipStream_t stream);

// ---- fused causal score + top-k (score_topk.hip).  cu_seqlens == nullptr -> one
// sequence of length T.  cand holds total * cap (key, index) pairs.
hipError_t launch_score_topk(const uint16_t *q, const uint16_t *k, const uint16_t *w,
                             const int32_t *cu_seqlens, int B, int64_t max_len, int64_t T,
                             int topk, int cap, uint32_t *cand_key, int32_t *cand_idx,
                             int32_t *idx, float *scores, hipStream_t stream);

// ---- decode (decode.hip).  score_buf holds B * max_seqlen floats.
hipError_t launch_decode(const uint16_t *q, const uint16_t *w, const uint16_t *k_cache,
                         const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                         int topk, float *score_buf, int32_t *idx, float *scores,
                         hipStream_t stream);

}  // namespace dsaidx
