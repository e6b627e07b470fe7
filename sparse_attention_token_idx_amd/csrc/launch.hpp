// Kernel launchers of libdsaidx (internal; the C-ABI in api.cpp validates and calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsaidx {

// Offset (in floats) of score row t in a sequence's triangular block of the prefill score
// workspace: row t holds kRowQuant * (t / kRowQuant + 1) scores (whole key tiles of the
// scoring kernel), rows packed back to back.  A sequence of L rows takes tri_row_offset(L).
constexpr int64_t kRowQuant = 128;
__host__ __device__ inline int64_t tri_row_offset(int64_t t) {
    const int64_t q = t / kRowQuant, r = t % kRowQuant;
    return kRowQuant * kRowQuant / 2 * q * (q + 1) + kRowQuant * r * (q + 1);
}

// ---- projections (project.hip).  ws (16-byte aligned) holds project_workspace(T) bytes:
// for T <= kSkinnyT the split-K path's fp32 partial sums, for larger T W_q transposed.
constexpr int64_t kSkinnyT = 64;
size_t project_workspace(int64_t T);
hipError_t launch_project(const uint16_t *x, int64_t ldx, const uint16_t *c_q, int64_t ldc,
                          int64_t T, const uint16_t *W_q, const uint16_t *W_k,
                          const uint16_t *W_w, const uint16_t *gamma, const uint16_t *beta,
                          float eps, uint16_t *q, uint16_t *k_base, const int64_t *k_slot,
                          uint16_t *w, float *ws, hipStream_t stream);

// ---- prefill scores (scores.hip).  cu_seqlens == nullptr -> one sequence of T query rows
// at positions pos0 .. pos0 + T - 1 (keys 0 .. pos0 + T - 1 of k); ragged batches start at
// position 0.  seq_base: B + 1 int64 (written here for varlen), out: triangular rows (row t
// at tri_row_offset(t) - tri_row_offset(pos0)), dummy: a row of kRowQuant * ceil((pos0 +
// max_len) / kRowQuant) floats that absorbs the stores of rows past a sequence end and past
// a row's own last key tile.
// launch_project with explicit row strides: of W_q (ldwq) and q (ldq) for the 4,096 q columns
// it computes, of W_w (ldww) and w (ldwo) for the 32 w columns; k_base may be nullptr (no key).
hipError_t launch_project_ex(const uint16_t *x, int64_t ldx, const uint16_t *c_q, int64_t ldc,
                             int64_t T, const uint16_t *W_q, int64_t ldwq, const uint16_t *W_k,
                             const uint16_t *W_w, int64_t ldww, const uint16_t *gamma,
                             const uint16_t *beta, float eps, uint16_t *q, int64_t ldq,
                             uint16_t *k_base, const int64_t *k_slot, uint16_t *w, int64_t ldwo,
                             float *ws, hipStream_t stream);
// The rotary step of the 64-head indexer, in place: dims (2i, 2i+1), i < 32, of every head of q
// (heads x 128 per row, rows ldq apart) and of k (rows ldk apart; either may be nullptr), token
// t at position pos0 + t.
hipError_t launch_rope(uint16_t *q, int64_t ldq, int heads, uint16_t *k, int64_t ldk, int64_t T, int64_t pos0,
                       double theta, hipStream_t stream);
// launch_scores with explicit row strides of q (ldq) and w (ldw) for the 32 heads it scores;
// accumulate: add to the score rows instead of writing them.
hipError_t launch_scores_ex(const uint16_t *q, int64_t ldq, const uint16_t *k, const uint16_t *w, int64_t ldw,
                            bool accumulate, const int32_t *cu_seqlens, int B, int64_t max_len, int64_t T,
                            int64_t pos0, int64_t *seq_base, float *out, float *dummy, hipStream_t stream);
hipError_t launch_scores(const uint16_t *q, const uint16_t *k, const uint16_t *w,
                         const int32_t *cu_seqlens, int B, int64_t max_len, int64_t T, int64_t pos0,
                         int64_t *seq_base, float *out, float *dummy, hipStream_t stream);

// ---- row top-k (topk.hip).  Prefill: rows = T (dense, query row g at position pos0 + g)
// or the packed total (varlen, longest sequence max_len), scores in the triangular layout of
// launch_scores.  Decode: B rows of stride ld (a multiple of 4), row b holding seqlens[b]
// scores.
hipError_t launch_row_topk_prefill(const float *scores, const int32_t *cu_seqlens,
                                   const int64_t *seq_base, int B, int64_t max_len, int64_t pos0,
                                   int64_t rows, int topk, int32_t *idx, float *out_scores,
                                   hipStream_t stream);
hipError_t launch_row_topk_decode(const float *scores, const int32_t *seqlens, int B, int64_t ld,
                                  int64_t nmax, int topk, int32_t *idx, float *out_scores,
                                  hipStream_t stream);

// ---- decode (decode.hip).  Score rows of decode_row_stride(max_seqlen) floats.
__host__ __device__ inline int64_t decode_row_stride(int64_t max_seqlen) {
    return (max_seqlen + 63) / 64 * 64;
}
// Parts of the decode workspace.
struct DecodeWs {
    int64_t *cu;        // [B + 1] prefix sums of the padded cache lengths
    uint64_t *plan;     // [B] per-row threshold plan
    int32_t *cnt;       // candidate counts per piece
    uint64_t *cand;     // candidate lists, flat-indexed
    float *score_buf;   // [B][decode_row_stride(max_seqlen)]
    uint32_t *skey;     // [B][8192] sampled score keys of the plan pass
    uint8_t *q8;        // FP8 path: [B][32][128] query codes
    float *qw;          // FP8 path: [B][32] folded head weights
};
// Bytes of the decode workspace (16-byte aligned base); with w and base, also its parts.
size_t decode_workspace(int B, int max_seqlen, bool fp8, DecodeWs *w = nullptr, void *base = nullptr);
// The 64-head indexer's decode: q [B][64][128], w [B][64]; the workspace as for launch_decode.
hipError_t launch_decode_v32(const uint16_t *q, const uint16_t *w, const uint16_t *k_cache,
                             const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                             int topk, void *ws, int32_t *idx, float *scores, hipStream_t stream);
hipError_t launch_decode(const uint16_t *q, const uint16_t *w, const uint16_t *k_cache,
                         const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                         int topk, void *ws, int32_t *idx, float *scores, hipStream_t stream);

// ---- FP8 key cache (fp8.hip).  Cache rows: 128 E4M3 bytes and one fp32 power-of-two scale.
hipError_t launch_quantize_keys(const uint16_t *k, int64_t ldk, int64_t N, const int64_t *slot, uint8_t *k8,
                                float *kscale, hipStream_t stream);
// The new queries: q8 [B][32][128] codes, qw[b][h] = w[b][h] * 2^eq[b][h].
hipError_t launch_quantize_queries(const uint16_t *q, const uint16_t *w, int B, int heads, uint8_t *q8,
                                   float *qw, hipStream_t stream);
// The 64-head indexer's decode against the FP8 key cache (workspace as for launch_decode_fp8).
hipError_t launch_decode_fp8_v32(const uint16_t *q, const uint16_t *w, const uint8_t *k8, const float *kscale,
                                 const int64_t *start, const int32_t *seqlens, int B, int max_seqlen, int topk,
                                 void *ws, int32_t *idx, float *scores, hipStream_t stream);
hipError_t launch_decode_fp8(const uint16_t *q, const uint16_t *w, const uint8_t *k8, const float *kscale,
                             const int64_t *start, const int32_t *seqlens, int B, int max_seqlen, int topk,
                             void *ws, int32_t *idx, float *scores, hipStream_t stream);

// ---- sparse MLA over the selected tokens (mla.hip).  Workspace: sparse_mla_workspace(T, topk)
// bytes (the splits' partial outputs; 0 when one split per query).
int sparse_mla_splits(int64_t T, int topk);
size_t sparse_mla_workspace(int64_t T, int topk);
hipError_t launch_sparse_mla(const uint16_t *q, const uint16_t *kv, const int32_t *idx, const int64_t *row0,
                             int64_t T, int topk, float scale, uint16_t *o, float *lse, float *ws,
                             hipStream_t stream);

}  // namespace dsaidx
