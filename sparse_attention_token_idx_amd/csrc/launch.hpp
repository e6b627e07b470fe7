// Kernel launchers of libdsaidx (internal; the C-ABI in api.cpp validates and calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

namespace dsaidx {

// Host-side set-up done once per device (kernel attributes), safe under concurrent calls from
// several threads: a lock-free check on the fast path, the set-up itself under a mutex.
constexpr int kMaxDevices = 64;
struct DeviceOnce {
    std::atomic<uint8_t> done[kMaxDevices] = {};
    std::mutex mu;
    template <class F> hipError_t run(F &&f) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
        if (done[dev].load(std::memory_order_acquire)) return hipSuccess;
        std::lock_guard<std::mutex> lk(mu);
        if (done[dev].load(std::memory_order_relaxed)) return hipSuccess;
        e = f();
        if (e == hipSuccess) done[dev].store(1, std::memory_order_release);
        return e;
    }
};

// A per-device integer computed on first use (every thread computes the same value, so a
// race only repeats the computation).
struct DeviceInt {
    std::atomic<int> v[kMaxDevices] = {};
    template <class F> int get(F &&f) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return f();
        int x = v[dev].load(std::memory_order_relaxed);
        if (x > 0) return x;
        x = f();
        v[dev].store(x, std::memory_order_relaxed);
        return x;
    }
};

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

// ---- prefill top-k with storage linear in the rows (prefill.hip).
constexpr int64_t kFilterRows = 65536;        // rows of one filter pass (32 heads; 64 heads: half)
constexpr int kListCap = 6144;                // candidates kept per (row, key segment)
constexpr int64_t kSampleBytes = 512LL << 20; // sample rows held at once
// Work split and workspace layout of one prefill call (host side).  rows: T (one sequence
// at positions pos0 ..) or the packed total (ragged batch of B sequences, longest max_len).
struct PrefillPlan {
    int heads;
    bool varlen;
    int64_t rows;
    int B;
    int64_t max_len, pos0;
    int64_t cf;        // rows of a filter chunk
    int64_t lists;     // candidate lists of a filter chunk (rows x key segments)
    int cap;           // entries per list
    int64_t ms;        // floats per sample row
    int64_t cs;        // rows of a sample sub-chunk
    int64_t ld;        // floats per fallback scratch row
    size_t off_hdr, off_theta, off_cnt, off_cand, off_srow, off_fblist, off_nbuf, off_obuf, off_scratch,
        off_dummy, bytes;
};
PrefillPlan prefill_plan(int heads, bool varlen, int64_t rows, int B, int64_t max_len, int64_t pos0);
// Scores and top-k of every row (q rows heads x 128, w rows heads); ws: plan.bytes, 256-byte
// aligned; its first word is the status (bit 0: a ring wait of a score kernel ran out of polls).
hipError_t launch_prefill_topk(const PrefillPlan &p, const uint16_t *q, const uint16_t *k, const uint16_t *w,
                               const int32_t *cu_seqlens, int topk, int32_t *idx, float *scores, void *ws,
                               hipStream_t stream);
// Raw causal score rows, 32 heads (cu_seqlens == nullptr: one sequence of T rows at positions
// pos0 ..; ragged batches start at 0).  seq_base: B + 1 int64 (written here for varlen), out:
// triangular rows (row t at tri_row_offset(t) - tri_row_offset(pos0) from its sequence's base),
// dummy: kRowQuant * ceil((pos0 + max_len) / kRowQuant) floats; status: cleared, then bit 0
// set if a ring wait ran out of polls.
hipError_t launch_scores(const uint16_t *q, const uint16_t *k, const uint16_t *w, const int32_t *cu_seqlens, int B,
                         int64_t max_len, int64_t T, int64_t pos0, int64_t *seq_base, float *out, float *dummy,
                         uint32_t *status, hipStream_t stream);
// Diagnostic timing of the phases of prefill top-k calls (process-wide): while on, every phase
// launch is bracketed by HIP events on its stream; prefill_phase_times synchronizes them and
// returns the summed milliseconds and launch counts per phase (then forgets them).
enum : int { kPhaseSample = 0, kPhaseThreshold = 1, kPhaseFilter = 2, kPhaseSelect = 3, kPhaseFallback = 4,
             kPhases = 5 };
void prefill_phase_timing(bool on);
hipError_t prefill_phase_times(double *ms, int *count, int n);
// Polls allowed per wait on a score kernel's key ring (default 2^20; 0 makes every wait that
// is not already satisfied give up, for tests of the status report).
void prefill_set_wait_budget(int polls);
int prefill_wait_budget();

// launch_project generalised: nq q columns (4,096 or 8,192) and hw w columns (32 or 64), with the
// row strides of W_q (ldwq), q (ldq), W_w (ldww) and w (ldwo); k_base may be nullptr (no key).
// theta > 0 applies the rotary step to dims 0..63 of every q head and of the key, token t at
// position pos0 + t, in the epilogues (the workspace then also holds the (cos, sin) table).
size_t project_workspace(int64_t T, int nq, int hw, bool rope);
hipError_t launch_project_ex(const uint16_t *x, int64_t ldx, const uint16_t *c_q, int64_t ldc,
                             int64_t T, const uint16_t *W_q, int64_t ldwq, int nq, const uint16_t *W_k,
                             const uint16_t *W_w, int64_t ldww, int hw, const uint16_t *gamma,
                             const uint16_t *beta, float eps, uint16_t *q, int64_t ldq,
                             uint16_t *k_base, const int64_t *k_slot, uint16_t *w, int64_t ldwo,
                             int64_t pos0, double theta, float *ws, hipStream_t stream);

// ---- row top-k (topk.hip).  Prefill: rows = T (dense, query row g at position pos0 + g)
// or the packed total (varlen, longest sequence max_len), scores in the triangular layout of
// launch_scores.  Decode: B rows of stride ld (a multiple of 4), row b holding seqlens[b]
// scores.
// status (may be nullptr): when its bit 0 is set (the scoring kernel's ring wait gave up) every
// row is written as index -2, score NaN instead of being selected.
hipError_t launch_row_topk_prefill(const float *scores, const int32_t *cu_seqlens,
                                   const int64_t *seq_base, int B, int64_t max_len, int64_t pos0,
                                   int64_t rows, int topk, int32_t *idx, float *out_scores,
                                   const uint32_t *status, hipStream_t stream);
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

// ---- calibration of the sustained bf16 MFMA rate (calib.hip): kCalibBlocks workgroups of 256
// threads, one float of `sink` per thread.
constexpr int kCalibBlocks = 1024;
int64_t mfma_calibrate_flop(int64_t iters);
hipError_t launch_mfma_calibrate(int64_t iters, int random_operands, float *sink, hipStream_t stream);

}  // namespace dsaidx
