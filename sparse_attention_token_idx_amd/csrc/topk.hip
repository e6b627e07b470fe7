// Row top-k of fp32 scores: for each row of n scores keep the topk largest, ties broken
// toward the lower index, and list them in ascending index order ("Qwen3.5-397B-A17B vs Kimi
// K3.1 Pro" compare page, sparse/compressed-attention row: each query keeps its top 2,048
// tokens).  Rows come from the prefill score workspace (triangular rows of scores.hip) or
// from the decode score buffer (one row per sequence).
//
// One workgroup of 4 waves per row, several workgroups per CU so that one row's selection
// overlaps other rows' loads.  Thread t handles 16 consecutive scores of each 4,096-score
// chunk (four 16-byte loads), so index order is thread order.
//   * Rows of at most 4,096 scores are held in registers and selected exactly.
//   * Longer rows: a threshold theta0 is placed from a sample of 4,096 scores (64 blocks of
//     64 consecutive scores spread over the row) so that about 1.4 topk keys of the row are
//     expected to reach it: one histogram pass over fine bins counted down from the sample's
//     largest key (2^13 key units per bin, which keeps the LDS atomics spread out) finds
//     the bin that holds the r-th largest sample key, and theta0 is that bin's lower edge.
//     One streaming pass compacts the keys >= theta0 into LDS in index order; when there are
//     between topk and 4,096 of them (the normal case) the exact select runs over those
//     candidates only, on their keys relative to theta0, with only as many 11-bit digit
//     passes as the candidates' key range needs.  Otherwise an exact select streams the
//     whole row (three digit passes) and a last pass writes the result.
// The exact select is a most-significant-digit radix select over the orderable key (11 + 11
// + 10 bits, an LDS histogram per digit): theta = the topk-th largest key, and how many keys
// equal to theta are kept (the lowest-index ones).
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

constexpr int kTkWaves = 4;
constexpr int kTkThreads = 64 * kTkWaves;
constexpr int kPer = 16;                        // scores per thread per chunk
constexpr int kChunk = kTkThreads * kPer;       // 4,096
constexpr int kCand = 4096;                     // candidates kept in LDS
constexpr int kBins = 2048;

struct TopkSmem {
    uint32_t cand_key[kCand];
    int32_t cand_idx[kCand];
    uint32_t hist[kBins];
    int32_t wsum[kTkWaves];
    uint32_t wmax[kTkWaves];
    int32_t bcast[2];
};

struct TopkArgs {
    const float *scores;
    int mode;                      // 0: prefill rows (triangular), 1: decode rows
    const int32_t *cu_seqlens;     // prefill varlen (nullptr: one sequence of length T)
    const int64_t *seq_base;
    int B;
    const int32_t *seqlens;        // decode: row b holds seqlens[b] (clamped to ld) scores
    int64_t ld;                    // decode: row stride
    int topk;
    int32_t *out_idx;
    float *out_score;              // may be nullptr
};

// Inclusive sum over the workgroup of one int per thread (the sum of all in `total`).
__device__ int block_inclusive_sum(int v, int &total, TopkSmem &sm) {
    const int lane = __lane_id(), wave = threadIdx.x >> 6;
    const int incl = wave_inclusive_sum(v);
    if (lane == 63) sm.wsum[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kTkWaves; ++i) {
        const int s = sm.wsum[i];
        before += i < wave ? s : 0;
        all += s;
    }
    __syncthreads();
    total = all;
    return before + incl;
}

// One digit of the radix select: given the histogram of the keys that match the digits
// found so far, return the digit of the need-th largest and subtract from need the keys in
// higher digits.  Thread t owns bins 8t .. 8t+7.
__device__ uint32_t pick_digit(int &need, TopkSmem &sm) {
    const int tid = threadIdx.x;
    int cnt[8], sum = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        cnt[j] = (int)sm.hist[8 * tid + j];
        sum += cnt[j];
    }
    int total;
    const int incl = block_inclusive_sum(sum, total, sm);
    int above = total - incl;   // keys in bins above 8t+7
#pragma unroll
    for (int j = 7; j >= 0; --j) {
        if (above < need && need <= above + cnt[j]) {
            sm.bcast[0] = 8 * tid + j;
            sm.bcast[1] = above;
        }
        above += cnt[j];
    }
    __syncthreads();
    const uint32_t d = (uint32_t)sm.bcast[0];
    need -= sm.bcast[1];
    __syncthreads();
    return d;
}

constexpr int kShift[3] = {21, 10, 0};
constexpr int kWidth[3] = {11, 11, 10};

// Exact select over keys held in registers (kPer per thread, 0 = no key): returns theta, the
// need-th largest key; on return need = how many keys equal to theta are among the need
// largest.
__device__ uint32_t select_regs(const uint32_t (&key)[kPer], int &need, TopkSmem &sm) {
    uint32_t prefix = 0, pmask = 0;
#pragma unroll 1
    for (int p = 0; p < 3; ++p) {
        const int shift = kShift[p];
        const uint32_t dmask = (1u << kWidth[p]) - 1u;
        for (int i = threadIdx.x; i < kBins; i += kTkThreads) sm.hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const uint32_t kv = key[i];
            if (kv != 0u && (kv & pmask) == prefix) atomicAdd(&sm.hist[(kv >> shift) & dmask], 1u);
        }
        __syncthreads();
        prefix |= pick_digit(need, sm) << shift;
        pmask |= dmask << shift;
    }
    return prefix;
}

// Largest of one key per thread over the workgroup.
__device__ uint32_t block_max(uint32_t v, TopkSmem &sm) {
    const int lane = __lane_id(), wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, d, 64);
        v = o > v ? o : v;
    }
    if (lane == 0) sm.wmax[wave] = v;
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kTkWaves; ++i) m = sm.wmax[i] > m ? sm.wmax[i] : m;
    __syncthreads();
    return m;
}

// Exact select over keys >= base held in registers (0 = no key), digits taken from the
// relative key (key - base) < 2^nbits, 11 bits at a time from the top: returns theta, the
// need-th largest key; on return need = how many keys equal to theta are among the need
// largest.
__device__ uint32_t select_rel(const uint32_t (&key)[kPer], uint32_t base, int nbits, int &need,
                               TopkSmem &sm) {
    uint32_t prefix = 0, pmask = 0;
    int hi = nbits;
#pragma unroll 1
    while (hi > 0) {
        const int w = hi < 11 ? hi : 11;
        const int shift = hi - w;
        const uint32_t dmask = (1u << w) - 1u;
        for (int i = threadIdx.x; i < kBins; i += kTkThreads) sm.hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const uint32_t rel = key[i] - base;
            if (key[i] != 0u && (rel & pmask) == prefix) atomicAdd(&sm.hist[(rel >> shift) & dmask], 1u);
        }
        __syncthreads();
        prefix |= pick_digit(need, sm) << shift;
        pmask |= dmask << shift;
        hi = shift;
    }
    return base + prefix;
}

// Writes, in index order, the keys above theta and the first `need` keys equal to theta among
// this thread's kPer keys (indices idx[i], increasing with thread and i); out_base = outputs
// already written and eq_base = keys equal to theta already seen (both block-uniform).
// Returns the number written by the whole workgroup; eq_base advances by the ties seen.
__device__ int emit_ordered(const uint32_t (&key)[kPer], const int32_t (&idx)[kPer], uint32_t theta,
                            int need, int out_base, int &eq_base, int32_t *oi, float *os,
                            TopkSmem &sm) {
    int eqc = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) eqc += key[i] == theta ? 1 : 0;
    int eq_total;
    int eq_rank = eq_base + block_inclusive_sum(eqc, eq_total, sm) - eqc;
    bool keep[kPer];
    int kc = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const bool e = key[i] == theta;
        keep[i] = key[i] > theta || (e && eq_rank < need);
        eq_rank += e ? 1 : 0;
        kc += keep[i] ? 1 : 0;
    }
    int keep_total;
    int pos = out_base + block_inclusive_sum(kc, keep_total, sm) - kc;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (keep[i]) {
            oi[pos] = idx[i];
            if (os) os[pos] = key_score(key[i]);
            ++pos;
        }
    }
    eq_base += eq_total;
    return keep_total;
}

__global__ __launch_bounds__(kTkThreads) void row_topk_kernel(TopkArgs a) {
    __shared__ TopkSmem sm;
    const int64_t g = blockIdx.x;
    const int tid = threadIdx.x;
    const int topk = a.topk;

    // ---- locate the row
    const float *row;
    int64_t n;
    if (a.mode == 0) {
        int64_t t = g, base = 0;
        if (a.cu_seqlens) {
            int lo = 0, hi = a.B - 1;   // last sequence with cu_seqlens[i] <= g
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if ((int64_t)a.cu_seqlens[mid] <= g) lo = mid;
                else hi = mid - 1;
            }
            t = g - a.cu_seqlens[lo];
            base = a.seq_base[lo];
        }
        row = a.scores + base + tri_row_offset(t);
        n = t + 1;
    } else {
        const int64_t L = a.seqlens[g];
        n = L < 0 ? 0 : (L > a.ld ? a.ld : L);
        row = a.scores + g * a.ld;
    }
    int32_t *oi = a.out_idx + g * topk;
    float *os = a.out_score ? a.out_score + g * topk : nullptr;
    if (n <= topk) {
        for (int i = tid; i < topk; i += kTkThreads) {
            const bool in = i < n;
            oi[i] = in ? i : -1;
            if (os) os[i] = in ? row[i] : -INFINITY;
        }
        return;
    }

    // 16 keys from element e0 (4-aligned; rows are padded to a multiple of 64 scores, so a
    // 16-byte group that starts below n lies inside the row)
    auto load16 = [&](int64_t e0, uint32_t (&key)[kPer]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t e = e0 + 4 * q;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (e < n) v = *reinterpret_cast<const f32x4 *>(row + e);
#pragma unroll
            for (int j = 0; j < 4; ++j) key[4 * q + j] = e + j < n ? score_key(v[j]) : 0u;   // 0: no key
        }
    };

    uint32_t key[kPer];
    int32_t kidx[kPer];
    if (n <= kChunk) {
        // ---- short row: all of it in registers
        load16(kPer * tid, key);
#pragma unroll
        for (int i = 0; i < kPer; ++i) kidx[i] = kPer * tid + i;
        int need = topk;
        const uint32_t theta = select_regs(key, need, sm);
        int eq_base = 0;
        emit_ordered(key, kidx, theta, need, 0, eq_base, oi, os, sm);
        return;
    }

    // ---- sample: 64 blocks of 64 consecutive scores spread over the row; thread t reads
    // quarter t % 4 of block t / 4
    {
        const int b = tid >> 2;
        const int64_t start = ((int64_t)b * (n - 64) / 63) & ~(int64_t)3;
        load16(start + 16 * (tid & 3), key);
    }
    // r such that about 1.4 topk keys of the row reach the r-th largest of the sample
    int r = (int)(((int64_t)topk * 7 * kChunk + (int64_t)5 * n - 1) / ((int64_t)5 * n)) + 8;
    if (r > kChunk) r = kChunk;
    uint32_t theta0;
    {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) m = key[i] > m ? key[i] : m;
        const uint32_t top = block_max(m, sm);
        // bins of 2^sb key units counted down from the largest sample key; a second try with
        // bins wide enough to hold every key if the first window holds fewer than r samples
        int sb = 13;
        for (;;) {
            for (int i = tid; i < kBins; i += kTkThreads) sm.hist[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const uint32_t d = (top - key[i]) >> sb;
                if (key[i] != 0u && d < (uint32_t)kBins) atomicAdd(&sm.hist[d], 1u);
            }
            __syncthreads();
            // bins in descending key order are ascending d: the first bin where the running
            // count reaches r (thread t owns bins 8t .. 8t+7)
            int cnt[8], sum = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                cnt[j] = (int)sm.hist[8 * tid + j];
                sum += cnt[j];
            }
            int total;
            int run = block_inclusive_sum(sum, total, sm) - sum;
            if (total >= r) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (run < r && r <= run + cnt[j]) sm.bcast[0] = 8 * tid + j;
                    run += cnt[j];
                }
            }
            __syncthreads();
            if (total >= r || sb >= 21) {
                const int64_t b = total >= r ? sm.bcast[0] : kBins - 1;
                const int64_t lo = (int64_t)top - ((b + 1) << sb) + 1;   // lowest key of bin b
                theta0 = lo < 1 ? 1u : (uint32_t)lo;
                __syncthreads();
                break;
            }
            __syncthreads();
            sb = 21;
        }
    }

    // ---- one streaming pass: compact the keys >= theta0 into LDS, in index order
    const int64_t nchunk = (n + kChunk - 1) / kChunk;
    int count = 0;
    uint32_t cmax = 0;
    uint32_t nxt[kPer];
    load16(kPer * tid, nxt);
#pragma unroll 1
    for (int64_t c = 0; c < nchunk; ++c) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) key[i] = nxt[i];
        if (c + 1 < nchunk) load16((c + 1) * kChunk + kPer * tid, nxt);
        int f = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const bool in = key[i] != 0u && key[i] >= theta0;
            f += in ? 1 : 0;
            cmax = in && key[i] > cmax ? key[i] : cmax;
        }
        int total;
        int pos = count + block_inclusive_sum(f, total, sm) - f;
        if (count + total <= kCand) {
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                if (key[i] != 0u && key[i] >= theta0) {
                    sm.cand_key[pos] = key[i];
                    sm.cand_idx[pos] = (int32_t)(c * kChunk + kPer * tid + i);
                    ++pos;
                }
            }
        }
        count += total;
        if (count > kCand) break;   // uniform: too many candidates
    }
    __syncthreads();

    int need = topk;
    if (count >= topk && count <= kCand) {
        // ---- exact select among the candidates: thread t holds candidates 16t .. 16t+15
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int ci = kPer * tid + i;
            key[i] = ci < count ? sm.cand_key[ci] : 0u;
            kidx[i] = ci < count ? sm.cand_idx[ci] : 0;
        }
        const uint32_t range = block_max(cmax, sm) - theta0;   // relative keys <= range
        const int nbits = range ? 32 - __builtin_clz(range) : 1;
        const uint32_t theta = select_rel(key, theta0, nbits, need, sm);
        int eq_base = 0;
        emit_ordered(key, kidx, theta, need, 0, eq_base, oi, os, sm);
        return;
    }

    // ---- general path: exact select streaming the whole row
    uint32_t prefix = 0, pmask = 0;
#pragma unroll 1
    for (int p = 0; p < 3; ++p) {
        const int shift = kShift[p];
        const uint32_t dmask = (1u << kWidth[p]) - 1u;
        for (int i = tid; i < kBins; i += kTkThreads) sm.hist[i] = 0u;
        __syncthreads();
#pragma unroll 1
        for (int64_t c = 0; c < nchunk; ++c) {
            load16(c * kChunk + kPer * tid, key);
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const uint32_t kv = key[i];
                if (kv != 0u && (kv & pmask) == prefix) atomicAdd(&sm.hist[(kv >> shift) & dmask], 1u);
            }
        }
        __syncthreads();
        prefix |= pick_digit(need, sm) << shift;
        pmask |= dmask << shift;
    }
    const uint32_t theta = prefix;
    int out = 0, eq_base = 0;
#pragma unroll 1
    for (int64_t c = 0; c < nchunk; ++c) {
        load16(c * kChunk + kPer * tid, key);
#pragma unroll
        for (int i = 0; i < kPer; ++i) kidx[i] = (int32_t)(c * kChunk + kPer * tid + i);
        out += emit_ordered(key, kidx, theta, need, out, eq_base, oi, os, sm);
    }
}

}  // namespace

hipError_t launch_row_topk_prefill(const float *scores, const int32_t *cu_seqlens,
                                   const int64_t *seq_base, int B, int64_t T, int64_t rows,
                                   int topk, int32_t *idx, float *out_scores, hipStream_t stream) {
    (void)T;
    if (rows == 0) return hipSuccess;
    TopkArgs a{};
    a.scores = scores;
    a.mode = 0;
    a.cu_seqlens = cu_seqlens;
    a.seq_base = seq_base;
    a.B = B;
    a.topk = topk;
    a.out_idx = idx;
    a.out_score = out_scores;
    hipLaunchKernelGGL(row_topk_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_row_topk_decode(const float *scores, const int32_t *seqlens, int B, int64_t ld,
                                  int topk, int32_t *idx, float *out_scores, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    TopkArgs a{};
    a.scores = scores;
    a.mode = 1;
    a.seqlens = seqlens;
    a.ld = ld;
    a.B = B;
    a.topk = topk;
    a.out_idx = idx;
    a.out_score = out_scores;
    hipLaunchKernelGGL(row_topk_kernel, dim3((unsigned)B), dim3(kTkThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
