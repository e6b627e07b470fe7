#pragma once
// Row top-k of fp32 scores (the internals, shared by the row top-k kernels and the decode
// select): for each row of n scores keep the topk largest, ties broken
// toward the lower index, and list them in ascending index order ("Qwen3.5-397B-A17B vs Kimi
// K3.1 Pro" compare page, sparse/compressed-attention row: each query keeps its top 2,048
// tokens).  Rows come from the prefill score workspace (triangular rows of scores.hip) or
// from the decode score buffer (one row per sequence).
//
// One workgroup of 4 waves per row, four workgroups per CU, so that one row's selection
// overlaps other rows' loads.  Scores become order-preserving uint32 keys (0 = no score).
//   * Rows of at most 4,096 scores are held in registers (16 consecutive per thread) and
//     selected exactly.
//   * Longer rows: a threshold theta0 is placed from a sample of 4,096 scores (64 blocks of
//     64 consecutive scores spread over the row) so that about 1.4 topk keys of the row are
//     expected to reach it (a histogram of the sample in 1,024 bins over its own key range
//     finds the bin that holds the r-th largest sample key; theta0 is that bin's lower
//     edge).  Then one streaming pass in which every wave works alone: wave w takes
//     the 1,024-key chunks w, w + 4, ... (16 consecutive keys per lane), keeps the keys >=
//     theta0, reserves room for them in an LDS candidate list with one LDS atomic and writes
//     them there in index order, recording where each chunk's run starts, and counts them in
//     a histogram of 1,024 bins above theta0 (sized from the sample's range).  No workgroup
//     barrier is crossed while the row streams, and each wave keeps two chunks of loads in
//     flight.  When between topk and 4,096 keys reach theta0 (the normal case), one scan of
//     that histogram finds the bin that holds the topk-th largest key; the few keys of that
//     bin are ranked against each other exactly (key, then lower index first), and every
//     candidate above the bin or ranked in wins.  The winners are placed in index order from
//     counts per chunk run and written from LDS with 16-byte stores.  A crowded bin is first
//     narrowed by an exact radix select; rows where the threshold misses (too few, too many
//     candidates) take an exact select that streams the whole row.
// The exact select is a most-significant-digit radix select: theta = the topk-th largest
// key, and how many keys equal to theta are kept (the lowest-index ones).
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace topk_impl {

// W = waves per workgroup (4 for the many rows of prefill, 16 for the few long rows of
// decode).  Per workgroup: 64 W threads; kPer keys per thread per block chunk of 64 W kPer keys
// (the register path and the full-row passes).
constexpr int kPer = 16;                        // keys per thread per chunk
constexpr int kWChunk = 64 * kPer;              // 1,024: one wave's chunk in the streaming pass
// candidate list capacity: one kPer group per thread
template <int W> constexpr int kCand = kPer * 64 * W;
// chunk runs: rows of up to 512K keys (W = 4) or 1M keys (W = 16)
template <int W> constexpr int kMaxRun = W <= 4 ? 512 : 1024;
// sample of a long row: 64 blocks of 64 scores (W = 4); W = 8 or 16 take up to 16 W blocks on
// rows long enough for them to stay a small share of the row
template <int W> constexpr int kSampleBlocks = W <= 4 ? 64 : 16 * W;
constexpr int kPrefetch = 2;                    // wave chunks in flight ahead of the current
constexpr int kRankMax = 128;                   // keys of the threshold bin ranked directly
constexpr int64_t kLongRow = 65536;             // longest prefill row of the 4-wave variant

// Histogram bins (digits of kDigit<W> bits): 512 for the 4-wave prefill workgroups, whose
// LDS footprint sets how many rows a CU holds, 1,024 for the 16-wave decode ones.
template <int W> constexpr int kDigit = W <= 4 ? 9 : 10;
template <int W> constexpr int kBins = 1 << kDigit<W>;
// bins owned by a thread in a histogram scan
template <int W> constexpr int kBinsPer = kBins<W> / (64 * W);
static_assert(kBinsPer<4> >= 1 && kBinsPer<16> >= 1 && kMaxRun<4> <= 2 * 64 * 4 &&
              kMaxRun<16> <= 2 * 64 * 16, "thread ownership of bins and runs");
static_assert(kSampleBlocks<4> * 4 <= 64 * 4 && kSampleBlocks<16> * 4 <= 64 * 16,
              "four threads per sample block");

// decode select (W = 16): pieces of a row's candidate list
template <int W> constexpr int kMaxPieces = W >= 16 ? 4096 : 1;

template <int W> struct TopkSmem {
    static constexpr int kW = W;
    union {
        struct {                   // a candidate: its key and its offset in its chunk
            uint32_t key[kCand<W>];
            uint16_t off[kCand<W>];
        } cand;
        struct {                   // emission: list prefix counts, staged output
            uint16_t pre[kCand<W>];
            int32_t out_idx[kMaxTopk];
            float out_score[kMaxTopk];
        } emit;
        struct {                   // decode select: start (flat position) and list offset of
            int64_t start[kMaxPieces<W>];   // each piece of the row's candidate list, and the
            int32_t off[kMaxPieces<W> + 1];   // piece of the first entry of every 64 entries
            int32_t blk[kCand<W> / 64];
        } pc;
        int32_t ecnt[kPer * W];    // decode select: winners per (entry row, wave), then prefixes
        struct {                   // decode select fallback: the row's query and head weights
            uint32_t q[2 * kHeads * kDim / 2];   // room for the 64-head indexer
            float w[2 * kHeads];
        } resc;
    } u;
    union {
        uint32_t hist[kBins<W>];   // digit histograms; per run: winners in earlier chunks
        struct {                   // the keys of the threshold bin: (key, index), list slot
            uint32_t key[kRankMax];
            int32_t idx[kRankMax];
            uint16_t slot[kRankMax];
        } bin;
    };
    uint32_t run[kMaxRun<W>];      // start | length << 16 of each chunk's run in the list
    uint32_t rlog[kMaxRun<W>];     // chunk | start << 16 of each run, in list order
    uint32_t win[kCand<W> / 32];   // ranked-in keys of the threshold bin, by list slot
    uint32_t count;                // candidates reserved so far | runs reserved << 16
    uint32_t nbin;                 // keys gathered from the threshold bin
    int32_t wsum[W];
    uint32_t wmax[W];
    int32_t bcast[3];
};

static_assert(sizeof(TopkSmem<4>) <= 32 * 1024, "five workgroups of 4 waves per CU");
static_assert(kMaxRun<4> <= kBins<4> && kMaxRun<16> <= kBins<16>, "per-run emission data lives in hist");
static_assert(kCand<16> <= 65536, "list positions are 16-bit");

struct TopkArgs {
    const float *scores;
    int mode;                      // 0: prefill rows (triangular), 1: decode rows
    const int32_t *cu_seqlens;     // prefill varlen (nullptr: one sequence of length T)
    const int64_t *seq_base;
    int64_t pos0;                  // prefill, one sequence: position of query row 0
    int64_t g0;                    // first row of this launch
    int B;
    const int32_t *seqlens;        // decode: row b holds seqlens[b] (clamped to nmax) scores
    int64_t ld;                    // decode: row stride (a multiple of 4)
    int64_t nmax;                  // decode: longest row
    int topk;
    int32_t *out_idx;
    float *out_score;              // may be nullptr
    const int64_t *out_row;        // output row of row g (nullptr: g)
    const uint32_t *status;        // row_topk_kernel: bit 0 set -> rows invalid (nullptr: none)
};


// Inclusive sum over the workgroup of one int per thread (the sum of all in `total`).
template <class Sm>
__device__ int block_inclusive_sum(int v, int &total, Sm &sm) {
    [[maybe_unused]] constexpr int W = Sm::kW;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int incl = wave_inclusive_sum(v);
    if (lane == 63) sm.wsum[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
        const int s = sm.wsum[i];
        before += i < wave ? s : 0;
        all += s;
    }
    __syncthreads();
    total = all;
    return before + incl;
}

// Exclusive prefix over the wave of one int per lane, and the wave's total.
__device__ __forceinline__ int wave_exclusive_sum(int v, int &total) {
    const int incl = row16_inclusive_sum(v);
    const int r0 = __builtin_amdgcn_readlane(incl, 15), r1 = __builtin_amdgcn_readlane(incl, 31);
    const int r2 = __builtin_amdgcn_readlane(incl, 47), r3 = __builtin_amdgcn_readlane(incl, 63);
    const int g = ((int)threadIdx.x & 63) >> 4;
    const int below = (g > 0 ? r0 : 0) + (g > 1 ? r1 : 0) + (g > 2 ? r2 : 0);
    total = r0 + r1 + r2 + r3;
    return below + incl - v;
}

// One digit of the radix select: given the histogram of the keys that match the digits
// found so far, return the digit of the need-th largest and subtract from need the keys in
// higher digits; in_bin = the keys in the returned digit's bin.  Thread t owns bins
// kBinsPer t .. kBinsPer t + kBinsPer - 1.
template <class Sm>
__device__ uint32_t pick_digit(int &need, Sm &sm, int *in_bin = nullptr) {
    [[maybe_unused]] constexpr int W = Sm::kW;
    const int tid = (int)threadIdx.x;
    int cnt[kBinsPer<W>], sum = 0;
#pragma unroll
    for (int j = 0; j < kBinsPer<W>; ++j) {
        cnt[j] = (int)sm.hist[kBinsPer<W> * tid + j];
        sum += cnt[j];
    }
    int total;
    const int incl = block_inclusive_sum(sum, total, sm);
    int above = total - incl;   // keys in bins above this thread's
#pragma unroll
    for (int j = kBinsPer<W> - 1; j >= 0; --j) {
        if (above < need && need <= above + cnt[j]) {
            sm.bcast[0] = kBinsPer<W> * tid + j;
            sm.bcast[1] = above;
            sm.bcast[2] = cnt[j];
        }
        above += cnt[j];
    }
    __syncthreads();
    const uint32_t d = (uint32_t)sm.bcast[0];
    need -= sm.bcast[1];
    if (in_bin) *in_bin = sm.bcast[2];
    __syncthreads();
    return d;
}

// Largest of one key per thread over the workgroup.
template <class Sm>
__device__ uint32_t block_max(uint32_t v, Sm &sm) {
    [[maybe_unused]] constexpr int W = Sm::kW;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, d, 64);
        v = o > v ? o : v;
    }
    if (lane == 0) sm.wmax[wave] = v;
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) m = sm.wmax[i] > m ? sm.wmax[i] : m;
    __syncthreads();
    return m;
}

// Exact select over keys >= base held in registers (0 = no key), digits taken from the
// relative key (key - base) < 2^nbits, kDigit<W> bits at a time from the top: returns theta,
// the need-th largest key; on return need = how many keys equal to theta are among the need
// largest.
template <class Sm>
__device__ uint32_t select_rel(const uint32_t (&key)[kPer], uint32_t base, int nbits, int &need,
                               Sm &sm) {
    [[maybe_unused]] constexpr int W = Sm::kW;
    uint32_t prefix = 0, pmask = 0;
    int hi = nbits;
#pragma unroll 1
    while (hi > 0) {
        const int w = hi < kDigit<W> ? hi : kDigit<W>;
        const int shift = hi - w;
        const uint32_t dmask = (1u << w) - 1u;
        for (int i = (int)threadIdx.x; i < kBins<W>; i += (64 * W)) sm.hist[i] = 0u;
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

// Number of significant bits of x (0 for x = 0).
__device__ __forceinline__ int bit_width(uint32_t x) { return x ? 32 - __builtin_clz(x) : 0; }

// Writes, in index order, the keys above theta and the first `need` keys equal to theta among
// this thread's kPer keys (indices idx0 + i, increasing with thread and i); out_base = outputs
// already written and eq_base = keys equal to theta already seen (both block-uniform).
// Returns the number written by the whole workgroup; eq_base advances by the ties seen.
template <class Sm>
__device__ int emit_ordered(const uint32_t (&key)[kPer], int32_t idx0, uint32_t theta,
                            int need, int out_base, int &eq_base, int32_t *oi, float *os,
                            Sm &sm) {
    [[maybe_unused]] constexpr int W = Sm::kW;
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
            oi[pos] = idx0 + i;
            if (os) os[pos] = key_score(key[i]);
            ++pos;
        }
    }
    eq_base += eq_total;
    return keep_total;
}

// emit_ordered for keys whose indices are given (kidx[i], increasing with thread and i).
template <class Sm>
__device__ int emit_ordered_idx(const uint32_t (&key)[kPer], const int32_t (&kidx)[kPer], uint32_t theta,
                                int need, int out_base, int &eq_base, int32_t *oi, float *os,
                                Sm &sm) {
    [[maybe_unused]] constexpr int W = Sm::kW;
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
            oi[pos] = kidx[i];
            if (os) os[pos] = key_score(key[i]);
            ++pos;
        }
    }
    eq_base += eq_total;
    return keep_total;
}

// Emission from the candidate list.  The list holds `count` candidates in runs, one run per
// wave chunk of kWChunk keys (sm.run[c] = start | length << 16), each run in index order; the
// runs themselves are in no particular order.  Thread t holds list entries kPer t .. kPer t +
// kPer - 1 and bit i of `win` says whether entry i is kept (exactly topk are).  A winner's output
// slot = winners in earlier chunks + winners before it in its run, both counted from prefix
// sums over the list.  The output row is staged in LDS and written with 16-byte stores.
template <int W>
__device__ void emit_winners(const uint32_t (&key)[kPer], const int32_t (&idx)[kPer],
                             uint32_t win, int count, int nrun, int topk, int32_t *oi,
                             float *os, TopkSmem<W> &sm) {
    const int tid = (int)threadIdx.x;
    const int tsum = __builtin_popcount(win);
    int all;
    const int ex0 = block_inclusive_sum(tsum, all, sm) - tsum;   // winners before this thread
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int ex = ex0 + __builtin_popcount(win & ((2u << i) - 1u));
        if (kPer * tid + i < count) sm.u.emit.pre[kPer * tid + i] = (uint16_t)ex;   // inclusive
    }
    __syncthreads();
    // per run, in chunk order (thread t: chunks 2t, 2t+1): winners nw, and winners before it
    // in the list (lo)
    uint32_t lo[2], nw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = 2 * tid + j;
        const uint32_t r = c < nrun ? sm.run[c] : 0u;
        const uint32_t s = r & 0xFFFFu, m = r >> 16;
        lo[j] = s > 0 ? sm.u.emit.pre[s - 1] : 0u;
        nw[j] = (m > 0 ? sm.u.emit.pre[s + m - 1] : lo[j]) - lo[j];
    }
    int tot;
    const int wb = block_inclusive_sum((int)(nw[0] + nw[1]), tot, sm) - (int)(nw[0] + nw[1]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = 2 * tid + j;
        if (c < nrun) {
            sm.hist[c] = (uint32_t)(wb + (j ? (int)nw[0] : 0));
            sm.run[c] = lo[j];
        }
    }
    __syncthreads();   // (also: every read of pre is done before the staged output overwrites it)
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (kPer * tid + i < count && ((win >> i) & 1u)) {
            const int c = idx[i] / kWChunk;
            const int exi = ex0 + __builtin_popcount(win & ((1u << i) - 1u));   // winners before
            const int pos = (int)sm.hist[c] + exi - (int)sm.run[c];
            sm.u.emit.out_idx[pos] = idx[i];
            sm.u.emit.out_score[pos] = key_score(key[i]);
        }
    }
    __syncthreads();
    // copy-out: 16-byte stores where the output rows allow them
    const uintptr_t align = reinterpret_cast<uintptr_t>(oi) | reinterpret_cast<uintptr_t>(os);
    if ((topk & 3) == 0 && (align & 15) == 0) {
        for (int p = 4 * tid; p < topk; p += 4 * (64 * W)) {
            *reinterpret_cast<u32x4 *>(oi + p) = *reinterpret_cast<const u32x4 *>(&sm.u.emit.out_idx[p]);
            if (os) *reinterpret_cast<u32x4 *>(os + p) = *reinterpret_cast<const u32x4 *>(&sm.u.emit.out_score[p]);
        }
    } else {
        for (int p = tid; p < topk; p += (64 * W)) {
            oi[p] = sm.u.emit.out_idx[p];
            if (os) os[p] = sm.u.emit.out_score[p];
        }
    }
}

// Row g's scores and their number.
__device__ __forceinline__ void locate_row(const TopkArgs &a, int64_t g, const float *&row, int64_t &n) {
    if (a.mode == 0) {
        int64_t t = a.pos0 + g, base = -tri_row_offset(a.pos0);
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
        n = L < 0 ? 0 : (L > a.nmax ? a.nmax : L);
        row = a.scores + g * a.ld;
    }
}

// 16 keys of a row of n scores from element e0 (4-aligned; rows are padded to a multiple of
// 64 scores, so a 16-byte group that starts below n lies inside the row); 0 past the end.
__device__ __forceinline__ void load16(const float *row, int64_t n, int64_t e0, uint32_t (&key)[kPer]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t e = e0 + 4 * q;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (e < n) v = *reinterpret_cast<const f32x4 *>(row + e);
#pragma unroll
        for (int j = 0; j < 4; ++j) key[4 * q + j] = e + j < n ? score_key(v[j]) : 0u;
    }
}

// The sample of a long row: nblk blocks of 64 consecutive scores spread over the row (n >
// 64 nblk); thread t reads quarter t % 4 of block t / 4.
__device__ __forceinline__ void load_sample(const float *row, int64_t n, int nblk, uint32_t (&key)[kPer]) {
    const int tid = (int)threadIdx.x;
    if (tid >= 4 * nblk) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) key[i] = 0u;
        return;
    }
    const int64_t start = ((int64_t)(tid >> 2) * (n - 64) / (nblk - 1)) & ~(int64_t)3;
    load16(row, n, start + 16 * (tid & 3), key);
}

// Top-k of row g, by one workgroup of 64 W threads.
template <int W>
__device__ __forceinline__ void row_topk_row(const TopkArgs &a, int64_t g, TopkSmem<W> &sm) {
    constexpr int kChunk = 64 * W * kPer;   // keys of the register path / one full-row pass step
    const int topk = a.topk;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t key[kPer];
    int32_t kidx[kPer];
    const float *row;
    int64_t n;
    locate_row(a, g, row, n);
    const int64_t go = a.out_row ? a.out_row[g] : g;
    int32_t *oi = a.out_idx + go * topk;
    float *os = a.out_score ? a.out_score + go * topk : nullptr;
    if (n <= topk) {
        for (int i = tid; i < topk; i += (64 * W)) {
            const bool in = i < n;
            oi[i] = in ? i : -1;
            if (os) os[i] = in ? row[i] : -INFINITY;
        }
        return;
    }

    if (n <= kChunk) {
        // ---- short row: all of it in registers
        load16(row, n, kPer * tid, key);
        uint32_t m = 0, mn = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            m = key[i] > m ? key[i] : m;
            mn = key[i] != 0u && key[i] < mn ? key[i] : mn;
        }
        const uint32_t top = block_max(m, sm);
        const uint32_t bot = ~block_max(~mn, sm);
        int need = topk;
        const uint32_t theta = select_rel(key, bot, bit_width(top - bot), need, sm);
        int eq_base = 0;
        emit_ordered(key, kPer * tid, theta, need, 0, eq_base, oi, os, sm);
        return;
    }

    // ---- sample; the wave's first chunks of the streaming pass are requested right behind
    // it, so they arrive while theta0 is placed.
#pragma unroll
    for (int j = 0; j < kBinsPer<W>; ++j) sm.hist[kBinsPer<W> * tid + j] = 0u;
    if (tid < kCand<W> / 32) sm.win[tid] = 0u;
    if (tid == 0) {
        sm.count = 0u;
        sm.nbin = 0u;
    }
    // sample blocks: 64, or on long rows of the 16-wave variant one per 4,096 scores
    int nblk = 64;
    if (W > 4) {
        const int64_t b = n >> 12;
        nblk = b < 64 ? 64 : (b > kSampleBlocks<W> ? kSampleBlocks<W> : (int)b);
    }
    const int ns = 64 * nblk;   // sampled scores
    load_sample(row, n, nblk, key);
    const int64_t nwc = (n + kWChunk - 1) / kWChunk;   // wave chunks
    uint32_t buf[kPrefetch][kPer];
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p) load16(row, n, (int64_t)(wave + W * p) * kWChunk + kPer * lane, buf[p]);

    // r such that about f topk keys of the row reach the r-th largest of the sample: f = 1.4
    // with 4 waves, 2 with 16 (whose list holds 16,384 candidates)
    constexpr int64_t kNum = W <= 4 ? 7 : 2, kDen = W <= 4 ? 5 : 1;
    int r = (int)(((int64_t)topk * kNum * ns + kDen * n - 1) / (kDen * n)) + 8;
    if (r > ns) r = ns;
    uint32_t theta0, top;
    {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) m = key[i] > m ? key[i] : m;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)m, d, 64);
            m = o > m ? o : m;
        }
        if (lane == 0) sm.wmax[wave] = m;
        __syncthreads();
        top = 0;
#pragma unroll
        for (int i = 0; i < W; ++i) top = sm.wmax[i] > top ? sm.wmax[i] : top;
        // The r-th largest sample key, to 2^(24 - D) key units: kBins = 2^D bins of 2^sb
        // units counted down from wtop.  First the window of two binades (2^24 units) below
        // the top; if it holds fewer than r sample keys, the whole key range in bins of
        // 2^(32 - D) units, then the bin found there in bins of 2^(32 - 2D).  Each thread
        // clears the bins it has read, so the histogram is zero again for the next pass and
        // for the streaming pass.
        constexpr int kD = kDigit<W>;
        int64_t wtop = top;
        int sb = 24 - kD, rr = r;
#pragma unroll 1
        for (;;) {
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int64_t d = (wtop - (int64_t)key[i]) >> sb;
                if (key[i] != 0u && d >= 0 && d < kBins<W>) atomicAdd(&sm.hist[d], 1u);
            }
            __syncthreads();
            // bins in descending key order are ascending d: the first bin where the running
            // count reaches rr
            int cnt[kBinsPer<W>], sum = 0;
#pragma unroll
            for (int j = 0; j < kBinsPer<W>; ++j) {
                cnt[j] = (int)sm.hist[kBinsPer<W> * tid + j];
                sum += cnt[j];
            }
            int total;
            int run = block_inclusive_sum(sum, total, sm) - sum;
#pragma unroll
            for (int j = 0; j < kBinsPer<W>; ++j) {
                if (run < rr && rr <= run + cnt[j]) {
                    sm.bcast[0] = kBinsPer<W> * tid + j;
                    sm.bcast[1] = run;
                }
                run += cnt[j];
                sm.hist[kBinsPer<W> * tid + j] = 0u;
            }
            __syncthreads();
            if (total >= rr) {
                const int64_t bb = sm.bcast[0];
                if (sb <= 24 - kD) {
                    const int64_t lo = wtop - ((bb + 1) << sb) + 1;   // lowest key of bin bb
                    theta0 = lo < 1 ? 1u : (uint32_t)lo;
                    break;
                }
                wtop -= bb << sb;   // the top of bin bb, split next in bins 2^D times finer
                rr -= sm.bcast[1];
                sb -= kD;
            } else if (sb < 32 - kD) {
                sb = 32 - kD;       // the whole key range
            } else {
                theta0 = 1u;        // (not reached: the sample holds at least r keys)
                break;
            }
            __syncthreads();        // bcast is read before the next pass writes it
        }
    }
    // bins of the streaming histogram: 2^sh key units above theta0, so that the sample's
    // range takes at most half of them; keys further up share the last bin
    const int sh = bit_width((top - theta0) >> (kDigit<W> - 1));


    // ---- streaming pass, every wave on its own: compact the keys >= theta0 of wave chunk c
    // into a run of the candidate list, in index order (no workgroup barrier until the end)
    const bool runs_fit = nwc <= kMaxRun<W>;
    uint32_t cmax = 0;
#pragma unroll 1
    for (int64_t c = wave; c < nwc; c += W) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) key[i] = buf[0][i];
#pragma unroll
        for (int p = 0; p + 1 < kPrefetch; ++p)
#pragma unroll
            for (int i = 0; i < kPer; ++i) buf[p][i] = buf[p + 1][i];
        const int64_t cn = c + W * kPrefetch;
        if (cn < nwc) load16(row, n, cn * kWChunk + kPer * lane, buf[kPrefetch - 1]);
        int f = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const bool in = key[i] >= theta0;   // theta0 >= 1: never a missing key
            f += in ? 1 : 0;
            cmax = in && key[i] > cmax ? key[i] : cmax;
        }
        int total;
        int pos = wave_exclusive_sum(f, total);
        // one LDS atomic reserves the run: list start in the low half, run number in the
        // high half (the low half stays below 2^16: reservations stop past kCand)
        uint32_t res = 0;
        if (lane == 0) res = atomicAdd(&sm.count, (uint32_t)total | 0x10000u);
        res = (uint32_t)__builtin_amdgcn_readfirstlane((int)res);
        const uint32_t start = res & 0xFFFFu;
        if (start + (uint32_t)total > (uint32_t)kCand<W> || !runs_fit) break;   // wave-uniform
        if (lane == 0) {
            sm.run[c] = start | ((uint32_t)total << 16);
            sm.rlog[res >> 16] = (uint32_t)c | (start << 16);
        }
        pos += (int)start;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            if (key[i] >= theta0) {
                const uint32_t d = (key[i] - theta0) >> sh;
                atomicAdd(&sm.hist[d < (uint32_t)kBins<W> ? d : kBins<W> - 1], 1u);
                sm.u.cand.key[pos] = key[i];
                sm.u.cand.off[pos] = (uint16_t)(kPer * lane + i);
                ++pos;
            }
        }
    }
    __syncthreads();
    const int count = (int)(sm.count & 0xFFFFu);
    const int nres = (int)(sm.count >> 16);

    int need = topk;
    if (runs_fit && count >= topk && count <= kCand<W>) {
        // ---- select among the candidates: thread t holds list entries 16t .. 16t+15
        // the run (and so the chunk) of list entry 16t: the last run starting at or below it
        // (runs are logged in list order; an empty run starts where the next one does)
        int rr0 = 0;
        {
            int lo = 0, hi = nres - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if ((int)(sm.rlog[mid] >> 16) <= kPer * tid) lo = mid;
                else hi = mid - 1;
            }
            rr0 = lo;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int ci = kPer * tid + i;
            while (rr0 + 1 < nres && (int)(sm.rlog[rr0 + 1] >> 16) <= ci) ++rr0;
            key[i] = ci < count ? sm.u.cand.key[ci] : 0u;
            kidx[i] = ci < count ? (int32_t)((sm.rlog[rr0] & 0xFFFFu) * kWChunk + sm.u.cand.off[ci]) : 0;
        }
        // the bin [blo, bhi] that holds the topk-th largest key; need = its keys that win
        int in_bin;
        const uint32_t d = pick_digit(need, sm, &in_bin);
        const uint64_t lo64 = (uint64_t)theta0 + ((uint64_t)d << sh);   // a key lies above it
        const uint64_t hi64 = lo64 + (1ull << sh) - 1ull;
        uint32_t blo = (uint32_t)lo64;
        uint32_t bhi = d == kBins<W> - 1 || hi64 > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)hi64;
        if (in_bin > kRankMax) {
            // a crowded bin: narrow it to one key value by an exact select over its keys
            uint32_t kb[kPer];
            uint32_t bmax = 0;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                kb[i] = key[i] >= blo && key[i] <= bhi ? key[i] : 0u;
                bmax = kb[i] > bmax ? kb[i] : bmax;
            }
            const uint32_t theta = select_rel(kb, blo, bit_width(block_max(bmax, sm) - blo), need, sm);
            int e = 0;
#pragma unroll
            for (int i = 0; i < kPer; ++i) e += key[i] == theta ? 1 : 0;
            block_inclusive_sum(e, in_bin, sm);
            blo = bhi = theta;
        }
        if (in_bin <= kRankMax) {
            // rank the bin's keys exactly: by key, then lower index first; the need best win
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                if (key[i] >= blo && key[i] <= bhi) {
                    const uint32_t j = atomicAdd(&sm.nbin, 1u);
                    sm.bin.key[j] = key[i];
                    sm.bin.idx[j] = kidx[i];
                    sm.bin.slot[j] = (uint16_t)(kPer * tid + i);
                }
            }
            __syncthreads();
            if (tid < in_bin) {
                const uint32_t mk = sm.bin.key[tid];
                const int32_t mi = sm.bin.idx[tid];
                int rank = 0;
                for (int j = 0; j < in_bin; ++j) {
                    const uint32_t ok = sm.bin.key[j];
                    rank += (ok > mk || (ok == mk && sm.bin.idx[j] < mi)) ? 1 : 0;
                }
                if (rank < need) {
                    const int sl = sm.bin.slot[tid];
                    atomicOr(&sm.win[sl >> 5], 1u << (sl & 31));
                }
            }
            __syncthreads();
            uint32_t win = 0;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int sl = kPer * tid + i;
                const bool w = key[i] > bhi || (key[i] >= blo && ((sm.win[sl >> 5] >> (sl & 31)) & 1u));
                win |= w ? 1u << i : 0u;
            }
            emit_winners(key, kidx, win, count, (int)nwc, topk, oi, os, sm);
            return;
        }
        need = topk;   // more than kRankMax equal keys at the threshold: the general path
    }

    // ---- general path: exact select streaming the whole row, absolute 10-bit digits from
    // the top (the last of the four has 2 bits)
    const int64_t nchunk = (n + kChunk - 1) / kChunk;
    uint32_t prefix = 0, pmask = 0;
#pragma unroll 1
    for (int hi = 32; hi > 0;) {
        const int w = hi < kDigit<W> ? hi : kDigit<W>;
        const int shift = hi - w;
        const uint32_t dmask = (1u << w) - 1u;
        for (int i = tid; i < kBins<W>; i += (64 * W)) sm.hist[i] = 0u;
        __syncthreads();
#pragma unroll 1
        for (int64_t c = 0; c < nchunk; ++c) {
            load16(row, n, c * kChunk + kPer * tid, key);
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const uint32_t kv = key[i];
                if (kv != 0u && (kv & pmask) == prefix) atomicAdd(&sm.hist[(kv >> shift) & dmask], 1u);
            }
        }
        __syncthreads();
        prefix |= pick_digit(need, sm) << shift;
        pmask |= dmask << shift;
        hi = shift;
    }
    const uint32_t theta = prefix;
    int out = 0, eq_base = 0;
#pragma unroll 1
    for (int64_t c = 0; c < nchunk; ++c) {
        load16(row, n, c * kChunk + kPer * tid, key);
        out += emit_ordered(key, (int32_t)(c * kChunk + kPer * tid), theta, need, out, eq_base, oi, os, sm);
    }
}

}  // namespace topk_impl
}  // namespace dsaidx
