// Decode: one new query per sequence scored against that sequence's cached indexer keys
// (serving engines cache the indexer keys: "Kimi K3.1 Pro vs GLM-5" compare page,
// low-precision row), then the top-k of the whole prefix (sparse/compressed-attention row of
// the "Qwen3.5-397B-A17B vs Kimi K3.1 Pro" page; long-context row of the "Kimi K3.1 Pro vs
// Gemma 4 31B" page).  The cache holds bf16 keys (256 bytes each) or FP8 keys (128 E4M3 bytes
// and a power-of-two scale; see fp8.hip).
//
// Three passes.  Streaming the cache is the bandwidth-bound part; writing every score back
// to HBM in the middle of that stream, and then a row top-k whose single workgroup per row
// streams those scores again, each cost a sizeable fraction of the stream itself.  So:
//  1. plan (four workgroups per sequence score a stratified sample of its keys, then one
//     workgroup per sequence turns the sample into a threshold): theta is such that, with
//     overwhelming probability, between topk and a few times topk of the row's scores
//     reach it;
//  2. filter (the flat split below): every key is scored, and only the keys whose score
//     reaches theta are written, as (score, index) pairs, in index order;
//  3. select (one workgroup per sequence): the exact top-k of those candidates, ties to the
//     lower index, in ascending index order.
// The result is exact whatever theta is: a row whose candidates turn out fewer than topk (a
// sample that overshoots) is scored again in full by its select workgroup and selected from
// all its scores; a row whose sample predicts too many candidates (many equal scores) has
// all its scores written by the filter pass and is selected from those.  Rows of at most
// kShortRow keys take every key as a candidate.
//
// The filter pass splits the flat range of all cached keys (each sequence padded to a
// multiple of 64 positions) evenly over its waves, so every wave streams the same number of
// bytes whatever the lengths.  Each 16-key slice is a pair of MFMA chains with the 32 heads
// as the M dimension (two halves of 16); ReLU and the w-weighted head sum stay in registers;
// a wave takes 64 consecutive keys (four slices) at a time, and issues the next group's loads
// before any store of this one, so that waiting for loads never waits for a store.  A wave's
// candidates go to a small LDS ring and leave it 64 at a time with full-width stores.
#include "common.hpp"
#include "launch.hpp"
#include "scorers.hpp"
#include "topk_impl.hpp"

namespace dsaidx {
namespace {
using namespace topk_impl;

constexpr int kFilterThreads = 256;
constexpr int kPlanThreads = 512;
constexpr int kSelectThreads = 1024;
constexpr int kShortRow = kPer * kSelectThreads;   // 16,384: every key a candidate
constexpr int kSampleMin = 1024, kSampleMax = 8192;
constexpr int64_t kDenseCount = 12288;              // predicted candidates of a dense row
constexpr int kPlanPrefixMax = 4096;                // batches whose prefix the plan pass computes
constexpr int kSampleParts = 4, kSampleThreads = 256;
static_assert(kMaxPieces<16> >= 8, "pieces per row");
static_assert(kSampleMin == 1024 && kSampleMax == 8192, "sample sizes 2^10 .. 2^13");

struct DecodePlan {
    uint32_t theta;   // candidates: order keys >= theta (0: every key)
    uint32_t dense;   // 1: the filter writes all scores of the row, the select takes them all
};

struct DecCommon {
    const int64_t *start;    // [B] first cache row of each sequence
    const int32_t *seqlens;  // [B] cached keys (clamped to [0, max_seqlen])
    int B;
    int max_seqlen;
    int topk;
    int filter_grid;         // workgroups of the filter pass (its geometry is recomputed)
    int64_t *cu;             // [B + 1] prefix sums of the padded lengths
    DecodePlan *plan;        // [B]
    int32_t *cnt;            // candidates of the piece starting at flat position p: cnt[p / 64]
    uint2 *cand;             // the piece's candidates from cand[p] on: (score bits, index)
    float *score_buf;        // [B][ld]: all scores of dense and re-scored rows
    uint32_t *skey;          // [B][kSampleMax] order keys of the sampled scores
    int64_t ld;
    int32_t *idx;            // [B][topk]
    float *scores;           // [B][topk] or nullptr
};

__device__ __forceinline__ int clamp_len(const DecCommon &a, int b) {
    return max(0, min(a.seqlens[b], a.max_seqlen));
}
__device__ __forceinline__ int64_t pad64(int64_t n) { return (n + 63) & ~(int64_t)63; }

// Keys per wave of the filter pass: an even split of the flat range over its waves, but long
// enough that a row has at most kMaxPieces pieces; a multiple of 64.
__device__ __forceinline__ int64_t decode_sub(int64_t total, int grid, int max_seqlen) {
    const int64_t waves = (int64_t)grid * (kFilterThreads / 64);
    const int64_t even = (total + waves - 1) / waves;
    const int64_t longest = ((int64_t)max_seqlen + kMaxPieces<16> - 3) / (kMaxPieces<16> - 2);
    return pad64(even > longest ? even : longest);
}

// Sample i of S = 2^lgS of a row of n >= S keys.  The sample is S / 8 runs of 8 consecutive
// keys (2 KB of bf16 keys: random single keys would cost a DRAM page each): run j lies in
// stratum [j n / (S/8), (j + 1) n / (S/8)) at an offset picked by an integer hash of
// (sequence, j) (the "lowbias32" mixer of C. Wellons) scaled to the stratum's width less 8,
// so that the runs are spread over the whole row and follow no fixed stride.
__device__ __forceinline__ int sample_pos(int b, int i, int n, int lgS) {
    const int j = i >> 3, lgR = lgS - 3;
    const int64_t lo = ((int64_t)j * n) >> lgR, hi = ((int64_t)(j + 1) * n) >> lgR;
    uint32_t x = (uint32_t)j + 0x9E3779B9u * (uint32_t)(b + 1);
    x ^= x >> 16;
    x *= 0x7FEB352Du;
    x ^= x >> 15;
    x *= 0x846CA68Bu;
    x ^= x >> 16;
    return (int)(lo + (int64_t)(((uint64_t)x * (uint64_t)(hi - lo - 7)) >> 32)) + (i & 7);
}

// ---------------------------------------------------------------- pass 1: plan
// S = 2^lgS samples of a row of n keys: at least n / 128 (1,024 .. 8,192).
__device__ __forceinline__ int sample_lg(int n) {
    int lgS = 10;
    while (lgS < 13 && (1 << lgS) < n / 128) ++lgS;
    return lgS;
}

// 1a. kSampleParts workgroups per sequence score a quarter of its sample each (one CU streams
// only some 20 GB/s, so a single workgroup per sequence took 12 us for its 256 KB sample)
// and write the order keys to the workspace.  Part 0 also writes cu[b] (own_prefix) and the
// plan of a short row.
template <class Sc, class Keys>
__global__ __launch_bounds__(kSampleThreads) void decode_sample_kernel(DecCommon a, Keys kp, int own_prefix) {
    __shared__ int64_t red[kSampleThreads / 64];
    const int b = blockIdx.x / kSampleParts, part = blockIdx.x % kSampleParts, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int n = clamp_len(a, b);
    if (own_prefix && part == 0) {
        int64_t s = 0;
        for (int i = tid; i < b; i += kSampleThreads) s += pad64(clamp_len(a, i));
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
        if (lane == 0) red[wave] = s;
        __syncthreads();
        if (tid == 0) {
            int64_t t = 0;
#pragma unroll
            for (int i = 0; i < kSampleThreads / 64; ++i) t += red[i];
            a.cu[b] = t;
            if (b == a.B - 1) a.cu[a.B] = t + pad64(n);
        }
    }
    if (n <= kShortRow) {
        if (part == 0 && tid == 0) a.plan[b] = DecodePlan{0u, 0u};
        return;
    }
    const int lgS = sample_lg(n);
    const int G = (1 << lgS) / 64 / kSampleParts;   // 64-key groups of this part
    Sc sc;
    sc.init(kp, a.start, b, l16, lg);
    uint32_t *out = a.skey + (int64_t)b * kSampleMax;
    for (int g = wave; g < G; g += kSampleThreads / 64) {
        const int j = part * G + g;
        int key[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) key[u] = sample_pos(b, 64 * j + 16 * u + l16, n, lgS);
        sc.load(key, lg);
        float p[4];
        sc.partial(p);
        out[64 * j + lane] = score_key(finish(sc, p, sc.scale(), lg));
    }
}

// 1b. One workgroup per sequence: the threshold from the sample keys.
__global__ __launch_bounds__(kPlanThreads) void decode_threshold_kernel(DecCommon a) {
    __shared__ uint32_t skey[kSampleMax];
    __shared__ uint32_t hist[1024];
    __shared__ int64_t red[kPlanThreads / 64];
    __shared__ uint32_t red2[kPlanThreads / 64];
    __shared__ int bc[2];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int kWaves = kPlanThreads / 64;
    auto block_sum = [&](int64_t v) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
        if (lane == 0) red[wave] = v;
        __syncthreads();
        int64_t t = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) t += red[i];
        __syncthreads();
        return t;
    };
    const int n = clamp_len(a, b);
    if (n <= kShortRow) return;   // planned by the sample pass
    const int S = 1 << sample_lg(n);
    const uint32_t *in = a.skey + (int64_t)b * kSampleMax;
    for (int x = 4 * tid; x < S; x += 4 * kPlanThreads)
        *reinterpret_cast<u32x4 *>(&skey[x]) = *reinterpret_cast<const u32x4 *>(in + x);
    __syncthreads();
    // r such that fewer than r of the S samples reach the topk-th largest score of the row
    // only with negligible probability (their number is about binomial with mean E)
    const float E = (float)S * (float)a.topk / (float)n;
    int r = (int)ceilf(E + 6.f * sqrtf(E) + 6.f);
    r = r > S ? S : r;
    // theta: the lower edge of the bin that holds the r-th largest sample key, first in 1,024
    // bins over the sample's key range, then in 1,024 bins over that bin (exact when the bins
    // reach single key values, otherwise at most 1/2^20 of the range lower)
    uint32_t top = 0, bot = 0xFFFFFFFFu;
    for (int x = tid; x < S; x += kPlanThreads) {
        const uint32_t k = skey[x];
        top = k > top ? k : top;
        bot = k < bot ? k : bot;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)top, d, 64), o2 = (uint32_t)__shfl_xor((int)bot, d, 64);
        top = o > top ? o : top;
        bot = o2 < bot ? o2 : bot;
    }
    if (lane == 0) {
        red[wave] = top;
        red2[wave] = bot;
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kWaves; ++x) {
        top = (uint32_t)red[x] > top ? (uint32_t)red[x] : top;
        bot = red2[x] < bot ? red2[x] : bot;
    }
    int nb = 32 - __builtin_clz((top - bot) | 1u);
    int sh = nb > 10 ? nb - 10 : 0;
    uint32_t base = bot, theta = bot;
    int rr = r;
    int span = 32;   // keys counted: base <= key < base + 2^span (pass 0: all)
    for (int pass = 0; pass < 2; ++pass) {
        hist[tid] = 0u;
        if (tid + kPlanThreads < 1024) hist[tid + kPlanThreads] = 0u;
        __syncthreads();
        for (int x = tid; x < S; x += kPlanThreads) {
            const uint32_t k = skey[x];
            const uint64_t rel = (uint64_t)k - base;
            if (k >= base && (rel >> span) == 0) atomicAdd(&hist[rel >> sh], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            int c[16], sum = 0;
#pragma unroll
            for (int q = 0; q < 16; ++q) {   // lane l: bins 1023 - 16 l - q, from the top
                c[q] = (int)hist[1023 - 16 * lane - q];
                sum += c[q];
            }
            int run = wave_inclusive_sum(sum) - sum;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                if (run < rr && rr <= run + c[q]) {
                    bc[0] = 1023 - 16 * lane - q;
                    bc[1] = run;
                }
                run += c[q];
            }
        }
        __syncthreads();
        base += (uint32_t)bc[0] << sh;
        rr -= bc[1];
        theta = base;
        __syncthreads();
        if (sh == 0) break;
        span = sh;
        sh = sh > 10 ? sh - 10 : 0;
    }
    int64_t reach = 0;
    for (int x = tid; x < S; x += kPlanThreads) reach += skey[x] >= theta ? 1 : 0;
    reach = block_sum(reach);
    if (tid == 0) a.plan[b] = DecodePlan{theta, reach * n / S > kDenseCount ? 1u : 0u};
}

// ---------------------------------------------------------------- pass 2: filter
// Keys stream through LDS: each wave copies its next 64-key group into its own slot with
// non-temporal whole-line loads (Sc::stage), reads the fragments of that group back (Sc::
// load_staged) and, before scoring them, already requests the group after it into the slot.
template <class Sc>
constexpr size_t filter_smem() { return (size_t)(kFilterThreads / 64) * Sc::kSlotBytes; }

template <class Sc, class Keys>
__global__ __launch_bounds__(kFilterThreads, 2) void decode_filter_kernel(DecCommon a, Keys kp) {
    __shared__ uint2 ring[kFilterThreads / 64][128];
    extern __shared__ __align__(16) unsigned char slots[];
    const int64_t total = a.cu[a.B];
    const int64_t sub = decode_sub(total, gridDim.x, a.max_seqlen);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    int64_t pos = ((int64_t)blockIdx.x * (kFilterThreads / 64) + wave) * sub;
    const int64_t end = min(total, pos + sub);
    if (pos >= end) return;
    uint2 *rw = ring[wave];
    // the last sequence with cu[b] <= pos (cu is non-decreasing: count the entries <= pos,
    // 64 at a time)
    int b = -1;
    for (int base = 0; base < a.B; base += 64) {
        const bool le = base + lane < a.B && a.cu[base + lane] <= pos;
        const uint64_t m = __ballot(le);
        b += (int)__popcll(m);
        if (m != ~0ull) break;
    }
    while (pos < end) {
        while (a.cu[b + 1] <= pos) ++b;   // skips empty sequences
        const int64_t seg_end = min(end, a.cu[b + 1]);
        // keys s_begin .. s_end - 1 of sequence b (s_begin a multiple of 64)
        const int s_begin = (int)(pos - a.cu[b]);
        const int s_end = min(clamp_len(a, b), (int)(seg_end - a.cu[b]));
        const DecodePlan pl = a.plan[b];
        Sc sc;
        sc.init(kp, a.start, b, l16, lg);
        unsigned char *const slot = slots + (size_t)wave * Sc::kSlotBytes;
        // keys past the end are the last key again
        int g0 = s_begin;
        if (g0 < s_end) sc.stage(slot, g0, s_end - 1, lane);
        // group g (staged) into registers, its scale kept, and group g + 64 requested into the slot
        auto next = [&](int g) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            sc.load_staged(slot, l16, lg);
            const float scl = sc.scale();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (g + 64 < s_end) sc.stage(slot, g + 64, s_end - 1, lane);
            return scl;
        };
        if (pl.dense) {
            // every lane stores (past the end lie the row's padding positions)
            float *out = a.score_buf + (int64_t)b * a.ld;
            for (; g0 < s_end; g0 += 64) {
                const float scl = next(g0);
                float p[4];
                sc.partial(p);
                out[g0 + lane] = finish(sc, p, scl, lg);
            }
        } else {
            // key >= theta  <=>  score >= the score of theta (the keys order the scores)
            const bool every = pl.theta == 0u;
            const float th = key_score(every ? 1u : pl.theta);
            uint2 *list = a.cand + pos;   // this piece's list (room for one entry per position)
            int nst = 0, nfl = 0;         // candidates staged, flushed
            for (; g0 < s_end; g0 += 64) {
                const float scl = next(g0);
                float p[4];
                sc.partial(p);
                const float v = finish(sc, p, scl, lg);
                const bool c = g0 + lane < s_end && (every || v >= th);
                const uint64_t m = __ballot(c);
                if (m) {
                    if (c) rw[(nst + (int)bits_below(m)) & 127] = make_uint2(__float_as_uint(v), (uint32_t)(g0 + lane));
                    nst += (int)__popcll(m);
                    __builtin_amdgcn_wave_barrier();
                    if (nst - nfl >= 64) {
                        list[nfl + lane] = rw[(nfl + lane) & 127];
                        nfl += 64;
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            if (lane < nst - nfl) list[nfl + lane] = rw[(nfl + lane) & 127];
            if (lane == 0) a.cnt[pos / 64] = nst;
        }
        pos = seg_end;
    }
}

// ---------------------------------------------------------------- pass 3: select
template <class Sc, class Keys>
__global__ __launch_bounds__(kSelectThreads) void decode_select_kernel(DecCommon a, Keys kp) {
    __shared__ TopkSmem<16> sm;
    const int b = blockIdx.x, tid = threadIdx.x;
    const int topk = a.topk;
    const int n = clamp_len(a, b);
    int32_t *oi = a.idx + (int64_t)b * topk;
    float *os = a.scores ? a.scores + (int64_t)b * topk : nullptr;
    TopkArgs ta{};
    ta.scores = a.score_buf;
    ta.mode = 1;
    ta.seqlens = a.seqlens;
    ta.ld = a.ld;
    ta.nmax = a.max_seqlen;
    ta.B = a.B;
    ta.topk = topk;
    ta.out_idx = a.idx;
    ta.out_score = a.scores;
    const DecodePlan pl = a.plan[b];
    // the row's pieces: one from cu[b], then one from every multiple of sub inside the row
    const int64_t c0 = a.cu[b];
    const int64_t sub = decode_sub(a.cu[a.B], a.filter_grid, a.max_seqlen);
    const int np = n > 0 ? (int)((c0 + n - 1) / sub - c0 / sub) + 1 : 0;
    const bool fits = np <= kMaxPieces<16>;
    int c = 0;
    if (!pl.dense && fits && np > 0) {
        int run = 0;
        for (int j0 = 0; j0 < np; j0 += kSelectThreads) {
            const int j = j0 + tid;
            int cj = 0;
            if (j < np) {
                const int64_t st = j == 0 ? c0 : (c0 / sub + j) * sub;
                sm.u.pc.start[j] = st;
                cj = a.cnt[st / 64];
            }
            int tot;
            const int incl = block_inclusive_sum(cj, tot, sm);
            if (j < np) sm.u.pc.off[j] = run + incl - cj;
            run += tot;
        }
        if (tid == 0) sm.u.pc.off[np] = run;
        c = run;
        __syncthreads();
    }
    const int need_min = n < topk ? n : topk;
    if (!pl.dense && (!fits || c < need_min || c > kCand<16>)) {
        // the sample overshot (or the list does not fit): score the whole row again
        Sc::stage(kp, b, sm.u.resc.q, sm.u.resc.w);
        __syncthreads();
        float *row = a.score_buf + (int64_t)b * a.ld;
        for (int s = tid; s < n; s += kSelectThreads)
            row[s] = Sc::rescore(kp, a.start, b, s, sm.u.resc.q, sm.u.resc.w);
        __threadfence();
        __syncthreads();
        c = -1;
    }
    if (pl.dense || c < 0) {   // all the row's scores are in score_buf
        row_topk_row<16>(ta, b, sm);
        return;
    }
    // Candidates to registers, entry e = tid + 1024 i (list order is index order), so that the
    // loads of a wave cover consecutive entries.  blk[k]: the piece of entry 64 k.
    for (int j = tid; j < np; j += kSelectThreads) {
        const int lo = sm.u.pc.off[j], hi = sm.u.pc.off[j + 1];
        for (int k = (lo + 63) >> 6; (k << 6) < hi; ++k) sm.u.pc.blk[k] = j;
    }
    __syncthreads();
    uint32_t key[kPer];
    int32_t kidx[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = tid + kSelectThreads * i;
        key[i] = 0u;
        kidx[i] = 0;
        if (e < c) {
            int j = sm.u.pc.blk[e >> 6];
            while (sm.u.pc.off[j + 1] <= e) ++j;
            const uint2 v = a.cand[sm.u.pc.start[j] + (e - sm.u.pc.off[j])];
            key[i] = score_key(__uint_as_float(v.x));
            kidx[i] = (int32_t)v.y;
        }
    }
    if (tid < kCand<16> / 32) sm.win[tid] = 0u;
    if (tid == 0) sm.nbin = 0u;
    __syncthreads();
    // Winners: keys above hi, plus, among keys in [lo, hi], those whose bit is set in win (the
    // bin ranked exactly) or, for a crowded bin narrowed to one value (lo == hi == theta), the
    // first eq_need of them in entry order.
    uint32_t lo = 1u, hi = 0u;   // c <= topk: every candidate wins
    int eq_need = -1;            // -1: bin members win by their bit
    if (c > topk) {
        uint32_t m = 0, mn = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            m = key[i] > m ? key[i] : m;
            mn = key[i] != 0u && key[i] < mn ? key[i] : mn;
        }
        const uint32_t top = block_max(m, sm);
        const uint32_t bot = ~block_max(~mn, sm);
        const int nb = bit_width(top - bot);
        const int sh = nb > kDigit<16> ? nb - kDigit<16> : 0;   // kBins bins of 2^sh from bot
        for (int x = tid; x < kBins<16>; x += kSelectThreads) sm.hist[x] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (key[i] != 0u) atomicAdd(&sm.hist[(key[i] - bot) >> sh], 1u);
        __syncthreads();
        int need = topk, in_bin;
        const uint32_t d = pick_digit(need, sm, &in_bin);   // need: winners inside bin d
        const uint64_t lo64 = (uint64_t)bot + ((uint64_t)d << sh);
        lo = (uint32_t)lo64;
        hi = (uint32_t)(lo64 + (1ull << sh) - 1ull);
        if (in_bin <= kRankMax) {
            // rank the bin's keys exactly: by key, then lower index first; the need best win
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                if (key[i] >= lo && key[i] <= hi) {
                    const uint32_t slot = atomicAdd(&sm.nbin, 1u);
                    sm.bin.key[slot] = key[i];
                    sm.bin.idx[slot] = kidx[i];
                    sm.bin.slot[slot] = (uint16_t)(tid + kSelectThreads * i);
                }
            }
            __syncthreads();
            if (tid < in_bin) {
                const uint32_t mk = sm.bin.key[tid];
                const int32_t mi = sm.bin.idx[tid];
                int rank = 0;
                for (int x = 0; x < in_bin; ++x) {
                    const uint32_t ok = sm.bin.key[x];
                    rank += (ok > mk || (ok == mk && sm.bin.idx[x] < mi)) ? 1 : 0;
                }
                if (rank < need) {
                    const int e = sm.bin.slot[tid];
                    atomicOr(&sm.win[e >> 5], 1u << (e & 31));
                }
            }
            __syncthreads();
        } else {
            // a crowded bin: narrow it to one key value by an exact select over its keys
            uint32_t kb[kPer];
            uint32_t bmax = 0;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                kb[i] = key[i] >= lo && key[i] <= hi ? key[i] : 0u;
                bmax = kb[i] > bmax ? kb[i] : bmax;
            }
            const uint32_t theta = select_rel(kb, lo, bit_width(block_max(bmax, sm) - lo), need, sm);
            lo = hi = theta;
            eq_need = need;
        }
    }
    // Output positions in entry order: per entry row i, the winners of the earlier rows, of
    // the earlier waves in row i and of the lower lanes.
    const int lane = tid & 63, wave = tid >> 6;
    bool win[kPer];
    if (eq_need >= 0) {
        // ties at theta: the first eq_need in entry order win
        uint64_t em[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            em[i] = __ballot(key[i] == lo);
            if (lane == 0) sm.u.ecnt[i * 16 + wave] = (int)__popcll(em[i]);
        }
        __syncthreads();
        if (tid < 64) {   // exclusive prefix over the 256 (row, wave) counts
            int v[4], sum = 0;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                v[x] = sm.u.ecnt[4 * tid + x];
                sum += v[x];
            }
            int run = wave_inclusive_sum(sum) - sum;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                sm.u.ecnt[4 * tid + x] = run;
                run += v[x];
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int r = sm.u.ecnt[i * 16 + wave] + (int)bits_below(em[i]);
            win[i] = key[i] > hi || (key[i] == lo && r < eq_need);
        }
        __syncthreads();
    } else {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = tid + kSelectThreads * i;
            win[i] = key[i] != 0u &&
                     (key[i] > hi || (key[i] >= lo && ((sm.win[e >> 5] >> (e & 31)) & 1u)));
        }
    }
    uint64_t wm[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        wm[i] = __ballot(win[i]);
        if (lane == 0) sm.u.ecnt[i * 16 + wave] = (int)__popcll(wm[i]);
    }
    __syncthreads();
    if (tid < 64) {
        int v[4], sum = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            v[x] = sm.u.ecnt[4 * tid + x];
            sum += v[x];
        }
        int run = wave_inclusive_sum(sum) - sum;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            sm.u.ecnt[4 * tid + x] = run;
            run += v[x];
        }
        if (tid == 63) sm.bcast[0] = run;
    }
    __syncthreads();
    const int wrote = sm.bcast[0];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (win[i]) {
            const int pos = sm.u.ecnt[i * 16 + wave] + (int)bits_below(wm[i]);
            oi[pos] = kidx[i];
            if (os) os[pos] = key_score(key[i]);
        }
    }
    for (int i = wrote + tid; i < topk; i += kSelectThreads) {
        oi[i] = -1;
        if (os) os[i] = -INFINITY;
    }
}

// cu[b] = sum over i < b of pad64(min(max(seqlens[i], 0), max_seqlen)), b = 0 .. B (batches
// too large for the plan pass to sum itself).
__global__ __launch_bounds__(1024) void decode_prefix_kernel(const int32_t *seqlens, int B,
                                                              int max_seqlen, int64_t *cu) {
    __shared__ int64_t part[1024];
    const int tid = threadIdx.x;
    const int per = (B + 1023) / 1024;
    const int i0 = tid * per, i1 = min(B, i0 + per);
    auto len = [&](int i) { return pad64(max(0, min(seqlens[i], max_seqlen))); };
    int64_t s = 0;
    for (int i = i0; i < i1; ++i) s += len(i);
    part[tid] = s;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {   // inclusive scan of the partial sums
        const int64_t o = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += o;
        __syncthreads();
    }
    int64_t run = tid ? part[tid - 1] : 0;
    for (int i = i0; i < i1; ++i) {
        cu[i] = run;
        run += len(i);
    }
    if (tid == 1023) cu[B] = part[1023];
}

template <class K>
int filter_grid(K kernel, size_t smem) {
    static DeviceInt cached;
    return cached.get([&] {
        int dev = 0, cus = 0, per = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kFilterThreads, smem) != hipSuccess || per <= 0)
            per = 2;
        return 2 * per * cus;   // two rounds of the workgroups resident at once
    });
}

// The filter's dynamic LDS (the key slots) may exceed the default limit: raised once per device.
template <class Sc, class Keys>
hipError_t filter_attr() {
    static DeviceOnce once;
    return once.run([] {
        return hipFuncSetAttribute(reinterpret_cast<const void *>(decode_filter_kernel<Sc, Keys>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)filter_smem<Sc>());
    });
}

template <class Sc, class Keys>
hipError_t run_decode(const Keys &kp, const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                      int topk, const DecodeWs &w, int32_t *idx, float *scores, hipStream_t stream) {
    DecCommon a{};
    a.start = start;
    a.seqlens = seqlens;
    a.B = B;
    a.max_seqlen = max_seqlen;
    a.topk = topk;
    a.cu = w.cu;
    a.plan = reinterpret_cast<DecodePlan *>(w.plan);
    a.cnt = w.cnt;
    a.cand = reinterpret_cast<uint2 *>(w.cand);
    a.score_buf = w.score_buf;
    a.skey = w.skey;
    a.ld = decode_row_stride(max_seqlen);
    a.idx = idx;
    a.scores = scores;
    const int64_t bound = ((int64_t)B * (decode_row_stride(max_seqlen) / 64) + 3) / 4;   // 4 waves of 64 keys
    hipError_t e = filter_attr<Sc, Keys>();
    if (e != hipSuccess) return e;
    const int g = filter_grid(decode_filter_kernel<Sc, Keys>, filter_smem<Sc>());
    a.filter_grid = (int)(bound < g ? (bound > 0 ? bound : 1) : g);
    const int own = B <= kPlanPrefixMax ? 1 : 0;
    if (!own) {
        hipLaunchKernelGGL(decode_prefix_kernel, dim3(1), dim3(1024), 0, stream, seqlens, B, max_seqlen, w.cu);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((decode_sample_kernel<Sc, Keys>), dim3(B * kSampleParts), dim3(kSampleThreads), 0, stream,
                       a, kp, own);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_threshold_kernel, dim3(B), dim3(kPlanThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_filter_kernel<Sc, Keys>), dim3(a.filter_grid), dim3(kFilterThreads), filter_smem<Sc>(),
                       stream, a, kp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_select_kernel<Sc, Keys>), dim3(B), dim3(kSelectThreads), 0, stream, a, kp);
    return hipGetLastError();
}

size_t r256(size_t b) { return (b + 255u) & ~(size_t)255u; }

}  // namespace

size_t decode_workspace(int B, int max_seqlen, bool fp8, DecodeWs *w, void *base) {
    const size_t Bs = (size_t)(B > 0 ? B : 0);
    const size_t flat = Bs * (size_t)decode_row_stride(max_seqlen);   // padded positions
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += r256(bytes);
        return o;
    };
    const size_t o_cu = take(8u * (Bs + 1));
    const size_t o_plan = take(8u * Bs);
    const size_t o_cnt = take(4u * (flat / 64 + 1));
    const size_t o_cand = take(8u * flat);
    const size_t o_sb = take(4u * flat);
    const size_t o_sk = take(4u * Bs * kSampleMax);
    const size_t o_q8 = fp8 ? take(Bs * 2 * kQOut) : 0;      // room for 64 heads
    const size_t o_qw = fp8 ? take(4u * Bs * 2 * kHeads) : 0;
    if (w && base) {
        char *p = static_cast<char *>(base);
        w->cu = reinterpret_cast<int64_t *>(p + o_cu);
        w->plan = reinterpret_cast<uint64_t *>(p + o_plan);
        w->cnt = reinterpret_cast<int32_t *>(p + o_cnt);
        w->cand = reinterpret_cast<uint64_t *>(p + o_cand);
        w->score_buf = reinterpret_cast<float *>(p + o_sb);
        w->skey = reinterpret_cast<uint32_t *>(p + o_sk);
        w->q8 = fp8 ? reinterpret_cast<uint8_t *>(p + o_q8) : nullptr;
        w->qw = fp8 ? reinterpret_cast<float *>(p + o_qw) : nullptr;
    }
    return off;
}

hipError_t launch_decode(const uint16_t *q, const uint16_t *w, const uint16_t *k_cache,
                         const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                         int topk, void *ws, int32_t *idx, float *scores, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    DecodeWs dw{};
    decode_workspace(B, max_seqlen, false, &dw, ws);
    return run_decode<Bf16Scorer>(Bf16Keys{q, w, k_cache}, start, seqlens, B, max_seqlen, topk, dw, idx,
                                  scores, stream);
}

hipError_t launch_decode_v32(const uint16_t *q, const uint16_t *w, const uint16_t *k_cache,
                             const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                             int topk, void *ws, int32_t *idx, float *scores, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    DecodeWs dw{};
    decode_workspace(B, max_seqlen, false, &dw, ws);
    return run_decode<Bf16ScorerT<4>>(Bf16Keys{q, w, k_cache}, start, seqlens, B, max_seqlen, topk, dw, idx,
                                      scores, stream);
}

hipError_t launch_decode_fp8(const uint16_t *q, const uint16_t *w, const uint8_t *k8, const float *kscale,
                             const int64_t *start, const int32_t *seqlens, int B, int max_seqlen, int topk,
                             void *ws, int32_t *idx, float *scores, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    DecodeWs dw{};
    decode_workspace(B, max_seqlen, true, &dw, ws);
    hipError_t e = launch_quantize_queries(q, w, B, kHeads, dw.q8, dw.qw, stream);
    if (e != hipSuccess) return e;
    return run_decode<Fp8Scorer>(Fp8Keys{dw.q8, dw.qw, k8, kscale}, start, seqlens, B, max_seqlen, topk, dw,
                                 idx, scores, stream);
}

hipError_t launch_decode_fp8_v32(const uint16_t *q, const uint16_t *w, const uint8_t *k8, const float *kscale,
                                 const int64_t *start, const int32_t *seqlens, int B, int max_seqlen, int topk,
                                 void *ws, int32_t *idx, float *scores, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    DecodeWs dw{};
    decode_workspace(B, max_seqlen, true, &dw, ws);
    hipError_t e = launch_quantize_queries(q, w, B, 2 * kHeads, dw.q8, dw.qw, stream);
    if (e != hipSuccess) return e;
    return run_decode<Fp8ScorerT<4>>(Fp8Keys{dw.q8, dw.qw, k8, kscale}, start, seqlens, B, max_seqlen, topk, dw,
                                     idx, scores, stream);
}

}  // namespace dsaidx
