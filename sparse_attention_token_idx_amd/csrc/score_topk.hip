// Fused causal indexer scores + streaming top-k for prefill (dense and varlen).
//
// Computes, for every query row t of a sequence, I[t,s] = sum_h w[t,h] * ReLU(q[t,h].k[s])
// over its whole causal prefix s <= t and keeps the topk largest (ties -> lower s), as
// fixed on the "Qwen3.5-397B-A17B vs Kimi K3.1 Pro" compare page (component table,
// sparse/compressed-attention row) with the whole prefix scored (long-context row of the
// "Kimi K3.1 Pro vs Gemma 4 31B" page).  The T x T score matrix never reaches memory.
//
// One workgroup (8 waves) owns 32 query rows and streams the keys of their prefix in
// tiles of 64:
//   * wave (qg, hg) keeps the bf16 q of 16 queries x 8 heads in registers (B operand) and
//     runs q.k for each head on v_mfma_f32_16x16x32_bf16 with the key tile (A operand, read
//     from LDS), then applies ReLU and the w-weighted sum over its 8 heads in registers;
//   * the four head groups' partial sums meet in LDS and are added in a fixed order;
//   * each wave then owns 4 rows.  A key whose score beats the row's emit threshold is
//     appended, in ascending s, to the row's candidate list in the workspace, and counted
//     in the row's LDS histogram: 512 bins of 1/32 binade over the orderable key, placed
//     just below the row's largest score.  As soon as the bins above the threshold's bin
//     hold topk candidates the threshold moves up to the next bin edge.  Later keys have
//     larger s and so lose every tie against candidates already kept, hence the strict
//     ">" emission rule never drops a winner.  Nothing is re-read while streaming, except
//     in the rare case that a list fills up (it is then compacted).
//   * at the end only the threshold bin needs an exact decision: its few candidates are
//     gathered, the exact boundary key and its tie count are found with a bitwise search,
//     and one ordered pass over the list writes the topk winners in ascending s.
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

constexpr int kBQ = 32;               // query rows per workgroup
constexpr int kBK = 64;               // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKStride = kDim + 8;    // bf16 per key row in LDS (272 B: conflict-free reads)
constexpr int kRStride = kBK + 4;     // floats per row of the partial-score tile (272 B)
constexpr int kNB = 256;              // histogram bins per row (8 binades)
constexpr int kRing = 128;            // per-row LDS staging ring of pending candidates
constexpr int kBinShift = 18;         // a bin is a 14-bit key prefix: 1/32 binade
constexpr int kGather = 1024;         // per-wave buffer for the threshold bin's keys

struct ScoreSmem {
    uint16_t k[2][kBK][kKStride];      // double-buffered key tile
    float red[2][4][kBQ][kRStride];    // double-buffered partial scores [buf][hg][query][key]
    uint32_t hist[kBQ / 2][kNB];       // candidate histograms, 16-bit counts, two rows a word
    uint64_t ring[kBQ][kRing];         // pending candidates (key | index << 32) per row
    uint64_t trash[kWaves][64];        // write target of lanes with nothing to emit
};
// the final phase reuses k and red as per-wave gather buffers
static_assert(kWaves * kGather * 4 <= sizeof(uint16_t) * 2 * kBK * kKStride + sizeof(float) * 8 * kBQ * kRStride,
              "gather buffers must fit in the key and partial-score tiles");

// One row's 16-bit histogram counters (the low or high halves of a shared word array).
// Both rows of a word belong to the same wave, so plain read-modify-writes are safe.
struct RowHist {
    uint32_t *w;
    int sh;
    __device__ int get(int b) const { return (int)((w[b] >> sh) & 0xFFFFu); }
    __device__ void inc(int b) const { atomicAdd(&w[b], 1u << sh); }
};

struct ScoreArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *w;
    const int32_t *cu_seqlens;  // nullptr: one sequence of length T
    int64_t T;
    int nrb;                    // grid.y: row blocks of the longest sequence
    int topk;
    int cap;                    // candidate slots per row
    uint32_t *cand_key;
    int32_t *cand_idx;
    int32_t *out_idx;
    float *out_score;           // may be nullptr
};

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------- histogram window
// Bins are consecutive 14-bit prefixes of the orderable key, bin 0 taking everything below
// the window and bin kNB-1 everything above.  The window ends one binade above the row's
// largest key seen when it was placed.
__device__ __forceinline__ int window_base(uint32_t kmax) {
    int top = (int)(kmax >> kBinShift) + 32;
    if (top > (1 << (32 - kBinShift)) - 1) top = (1 << (32 - kBinShift)) - 1;
    const int base = top - (kNB - 1);
    return base < 0 ? 0 : base;
}
__device__ __forceinline__ int bin_of(uint32_t key, int pbase) {
    const int b = (int)(key >> kBinShift) - pbase;
    return b < 0 ? 0 : (b >= kNB ? kNB - 1 : b);
}
// Smallest key of bin b (b >= 1).
__device__ __forceinline__ uint32_t bin_edge(int b, int pbase) {
    return (uint32_t)(pbase + b) << kBinShift;
}

// Maximum over each 16-lane row (DPP row-shift max scan, then the row's last lane).
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
    int x = (int)v;
#define DSA_ROWMAX_STEP(ctrl)                                                         \
    {                                                                                 \
        const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, x, ctrl, 0xF, 0xF, true); \
        x = (int)(o > (uint32_t)x ? o : (uint32_t)x);                                 \
    }
    DSA_ROWMAX_STEP(0x111) DSA_ROWMAX_STEP(0x112) DSA_ROWMAX_STEP(0x114) DSA_ROWMAX_STEP(0x118)
#undef DSA_ROWMAX_STEP
    return (uint32_t)row16_last(x);
}

__device__ __forceinline__ uint32_t group16_max(uint32_t v) {
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)v, d, 64);
        v = o > v ? o : v;
    }
    return v;
}

// ---------------------------------------------------------------- whole-wave list passes
// Histogram of keys[0..n) into hist[kNB] (zeroed first).  Entries are read in batches of B
// per lane so that many loads are in flight.
template <int B>
__device__ void wave_fill_hist(const uint32_t *keys, int n, RowHist hist, int pbase) {
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < kNB / 64; ++i) hist.w[lane + 64 * i] &= ~(0xFFFFu << hist.sh);
    wave_sync_lds();
    for (int base = 0; base < n; base += 64 * B) {
        uint32_t kv[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int i = base + 64 * j + lane;
            kv[j] = keys[i < n ? i : n - 1];
        }
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (base + 64 * j + lane < n) hist.inc(bin_of(kv[j], pbase));
    }
    wave_sync_lds();
}

// Stable in-place compaction keeping keys >= min_key; returns the new length.  A batch is
// loaded before any of its slots is written and writes never pass the batch being read.
template <int B>
__device__ int wave_keep_at_least(uint32_t *keys, int32_t *ids, int n, uint32_t min_key) {
    const int lane = lane_id();
    int out = 0;
    for (int base = 0; base < n; base += 64 * B) {
        uint32_t kv[B];
        int32_t iv[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int i = base + 64 * j + lane;
            kv[j] = keys[i < n ? i : n - 1];
            iv[j] = ids[i < n ? i : n - 1];
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const bool keep = base + 64 * j + lane < n && kv[j] >= min_key;
            const uint64_t km = ballot(keep);
            if (keep) {
                const int pos = out + (int)bits_below(km);
                keys[pos] = kv[j];
                ids[pos] = iv[j];
            }
            out += __popcll(km);
        }
    }
    __threadfence();
    return out;
}

// Exact selection over a whole list (the rare path): an MSD radix select on 8-bit digits
// finds theta, the topk-th largest key, and how many entries equal to theta win the tie
// (the lowest indices, i.e. the earliest list positions); the list is then compacted in
// place (stable) to exactly those topk entries.  s0 and s1 are two scratch histograms of
// 256 words each (lanes alternate between them).  Returns theta.
template <int B>
__device__ uint32_t wave_exact_select(uint32_t *keys, int32_t *ids, int n, int topk, uint32_t *s0,
                                      uint32_t *s1) {
    const int lane = lane_id();
    uint32_t prefix = 0, pmask = 0;
    int need = topk;
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s0[lane + 64 * i] = 0u;
            s1[lane + 64 * i] = 0u;
        }
        wave_sync_lds();
        uint32_t *h = (lane & 1) ? s1 : s0;
        for (int base = 0; base < n; base += 64 * B) {
            uint32_t kv[B];
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const int i = base + 64 * j + lane;
                kv[j] = keys[i < n ? i : n - 1];
            }
#pragma unroll
            for (int j = 0; j < B; ++j)
                if (base + 64 * j + lane < n && (kv[j] & pmask) == prefix)
                    atomicAdd(&h[(kv[j] >> shift) & 255u], 1u);
        }
        wave_sync_lds();
        int c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 4 * lane + j;
            c[j] = (int)(s0[b] + s1[b]);
        }
        const int incl = wave_inclusive_sum(c[0] + c[1] + c[2] + c[3]);
        int above = readlane(incl, 63) - incl;   // entries in digits above 4*lane+3
        int found = -1, found_above = 0;
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            if (found < 0 && above < need && need <= above + c[j]) {
                found = 4 * lane + j;
                found_above = above;
            }
            above += c[j];
        }
        const int src = (int)__builtin_ctzll(ballot(found >= 0));
        need -= readlane(found_above, src);
        prefix |= (uint32_t)readlane(found, src) << shift;
        pmask |= 255u << shift;
        wave_sync_lds();
    }
    const uint32_t theta = prefix;
    int out = 0, ties = 0;
    for (int base = 0; base < n; base += 64 * B) {
        uint32_t kv[B];
        int32_t iv[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int i = base + 64 * j + lane;
            kv[j] = keys[i < n ? i : n - 1];
            iv[j] = ids[i < n ? i : n - 1];
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const bool in = base + 64 * j + lane < n;
            const bool eq = in && kv[j] == theta;
            const uint64_t em = ballot(eq);
            const bool keep = (in && kv[j] > theta) || (eq && ties + (int)bits_below(em) < need);
            const uint64_t km = ballot(keep);
            if (keep) {
                const int pos = out + (int)bits_below(km);
                keys[pos] = kv[j];
                ids[pos] = iv[j];
            }
            out += __popcll(km);
            ties += __popcll(em);
        }
    }
    __threadfence();
    return theta;
}

// Largest v such that at least `need` of the m keys in g (m <= 1024, zero padded) are >= v:
// the need-th largest key.  Bitwise search, counts reduced over the wave.
__device__ uint32_t wave_kth_largest(const uint32_t (&g)[kGather / 64], int need) {
    uint32_t v = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = v | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < kGather / 64; ++j) cnt += g[j] >= c ? 1 : 0;
        if (wave_sum(cnt) >= need) v = c;
    }
    return v;
}

__global__ __launch_bounds__(kThreads, 1) void score_topk_kernel(ScoreArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ScoreSmem &sm = *reinterpret_cast<ScoreSmem *>(smem_raw);

    const int seq = blockIdx.x;
    const int rb = a.nrb - 1 - (int)blockIdx.y;   // longest rows first
    int64_t seq_start = 0, L = a.T;
    if (a.cu_seqlens) {
        seq_start = a.cu_seqlens[seq];
        L = (int64_t)a.cu_seqlens[seq + 1] - seq_start;
    }
    const int64_t r0 = (int64_t)rb * kBQ;
    if (r0 >= L) return;
    const int rows_here = (int)(L - r0 < kBQ ? L - r0 : kBQ);
    const int64_t r_last = r0 + rows_here - 1;
    const int nkt = (int)(r_last / kBK) + 1;
    const int topk = a.topk, cap = a.cap;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int qg = wave & 1, hg = wave >> 1;
    const int l16 = lane & 15, lg = lane >> 4;

    // ---- q fragments (B operand) and head weights for 16 queries x 8 heads
    u32x4 qf[8][4];
    float wv[8];
    {
        const int row = 16 * qg + l16;
        const bool ok = row < rows_here;
        const int64_t g = seq_start + r0 + (ok ? row : 0);
        const uint16_t *qrow = a.q + g * kQOut + (8 * hg) * kDim + 8 * lg;
#pragma unroll
        for (int h = 0; h < 8; ++h) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qf[h][ks] = *reinterpret_cast<const u32x4 *>(qrow + h * kDim + 32 * ks);
            wv[h] = bf16_to_f32(a.w[g * kHeads + 8 * hg + h]);
        }
        if (!ok) {   // rows past the end: zero queries (row 0's data was loaded in their place)
#pragma unroll
            for (int h = 0; h < 8; ++h) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) qf[h][ks] = u32x4{0u, 0u, 0u, 0u};
                wv[h] = 0.f;
            }
        }
    }

    // ---- key tile staging: thread -> key tid/8, 32 bytes at dim 16*(tid%8)
    const int st_key = tid >> 3, st_dim = 16 * (tid & 7);
    u32x4 kv0, kv1;
    // Keys past the sequence end are loaded from its last row instead (never a branch, so
    // the load never waits for earlier stores); the causal mask discards their scores.
    auto load_k = [&](int kt) {
        int64_t s = (int64_t)kt * kBK + st_key;
        s = s < L ? s : L - 1;
        const uint16_t *p = a.k + (seq_start + s) * kDim + st_dim;
        kv0 = *reinterpret_cast<const u32x4 *>(p);
        kv1 = *reinterpret_cast<const u32x4 *>(p + 8);
    };
    auto store_k = [&](int buf) {
        uint16_t *p = &sm.k[buf][st_key][st_dim];
        *reinterpret_cast<u32x4 *>(p) = kv0;
        *reinterpret_cast<u32x4 *>(p + 8) = kv1;
    };

    // ---- state of the row this lane's 16-lane group emits for (row 4*wave + lg);
    // every value except kmax is uniform within the group
    const int er = 4 * wave + lg;
    const bool erow_ok = er < rows_here;
    const int et32 = (int)(r0 + er);                     // its position in the sequence
    const int64_t egrow = seq_start + r0 + (erow_ok ? er : 0);
    uint32_t *ck = a.cand_key + egrow * cap;
    int32_t *ci = a.cand_idx + egrow * cap;
    uint64_t *ring = sm.ring[er];
    const RowHist rh{sm.hist[er >> 1], 16 * (er & 1)};
    // emit key > theta (0 is below every finite score's key; rows past the end never emit)
    uint32_t theta = erow_ok ? 0u : 0xFFFFFFFFu;
    int n = 0;             // candidates already in the list in memory
    int p = 0;             // candidates pending in the LDS ring, starting at slot head
    int head = 0;
    bool hv = false;       // histogram placed
    int pbase = 0;         // histogram window
    int bth = 0;           // bin of the threshold: bins >= bth hold the live candidates
    int cum = 0;           // number of candidates in bins >= bth
    uint32_t kmax = 0u;    // largest key this lane has written to the list
    uint64_t *const trash = &sm.trash[wave][lane];

    int live_pend = 0;     // flushed candidates in bins >= bth not yet added to cum (per lane)
    bool dirty = false;    // flushed since the last advance

    // Move the threshold up while the bins above bth alone hold topk candidates.
    auto advance = [&]() {
        for (;;) {
            const int h = rh.get(bth);
            if (bth < kNB - 1 && cum - h >= topk) {
                cum -= h;
                ++bth;
                const uint32_t e = bin_edge(bth, pbase);
                theta = e > theta ? e : theta;
            } else {
                break;
            }
        }
    };
    // Fold the flushed candidates into cum and advance (row-wide).
    auto settle = [&]() {
        cum += row16_last(row16_inclusive_sum(live_pend));
        live_pend = 0;
        dirty = false;
        advance();
    };
    // Place the histogram window for a row whose largest candidate so far is m.
    auto place = [&](uint32_t m) {
        pbase = window_base(m);
        hv = true;
        bth = 0;
        cum = 0;
    };
    auto account = [&](uint32_t key) {
        kmax = key > kmax ? key : kmax;
        const int b = bin_of(key, pbase);
        rh.inc(b);
        live_pend += b >= bth ? 1 : 0;
    };
    // Write 64 pending candidates of the ring to the list with 16-byte stores (row-wide).
    // The first flush of a row places its histogram window from these 64 keys.
    auto flush64 = [&]() {
        const uint64_t *src = ring + head + 4 * l16;
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(src);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(src + 2);
        const u32x4a4 kv = {lo[0], lo[2], hi[0], hi[2]};
        const u32x4a4 iv = {lo[1], lo[3], hi[1], hi[3]};
        *reinterpret_cast<u32x4a4 *>(ck + n + 4 * l16) = kv;
        *reinterpret_cast<u32x4a4 *>(ci + n + 4 * l16) = iv;
        if (!hv) {
            uint32_t m = kv[0] > kv[1] ? kv[0] : kv[1];
            const uint32_t m2 = kv[2] > kv[3] ? kv[2] : kv[3];
            place(row16_max(m > m2 ? m : m2));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) account(kv[i]);
        n += 64;
        p -= 64;
        head ^= 64;
        dirty = true;
    };
    // Write every pending candidate of the ring to the list and settle (row-wide).
    auto flush_all = [&]() {
        if (!hv && n + p > topk) {
            uint32_t m = kmax;
            for (int i = l16; i < p; i += 16) {
                const uint32_t k = (uint32_t)ring[(head + i) & (kRing - 1)];
                m = k > m ? k : m;
            }
            place(row16_max(m));
            // candidates already in the list were written before the window existed
            for (int i = l16; i < n; i += 16) account(ck[i]);
        }
        for (int i = l16; i < p; i += 16) {
            const uint64_t e = ring[(head + i) & (kRing - 1)];
            ck[n + i] = (uint32_t)e;
            ci[n + i] = (int32_t)(e >> 32);
            if (hv) account((uint32_t)e);
        }
        n += p;
        p = 0;
        head = 0;
        if (hv) {
            wave_sync_lds();
            settle();
        }
    };

    // ---- candidates of tile ke for row er: this lane covers keys 4*l16 .. 4*l16+3.
    // Only LDS is touched: every lane writes all four slots, the losers to its trash slot,
    // and positions come from a prefix sum over the row's 16 lanes.  Straight-line code (en
    // false: nothing is emitted), so that it can be interleaved with the matrix products.
    // A summed score is never -0 (every partial sum starts from +0, and in round-to-nearest
    // an exact zero of nonzero terms is +0), so the shorter key map applies.
    auto emit_core = [&](int ke, bool en) {
        const int rb2 = ke & 1;
        f32x4 v = *reinterpret_cast<const f32x4 *>(&sm.red[rb2][0][er][4 * l16]);
#pragma unroll
        for (int g = 1; g < 4; ++g) v += *reinterpret_cast<const f32x4 *>(&sm.red[rb2][g][er][4 * l16]);
        const int s0 = ke * kBK + 4 * l16;
        uint32_t kk[4];
        bool e[4];
        int c = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            kk[j] = score_key_nz(v[j]);
            e[j] = en && kk[j] > theta && s0 + j <= et32;
            c += e[j] ? 1 : 0;
        }
        const int incl = row16_inclusive_sum(c);
        int pos = head + p + incl - c;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint64_t *dst = e[j] ? ring + (pos & (kRing - 1)) : trash;
            *dst = (uint64_t)kk[j] | ((uint64_t)(uint32_t)(s0 + j) << 32);
            pos += e[j] ? 1 : 0;
        }
        p += row16_last(incl);
    };

    // ---- one key tile on the matrix cores, software pipelined.  A unit is 16 keys (one
    // subtile) x 16 queries x 4 heads: four independent MFMA chains over the 128 dims.  The
    // ReLU / w epilogue of each unit runs under the products of the next one, and the
    // candidates of the previous tile (emit_core) are interleaved as well; the scheduling
    // groups at the end of every unit ask for one MFMA followed by up to three VALU ops.
    // Keys past the causal end are computed like the others and masked when emitted.
    auto tile_block = [&](int kt) {
        const int buf = kt & 1;
        const uint16_t *kb = &sm.k[buf][l16][8 * lg];
        u32x4 a[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a[ks] = *reinterpret_cast<const u32x4 *>(kb + 32 * ks);
        emit_core(kt - 1, kt > 0);
        float *dst = &sm.red[buf][hg][16 * qg + l16][4 * lg];
        f32x4 prev[4];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                f32x4 cur[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) cur[h] = mfma16x16x32(a[0], qf[4 * u + h][0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int ks = 1; ks < 4; ++ks)
#pragma unroll
                    for (int h = 0; h < 4; ++h) cur[h] = mfma16x16x32(a[ks], qf[4 * u + h][ks], cur[h]);
                if (u == 1 && st < 3) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        a[ks] = *reinterpret_cast<const u32x4 *>(kb + (16 * (st + 1)) * kKStride + 32 * ks);
                }
                if (st > 0 || u > 0) {
                    // epilogue of the previous unit (heads 4*(1-u) .. of subtile st-(u==0))
                    const int pu = 1 - u;
#pragma unroll
                    for (int h = 0; h < 4; ++h)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[r] = fmaf(wv[4 * pu + h], relu(prev[h][r]), acc[r]);
                    if (u == 0) {
                        *reinterpret_cast<f32x4 *>(dst + 16 * (st - 1)) = acc;
                        acc = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
                if (u == 1 && st < 3) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
                }
#pragma unroll
                for (int h = 0; h < 4; ++h) prev[h] = cur[h];
            }
        }
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = fmaf(wv[4 + h], relu(prev[h][r]), acc[r]);
        *reinterpret_cast<f32x4 *>(dst + 48) = acc;
    };

    // ---- rare per-row work, done by the whole wave one row at a time: place the histogram
    // once a row holds more than topk candidates; compact a full list.  scratch: two
    // 256-word areas only this wave uses right now.
    auto rare = [&](uint32_t *scr0, uint32_t *scr1) {
        const uint64_t want = ballot(n + p > cap - 2 * kBK);
        if (!want) return;
        if ((want >> (16 * lg)) & 1ull) flush_all();
        const uint32_t gkmax = group16_max(kmax);
#pragma unroll 1
        for (int g = 0; g < 4; ++g) {
            if (!((want >> (16 * g)) & 1ull)) continue;
            const int row = 4 * wave + g;
            const int64_t grow = seq_start + r0 + row;
            uint32_t *rk = a.cand_key + grow * cap;
            int32_t *ri = a.cand_idx + grow * cap;
            const RowHist hist{sm.hist[row >> 1], 16 * (row & 1)};
            int ng = readlane(n, 16 * g);
            const uint32_t km = (uint32_t)readlane((int)gkmax, 16 * g);
            uint32_t th = (uint32_t)readlane((int)theta, 16 * g);
            int pb = readlane(pbase, 16 * g), bt = readlane(bth, 16 * g), cm = readlane(cum, 16 * g);
            __threadfence();
            if (bt > 0 && cm <= cap / 2) {
                // drop the dead candidates (bins below the threshold bin)
                ng = wave_keep_at_least<8>(rk, ri, ng, bin_edge(bt, pb));
                cm = ng;
            } else {
                // too many live candidates: exact select, then re-place the window
                th = wave_exact_select<8>(rk, ri, ng, topk, scr0, scr1);
                ng = topk;
                pb = window_base(km);
                wave_fill_hist<8>(rk, ng, hist, pb);
                bt = 0;
                cm = ng;
                for (;;) {
                    const int h = hist.get(bt);
                    if (bt < kNB - 1 && cm - h >= topk) {
                        cm -= h;
                        ++bt;
                        const uint32_t ed = bin_edge(bt, pb);
                        th = ed > th ? ed : th;
                    } else {
                        break;
                    }
                }
            }
            if (lg == g) {
                n = ng;
                theta = th;
                pbase = pb;
                bth = bt;
                cum = cm;
            }
        }
    };

    // ---- the stream: tile kt's products run while tile kt-1's candidates are emitted;
    // one barrier per tile
    for (int i = tid; i < (kBQ / 2) * kNB; i += kThreads) (&sm.hist[0][0])[i] = 0u;
    load_k(0);
    store_k(0);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        // always fetch a tile (the last one again at the end) and always stage it: with no
        // conditional load the compiler never waits at the top of the loop, and a wait there
        // would also wait for the candidate stores (vmcnt counts loads and stores in order)
        load_k(kt + 1 < nkt ? kt + 1 : nkt - 1);
        // fold in the last flush (its histogram updates completed before the barrier)
        if (dirty) settle();
        tile_block(kt);
        store_k((kt + 1) & 1);
        if (kt > 0) {
            // global stores go after the tile load has been consumed, so that waiting for
            // the next tile does not also wait for them
            if (p >= 64) flush64();
            const int rb2 = (kt - 1) & 1;
            rare(reinterpret_cast<uint32_t *>(&sm.red[rb2][0][4 * wave][0]),
                 reinterpret_cast<uint32_t *>(&sm.red[rb2][1][4 * wave][0]));
        }
        __syncthreads();
    }
    // candidates of the last tile
    if (dirty) settle();
    emit_core(nkt - 1, true);
    if (p >= 64) flush64();
    {
        const int rb2 = (nkt - 1) & 1;
        rare(reinterpret_cast<uint32_t *>(&sm.red[rb2][0][4 * wave][0]),
             reinterpret_cast<uint32_t *>(&sm.red[rb2][1][4 * wave][0]));
    }
    __syncthreads();

    // ---- final selection and output, one row at a time per wave
    flush_all();
    uint32_t *G = reinterpret_cast<uint32_t *>(smem_raw) + wave * kGather;
    __threadfence();
#pragma unroll 1
    for (int g = 0; g < 4; ++g) {
        const int row = 4 * wave + g;
        if (row >= rows_here) break;
        const int64_t grow = seq_start + r0 + row;
        uint32_t *rk = a.cand_key + grow * cap;
        int32_t *ri = a.cand_idx + grow * cap;
        int32_t *oi = a.out_idx + grow * topk;
        float *os = a.out_score ? a.out_score + grow * topk : nullptr;
        const int ng = readlane(n, 16 * g);
        if (ng <= topk) {
            // short row: the list is the whole causal prefix
            for (int i = lane; i < topk; i += 64) {
                const bool in = i < ng;
                oi[i] = in ? ri[i] : -1;
                if (os) os[i] = in ? key_score(rk[i]) : -INFINITY;
            }
            continue;
        }
        const int pb = readlane(pbase, 16 * g), bt = readlane(bth, 16 * g), cm = readlane(cum, 16 * g);
        const bool hvg = readlane(hv ? 1 : 0, 16 * g) != 0;
        const int m = hvg ? RowHist{sm.hist[row >> 1], 16 * (row & 1)}.get(bt) : 0;   // in the threshold bin
        const int need = topk - (cm - m);                // how many of them win
        if (!hvg || m > kGather) {
            // rare: too many candidates share the threshold bin -- exact select of the list
            wave_exact_select<8>(rk, ri, ng, topk, G, G + 256);
            for (int i = lane; i < topk; i += 64) {
                oi[i] = ri[i];
                if (os) os[i] = key_score(rk[i]);
            }
            continue;
        }
        // gather the threshold bin's keys
        int gpos = 0;
        for (int base = 0; base < ng; base += 64 * 16) {
            uint32_t kv[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int i = base + 64 * j + lane;
                kv[j] = rk[i < ng ? i : ng - 1];
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const bool sel = base + 64 * j + lane < ng && bin_of(kv[j], pb) == bt;
                const uint64_t mk = ballot(sel);
                const int q = gpos + (int)bits_below(mk);
                if (sel && q < kGather) G[q] = kv[j];
                gpos += __popcll(mk);
            }
        }
        wave_sync_lds();
        uint32_t gk[kGather / 64];
#pragma unroll
        for (int j = 0; j < kGather / 64; ++j) {
            const int i = lane + 64 * j;
            gk[j] = i < gpos ? G[i] : 0u;
        }
        wave_sync_lds();
        const uint32_t v = wave_kth_largest(gk, need);
        int gt = 0;
#pragma unroll
        for (int j = 0; j < kGather / 64; ++j) gt += gk[j] > v ? 1 : 0;
        const int ties_need = need - wave_sum(gt);
        // one ordered pass writes the winners in ascending index order
        int out = 0, ties = 0;
        for (int base = 0; base < ng; base += 64 * 8) {
            uint32_t kv[8];
            int32_t iv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = base + 64 * j + lane;
                kv[j] = rk[i < ng ? i : ng - 1];
                iv[j] = ri[i < ng ? i : ng - 1];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool in = base + 64 * j + lane < ng;
                const int b = bin_of(kv[j], pb);
                const bool eq = in && b == bt && kv[j] == v;
                const uint64_t em = ballot(eq);
                const bool keep = in && (b > bt || (b == bt && kv[j] > v) ||
                                         (eq && ties + (int)bits_below(em) < ties_need));
                const uint64_t km = ballot(keep);
                if (keep) {
                    const int pos = out + (int)bits_below(km);
                    if (pos < topk) {
                        oi[pos] = iv[j];
                        if (os) os[pos] = key_score(kv[j]);
                    }
                }
                out += __popcll(km);
                ties += __popcll(em);
            }
        }
    }
}

}  // namespace

int candidate_capacity(int topk) {
    // room for about four times topk candidates before a list has to be compacted
    const int c = ((4 * topk + kBK - 1) / kBK) * kBK;
    return c < 256 ? 256 : c;
}

hipError_t launch_score_topk(const uint16_t *q, const uint16_t *k, const uint16_t *w,
                             const int32_t *cu_seqlens, int B, int64_t max_len, int64_t T,
                             int topk, int cap, uint32_t *cand_key, int32_t *cand_idx,
                             int32_t *idx, float *scores, hipStream_t stream) {
    static bool attr_done = false;
    const size_t smem = sizeof(ScoreSmem);
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(score_topk_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    ScoreArgs a;
    a.q = q;
    a.k = k;
    a.w = w;
    a.cu_seqlens = cu_seqlens;
    a.T = T;
    a.nrb = (int)((max_len + kBQ - 1) / kBQ);
    a.topk = topk;
    a.cap = cap;
    a.cand_key = cand_key;
    a.cand_idx = cand_idx;
    a.out_idx = idx;
    a.out_score = scores;
    if (a.nrb == 0 || B == 0) return hipSuccess;
    hipLaunchKernelGGL(score_topk_kernel, dim3(B, a.nrb), dim3(kThreads), smem, stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
