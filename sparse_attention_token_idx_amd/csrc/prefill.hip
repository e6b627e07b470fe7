// Prefill: causal indexer scores and the top-k of every query row, with storage that grows
// linearly in the number of rows (no T x T score matrix is ever written).
//
//         I[t,s] = sum_h w[t,h] * ReLU( q[t,h,:] . k[s,:] ),   s <= t
//
// ("Qwen3.5-397B-A17B vs Kimi K3.1 Pro" compare page, component table, sparse/compressed-
// attention row: H = 32, D = 128, the top 2,048 keys per query; every key of the prefix is
// scored: long-context row of the "Kimi K3.1 Pro vs Gemma 4 31B" page; H = 64 with a rotary
// step for the DeepSeek-V3.2-shaped variant, same sparse-attention row and that page's RoPE
// row).  The pages describe the operation, not an algorithm for it; the one here:
//
//  1. sample: every row scores one key per stratum of kSampleStride keys (at a hashed offset
//     inside the stratum), on the same matrix-core kernel as step 3 (~3% of its work);
//  2. threshold: per row, theta = a lower bound of the r-th largest sample score, with r set
//     so that the true topk-th score lies above theta with overwhelming probability while
//     only about 1.8 topk keys of the row reach it (rows of at most kAllKeys keys: theta =
//     -inf);
//  3. score and filter: the full causal score stream; a key leaves the kernel only if its
//     score reaches its row's theta, as a (score, index) pair appended to the row's list in
//     index order;
//  4. select: the exact top-k of each row's list, ties to the lower index, in ascending index
//     order;
//  5. fallback: a row whose list holds fewer than min(topk, t + 1) keys (theta too high) or
//     overflowed (theta too low, or many equal scores) is scored again in full into a bounded
//     scratch row and selected from all its scores.
// Steps 3 and 4 are exact whatever theta is, so the result equals the full sort of the row.
//
// Score kernel layout: a workgroup of 8 waves (2 per SIMD) owns kBQ query rows (32 for 32
// heads, 16 for 64); wave w owns kQPW = 128 / H rows alone, its q (kQPW queries x H heads,
// bf16) resident in VGPRs as the A operand of v_mfma_f32_16x16x32_bf16.  The 16 rows of one
// product are (query, head) pairs, kH / 8 heads of each of the wave's queries, the 16 columns
// are 16 keys (B operand, from LDS); each lane receives four head dot products of one query
// for one key, and ReLU and the w-weighted head sum stay in its registers (64 heads: one
// exchange with the lane 16 apart adds the other half of the heads).  A 128-key tile's eight
// 16-key slices give each lane the scores of eight consecutive keys.  Keys stream through a
// ring of LDS tiles that every wave stages one eighth of; progress counters in LDS, not
// workgroup barriers, order the ring, so the waves may drift two tiles apart.
#include <algorithm>
#include <functional>
#include <mutex>
#include <type_traits>
#include <vector>

#include "common.hpp"
#include "launch.hpp"
#include "scorers.hpp"
#include "topk_impl.hpp"

namespace dsaidx {
namespace {
using namespace topk_impl;

enum : int { kModeRows = 0, kModeSample = 1, kModeFilter = 2 };

constexpr int kBK = 128;               // keys per tile (= kRowQuant)
constexpr int kSlices = kBK / 16;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKR = 4;                 // key tiles in the LDS ring
constexpr int kSignalSlice = 2;        // slice of a tile after which the next tile's DMA is awaited
constexpr int kFillWg = 2048;          // workgroups a split launch aims for (8 per CU)
constexpr int kMinSegTiles = 64;       // shortest key segment of a split launch (8,192 keys)
constexpr int kFewRowBlocks = 128;     // at most this many row blocks (half the CUs or fewer) ...
constexpr int kMinSegTilesFew = 8;     // ... may split their keys into segments this short
constexpr int kMaxSeg = 512;           // most key segments of a split launch
static_assert(kBK == kRowQuant, "a tile is one row quantum of the triangular layout");

struct ScoreSmem {
    // key ring: row n of a tile holds its key n, slice st is rows 16 st .. 16 st + 15.  Row R
    // keeps its dims chunk c (16 bytes) at chunk position c ^ (R % 16), so that the 16 rows a
    // fragment read touches hit 16 different bank groups.
    uint16_t k[kKR][kBK][kDim];
    uint32_t k_staged[kWaves];         // key tiles whose eighth wave w has staged
    uint32_t k_used[kWaves];           // key tiles whose products wave w has finished
};

template <int kH> struct Geo {
    static constexpr int kQPW = 128 / kH;       // queries per wave: 4 or 2
    static constexpr int kBQ = kQPW * kWaves;   // query rows per workgroup: 32 or 16
    static constexpr int kHG = kH / 8;          // heads of one query in a product: 4 or 8
};

struct ScoreArgs {
    const uint16_t *q, *k, *w;
    int64_t ldq, ldw;           // row strides of q (elements: H x 128) and w (H)
    const int32_t *cu_seqlens;  // nullptr: one sequence of T rows
    int64_t T;
    int64_t pos0;               // one sequence: position of row 0 (its keys: rows 0 .. pos0 + T - 1)
    int64_t g_lo, g_hi;         // only packed rows g_lo <= g < g_hi produce output
    int nrb;                    // grid.y: row blocks of the longest sequence
    int seg_tiles;              // one sequence: key tiles per workgroup (0: none)
    int seg_y;                  // one sequence: segments on grid.y, row blocks on grid.x
    int spin;                   // polls allowed per wait on the key ring
    uint32_t *status;           // bit 0 set when a wait ran out of polls
    float *dummy;               // store target of rows with no output
    // kModeRows: triangular rows (row g at tri_row_offset(pos) - tri_row_offset(pos0) + base)
    float *tri;
    const int64_t *seq_base;
    // kModeSample: sample scores, row g at srow + (g - g_lo) * ms
    float *srow;
    int64_t ms;
    // kModeFilter: per (row, segment) candidate lists and counts
    const uint32_t *theta;      // [g - g_lo] order-key threshold
    uint2 *cand;                // [(g - g_lo) * nseg + seg][cap + 64]: (score bits, key position)
    int32_t *cnt;               // [(g - g_lo) * nseg + seg]
    int nseg, cap;              // lists are cap + 64 slots apart: a list ends in 64 sentinel pairs
};

// Polls `ctr` (the smallest of kWaves counters) until it reaches `target`, at most `budget`
// times after the first look.  Every target is reachable (a wave waits only for tiles that
// slower waves can finish without waiting for it); running out of polls means a broken
// invariant, which the caller reports through the status word rather than hanging.
__device__ __forceinline__ bool wait_min_geq(const uint32_t *ctr, uint32_t target, int budget) {
    for (int i = 0;; ++i) {
        uint32_t m = 0xFFFFFFFFu;
#pragma unroll
        for (int j = 0; j < kWaves; ++j) {
            const uint32_t v = __hip_atomic_load(ctr + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            m = v < m ? v : m;
        }
        if (m >= target) break;
        if (i >= budget) return false;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
    return true;
}

// Publishes this wave's LDS accesses so far (they are performed in order) and bumps `ctr`
// by one (lane 0 adds 1, the others 0: no branch, which would split the scheduling region).
__device__ __forceinline__ void signal(uint32_t *ctr) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __hip_atomic_fetch_add(ctr, __lane_id() == 0 ? 1u : 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Bumps `ctr` once this wave's direct-to-LDS loads have landed (they count in vmcnt).
__device__ __forceinline__ void signal_dma(uint32_t *ctr) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __hip_atomic_fetch_add(ctr, __lane_id() == 0 ? 1u : 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte-per-lane global -> LDS load (lane i lands at lds_addr + 16 i).  Written out so
// that the compiler, which cannot tell the tiles in flight from the ones being read, does not
// wait for these loads before every LDS access; the kernel waits for them itself (vmcnt).  The
// instruction has no result registers and reads its address registers when it issues.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_addr)
                 : "memory", "m0");
}

template <int kH, int kMode>
__global__ __launch_bounds__(kThreads, 1) void score_kernel(ScoreArgs a) {
    using G = Geo<kH>;
    constexpr int kQPW = G::kQPW, kBQ = G::kBQ, kHG = G::kHG;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ScoreSmem &sm = *reinterpret_cast<ScoreSmem *>(smem_raw);

    // One sequence: grid (key segments, row blocks), or (row blocks, key segments) with seg_y.
    // Ragged batches: grid (row blocks, sequences), so that consecutive workgroups -- which the
    // dispatcher deals to the 8 XCDs in turn -- are row blocks of one sequence rather than one
    // row block of every sequence (which would pin each sequence to one XCD).  Longest rows
    // first either way.
    const bool rb_x = a.cu_seqlens || a.seg_y;
    const int seq = a.cu_seqlens ? (int)blockIdx.y : 0;
    const int rb = a.nrb - 1 - (int)(rb_x ? blockIdx.x : blockIdx.y);
    int64_t seq_start = 0, L = a.T;
    if (a.cu_seqlens) {
        seq_start = a.cu_seqlens[seq];
        L = (int64_t)a.cu_seqlens[seq + 1] - seq_start;
    }
    const int64_t r0 = (int64_t)rb * kBQ;
    if (r0 >= L) return;
    const int rows_here = (int)(L - r0 < kBQ ? L - r0 : kBQ);
    if (seq_start + r0 >= a.g_hi || seq_start + r0 + rows_here <= a.g_lo) return;
    // rows r0 .. r0 + rows_here - 1 sit at positions p0 + r0 ..; the block streams the key
    // tiles of its last row
    const int64_t p0 = a.pos0;
    const int64_t nkeys = p0 + L;
    int nkt;
    int64_t nsamp = 0;   // kModeSample: strata of the sequence
    if constexpr (kMode == kModeSample) {
        const int64_t n_last = p0 + r0 + rows_here;   // keys of the block's last row
        if (n_last <= kAllKeys) return;               // no row of the block uses a sample
        nsamp = nkeys / kSampleStride;
        nkt = (int)((n_last / kSampleStride + kBK - 1) / kBK);
    } else {
        nkt = (int)((p0 + r0 + rows_here - 1) / kBK) + 1;
    }
    int kt0 = 0, nt = nkt, seg = 0;
    if (a.seg_tiles > 0) {
        seg = (int)(a.seg_y ? blockIdx.y : blockIdx.x);
        kt0 = seg * a.seg_tiles;
        if (kt0 >= nkt) return;
        nt = nkt - kt0 < a.seg_tiles ? nkt - kt0 : a.seg_tiles;
    }

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, lg = lane >> 4;

    if (tid < 2 * kWaves) (&sm.k_staged[0])[tid] = 0u;
    __syncthreads();
    bool expired = false;

    // ---- q fragments: product g covers heads kHG g .. kHG g + kHG - 1 of each of the wave's
    // queries; A row m = kHG * (query) + (head - kHG g); lane l supplies row l % 16 and the 8
    // dims 32 ks + 8 (l / 16) .. +7 of k-step ks (the key fragments use the same dims).
    // Output element r of lane l is then row m = 4 (l / 16) + r: query m / kHG, key l % 16.
    u32x4 qa[8][4];
    f32x4 wv[8];   // head weights of the lane's four output rows, by product
    const int oq = 4 * lg / kHG;   // this lane's output query within the wave
    {
        const int qrow = kQPW * wave + l16 / kHG;
        const bool qok = qrow < rows_here;
        const int64_t gq = seq_start + r0 + (qok ? qrow : 0);
        const uint16_t *qp = a.q + gq * a.ldq + (l16 % kHG) * kDim + 8 * lg;
#pragma unroll
        for (int g = 0; g < 8; ++g)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(qp + (kHG * g) * kDim + 32 * ks);
                qa[g][ks] = qok ? v : u32x4{0u, 0u, 0u, 0u};   // rows past the end: zero
            }
        const int wrow = kQPW * wave + oq;
        const bool wok = wrow < rows_here;
        const int64_t gw = seq_start + r0 + (wok ? wrow : 0);
        const int h0 = (4 * lg) % kHG;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const uint2 w4 = *reinterpret_cast<const uint2 *>(a.w + gw * a.ldw + kHG * g + h0);
            wv[g] = wok ? f32x4{bf16_to_f32(w4.x & 0xFFFFu), bf16_to_f32(w4.x >> 16),
                                bf16_to_f32(w4.y & 0xFFFFu), bf16_to_f32(w4.y >> 16)}
                        : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // this lane's output row (64 heads: the two lanes of a pair hold the same row and scores;
    // only the even one emits candidates)
    const int orow_in = kQPW * wave + oq;
    const int64_t gpk = seq_start + r0 + orow_in;                 // packed row
    const bool row_ok = orow_in < rows_here && gpk >= a.g_lo && gpk < a.g_hi;
    const int64_t pos = p0 + r0 + orow_in;                         // its position
    float *const drow = a.dummy + l16;
    float *orow = drow;
    int row_nt = nkt;                                              // kModeRows: its key tiles
    int my_lim = -1;                                               // kModeFilter: last key, -1: none
    float my_thf = INFINITY;                                       // its threshold
    uint32_t my_list = 0;                                          // first entry of the row's list
    if constexpr (kMode == kModeRows) {
        if (row_ok) {
            orow = a.tri + (a.cu_seqlens ? a.seq_base[seq] : 0) + tri_row_offset(pos) - tri_row_offset(p0) + l16;
            row_nt = (int)(pos / kBK) + 1;
        }
    } else if constexpr (kMode == kModeSample) {
        if (row_ok) orow = a.srow + (gpk - a.g_lo) * a.ms + l16;
    } else {
        if (row_ok && (kH == 32 || (lg & 1) == 0)) {
            my_lim = (int)pos;
            const uint32_t th = a.theta[gpk - a.g_lo];
            my_thf = th ? key_score(th) : -INFINITY;   // order key 0: every key
            my_list = (uint32_t)(((gpk - a.g_lo) * a.nseg + seg) * (int64_t)(a.cap + 64));
        }
    }
    int rowcnt = 0;   // kModeFilter: keys of this row emitted so far (same in its 16 lanes)
    uint2 *const dummy_pair = reinterpret_cast<uint2 *>(a.dummy);

    // ---- key staging by direct global -> LDS loads: wave w fills rows (keys) 16 w .. 16 w + 15
    // of every tile with four 1 KB loads; lane l of load i writes chunk position l % 16 of row
    // 16 w + n, n = 4 i + l / 16, so it fetches dims chunk (l % 16) ^ n of that key.  Keys past
    // the end repeat the last key; their scores are masked or never read.
    auto issue_k = [&](int u) {   // this workgroup's u-th tile (clamped) into slot u % kKR
        const int uu = u < nt ? u : nt - 1;
        const int64_t tb = (int64_t)(kt0 + uu) * kBK;
        uint16_t *slot = &sm.k[u % kKR][0][0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = 4 * i + (lane >> 4);
            int64_t s = tb + 16 * wave + n;
            if constexpr (kMode == kModeSample) {
                s = s < nsamp ? s : nsamp - 1;
                s = s * kSampleStride + sample_offset(s);
            } else {
                s = s < nkeys ? s : nkeys - 1;
            }
            const uint16_t *src = a.k + (seq_start + s) * kDim + 8 * ((lane & 15) ^ n);
            dma16(src, (uint32_t)__builtin_amdgcn_readfirstlane(
                           (int)(uint32_t)(uintptr_t)(lds_void *)(slot + (16 * wave + 4 * i) * kDim)));
        }
    };
    // lane (l16, lg) reads dims chunk 4 ks + lg of row 16 st + l16: chunk position (4 ks + lg) ^ l16
    int frag_off[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) frag_off[ks] = l16 * kDim + 8 * ((4 * ks + lg) ^ l16);
    // tiles 0 and 1 before the stream; tile t + 2 is requested at the end of tile t (into the
    // slot of tile t - 2, once every wave is done with it) and announced kSignalSlice slices
    // into tile t + 1, so waves may drift almost two tiles apart
    issue_k(0);
    issue_k(1);
    signal_dma(&sm.k_staged[wave]);
    __hip_atomic_fetch_add(&sm.k_staged[wave], __lane_id() == 0 ? 1u : 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    bool pending = false;

    // ---- the stream.  Software pipeline inside a tile: a unit is kUG products g of one 16-key
    // slice, kUG independent MFMA chains over the 128 dims.  The ReLU / w epilogue of each
    // unit runs under the next unit's products, the next slice's key fragments are read a
    // whole slice ahead, and the scheduling groups ask for one MFMA followed by up to two VALU
    // ops.
    constexpr int kUG = 2;
    constexpr int kUnits = 8 / kUG;
    f32x4 prev[kUG];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};    // per-output-row sums of the open slice
    auto epilogue = [&](int g0) {
#pragma unroll
        for (int i = 0; i < kUG; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = fmaf(wv[g0 + i][r], relu(prev[i][r]), acc[r]);
    };
    auto close_slice = [&]() {
        float v = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        if constexpr (kH == 64) v += __shfl_xor(v, 16, 64);   // the other 32 heads of the query
        // the score is formed here, in a register: left to itself the compiler sinks these
        // sums to their use after the tile, keeping the per-head partials live (and spilling)
        asm volatile("" : "+v"(v));
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
        return v;
    };
    // The score v of key 16 st + l16 of tile kt for this lane's row leaves the kernel at once,
    // inside the MFMA stream and without branches: one store per lane and slice.  Rows and
    // samples store it; the filter keeps it if it reaches the row's threshold (the row's 16
    // lanes take consecutive list slots from a ballot; the other lanes store to a dummy slot).
    auto out_slice = [&](int kt, int st, float v) {
        if constexpr (kMode == kModeFilter) {
            const int key = kt * kBK + 16 * st + l16;
            const bool p = (key <= my_lim) & (v >= my_thf);
            // this lane's row in the ballot, and its lanes before this one
            const uint32_t rm = (uint32_t)(__ballot(p) >> (16u * (uint32_t)(__lane_id() >> 4))) & 0xFFFFu;
            const int slot = rowcnt + __builtin_popcount(rm & ((1u << (__lane_id() & 15u)) - 1u));
            rowcnt += __builtin_popcount(rm);
            uint2 *const dst = (p & (slot < a.cap)) ? a.cand + (my_list + (uint32_t)slot) : dummy_pair;
            *dst = uint2{__float_as_uint(v), (uint32_t)key};
        } else {
            float *const dst = (kt < row_nt ? orow : drow) + (int64_t)kt * kBK + 16 * st;
            *dst = v;
        }
    };
#pragma unroll 1
    for (int t = 0; t < nt; ++t) {
        const int kt = kt0 + t;
        if (!wait_min_geq(sm.k_staged, (uint32_t)(t + 1), expired ? 0 : a.spin)) expired = true;
        const uint16_t *kb = &sm.k[t % kKR][0][0];
        u32x4 b[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) b[ks] = *reinterpret_cast<const u32x4 *>(kb + frag_off[ks]);
#pragma unroll
        for (int st = 0; st < kSlices; ++st) {
            u32x4 bn[4];
            if (st < kSlices - 1) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    bn[ks] = *reinterpret_cast<const u32x4 *>(kb + (16 * (st + 1)) * kDim + frag_off[ks]);
            }
#pragma unroll
            for (int u = 0; u < kUnits; ++u) {
                f32x4 cur[kUG];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
                    for (int i = 0; i < kUG; ++i)
                        cur[i] = mfma16x16x32(qa[kUG * u + i][ks], b[ks],
                                              ks ? cur[i] : f32x4{0.f, 0.f, 0.f, 0.f});
                }
                if (st > 0 || u > 0) {
                    epilogue(kUG * ((u + kUnits - 1) % kUnits));
                    if (u == 0) out_slice(kt, st - 1, close_slice());
                }
#pragma unroll
                for (int i = 0; i < 4 * kUG; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // VALU
                }
#pragma unroll
                for (int i = 0; i < kUG; ++i) prev[i] = cur[i];
            }
            if (st < kSlices - 1) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) b[ks] = bn[ks];
            }
            if (st == kSignalSlice) {
                // the tile requested at the end of the last one (if any) has landed once at most
                // this tile's kSignalSlice slice stores are still in flight
                static_assert(kSignalSlice == 2, "the wait below counts two stores");
                asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
                __hip_atomic_fetch_add(&sm.k_staged[wave], __lane_id() == 0 && pending ? 1u : 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
                pending = false;
            }
        }
        epilogue(8 - kUG);
        out_slice(kt, kSlices - 1, close_slice());
        signal(&sm.k_used[wave]);             // every read of key slot t % kKR is done
        // request tile t + 2 into the slot of tile t - 2 once every wave is done with that tile
        if (t + 2 < nt) {
            if (!wait_min_geq(sm.k_used, (uint32_t)(t - 1 > 0 ? t - 1 : 0), expired ? 0 : a.spin)) expired = true;
            issue_k(t + 2);
            pending = true;
        }
    }
    if constexpr (kMode == kModeFilter) {
        if (my_lim >= 0) {
            if (l16 == 0) a.cnt[(gpk - a.g_lo) * a.nseg + seg] = rowcnt;
            // 64 sentinel pairs (score bits 0xFFFFFFFF: order key 0) after the list, so that a
            // select may read whole 64-entry groups past its end
            if (rowcnt <= a.cap) {
                uint2 *sp = a.cand + my_list + (uint32_t)rowcnt + 4u * (uint32_t)l16;
#pragma unroll
                for (int j = 0; j < 4; ++j) sp[j] = uint2{0xFFFFFFFFu, 0u};
            }
        }
    }
    if (expired && lane == 0) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- row location
struct RowMap {
    const int32_t *cu_seqlens;   // nullptr: one sequence, row g at position pos0 + g
    int B;
    int64_t pos0;
};

// Position of packed row g in its sequence and the sequence's first packed row.
__device__ __forceinline__ void locate(const RowMap &m, int64_t g, int64_t &pos, int64_t &seq_start) {
    if (!m.cu_seqlens) {
        pos = m.pos0 + g;
        seq_start = 0;
        return;
    }
    int lo = 0, hi = m.B - 1;   // last sequence with cu_seqlens[i] <= g
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)m.cu_seqlens[mid] <= g) lo = mid;
        else hi = mid - 1;
    }
    seq_start = m.cu_seqlens[lo];
    pos = g - seq_start;
}

// ---------------------------------------------------------------- threshold
struct ThrArgs {
    RowMap map;
    int64_t s0, s1;       // packed rows of this sub-chunk
    int64_t f0;           // first packed row of the filter chunk (theta index base)
    const float *srow;    // sample rows: row g at srow + (g - s0) * ms
    int64_t ms;
    int topk;
    uint32_t *theta;
};

// Count of order keys in 256 bins (this wave's histogram) from the top bin down: returns the
// bin b that holds the r-th largest key and sets above = keys in bins above b.
__device__ __forceinline__ int find_bin_from_top(const uint32_t *hist, int r, int &above) {
    const int lane = __lane_id();
    int c[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        c[i] = (int)hist[4 * lane + i];
        s += c[i];
    }
    const int incl = wave_inclusive_sum(s);
    const int total = __shfl(incl, 63, 64);
    int run = total - incl;   // keys in the bins of higher lanes
    int found = -1, found_above = 0;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
        if (found < 0 && run < r && r <= run + c[i]) {
            found = 4 * lane + i;
            found_above = run;
        }
        run += c[i];
    }
    const uint64_t who = __ballot(found >= 0);
    const int src = who ? (int)__builtin_ctzll(who) : 0;
    above = __shfl(found_above, src, 64);
    return who ? __shfl(found, src, 64) : 0;
}

// One wave per row: theta = order key at or below the r-th largest of the row's m sampled
// scores, r = E + c sqrt(E) + c (E = m topk / n, the expected number of samples at or above
// the row's topk-th score; c = kThetaMargin), found by two 256-bin histogram passes over
// [min, max] of the sample keys.  Rows of at most kAllKeys keys take every key (theta 0).
__global__ __launch_bounds__(256) void threshold_kernel(ThrArgs a) {
    __shared__ uint32_t hist_all[4][256];
    const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
    const int64_t g = a.s0 + (int64_t)blockIdx.x * 4 + wave;
    if (g >= a.s1) return;
    int64_t pos, ss;
    locate(a.map, g, pos, ss);
    const int64_t n = pos + 1;
    uint32_t theta = 0u;
    if (n > kAllKeys) {
        uint32_t *hist = hist_all[wave];
        const int m = (int)(n / kSampleStride);
        const double E = (double)m * (double)a.topk / (double)n;
        int r = (int)ceil(E + kThetaMargin * sqrt(E) + kThetaMargin);
        r = r < m ? r : m;
        const float *row = a.srow + (g - a.s0) * a.ms;
        // keys of the row, 256 at a time (rows are padded to a multiple of 128 floats)
        auto chunk = [&](int j0, uint32_t (&key)[4]) {
            f32x4 v = *reinterpret_cast<const f32x4 *>(row + j0);
#pragma unroll
            for (int i = 0; i < 4; ++i) key[i] = j0 + i < m ? score_key(v[i]) : 0u;
        };
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
        for (int j0 = 4 * lane; j0 < m; j0 += 256) {
            uint32_t key[4];
            chunk(j0, key);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (key[i]) {
                    lo = key[i] < lo ? key[i] : lo;
                    hi = key[i] > hi ? key[i] : hi;
                }
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            const uint32_t olo = (uint32_t)__shfl_xor((int)lo, d, 64), ohi = (uint32_t)__shfl_xor((int)hi, d, 64);
            lo = olo < lo ? olo : lo;
            hi = ohi > hi ? ohi : hi;
        }
        const uint32_t range = hi - lo;
        const int shA = bit_width(range) > 8 ? bit_width(range) - 8 : 0;
        const int shB = shA > 8 ? shA - 8 : 0;
        // pass A: bins of 2^shA key units above lo
#pragma unroll
        for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0u;
        __builtin_amdgcn_wave_barrier();
        for (int j0 = 4 * lane; j0 < m; j0 += 256) {
            uint32_t key[4];
            chunk(j0, key);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (key[i]) atomicAdd(&hist[(key[i] - lo) >> shA], 1u);
        }
        __builtin_amdgcn_wave_barrier();
        int above = 0;
        const int bA = find_bin_from_top(hist, r, above);
        uint32_t th = lo + ((uint32_t)bA << shA);
        if (shA > 0) {
            // pass B: the keys of bin bA in 256 bins of 2^shB units
            const int rB = r - above;
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0u;
            __builtin_amdgcn_wave_barrier();
            for (int j0 = 4 * lane; j0 < m; j0 += 256) {
                uint32_t key[4];
                chunk(j0, key);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t rel = key[i] - lo;
                    if (key[i] && (int)(rel >> shA) == bA) atomicAdd(&hist[(rel >> shB) & 255u], 1u);
                }
            }
            __builtin_amdgcn_wave_barrier();
            int aboveB = 0;
            const int bB = find_bin_from_top(hist, rB, aboveB);
            th += (uint32_t)bB << shB;
        }
        theta = th;
    }
    if (lane == 0) a.theta[g - a.f0] = theta;
}

// ---------------------------------------------------------------- exact select of the lists
// A row whose kept keys are one list: a workgroup of kSelW waves, wave h holding a contiguous
// quarter of the list's 64-entry groups (entry 64 (g0 + i) + lane in key[i] and pos[i]), the
// order key and the key position of every entry in registers, so the list is read once.  An MSD
// radix select over the order keys relative to their minimum, 8 bits at a time with a shared
// 256-bin LDS histogram, finds theta = the need-th largest key and how many keys equal to
// theta win (the lowest-index ones).  Each wave then counts its keys above and equal to theta;
// from the counts of the waves before it, it knows where its winners start and how many of its
// keys equal to theta still win, and writes its winners in list order, which is index order,
// from ballots.
constexpr int kSelW = 4;                               // waves per row
constexpr int kSelKeys = kListCap / (64 * kSelW);      // entries per lane: 24
constexpr int kSelCap = kSelKeys * 64 * kSelW;         // kept keys a row may have
static_assert(kSelCap == kListCap, "a row's list fits the select");
constexpr int kSelBlk = 8;                             // loads in flight per lane
static_assert(kSelKeys % kSelBlk == 0, "whole load blocks");

struct SelArgs {
    RowMap map;
    int64_t f0, f1;            // packed rows of the filter chunk
    const uint2 *cand;
    const int32_t *cnt;
    int nseg, cap, seg_tiles;  // lists cap + 64 slots apart
    int topk;
    const uint32_t *status;
    uint32_t *fb;              // [1] rows sent to the fallback
    int64_t *fb_list;
    int32_t *idx;
    float *scores;
    int32_t *dummy_i;          // store target of the lanes that write nothing (2 words a wave)
};

// A row's list: the entries of up to kSelSegs pieces, one per key segment of the row (a row
// whose key tiles were split over workgroups), the keys of each piece all above those of the
// pieces before it.  Entry e is in the last piece j with off[j] <= e, at l[j] + (e - off[j]);
// pieces the row does not have start at INT32_MAX.
constexpr int kSelSegs = 4;
struct SelList {
    const uint2 *l[kSelSegs];
    int off[kSelSegs];
};

// This wave's order keys and key positions: entry e0 + 64 i + lane of the row's list in key[i],
// pos[i], kSelBlk loads in flight at a time.
// Blocks past the wave's nit groups are not read; inside a block, a group i >= nit reads the
// wave's last group again (a uniform index, so no branch) and its keys are zeroed; entries past
// the list's end inside its last group read the sentinel run that follows its last piece,
// whose key is 0.
// The scores are never -0 (each is a sum from +0 of products and ReLUs), so the cheaper key
// serves; the sentinels (all bits set) get key 0.
template <int NS>
__device__ __forceinline__ void sel_load(uint32_t (&key)[kSelKeys], int32_t (&pos)[kSelKeys], const SelList &sl,
                                         int e0, int lane, int nit) {
    nit = __builtin_amdgcn_readfirstlane(nit);
#pragma unroll
    for (int blk = 0; blk < kSelKeys / kSelBlk; ++blk) {
        if (kSelBlk * blk < nit) {
            uint2 e[kSelBlk];
#pragma unroll
            for (int j = 0; j < kSelBlk; ++j) {
                const int gi = min(kSelBlk * blk + j, nit - 1);
                const int en = e0 + 64 * gi + lane;
                const uint2 *src = sl.l[0] + en;
#pragma unroll
                for (int q = 1; q < NS; ++q) src = en >= sl.off[q] ? sl.l[q] + (en - sl.off[q]) : src;
                e[j] = *src;
            }
#pragma unroll
            for (int j = 0; j < kSelBlk; ++j) {
                const uint32_t k = score_key_nz(__uint_as_float(e[j].x));
                key[kSelBlk * blk + j] = kSelBlk * blk + j < nit ? k : 0u;
                pos[kSelBlk * blk + j] = (int32_t)e[j].y;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kSelBlk; ++j) {
                key[kSelBlk * blk + j] = 0u;
                pos[kSelBlk * blk + j] = 0;
            }
        }
    }
}

// NS: most pieces a row's list has (1: the key tiles of a row were not split)
template <int NS>
__global__ __launch_bounds__(64 * kSelW) void select_kernel(SelArgs a) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t xch[2 * kSelW];
    const int tid = (int)threadIdx.x;
    const int h = tid >> 6, lane = tid & 63;
    const int64_t g = a.f0 + (int64_t)blockIdx.x;
    int64_t pos_t, ss;
    locate(a.map, g, pos_t, ss);
    const int64_t n = pos_t + 1;
    const int topk = a.topk;
    const int need = n < topk ? (int)n : topk;
    int32_t *oi = a.idx + g * topk;
    float *os = a.scores ? a.scores + g * topk : nullptr;
    if (*a.status & 1u) {
        // a wait of the scoring kernel ran out of polls: its scores are not to be trusted,
        // so the row is marked invalid (index -2, NaN) instead of returning a wrong selection
        for (int i = tid; i < topk; i += 64 * kSelW) {
            oi[i] = -2;
            if (os) os[i] = __builtin_nanf("");
        }
        return;
    }
    // the row's list: one piece per key segment of the row (one, or up to NS when its key tiles
    // were split over workgroups)
    const int64_t lrow = g - a.f0;
    const int nsr = NS > 1 && a.seg_tiles > 0 ? (int)((pos_t / kBK) / a.seg_tiles) + 1 : 1;
    SelList sl;
    int total = 0;
    bool over = false;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int c = j < nsr ? a.cnt[lrow * a.nseg + j] : 0;
        over |= c > a.cap;
        sl.l[j] = a.cand + (lrow * a.nseg + (j < nsr ? j : 0)) * (int64_t)(a.cap + 64);
        sl.off[j] = j == 0 ? 0 : j < nsr ? total : INT32_MAX;
        total += c > a.cap ? a.cap : c;
    }
    if (over || total > kSelCap || total < need) {
        if (tid == 0) {
            const uint32_t i = atomicAdd(&a.fb[1], 1u);
            a.fb_list[i] = g;
        }
        return;
    }
    const int nit_all = (total + 63) >> 6;
    const int per = (nit_all + kSelW - 1) / kSelW;
    const int g0 = min(h * per, nit_all);
    const int nit = min(per, nit_all - g0);
    uint32_t key[kSelKeys];
    int32_t pos[kSelKeys];
    sel_load<NS>(key, pos, sl, 64 * g0, lane, nit);
    // Every candidate wins when there are only `need` of them (a row of at most topk keys): theta
    // 0 and no key to place by ties keep every key present and no empty slot.
    uint32_t base = 0u, prefix = 0u;
    int left = 0;             // winners still to place among the keys matching the prefix
    if (total > need) {
        // the smallest and largest keys present (key - 1 wraps 0, no key, to the top)
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
        for (int i = 0; i < kSelKeys; i += 2) {
            lo = min(lo, min(key[i] - 1u, key[i + 1] - 1u));
            hi = max(hi, max(key[i], key[i + 1]));
        }
        lo += 1u;
        if (lo == 0u) lo = 0xFFFFFFFFu;   // no key in this lane
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            const uint32_t olo = (uint32_t)__shfl_xor((int)lo, d, 64), ohi = (uint32_t)__shfl_xor((int)hi, d, 64);
            lo = olo < lo ? olo : lo;
            hi = ohi > hi ? ohi : hi;
        }
        if (lane == 0) {
            xch[2 * h] = lo;
            xch[2 * h + 1] = hi;
        }
        __syncthreads();
#pragma unroll
        for (int v = 0; v < kSelW; ++v) {
            lo = xch[2 * v] < lo ? xch[2 * v] : lo;
            hi = xch[2 * v + 1] > hi ? xch[2 * v + 1] : hi;
        }
        // Radix select over r = key - (lo - 1), in [1, hi - lo + 1] for the keys present, 8 bits
        // at a time from the top; the empty slots keep r = 0 and stay out of the histograms
        // (counted, their crowd in one bin would serialise the LDS atomics).
        base = lo - 1u;
#pragma unroll
        for (int i = 0; i < kSelKeys; ++i) key[i] = key[i] ? key[i] - base : 0u;
        left = need;
        uint32_t pmask = 0;
        int hb = bit_width(hi - base);
#pragma unroll 1
        while (hb > 0) {
            const int wd = hb < 8 ? hb : 8;
            const int shift = hb - wd;
            const uint32_t dmask = (1u << wd) - 1u;
            hist[tid] = 0u;       // 256 threads, 256 bins
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kSelKeys; ++i)
                if (key[i] && (key[i] & pmask) == prefix)
                    atomicAdd(&hist[__builtin_amdgcn_ubfe(key[i], (uint32_t)shift, (uint32_t)wd)], 1u);
            __syncthreads();
            int above = 0;
            const int d = find_bin_from_top(hist, left, above);
            left -= above;
            prefix |= (uint32_t)d << shift;
            pmask |= dmask << shift;
            hb = shift;
            __syncthreads();   // every read of this pass's histogram is done
        }
    }
    const uint32_t theta = prefix;   // r of the need-th largest key; `left` keys equal to it win
    // this wave's keys above theta and equal to it; from those of the waves before it, where
    // its winners start and how many keys equal to theta were seen before it
    // (theta >= 1, so neither test holds for an empty slot)
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < kSelKeys; ++i) {
        gt += (int)__popcll(__ballot(key[i] > theta));
        eq += (int)__popcll(__ballot(key[i] == theta));
    }
    if (lane == 0) {
        xch[2 * h] = (uint32_t)gt;
        xch[2 * h + 1] = (uint32_t)eq;
    }
    __syncthreads();
    int out = 0, eq_seen = 0;
#pragma unroll
    for (int v = 0; v < kSelW; ++v) {
        if (v < h) {
            const int gv = (int)xch[2 * v], ev = (int)xch[2 * v + 1];
            const int ek = left - eq_seen;   // keys equal to theta that still win
            out += gv + (ek <= 0 ? 0 : (ek < ev ? ek : ev));
            eq_seen += ev;
        }
    }
    // the winners, in list order
#pragma unroll
    for (int blk = 0; blk < kSelKeys / kSelBlk; ++blk) {
        if (kSelBlk * blk < nit) {
#pragma unroll
            for (int j = 0; j < kSelBlk; ++j) {
                const int i = kSelBlk * blk + j;
                bool keep = key[i] > theta;
                const uint64_t em = __ballot(key[i] == theta);
                if (em) {   // the group holds keys equal to theta (a uniform branch, rarely taken)
                    keep |= (key[i] == theta) & (eq_seen + (int)bits_below(em) < left);
                    eq_seen += (int)__popcll(em);
                }
                const uint64_t km = __ballot(keep);
                if (keep) {
                    const uint32_t p4 = 4u * ((uint32_t)out + bits_below(km));   // byte offset of the slot
                    *reinterpret_cast<int32_t *>(reinterpret_cast<char *>(oi) + p4) = pos[i];
                    if (os) *reinterpret_cast<float *>(reinterpret_cast<char *>(os) + p4) = key_score(key[i] + base);
                }
                out += (int)__popcll(km);
            }
        }
    }
    for (int i = need + tid; i < topk; i += 64 * kSelW) {
        oi[i] = -1;
        if (os) os[i] = -INFINITY;
    }
}

// Rows whose list is split over key segments (launches that split a row block's keys over
// several workgroups): one 8-wave workgroup per row, 16 list entries per thread in list order,
// an exact radix select and an ordered emission over the workgroup.
constexpr int kSelMW = 8;
struct SelMSmem {
    static constexpr int kW = kSelMW;
    uint32_t hist[kBins<kSelMW>];
    int32_t wsum[kSelMW];
    uint32_t wmax[kSelMW];
    int32_t bcast[3];
    int32_t segoff[kMaxSeg + 1];
};
static_assert(kPer * 64 * kSelMW >= kSelCap, "the workgroup holds a whole list");

__global__ __launch_bounds__(64 * kSelMW) void select_multi_kernel(SelArgs a) {
    __shared__ SelMSmem sm;
    const int tid = (int)threadIdx.x;
    const int64_t g = a.f0 + (int64_t)blockIdx.x;
    int64_t pos, ss;
    locate(a.map, g, pos, ss);
    const int64_t n = pos + 1;
    const int topk = a.topk;
    const int need = n < topk ? (int)n : topk;
    int32_t *oi = a.idx + g * topk;
    float *os = a.scores ? a.scores + g * topk : nullptr;
    if (*a.status & 1u) {
        for (int i = tid; i < topk; i += 64 * kSelMW) {
            oi[i] = -2;
            if (os) os[i] = __builtin_nanf("");
        }
        return;
    }
    const int64_t lrow = g - a.f0;
    const int nsr = (int)((pos / kBK) / a.seg_tiles) + 1;
    int c = tid < nsr ? a.cnt[lrow * a.nseg + tid] : 0;
    const bool over = __syncthreads_or(c > a.cap);
    c = c > a.cap ? a.cap : c;
    int total;
    const int incl = block_inclusive_sum(c, total, sm);
    if (tid < nsr) sm.segoff[tid + 1] = incl;
    if (tid == 0) sm.segoff[0] = 0;
    __syncthreads();
    if (over || total < need || total > kSelCap) {
        if (tid == 0) {
            const uint32_t i = atomicAdd(&a.fb[1], 1u);
            a.fb_list[i] = g;
        }
        return;
    }
    uint32_t key[kPer];
    int32_t kidx[kPer];
    {
        const int e0 = kPer * tid;
        int s = 0;
        if (e0 < total) {
            int lo = 0, hi = nsr - 1;   // last segment with segoff[s] <= e0
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sm.segoff[mid] <= e0) lo = mid;
                else hi = mid - 1;
            }
            s = lo;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = e0 + i;
            key[i] = 0u;
            kidx[i] = 0;
            if (e < total) {
                while (sm.segoff[s + 1] <= e) ++s;
                const uint2 v = a.cand[(lrow * a.nseg + s) * (int64_t)(a.cap + 64) + (e - sm.segoff[s])];
                key[i] = score_key(__uint_as_float(v.x));
                kidx[i] = (int32_t)v.y;
            }
        }
    }
    // every candidate wins when there are only `need` of them (a row of at most topk keys):
    // theta 0 keeps every key present (and no empty slot)
    uint32_t theta = 0u;
    int keep = 0;
    if (total > need) {
        uint32_t m = 0, mn = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            m = key[i] > m ? key[i] : m;
            mn = key[i] != 0u && key[i] < mn ? key[i] : mn;
        }
        const uint32_t top = block_max(m, sm);
        const uint32_t bot = ~block_max(~mn, sm);
        keep = need;
        theta = select_rel(key, bot, bit_width(top - bot), keep, sm);
    }
    int eq_base = 0;
    emit_ordered_idx(key, kidx, theta, keep, 0, eq_base, oi, os, sm);
    for (int i = need + tid; i < topk; i += 64 * kSelMW) {
        oi[i] = -1;
        if (os) os[i] = -INFINITY;
    }
}

// ---------------------------------------------------------------- exact fallback
constexpr int kFbWg = 128;          // persistent workgroups of the fallback pass
constexpr int kFbW = 8;             // their waves

struct FbArgs {
    RowMap map;
    const uint16_t *q, *k, *w;
    int64_t ldq, ldw;
    int topk;
    uint32_t *fb;                   // [1] rows listed, [2] rows taken
    const int64_t *fb_list;
    float *scratch;                 // [kFbWg][ld]
    int64_t ld;
    int32_t *nbuf;                  // [kFbWg] length of the row in the scratch row
    int64_t *obuf;                  // [kFbWg] its packed row
    int32_t *idx;
    float *scores;
};

// Each workgroup takes listed rows one by one: scores the whole row into its scratch row
// (64-key groups per wave, the decode scorer) and selects from it with the row top-k.
template <int HB>
__global__ __launch_bounds__(64 * kFbW, 1) void fallback_kernel(FbArgs a) {
    __shared__ TopkSmem<kFbW> sm;
    __shared__ int64_t cur;
    const int tid = (int)threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, lg = lane >> 4;
    float *const row = a.scratch + (int64_t)blockIdx.x * a.ld;
    for (;;) {
        if (tid == 0) {
            const uint32_t i = atomicAdd(&a.fb[2], 1u);
            cur = i < __hip_atomic_load(&a.fb[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ? a.fb_list[i] : -1;
        }
        __syncthreads();
        const int64_t g = cur;
        __syncthreads();
        if (g < 0) break;
        int64_t pos, ss;
        locate(a.map, g, pos, ss);
        const int64_t n = pos + 1;
        Bf16ScorerT<HB> sc;
        sc.init_row(a.q + g * a.ldq, a.w + g * a.ldw, a.k + ss * kDim, l16, lg);
        for (int64_t grp = wave; grp * 64 < n; grp += kFbW) {
            int key[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t s = grp * 64 + 16 * u + l16;
                key[u] = (int)(s < n ? s : n - 1);
            }
            sc.load(key, lg);
            float p[4];
            sc.partial(p);
            const float v = group_scores(p, lg);
            const int64_t s = grp * 64 + 16 * lg + l16;
            if (s < n) row[s] = v;
        }
        if (tid == 0) {
            a.nbuf[blockIdx.x] = (int32_t)n;
            a.obuf[blockIdx.x] = g;
        }
        __syncthreads();
        TopkArgs ta{};
        ta.scores = a.scratch;
        ta.mode = 1;
        ta.seqlens = a.nbuf;
        ta.ld = a.ld;
        ta.nmax = a.ld;
        ta.B = (int)gridDim.x;
        ta.topk = a.topk;
        ta.out_idx = a.idx;
        ta.out_score = a.scores;
        ta.out_row = a.obuf;
        row_topk_row<kFbW>(ta, (int64_t)blockIdx.x, sm);
        __syncthreads();
    }
}

// Clears the fallback counters (and the status word on a call's first chunk) and sets the first
// n_zero thresholds to 0 (every key), for chunks that need no sample.
__global__ __launch_bounds__(256) void prefill_reset_kernel(uint32_t *fb, int clear_status, uint32_t *theta,
                                                            int64_t n_zero) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i == 0) {
        if (clear_status) fb[0] = 0u;
        fb[1] = 0u;
        fb[2] = 0u;
    }
    if (i < n_zero) theta[i] = 0u;
}

// seq_base[i] = sum over sequences j < i of tri_row_offset(L_j), i = 0 .. B (one workgroup).
__global__ __launch_bounds__(1024) void seq_base_kernel(const int32_t *cu_seqlens, int B, int64_t *seq_base) {
    __shared__ int64_t part[1024];
    const int tid = threadIdx.x;
    const int per = (B + 1023) / 1024;
    const int i0 = tid * per, i1 = min(B, i0 + per);
    int64_t s = 0;
    for (int i = i0; i < i1; ++i) s += tri_row_offset((int64_t)cu_seqlens[i + 1] - cu_seqlens[i]);
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
        seq_base[i] = run;
        run += tri_row_offset((int64_t)cu_seqlens[i + 1] - cu_seqlens[i]);
    }
    if (tid == 1023) seq_base[B] = part[1023];
}

// ---------------------------------------------------------------- host side
std::atomic<int> g_spin{1 << 20};   // polls per wait of the score kernels

// Diagnostic phase timing: while on, each phase launch of a prefill top-k call is bracketed by
// two HIP events on its stream; the records are read (and released) by prefill_phase_times.
std::atomic<bool> g_timing{false};
struct PhaseRec {
    int phase;
    hipEvent_t a, b;
};
std::mutex g_tmu;
std::vector<PhaseRec> g_trecs;

struct PhaseMark {
    int phase;
    hipStream_t st;
    hipEvent_t a = nullptr;
    PhaseMark(int p, hipStream_t s) : phase(p), st(s) {
        if (!g_timing.load(std::memory_order_relaxed)) return;
        if (hipEventCreate(&a) != hipSuccess || hipEventRecord(a, st) != hipSuccess) {
            if (a) (void)hipEventDestroy(a);
            a = nullptr;
        }
    }
    ~PhaseMark() {
        if (!a) return;
        hipEvent_t b = nullptr;
        if (hipEventCreate(&b) != hipSuccess || hipEventRecord(b, st) != hipSuccess) {
            if (b) (void)hipEventDestroy(b);
            (void)hipEventDestroy(a);
            return;
        }
        std::lock_guard<std::mutex> lk(g_tmu);
        g_trecs.push_back({phase, a, b});
    }
};

template <int kH, int kMode>
hipError_t set_attr() {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(score_kernel<kH, kMode>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(ScoreSmem));
}

hipError_t ensure_attrs() {
    static DeviceOnce once;
    return once.run([] {
        hipError_t e = set_attr<32, kModeRows>();
        if (e == hipSuccess) e = set_attr<32, kModeSample>();
        if (e == hipSuccess) e = set_attr<32, kModeFilter>();
        if (e == hipSuccess) e = set_attr<64, kModeSample>();
        if (e == hipSuccess) e = set_attr<64, kModeFilter>();
        return e;
    });
}

// Key tiles per workgroup of a launch over nrb row blocks of one sequence whose longest row
// streams max_nkt tiles (0: no split).
int split_tiles(int64_t nrb, int64_t max_nkt) {
    // a launch of a few row blocks leaves most CUs idle and waits on its longest row block, so
    // it takes short segments; otherwise a segment is long enough for its workgroup to pay for
    // loading its queries and filling the key ring
    const int64_t min_seg = nrb <= kFewRowBlocks ? kMinSegTilesFew : kMinSegTiles;
    if (nrb >= kFillWg || max_nkt <= min_seg) return 0;
    const int64_t want = (kFillWg + nrb - 1) / nrb;
    int64_t st = (max_nkt + want - 1) / want;
    st = st < min_seg ? min_seg : st;
    const int64_t few = (max_nkt + kMaxSeg - 1) / kMaxSeg;   // at most kMaxSeg segments
    st = st < few ? few : st;
    return st < max_nkt ? (int)st : 0;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kCUs = 256;              // compute units of a gfx950 device
constexpr int kSimOverhead = 2;        // a filter workgroup's query load and ring fill, in key tiles

// How a one-sequence filter launch splits its key tiles: seg key tiles per workgroup (0: no
// split), with the segments on grid.y (seg_y) or grid.x.
struct FilterSplit {
    int seg;
    bool seg_y;
};

// The split of a filter launch over the rows rows at positions pos0 .. of one sequence, in row
// blocks of bq.  With between a few row blocks and one and a half per CU, starting at most their
// own count into the sequence, the launch is one or two rounds of workgroups whose time is that
// of the busiest CU, set by the longest row blocks (at T = 8,192 the last one streams 64 key tiles
// against 33 on average).  There the choice is between no split and the longest row block in two
// segments (a row's two lists are then merged by the select), with the row blocks on grid.x:
// the dispatcher deals consecutive workgroups to the 8 XCDs in turn and each XCD gives its next
// workgroup to the CU that frees first, so the whole first segments go out longest first over
// every XCD and the second segments follow on the CUs that the short ones free.  (With the
// segments on grid.x instead, a row block's two halves alternate between even and odd XCDs and
// the even ones get every long half.)  The choice with the least busy CU in that deal is kept,
// and remembered per shape.  Otherwise split_tiles decides.
int filter_span(int64_t rows, int bq, int64_t pos0, int64_t nrb, int seg) {
    constexpr int kXcds = 8, kXcdCUs = kCUs / kXcds;
    std::vector<int64_t> busy(kCUs, 0);   // XCD x's CUs at [kXcdCUs x, kXcdCUs x + kXcdCUs)
    const int64_t nseg = seg ? cdiv((pos0 + rows - 1) / kBK + 1, seg) : 1;
    int64_t span = 0, id = 0;
    for (int64_t y = 0; y < nseg; ++y)
        for (int64_t x = 0; x < nrb; ++x, ++id) {
            const int64_t r0 = (nrb - 1 - x) * bq;
            const int64_t nrows = rows - r0 < bq ? rows - r0 : bq;
            const int64_t nkt = (pos0 + r0 + nrows - 1) / kBK + 1;
            const int64_t kt0 = y * seg;
            if (kt0 >= nkt) continue;   // exits at once
            const int64_t len = seg && nkt - kt0 > seg ? seg : nkt - kt0;
            int64_t *cu = &busy[(size_t)(id % kXcds) * kXcdCUs];
            int64_t *m = std::min_element(cu, cu + kXcdCUs);
            *m += len + kSimOverhead;
            span = *m > span ? *m : span;
        }
    return (int)span;
}

FilterSplit filter_split(int64_t rows, int bq, int64_t pos0) {
    const int64_t nrb = cdiv(rows, bq);
    const int64_t max_nkt = (pos0 + rows - 1) / kBK + 1;
    // the rows' key counts differ by less than 2x when the prefix is longer than the rows
    if (nrb <= kFewRowBlocks || 2 * nrb > 3 * kCUs || pos0 >= rows)
        return FilterSplit{split_tiles(nrb, max_nkt), false};
    struct Shape {
        int64_t rows, pos0;
        int bq, seg;
    };
    static std::mutex mu;
    static std::vector<Shape> seen;   // at most kSeenShapes shapes, first come
    constexpr size_t kSeenShapes = 64;
    {
        std::lock_guard<std::mutex> lk(mu);
        for (const Shape &sh : seen)
            if (sh.rows == rows && sh.pos0 == pos0 && sh.bq == bq) return FilterSplit{sh.seg, sh.seg > 0};
    }
    const int half = (int)cdiv(max_nkt, 2);
    const int seg = half >= kMinSegTilesFew && filter_span(rows, bq, pos0, nrb, half) < filter_span(rows, bq, pos0, nrb, 0)
                        ? half
                        : 0;
    std::lock_guard<std::mutex> lk(mu);
    if (seen.size() < kSeenShapes) seen.push_back(Shape{rows, pos0, bq, seg});
    return FilterSplit{seg, seg > 0};
}

template <int kH>
hipError_t launch_score(int mode, const ScoreArgs &a, unsigned gx, hipStream_t st) {
    const size_t smem = sizeof(ScoreSmem);
    // ragged batches: grid (row blocks, sequences), gx = the sequence count; one sequence: gx
    // key segments, on grid.y with seg_y
    const dim3 grid = a.cu_seqlens || a.seg_y ? dim3((unsigned)a.nrb, gx) : dim3(gx, (unsigned)a.nrb);
    if constexpr (kH == 32) {
        if (mode == kModeRows) {
            hipLaunchKernelGGL((score_kernel<32, kModeRows>), grid, dim3(kThreads), smem, st, a);
            return hipGetLastError();
        }
    }
    if (mode == kModeSample)
        hipLaunchKernelGGL((score_kernel<kH, kModeSample>), grid, dim3(kThreads), smem, st, a);
    else
        hipLaunchKernelGGL((score_kernel<kH, kModeFilter>), grid, dim3(kThreads), smem, st, a);
    return hipGetLastError();
}

}  // namespace

void prefill_phase_timing(bool on) {
    g_timing.store(on, std::memory_order_relaxed);
}

hipError_t prefill_phase_times(double *ms, int *count, int n) {
    std::lock_guard<std::mutex> lk(g_tmu);
    for (int i = 0; i < n; ++i) {
        ms[i] = 0.0;
        count[i] = 0;
    }
    hipError_t err = hipSuccess;
    for (const PhaseRec &r : g_trecs) {
        float t = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
        if (e != hipSuccess && err == hipSuccess) err = e;
        if (e == hipSuccess && r.phase >= 0 && r.phase < n) {
            ms[r.phase] += t;
            count[r.phase] += 1;
        }
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    g_trecs.clear();
    return err;
}

void prefill_set_wait_budget(int polls) { g_spin.store(polls < 0 ? 0 : polls, std::memory_order_relaxed); }
int prefill_wait_budget() { return g_spin.load(std::memory_order_relaxed); }

// ---- plan and workspace of a prefill call
PrefillPlan prefill_plan(int heads, bool varlen, int64_t rows, int B, int64_t max_len, int64_t pos0) {
    PrefillPlan p{};
    p.heads = heads;
    p.varlen = varlen;
    p.rows = rows;
    p.B = varlen ? B : 1;
    p.max_len = varlen ? max_len : rows;
    p.pos0 = varlen ? 0 : pos0;
    const int bq = heads == 64 ? Geo<64>::kBQ : Geo<32>::kBQ;
    const int64_t nkeys = p.pos0 + p.max_len;     // keys of the longest row
    // filter chunks of equal size: a short last chunk would be a launch of few row blocks
    const int64_t cmax = heads == 64 ? kFilterRows / 2 : kFilterRows;
    p.cf = rows > 0 ? cdiv(rows, cdiv(rows, cmax)) : 0;
    // lists of a filter chunk: rows x segments (dense chunks may split their key tiles)
    p.lists = 0;
    for (int64_t f0 = 0; f0 < rows; f0 += p.cf) {
        const int64_t f1 = f0 + p.cf < rows ? f0 + p.cf : rows;
        int64_t nseg = 1;
        if (!varlen) {
            const int st = filter_split(f1 - f0, bq, p.pos0 + f0).seg;
            if (st) nseg = cdiv((p.pos0 + f1 - 1) / kBK + 1, st);
        }
        const int64_t l = (varlen ? p.cf : (f1 - f0)) * nseg;
        p.lists = l > p.lists ? l : p.lists;
    }
    p.cap = kListCap;
    // sample rows: m = n / stride scores per row, in whole tiles
    const int64_t mmax = nkeys / kSampleStride;
    p.ms = cdiv(mmax > 0 ? mmax : 1, kBK) * kBK;
    int64_t cs = kSampleBytes / (4 * p.ms);
    cs = cs / bq * bq;
    cs = cs < bq ? bq : cs;
    p.cs = cs < p.cf ? cs : p.cf;
    p.ld = cdiv(nkeys > 0 ? nkeys : 1, 64) * 64;
    // workspace parts, each 256-byte aligned
    auto r256 = [](size_t b) { return (b + 255u) & ~(size_t)255u; };
    size_t off = 0;
    p.off_hdr = off;      off += 256;
    p.off_theta = off;    off += r256(4u * (size_t)p.cf);
    p.off_cnt = off;      off += r256(4u * (size_t)p.lists);
    p.off_cand = off;     off += r256(8u * (size_t)p.lists * (size_t)(p.cap + 64));
    p.off_srow = off;     off += r256(4u * (size_t)p.cs * (size_t)p.ms);
    p.off_fblist = off;   off += r256(8u * (size_t)p.cf);
    p.off_nbuf = off;     off += r256(4u * kFbWg);
    p.off_obuf = off;     off += r256(8u * kFbWg);
    p.off_scratch = off;  off += r256(4u * (size_t)kFbWg * (size_t)p.ld);
    p.off_dummy = off;    off += r256(4u * (size_t)(p.ms > p.ld ? p.ms : p.ld) + 4u * kBK);
    p.bytes = off;
    return p;
}

hipError_t launch_prefill_topk(const PrefillPlan &p, const uint16_t *q, const uint16_t *k, const uint16_t *w,
                               const int32_t *cu_seqlens, int topk, int32_t *idx, float *scores, void *ws,
                               hipStream_t st) {
    if (p.rows == 0) return hipSuccess;
    hipError_t e = ensure_attrs();
    if (e != hipSuccess) return e;
    char *base = static_cast<char *>(ws);
    uint32_t *fb = reinterpret_cast<uint32_t *>(base + p.off_hdr);
    uint32_t *theta = reinterpret_cast<uint32_t *>(base + p.off_theta);
    int32_t *cnt = reinterpret_cast<int32_t *>(base + p.off_cnt);
    uint2 *cand = reinterpret_cast<uint2 *>(base + p.off_cand);
    float *srow = reinterpret_cast<float *>(base + p.off_srow);
    int64_t *fb_list = reinterpret_cast<int64_t *>(base + p.off_fblist);
    int32_t *nbuf = reinterpret_cast<int32_t *>(base + p.off_nbuf);
    int64_t *obuf = reinterpret_cast<int64_t *>(base + p.off_obuf);
    float *scratch = reinterpret_cast<float *>(base + p.off_scratch);
    float *dummy = reinterpret_cast<float *>(base + p.off_dummy);
    const int H = p.heads;
    const int bq = H == 64 ? Geo<64>::kBQ : Geo<32>::kBQ;
    const int64_t ldq = (int64_t)H * kDim, ldw = H;
    RowMap map{cu_seqlens, p.B, p.pos0};

    for (int64_t f0 = 0; f0 < p.rows; f0 += p.cf) {
        const int64_t f1 = f0 + p.cf < p.rows ? f0 + p.cf : p.rows;
        // rows of at most kAllKeys keys keep every key: when the chunk's longest row is one of
        // them, no sample is needed and every threshold is 0
        const bool all_keys = p.varlen ? p.max_len <= kAllKeys : p.pos0 + f1 <= kAllKeys;
        const int64_t nz = all_keys ? f1 - f0 : 0;
        hipLaunchKernelGGL(prefill_reset_kernel, dim3((unsigned)(nz > 0 ? cdiv(nz, 256) : 1)), dim3(256), 0, st, fb,
                           f0 == 0 ? 1 : 0, theta, nz);
        // 1 + 2. sample scores and thresholds, in sub-chunks of the sample buffer
        for (int64_t s0 = f0; s0 < f1 && !all_keys; s0 += p.cs) {
            const int64_t s1 = s0 + p.cs < f1 ? s0 + p.cs : f1;
            ScoreArgs a{};
            a.k = k;
            a.ldq = ldq;
            a.ldw = ldw;
            a.spin = g_spin.load(std::memory_order_relaxed);
            a.status = fb;
            a.dummy = dummy;
            a.srow = srow;
            a.ms = p.ms;
            unsigned gx;
            if (p.varlen) {
                a.q = q; a.w = w; a.cu_seqlens = cu_seqlens;
                a.T = p.rows; a.pos0 = 0; a.g_lo = s0; a.g_hi = s1;
                a.nrb = (int)cdiv(p.max_len, bq);
                a.seg_tiles = 0;
                gx = (unsigned)p.B;
            } else {
                a.q = q + s0 * ldq; a.w = w + s0 * ldw; a.cu_seqlens = nullptr;
                a.T = s1 - s0; a.pos0 = p.pos0 + s0; a.g_lo = 0; a.g_hi = s1 - s0;
                a.nrb = (int)cdiv(s1 - s0, bq);
                const int64_t mt = cdiv((p.pos0 + s1) / kSampleStride, kBK);
                a.seg_tiles = split_tiles(a.nrb, mt);
                gx = a.seg_tiles ? (unsigned)cdiv(mt, a.seg_tiles) : 1u;
            }
            {
                PhaseMark pm(kPhaseSample, st);
                e = H == 64 ? launch_score<64>(kModeSample, a, gx, st) : launch_score<32>(kModeSample, a, gx, st);
            }
            if (e != hipSuccess) return e;
            ThrArgs t{map, s0, s1, f0, srow, p.ms, topk, theta};
            {
                PhaseMark pm(kPhaseThreshold, st);
                hipLaunchKernelGGL(threshold_kernel, dim3((unsigned)cdiv(s1 - s0, 4)), dim3(256), 0, st, t);
                e = hipGetLastError();
            }
            if (e != hipSuccess) return e;
        }
        // 3. the full score stream, emitting the keys at or above each row's threshold
        ScoreArgs a{};
        a.k = k;
        a.ldq = ldq;
        a.ldw = ldw;
        a.spin = g_spin.load(std::memory_order_relaxed);
        a.status = fb;
        a.dummy = dummy;
        a.theta = theta;
        a.cand = cand;
        a.cnt = cnt;
        a.cap = p.cap;
        unsigned gx;
        if (p.varlen) {
            a.q = q; a.w = w; a.cu_seqlens = cu_seqlens;
            a.T = p.rows; a.pos0 = 0; a.g_lo = f0; a.g_hi = f1;
            a.nrb = (int)cdiv(p.max_len, bq);
            a.seg_tiles = 0;
            a.nseg = 1;
            gx = (unsigned)p.B;
        } else {
            a.q = q + f0 * ldq; a.w = w + f0 * ldw; a.cu_seqlens = nullptr;
            a.T = f1 - f0; a.pos0 = p.pos0 + f0; a.g_lo = 0; a.g_hi = f1 - f0;
            a.nrb = (int)cdiv(f1 - f0, bq);
            const int64_t mt = (p.pos0 + f1 - 1) / kBK + 1;
            const FilterSplit fs = filter_split(f1 - f0, bq, p.pos0 + f0);
            a.seg_tiles = fs.seg;
            a.seg_y = fs.seg_y ? 1 : 0;
            a.nseg = a.seg_tiles ? (int)cdiv(mt, a.seg_tiles) : 1;
            gx = (unsigned)a.nseg;
        }
        {
            PhaseMark pm(kPhaseFilter, st);
            e = H == 64 ? launch_score<64>(kModeFilter, a, gx, st) : launch_score<32>(kModeFilter, a, gx, st);
        }
        if (e != hipSuccess) return e;
        // 4. exact select of every row's list
        SelArgs s{};
        s.map = map;
        s.f0 = f0;
        s.f1 = f1;
        s.cand = cand;
        s.cnt = cnt;
        s.nseg = a.nseg;
        s.cap = p.cap;
        s.seg_tiles = a.seg_tiles;
        s.topk = topk;
        s.status = fb;
        s.fb = fb;
        s.fb_list = fb_list;
        s.idx = idx;
        s.scores = scores;
        s.dummy_i = reinterpret_cast<int32_t *>(dummy);
        {
            PhaseMark pm(kPhaseSelect, st);
            if (a.nseg > kSelSegs)
                hipLaunchKernelGGL(select_multi_kernel, dim3((unsigned)(f1 - f0)), dim3(64 * kSelMW), 0, st, s);
            else if (a.nseg > 1)
                hipLaunchKernelGGL(select_kernel<kSelSegs>, dim3((unsigned)(f1 - f0)), dim3(64 * kSelW), 0, st, s);
            else
                hipLaunchKernelGGL(select_kernel<1>, dim3((unsigned)(f1 - f0)), dim3(64 * kSelW), 0, st, s);
            e = hipGetLastError();
        }
        if (e != hipSuccess) return e;
        // 5. rows whose list could not decide them
        FbArgs fa{map, q, k, w, ldq, ldw, topk, fb, fb_list, scratch, p.ld, nbuf, obuf, idx, scores};
        {
            PhaseMark pm(kPhaseFallback, st);
            if (H == 64)
                hipLaunchKernelGGL(fallback_kernel<4>, dim3(kFbWg), dim3(64 * kFbW), 0, st, fa);
            else
                hipLaunchKernelGGL(fallback_kernel<2>, dim3(kFbWg), dim3(64 * kFbW), 0, st, fa);
            e = hipGetLastError();
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---- raw causal score rows (triangular layout), 32 heads
hipError_t launch_scores(const uint16_t *q, const uint16_t *k, const uint16_t *w, const int32_t *cu_seqlens, int B,
                         int64_t max_len, int64_t T, int64_t pos0, int64_t *seq_base, float *out, float *dummy,
                         uint32_t *status, hipStream_t stream) {
    hipError_t e = ensure_attrs();
    if (e != hipSuccess) return e;
    if (B == 0 || max_len == 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_reset_kernel, dim3(1), dim3(64), 0, stream, status, 1, (uint32_t *)nullptr, (int64_t)0);
    if (cu_seqlens) hipLaunchKernelGGL(seq_base_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, B, seq_base);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int bq = Geo<32>::kBQ;
    ScoreArgs a{};
    a.q = q;
    a.k = k;
    a.w = w;
    a.ldq = kQOut;
    a.ldw = kHeads;
    a.cu_seqlens = cu_seqlens;
    a.T = T;
    a.pos0 = cu_seqlens ? 0 : pos0;
    a.g_lo = 0;
    a.g_hi = INT64_MAX;
    a.nrb = (int)cdiv(max_len, bq);
    a.spin = g_spin.load(std::memory_order_relaxed);
    a.status = status;
    a.dummy = dummy;
    a.tri = out;
    a.seq_base = seq_base;
    a.seg_tiles = 0;
    unsigned gx = (unsigned)B;
    if (!cu_seqlens) {
        const int64_t mt = (a.pos0 + T - 1) / kBK + 1;
        a.seg_tiles = split_tiles(a.nrb, mt);
        if (a.seg_tiles) gx = (unsigned)cdiv(mt, a.seg_tiles);
    }
    return launch_score<32>(kModeRows, a, gx, stream);
}

}  // namespace dsaidx
