// Causal indexer scores for prefill (dense and varlen), the matrix-core half of the prefill
// path.  For every query row t of a sequence and every key s <= t it computes
//
//         I[t,s] = sum_h w[t,h] * ReLU( q[t,h,:] . k[s,:] )
//
// ("Qwen3.5-397B-A17B vs Kimi K3.1 Pro" compare page, component table, sparse/compressed-
// attention row; whole prefix scored: long-context row of the "Kimi K3.1 Pro vs Gemma 4 31B"
// page) and writes the fp32 scores to the workspace, one row per query in a triangular
// layout (row t holds keys 0 .. 128*(t/128) + 127; the tail past t is never read).  The row
// top-k (topk.hip) consumes them.
//
// One workgroup owns 32 query rows; its 8 waves (2 per SIMD) are symmetric.  Wave w owns rows
// 4w .. 4w+3 completely: its q (4 queries x 32 heads, bf16) stays in registers as the A
// operand of v_mfma_f32_16x16x32_bf16.  The 16 output rows of one product are 4 queries x 4
// heads and the 16 columns are 16 keys (B operand, read from LDS), so each lane gets one
// query's four head dot products for one key; ReLU and the w-weighted sum over the 32 heads
// stay in that lane's registers (no exchange between waves), and a 128-key tile's eight
// 16-key slices give each lane the scores of eight consecutive keys, stored as 32 bytes.
// The keys stream through a ring of LDS tiles that every wave stages one eighth of; progress
// counters in LDS, not workgroup barriers, order the ring, so waves may drift two tiles apart.
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

constexpr int kBQ = 32;               // query rows per workgroup
constexpr int kBK = 128;              // keys per tile (= kRowQuant)
constexpr int kSlices = kBK / 16;
constexpr int kWaves = 8;             // 4 rows each
constexpr int kThreads = 64 * kWaves;
constexpr int kKR = 4;                // key tiles in the LDS ring
constexpr int kKStride = kDim + 8;    // bf16 per key row in LDS (272 B: conflict-free reads)
constexpr int kFillWg = 2048;         // workgroups a split launch aims for (8 per CU)
constexpr int kMinSegTiles = 64;      // shortest key segment of a split launch (8,192 keys)

struct ScoreSmem {
    // key ring; key 8n + st of a tile sits in row 16 st + n, so that the 16-key slice st
    // holds every eighth key and a lane's eight slice results are eight consecutive keys
    uint16_t k[kKR][kBK][kKStride];
    uint32_t k_staged[kWaves];         // key tiles whose eighth wave w has staged
    uint32_t k_used[kWaves];           // key tiles whose products wave w has finished
};

static_assert(kBK == kRowQuant, "a tile is one row quantum of the score layout");

struct ScoreArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *w;
    const int32_t *cu_seqlens;  // nullptr: one sequence of length T
    const int64_t *seq_base;    // start of each sequence's rows in `out` (varlen)
    int64_t T;
    int64_t pos0;               // one sequence: position of its first query row; its keys are
                                // rows 0 .. pos0 + T - 1 of k (0 for ragged batches)
    int nrb;                    // grid.y: row blocks of the longest sequence
    int seg_tiles;              // one sequence: key tiles per workgroup along grid.x (0: all
                                // of a row block's tiles in one workgroup, grid.x = sequence)
    float *out;                 // triangular score rows
    float *dummy;               // write target of rows past a sequence end
    int64_t ldq;                // row stride of q (elements): 4,096, or 8,192 for 64 heads
    int64_t ldw;                // row stride of w: 32, or 64
};

// Polls `ctr` (the smallest of kWaves counters) until it reaches `target`.  Every target is
// reachable (a wave waits only for tiles that slower waves can finish without waiting for
// it), but as a guard against a broken invariant the polls of one wave share a budget of
// about a second in total: once it is spent, waits return at once and the kernel ends.
__device__ __forceinline__ void wait_min_geq(const uint32_t *ctr, uint32_t target, int &budget) {
    for (; budget > 0; --budget) {
        uint32_t m = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            const uint32_t v = __hip_atomic_load(ctr + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            m = v < m ? v : m;
        }
        if (m >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// Publishes this wave's LDS accesses so far (they are performed in order) and bumps `ctr`
// by one (lane 0 adds 1, the others 0: no branch, which would split the scheduling region).
__device__ __forceinline__ void signal(uint32_t *ctr) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __hip_atomic_fetch_add(ctr, __lane_id() == 0 ? 1u : 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// kAccum: add the scores to the rows already there (the second half of a 64-head score,
// whose head sum splits into two 32-head sums) instead of writing them.
template <bool kAccum>
__global__ __launch_bounds__(kThreads, 1) void score_rows_kernel(ScoreArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ScoreSmem &sm = *reinterpret_cast<ScoreSmem *>(smem_raw);

    const int seq = a.seg_tiles > 0 ? 0 : (int)blockIdx.x;
    const int rb = a.nrb - 1 - (int)blockIdx.y;   // longest rows first
    int64_t seq_start = 0, L = a.T, base = 0;
    if (a.cu_seqlens) {
        seq_start = a.cu_seqlens[seq];
        L = (int64_t)a.cu_seqlens[seq + 1] - seq_start;
        base = a.seq_base[seq];
    }
    const int64_t r0 = (int64_t)rb * kBQ;
    if (r0 >= L) return;
    const int rows_here = (int)(L - r0 < kBQ ? L - r0 : kBQ);
    // rows r0 .. r0 + rows_here - 1 sit at positions p0 + r0 .. ; the block streams the key
    // tiles of its last row, and a row whose own last tile comes earlier sends the rest of
    // its stores to the dummy row (only when p0 is not a multiple of kBQ)
    const int64_t p0 = a.pos0;
    const int64_t nkeys = p0 + L;
    const int nkt = (int)((p0 + r0 + rows_here - 1) / kBK) + 1;
    // this workgroup's key tiles: kt0 .. kt0 + nt - 1
    int kt0 = 0, nt = nkt;
    if (a.seg_tiles > 0) {
        kt0 = (int)blockIdx.x * a.seg_tiles;
        if (kt0 >= nkt) return;
        nt = nkt - kt0 < a.seg_tiles ? nkt - kt0 : a.seg_tiles;
    }

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, lg = lane >> 4;

    if (tid < 2 * kWaves) (&sm.k_staged[0])[tid] = 0u;
    __syncthreads();
    int spin = 1 << 22;

    // ---- q fragments: product g covers heads 4g .. 4g+3; A row m = 4 * (query) + (head -
    // 4g); lane l supplies row l % 16 and the 8 dims 32 ks + 8 (l / 16) .. +7 of k-step ks
    // (the key fragments use the same dims).  Output element r of lane l is then query
    // l / 16, head 4g + r, key l % 16 of the slice.
    u32x4 qa[8][4];
    f32x4 wv[8];   // head weights of this lane's output query: w[4g + r] of products g
    {
        const int qrow = 4 * wave + (l16 >> 2);
        const bool qok = qrow < rows_here;
        const int64_t gq = seq_start + r0 + (qok ? qrow : 0);
        const uint16_t *qp = a.q + gq * a.ldq + (l16 & 3) * kDim + 8 * lg;
#pragma unroll
        for (int g = 0; g < 8; ++g)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(qp + (4 * g) * kDim + 32 * ks);
                qa[g][ks] = qok ? v : u32x4{0u, 0u, 0u, 0u};   // rows past the end: zero
            }
        const int wrow = 4 * wave + lg;
        const bool wok = wrow < rows_here;
        const int64_t gw = seq_start + r0 + (wok ? wrow : 0);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const uint2 w4 = *reinterpret_cast<const uint2 *>(a.w + gw * a.ldw + 4 * g);
            wv[g] = wok ? f32x4{bf16_to_f32(w4.x & 0xFFFFu), bf16_to_f32(w4.x >> 16),
                                bf16_to_f32(w4.y & 0xFFFFu), bf16_to_f32(w4.y >> 16)}
                        : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // this lane's output row; rows past the end write to the dummy row, so that every store
    // is issued (a conditional store would make each later wait on a load wait for it too)
    float *const drow = a.dummy + 8 * l16;
    float *orow;
    int row_nt;                          // key tiles of this lane's row
    {
        const int row = 4 * wave + lg;
        const int64_t pos = p0 + r0 + row;
        const bool ok = row < rows_here;
        orow = ok ? a.out + base + tri_row_offset(pos) - tri_row_offset(p0) + 8 * l16 : drow;
        row_nt = ok ? (int)(pos / kBK) + 1 : nkt;
    }

    // ---- key staging: wave w stages keys 16w .. 16w + 15 of every tile, lane -> key
    // 16w + lane/4, 64 bytes at dim 32*(lane%4).  Keys past the sequence end are loaded from
    // its last row; their scores are never read.
    const int sk = 16 * wave + (lane >> 2), sd = 32 * (lane & 3);
    u32x4 kv[4];
    auto load_k = [&](int u) {   // the u-th tile of this workgroup
        int64_t s = (int64_t)(kt0 + u) * kBK + sk;
        s = s < nkeys ? s : nkeys - 1;
        const uint16_t *src = a.k + (seq_start + s) * kDim + sd;
#pragma unroll
        for (int j = 0; j < 4; ++j) kv[j] = *reinterpret_cast<const u32x4 *>(src + 8 * j);
    };
    auto store_k = [&](int slot) {
        uint16_t *dst = &sm.k[slot][16 * (sk & 7) + (sk >> 3)][sd];
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4 *>(dst + 8 * j) = kv[j];
    };
    // the first kKR - 2 tiles go to fresh slots
    for (int u = 0; u < kKR - 2; ++u) {
        load_k(u < nt ? u : nt - 1);
        store_k(u);
        signal(&sm.k_staged[wave]);
    }
    load_k(kKR - 2 < nt ? kKR - 2 : nt - 1);

    // ---- the stream.  Software pipeline inside a tile: a unit is kUG products g (4 heads
    // each) of one 16-key slice, kUG independent MFMA chains over the 128 dims.  The ReLU / w
    // epilogue of each unit runs under the next unit's products, the next slice's key
    // fragments are read a whole slice ahead, and the scheduling groups ask for one MFMA
    // followed by up to two VALU ops.
    constexpr int kUG = 2;
    constexpr int kUnits = 8 / kUG;
    f32x4 prev[kUG];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};    // per-head-slot sums of the open slice
    float sc[kSlices];                   // scores of the tile, by slice
    auto epilogue = [&](int g0) {
#pragma unroll
        for (int i = 0; i < kUG; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = fmaf(wv[g0 + i][r], relu(prev[i][r]), acc[r]);
    };
    auto close_slice = [&]() {
        const float v = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
        return v;
    };
#pragma unroll 1
    for (int t = 0; t < nt; ++t) {
        wait_min_geq(sm.k_staged, (uint32_t)(t + 1), spin);   // tile t staged by every wave
        f32x4 old0, old1;   // kAccum: this tile's scores so far, loaded under the tile's products
        if constexpr (kAccum) {
            const float *src = (kt0 + t < row_nt ? orow : drow) + (int64_t)(kt0 + t) * kBK;
            old0 = *reinterpret_cast<const f32x4 *>(src);
            old1 = *reinterpret_cast<const f32x4 *>(src + 4);
        }
        const uint16_t *kb = &sm.k[t % kKR][l16][8 * lg];
        u32x4 b[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) b[ks] = *reinterpret_cast<const u32x4 *>(kb + 32 * ks);
#pragma unroll
        for (int st = 0; st < kSlices; ++st) {
            // the next slice's key fragments, a whole slice ahead of their use
            u32x4 bn[4];
            if (st < kSlices - 1) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    bn[ks] = *reinterpret_cast<const u32x4 *>(kb + (16 * (st + 1)) * kKStride + 32 * ks);
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
                    if (u == 0) sc[st - 1] = close_slice();
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
        }
        epilogue(8 - kUG);
        sc[kSlices - 1] = close_slice();
        signal(&sm.k_used[wave]);             // every read of key slot t % kKR is done
        // one store and one load per tile, unconditionally and in this order, so that the
        // wait for the load in the next tile never has to include a store
        float *const dst = (kt0 + t < row_nt ? orow : drow) + (int64_t)(kt0 + t) * kBK;
        if constexpr (kAccum) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sc[r] += old0[r];
                sc[4 + r] += old1[r];
            }
        }
        *reinterpret_cast<f32x4 *>(dst) = f32x4{sc[0], sc[1], sc[2], sc[3]};
        *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{sc[4], sc[5], sc[6], sc[7]};
        // stage tile t + kKR - 2 into the slot of tile t - 2 once every wave is done with it
        // (so waves may drift up to two tiles apart); its loads were issued a tile earlier
        const int u = t + kKR - 2;
        if (u < nt) {
            wait_min_geq(sm.k_used, (uint32_t)(t - 1 > 0 ? t - 1 : 0), spin);
            store_k(u % kKR);
            signal(&sm.k_staged[wave]);
        }
        load_k(u + 1 < nt ? u + 1 : nt - 1);
    }
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

}  // namespace

hipError_t launch_scores(const uint16_t *q, const uint16_t *k, const uint16_t *w,
                         const int32_t *cu_seqlens, int B, int64_t max_len, int64_t T, int64_t pos0,
                         int64_t *seq_base, float *out, float *dummy, hipStream_t stream) {
    return launch_scores_ex(q, kQOut, k, w, kHeads, false, cu_seqlens, B, max_len, T, pos0, seq_base, out, dummy,
                            stream);
}

hipError_t launch_scores_ex(const uint16_t *q, int64_t ldq, const uint16_t *k, const uint16_t *w, int64_t ldw,
                            bool accumulate, const int32_t *cu_seqlens, int B, int64_t max_len, int64_t T,
                            int64_t pos0, int64_t *seq_base, float *out, float *dummy, hipStream_t stream) {
    static bool attr_done = false;
    const size_t smem = sizeof(ScoreSmem);
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(score_rows_kernel<false>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(score_rows_kernel<true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    if (B == 0 || max_len == 0) return hipSuccess;
    if (cu_seqlens) {
        hipLaunchKernelGGL(seq_base_kernel, dim3(1), dim3(1024), 0, stream, cu_seqlens, B, seq_base);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    ScoreArgs a;
    a.q = q;
    a.k = k;
    a.w = w;
    a.cu_seqlens = cu_seqlens;
    a.seq_base = seq_base;
    a.T = T;
    a.pos0 = cu_seqlens ? 0 : pos0;
    a.nrb = (int)((max_len + kBQ - 1) / kBQ);
    a.out = out;
    a.dummy = dummy;
    a.ldq = ldq;
    a.ldw = ldw;
    // One sequence with few row blocks (a chunk of queries against a long prefix): split each
    // row block's key tiles over several workgroups, for about kFillWg workgroups of at least
    // kMinSegTiles tiles.  A score needs no reduction across keys, so segments are independent.
    a.seg_tiles = 0;
    unsigned gx = (unsigned)B;
    if (!cu_seqlens && a.nrb < kFillWg) {
        const int64_t max_nkt = (a.pos0 + T - 1) / kBK + 1;
        const int64_t want = (kFillWg + a.nrb - 1) / a.nrb;
        int64_t st = (max_nkt + want - 1) / want;
        st = st < kMinSegTiles ? kMinSegTiles : st;
        if (st < max_nkt) {
            a.seg_tiles = (int)st;
            gx = (unsigned)((max_nkt + st - 1) / st);
        }
    }
    if (accumulate)
        hipLaunchKernelGGL(score_rows_kernel<true>, dim3(gx, a.nrb), dim3(kThreads), smem, stream, a);
    else
        hipLaunchKernelGGL(score_rows_kernel<false>, dim3(gx, a.nrb), dim3(kThreads), smem, stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
