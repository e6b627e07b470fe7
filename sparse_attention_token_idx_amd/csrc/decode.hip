// Decode: one new query per sequence scored against that sequence's cached indexer keys
// (serving engines cache the indexer keys: "Kimi K3.1 Pro vs GLM-5" compare page,
// low-precision row), then the top-k of the whole prefix (sparse/compressed-attention
// row of the "Qwen3.5-397B-A17B vs Kimi K3.1 Pro" page; long-context row of the
// "Kimi K3.1 Pro vs Gemma 4 31B" page).
//
// Pass 1 streams the key cache once (256 bytes per key, the bandwidth-bound part), split
// evenly over the grid across sequences: each 16-key slice is one pair of
// v_mfma_f32_16x16x32_bf16 chains with the 32 heads as the M dimension (two halves of 16),
// ReLU and the w-weighted head sum in registers, and one fp32 score per key written to the
// workspace (4 bytes against 256 read).  A wave takes 64 consecutive keys (four slices) at a
// time and writes their scores with one 256-byte store: every lane stores one score, at a
// 256-byte aligned address (each sequence's range in the flat split starts at a multiple of
// 64), because scattered 64-byte stores of the scores slow the read stream measurably.
// Pass 2 is the row top-k of topk.hip, one workgroup of 16 waves per sequence: a sampled
// threshold, one streaming pass that keeps the keys above it, an exact select among those,
// and the winners in ascending index order.
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

constexpr int kDecThreads = 256;
constexpr int kSplit = 64;            // a workgroup's share of keys is a multiple of this

struct DecArgs {
    const uint16_t *q;
    const uint16_t *w;
    const uint16_t *k_cache;
    const int64_t *start;
    const int64_t *cu;  // [B + 1] prefix sums of the clamped cache lengths rounded up to 64
    const int32_t *seqlens;
    int max_seqlen;
    int B;
    int64_t ld;         // score row stride (a multiple of 64)
    float *score_buf;   // [B][ld]
};

// cu[b] = sum over i < b of L_i = min(max(seqlens[i], 0), max_seqlen) rounded up to a
// multiple of 64, for b = 0 .. B.
__global__ __launch_bounds__(1024) void decode_prefix_kernel(const int32_t *seqlens, int B,
                                                              int max_seqlen, int64_t *cu) {
    __shared__ int64_t part[1024];
    const int tid = threadIdx.x;
    const int per = (B + 1023) / 1024;
    const int i0 = tid * per, i1 = min(B, i0 + per);
    auto len = [&](int i) { return ((int64_t)max(0, min(seqlens[i], max_seqlen)) + 63) & ~(int64_t)63; };
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

// The cached keys of all sequences, taken as one flat range of cu[B] positions (each
// sequence's keys padded to a multiple of 64), are split evenly over the grid, so every
// workgroup streams the same number of bytes whatever the lengths.  A workgroup's share may
// cross sequence boundaries; each piece uses its sequence's q and w.  Within a piece, wave w
// takes the 64-key groups w, w + 4, ...
__global__ __launch_bounds__(kDecThreads) void decode_score_kernel(DecArgs a) {
    const int64_t total = a.cu[a.B];
    const int64_t per = ((total + gridDim.x - 1) / gridDim.x + kSplit - 1) / kSplit * kSplit;
    int64_t pos = (int64_t)blockIdx.x * per;
    const int64_t end = min(total, pos + per);
    if (pos >= end) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    int b = 0;
    {
        int lo = 0, hi = a.B - 1;   // the last sequence with cu[b] <= pos
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu[mid] <= pos) lo = mid;
            else hi = mid - 1;
        }
        b = lo;
    }
    while (pos < end) {
        while (a.cu[b + 1] <= pos) ++b;   // skips empty sequences
        const int64_t seg_end = min(end, a.cu[b + 1]);
        // keys s_begin .. s_end - 1 of sequence b (s_begin a multiple of 64; below max_seqlen)
        const int len = max(0, min(a.seqlens[b], a.max_seqlen));
        const int s_begin = (int)(pos - a.cu[b]), s_end = min(len, (int)(seg_end - a.cu[b]));

        // A operand: head 16*hh + l16, k-slot chunk 4*ks + lg (8 dims)
        u32x4 qa[2][4];
        float wv[2][4];
        const uint16_t *qb = a.q + (int64_t)b * kQOut;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qa[hh][ks] = *reinterpret_cast<const u32x4 *>(qb + (16 * hh + l16) * kDim + 8 * (4 * ks + lg));
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[hh][r] = bf16_to_f32(a.w[(int64_t)b * kHeads + 16 * hh + 4 * lg + r]);
        }
        const uint16_t *kc = a.k_cache + a.start[b] * kDim;
        float *out = a.score_buf + (int64_t)b * a.ld;

        // The next group's loads are issued before this group's store, and every lane stores
        // (positions past the end are the row's padding), so that waiting for loads never
        // waits for a store.  Key rows past the end are clamped to the last one.
        u32x4 kb[4][4];
        auto load = [&](int g) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int key = min(g + 16 * u + l16, s_end - 1);
                const uint32_t off = (uint32_t)key * (uint32_t)kDim + 8u * (uint32_t)lg;   // elements
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) kb[u][ks] = *reinterpret_cast<const u32x4 *>(kc + off + 32 * ks);
            }
        };
        int g0 = s_begin + 64 * wave;
        if (g0 < s_end) load(g0);
        for (; g0 < s_end; g0 += 256) {
            float p[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                f32x4 s_lo = {0.f, 0.f, 0.f, 0.f}, s_hi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    s_lo = mfma16x16x32(qa[0][ks], kb[u][ks], s_lo);
                    s_hi = mfma16x16x32(qa[1][ks], kb[u][ks], s_hi);
                }
                float v = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) v = fmaf(wv[0][r], relu(s_lo[r]), v);
#pragma unroll
                for (int r = 0; r < 4; ++r) v = fmaf(wv[1][r], relu(s_hi[r]), v);
                p[u] = v;
            }
            if (g0 + 256 < s_end) load(g0 + 256);
            out[g0 + lane] = group_scores(p, lg);
        }
        pos = seg_end;
    }
}

int decode_grid() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 2048;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_score_kernel, kDecThreads, 0) != hipSuccess || per <= 0)
        per = 2;
    const int g = 8 * per * cus;   // eight rounds of the workgroups resident at once: short shares
    if (dev < 64) cached[dev] = g;
    return g;
}

}  // namespace

hipError_t launch_decode_prefix(const int32_t *seqlens, int B, int max_seqlen, int64_t *cu, hipStream_t stream) {
    hipLaunchKernelGGL(decode_prefix_kernel, dim3(1), dim3(1024), 0, stream, seqlens, B, max_seqlen, cu);
    return hipGetLastError();
}

hipError_t launch_decode(const uint16_t *q, const uint16_t *w, const uint16_t *k_cache,
                         const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                         int topk, int64_t *cu, float *score_buf, int32_t *idx, float *scores,
                         hipStream_t stream) {
    if (B == 0) return hipSuccess;
    hipError_t e = launch_decode_prefix(seqlens, B, max_seqlen, cu, stream);
    if (e != hipSuccess) return e;
    const int64_t ld = decode_row_stride(max_seqlen);
    DecArgs a{q, w, k_cache, start, cu, seqlens, max_seqlen, B, ld, score_buf};
    const int64_t bound = (int64_t)B * ((max_seqlen + kSplit - 1) / kSplit);   // shares of kSplit keys
    const int64_t grid = bound < decode_grid() ? bound : decode_grid();
    hipLaunchKernelGGL(decode_score_kernel, dim3((unsigned)grid), dim3(kDecThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_row_topk_decode(score_buf, seqlens, B, ld, max_seqlen, topk, idx, scores, stream);
}

}  // namespace dsaidx
