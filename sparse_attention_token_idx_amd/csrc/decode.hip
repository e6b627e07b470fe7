// Decode: one new query per sequence scored against that sequence's cached indexer keys
// (serving engines cache the indexer keys: "Kimi K3.1 Pro vs GLM-5" compare page,
// low-precision row), then the top-k of the whole prefix (sparse/compressed-attention
// row of the "Qwen3.5-397B-A17B vs Kimi K3.1 Pro" page; long-context row of the
// "Kimi K3.1 Pro vs Gemma 4 31B" page).
//
// Pass 1 streams the key cache once (256 bytes per key, the bandwidth-bound part): each
// 16-key slice is one pair of v_mfma_f32_16x16x32_bf16 chains with the 32 heads as the M
// dimension (two halves of 16), ReLU and the w-weighted head sum in registers, and one fp32
// score per key written to the workspace (4 bytes against 256 read).
// Pass 2 selects per sequence with an exact most-significant-digit radix select over the
// orderable score keys (11 + 11 + 10 bits), then a stable compaction that keeps every key
// above the threshold plus the lowest-index ties, in ascending index order.
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

constexpr int kChunk = 2048;          // keys per workgroup in pass 1
constexpr int kWaveKeys = kChunk / 4; // keys per wave
constexpr int kUnroll = 4;            // 16-key slices in flight per wave

struct DecArgs {
    const uint16_t *q;
    const uint16_t *w;
    const uint16_t *k_cache;
    const int64_t *start;
    const int32_t *seqlens;
    int max_seqlen;
    float *score_buf;   // [B][max_seqlen]
};

__global__ __launch_bounds__(256) void decode_score_kernel(DecArgs a) {
    const int b = blockIdx.y;
    const int L = max(0, min(a.seqlens[b], a.max_seqlen));
    const int c0 = blockIdx.x * kChunk;
    if (c0 >= L) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;

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
    float *out = a.score_buf + (int64_t)b * a.max_seqlen;
    const int s_begin = c0 + wave * kWaveKeys;
    const int s_end = min(min(c0 + kChunk, L), s_begin + kWaveKeys);

    for (int s0 = s_begin; s0 < s_end; s0 += 16 * kUnroll) {
        u32x4 kb[kUnroll][4];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int key = s0 + 16 * u + l16;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                kb[u][ks] = key < s_end ? *reinterpret_cast<const u32x4 *>(kc + (int64_t)key * kDim + 8 * (4 * ks + lg))
                                        : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            f32x4 s_lo = {0.f, 0.f, 0.f, 0.f}, s_hi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                s_lo = mfma16x16x32(qa[0][ks], kb[u][ks], s_lo);
                s_hi = mfma16x16x32(qa[1][ks], kb[u][ks], s_hi);
            }
            float p = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) p = fmaf(wv[0][r], relu(s_lo[r]), p);
#pragma unroll
            for (int r = 0; r < 4; ++r) p = fmaf(wv[1][r], relu(s_hi[r]), p);
            p += __shfl_xor(p, 16, 64);
            p += __shfl_xor(p, 32, 64);
            const int key = s0 + 16 * u + l16;
            if (lg == 0 && key < s_end) out[key] = p;
        }
    }
}

// ---------------------------------------------------------------- pass 2
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

struct SelSmem {
    uint32_t hist[4][2048];
    int wtot[kSelWaves];
    int bcast[4];
};

// Block-wide exclusive prefix sum of v (all threads must call); returns the total too.
__device__ int block_exclusive_sum(int v, int &total, SelSmem &sm) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_inclusive_sum(v);
    if (lane == 63) sm.wtot[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
        const int t = sm.wtot[i];
        before += i < wave ? t : 0;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return before + incl - v;
}

__global__ __launch_bounds__(kSelThreads) void decode_select_kernel(const float *__restrict__ score_buf,
                                                                    const int32_t *__restrict__ seqlens,
                                                                    int max_seqlen, int topk,
                                                                    int32_t *__restrict__ out_idx,
                                                                    float *__restrict__ out_score) {
    __shared__ SelSmem sm;
    const int b = blockIdx.x;
    const int L = max(0, min(seqlens[b], max_seqlen));
    const int tid = threadIdx.x;
    const float *sc = score_buf + (int64_t)b * max_seqlen;
    int32_t *oi = out_idx + (int64_t)b * topk;
    float *os = out_score ? out_score + (int64_t)b * topk : nullptr;
    if (L <= topk) {
        for (int i = tid; i < topk; i += kSelThreads) {
            oi[i] = i < L ? i : -1;
            if (os) os[i] = i < L ? sc[i] : -INFINITY;
        }
        return;
    }

    uint32_t prefix = 0, pmask = 0;
    int need = topk;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
    for (int p = 0; p < 3; ++p) {
        const int shift = shifts[p];
        const uint32_t dmask = (1u << widths[p]) - 1u;
        for (int i = tid; i < 4 * 2048; i += kSelThreads) (&sm.hist[0][0])[i] = 0u;
        __syncthreads();
        uint32_t *h = sm.hist[tid & 3];
        for (int i = tid; i < L; i += kSelThreads) {
            const uint32_t kv = score_key(sc[i]);
            if ((kv & pmask) == prefix) atomicAdd(&h[(kv >> shift) & dmask], 1u);
        }
        __syncthreads();
        // thread t owns bins 2t, 2t+1
        const int c0 = (int)(sm.hist[0][2 * tid] + sm.hist[1][2 * tid] + sm.hist[2][2 * tid] + sm.hist[3][2 * tid]);
        const int c1 = (int)(sm.hist[0][2 * tid + 1] + sm.hist[1][2 * tid + 1] + sm.hist[2][2 * tid + 1] +
                             sm.hist[3][2 * tid + 1]);
        int total;
        const int excl = block_exclusive_sum(c0 + c1, total, sm);
        const int above_hi = total - excl - c0 - c1;   // entries in bins > 2t+1
        if (above_hi < need && need <= above_hi + c1) {
            sm.bcast[0] = 2 * tid + 1;
            sm.bcast[1] = above_hi;
        } else if (above_hi + c1 < need && need <= above_hi + c1 + c0) {
            sm.bcast[0] = 2 * tid;
            sm.bcast[1] = above_hi + c1;
        }
        __syncthreads();
        const int d = sm.bcast[0];
        need -= sm.bcast[1];
        prefix |= (uint32_t)d << shift;
        pmask |= dmask << shift;
        __syncthreads();
    }

    // stable compaction: keep key > theta, and the first `need` keys == theta
    const uint32_t theta = prefix;
    int out = 0, ties = 0;
    for (int base = 0; base < L; base += 4 * kSelThreads) {
        uint32_t kv[4];
        int eqc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = base + 4 * tid + j;
            kv[j] = i < L ? score_key(sc[i]) : 0u;
            eqc += (i < L && kv[j] == theta) ? 1 : 0;
        }
        int eq_total;
        int eq_rank = ties + block_exclusive_sum(eqc, eq_total, sm);
        bool keep[4];
        int kc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = base + 4 * tid + j;
            const bool in = i < L;
            const bool eq = in && kv[j] == theta;
            keep[j] = in && (kv[j] > theta || (eq && eq_rank < need));
            eq_rank += eq ? 1 : 0;
            kc += keep[j] ? 1 : 0;
        }
        int keep_total;
        int pos = out + block_exclusive_sum(kc, keep_total, sm);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (keep[j] && pos < topk) {
                const int i = base + 4 * tid + j;
                oi[pos] = i;
                if (os) os[pos] = key_score(kv[j]);
                ++pos;
            }
        }
        out += keep_total;
        ties += eq_total;
    }
}

}  // namespace

hipError_t launch_decode(const uint16_t *q, const uint16_t *w, const uint16_t *k_cache,
                         const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                         int topk, float *score_buf, int32_t *idx, float *scores,
                         hipStream_t stream) {
    if (B == 0) return hipSuccess;
    DecArgs a{q, w, k_cache, start, seqlens, max_seqlen, score_buf};
    const int nch = (max_seqlen + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(decode_score_kernel, dim3(nch, B), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_select_kernel, dim3(B), dim3(kSelThreads), 0, stream, score_buf,
                       seqlens, max_seqlen, topk, idx, scores);
    return hipGetLastError();
}

}  // namespace dsaidx
