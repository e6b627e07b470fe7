// FP8 indexer-key cache (serving engines cache the indexer keys in FP8: "Kimi K3.1 Pro vs
// GLM-5" compare page, low-precision row).  The pages give no format or scale; the reading
// here: OCP E4M3 codes (bias 7, largest finite 448, no infinities) with one power-of-two
// scale per cached key (per query head for the new query), the smallest 2^e with
// max|x| <= 448 * 2^e.  x / 2^e is then exact and the only rounding is round-to-nearest-even
// onto E4M3.  A key costs 128 + 4 bytes instead of 256.
//
// The decode score of the FP8 path is the indexer formula on the dequantised vectors
// ("Qwen3.5-397B-A17B vs Kimi K3.1 Pro" page, sparse/compressed-attention row):
//     I[s] = 2^ek[s] * sum_h (w_h 2^eq_h) * ReLU(q8_h . k8[s])
// (the scales are positive, so they leave the ReLU), with the E4M3 dot products on
// v_mfma_f32_16x16x32_fp8_fp8 (gfx950 reads its operands as OCP E4M3).
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

// Exponent e of the smallest power-of-two scale with amax <= 448 * 2^e (0 for amax = 0).
// amax = m * 2^x with m in [0.5, 1): amax <= 448 * 2^e  <=>  2m * 2^(x-1) <= 1.75 * 2^(e+8),
// so e = x - 9 when 2m <= 1.75, else x - 8.  frexpf is exact, subnormals included.
__device__ __forceinline__ int pow2_scale_exp(float amax) {
    if (!(amax > 0.f)) return 0;
    int x;
    const float m = frexpf(amax, &x);
    return m <= 0.875f ? x - 9 : x - 8;
}

// E4M3 code of v (|v| <= 448), round to nearest even, from the float's bits: in the binade
// [2^E, 2^(E+1)), E >= -6, the 24-bit significand keeps its top 4 bits (1 + 3 mantissa
// bits) with the 20 below rounded off; below 2^-6 the subnormal spacing is 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sgn = (u >> 24) & 0x80u;
    const float a = fabsf(v);
    uint32_t mag;
    if (a < 0.015625f) {                                   // 2^-6
        mag = (uint32_t)__builtin_rintf(a * 512.f);        // exact product, rint: ties to even
    } else {
        const int E = (int)((u >> 23) & 0xFFu) - 127;
        const uint32_t sig = (u & 0x7FFFFFu) | 0x800000u;
        uint32_t q = sig >> 20;                            // 8 .. 15
        const uint32_t rem = sig & 0xFFFFFu;
        q += (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u;   // 8 .. 16
        mag = 8u * (uint32_t)(E + 6) + q;
    }
    return sgn | mag;
}

// One wave per vector of 128 bf16: codes to dst (128 bytes), the scale 2^e to *scale, and
// for the query path also the weight folded with the scale.
__device__ __forceinline__ void quantize_row(const uint16_t *src, uint8_t *dst, float *scale_out) {
    const int lane = __lane_id();
    const uint32_t pair = *reinterpret_cast<const uint32_t *>(src + 2 * lane);
    const float v0 = bf16_to_f32(pair & 0xFFFFu), v1 = bf16_to_f32(pair >> 16);
    float m = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
    const int e = pow2_scale_exp(m);
    const uint32_t c0 = e4m3_rne(ldexpf(v0, -e)), c1 = e4m3_rne(ldexpf(v1, -e));
    *reinterpret_cast<uint16_t *>(dst + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
    if (lane == 0) *scale_out = ldexpf(1.f, e);
}

__global__ __launch_bounds__(256) void quantize_keys_kernel(const uint16_t *__restrict__ k, int64_t ldk,
                                                            int64_t N, const int64_t *__restrict__ slot,
                                                            uint8_t *__restrict__ k8, float *__restrict__ kscale) {
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= N) return;
    const int64_t r = slot ? slot[i] : i;
    quantize_row(k + i * ldk, k8 + r * kDim, kscale + r);
}

// The new queries: q8 [B][32][128] codes and qw[b][h] = w[b][h] * 2^eq[b][h] (exact in fp32).
__global__ __launch_bounds__(256) void quantize_queries_kernel(const uint16_t *__restrict__ q,
                                                               const uint16_t *__restrict__ w, int B,
                                                               uint8_t *__restrict__ q8, float *__restrict__ qw) {
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (b, h)
    if (i >= (int64_t)B * kHeads) return;
    float sc;
    quantize_row(q + i * kDim, q8 + i * kDim, &sc);
    if (__lane_id() == 0) qw[i] = bf16_to_f32(w[i]) * sc;
}

constexpr int kDecThreads = 256;
constexpr int kSplit = 64;            // a workgroup's share of keys is a multiple of this

struct Fp8Args {
    const uint8_t *q8;
    const float *qw;
    const uint8_t *k8;
    const float *kscale;
    const int64_t *start;
    const int64_t *cu;             // prefix sums of the cache lengths rounded up to 64
    const int32_t *seqlens;
    int max_seqlen;
    int B;
    int64_t ld;
    float *score_buf;
};

__device__ __forceinline__ f32x4 mfma_fp8(uint64_t a, uint64_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)a, (long)b, c, 0, 0, 0);
}

// As the bf16 decode score pass: the flat range of all cached keys (each sequence padded to a
// multiple of 64) split evenly over the grid, 64-key groups per wave, one 256-byte store of
// scores per group; lane (l16, lg) of a 16-key slice reads bytes 32 lg .. 32 lg + 31 of key
// l16 (two 16-byte loads), k-step ks uses bytes 32 lg + 8 ks .. + 7 of the key and of the
// query head (rows of the A operand: head 16 hh + l16).  The key scales of a group are read
// with one 256-byte load, lane i taking key i's.
__global__ __launch_bounds__(kDecThreads) void decode_score_fp8_kernel(Fp8Args a) {
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
        while (a.cu[b + 1] <= pos) ++b;
        const int64_t seg_end = min(end, a.cu[b + 1]);
        const int len = max(0, min(a.seqlens[b], a.max_seqlen));
        const int s_begin = (int)(pos - a.cu[b]), s_end = min(len, (int)(seg_end - a.cu[b]));

        uint64_t qa[2][4];
        float wv[2][4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint8_t *qr = a.q8 + ((int64_t)b * kHeads + 16 * hh + l16) * kDim + 32 * lg;
            const u32x4 v0 = *reinterpret_cast<const u32x4 *>(qr);
            const u32x4 v1 = *reinterpret_cast<const u32x4 *>(qr + 16);
            qa[hh][0] = (uint64_t)v0[0] | ((uint64_t)v0[1] << 32);
            qa[hh][1] = (uint64_t)v0[2] | ((uint64_t)v0[3] << 32);
            qa[hh][2] = (uint64_t)v1[0] | ((uint64_t)v1[1] << 32);
            qa[hh][3] = (uint64_t)v1[2] | ((uint64_t)v1[3] << 32);
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[hh][r] = a.qw[(int64_t)b * kHeads + 16 * hh + 4 * lg + r];
        }
        const uint8_t *kc = a.k8 + a.start[b] * kDim;
        const float *ks = a.kscale + a.start[b];
        float *out = a.score_buf + (int64_t)b * a.ld;

        // next group's loads before this group's store; every lane stores (see the bf16 pass)
        u32x4 kb[4][2];
        float kscale;
        auto load = [&](int g) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int key = min(g + 16 * u + l16, s_end - 1);
                const uint32_t off = (uint32_t)key * (uint32_t)kDim + 32u * (uint32_t)lg;
                kb[u][0] = *reinterpret_cast<const u32x4 *>(kc + off);
                kb[u][1] = *reinterpret_cast<const u32x4 *>(kc + off + 16);
            }
            kscale = ks[min(g + lane, s_end - 1)];
        };
        int g0 = s_begin + 64 * wave;
        if (g0 < s_end) load(g0);
        for (; g0 < s_end; g0 += 256) {
            float p[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint64_t b0 = (uint64_t)kb[u][0][0] | ((uint64_t)kb[u][0][1] << 32);
                const uint64_t b1 = (uint64_t)kb[u][0][2] | ((uint64_t)kb[u][0][3] << 32);
                const uint64_t b2 = (uint64_t)kb[u][1][0] | ((uint64_t)kb[u][1][1] << 32);
                const uint64_t b3 = (uint64_t)kb[u][1][2] | ((uint64_t)kb[u][1][3] << 32);
                f32x4 s_lo = {0.f, 0.f, 0.f, 0.f}, s_hi = {0.f, 0.f, 0.f, 0.f};
                s_lo = mfma_fp8(qa[0][0], b0, s_lo);
                s_hi = mfma_fp8(qa[1][0], b0, s_hi);
                s_lo = mfma_fp8(qa[0][1], b1, s_lo);
                s_hi = mfma_fp8(qa[1][1], b1, s_hi);
                s_lo = mfma_fp8(qa[0][2], b2, s_lo);
                s_hi = mfma_fp8(qa[1][2], b2, s_hi);
                s_lo = mfma_fp8(qa[0][3], b3, s_lo);
                s_hi = mfma_fp8(qa[1][3], b3, s_hi);
                float v = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) v = fmaf(wv[0][r], relu(s_lo[r]), v);
#pragma unroll
                for (int r = 0; r < 4; ++r) v = fmaf(wv[1][r], relu(s_hi[r]), v);
                p[u] = v;
            }
            const float scale = kscale;
            if (g0 + 256 < s_end) load(g0 + 256);
            out[g0 + lane] = group_scores(p, lg) * scale;
        }
        pos = seg_end;
    }
}

int decode_fp8_grid() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 2048;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_score_fp8_kernel, kDecThreads, 0) != hipSuccess ||
        per <= 0)
        per = 2;
    const int g = 8 * per * cus;   // eight rounds of the workgroups resident at once: short shares
    if (dev < 64) cached[dev] = g;
    return g;
}

}  // namespace

hipError_t launch_quantize_keys(const uint16_t *k, int64_t ldk, int64_t N, const int64_t *slot, uint8_t *k8,
                                float *kscale, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_keys_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, stream, k, ldk, N, slot,
                       k8, kscale);
    return hipGetLastError();
}

hipError_t launch_decode_fp8(const uint16_t *q, const uint16_t *w, const uint8_t *k8, const float *kscale,
                             const int64_t *start, const int32_t *seqlens, int B, int max_seqlen, int topk,
                             int64_t *cu, float *score_buf, uint8_t *q8, float *qw, int32_t *idx,
                             float *scores, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    hipError_t e = launch_decode_prefix(seqlens, B, max_seqlen, cu, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(quantize_queries_kernel, dim3((unsigned)(((int64_t)B * kHeads + 3) / 4)), dim3(256), 0,
                       stream, q, w, B, q8, qw);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ld = decode_row_stride(max_seqlen);
    Fp8Args a{q8, qw, k8, kscale, start, cu, seqlens, max_seqlen, B, ld, score_buf};
    const int64_t bound = (int64_t)B * ((max_seqlen + kSplit - 1) / kSplit);
    const int64_t grid = bound < decode_fp8_grid() ? bound : decode_fp8_grid();
    hipLaunchKernelGGL(decode_score_fp8_kernel, dim3((unsigned)grid), dim3(kDecThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_row_topk_decode(score_buf, seqlens, B, ld, max_seqlen, topk, idx, scores, stream);
}

}  // namespace dsaidx
