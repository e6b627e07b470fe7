// FP8 indexer-key cache (serving engines cache the indexer keys in FP8: "Kimi K3.1 Pro vs
// GLM-5" compare page, low-precision row).  The pages give no format or scale; the reading
// here: OCP E4M3 codes (bias 7, largest finite 448, no infinities) with one power-of-two
// scale per cached key (per query head for the new query), the smallest 2^e with
// max|x| <= 448 * 2^e.  x / 2^e is then exact and the only rounding is round-to-nearest-even
// onto E4M3.  A key costs 128 + 4 bytes instead of 256.
//
// The decode score of the FP8 path (decode.hip) is the indexer formula on the dequantised
// vectors ("Qwen3.5-397B-A17B vs Kimi K3.1 Pro" page, sparse/compressed-attention row):
//     I[s] = 2^ek[s] * sum_h (w_h 2^eq_h) * ReLU(q8_h . k8[s])
// (the scales are positive, so they leave the ReLU), with the E4M3 dot products on
// v_mfma_f32_16x16x32_fp8_fp8 (gfx950 reads its operands as OCP E4M3).  This file holds the
// quantisation of the cached keys and of the new queries.
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

// The new queries: q8 [B][H][128] codes and qw[b][h] = w[b][h] * 2^eq[b][h] (exact in fp32).
__global__ __launch_bounds__(256) void quantize_queries_kernel(const uint16_t *__restrict__ q,
                                                               const uint16_t *__restrict__ w, int64_t n,
                                                               uint8_t *__restrict__ q8, float *__restrict__ qw) {
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (b, h), n = B H of them
    if (i >= n) return;
    float sc;
    quantize_row(q + i * kDim, q8 + i * kDim, &sc);
    if (__lane_id() == 0) qw[i] = bf16_to_f32(w[i]) * sc;
}

}  // namespace

hipError_t launch_quantize_keys(const uint16_t *k, int64_t ldk, int64_t N, const int64_t *slot, uint8_t *k8,
                                float *kscale, hipStream_t stream) {
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_keys_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, stream, k, ldk, N, slot,
                       k8, kscale);
    return hipGetLastError();
}

hipError_t launch_quantize_queries(const uint16_t *q, const uint16_t *w, int B, int heads, uint8_t *q8,
                                   float *qw, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    const int64_t n = (int64_t)B * heads;
    hipLaunchKernelGGL(quantize_queries_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream, q, w, n, q8,
                       qw);
    return hipGetLastError();
}

}  // namespace dsaidx
