// The rotary step of the DeepSeek-V3.2-shaped indexer.  The pages give it 64 heads (sparse-
// attention row of the "Qwen3.5-397B-A17B vs Kimi K3.1 Pro" compare page) and say it rotates
// 64 of its 128 dims (RoPE row of the "Kimi K3.1 Pro vs Gemma 4 31B" page).  Read here as:
// dims (2i, 2i+1), i < 32, of every query head and of the key turn by the angle
// pos * theta^(-2i/64), applied to the projections as stored in bf16 and rounded to bf16
// once more; dims 64..127 stay.
//
// One thread per (token, pair): it forms the angle and its sine and cosine in fp64 (positions
// reach 2^20, where an fp32 angle would be off by tenths of a radian), turns the pair of every
// head and of the key in fp64, and rounds each result to bf16 directly (round to odd into fp32,
// then to nearest even into bf16, which is the correctly rounded bf16 value).  The 32 threads
// of a token touch 128 contiguous bytes of each head.  A thread loads the pairs of kBatch
// heads before it turns and stores them, so each thread waits on a few memory round trips
// instead of one per head; the key and the first batch are in flight while it forms the
// sine and cosine.
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

constexpr int kRotPairs = 32;   // pairs turned per head: 64 of the 128 dims

__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    float f = __double2float_rz(x);
    if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);   // round to odd (NaN stays NaN)
    return (uint16_t)f32_to_bf16(f);
}

constexpr int kBatch = 16;      // head pairs loaded before the first of them is turned

__device__ __forceinline__ uint32_t turn(uint32_t v, double c, double s) {
    const double x = (double)bf16_to_f32(v & 0xFFFFu), y = (double)bf16_to_f32(v >> 16);
    return (uint32_t)f64_to_bf16(x * c - y * s) | ((uint32_t)f64_to_bf16(x * s + y * c) << 16);
}

__global__ __launch_bounds__(256) void rope_kernel(uint16_t *q, int64_t ldq, int heads, uint16_t *k, int64_t ldk,
                                                   int64_t T, int64_t pos0, double theta) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t t = g / kRotPairs;
    const int i = (int)(g % kRotPairs);
    if (t >= T) return;
    uint32_t *kp = k ? reinterpret_cast<uint32_t *>(k + t * ldk + 2 * i) : nullptr;
    uint32_t *qp = q ? reinterpret_cast<uint32_t *>(q + t * ldq + 2 * i) : nullptr;
    constexpr int64_t kHeadStride = kDim / 2;   // uint32 pairs between heads
    uint32_t kv = 0, v[kBatch];
    auto load_batch = [&](int h0) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (h0 + j < heads) v[j] = qp[(int64_t)(h0 + j) * kHeadStride];
    };
    if (kp) kv = *kp;
    if (qp) load_batch(0);
    const double ang = (double)(pos0 + t) * pow(theta, -2.0 * i / (2 * kRotPairs));
    double s, c;
    sincos(ang, &s, &c);
    if (qp) {
        for (int h0 = 0;;) {
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (h0 + j < heads) qp[(int64_t)(h0 + j) * kHeadStride] = turn(v[j], c, s);
            h0 += kBatch;
            if (h0 >= heads) break;
            load_batch(h0);
        }
    }
    if (kp) *kp = turn(kv, c, s);
}

}  // namespace

hipError_t launch_rope(uint16_t *q, int64_t ldq, int heads, uint16_t *k, int64_t ldk, int64_t T, int64_t pos0,
                       double theta, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int64_t n = T * kRotPairs;
    hipLaunchKernelGGL(rope_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, q, ldq, heads, k, ldk,
                       T, pos0, theta);
    return hipGetLastError();
}

}  // namespace dsaidx
