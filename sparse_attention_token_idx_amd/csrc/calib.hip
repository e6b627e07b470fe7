// Calibration (not part of the indexer): the sustained bf16 matrix-core rate of this device,
// the ceiling that the score pass and the projections are measured against beside the
// published peak (which assumes the top clock; under a full MFMA load the clock drops).
//
// Every SIMD runs one wave of 16 independent v_mfma_f32_16x16x32_bf16 accumulation chains
// on operands held in registers, so the matrix core never waits for a dependency or for
// memory; four such waves per workgroup (one per SIMD), kCalibBlocks workgroups.  The
// operands are zero or bf16 values with random mantissas and signs in [-2, -0.5] u [0.5, 2]
// (the multipliers' power, hence the clock, depends on the data).  Each lane adds up its
// accumulators into `sink` so that the work cannot be dropped.
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

constexpr int kCalibChains = 16;

__device__ __forceinline__ uint32_t calib_hash(uint32_t x) {   // lowbias32
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// A bf16 pair with random signs, exponents 126 or 127 and random mantissas.
__device__ __forceinline__ uint32_t calib_pair(uint32_t h) {
    const uint32_t lo = (h & 0x80FFu) | 0x3F00u;
    const uint32_t hi = ((h >> 16) & 0x80FFu) | 0x3F00u;
    return lo | hi << 16;
}

__global__ __launch_bounds__(256) void mfma_calibrate_kernel(int64_t iters, int random_operands, float *sink) {
    const uint32_t id = blockIdx.x * 256u + threadIdx.x;
    u32x4 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t h = calib_hash(id * 64u + 8u * j + r);
            const uint32_t g = calib_hash(h ^ 0x9e3779b9u);
            a[j][r] = random_operands ? calib_pair(h) : 0u;
            b[j][r] = random_operands ? calib_pair(g) : 0u;
        }
    f32x4 acc[kCalibChains];
#pragma unroll
    for (int i = 0; i < kCalibChains; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kCalibChains; ++i) acc[i] = mfma16x16x32(a[i & 3], b[i >> 2], acc[i]);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kCalibChains; ++i) s += (acc[i][0] + acc[i][1]) + (acc[i][2] + acc[i][3]);
    sink[id] = s;
}

}  // namespace

int64_t mfma_calibrate_flop(int64_t iters) {
    // 16 x 16 x 32 multiply-adds per product, kCalibChains products per lane group of 64
    return (int64_t)kCalibBlocks * 4 * iters * kCalibChains * (2LL * 16 * 16 * 32);
}

hipError_t launch_mfma_calibrate(int64_t iters, int random_operands, float *sink, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_calibrate_kernel, dim3(kCalibBlocks), dim3(256), 0, stream, iters, random_operands, sink);
    return hipGetLastError();
}

}  // namespace dsaidx
