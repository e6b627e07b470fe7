// Device-side building blocks shared by the libdsaidx kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsaidx {

constexpr int kHeads = 32;
constexpr int kDim = 128;
constexpr int kQLat = 1536;
constexpr int kQOut = 4096;
constexpr int kHidden = 7168;
constexpr int kMaxTopk = 2048;

// ---------------------------------------------------------------- prefill sampling
// A prefill row samples one key per stratum of kSampleStride consecutive keys (at an offset
// inside the stratum picked by an integer hash of the stratum), to place its threshold; rows
// of at most kAllKeys keys keep every key as a candidate.  The threshold is the r-th largest
// sample score with r = E + kThetaMargin (sqrt(E) + 1), E the expected number of samples at or
// above the row's topk-th score.
constexpr int kSampleStride = 32;
constexpr int64_t kAllKeys = 4096;
constexpr double kThetaMargin = 6.0;

// The "lowbias32" integer mixer (C. Wellons' hash prospector).
__host__ __device__ inline uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7FEB352Du;
    x ^= x >> 15;
    x *= 0x846CA68Bu;
    x ^= x >> 16;
    return x;
}

// Offset of stratum j's sampled key inside the stratum.
__host__ __device__ inline int sample_offset(int64_t j) {
    return (int)(mix32((uint32_t)j + 0x9E3779B9u) & (uint32_t)(kSampleStride - 1));
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// 16-byte vector with 4-byte alignment, for global stores at any dword offset
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));

// ---------------------------------------------------------------- bf16
typedef __attribute__((address_space(3))) void lds_void;

// LDS address of a pointer into shared memory, uniform over the wave (an SGPR operand).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(const lds_void *)p);
}

// A read of data streamed once (the key caches of the decode): one 16-byte-per-lane
// global -> LDS load, lane i landing at lds + 16 i, marked non-temporal.  Issued so that each
// instruction covers whole cache lines (1 KB, contiguous), a read-only stream over 1.3 GB of
// device memory runs at about 6.9 TB/s this way, against 6.1 TB/s with plain loads, and 5.6
// TB/s with non-temporal loads of the 64-byte row pieces that a matrix-core fragment wants.
// Written out so that the compiler does not wait for it before every LDS access; the caller
// waits (vmcnt) before reading the data.  It has no result registers.
__device__ __forceinline__ void stream_to_lds(const void *src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds)
                 : "memory", "m0");
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------- MFMA
// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.  Lane l supplies
// A[l % 16][kk] and B[kk][l % 16] for the 8 values kk of its k-slot (any assignment of
// the 32 k values to (lane / 16, element) works as long as A and B use the same one),
// and receives D[4 * (l / 16) + r][l % 16] in element r.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// max(x, 0) as one integer max on the bit pattern: non-negative floats order like their
// bits read as int32, and every negative float (-0 included) is a negative int32, which the
// max turns into +0.  A float max would first canonicalize x, costing a second instruction.
__device__ __forceinline__ float relu(float x) {
    const int b = __float_as_int(x);
    return __int_as_float(b > 0 ? b : 0);
}

// ---------------------------------------------------------------- ordering keys
// Monotone map fp32 -> uint32 (larger score -> larger key); -0 is mapped as +0 so the two
// zeros tie.  NaN is outside the contract.
__device__ __forceinline__ uint32_t score_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// score_key for a value known not to be -0 (the two zeros would get different keys): one
// arithmetic shift and two bitwise ops.
__device__ __forceinline__ uint32_t score_key_nz(float v) {
    const uint32_t u = __float_as_uint(v);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// ---------------------------------------------------------------- wave64 helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of `mask` in lanes strictly below the calling lane.
__device__ __forceinline__ uint32_t bits_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int readlane(int v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}

// Inclusive prefix sum across the 64 lanes.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    const int l = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(v, d, 64);
        if (l >= d) v += o;
    }
    return v;
}

// Inclusive prefix sum within each 16-lane row of the wave (DPP row shifts).
__device__ __forceinline__ int row16_inclusive_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    return x;
}

// Value of the last lane (15) of the calling lane's 16-lane row: four lane reads and a
// select, all on the VALU (no LDS round trip on a latency-bound path).
__device__ __forceinline__ int row16_last(int x) {
    const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
    const int r2 = __builtin_amdgcn_readlane(x, 47), r3 = __builtin_amdgcn_readlane(x, 63);
    const int g = __lane_id() >> 4;
    return g == 0 ? r0 : (g == 1 ? r1 : (g == 2 ? r2 : r3));
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

// Sum over the four lane groups (lg = lane / 16) of this lane's partial scores p[u] of the
// four slices u of a 64-key group, returned so that lane (l16, lg) holds slice lg's total:
// the score of key 16 lg + l16 of the group.  Two exchanges across lg bit 1, one across bit 0.
__device__ __forceinline__ float group_scores(const float (&p)[4], int lg) {
    const bool h = (lg >> 1) & 1, e = lg & 1;
    const float x0 = (h ? p[2] : p[0]) + __shfl_xor(h ? p[0] : p[2], 32, 64);   // slice 2h
    const float x1 = (h ? p[3] : p[1]) + __shfl_xor(h ? p[1] : p[3], 32, 64);   // slice 2h + 1
    return (e ? x1 : x0) + __shfl_xor(e ? x0 : x1, 16, 64);
}

}  // namespace dsaidx
