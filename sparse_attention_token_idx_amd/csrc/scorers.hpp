#pragma once
// Key scorers of one query row against keys in global memory, 64 keys per wave at a time
// (used by the decode passes and by the exact re-scoring of prefill rows).  Each 16-key
// slice is a chain of v_mfma_f32_16x16x32 products with the heads as the M dimension (blocks
// of 16), the keys as N; ReLU and the w-weighted head sum stay in the lane's registers
// (I = sum_h w_h ReLU(q_h . k): "Qwen3.5-397B-A17B vs Kimi K3.1 Pro" compare page,
// sparse/compressed-attention row).
#include "common.hpp"

namespace dsaidx {
// ---------------------------------------------------------------- key scorers
// A scorer holds one sequence's query (the MFMA A operand) and head weights, loads the keys
// of one 64-key group (key[u]: this lane's key, row of the sequence, in slice u) and turns
// them into this lane's partial scores p[u] (its 8 heads).  group_scores then gives lane
// (l16, lg) the score of slice lg's key l16, which the scorer's scale() finishes.

struct Bf16Keys {
    const uint16_t *q, *w, *k_cache;
};

// HB blocks of 16 heads: 2 for the 32-head indexer, 4 for the 64-head one.
template <int HB>
struct Bf16ScorerT {
    static constexpr int kH = 16 * HB;                 // heads
    u32x4 qa[HB][4];   // A operand: head 16 hh + l16, k-slot chunk 4 ks + lg (8 dims)
    float wv[HB][4];
    const uint16_t *kc;
    u32x4 kb[4][4];

    // qb: the row's [kH][128] query, wb: its [kH] head weights, kbase: key 0 of the row
    __device__ __forceinline__ void init_row(const uint16_t *qb, const uint16_t *wb, const uint16_t *kbase,
                                             int l16, int lg) {
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qa[hh][ks] = *reinterpret_cast<const u32x4 *>(qb + (16 * hh + l16) * kDim + 8 * (4 * ks + lg));
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[hh][r] = bf16_to_f32(wb[16 * hh + 4 * lg + r]);
        }
        kc = kbase;
    }
    __device__ __forceinline__ void init(const Bf16Keys &p, const int64_t *start, int b, int l16, int lg) {
        init_row(p.q + (int64_t)b * kH * kDim, p.w + (int64_t)b * kH, p.k_cache + start[b] * kDim, l16, lg);
    }
    __device__ __forceinline__ void load(const int (&key)[4], int lg) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t off = (uint32_t)key[u] * (uint32_t)kDim + 8u * (uint32_t)lg;   // elements
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) kb[u][ks] = *reinterpret_cast<const u32x4 *>(kc + off + 32 * ks);
        }
    }
    // The streamed form of load (the decode filter): stage() copies keys g .. g + 63 of the row
    // (clamped to `last`) into a 16 KB LDS slot, 4 keys of 256 bytes per instruction, row r of
    // the slot keeping its 16-byte chunk c at position c ^ (r % 16) (the 16 rows that one
    // fragment read touches then hit 16 different bank groups); once the loads have landed
    // (vmcnt), load_staged() reads the fragments load() would have read.
    static constexpr int kSlotBytes = 64 * kDim * 2;
    __device__ __forceinline__ void stage(unsigned char *slot, int g, int last, int lane) const {
        const uint32_t base = lds_addr(slot);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 4 * i + (lane >> 4);
            const int key = g + r < last ? g + r : last;
            stream_to_lds(kc + (uint32_t)key * (uint32_t)kDim + 8 * ((lane & 15) ^ (r & 15)), base + 1024u * i);
        }
    }
    __device__ __forceinline__ void load_staged(const unsigned char *slot, int l16, int lg) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                kb[u][ks] = *reinterpret_cast<const u32x4 *>(slot + (16 * u + l16) * (2 * kDim) + 16 * ((lg + 4 * ks) ^ l16));
    }
    __device__ __forceinline__ void partial(float (&p)[4]) const {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            f32x4 s[HB];
#pragma unroll
            for (int hh = 0; hh < HB; ++hh) s[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int hh = 0; hh < HB; ++hh) s[hh] = mfma16x16x32(qa[hh][ks], kb[u][ks], s[hh]);
            float v = 0.f;
#pragma unroll
            for (int hh = 0; hh < HB; ++hh)
#pragma unroll
                for (int r = 0; r < 4; ++r) v = fmaf(wv[hh][r], relu(s[hh][r]), v);
            p[u] = v;
        }
    }
    __device__ __forceinline__ float scale() const { return 1.f; }
    static constexpr bool kScaled = false;

    // The plain (non-MFMA) score of key s, for the select's re-scoring of a row: the query
    // (bf16 pairs) and weights of the row are in LDS.
    static __device__ void stage(const Bf16Keys &p, int b, uint32_t *q_lds, float *w_lds) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(p.q + (int64_t)b * kH * kDim);
        for (int i = (int)threadIdx.x; i < kH * kDim / 2; i += (int)blockDim.x) q_lds[i] = src[i];
        if ((int)threadIdx.x < kH) w_lds[threadIdx.x] = bf16_to_f32(p.w[(int64_t)b * kH + threadIdx.x]);
    }
    static __device__ float rescore(const Bf16Keys &p, const int64_t *start, int b, int s,
                                    const uint32_t *q_lds, const float *w_lds) {
        const uint16_t *kr = p.k_cache + (start[b] + s) * kDim;
        float sc = 0.f;
#pragma unroll 1
        for (int h = 0; h < kH; ++h) {
            float dot = 0.f;
#pragma unroll 1
            for (int c = 0; c < kDim / 8; ++c) {
                const u32x4 kv = *reinterpret_cast<const u32x4 *>(kr + 8 * c);
                const uint32_t *qr = q_lds + h * (kDim / 2) + 4 * c;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    dot = fmaf(bf16_to_f32(qr[j] & 0xFFFFu), bf16_to_f32(kv[j] & 0xFFFFu), dot);
                    dot = fmaf(bf16_to_f32(qr[j] >> 16), bf16_to_f32(kv[j] >> 16), dot);
                }
            }
            sc = fmaf(w_lds[h], relu(dot), sc);
        }
        return sc;
    }
};
using Bf16Scorer = Bf16ScorerT<2>;
static_assert(Bf16Scorer::kH == kHeads, "the 32-head scorer");

struct Fp8Keys {
    const uint8_t *q8;     // [B][32][128] E4M3 codes of the new queries
    const float *qw;       // [B][32] w * 2^eq
    const uint8_t *k8;     // [*][128] E4M3 codes of the cached keys
    const float *kscale;   // [*] 2^ek
};

__device__ __forceinline__ f32x4 mfma_fp8(uint64_t a, uint64_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)a, (long)b, c, 0, 0, 0);
}

// Value of an E4M3 code (bias 7; the codes 0x7F / 0xFF, NaN, never occur in the cache).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return (c & 0x80u) ? -mag : mag;
}

// Lane (l16, lg) of a 16-key slice reads bytes 32 lg .. 32 lg + 31 of key l16 (two 16-byte
// loads); k-step ks uses bytes 32 lg + 8 ks .. + 7 of the key and of the query head.
template <int HB>
struct Fp8ScorerT {
    static constexpr int kH = 16 * HB;                 // heads: 32 or 64
    uint64_t qa[HB][4];
    float wv[HB][4];
    const uint8_t *kc;
    const float *ks;
    u32x4 kb[4][2];
    float kscale;

    __device__ __forceinline__ void init(const Fp8Keys &p, const int64_t *start, int b, int l16, int lg) {
#pragma unroll
        for (int hh = 0; hh < HB; ++hh) {
            const uint8_t *qr = p.q8 + ((int64_t)b * kH + 16 * hh + l16) * kDim + 32 * lg;
            const u32x4 v0 = *reinterpret_cast<const u32x4 *>(qr);
            const u32x4 v1 = *reinterpret_cast<const u32x4 *>(qr + 16);
            qa[hh][0] = (uint64_t)v0[0] | ((uint64_t)v0[1] << 32);
            qa[hh][1] = (uint64_t)v0[2] | ((uint64_t)v0[3] << 32);
            qa[hh][2] = (uint64_t)v1[0] | ((uint64_t)v1[1] << 32);
            qa[hh][3] = (uint64_t)v1[2] | ((uint64_t)v1[3] << 32);
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[hh][r] = p.qw[(int64_t)b * kH + 16 * hh + 4 * lg + r];
        }
        kc = p.k8 + start[b] * kDim;
        ks = p.kscale + start[b];
    }
    __device__ __forceinline__ void load(const int (&key)[4], int lg) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t off = (uint32_t)key[u] * (uint32_t)kDim + 32u * (uint32_t)lg;
            kb[u][0] = *reinterpret_cast<const u32x4 *>(kc + off);
            kb[u][1] = *reinterpret_cast<const u32x4 *>(kc + off + 16);
        }
        kscale = ks[key[lg]];   // this lane's output key: slice lg, key l16
    }
    // Streamed form (the decode filter), as for bf16 keys: an 8 KB slot, 8 keys of 128 bytes per
    // instruction, row r keeping its chunk c at position c ^ (r % 8); the scales are loaded
    // directly.
    static constexpr int kSlotBytes = 64 * kDim;
    __device__ __forceinline__ void stage(unsigned char *slot, int g, int last, int lane) {
        const uint32_t base = lds_addr(slot);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * i + (lane >> 3);
            const int key = g + r < last ? g + r : last;
            stream_to_lds(kc + (uint32_t)key * (uint32_t)kDim + 16 * ((lane & 7) ^ (r & 7)), base + 1024u * i);
        }
        const int own = g + 16 * (lane >> 4) + (lane & 15);   // this lane's output key: slice lg, key l16
        kscale = __builtin_nontemporal_load(ks + (own < last ? own : last));
    }
    __device__ __forceinline__ void load_staged(const unsigned char *slot, int l16, int lg) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                kb[u][j] = *reinterpret_cast<const u32x4 *>(slot + (16 * u + l16) * kDim + 16 * ((2 * lg + j) ^ (l16 & 7)));
    }
    __device__ __forceinline__ void partial(float (&p)[4]) const {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint64_t b0 = (uint64_t)kb[u][0][0] | ((uint64_t)kb[u][0][1] << 32);
            const uint64_t b1 = (uint64_t)kb[u][0][2] | ((uint64_t)kb[u][0][3] << 32);
            const uint64_t b2 = (uint64_t)kb[u][1][0] | ((uint64_t)kb[u][1][1] << 32);
            const uint64_t b3 = (uint64_t)kb[u][1][2] | ((uint64_t)kb[u][1][3] << 32);
            const uint64_t bk[4] = {b0, b1, b2, b3};
            f32x4 s[HB];
#pragma unroll
            for (int hh = 0; hh < HB; ++hh) s[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int hh = 0; hh < HB; ++hh) s[hh] = mfma_fp8(qa[hh][c], bk[c], s[hh]);
            float v = 0.f;
#pragma unroll
            for (int hh = 0; hh < HB; ++hh)
#pragma unroll
                for (int r = 0; r < 4; ++r) v = fmaf(wv[hh][r], relu(s[hh][r]), v);
            p[u] = v;
        }
    }
    __device__ __forceinline__ float scale() const { return kscale; }
    static constexpr bool kScaled = true;

    static __device__ void stage(const Fp8Keys &p, int b, uint32_t *q_lds, float *w_lds) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(p.q8 + (int64_t)b * kH * kDim);
        for (int i = (int)threadIdx.x; i < kH * kDim / 4; i += (int)blockDim.x) q_lds[i] = src[i];
        if ((int)threadIdx.x < kH) w_lds[threadIdx.x] = p.qw[(int64_t)b * kH + threadIdx.x];
    }
    static __device__ float rescore(const Fp8Keys &p, const int64_t *start, int b, int s,
                                    const uint32_t *q_lds, const float *w_lds) {
        const uint8_t *kr = p.k8 + (start[b] + s) * kDim;
        float sc = 0.f;
#pragma unroll 1
        for (int h = 0; h < kH; ++h) {
            float dot = 0.f;
#pragma unroll 1
            for (int c = 0; c < kDim / 16; ++c) {
                const u32x4 kv = *reinterpret_cast<const u32x4 *>(kr + 16 * c);
                const uint32_t *qr = q_lds + h * (kDim / 4) + 4 * c;
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    dot = fmaf(e4m3_value((qr[j / 4] >> (8 * (j % 4))) & 0xFFu),
                               e4m3_value((kv[j / 4] >> (8 * (j % 4))) & 0xFFu), dot);
            }
            sc = fmaf(w_lds[h], relu(dot), sc);
        }
        return sc * p.kscale[start[b] + s];
    }
};
using Fp8Scorer = Fp8ScorerT<2>;

template <class Sc>
__device__ __forceinline__ float finish(const Sc &sc, const float (&p)[4], float scl, int lg) {
    const float v = group_scores(p, lg);
    return Sc::kScaled ? v * scl : v;
}


}  // namespace dsaidx
