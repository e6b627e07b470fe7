// Sparse MLA over the selected tokens: the consumer of the indexer's selection ("Qwen3.5-397B-
// A17B vs Kimi K3.1 Pro" compare page, gated-MLA row: 96 heads, keys and values from a 512-dim
// latent plus a 64-dim shared key slot, 576 cached values per token, each query attending only
// to the 2,048 tokens its layer's indexer selects; no rotary step, RoPE row of the "Kimi K3.1
// Pro vs Gemma 4 31B" page).  Queries arrive in the absorbed latent form q~ [96][576], so head
// h's logit for a selected token s is scale * q~_h . kv[s] over the 576 cached values, the
// softmax runs over the selected tokens, and the head's output is the softmax-weighted sum of
// the 512-dim latents (value up-projection, output gate and output projection follow as dense
// products).
//
// One workgroup takes one query and a contiguous split of its selections; its 12 waves pair up
// on 16 heads each, one wave of a pair taking the first half of the 576 logit dims and of the
// 512 output dims, the other the second halves, so that a wave holds its query slice (36
// VGPRs) and its output (64) with three waves per SIMD.  The selected cache rows stream
// through LDS 32 at a time with direct global->LDS loads (double-buffered): row-major for the
// logits S^T = K q~^T (v_mfma_f32_16x16x32_bf16, the wave's q~ as the B operand), whose two
// halves the pair adds through LDS, and transposed (latent dim major) for O^T += V^T P^T,
// whose B operand is the wave's probabilities straight from the logit accumulators (the 32
// tokens of a tile taken in the order the accumulators hold them).  The softmax is online, in
// the log2 domain; with several splits per query, a second kernel merges the splits' (max,
// sum, unnormalised output).
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

constexpr int kMlaHeads = 96;
constexpr int kKv = 576;                 // cached values per token
constexpr int kV = 512;                  // latent (value) dims
constexpr int kWavesMla = 2 * (kMlaHeads / 16);   // a pair per 16 heads
constexpr int kMlaThreads = 64 * kWavesMla;
constexpr int kTile = 32;                // selected tokens per LDS tile
constexpr int kPieces = kKv / 8;         // 16-byte pieces of a cache row: 72
constexpr int kSlots = kTile * kPieces;  // of a tile: 2,304 = 36 load instructions of 64 lanes
constexpr int kSlotsPerWave = kSlots / kMlaThreads;   // 3
constexpr int kVRow = 36;                // bf16 per latent-dim row of the V^T area (72 bytes)
constexpr int kMaxSel = 2048;            // selections per split held in LDS
static_assert(kSlots % kMlaThreads == 0 && kPieces % 8 == 0, "tile geometry");

typedef __attribute__((address_space(3))) void lds_void;

struct MlaSmem {
    // token rows of two tiles: piece u of token tau sits in slot 72 tau + (u ^ (tau & 7)) (16
    // bytes each), which spreads the 16 rows one MFMA operand read touches over the banks
    uint16_t k[2][kSlots * 8];
    uint16_t vt[kV][kVRow];      // the current tile, latent-dim major (token contiguous)
    int32_t sel[kMaxSel];        // this split's selections (-1: none)
    f32x4 sx[kWavesMla][2][64];  // each wave's half of the logits, for its partner
};

struct MlaArgs {
    const uint16_t *q;       // [T][96][576]
    const uint16_t *kv;      // [*][576]
    const int32_t *idx;      // [T][topk]
    const int64_t *row0;     // [T] or nullptr
    int64_t T;
    int topk;
    int nsplit;
    int per;                 // selections per split (a multiple of kTile, at most kMaxSel)
    float scale_log2;        // scale * log2(e)
    uint16_t *o;             // [T][96][512] (nsplit == 1)
    float *lse;              // [T][96] or nullptr (nsplit == 1)
    float *part_o;           // [nsplit][T][96][512] unnormalised (nsplit > 1)
    float *part_ml;          // [nsplit][T][96][2]: running max (log2 domain), sum
};

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) { return pack_bf16x2(lo, hi); }

// Workgroup barrier over LDS traffic only: __syncthreads() would also wait for every global
// load in flight, the next tile's included.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ __launch_bounds__(kMlaThreads, 1) void sparse_mla_kernel(MlaArgs a) {
    static_assert(kV / 16 / 2 * 2 == kV / 16 && kKv / 32 % 2 == 0, "halves");
    extern __shared__ __align__(16) unsigned char smem_raw[];
    MlaSmem &sm = *reinterpret_cast<MlaSmem *>(smem_raw);
    const int split = blockIdx.x;
    const int64_t t = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const int hg = wave >> 1, half = wave & 1;   // heads 16 hg .. + 15; dims half
    constexpr int kKs = kKv / 32 / 2;             // logit k-steps of a half: 9
    constexpr int kMt = kV / 16 / 2;              // 16-dim output tiles of a half: 16
    const int sel0 = split * a.per;
    const int nsel = max(0, min(a.topk, sel0 + a.per) - sel0);
    const int ntile = (nsel + kTile - 1) / kTile;
    const int64_t base = a.row0 ? a.row0[t] : 0;
    for (int x = tid; x < ntile * kTile; x += kMlaThreads)
        sm.sel[x] = x < nsel ? a.idx[t * (int64_t)a.topk + sel0 + x] : -1;

    // this wave's q~ as the B operand of S^T = K q~^T: lane (l16, g) holds head 16 hg + l16,
    // dims 32 (kKs half + ks) + 8 g .. + 7
    u32x4 qb[kKs];
    {
        const uint16_t *qh = a.q + (t * kMlaHeads + 16 * hg + l16) * (int64_t)kKv + 32 * kKs * half + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) qb[ks] = *reinterpret_cast<const u32x4 *>(qh + 32 * ks);
    }
    __syncthreads();   // sel

    // A tile goes to LDS with direct global->LDS loads: slot 64 (6 wave + j) + lane of
    // instruction j holds piece u = (slot % 72) ^ (tau & 7) of token tau = slot / 72.  A token
    // with no selection reads cache row 0 instead (its logit is masked, its weight is 0).
    auto load_tile = [&](int tile, int buf) {
#pragma unroll
        for (int j = 0; j < kSlotsPerWave; ++j) {
            const int slot0 = 64 * (kSlotsPerWave * wave + j);
            const int slot = slot0 + lane;
            const int tau = slot / kPieces, u = (slot % kPieces) ^ (tau & 7);
            const int32_t r = sm.sel[tile * kTile + tau];
            const int64_t row = r >= 0 ? base + r : 0;
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(a.kv + row * kKv + 8 * u),
                                             (lds_void *)(&sm.k[buf][8 * slot0]), 16, 0, 0);
        }
    };
    // the latent part of a tile, transposed into vt: thread i < 512 takes 4 consecutive tokens
    // 4 (i % 8) .. + 3 of piece u = i / 8 (8 dims) and writes each dim's 4 tokens as 8 bytes
    auto transpose = [&](int buf) {
        if (tid < (kTile / 4) * (kV / 8)) {
            const int tq = tid & 7, u = tid >> 3;
            u32x4 v[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int tau = 4 * tq + x;
                v[x] = *reinterpret_cast<const u32x4 *>(&sm.k[buf][8 * (kPieces * tau + (u ^ (tau & 7)))]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // dims 8 u + 2 j (low halves) and 8 u + 2 j + 1 (high halves) of the 4 tokens
                const uint2 lo = {(v[0][j] & 0xFFFFu) | (v[1][j] << 16), (v[2][j] & 0xFFFFu) | (v[3][j] << 16)};
                const uint2 hi = {(v[0][j] >> 16) | (v[1][j] & 0xFFFF0000u), (v[2][j] >> 16) | (v[3][j] & 0xFFFF0000u)};
                *reinterpret_cast<uint2 *>(&sm.vt[8 * u + 2 * j][4 * tq]) = lo;
                *reinterpret_cast<uint2 *>(&sm.vt[8 * u + 2 * j + 1][4 * tq]) = hi;
            }
        }
    };

    f32x4 acc_o[kMt];   // O^T: lane (l16, g) holds dims 256 half + 16 mt + 4 g + r of head 16 hg + l16
#pragma unroll
    for (int mt = 0; mt < kMt; ++mt) acc_o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // running max of the head's logits (log2 domain)
    float l_run = 0.f;         // this lane's part of the running sum

    if (ntile > 0) load_tile(0, 0);
    __syncthreads();   // (waits for the loads)
    if (ntile > 0) transpose(0);
    __syncthreads();
#pragma unroll 1
    for (int tile = 0; tile < ntile; ++tile) {
        const int buf = tile & 1;
        if (tile + 1 < ntile) load_tile(tile + 1, buf ^ 1);   // in flight during this tile
        // logits: S^T rows are tokens (two 16-token halves), columns the pair's 16 heads; this
        // wave sums its half of the dims, the partner's half comes through LDS
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        const uint16_t *kb = sm.k[buf];
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
            const int u = 4 * (kKs * half + ks) + g;
            const u32x4 k0 = *reinterpret_cast<const u32x4 *>(kb + 8 * (kPieces * l16 + (u ^ (l16 & 7))));
            const u32x4 k1 = *reinterpret_cast<const u32x4 *>(
                kb + 8 * (kPieces * (16 + l16) + (u ^ (l16 & 7))));
            s0 = mfma16x16x32(k0, qb[ks], s0);
            s1 = mfma16x16x32(k1, qb[ks], s1);
        }
        sm.sx[wave][0][lane] = s0;
        sm.sx[wave][1][lane] = s1;
        lds_barrier();
        {   // mine + partner's: both waves of a pair add the same two numbers, so they agree
            const f32x4 o0 = sm.sx[wave ^ 1][0][lane], o1 = sm.sx[wave ^ 1][1][lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                s0[r] += o0[r];
                s1[r] += o1[r];
            }
        }
        // lane (l16, g): head 16 hg + l16, tokens 4 g + r (s0) and 16 + 4 g + r (s1)
        float z[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            z[r] = sm.sel[tile * kTile + 4 * g + r] >= 0 ? s0[r] * a.scale_log2 : -INFINITY;
            z[4 + r] = sm.sel[tile * kTile + 16 + 4 * g + r] >= 0 ? s1[r] * a.scale_log2 : -INFINITY;
        }
        float mx = z[0];
#pragma unroll
        for (int r = 1; r < 8; ++r) mx = fmaxf(mx, z[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        float p[8];
        float factor = 1.f;
        if (m_new == -INFINITY) {
#pragma unroll
            for (int r = 0; r < 8; ++r) p[r] = 0.f;
        } else {
            factor = exp2f(m_run - m_new);   // 0 when m_run is -inf
#pragma unroll
            for (int r = 0; r < 8; ++r) p[r] = exp2f(z[r] - m_new);
        }
        m_run = m_new;
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) ps += p[r];
        l_run = l_run * factor + ps;
        // P^T as the B operand: k slots 8 g .. 8 g + 7 are the lane's 8 tokens, and the V^T
        // operand reads the same tokens (4 g .. 4 g + 3 and 16 + 4 g .. + 3)
        const u32x4 pb = {bf16_pair(p[0], p[1]), bf16_pair(p[2], p[3]), bf16_pair(p[4], p[5]),
                          bf16_pair(p[6], p[7])};
#pragma unroll
        for (int mt = 0; mt < kMt; ++mt) {
            const uint16_t *vr = &sm.vt[256 * half + 16 * mt + l16][0];
            const uint2 lo = *reinterpret_cast<const uint2 *>(vr + 4 * g);
            const uint2 hi = *reinterpret_cast<const uint2 *>(vr + 16 + 4 * g);
            const u32x4 va = {lo.x, lo.y, hi.x, hi.y};
            f32x4 o = acc_o[mt];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] *= factor;
            acc_o[mt] = mfma16x16x32(va, pb, o);
        }
        // vt and k[buf] read by every wave, and (after each wave's wait) the next tile's loads
        // have landed
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        if (tile + 1 < ntile) transpose(buf ^ 1);
        lds_barrier();
    }

    // the head's sum over its 4 lane groups
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int head = 16 * hg + l16;
    if (a.nsplit == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t *oh = a.o + (t * kMlaHeads + head) * (int64_t)kV + 256 * half;
#pragma unroll
        for (int mt = 0; mt < kMt; ++mt) {
            const f32x4 o = acc_o[mt];
            const uint2 v = {bf16_pair(o[0] * inv, o[1] * inv), bf16_pair(o[2] * inv, o[3] * inv)};
            *reinterpret_cast<uint2 *>(oh + 16 * mt + 4 * g) = v;
        }
        if (a.lse && g == 0 && half == 0)
            a.lse[t * kMlaHeads + head] = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    } else {
        const int64_t ph = ((int64_t)split * a.T + t) * kMlaHeads + head;
        float *oh = a.part_o + ph * kV + 256 * half;
#pragma unroll
        for (int mt = 0; mt < kMt; ++mt) *reinterpret_cast<f32x4 *>(oh + 16 * mt + 4 * g) = acc_o[mt];
        if (g == 0 && half == 0) {
            a.part_ml[2 * ph] = m_run;
            a.part_ml[2 * ph + 1] = l_tot;
        }
    }
}

// Merge of the splits of one (query, head): one wave per (query, head), lane i owns dims
// 8 i .. 8 i + 7.
__global__ __launch_bounds__(256) void sparse_mla_merge_kernel(MlaArgs a) {
    const int64_t qh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // t * 96 + head
    if (qh >= a.T * kMlaHeads) return;
    const int lane = threadIdx.x & 63;
    float M = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_ml[2 * ((int64_t)s * a.T * kMlaHeads + qh)]);
    float L = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        for (int s = 0; s < a.nsplit; ++s) {
            const int64_t ph = (int64_t)s * a.T * kMlaHeads + qh;
            const float ms = a.part_ml[2 * ph];
            if (ms == -INFINITY) continue;
            const float f = exp2f(ms - M);
            L += f * a.part_ml[2 * ph + 1];
            const f32x4 x0 = *reinterpret_cast<const f32x4 *>(a.part_o + ph * kV + 8 * lane);
            const f32x4 x1 = *reinterpret_cast<const f32x4 *>(a.part_o + ph * kV + 8 * lane + 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[r] = fmaf(f, x0[r], acc[r]);
                acc[4 + r] = fmaf(f, x1[r], acc[4 + r]);
            }
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const u32x4 v = {bf16_pair(acc[0] * inv, acc[1] * inv), bf16_pair(acc[2] * inv, acc[3] * inv),
                     bf16_pair(acc[4] * inv, acc[5] * inv), bf16_pair(acc[6] * inv, acc[7] * inv)};
    *reinterpret_cast<u32x4 *>(a.o + qh * kV + 8 * lane) = v;
    if (a.lse && lane == 0) a.lse[qh] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

int mla_cus() {
    static int cached = 0;
    if (cached > 0) return cached;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    cached = cus;
    return cus;
}

}  // namespace

int sparse_mla_splits(int64_t T, int topk) {
    if (T <= 0 || topk <= 0) return 1;
    const int64_t want = (2 * (int64_t)mla_cus() + T - 1) / T;           // about 2 workgroups per CU
    const int64_t most = ((int64_t)topk + 8 * kTile - 1) / (8 * kTile);   // at least 8 tiles a split
    const int64_t least = ((int64_t)topk + kMaxSel - 1) / kMaxSel;         // at most kMaxSel a split
    int64_t n = want < most ? want : most;
    n = n < least ? least : n;
    return (int)(n < 1 ? 1 : n);
}

size_t sparse_mla_workspace(int64_t T, int topk) {
    const int ns = sparse_mla_splits(T, topk);
    if (ns <= 1) return 0;
    return (size_t)ns * (size_t)T * kMlaHeads * (kV + 2) * 4u;
}

hipError_t launch_sparse_mla(const uint16_t *q, const uint16_t *kv, const int32_t *idx, const int64_t *row0,
                             int64_t T, int topk, float scale, uint16_t *o, float *lse, float *ws,
                             hipStream_t stream) {
    static bool attr_done = false;
    const size_t smem = sizeof(MlaSmem);
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(sparse_mla_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    if (T == 0) return hipSuccess;
    MlaArgs a{};
    a.q = q;
    a.kv = kv;
    a.idx = idx;
    a.row0 = row0;
    a.T = T;
    a.topk = topk;
    a.nsplit = sparse_mla_splits(T, topk);
    a.per = ((topk + a.nsplit - 1) / a.nsplit + kTile - 1) / kTile * kTile;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.o = o;
    a.lse = lse;
    a.part_o = ws;
    a.part_ml = ws ? ws + (size_t)a.nsplit * (size_t)T * kMlaHeads * kV : nullptr;
    hipLaunchKernelGGL(sparse_mla_kernel, dim3(a.nsplit, (unsigned)T), dim3(kMlaThreads), smem, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    hipLaunchKernelGGL(sparse_mla_merge_kernel, dim3((unsigned)((T * kMlaHeads + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
