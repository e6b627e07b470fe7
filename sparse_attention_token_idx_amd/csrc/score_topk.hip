// Fused causal indexer scores + streaming top-k for prefill (dense and varlen).
//
// Computes, for every query row t of a sequence, I[t,s] = sum_h w[t,h] * ReLU(q[t,h].k[s])
// over its whole causal prefix s <= t and keeps the topk largest (ties -> lower s), as
// fixed on the "Qwen3.5-397B-A17B vs Kimi K3.1 Pro" compare page (component table,
// sparse/compressed-attention row) with the whole prefix scored (long-context row of the
// "Kimi K3.1 Pro vs Gemma 4" page).  The T x T score matrix never reaches memory.
//
// One workgroup (8 waves) owns 32 query rows and streams the keys of their prefix in
// tiles of 64:
//   * wave (qg, hg) keeps the bf16 q of 16 queries x 8 heads in registers (B operand) and
//     runs q.k for each head on v_mfma_f32_16x16x32_bf16 with the key tile (A operand, read
//     from LDS), then applies ReLU and the w-weighted sum over its 8 heads in registers;
//   * the four head groups' partial sums meet in LDS and are added in a fixed order;
//   * each wave then owns 4 rows: keys above the row's running threshold are appended,
//     in ascending s, to the row's candidate list in the workspace.  When a list nears its
//     capacity the owning wave runs an exact radix select over it, keeps exactly topk
//     entries (stable) and raises the threshold to the topk-th key.  Later keys have
//     larger s and so lose every tie against kept entries, hence the strict ">" rule is
//     exact.
//   * at the end each row's list is selected once more and written out in ascending s.
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

constexpr int kBQ = 32;               // query rows per workgroup
constexpr int kBK = 64;               // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKStride = kDim + 8;    // bf16 per key row in LDS (272 B: conflict-free reads)
constexpr int kRStride = kBK + 4;     // floats per row of the partial-score tile (272 B)

struct ScoreSmem {
    uint16_t k[2][kBK][kKStride];      // double-buffered key tile
    float red[4][kBQ][kRStride];       // per head-group partial scores [hg][query][key]
    uint32_t hist[kWaves][4][256];     // radix-select histograms, 4 copies per wave
};

struct ScoreArgs {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *w;
    const int32_t *cu_seqlens;  // nullptr: one sequence of length T
    int64_t T;
    int nrb;                    // grid.y: row blocks of the longest sequence
    int topk;
    int cap;                    // candidate slots per row
    uint32_t *cand_key;
    int32_t *cand_idx;
    int32_t *out_idx;
    float *out_score;           // may be nullptr
};

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Exact selection over one candidate list, run by one whole wave.
// keys/ids[0..n) hold (orderable score key, token index) in ascending index order, n > topk.
// Finds theta = the topk-th largest key, then compacts the list in place (stable) to the
// topk entries that win under (key desc, index asc): every key > theta plus the first
// topk - #(key > theta) entries equal to theta.  Returns theta.
__device__ uint32_t wave_select(uint32_t *keys, int32_t *ids, int n, int topk, uint32_t *hist) {
    const int lane = lane_id();
    uint32_t prefix = 0, pmask = 0;
    int need = topk;
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int i = 0; i < 16; ++i) hist[lane + 64 * i] = 0u;
        wave_sync_lds();
        uint32_t *h = hist + 256 * (lane & 3);
        for (int i = lane; i < n; i += 64) {
            const uint32_t kv = keys[i];
            if ((kv & pmask) == prefix) atomicAdd(&h[(kv >> shift) & 255u], 1u);
        }
        wave_sync_lds();
        int c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 4 * lane + j;
            c[j] = (int)(hist[b] + hist[256 + b] + hist[512 + b] + hist[768 + b]);
        }
        const int s = c[0] + c[1] + c[2] + c[3];
        const int incl = wave_inclusive_sum(s);
        const int total = readlane(incl, 63);
        int above = total - incl;   // entries in bins above 4*lane+3
        int found = -1, found_above = 0;
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            if (found < 0 && above < need && need <= above + c[j]) {
                found = 4 * lane + j;
                found_above = above;
            }
            above += c[j];
        }
        const uint64_t bm = ballot(found >= 0);
        const int src = (int)__builtin_ctzll(bm);
        const int d = readlane(found, src);
        need -= readlane(found_above, src);
        prefix |= (uint32_t)d << shift;
        pmask |= 255u << shift;
        wave_sync_lds();
    }
    // stable in-place compaction: each chunk is read before any of its slots is written,
    // and writes never reach beyond the chunk being read
    const uint32_t theta = prefix;
    int out = 0, ties = 0;
    for (int base = 0; base < n; base += 64) {
        const int i = base + lane;
        const bool in = i < n;
        const uint32_t kv = in ? keys[i] : 0u;
        const int32_t iv = in ? ids[i] : 0;
        const bool gt = in && kv > theta;
        const bool eq = in && kv == theta;
        const uint64_t em = ballot(eq);
        const bool keep = gt || (eq && ties + (int)bits_below(em) < need);
        const uint64_t km = ballot(keep);
        if (keep) {
            const int pos = out + (int)bits_below(km);
            keys[pos] = kv;
            ids[pos] = iv;
        }
        out += __popcll(km);
        ties += __popcll(em);
    }
    __threadfence();
    return theta;
}

__global__ __launch_bounds__(kThreads, 1) void score_topk_kernel(ScoreArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ScoreSmem &sm = *reinterpret_cast<ScoreSmem *>(smem_raw);

    const int seq = blockIdx.x;
    const int rb = a.nrb - 1 - (int)blockIdx.y;   // longest rows first
    int64_t seq_start = 0, L = a.T;
    if (a.cu_seqlens) {
        seq_start = a.cu_seqlens[seq];
        L = (int64_t)a.cu_seqlens[seq + 1] - seq_start;
    }
    const int64_t r0 = (int64_t)rb * kBQ;
    if (r0 >= L) return;
    const int rows_here = (int)(L - r0 < kBQ ? L - r0 : kBQ);
    const int64_t r_last = r0 + rows_here - 1;
    const int nkt = (int)(r_last / kBK) + 1;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int qg = wave & 1, hg = wave >> 1;
    const int l16 = lane & 15, lg = lane >> 4;

    // ---- q fragments (B operand) and head weights for 16 queries x 8 heads
    u32x4 qf[8][4];
    float wv[8];
    {
        const int row = 16 * qg + l16;
        const bool ok = row < rows_here;
        const int64_t g = seq_start + r0 + (ok ? row : 0);
        const uint16_t *qrow = a.q + g * kQOut + (8 * hg) * kDim + 8 * lg;
#pragma unroll
        for (int h = 0; h < 8; ++h) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qf[h][ks] = ok ? *reinterpret_cast<const u32x4 *>(qrow + h * kDim + 32 * ks)
                               : u32x4{0u, 0u, 0u, 0u};
            wv[h] = ok ? bf16_to_f32(a.w[g * kHeads + 8 * hg + h]) : 0.f;
        }
    }

    // ---- key tile staging: thread -> key tid/8, 32 bytes at dim 16*(tid%8)
    const int st_key = tid >> 3, st_dim = 16 * (tid & 7);
    u32x4 kv0, kv1;
    auto load_k = [&](int kt) {
        const int64_t s = (int64_t)kt * kBK + st_key;
        if (s < L) {
            const uint16_t *p = a.k + (seq_start + s) * kDim + st_dim;
            kv0 = *reinterpret_cast<const u32x4 *>(p);
            kv1 = *reinterpret_cast<const u32x4 *>(p + 8);
        } else {
            kv0 = u32x4{0u, 0u, 0u, 0u};
            kv1 = kv0;
        }
    };
    auto store_k = [&](int buf) {
        uint16_t *p = &sm.k[buf][st_key][st_dim];
        *reinterpret_cast<u32x4 *>(p) = kv0;
        *reinterpret_cast<u32x4 *>(p + 8) = kv1;
    };

    // ---- row state for the 4 rows this wave emits (row 4*wave + lg, uniform per 16 lanes)
    const int er = 4 * wave + lg;
    const bool erow_ok = er < rows_here;
    const int64_t et = r0 + er;                          // its position in the sequence
    const int64_t egrow = seq_start + r0 + (erow_ok ? er : 0);
    uint32_t *ck = a.cand_key + egrow * a.cap;
    int32_t *ci = a.cand_idx + egrow * a.cap;
    uint32_t theta = 0u;   // emit key > theta; 0 is below every finite score's key
    int n = 0;
    uint32_t *whist = &sm.hist[wave][0][0];
    const uint64_t gmask = 0xFFFFull << (16 * lg);
    const int64_t wave_last_row = r0 + 16 * qg + 15;

    load_k(0);
    store_k(0);
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < nkt;
        if (more) load_k(kt + 1);

        f32x4 acc[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            acc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
            if ((int64_t)kt * kBK + 16 * st <= wave_last_row) {
                u32x4 af[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    af[ks] = *reinterpret_cast<const u32x4 *>(&sm.k[buf][16 * st + l16][32 * ks + 8 * lg]);
#pragma unroll
                for (int h = 0; h < 8; ++h) {
                    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) s = mfma16x16x32(af[ks], qf[h][ks], s);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[st][r] = fmaf(wv[h], fmaxf(s[r], 0.f), acc[st][r]);
                }
            }
        }
#pragma unroll
        for (int st = 0; st < 4; ++st)
            *reinterpret_cast<f32x4 *>(&sm.red[hg][16 * qg + l16][16 * st + 4 * lg]) = acc[st];
        if (more) store_k(buf ^ 1);
        __syncthreads();

        // ---- emission: this lane covers keys 4*l16 .. 4*l16+3 of the tile for row er
        {
            f32x4 v = *reinterpret_cast<const f32x4 *>(&sm.red[0][er][4 * l16]);
#pragma unroll
            for (int g = 1; g < 4; ++g) v += *reinterpret_cast<const f32x4 *>(&sm.red[g][er][4 * l16]);
            const int64_t s0 = (int64_t)kt * kBK + 4 * l16;
            uint32_t kk[4];
            bool e[4];
            int before = 0, total = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kk[j] = score_key(v[j]);
                e[j] = erow_ok && (s0 + j <= et) && (kk[j] > theta);
                const uint64_t b = ballot(e[j]) & gmask;
                before += (int)bits_below(b);
                total += __popcll(b);
            }
            int pos = n + before;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (e[j]) {
                    ck[pos] = kk[j];
                    ci[pos] = (int32_t)(s0 + j);
                    ++pos;
                }
            }
            n += total;
        }
        // ---- compaction of rows whose list could overflow on the next tile
        {
            const uint64_t full = ballot(n > a.cap - kBK);
            if (full) {
#pragma unroll 1
                for (int g = 0; g < 4; ++g) {
                    if (!((full >> (16 * g)) & 1ull)) continue;
                    const int row = 4 * wave + g;
                    const int64_t grow = seq_start + r0 + row;
                    const int ng = readlane(n, 16 * g);
                    __threadfence();
                    const uint32_t th = wave_select(a.cand_key + grow * a.cap,
                                                    a.cand_idx + grow * a.cap, ng, a.topk, whist);
                    if (lg == g) {
                        theta = th;
                        n = a.topk;
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- final selection and output, one row at a time per wave
    __threadfence();
#pragma unroll 1
    for (int g = 0; g < 4; ++g) {
        const int row = 4 * wave + g;
        if (row >= rows_here) break;
        const int64_t grow = seq_start + r0 + row;
        int ng = readlane(n, 16 * g);
        uint32_t *rk = a.cand_key + grow * a.cap;
        int32_t *ri = a.cand_idx + grow * a.cap;
        if (ng > a.topk) {
            wave_select(rk, ri, ng, a.topk, whist);
            ng = a.topk;
        }
        int32_t *oi = a.out_idx + grow * a.topk;
        float *os = a.out_score ? a.out_score + grow * a.topk : nullptr;
        for (int i = lane; i < a.topk; i += 64) {
            const bool in = i < ng;
            oi[i] = in ? ri[i] : -1;
            if (os) os[i] = in ? key_score(rk[i]) : -INFINITY;
        }
    }
}

}  // namespace

int candidate_capacity(int topk) {
    // room for topk survivors plus at least topk fresh emissions and one tile of slack
    return ((2 * topk + kBK - 1) / kBK) * kBK + kBK;
}

hipError_t launch_score_topk(const uint16_t *q, const uint16_t *k, const uint16_t *w,
                             const int32_t *cu_seqlens, int B, int64_t max_len, int64_t T,
                             int topk, int cap, uint32_t *cand_key, int32_t *cand_idx,
                             int32_t *idx, float *scores, hipStream_t stream) {
    static bool attr_done = false;
    const size_t smem = sizeof(ScoreSmem);
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(score_topk_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    ScoreArgs a;
    a.q = q;
    a.k = k;
    a.w = w;
    a.cu_seqlens = cu_seqlens;
    a.T = T;
    a.nrb = (int)((max_len + kBQ - 1) / kBQ);
    a.topk = topk;
    a.cap = cap;
    a.cand_key = cand_key;
    a.cand_idx = cand_idx;
    a.out_idx = idx;
    a.out_score = scores;
    if (a.nrb == 0 || B == 0) return hipSuccess;
    hipLaunchKernelGGL(score_topk_kernel, dim3(B, a.nrb), dim3(kThreads), smem, stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
