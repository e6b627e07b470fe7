// Indexer projections: q = c_q W_q (1,536 -> 4,096), k = LayerNorm(x W_k) (7,168 -> 128),
// w = x W_w (7,168 -> 32), as listed for the Kimi K3.1 Pro indexer on the
// "Qwen3.5-397B-A17B vs Kimi K3.1 Pro" compare page (sparse/compressed-attention row; the
// LayerNorm on the key is the QK-norm row).  bf16 in, fp32 accumulation on
// v_mfma_f32_16x16x32_bf16, bf16 (round to nearest even) out.
//
// One tiled GEMM serves both products.  The weights arrive [K][N] (N contiguous) while the
// MFMA wants 8 consecutive k per lane for both operands, so each B tile is transposed on
// its way into LDS: a thread loads an 8(k) x 8(n) block with 16-byte loads, transposes it
// in registers and writes 8 k-contiguous 16-byte chunks.  Both LDS tiles are stored as
// 128-byte rows of eight 16-byte chunks, chunk c of row r at slot c ^ (r & 7), which keeps
// the 16-byte MFMA operand reads and the transposed writes free of bank conflicts.
// The k/w product (N = 160) keeps whole rows in one wave, so the LayerNorm over the 128
// key columns runs in the epilogue on the fp32 accumulators before rounding.
//
// A handful of tokens (a decode step: T <= kSkinnyT) would give the tiled GEMM a handful
// of workgroups, each streaming whole weight matrices.  There the work is tiny and the
// weights are the bytes that matter, so K is split over many workgroups instead: each one
// runs the same tiled core on one 64-row tile and its K-slice and writes fp32 partial sums
// to the workspace; a second kernel adds the slices in order (deterministic), then
// rounds, with the LayerNorm for k.
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

constexpr int kBK = 64;  // k per LDS tile (8 chunks of 8)

__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + 8 * (chunk ^ (row & 7)); }

template <int BM, int BN>
struct GemmSmem {
    uint16_t a[2][BM * kBK];
    uint16_t b[2][BN * kBK];
};

// C tile = A[m0:m0+BM, :] x B[:, n0:n0+BN]; wave (wm, wn) of a WM x WN grid owns a
// (BM/WM) x (BN/WN) sub-tile as SM x SN MFMA tiles of 16 x 16.
template <int BM, int BN, int WM, int WN>
struct GemmCore {
    static constexpr int SM = BM / WM / 16;
    static constexpr int SN = BN / WN / 16;
    static constexpr int A_CHUNKS = BM * 8 / 256;   // 16-byte A chunks per thread per tile

    // Columns n < nsplit of B come from B0 ([K][ld0]), the others from B1 ([K][ld1], column
    // n - nsplit).
    __device__ static void run(const uint16_t *__restrict__ A, int64_t lda, int64_t M, int64_t m0,
                               const uint16_t *__restrict__ B0, int ld0, const uint16_t *__restrict__ B1,
                               int ld1, int nsplit, int n0, int K, GemmSmem<BM, BN> &sm,
                               f32x4 (&acc)[SM][SN]) {
        const int tid = threadIdx.x;
        const int wave = tid >> 6, lane = tid & 63;
        const int wm = wave / WN, wn = wave % WN;
        const int l16 = lane & 15, lg = lane >> 4;
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        u32x4 ra[A_CHUNKS];
        u32x4 rb[8];
        const bool b_thread = tid < BN;
        const int bkb = tid & 7, bnb = tid >> 3;   // B block: k rows 8*bkb.., n cols 8*bnb..
        const int bn = n0 + 8 * bnb;
        const uint16_t *bsrc = bn < nsplit ? B0 + bn : B1 + (bn - nsplit);
        const int ldb = bn < nsplit ? ld0 : ld1;
        auto load = [&](int kt) {
            const int k0 = kt * kBK;
#pragma unroll
            for (int i = 0; i < A_CHUNKS; ++i) {
                const int c = tid + 256 * i;
                const int row = c >> 3, kc = c & 7;
                const int64_t gm = m0 + row;
                ra[i] = gm < M ? *reinterpret_cast<const u32x4 *>(A + gm * lda + k0 + 8 * kc)
                               : u32x4{0u, 0u, 0u, 0u};
            }
            if (b_thread) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    rb[i] = *reinterpret_cast<const u32x4 *>(bsrc + (int64_t)(k0 + 8 * bkb + i) * ldb);
            }
        };
        auto store = [&](int buf) {
#pragma unroll
            for (int i = 0; i < A_CHUNKS; ++i) {
                const int c = tid + 256 * i;
                *reinterpret_cast<u32x4 *>(&sm.a[buf][swz(c >> 3, c & 7)]) = ra[i];
            }
            if (b_thread) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    // column j of the 8x8 block: element i = row i's bf16 j
                    const int sh = 16 * (j & 1), dw = j >> 1;
                    u32x4 o;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const uint32_t lo = (rb[2 * m][dw] >> sh) & 0xFFFFu;
                        const uint32_t hi = (rb[2 * m + 1][dw] >> sh) & 0xFFFFu;
                        o[m] = lo | (hi << 16);
                    }
                    *reinterpret_cast<u32x4 *>(&sm.b[buf][swz(8 * bnb + j, bkb)]) = o;
                }
            }
        };

        const int nk = K / kBK;
        load(0);
        store(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int buf = kt & 1;
            if (kt + 1 < nk) load(kt + 1);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int kc = 4 * ks + lg;
                u32x4 af[SM], bf[SN];
#pragma unroll
                for (int i = 0; i < SM; ++i)
                    af[i] = *reinterpret_cast<const u32x4 *>(&sm.a[buf][swz(wm * (BM / WM) + 16 * i + l16, kc)]);
#pragma unroll
                for (int j = 0; j < SN; ++j)
                    bf[j] = *reinterpret_cast<const u32x4 *>(&sm.b[buf][swz(wn * (BN / WN) + 16 * j + l16, kc)]);
#pragma unroll
                for (int i = 0; i < SM; ++i)
#pragma unroll
                    for (int j = 0; j < SN; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
            }
            if (kt + 1 < nk) store(buf ^ 1);
            __syncthreads();
        }
    }
};

// ---------------------------------------------------------------- q for many tokens
// q = bf16(c_q . W_q) with W_q first transposed into the workspace (W_qT [4096][1536], a
// few microseconds), so that both operands are k-contiguous and every tile can be copied
// from global memory into LDS by the direct global->LDS loads (16 bytes per lane, no
// registers, no VALU transpose).  256 x 256 block tiles, 4 waves of 128 x 128 (the 64
// accumulator tiles live in AGPRs), K-steps of 32 through a ring of kQStages LDS stages
// refilled kQStages steps ahead; the next step's MFMA fragments are read while the current
// step's MFMAs run.  One wave instruction fills 1 KB = 16 rows of 64 bytes, so each MFMA
// fragment read is one contiguous 1 KB (no bank conflicts, no swizzle).
typedef __attribute__((address_space(3))) void lds_void;
constexpr int kQBM = 256, kQBN = 256, kQKB = 32, kQStages = 3;
constexpr int kQStage = (kQBM + kQBN) * kQKB;   // bf16 per stage

// W_qT[n][k] = W_q[k][n], 64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void transpose_wq_kernel(const uint16_t *__restrict__ Wq, int64_t ldw,
                                                           uint16_t *__restrict__ WqT) {
    __shared__ uint16_t t[64][72];
    const int n0 = 64 * blockIdx.x, k0 = 64 * blockIdx.y;
    const int r = threadIdx.x >> 2, c = 16 * (threadIdx.x & 3);
    const u32x4 v0 = *reinterpret_cast<const u32x4 *>(Wq + (int64_t)(k0 + r) * ldw + n0 + c);
    const u32x4 v1 = *reinterpret_cast<const u32x4 *>(Wq + (int64_t)(k0 + r) * ldw + n0 + c + 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        t[r][c + 2 * j] = (uint16_t)(v0[j] & 0xFFFFu);
        t[r][c + 2 * j + 1] = (uint16_t)(v0[j] >> 16);
        t[r][c + 8 + 2 * j] = (uint16_t)(v1[j] & 0xFFFFu);
        t[r][c + 8 + 2 * j + 1] = (uint16_t)(v1[j] >> 16);
    }
    __syncthreads();
    u32x4 o0, o1;   // row n0 + r of W_qT, k = k0 + c .. k0 + c + 15
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o0[j] = (uint32_t)t[c + 2 * j][r] | ((uint32_t)t[c + 2 * j + 1][r] << 16);
        o1[j] = (uint32_t)t[c + 8 + 2 * j][r] | ((uint32_t)t[c + 8 + 2 * j + 1][r] << 16);
    }
    *reinterpret_cast<u32x4 *>(WqT + (int64_t)(n0 + r) * kQLat + k0 + c) = o0;
    *reinterpret_cast<u32x4 *>(WqT + (int64_t)(n0 + r) * kQLat + k0 + c + 8) = o1;
}

__global__ __launch_bounds__(256, 1) void proj_q_kernel(const uint16_t *__restrict__ cq, int64_t ldc,
                                                        int64_t T, const uint16_t *__restrict__ WqT,
                                                        uint16_t *__restrict__ q, int64_t ldq) {
    constexpr int SM = 8, SN = 8, S = kQStages, KB = kQKB;
    extern __shared__ __align__(16) uint16_t qsm[];
    const int ntn = kQOut / kQBN;
    const int64_t m0 = (int64_t)(blockIdx.x / ntn) * kQBM;
    const int n0 = (blockIdx.x % ntn) * kQBN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1, l16 = lane & 15, lg = lane >> 4;
    f32x4 acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // stage of K-step kt: A rows 0..255 then B rows 0..255, 32 bf16 each; wave w fills rows
    // 64w .. 64w+63 of both, 8 load instructions per wave (rows past T repeat row T - 1)
    auto issue = [&](int kt) {
        uint16_t *st = qsm + (kt % S) * kQStage;
        const int k0 = kt * KB;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 64 * wave + 16 * i + (lane >> 2);
            const int kc = 8 * (lane & 3);
            const int64_t ga = m0 + row < T ? m0 + row : T - 1;
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(cq + ga * ldc + k0 + kc),
                                             (lds_void *)(st + (64 * wave + 16 * i) * KB), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(WqT + (int64_t)(n0 + row) * kQLat + k0 + kc),
                                             (lds_void *)(st + kQBM * KB + (64 * wave + 16 * i) * KB),
                                             16, 0, 0);
        }
    };
    // Until this wave's loads of stage kt are done (8 per later stage may stay in flight),
    // then this wave's fragment reads of older stages (before anyone refills them), then a
    // barrier without the fence of __syncthreads (which would wait for every load in flight).
    const int nk = kQLat / KB;
    auto wait_stage = [&](int kt) {
        const int later = min(S - 2, nk - 1 - kt);
        if (later >= 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else if (later == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    u32x4 fa[2][SM], fb[2][SN];
    auto read_frags = [&](int kt, int p) {
        const uint16_t *st = qsm + (kt % S) * kQStage;
#pragma unroll
        for (int i = 0; i < SM; ++i)
            fa[p][i] = *reinterpret_cast<const u32x4 *>(st + (wm * 128 + 16 * i + l16) * KB + 8 * lg);
#pragma unroll
        for (int j = 0; j < SN; ++j)
            fb[p][j] = *reinterpret_cast<const u32x4 *>(st + kQBM * KB + (wn * 128 + 16 * j + l16) * KB + 8 * lg);
    };
    // the ring holds S stages; step k refills the slot of stage k, already in registers
#pragma unroll
    for (int p = 0; p < S; ++p)
        if (p < nk) issue(p);
    wait_stage(0);
    read_frags(0, 0);
    for (int kt = 0; kt < nk; kt += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {   // fragments of step kt + h in register set h
            const int k = kt + h;
            if (k < nk) {
                if (k + 1 < nk) {
                    wait_stage(k + 1);
                    if (k + S < nk) issue(k + S);
                    read_frags(k + 1, h ^ 1);
                }
#pragma unroll
                for (int i = 0; i < SM; ++i)
#pragma unroll
                    for (int j = 0; j < SN; ++j) acc[i][j] = mfma16x16x32(fa[h][i], fb[h][j], acc[i][j]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wm * 128 + 16 * i + 4 * lg + r;
            if (row >= T) continue;
#pragma unroll
            for (int j = 0; j < SN; ++j)
                q[row * ldq + n0 + wn * 128 + 16 * j + l16] = (uint16_t)f32_to_bf16(acc[i][j][r]);
        }
}

static_assert(kQLat % (2 * kQKB) == 0 && kQOut % kQBN == 0, "q tiles");

// [k | w] = x . [W_k | W_w] (N = 128 + 32), LayerNorm on the k part: 128-row tiles, each
// of the 4 waves owns 32 full rows.  The two weight matrices are read as one [7168][160]
// operand whose first 16 column-chunks come from W_k and the last 4 from W_w.
struct KWArgs {
    const uint16_t *x;
    int64_t ldx;
    int64_t T;
    const uint16_t *Wk;
    const uint16_t *Ww;
    const uint16_t *gamma;
    const uint16_t *beta;
    float eps;
    uint16_t *k_base;           // nullptr: compute no key
    const int64_t *k_slot;
    uint16_t *w;
    int64_t ldww;               // row stride of W_w (elements)
    int64_t ldwo;               // row stride of w
};

__global__ __launch_bounds__(256) void proj_kw_kernel(KWArgs a) {
    constexpr int BM = 128, BN = 160, SM = 2, SN = 10;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    auto &sm = *reinterpret_cast<GemmSmem<BM, BN> *>(smem_raw);
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, lg = lane >> 4;

    f32x4 acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int A_CHUNKS = BM * 8 / 256;
    u32x4 ra[A_CHUNKS];
    u32x4 rb[8];
    const bool b_thread = tid < BN;
    const int bkb = tid & 7, bnb = tid >> 3;   // bnb in 0..19: 0..15 -> W_k, 16..19 -> W_w
    auto load = [&](int kt) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 3, kc = c & 7;
            const int64_t gm = m0 + row;
            ra[i] = gm < a.T ? *reinterpret_cast<const u32x4 *>(a.x + gm * a.ldx + k0 + 8 * kc)
                             : u32x4{0u, 0u, 0u, 0u};
        }
        if (b_thread) {
            const uint16_t *src = bnb < 16 ? a.Wk + 8 * bnb : a.Ww + 8 * (bnb - 16);
            const int ld = bnb < 16 ? kDim : (int)a.ldww;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                rb[i] = *reinterpret_cast<const u32x4 *>(src + (int64_t)(k0 + 8 * bkb + i) * ld);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = tid + 256 * i;
            *reinterpret_cast<u32x4 *>(&sm.a[buf][swz(c >> 3, c & 7)]) = ra[i];
        }
        if (b_thread) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int sh = 16 * (j & 1), dw = j >> 1;
                u32x4 o;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint32_t lo = (rb[2 * m][dw] >> sh) & 0xFFFFu;
                    const uint32_t hi = (rb[2 * m + 1][dw] >> sh) & 0xFFFFu;
                    o[m] = lo | (hi << 16);
                }
                *reinterpret_cast<u32x4 *>(&sm.b[buf][swz(8 * bnb + j, bkb)]) = o;
            }
        }
    };

    const int nk = kHidden / kBK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load(kt + 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int kc = 4 * ks + lg;
            u32x4 af[SM], bf[SN];
#pragma unroll
            for (int i = 0; i < SM; ++i)
                af[i] = *reinterpret_cast<const u32x4 *>(&sm.a[buf][swz(wave * 32 + 16 * i + l16, kc)]);
#pragma unroll
            for (int j = 0; j < SN; ++j)
                bf[j] = *reinterpret_cast<const u32x4 *>(&sm.b[buf][swz(16 * j + l16, kc)]);
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
        }
        if (kt + 1 < nk) store(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: LayerNorm over the 128 key columns (mean-centred, biased variance)
    float g[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        g[j] = bf16_to_f32(a.gamma[16 * j + l16]);
        b[j] = bf16_to_f32(a.beta[16 * j + l16]);
    }
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wave * 32 + 16 * i + 4 * lg + r;
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) s += acc[i][j][r];
#pragma unroll
            for (int d = 1; d < 16; d <<= 1) s += __shfl_xor(s, d, 64);
            const float mu = s * (1.0f / kDim);
            float v = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float c = acc[i][j][r] - mu;
                v = fmaf(c, c, v);
            }
#pragma unroll
            for (int d = 1; d < 16; d <<= 1) v += __shfl_xor(v, d, 64);
            const float inv = 1.0f / sqrtf(v * (1.0f / kDim) + a.eps);
            if (row >= a.T) continue;
            if (a.k_base) {
                const int64_t slot = a.k_slot ? a.k_slot[row] : row;
                uint16_t *kr = a.k_base + slot * kDim;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    kr[16 * j + l16] = (uint16_t)f32_to_bf16(fmaf((acc[i][j][r] - mu) * inv, g[j], b[j]));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
                a.w[row * a.ldwo + 16 * j + l16] = (uint16_t)f32_to_bf16(acc[i][8 + j][r]);
        }
}

// ---------------------------------------------------------------- small T (split K)
// part[s][t][n] for one 64-row tile (all T <= 64 rows) and one BN-column tile n0 = BN x:
// the product of A[:, k0:k0+KS] and B[k0:k0+KS, n0:n0+BN], k0 = KS s, on the tiled core.
template <int BN, int WM, int WN, int KS>
__global__ __launch_bounds__(256) void skinny_partial_kernel(const uint16_t *__restrict__ A, int64_t lda,
                                                             int T, const uint16_t *__restrict__ B0, int ld0,
                                                             const uint16_t *__restrict__ B1, int ld1,
                                                             int nsplit, int N, float *__restrict__ part) {
    using Core = GemmCore<64, BN, WM, WN>;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    auto &sm = *reinterpret_cast<GemmSmem<64, BN> *>(smem_raw);
    const int n0 = BN * blockIdx.x;
    const int s = blockIdx.y;
    const int k0 = KS * s;
    f32x4 acc[Core::SM][Core::SN];
    Core::run(A + k0, lda, T, 0, B0 + (int64_t)k0 * ld0, ld0, B1 + (int64_t)k0 * ld1, ld1, nsplit, n0, KS,
              sm, acc);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave / WN, wn = wave % WN;
    const int l16 = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int i = 0; i < Core::SM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wm * (64 / WM) + 16 * i + 4 * lg + r;
            if (row >= T) continue;
            float *pr = part + ((int64_t)s * T + row) * N + n0 + wn * (BN / WN) + l16;
#pragma unroll
            for (int j = 0; j < Core::SN; ++j) pr[16 * j] = acc[i][j][r];
        }
}

// q[t][n] = bf16(sum over the S slices of part[s][t][n]), q rows ldq apart; thread: 4
// consecutive n.
__global__ __launch_bounds__(256) void skinny_reduce_q_kernel(const float *__restrict__ part, int S, int T,
                                                              uint16_t *__restrict__ q, int64_t ldq) {
    const int64_t e = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
    if (e >= (int64_t)T * kQOut) return;
    f32x4 v = *reinterpret_cast<const f32x4 *>(part + e);
    for (int s = 1; s < S; ++s) {
        const f32x4 p = *reinterpret_cast<const f32x4 *>(part + (int64_t)s * T * kQOut + e);
        v = f32x4{v[0] + p[0], v[1] + p[1], v[2] + p[2], v[3] + p[3]};
    }
    const int64_t t = e / kQOut, n = e % kQOut;
    *reinterpret_cast<u32x2 *>(q + t * ldq + n) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// One workgroup per token: wave j adds the slices s = j, j + 4, ... of the 160 columns of
// [k | w] (lane: columns lane, 64 + lane, and 128 + lane for lane < 32); the four wave sums
// are added in a fixed order, then wave 0 applies the LayerNorm over the 128 key columns
// (as in the tiled kernel's epilogue), rounds to bf16 and writes k to its slot.
__global__ __launch_bounds__(256) void skinny_reduce_kw_kernel(const float *__restrict__ part, int S, KWArgs a) {
    constexpr int N = kDim + kHeads;
    __shared__ float red[4][3][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = blockIdx.x;
    const int64_t ss = (int64_t)a.T * N;  // slice stride
    const float *p = part + t * N;
    float v0 = 0.f, v1 = 0.f, vw = 0.f;
#pragma unroll 4
    for (int s = wave; s < S; s += 4) {
        v0 += p[s * ss + lane];
        v1 += p[s * ss + 64 + lane];
        vw += lane < kHeads ? p[s * ss + kDim + lane] : 0.f;
    }
    red[wave][0][lane] = v0;
    red[wave][1][lane] = v1;
    red[wave][2][lane] = vw;
    __syncthreads();
    if (wave) return;
    v0 = ((red[0][0][lane] + red[1][0][lane]) + red[2][0][lane]) + red[3][0][lane];
    v1 = ((red[0][1][lane] + red[1][1][lane]) + red[2][1][lane]) + red[3][1][lane];
    vw = ((red[0][2][lane] + red[1][2][lane]) + red[2][2][lane]) + red[3][2][lane];
    float sum = v0 + v1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) sum += __shfl_xor(sum, d, 64);
    const float mu = sum * (1.0f / kDim);
    const float c0 = v0 - mu, c1 = v1 - mu;
    float var = fmaf(c0, c0, c1 * c1);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) var += __shfl_xor(var, d, 64);
    const float inv = 1.0f / sqrtf(var * (1.0f / kDim) + a.eps);
    if (a.k_base) {
        const int64_t slot = a.k_slot ? a.k_slot[t] : t;
        uint16_t *kr = a.k_base + slot * kDim;
        kr[lane] = (uint16_t)f32_to_bf16(fmaf(c0 * inv, bf16_to_f32(a.gamma[lane]), bf16_to_f32(a.beta[lane])));
        kr[64 + lane] = (uint16_t)f32_to_bf16(fmaf(c1 * inv, bf16_to_f32(a.gamma[64 + lane]), bf16_to_f32(a.beta[64 + lane])));
    }
    if (lane < kHeads) a.w[t * a.ldwo + lane] = (uint16_t)f32_to_bf16(vw);
}

constexpr int kSkQSlice = 256;    // q: K = 1,536 in 6 slices x 32 column tiles
constexpr int kSkKWSlice = 128;   // k/w: K = 7,168 in 56 slices

}  // namespace

size_t project_workspace(int64_t T) {
    if (T <= 0) return 0;
    if (T > kSkinnyT) return (size_t)kQOut * kQLat * 2;   // W_q transposed
    return 4u * (size_t)T * ((size_t)(kQLat / kSkQSlice) * kQOut + (size_t)(kHidden / kSkKWSlice) * (kDim + kHeads));
}

hipError_t launch_project(const uint16_t *x, int64_t ldx, const uint16_t *c_q, int64_t ldc,
                          int64_t T, const uint16_t *W_q, const uint16_t *W_k,
                          const uint16_t *W_w, const uint16_t *gamma, const uint16_t *beta,
                          float eps, uint16_t *q, uint16_t *k_base, const int64_t *k_slot,
                          uint16_t *w, float *ws, hipStream_t stream) {
    return launch_project_ex(x, ldx, c_q, ldc, T, W_q, kQOut, W_k, W_w, kHeads, gamma, beta, eps, q, kQOut,
                             k_base, k_slot, w, kHeads, ws, stream);
}

hipError_t launch_project_ex(const uint16_t *x, int64_t ldx, const uint16_t *c_q, int64_t ldc,
                             int64_t T, const uint16_t *W_q, int64_t ldwq, const uint16_t *W_k,
                             const uint16_t *W_w, int64_t ldww, const uint16_t *gamma,
                             const uint16_t *beta, float eps, uint16_t *q, int64_t ldq,
                             uint16_t *k_base, const int64_t *k_slot, uint16_t *w, int64_t ldwo,
                             float *ws, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    if (T <= kSkinnyT) {
        const int t = (int)T;
        float *part_q = ws;
        float *part_kw = ws + (size_t)(kQLat / kSkQSlice) * T * kQOut;
        static DeviceOnce sk_attr;
        hipError_t ea = sk_attr.run([] {
            hipError_t e = hipFuncSetAttribute(
                reinterpret_cast<const void *>(skinny_partial_kernel<128, 1, 4, kSkQSlice>),
                hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(GemmSmem<64, 128>));
            if (e != hipSuccess) return e;
            return hipFuncSetAttribute(reinterpret_cast<const void *>(skinny_partial_kernel<160, 2, 2, kSkKWSlice>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(GemmSmem<64, 160>));
        });
        if (ea != hipSuccess) return ea;
        if (q) {
            hipLaunchKernelGGL((skinny_partial_kernel<128, 1, 4, kSkQSlice>), dim3(kQOut / 128, kQLat / kSkQSlice),
                               dim3(256), sizeof(GemmSmem<64, 128>), stream, c_q, ldc, t, W_q, (int)ldwq, W_q,
                               (int)ldwq, kQOut, kQOut, part_q);
            hipLaunchKernelGGL(skinny_reduce_q_kernel, dim3((unsigned)((T * kQOut / 4 + 255) / 256)), dim3(256),
                               0, stream, part_q, kQLat / kSkQSlice, t, q, ldq);
        }
        hipLaunchKernelGGL((skinny_partial_kernel<160, 2, 2, kSkKWSlice>), dim3(1, kHidden / kSkKWSlice), dim3(256),
                           sizeof(GemmSmem<64, 160>), stream, x, ldx, t, W_k, kDim, W_w, (int)ldww, kDim,
                           kDim + kHeads, part_kw);
        KWArgs a{x, ldx, T, W_k, W_w, gamma, beta, eps, k_base, k_slot, w, ldww, ldwo};
        hipLaunchKernelGGL(skinny_reduce_kw_kernel, dim3((unsigned)T), dim3(256), 0, stream, part_kw,
                           kHidden / kSkKWSlice, a);
        return hipGetLastError();
    }
    static DeviceOnce attr;
    const size_t smem_q = sizeof(uint16_t) * kQStage * kQStages;
    const size_t smem_kw = sizeof(GemmSmem<128, 160>);
    hipError_t ea = attr.run([&] {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(proj_q_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem_q);
        if (e != hipSuccess) return e;
        return hipFuncSetAttribute(reinterpret_cast<const void *>(proj_kw_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem_kw);
    });
    if (ea != hipSuccess) return ea;
    const int64_t mt = (T + 127) / 128;
    if (q) {
        uint16_t *WqT = reinterpret_cast<uint16_t *>(ws);
        hipLaunchKernelGGL(transpose_wq_kernel, dim3(kQOut / 64, kQLat / 64), dim3(256), 0, stream, W_q, ldwq,
                           WqT);
        const int64_t qt = (T + kQBM - 1) / kQBM;
        hipLaunchKernelGGL(proj_q_kernel, dim3((unsigned)(qt * (kQOut / kQBN))), dim3(256), smem_q, stream,
                           c_q, ldc, T, WqT, q, ldq);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    KWArgs a{x, ldx, T, W_k, W_w, gamma, beta, eps, k_base, k_slot, w, ldww, ldwo};
    hipLaunchKernelGGL(proj_kw_kernel, dim3((unsigned)mt), dim3(256), smem_kw, stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
