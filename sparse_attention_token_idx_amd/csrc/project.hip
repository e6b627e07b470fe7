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
// The DeepSeek-V3.2-shaped indexer (64 heads: 8,192 q columns and 64 w columns; a rotary step
// on dims 0..63 of every q head and of the key, "Kimi K3.1 Pro vs Gemma 4 31B" page, RoPE row)
// runs through the same kernels in one pass: the rotation is applied in the epilogues to the
// fp32 results (for k after the LayerNorm), with (cos, sin) of every (token, pair) taken from a
// table formed once per call in fp64, and each element is rounded to bf16 once.  Pair (2i, 2i+1)
// sits in two neighbouring lanes of an MFMA result tile, which swap values with one exchange.
//
// A handful of tokens (a decode step: T <= kSkinnyT) would give the tiled GEMM a handful
// of workgroups, each streaming whole weight matrices.  There the work is tiny and the
// weights are the bytes that matter, so K is split over many workgroups instead: each one
// runs the same tiled core on one 64-row tile and its K-slice and writes fp32 partial sums
// to the workspace; a second kernel adds the slices in order (deterministic), then
// rounds, with the LayerNorm for k.  The [k | w] product does the same up to kKwSplitT
// tokens (its 128-row tiles would fill only part of the chip: 64 workgroups at T = 8,192),
// with as many K slices as bring the workgroups to about 1,024.
#include <utility>

#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

constexpr int kBK = 64;  // k per LDS tile (8 chunks of 8)

__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + 8 * (chunk ^ (row & 7)); }

constexpr int kRotPairs = 32;   // rotated pairs per head (dims 0..63)

// The rotation of pair (x, y) by (c, s), for the element this lane holds: x' = x c - y s (even
// dim), y' = x s + y c (odd dim); `other` is the pair's other element.
__device__ __forceinline__ float rotate(float v, float other, float2 cs, bool odd) {
    return odd ? fmaf(other, cs.y, v * cs.x) : fmaf(v, cs.x, -(other * cs.y));
}

// (cos, sin) of angle (pos0 + t) theta^(-2i/64), t < T, i < 32: the angle and its sine and cosine in
// fp64 (positions reach 2^20, where an fp32 angle would be off by tenths of a radian), stored in fp32.
__global__ __launch_bounds__(256) void rope_table_kernel(float2 *tab, int64_t T, int64_t pos0, double theta) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= T * kRotPairs) return;
    const int i = (int)(g % kRotPairs);
    const double ang = (double)(pos0 + g / kRotPairs) * pow(theta, -2.0 * i / (2 * kRotPairs));
    double sn, cs;
    sincos(ang, &sn, &cs);
    tab[g] = make_float2((float)cs, (float)sn);
}

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
// q = bf16(c_q . W_q) with W_q first transposed into the workspace (W_qT [N][1536], a few
// microseconds), so that both operands are k-contiguous and every tile can be copied from
// global memory into LDS by the direct global->LDS loads (16 bytes per lane, no registers, no
// VALU transpose).  256 x 256 block tiles over 8 waves, two per SIMD, each a 128 x 64 quadrant
// (32 accumulator tiles), so that one wave's MFMAs run while the other waits at a barrier or
// for LDS; K-steps of 32 through a ring of kQStages LDS stages refilled kQStages steps ahead;
// the next step's MFMA fragments are read while the current step's MFMAs run.  One wave
// instruction fills 1 KB = 16 rows of 64 bytes, so each MFMA fragment read is one contiguous
// 1 KB (no bank conflicts, no swizzle).
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

struct QArgs {
    const uint16_t *cq;
    int64_t ldc, T;
    const uint16_t *WqT;        // [N][1536]
    int N;                      // q columns: 4,096 or 8,192
    uint16_t *q;
    int64_t ldq;
    const float2 *rope;         // [T][32] (cos, sin), or nullptr: no rotary step
};

// Tile of workgroup `bid`: m-block bid / ntn, n-block bid % ntn.  Workgroup i runs on XCD i mod 8,
// so each XCD only ever needs the ntn / 8 W_qT blocks n = x, x + 8, ... (1.5 or 3 MB, resident in
// its L2 for the whole launch), and the tiles of one m-block that share an XCD run together.
__device__ __forceinline__ bool q_tile(int bid, int64_t qt, int ntn, int64_t &mb, int &nb) {
    mb = bid / ntn;
    nb = bid % ntn;
    return mb < qt;
}

__global__ __launch_bounds__(512, 1) void proj_q_kernel(QArgs a) {
    constexpr int SM = 8, SN = 4, S = kQStages, KB = kQKB;
    extern __shared__ __align__(16) uint16_t qsm[];
    const int ntn = a.N / kQBN;
    int64_t mb;
    int nb;
    if (!q_tile(blockIdx.x, (a.T + kQBM - 1) / kQBM, ntn, mb, nb)) return;
    const int64_t m0 = mb * kQBM, T = a.T;
    const int n0 = nb * kQBN;
    const uint16_t *__restrict__ cq = a.cq;
    const uint16_t *__restrict__ WqT = a.WqT;
    const int64_t ldc = a.ldc;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 2, wn = wave & 3, l16 = lane & 15, lg = lane >> 4;
    f32x4 acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto issue = [&](int kt) {
        uint16_t *st = qsm + (kt % S) * kQStage;
        const int k0 = kt * KB;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = 32 * wave + 16 * i + (lane >> 2);
            const int kc = 8 * (lane & 3);
            const int64_t ga = m0 + row < T ? m0 + row : T - 1;
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(cq + ga * ldc + k0 + kc),
                                             (lds_void *)(st + (32 * wave + 16 * i) * KB), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(WqT + (int64_t)(n0 + row) * kQLat + k0 + kc),
                                             (lds_void *)(st + kQBM * KB + (32 * wave + 16 * i) * KB),
                                             16, 0, 0);
        }
    };
    const int nk = kQLat / KB;
    // The waits are the compiler's own s_waitcnt (not inline assembly), so that it knows every
    // LDS read issued so far has completed at the barrier: otherwise it waits for the next
    // stage's fragment reads as well before the products of this one (their latency then
    // adds to every k-step).  Encoding (gfx9): vmcnt in bits 3:0 and 15:14, expcnt 6:4,
    // lgkmcnt 11:8; expcnt stays at its maximum.
    auto wait_stage = [&](int kt) {
        const int later = min(S - 2, nk - 1 - kt);
        if (later >= 2) __builtin_amdgcn_s_waitcnt(0x0078);        // vmcnt(8) lgkmcnt(0)
        else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0074);   // vmcnt(4) lgkmcnt(0)
        else __builtin_amdgcn_s_waitcnt(0x0070);                   // vmcnt(0) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
    };
    u32x4 fa[2][SM], fb[2][SN];
    auto read_frags = [&](int kt, int p) {
        const uint16_t *st = qsm + (kt % S) * kQStage;
#pragma unroll
        for (int i = 0; i < SM; ++i)
            fa[p][i] = *reinterpret_cast<const u32x4 *>(st + (wm * 128 + 16 * i + l16) * KB + 8 * lg);
#pragma unroll
        for (int j = 0; j < SN; ++j)
            fb[p][j] = *reinterpret_cast<const u32x4 *>(st + kQBM * KB + (wn * 64 + 16 * j + l16) * KB + 8 * lg);
    };
#pragma unroll
    for (int p = 0; p < S; ++p)
        if (p < nk) issue(p);
    wait_stage(0);
    read_frags(0, 0);
    for (int kt = 0; kt < nk; kt += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = kt + h;
            if (k + 1 < nk) {
                wait_stage(k + 1);
                if (k + S < nk) issue(k + S);
            }
            // the next step's fragments (after the last step: a stage read again, unused) are
            // read between this step's products, one read after each of the first 12
            read_frags(k + 1 < nk ? k + 1 : k, h ^ 1);
#pragma unroll
            for (int i = 0; i < SM; ++i)
#pragma unroll
                for (int j = 0; j < SN; ++j) acc[i][j] = mfma16x16x32(fa[h][i], fb[h][j], acc[i][j]);
#pragma unroll
            for (int x = 0; x < SM + SN; ++x) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, SM * SN - SM - SN, 0);
        }
    }
    const bool odd = l16 & 1;
    const bool rot = a.rope && (wn & 1) == 0;   // this wave's 64 columns are dims 0..63 of a head
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wm * 128 + 16 * i + 4 * lg + r;
            const int64_t rr = row < T ? row : T - 1;
            float v[SN];
#pragma unroll
            for (int j = 0; j < SN; ++j) v[j] = acc[i][j][r];
            if (rot) {
#pragma unroll
                for (int j = 0; j < SN; ++j) {
                    const float other = __shfl_xor(v[j], 1, 64);
                    v[j] = rotate(v[j], other, a.rope[rr * kRotPairs + 8 * j + (l16 >> 1)], odd);
                }
            }
            if (row >= T) continue;
#pragma unroll
            for (int j = 0; j < SN; ++j)
                a.q[row * a.ldq + n0 + wn * 64 + 16 * j + l16] = (uint16_t)f32_to_bf16(v[j]);
        }
}

static_assert(kQLat % (2 * kQKB) == 0 && kQOut % kQBN == 0 && kQBN % kDim == 0, "q tiles");

// [k | w] = x . [W_k | W_w] (N = 128 + HW, HW = 32 or 64 w columns), LayerNorm on the k part:
// 128-row tiles, each of the 4 waves owns 32 full rows.  The two weight matrices are read as one
// [7168][128 + HW] operand whose first 16 column-chunks come from W_k and the rest from W_w.
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
    const float2 *rope;         // [T][32] (cos, sin) for the key, or nullptr: no rotary step
};

template <int HW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void proj_kw_kernel(KWArgs a) {
    constexpr int BM = 128, BN = kDim + HW, SM = 2, SN = BN / 16;
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
    const int bkb = tid & 7, bnb = tid >> 3;   // bnb < 16 -> W_k, the rest -> W_w
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
            const int64_t rr = row < a.T ? row : a.T - 1;
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
            float kv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) kv[j] = fmaf((acc[i][j][r] - mu) * inv, g[j], b[j]);
            if (a.rope) {   // key dims 0..63 (j < 4) turn with the neighbouring lane's value
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float other = __shfl_xor(kv[j], 1, 64);
                    kv[j] = rotate(kv[j], other, a.rope[rr * kRotPairs + 8 * j + (l16 >> 1)], l16 & 1);
                }
            }
            if (row >= a.T) continue;
            if (a.k_base) {
                const int64_t slot = a.k_slot ? a.k_slot[row] : row;
                uint16_t *kr = a.k_base + slot * kDim;
#pragma unroll
                for (int j = 0; j < 8; ++j) kr[16 * j + l16] = (uint16_t)f32_to_bf16(kv[j]);
            }
#pragma unroll
            for (int j = 0; j < HW / 16; ++j)
                a.w[row * a.ldwo + 16 * j + l16] = (uint16_t)f32_to_bf16(acc[i][8 + j][r]);
        }
}

// ---------------------------------------------------------------- split K
// part[s][t][n] for the 64-row tile m0 = 64 blockIdx.z and the BN-column tile n0 = BN blockIdx.x:
// the product of A[m0 : m0 + 64, k0 : k0 + ks] and B[k0 : k0 + ks, n0 : n0 + BN], k0 = ks
// blockIdx.y, on the tiled core.  Used where the tiled kernels would leave most CUs idle: q and
// [k | w] of a decode step (T <= kSkinnyT), and [k | w] up to kKwSplitT tokens.
template <int BN, int WM, int WN>
__global__ __launch_bounds__(256) void skinny_partial_kernel(const uint16_t *__restrict__ A, int64_t lda,
                                                             int T, const uint16_t *__restrict__ B0, int ld0,
                                                             const uint16_t *__restrict__ B1, int ld1,
                                                             int nsplit, int N, int ks, float *__restrict__ part) {
    using Core = GemmCore<64, BN, WM, WN>;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    auto &sm = *reinterpret_cast<GemmSmem<64, BN> *>(smem_raw);
    const int n0 = BN * blockIdx.x;
    const int s = blockIdx.y;
    const int m0 = 64 * blockIdx.z;
    const int k0 = ks * s;
    f32x4 acc[Core::SM][Core::SN];
    Core::run(A + k0, lda, T, m0, B0 + (int64_t)k0 * ld0, ld0, B1 + (int64_t)k0 * ld1, ld1, nsplit, n0, ks,
              sm, acc);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave / WN, wn = wave % WN;
    const int l16 = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int i = 0; i < Core::SM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + wm * (64 / WM) + 16 * i + 4 * lg + r;
            if (row >= T) continue;
            float *pr = part + ((int64_t)s * T + row) * N + n0 + wn * (BN / WN) + l16;
#pragma unroll
            for (int j = 0; j < Core::SN; ++j) pr[16 * j] = acc[i][j][r];
        }
}

// q[t][n] = bf16(sum over the S slices of part[s][t][n]), N columns, q rows ldq apart; thread:
// 4 consecutive n (two rotary pairs when n mod 128 < 64 and rope is given).
__global__ __launch_bounds__(256) void skinny_reduce_q_kernel(const float *__restrict__ part, int S, int T, int N,
                                                              uint16_t *__restrict__ q, int64_t ldq,
                                                              const float2 *__restrict__ rope) {
    const int64_t e = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
    if (e >= (int64_t)T * N) return;
    f32x4 v = *reinterpret_cast<const f32x4 *>(part + e);
    for (int s = 1; s < S; ++s) {
        const f32x4 p = *reinterpret_cast<const f32x4 *>(part + (int64_t)s * T * N + e);
        v = f32x4{v[0] + p[0], v[1] + p[1], v[2] + p[2], v[3] + p[3]};
    }
    const int64_t t = e / N, n = e % N;
    if (rope && (n % kDim) < 2 * kRotPairs) {
        const int i = (int)(n % kDim) / 2;
        const float2 c0 = rope[t * kRotPairs + i], c1 = rope[t * kRotPairs + i + 1];
        v = f32x4{rotate(v[0], v[1], c0, false), rotate(v[1], v[0], c0, true), rotate(v[2], v[3], c1, false),
                  rotate(v[3], v[2], c1, true)};
    }
    *reinterpret_cast<u32x2 *>(q + t * ldq + n) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// One workgroup per token: wave j adds the slices s = j, j + 4, ... of the 128 + HW columns of
// [k | w] (lane: columns lane, 64 + lane, and 128 + lane for lane < HW); the four wave sums
// are added in a fixed order, then wave 0 applies the LayerNorm over the 128 key columns
// (as in the tiled kernel's epilogue) and the rotary step on dims 0..63 if rope is given,
// rounds to bf16 and writes k to its slot.
template <int HW>
__global__ __launch_bounds__(256) void skinny_reduce_kw_kernel(const float *__restrict__ part, int S, KWArgs a) {
    constexpr int N = kDim + HW;
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
        vw += lane < HW ? p[s * ss + kDim + lane] : 0.f;
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
    float k0 = fmaf(c0 * inv, bf16_to_f32(a.gamma[lane]), bf16_to_f32(a.beta[lane]));
    const float k1 = fmaf(c1 * inv, bf16_to_f32(a.gamma[64 + lane]), bf16_to_f32(a.beta[64 + lane]));
    if (a.rope) {
        const float other = __shfl_xor(k0, 1, 64);
        k0 = rotate(k0, other, a.rope[t * kRotPairs + (lane >> 1)], lane & 1);
    }
    if (a.k_base) {
        const int64_t slot = a.k_slot ? a.k_slot[t] : t;
        uint16_t *kr = a.k_base + slot * kDim;
        kr[lane] = (uint16_t)f32_to_bf16(k0);
        kr[64 + lane] = (uint16_t)f32_to_bf16(k1);
    }
    if (lane < HW) a.w[t * a.ldwo + lane] = (uint16_t)f32_to_bf16(vw);
}

constexpr int kSkQSlice = 256;    // q of a decode step: K = 1,536 in 6 slices x (N / 128) column tiles
constexpr int64_t kKwSplitT = 32768;   // [k | w] up to this many tokens: split K

size_t r256(size_t b) { return (b + 255u) & ~(size_t)255u; }

// K slices of the [k | w] product for T tokens (0: the tiled kernel): enough 64-row-tile x slice
// workgroups to fill the chip (about 1,024), each slice a whole number of 64-wide K blocks.
int kw_slices(int64_t T) {
    if (T > kKwSplitT) return 0;
    const int64_t tiles = (T + 63) / 64;
    static const int kDivs[] = {1, 2, 4, 7, 8, 14, 16, 28, 56};   // divisors of 7,168 / 64 = 112
    for (int d : kDivs)
        if (tiles * d >= 1024) return d;
    return 56;
}

size_t kw_part_bytes(int64_t T, int hw) {
    const int S = kw_slices(T);
    return S ? 4u * (size_t)S * (size_t)T * (size_t)(kDim + hw) : 0;
}

size_t main_workspace(int64_t T, int nq, int hw) {
    const size_t q = T > kSkinnyT ? (size_t)nq * kQLat * 2           // W_q transposed
                                  : 4u * (size_t)T * (size_t)(kQLat / kSkQSlice) * nq;   // q partial sums
    return r256(q) + kw_part_bytes(T, hw);
}

template <int HW>
hipError_t launch_kw(const KWArgs &a, float *part_kw, size_t smem_kw, hipStream_t stream) {
    const int S = kw_slices(a.T);
    if (S) {
        const unsigned tiles = (unsigned)((a.T + 63) / 64);
        hipLaunchKernelGGL((skinny_partial_kernel<kDim + HW, 2, 2>), dim3(1, S, tiles), dim3(256),
                           sizeof(GemmSmem<64, kDim + HW>), stream, a.x, a.ldx, (int)a.T, a.Wk, kDim, a.Ww,
                           (int)a.ldww, kDim, kDim + HW, kHidden / S, part_kw);
        hipLaunchKernelGGL(skinny_reduce_kw_kernel<HW>, dim3((unsigned)a.T), dim3(256), 0, stream, part_kw, S, a);
    } else {
        hipLaunchKernelGGL(proj_kw_kernel<HW>, dim3((unsigned)((a.T + 127) / 128)), dim3(256), smem_kw, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

size_t project_workspace(int64_t T, int nq, int hw, bool rope) {
    if (T <= 0) return 0;
    const size_t m = main_workspace(T, nq, hw);
    return rope ? r256(m) + 8u * (size_t)T * kRotPairs : m;
}

size_t project_workspace(int64_t T) { return project_workspace(T, kQOut, kHeads, false); }

hipError_t launch_project(const uint16_t *x, int64_t ldx, const uint16_t *c_q, int64_t ldc,
                          int64_t T, const uint16_t *W_q, const uint16_t *W_k,
                          const uint16_t *W_w, const uint16_t *gamma, const uint16_t *beta,
                          float eps, uint16_t *q, uint16_t *k_base, const int64_t *k_slot,
                          uint16_t *w, float *ws, hipStream_t stream) {
    return launch_project_ex(x, ldx, c_q, ldc, T, W_q, kQOut, kQOut, W_k, W_w, kHeads, kHeads, gamma, beta, eps,
                             q, kQOut, k_base, k_slot, w, kHeads, 0, 0.0, ws, stream);
}

hipError_t launch_project_ex(const uint16_t *x, int64_t ldx, const uint16_t *c_q, int64_t ldc,
                             int64_t T, const uint16_t *W_q, int64_t ldwq, int nq, const uint16_t *W_k,
                             const uint16_t *W_w, int64_t ldww, int hw, const uint16_t *gamma,
                             const uint16_t *beta, float eps, uint16_t *q, int64_t ldq,
                             uint16_t *k_base, const int64_t *k_slot, uint16_t *w, int64_t ldwo,
                             int64_t pos0, double theta, float *ws, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    if ((nq != kQOut && nq != 2 * kQOut) || (hw != kHeads && hw != 2 * kHeads)) return hipErrorInvalidValue;
    static DeviceOnce attr;
    const size_t smem_q = sizeof(uint16_t) * kQStage * kQStages;
    hipError_t ea = attr.run([&] {
        const std::pair<const void *, size_t> fs[] = {
            {reinterpret_cast<const void *>(proj_q_kernel), smem_q},
            {reinterpret_cast<const void *>(proj_kw_kernel<kHeads>), sizeof(GemmSmem<128, kDim + kHeads>)},
            {reinterpret_cast<const void *>(proj_kw_kernel<2 * kHeads>), sizeof(GemmSmem<128, kDim + 2 * kHeads>)},
            {reinterpret_cast<const void *>(skinny_partial_kernel<128, 1, 4>), sizeof(GemmSmem<64, 128>)},
            {reinterpret_cast<const void *>(skinny_partial_kernel<kDim + kHeads, 2, 2>),
             sizeof(GemmSmem<64, kDim + kHeads>)},
            {reinterpret_cast<const void *>(skinny_partial_kernel<kDim + 2 * kHeads, 2, 2>),
             sizeof(GemmSmem<64, kDim + 2 * kHeads>)}};
        for (const auto &f : fs) {
            hipError_t e = hipFuncSetAttribute(f.first, hipFuncAttributeMaxDynamicSharedMemorySize, (int)f.second);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    });
    if (ea != hipSuccess) return ea;
    const bool rot = theta > 0.0;
    float2 *rope = nullptr;
    if (rot) {
        rope = reinterpret_cast<float2 *>(reinterpret_cast<char *>(ws) + r256(main_workspace(T, nq, hw)));
        hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((T * kRotPairs + 255) / 256)), dim3(256), 0, stream,
                           rope, T, pos0, theta);
    }
    KWArgs a{x, ldx, T, W_k, W_w, gamma, beta, eps, k_base, k_slot, w, ldww, ldwo, rope};
    // the [k | w] partial sums (split K) follow the q part of the workspace
    float *part_kw = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) +
                                               (main_workspace(T, nq, hw) - kw_part_bytes(T, hw)));
    if (T <= kSkinnyT) {
        const int t = (int)T;
        float *part_q = ws;
        if (q) {
            hipLaunchKernelGGL((skinny_partial_kernel<128, 1, 4>), dim3(nq / 128, kQLat / kSkQSlice, 1),
                               dim3(256), sizeof(GemmSmem<64, 128>), stream, c_q, ldc, t, W_q, (int)ldwq, W_q,
                               (int)ldwq, nq, nq, kSkQSlice, part_q);
            hipLaunchKernelGGL(skinny_reduce_q_kernel, dim3((unsigned)((T * nq / 4 + 255) / 256)), dim3(256), 0,
                               stream, part_q, kQLat / kSkQSlice, t, nq, q, ldq, (const float2 *)rope);
        }
    } else if (q) {
        uint16_t *WqT = reinterpret_cast<uint16_t *>(ws);
        hipLaunchKernelGGL(transpose_wq_kernel, dim3(nq / 64, kQLat / 64), dim3(256), 0, stream, W_q, ldwq, WqT);
        const int64_t tiles = (T + kQBM - 1) / kQBM * (nq / kQBN);
        QArgs qa{c_q, ldc, T, WqT, nq, q, ldq, rope};
        hipLaunchKernelGGL(proj_q_kernel, dim3((unsigned)tiles), dim3(512), smem_q, stream, qa);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t smem_kw = hw == kHeads ? sizeof(GemmSmem<128, kDim + kHeads>) : sizeof(GemmSmem<128, kDim + 2 * kHeads>);
    return hw == kHeads ? launch_kw<kHeads>(a, part_kw, smem_kw, stream)
                        : launch_kw<2 * kHeads>(a, part_kw, smem_kw, stream);
}

}  // namespace dsaidx
