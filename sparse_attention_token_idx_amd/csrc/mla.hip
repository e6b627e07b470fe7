// Sparse MLA over the selected tokens: the consumer of the indexer's selection ("Qwen3.5-397B-
// A17B vs Kimi K3.1 Pro" compare page, gated-MLA row).  Shapes from that row: H = 96, a cache
// row per token of 512 + 64 = 576 bf16 values (latent, then the position key slot), and the
// key set of query t is the <= 2,048 rows its indexer picked; MLA turns no rotary step ("Kimi
// K3.1 Pro vs Gemma 4 31B" page, RoPE row).  Queries arrive in the absorbed latent form
// q~ [96][576]: logit(h, s) = scale * q~_h . kv[s] over all 576 values, a softmax over the
// picked rows, and out_h = sum_s p_h(s) kv[s][0:512] (the dense value up-projection, gate and
// output projection come after this step).
//
// One workgroup takes one query and a contiguous split of its selections; its 3 waves, one per
// SIMD, take 32 heads each (two 16-head MFMA groups) over all 576 logit dims and all 512 output
// dims, so that every tile is read from LDS once per 32 heads: the wave's query slice stays in
// 144 VGPRs and its output in the 256 accumulation registers.  The selected cache rows stream
// through LDS 32 at a time with direct global->LDS loads, four tiles deep, row-major (a
// token's 72 16-byte pieces in a row, the piece order swizzled by the token so that the rows
// one operand read touches fall in different banks).  The logits S^T = K q~^T
// (v_mfma_f32_16x16x32_bf16, the wave's q~ as the B operand) take K straight from those rows.
// The output O^T += V^T P^T takes V^T from the same rows with the transposing LDS read of
// gfx950 (ds_read_b64_tr_b16: each 16-lane group loads 4 tokens x 16 dims and every lane
// receives one dim of the 4 tokens), and P^T straight from the logit accumulators (the 32
// tokens of a tile taken in the order the accumulators hold them).  The softmax is in the log2
// domain against a fixed reference per head (the first tile's maximum), so the accumulated
// output is never rescaled; a split whose logits outrun the reference by more than 2^64 is run
// again against the true maxima.  With several splits per query, each split writes its (max,
// sum) and its output normalised by its own sum, in bf16 (a convex combination of latents, so
// in their range), and a second kernel merges them.
#include "common.hpp"
#include "launch.hpp"

namespace dsaidx {
namespace {

constexpr int kMlaHeads = 96;
constexpr int kKv = 576;                 // cached values per token
constexpr int kV = 512;                  // latent (value) dims
constexpr int kHeadsPerWave = 32;        // two 16-head MFMA groups, every logit and output dim
constexpr int kWavesMla = kMlaHeads / kHeadsPerWave;   // 3, one per SIMD
constexpr int kMlaThreads = 64 * kWavesMla;
constexpr int kTile = 32;                // selected tokens per LDS tile
constexpr int kPieces = kKv / 8;         // 16-byte pieces of a cache row: 72
constexpr int kSlots = kTile * kPieces;  // of a tile: 2,304 = 36 load instructions of 64 lanes
constexpr int kSlotsPerWave = kSlots / kMlaThreads;   // 12
constexpr int kBufs = 4;                 // tiles in LDS: being read, being added, two in flight
constexpr int kMaxSel = 2048;            // selections per split held in LDS
constexpr int kTileBytes = kSlots * 16;
constexpr int kHalfTileBytes = kTileBytes / 2;        // tokens 16..31 start here
static_assert(kSlots % kMlaThreads == 0 && kPieces == 72 && kV == 512, "tile geometry");

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

struct MlaSmem {
    uint16_t k[kBufs][kSlots * 8];   // token tau's piece u sits in slot 72 tau + (u ^ swz(tau))
    int32_t sel[kMaxSel];            // this split's cache rows (INT_MIN: none)
    uint32_t slot_pk[kWavesMla][kSlotsPerWave / 2][64];   // each lane's tile-load constants
};

// Piece u of token tau sits at position u ^ swz(tau) among the token's 72 slots: a permutation
// within each aligned group of 8 pieces, so that a piece's offset from the group start, and
// hence every operand address below, is a per-lane base plus a constant.  The LDS serves 256
// bytes (64 banks) at a time and the rows are 1,152 bytes apart, so rows of equal parity start
// in the same bank, odd ones 128 bytes on.  swz takes all 8 values on the 8 even and on the 8
// odd tokens of each 16 (a logit-operand read: 16 rows x 16 bytes), and 4 different even
// values on the 4 tokens of equal parity among any 8 tokens 8 m .. 8 m + 7 (a transposing read:
// 32 lanes, 8 tokens x 32 bytes), so that both fill the banks once.  An involution.
__device__ __forceinline__ int swz(int tau) { return (2 * ((tau >> 1) & 3) + ((tau >> 3) & 1)) & 7; }
template <bool B> struct Flag {
    static constexpr bool value = B;
};

constexpr float kRefRange = 64.f;   // logits may exceed a head's reference by this much (log2 units)

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
    uint16_t *part_o;        // [nsplit][T][96][512] bf16, normalised by the split's sum (nsplit > 1)
    float *part_ml;          // [nsplit][T][96][2]: running max (log2 domain), sum
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to bf16 (round to nearest even), with gfx950's packing conversion.
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// 2^x with the hardware instruction: the arguments here are at most kRefRange = 64 (or -inf),
// and a result below the normal range (a weight under 2^-126 of the reference) may flush to 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier over LDS traffic only: __syncthreads() would also wait for every global
// load in flight, the tiles ahead included.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One 16-byte-per-lane global->LDS load (lane i lands at lds_addr + 16 i).  Written out so that
// the compiler, which cannot tell the tiles in flight from the one being read, does not wait for
// them before every LDS read; the kernel counts these loads and waits for them itself.  The
// instruction has no result registers and reads its address registers when it issues.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_addr) : "memory", "m0");
}

__device__ __forceinline__ uint2 tr_read(const lds_char *p) {
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p);
    return __builtin_bit_cast(uint2, v);
}

__global__ __launch_bounds__(kMlaThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_mla_kernel(MlaArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    MlaSmem &sm = *reinterpret_cast<MlaSmem *>(smem_raw);
    const lds_char *lds_k = (const lds_char *)smem_raw;   // the tile buffers start the area
    // The splits of a query run on one XCD (workgroup i runs on XCD i mod 8), so its q~ comes from
    // HBM once and from that XCD's L2 for the other splits: query t sits on XCD t mod 8, and
    // workgroups past the last query end at once.
    const int xcd = blockIdx.x & 7, chunk = blockIdx.x >> 3;
    const int split = chunk % a.nsplit;
    const int64_t t = 8 * (int64_t)(chunk / a.nsplit) + xcd;
    if (t >= a.T) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    constexpr int kKs = kKv / 32;                 // logit k-steps: 18
    constexpr int kMt = kV / 16;                  // 16-dim output tiles: 32
    constexpr int kG = kHeadsPerWave / 16;        // head groups of a wave: 2
    const int sel0 = split * a.per;
    const int nsel = max(0, min(a.topk, sel0 + a.per) - sel0);
    const int ntile = (nsel + kTile - 1) / kTile;
    const int64_t base = a.row0 ? a.row0[t] : 0;
    for (int x = tid; x < ntile * kTile; x += kMlaThreads) {
        // the cache row of each selection (below 2^31), or INT_MIN for none
        const int32_t r = x < nsel ? a.idx[t * (int64_t)a.topk + sel0 + x] : -1;
        sm.sel[x] = r >= 0 ? (int32_t)(base + r) : INT_MIN;
    }

    // this wave's q~ as the B operand of S^T = K q~^T: lane (l16, g) holds head
    // 32 wave + 16 e + l16, dims 32 ks + 8 g .. + 7
    u32x4 qb[kG][kKs];   // loaded after tile 0's loads are issued (below)
    __syncthreads();   // sel

    // A tile goes to LDS with direct global->LDS loads: lane i of instruction j of a wave fills
    // slot 64 (12 wave + j) + i, i.e. piece (slot - 72 tau) ^ swz(tau) of token tau = slot / 72.
    // A token with no selection reads cache row 0 instead (its logit is masked, its weight is
    // 0).  Exactly kSlotsPerWave vector-memory instructions per tile and wave: the waits below
    // count on it.  tau and the piece are the same for every tile, so they are worked out once
    // into LDS, 16 bits per instruction (tau in bits 0-4, the piece in bits 5-11), two
    // instructions per word: in registers they would crowd out the loop's.
    const char *kv_bytes = reinterpret_cast<const char *>(a.kv);
    const uint32_t lds_k0 = (uint32_t)(uintptr_t)(lds_void *)sm.k[0];
#pragma unroll
    for (int j = 0; j < kSlotsPerWave; j += 2) {
        uint32_t v = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int slot = 64 * (kSlotsPerWave * wave + j + h) + lane;
            const int tau = slot / kPieces;
            const int piece = (slot - kPieces * tau) ^ swz(tau);
            v |= (uint32_t)(tau | piece << 5) << (16 * h);
        }
        sm.slot_pk[wave][j / 2][lane] = v;   // read back by this lane only
    }
    auto load_tile = [&](int tile, int buf_off) {
        // every row first: the loads are opaque to the compiler, which would otherwise wait for
        // each LDS read in turn
        uint32_t pk[kSlotsPerWave / 2], rw[kSlotsPerWave];
#pragma unroll
        for (int i = 0; i < kSlotsPerWave / 2; ++i) pk[i] = sm.slot_pk[wave][i][lane];
#pragma unroll
        for (int j = 0; j < kSlotsPerWave; ++j) {
            const uint32_t tau = (pk[j / 2] >> (16 * (j & 1))) & 31u;
            rw[j] = (uint32_t)sm.sel[tile * kTile + tau];
        }
#pragma unroll
        for (int j = 0; j < kSlotsPerWave; ++j) {
            const uint32_t u16 = ((pk[j / 2] >> (16 * (j & 1))) >> 1) & 0x7f0u;
            // a token with no selection reads cache row 0 (its logit is masked, its weight is 0)
            const uint64_t row = rw[j] & 0x7fffffffu;
            dma16(kv_bytes + u16 + row * (2 * kKv),
                  __builtin_amdgcn_readfirstlane(lds_k0 + buf_off + 16 * 64 * (kSlotsPerWave * wave + j)));
        }
    };

    // LDS byte offsets (within a tile) of this lane's operand reads.  Logits, k-step ks: token
    // l16 (and 16 + l16, kHalfTileBytes further: the same swizzle), piece 4 ks + g, at
    // qk_base[ks & 1] + 128 (ks >> 1).
    int qk_base[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) qk_base[h] = 16 * (kPieces * l16 + ((4 * h + g) ^ swz(l16)));
    // Values, tile mt (dims 16 mt ..): this lane loads token 4 g + (l16 >> 2) (and 16 + that,
    // kHalfTileBytes further), dims 4 (l16 & 3) .. + 3 of the tile, i.e. piece
    // 2 mt + ((l16 & 3) >> 1), bytes 8 (l16 & 1) .., at pv_base[mt & 3] + 128 (mt >> 2)
    const int vtok = 4 * g + (l16 >> 2);
    int pv_base[4];
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4)
        pv_base[m4] = 16 * (kPieces * vtok + ((2 * m4 + ((l16 & 3) >> 1)) ^ swz(vtok))) + 8 * (l16 & 1);

    f32x4 acc_o[kG][kMt];   // O^T: lane (l16, g) holds dims 16 mt + 4 g + r of head 32 wave + 16 e + l16
#pragma unroll
    for (int e = 0; e < kG; ++e)
#pragma unroll
        for (int mt = 0; mt < kMt; ++mt) acc_o[e][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The weights are exp2(logit - m_ref), m_ref a reference per head: the first finite tile max,
    // so that no accumulated output ever needs rescaling (the accumulators stay in the matrix
    // cores' registers).  A later tile may exceed it by up to kRefRange (weights up to 2^64,
    // well inside fp32 and bf16); if any head's logits go further, the split is run again with
    // each head's true maximum as its reference, which the first run has found by then.
    float m_ref[kG], m_all[kG], l_run[kG];
    u32x4 pb[kG];                 // P^T of the tile whose values are added next (bf16 pairs)
    bool over = false;            // this lane's heads went past their reference range

    auto head_max = [](float x) {   // over the 4 lane groups that hold one head's tokens
        x = fmaxf(x, __shfl_xor(x, 16, 64));
        return fmaxf(x, __shfl_xor(x, 32, 64));
    };
    auto vread = [&](const lds_char *vb, int mt) {
        const lds_char *vp = vb + pv_base[mt & 3] + 128 * (mt >> 2);
        const uint2 lo = tr_read(vp);
        const uint2 hi = tr_read(vp + kHalfTileBytes);
        return u32x4{lo.x, lo.y, hi.x, hi.y};
    };
    // One pipeline step over tile `tile` (buffer kb):
    //  A. its logits (matrix instructions only, the K operands read two k-steps ahead);
    //  B. its weights (vector instructions), under the output update of the previous tile's
    //     values (buffer vb, O^T += V^T P^T, both head groups from one read of V^T) when pv_tag
    //     says so; the next step's update takes the new weights from pb.
    auto step = [&](auto pv_tag, int tile, const lds_char *kb, const lds_char *vb) {
        constexpr bool kPv = decltype(pv_tag)::value;
        // A. S^T rows are tokens (two 16-token halves), columns the group's 16 heads
        f32x4 s[kG][2];
#pragma unroll
        for (int e = 0; e < kG; ++e) s[e][0] = s[e][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto kread = [&](int ks, u32x4 &k0, u32x4 &k1) {
            const int off = qk_base[ks & 1] + 128 * (ks >> 1);
            k0 = *(const lds_u32x4 *)(kb + off);
            k1 = *(const lds_u32x4 *)(kb + off + kHalfTileBytes);
        };
        // K operands read two k-steps ahead of the matrix instructions that take them
        u32x4 k0, k1, m0, m1;
        kread(0, k0, k1);
        kread(1, m0, m1);
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
            u32x4 n0, n1;
            if (ks + 2 < kKs) kread(ks + 2, n0, n1);
#pragma unroll
            for (int e = 0; e < kG; ++e) {
                s[e][0] = mfma16x16x32(k0, qb[e][ks], s[e][0]);
                s[e][1] = mfma16x16x32(k1, qb[e][ks], s[e][1]);
            }
            k0 = m0;
            k1 = m1;
            m0 = n0;
            m1 = n1;
            // keep each k-step's four accumulation chains in order: a chain's next product then
            // comes four matrix instructions (64 cycles) after its last
            __builtin_amdgcn_sched_barrier(0);
        }
        // B. lane (l16, g): head 16 e + l16 of the wave's 32, tokens 4 g + r (s[e][0]) and
        // 16 + 4 g + r (s[e][1])
        const int4 sa = *reinterpret_cast<const int4 *>(&sm.sel[tile * kTile + 4 * g]);
        const int4 sb = *reinterpret_cast<const int4 *>(&sm.sel[tile * kTile + 16 + 4 * g]);
        const int sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
        float z[kG][8], mx[kG];
#pragma unroll
        for (int e = 0; e < kG; ++e) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                z[e][r] = sv[r] >= 0 ? s[e][0][r] * a.scale_log2 : -INFINITY;
                z[e][4 + r] = sv[4 + r] >= 0 ? s[e][1][r] * a.scale_log2 : -INFINITY;
            }
            mx[e] = z[e][0];
#pragma unroll
            for (int r = 1; r < 8; ++r) mx[e] = fmaxf(mx[e], z[e][r]);
            m_all[e] = fmaxf(m_all[e], mx[e]);
        }
        // a head without a reference yet (nothing weighed so far) takes this tile's maximum;
        // the wave agrees on it (a branch the whole wave takes, on the first tiles only)
        bool unset = false;
#pragma unroll
        for (int e = 0; e < kG; ++e) unset |= m_ref[e] == -INFINITY;
        if (__builtin_amdgcn_ballot_w64(unset)) {
#pragma unroll
            for (int e = 0; e < kG; ++e) {
                const float hm = head_max(mx[e]);
                m_ref[e] = m_ref[e] == -INFINITY ? hm : m_ref[e];
            }
        }
        // the new weights of head group e, their vector instructions placed between the output
        // update's matrix instructions
        u32x4 pn[kG];
        auto weights = [&](int e) {
            over |= mx[e] > m_ref[e] + kRefRange;
            const bool none = m_ref[e] == -INFINITY;
            float p[8], ps = 0.f;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                p[r] = none ? 0.f : exp2_hw(z[e][r] - m_ref[e]);
                ps += p[r];
            }
            l_run[e] += ps;
            // P^T as the B operand: k slots 8 g .. 8 g + 7 are the lane's 8 tokens, and the V^T
            // operand holds the same tokens (4 g .. 4 g + 3 and 16 + 4 g .. + 3)
            pn[e] = u32x4{bf16_pair(p[0], p[1]), bf16_pair(p[2], p[3]), bf16_pair(p[4], p[5]), bf16_pair(p[6], p[7])};
        };
        if (kPv) {
            u32x4 v = vread(vb, 0);
#pragma unroll
            for (int mt = 0; mt < kMt; ++mt) {
                u32x4 vn;
                if (mt + 1 < kMt) vn = vread(vb, mt + 1);
#pragma unroll
                for (int e = 0; e < kG; ++e) acc_o[e][mt] = mfma16x16x32(v, pb[e], acc_o[e][mt]);
                if (mt == 2) weights(0);
                if (mt == 10) weights(1);
                if (mt == 2 || mt == 10) __builtin_amdgcn_sched_barrier(0);
                v = vn;
            }
        } else {
            weights(0);
            weights(1);
        }
#pragma unroll
        for (int e = 0; e < kG; ++e) pb[e] = pn[e];
    };

    // the queries, their latency under that of tile 0's loads
    auto load_queries = [&] {
#pragma unroll
        for (int e = 0; e < kG; ++e) {
            const uint16_t *qh = a.q + (t * kMlaHeads + kHeadsPerWave * wave + 16 * e + l16) * (int64_t)kKv + 8 * g;
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) qb[e][ks] = *reinterpret_cast<const u32x4 *>(qh + 32 * ks);
        }
        // use them here, so that the compiler waits for these loads before the tile loop rather
        // than inside it, where its count of loads in flight would not include the tiles' (the
        // wait drains the tiles' loads issued before them too: the first tile needs them anyway)
#pragma unroll
        for (int e = 0; e < kG; ++e)
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) asm volatile("" ::"v"(qb[e][ks]));
    };
    // Tiles 0 and 1 are loaded ahead and tile t + 2 during step t, into buffer (t + 2) % 4, whose
    // tile t - 2 step t - 1 consumed.  So when step t begins, only tile t + 1's loads may still be
    // in flight beside tile t's.
#pragma unroll 1
    for (int run = 0; run < 2; ++run) {
#pragma unroll
        for (int e = 0; e < kG; ++e) {
#pragma unroll
            for (int mt = 0; mt < kMt; ++mt) acc_o[e][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            m_ref[e] = run ? head_max(m_all[e]) : -INFINITY;   // a run again: the true maxima
            m_all[e] = -INFINITY;
            l_run[e] = 0.f;
            pb[e] = u32x4{0u, 0u, 0u, 0u};
        }
        over = false;
        // tile 0 and the queries first; the wait for the queries (which drains tile 0's loads,
        // issued before them) then leaves tile 1's loads in flight into step 0
        if (ntile > 0) load_tile(0, 0);
        if (run == 0) load_queries();
        if (ntile > 1) load_tile(1, kTileBytes);
        auto body = [&](auto pv_tag, int tile) {
            if (tile + 1 < ntile)
                asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            // every wave's loads of this tile have landed, and every wave is done with step
            // tile - 1, i.e. with the values of tile - 2 (whose buffer tile + 2 takes)
            lds_barrier();
            if (tile + 2 < ntile) load_tile(tile + 2, ((tile + 2) & (kBufs - 1)) * kTileBytes);
            const lds_char *kb = lds_k + (tile & (kBufs - 1)) * kTileBytes;
            const lds_char *vb = lds_k + ((tile - 1) & (kBufs - 1)) * kTileBytes;
            step(pv_tag, tile, kb, vb);
        };
        if (ntile > 0) body(Flag<false>{}, 0);
#pragma unroll 1
        for (int tile = 1; tile < ntile; ++tile) body(Flag<true>{}, tile);
        if (ntile > 0) {   // the last tile's values
            const lds_char *vb = lds_k + ((ntile - 1) & (kBufs - 1)) * kTileBytes;
#pragma unroll
            for (int mt = 0; mt < kMt; ++mt) {
                const u32x4 va = vread(vb, mt);
#pragma unroll
                for (int e = 0; e < kG; ++e) acc_o[e][mt] = mfma16x16x32(va, pb[e], acc_o[e][mt]);
            }
        }
        // run again (every wave: they share the tile ring) if any head left its range
        if (!__syncthreads_or(over)) break;
    }

#pragma unroll
    for (int e = 0; e < kG; ++e) {
        // the head's sum over its 4 lane groups
        float l_tot = l_run[e] + __shfl_xor(l_run[e], 16, 64);
        l_tot += __shfl_xor(l_tot, 32, 64);
        const int head = kHeadsPerWave * wave + 16 * e + l16;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (a.nsplit == 1) {
            uint16_t *oh = a.o + (t * kMlaHeads + head) * (int64_t)kV + 4 * g;
#pragma unroll
            for (int mt = 0; mt < kMt; ++mt) {
                const f32x4 o = acc_o[e][mt];
                const uint2 v = {bf16_pair(o[0] * inv, o[1] * inv), bf16_pair(o[2] * inv, o[3] * inv)};
                *reinterpret_cast<uint2 *>(oh + 16 * mt) = v;
            }
            if (a.lse && g == 0)
                a.lse[t * kMlaHeads + head] = l_tot > 0.f ? (m_ref[e] + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
        } else {
            const int64_t ph = ((int64_t)split * a.T + t) * kMlaHeads + head;
            uint16_t *oh = a.part_o + ph * kV + 4 * g;
#pragma unroll
            for (int mt = 0; mt < kMt; ++mt) {
                const f32x4 o = acc_o[e][mt];
                const uint2 v = {bf16_pair(o[0] * inv, o[1] * inv), bf16_pair(o[2] * inv, o[3] * inv)};
                *reinterpret_cast<uint2 *>(oh + 16 * mt) = v;
            }
            if (g == 0) {
                a.part_ml[2 * ph] = m_ref[e];
                a.part_ml[2 * ph + 1] = l_tot;
            }
        }
    }
}

// Merge of the splits of one (query, head): one wave per (query, head), lane i owns dims
// 8 i .. 8 i + 7.
__global__ __launch_bounds__(256) void sparse_mla_merge_kernel(MlaArgs a) {
    // Query t's partials were written on XCD t mod 8 (the main kernel's order) and are still in
    // that XCD's L2: its heads are merged there too, 4 per workgroup.
    const int xcd = blockIdx.x & 7, chunk = blockIdx.x >> 3;
    const int64_t t = 8 * (int64_t)(chunk / (kMlaHeads / 4)) + xcd;
    if (t >= a.T) return;
    const int64_t qh = t * kMlaHeads + 4 * (chunk % (kMlaHeads / 4)) + (threadIdx.x >> 6);   // t * 96 + head
    const int lane = threadIdx.x & 63;
    const int64_t stride = a.T * kMlaHeads;   // between splits
    float M = -INFINITY;
#pragma unroll 4
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_ml[2 * (s * stride + qh)]);
    float L = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll 4
        for (int s = 0; s < a.nsplit; ++s) {
            const int64_t ph = s * stride + qh;
            const float ms = a.part_ml[2 * ph];
            // the split's normalised output weighs by its share of the sum, f * l_s (0 for a
            // split with nothing selected)
            const float fl = ms == -INFINITY ? 0.f : exp2f(ms - M) * a.part_ml[2 * ph + 1];
            L += fl;
            const u32x4 x = *reinterpret_cast<const u32x4 *>(a.part_o + ph * kV + 8 * lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[2 * r] = fmaf(fl, bf16_to_f32(x[r] & 0xFFFFu), acc[2 * r]);
                acc[2 * r + 1] = fmaf(fl, bf16_to_f32(x[r] >> 16), acc[2 * r + 1]);
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
    static DeviceInt cached;
    return cached.get([] {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        return cus;
    });
}

}  // namespace

int sparse_mla_splits(int64_t T, int topk) {
    if (T <= 0 || topk <= 0) return 1;
    const int64_t want = ((int64_t)mla_cus() + T - 1) / T;               // a workgroup per CU (LDS fits one)
    const int64_t most = ((int64_t)topk + 8 * kTile - 1) / (8 * kTile);   // at least 8 tiles a split
    const int64_t least = ((int64_t)topk + kMaxSel - 1) / kMaxSel;         // at most kMaxSel a split
    int64_t n = want < most ? want : most;
    n = n < least ? least : n;
    return (int)(n < 1 ? 1 : n);
}

size_t sparse_mla_workspace(int64_t T, int topk) {
    const int ns = sparse_mla_splits(T, topk);
    if (ns <= 1) return 0;
    return (size_t)ns * (size_t)T * kMlaHeads * (kV * 2u + 2 * 4u);
}

hipError_t launch_sparse_mla(const uint16_t *q, const uint16_t *kv, const int32_t *idx, const int64_t *row0,
                             int64_t T, int topk, float scale, uint16_t *o, float *lse, float *ws,
                             hipStream_t stream) {
    static DeviceOnce attr;
    const size_t smem = sizeof(MlaSmem);
    hipError_t ea = attr.run([&] {
        return hipFuncSetAttribute(reinterpret_cast<const void *>(sparse_mla_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    });
    if (ea != hipSuccess) return ea;
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
    a.part_o = reinterpret_cast<uint16_t *>(ws);
    a.part_ml = ws ? reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + (size_t)a.nsplit * (size_t)T * kMlaHeads * kV * 2u)
                   : nullptr;
    const int64_t groups = (T + 7) / 8;   // of 8 queries, one per XCD
    hipLaunchKernelGGL(sparse_mla_kernel, dim3((unsigned)(groups * 8 * a.nsplit)), dim3(kMlaThreads), smem, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    hipLaunchKernelGGL(sparse_mla_merge_kernel, dim3((unsigned)(groups * 8 * (kMlaHeads / 4))), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
