// Sparse MLA over the selected tokens: the consumer of the indexer's selection ("Qwen3.5-397B-
// A17B vs Kimi K3.1 Pro" compare page, gated-MLA row).  Shapes from that row: H = 96, a cache
// row per token of 512 + 64 = 576 bf16 values (latent, then the position key slot), and the
// key set of query t is the <= 2,048 rows its indexer picked; MLA turns no rotary step ("Kimi
// K3.1 Pro vs Gemma 4 31B" page, RoPE row).  Queries arrive in the absorbed latent form
// q~ [96][576]: logit(h, s) = scale * q~_h . kv[s] over all 576 values, a softmax over the
// picked rows, and out_h = sum_s p_h(s) kv[s][0:512] (the dense value up-projection, gate and
// output projection come after this step).
//
// One workgroup takes one query and a contiguous split of its selections; its 12 waves pair up
// on 16 heads each, the two waves of a pair taking alternate 32-dim k-steps of the 576 logit
// dims and alternate 16-dim tiles of the 512 output dims, so that a wave holds its query
// slice (36 VGPRs) and its output (64) with three waves per SIMD.  The selected cache rows
// stream through LDS 32 at a time with direct global->LDS loads, three tiles deep, row-major
// (a token's 72 16-byte pieces in a row, the piece order swizzled by the token so that the
// rows one operand read touches fall in different banks).  The logits S^T = K q~^T
// (v_mfma_f32_16x16x32_bf16, the wave's q~ as the B operand) take K straight from those rows;
// the pair adds its two halves through LDS.  The output O^T += V^T P^T takes V^T from the same
// rows with the transposing LDS read of gfx950 (ds_read_b64_tr_b16: each 16-lane group loads 4
// tokens x 16 dims and every lane receives one dim of the 4 tokens), and P^T straight from the
// logit accumulators (the 32 tokens of a tile taken in the order the accumulators hold them).
// The softmax is online, in the log2 domain; with several splits per query, each split writes
// its (max, sum) and its output normalised by its own sum, in bf16 (a convex combination of
// latents, so in their range), and a second kernel merges them.
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
constexpr int kBufs = 3;                 // tiles in LDS: the current one and two in flight
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
    int32_t sel[kMaxSel];            // this split's selections (-1: none)
    f32x4 sx[kWavesMla][2][64];      // each wave's half of the logits, for its partner
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
constexpr float kLazy = 8.f;   // a head's reference max moves only when exceeded by 2^8

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

// 2^x with the hardware instruction: the arguments here are at most 8 (or -inf), and a result
// below the normal range (a weight under 2^-126 of the largest) may flush to 0.
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

__global__ __launch_bounds__(kMlaThreads, 1) void sparse_mla_kernel(MlaArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    MlaSmem &sm = *reinterpret_cast<MlaSmem *>(smem_raw);
    const lds_char *lds_k = (const lds_char *)smem_raw;   // the tile buffers start the area
    const int split = blockIdx.x;
    const int64_t t = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int hg = wave >> 1, half = wave & 1;   // heads 16 hg .. + 15; alternate k-steps / tiles
    constexpr int kKs = kKv / 32 / 2;             // logit k-steps of a wave: 9
    constexpr int kMt = kV / 16 / 2;              // 16-dim output tiles of a wave: 16
    const int sel0 = split * a.per;
    const int nsel = max(0, min(a.topk, sel0 + a.per) - sel0);
    const int ntile = (nsel + kTile - 1) / kTile;
    const int64_t base = a.row0 ? a.row0[t] : 0;
    for (int x = tid; x < ntile * kTile; x += kMlaThreads)
        sm.sel[x] = x < nsel ? a.idx[t * (int64_t)a.topk + sel0 + x] : -1;

    // this wave's q~ as the B operand of S^T = K q~^T: lane (l16, g) holds head 16 hg + l16,
    // dims 32 (2 ks + half) + 8 g .. + 7
    u32x4 qb[kKs];   // loaded after the first tiles' loads are issued (below)
    __syncthreads();   // sel

    // A tile goes to LDS with direct global->LDS loads: lane i of instruction j of a wave fills
    // slot 64 (3 wave + j) + i, i.e. piece (slot % 72) ^ swz(tau) of token tau = slot / 72.  A token
    // with no selection reads cache row 0 instead (its logit is masked, its weight is 0).
    // Exactly kSlotsPerWave vector-memory instructions per tile and wave: the waits below count
    // on it.
    const char *kv_bytes = reinterpret_cast<const char *>(a.kv);
    const uint32_t lds_k0 = (uint32_t)(uintptr_t)(lds_void *)sm.k[0];
    auto load_tile = [&](int tile, int buf_off) {
        // the slot geometry is recomputed per tile from the lane index, itself recomputed here
        // (v_mbcnt): held across the loop it would cost registers the operands need
        int ln;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        int tau[kSlotsPerWave];
        int32_t r[kSlotsPerWave];
#pragma unroll
        for (int j = 0; j < kSlotsPerWave; ++j) {
            tau[j] = (64 * (kSlotsPerWave * wave + j) + ln) / kPieces;
            r[j] = sm.sel[tile * kTile + tau[j]];
        }
#pragma unroll
        for (int j = 0; j < kSlotsPerWave; ++j) {
            const int slot0 = 64 * (kSlotsPerWave * wave + j);
            const int slot = slot0 + ln;
            const int u16 = 16 * ((slot - kPieces * tau[j]) ^ swz(tau[j]));
            const int64_t row = r[j] >= 0 ? base + r[j] : 0;
            dma16(kv_bytes + (row * (2 * kKv) + u16),
                  __builtin_amdgcn_readfirstlane(lds_k0 + buf_off + 16 * slot0));
        }
    };

    // LDS byte offsets (within a tile) of this lane's operand reads.  Logits, k-step ks: token
    // l16 (and 16 + l16, kHalfTileBytes further: the same swizzle), piece 8 ks + 4 half + g, at
    // qk_base + 128 ks.
    const int qk_base = 16 * (kPieces * l16 + ((4 * half + g) ^ swz(l16)));
    // Values, tile mt (dims 16 (2 mt + half) ..): this lane loads token 4 g + (l16 >> 2) (and
    // 16 + that, kHalfTileBytes further), dims 4 (l16 & 3) .. + 3 of the tile, i.e. piece
    // 4 mt + 2 half + ((l16 & 3) >> 1), bytes 8 (l16 & 1) .., at pv_base[mt & 1] + 128 (mt >> 1)
    const int vtok = 4 * g + (l16 >> 2);
    int pv_base[2];
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2)
        pv_base[m2] = 16 * (kPieces * vtok + ((4 * m2 + 2 * half + ((l16 & 3) >> 1)) ^ swz(vtok))) + 8 * (l16 & 1);

    f32x4 acc_o[kMt];   // O^T: lane (l16, g) holds dims 16 (2 mt + half) + 4 g + r of head 16 hg + l16
#pragma unroll
    for (int mt = 0; mt < kMt; ++mt) acc_o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;   // running max of the head's logits (log2 domain)
    float l_run = 0.f;         // this lane's part of the running sum

    u32x4 pb = {0u, 0u, 0u, 0u};   // P^T of the tile whose values are added next (bf16 pairs)
    float factor = 1.f;            // and the rescaling of the output that must come first
    bool rescale = false;

    // Output update with the previous tile's values: O^T += V^T P^T over one 16-dim tile mt.
    auto pv = [&](const lds_char *vb, int mt) {
        const lds_char *vp = vb + pv_base[mt & 1] + 128 * (mt >> 1);
        const uint2 lo = tr_read(vp);
        const uint2 hi = tr_read(vp + kHalfTileBytes);
        acc_o[mt] = mfma16x16x32(u32x4{lo.x, lo.y, hi.x, hi.y}, pb, acc_o[mt]);
    };
    auto apply_rescale = [&] {
        if (__builtin_expect(rescale, 0)) {   // wave-uniform, rarely taken after the first tiles
#pragma unroll
            for (int mt = 0; mt < kMt; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc_o[mt][r] *= factor;
        }
    };
    // One pipeline step: the logits of tile `tile` (buffer kb); then, when with_pv, the output
    // update with the previous tile's values (buffer vb), issued just before the barrier of the
    // logit exchange so that the matrix cores work through it while the waves compute the
    // softmax (a barrier does not wait for them); then the softmax, which leaves the weights
    // for the next step's output update in pb / factor / rescale.
    auto step = [&](int tile, const lds_char *kb, const lds_char *vb, bool with_pv) {
        // logits: S^T rows are tokens (two 16-token halves), columns the pair's 16 heads; this
        // wave sums its k-steps, the partner's come through LDS
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
            const int off = qk_base + 128 * ks;
            const u32x4 k0 = *(const lds_u32x4 *)(kb + off);
            const u32x4 k1 = *(const lds_u32x4 *)(kb + off + kHalfTileBytes);
            s0 = mfma16x16x32(k0, qb[ks], s0);
            s1 = mfma16x16x32(k1, qb[ks], s1);
        }
        sm.sx[wave][0][lane] = s0;
        sm.sx[wave][1][lane] = s1;
        if (with_pv) {
            apply_rescale();
#pragma unroll
            for (int mt = 0; mt < kMt; ++mt) pv(vb, mt);
        }
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
        const int4 sa = *reinterpret_cast<const int4 *>(&sm.sel[tile * kTile + 4 * g]);
        const int4 sb = *reinterpret_cast<const int4 *>(&sm.sel[tile * kTile + 16 + 4 * g]);
        const int sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
        float z[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            z[r] = sv[r] >= 0 ? s0[r] * a.scale_log2 : -INFINITY;
            z[4 + r] = sv[4 + r] >= 0 ? s1[r] * a.scale_log2 : -INFINITY;
        }
        float mx = z[0];
#pragma unroll
        for (int r = 1; r < 8; ++r) mx = fmaxf(mx, z[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // The reference max m_run only moves when the tile's max exceeds it by more than 2^8
        // (so the weights below stay under 256): the output and sum are kept relative to m_run,
        // and most tiles then need no rescaling at all.  Both waves of a pair hold the same
        // logits, so they move it together.
        const bool move = mx > m_run + kLazy;
        const float m_new = move ? mx : m_run;
        factor = move ? exp2_hw(m_run - m_new) : 1.f;   // 0 when m_run is -inf
        float p[8];
        if (m_new == -INFINITY) {
#pragma unroll
            for (int r = 0; r < 8; ++r) p[r] = 0.f;
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) p[r] = exp2_hw(z[r] - m_new);
        }
        m_run = m_new;
        rescale = __ballot(move) != 0;
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) ps += p[r];
        l_run = l_run * factor + ps;
        // P^T as the B operand: k slots 8 g .. 8 g + 7 are the lane's 8 tokens, and the V^T
        // operand holds the same tokens (4 g .. 4 g + 3 and 16 + 4 g .. + 3)
        pb = u32x4{bf16_pair(p[0], p[1]), bf16_pair(p[2], p[3]), bf16_pair(p[4], p[5]), bf16_pair(p[6], p[7])};
    };

    // Tiles 0 and 1 are loaded ahead, tile 2 during step 0, and tile t + 1 (t >= 2) during step
    // t, into the buffer of tile t - 2, whose values step t - 1 consumed.  So when step t
    // begins, the loads of tile t + 1 are still in flight only for t <= 1.
    if (ntile > 0) load_tile(0, 0);
    if (ntile > 1) load_tile(1, kTileBytes);
    {   // the queries, their latency under that of the first tiles' loads
        const uint16_t *qh = a.q + (t * kMlaHeads + 16 * hg + l16) * (int64_t)kKv + 32 * half + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) qb[ks] = *reinterpret_cast<const u32x4 *>(qh + 64 * ks);
        // use them here, so that the compiler waits for these loads before the tile loop rather
        // than inside it, where its count of loads in flight would not include the tiles' (the
        // wait drains the tiles' loads issued before them too: the first tile needs them anyway)
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) asm volatile("" ::"v"(qb[ks]));
    }
    // byte offsets of the current and previous tiles' buffers, kept in scalar registers
    // (computing them from the tile index costs vector instructions on every operand address)
    int cur_off = 0, prev_off = 0;
#pragma unroll 1
    for (int tile = 0; tile < ntile; ++tile) {
        if (tile + 1 < ntile && tile <= 1)
            asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // every wave's loads of this tile have landed, and every wave is done with step
        // tile - 1, i.e. with the values of tile - 2
        lds_barrier();
        const int next_off = cur_off == (kBufs - 1) * kTileBytes ? 0 : cur_off + kTileBytes;
        if (tile == 0) {
            if (ntile > 2) load_tile(2, 2 * kTileBytes);
        } else if (tile >= 2 && tile + 1 < ntile) {
            load_tile(tile + 1, next_off);
        }
        const lds_char *kb = lds_k + __builtin_amdgcn_readfirstlane(cur_off);
        const lds_char *vb = lds_k + __builtin_amdgcn_readfirstlane(prev_off);
        step(tile, kb, vb, tile > 0);
        prev_off = cur_off;
        cur_off = next_off;
    }
    if (ntile > 0) {   // the last tile's values
        const lds_char *vb = lds_k + __builtin_amdgcn_readfirstlane(prev_off);
        apply_rescale();
#pragma unroll
        for (int mt = 0; mt < kMt; ++mt) pv(vb, mt);
    }

    // the head's sum over its 4 lane groups
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int head = 16 * hg + l16;
    if (a.nsplit == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t *oh = a.o + (t * kMlaHeads + head) * (int64_t)kV + 16 * half + 4 * g;
#pragma unroll
        for (int mt = 0; mt < kMt; ++mt) {
            const f32x4 o = acc_o[mt];
            const uint2 v = {bf16_pair(o[0] * inv, o[1] * inv), bf16_pair(o[2] * inv, o[3] * inv)};
            *reinterpret_cast<uint2 *>(oh + 32 * mt) = v;
        }
        if (a.lse && g == 0 && half == 0)
            a.lse[t * kMlaHeads + head] = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    } else {
        const int64_t ph = ((int64_t)split * a.T + t) * kMlaHeads + head;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t *oh = a.part_o + ph * kV + 16 * half + 4 * g;
#pragma unroll
        for (int mt = 0; mt < kMt; ++mt) {
            const f32x4 o = acc_o[mt];
            const uint2 v = {bf16_pair(o[0] * inv, o[1] * inv), bf16_pair(o[2] * inv, o[3] * inv)};
            *reinterpret_cast<uint2 *>(oh + 32 * mt) = v;
        }
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
            // the split's normalised output weighs by its share of the sum, f * l_s
            const float fl = f * a.part_ml[2 * ph + 1];
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
    hipLaunchKernelGGL(sparse_mla_kernel, dim3(a.nsplit, (unsigned)T), dim3(kMlaThreads), smem, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    hipLaunchKernelGGL(sparse_mla_merge_kernel, dim3((unsigned)((T * kMlaHeads + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
