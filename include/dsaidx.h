/*
 * libdsaidx -- forward pass of a DSA lightning indexer on AMD MI355X (gfx950).
 *
 * The operation is the one fixed on the archdiff.com compare page "Qwen3.5-397B-A17B vs
 * Kimi K3.1 Pro" (component table, sparse/compressed-attention row, Kimi K3.1 Pro cell):
 * each MLA layer has an indexer with H = 32, D = 128: q = c_q W_q (W_q [1536][4096]),
 * k = LayerNorm(x W_k) (W_k [7168][128], one key vector per token for all heads) and
 * w = x W_w (W_w [7168][32]); the score of key token s for query token t is
 *
 *         I[t,s] = sum_h w[t,h] * ReLU( q[t,h,:] . k[s,:] ),
 *
 * and each query keeps the 2,048 tokens with the largest scores, which become the only
 * keys its MLA attends (gated-MLA row of the same table).  The key LayerNorm is named in
 * the QK-norm row; the indexer applies no rotary embedding ("Kimi K3.1 Pro vs Gemma 4 31B"
 * page, RoPE row) and every key s <= t is scored (same page, long-context row).  Serving
 * engines cache the indexer keys across decode steps ("Kimi K3.1 Pro vs GLM-5" page,
 * low-precision row); dsa_idx_decode scores against such a cache.
 *
 * Readings taken where the pages say nothing (fixed here, identical in the oracle):
 *   - causal prefix s <= t: a query scores itself;
 *   - a query with fewer than topk causal tokens keeps all t+1 of them; unused output
 *     slots hold index -1 and score -inf;
 *   - equal scores are broken toward the lower token index (-0 and +0 are equal);
 *   - selected indices are listed in ascending order;
 *   - no score scale, no projection biases, w has no activation (may be negative);
 *   - LayerNorm = mean-centred, biased variance over the 128 key dims, eps from the
 *     caller, gain and bias, applied before rounding k to bf16;
 *   - q, k and w are stored as bf16 (round to nearest even from the fp32 accumulators);
 *     scores are computed in fp32;
 *   - q is head-major: head h is columns [128h, 128h + 128) of the 4,096.
 *
 * Conventions of every entry point:
 *   - Tensor pointers are DEVICE pointers unless stated; bf16 is passed as uint16_t bit
 *     patterns.  Rows are contiguous (row-major) unless a leading dimension is given.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are asynchronous:
 *     they enqueue kernels and return; they never synchronize.  The caller keeps every
 *     buffer alive until the stream work completes.
 *   - The library allocates no device memory and keeps no pointer after returning.
 *     Scratch memory is the caller's workspace `ws` of `ws_bytes` bytes, sized with
 *     dsa_idx_workspace_size(); it must not be shared by calls that may overlap.
 *   - Status: DSA_IDX_OK (0) or a negative code below; on error nothing is launched and
 *     outputs are untouched, and dsa_idx_last_error() returns a message (thread-local).
 *   - Identical inputs give bitwise-identical outputs (no floating-point atomics).
 *   - The device must be gfx950 (checked once per device).
 */
#ifndef DSAIDX_H
#define DSAIDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_IDX_HEADS 32     /* indexer heads */
#define DSA_IDX_DIM 128      /* dims per head, and the shared key width */
#define DSA_IDX_QLAT 1536    /* query latent width (input of the q projection) */
#define DSA_IDX_QOUT 4096    /* 32 x 128 */
#define DSA_IDX_HIDDEN 7168  /* hidden width (input of the key and weight projections) */
#define DSA_IDX_MAX_TOPK 2048

/* status codes */
#define DSA_IDX_OK 0
#define DSA_IDX_EINVAL (-1)      /* null pointer, negative size, misalignment, ld too small */
#define DSA_IDX_EUNSUPPORTED (-2)/* topk outside [1, 2048], device not gfx950, size too large */
#define DSA_IDX_EWORKSPACE (-3)  /* ws_bytes below dsa_idx_workspace_size() */
#define DSA_IDX_EHIP (-4)        /* a HIP runtime call failed (message names it) */
#define DSA_IDX_ESTALL (-5)      /* dsa_idx_workspace_status: a score kernel's ring wait gave up */

/* operations for dsa_idx_workspace_size */
#define DSA_IDX_OP_PROJECT 0
#define DSA_IDX_OP_SCORE_TOPK 1
#define DSA_IDX_OP_SCORE_TOPK_VARLEN 2
#define DSA_IDX_OP_DECODE 3
#define DSA_IDX_OP_DECODE_FP8 4
#define DSA_IDX_OP_PREFILL_CHUNK 5
#define DSA_IDX_OP_SPARSE_MLA 6
#define DSA_IDX_OP_V32_PROJECT 7
#define DSA_IDX_OP_V32_SCORE_TOPK 8
#define DSA_IDX_OP_V32_SCORE_TOPK_VARLEN 9
#define DSA_IDX_OP_V32_PREFILL_CHUNK 10
#define DSA_IDX_OP_PREFILL_ROWS 11   /* dsa_idx_prefill_scores / dsa_idx_prefill_select */

typedef uint16_t dsa_idx_bf16;

/* One layer's indexer weights (device pointers, borrowed for the call).  The 24 MLA layers
 * have 24 separate sets; no layer reuses another's selection (sparse/compressed-attention
 * row). */
typedef struct {
    const dsa_idx_bf16 *W_q;      /* [1536][4096] row-major: q = c_q . W_q            */
    const dsa_idx_bf16 *W_k;      /* [7168][128]  row-major: k = LN(x . W_k)           */
    const dsa_idx_bf16 *W_w;      /* [7168][32]   row-major: w = x . W_w               */
    const dsa_idx_bf16 *ln_gamma; /* [128] LayerNorm gain on the key                   */
    const dsa_idx_bf16 *ln_beta;  /* [128] LayerNorm bias on the key                   */
    float ln_eps;                 /* LayerNorm epsilon (> 0)                           */
} dsa_idx_weights;

/* Library version string (static storage). */
const char *dsa_idx_version(void);

/* Message of the last non-OK status returned on the calling thread ("" if none). */
const char *dsa_idx_last_error(void);

/* Whether the library's kernels run on a device whose architecture name (hipDeviceProp_t::
 * gcnArchName, e.g. "gfx950:sramecc+:xnack-") is arch_name: DSA_IDX_OK for gfx950 with any
 * feature suffix, DSA_IDX_EUNSUPPORTED (with a message) for any other name, DSA_IDX_EINVAL for a
 * null pointer.  Host-only; every entry point that launches work applies this check to the
 * current device (once per device) and returns its status. */
int dsa_idx_arch_supported(const char *arch_name);

/* Bytes of workspace an operation needs (host-only, no device access).
 *   op               one of DSA_IDX_OP_*
 *   total_tokens     T for PROJECT, SCORE_TOPK, SPARSE_MLA, V32_PROJECT and V32_SCORE_TOPK;
 *                    the packed token count for the VARLEN ops and PREFILL_ROWS; the chunk's
 *                    query count C for the PREFILL_CHUNK ops
 *   B                number of sequences (VARLEN ops, DECODE ops; PREFILL_ROWS: 0 for one
 *                    sequence of total_tokens tokens); ignored otherwise
 *   max_seqlen       longest sequence (VARLEN ops, PREFILL_ROWS with B > 0), keys of the
 *                    longest cache for the DECODE ops; the cached prefix length for the
 *                    PREFILL_CHUNK ops
 *   topk             tokens kept (selected, for SPARSE_MLA) per query, 1..2048; ignored
 *                    for PROJECT and V32_PROJECT
 * Writes *bytes (0 is a valid answer).  Returns a status. */
int dsa_idx_workspace_size(int op, int64_t total_tokens, int B, int max_seqlen, int topk,
                           size_t *bytes);

/* Projections of one indexer layer for T tokens (sparse-attention row; key LayerNorm
 * from the QK-norm row):
 *   q[t]  = bf16( c_q[t] . W_q )                   q    [T][4096]  (= [T][32][128])
 *   k     = bf16( LayerNorm( x[t] . W_k ) )        row k_slot[t] (or t when k_slot is
 *                                                  NULL) of k_base, rows of 128
 *   w[t]  = bf16( x[t] . W_w )                     w    [T][32]
 * x is [T][ldx] (ldx >= 7168), c_q is [T][ldc] (ldc >= 1536); ldx and ldc are in
 * elements and must be multiples of 8; x, c_q, q, k_base, w must be 16-byte aligned.
 * k_slot (device, int64 [T], may be NULL) scatters the keys into a cache (decode).
 * Needs dsa_idx_workspace_size(DSA_IDX_OP_PROJECT, T, ...) bytes of workspace. */
int dsa_idx_project(const dsa_idx_weights *weights, const dsa_idx_bf16 *x, int64_t ldx,
                    const dsa_idx_bf16 *c_q, int64_t ldc, int64_t T, dsa_idx_bf16 *q,
                    dsa_idx_bf16 *k_base, const int64_t *k_slot, dsa_idx_bf16 *w, void *ws,
                    size_t ws_bytes, void *stream);

/* Causal scores and top-k of one sequence of T tokens (sparse-attention row: score
 * formula and top-2,048; long-context row: whole prefix scored):
 *   q [T][32][128], k [T][128], w [T][32]   bf16, 16-byte aligned
 *   idx    [T][topk] int32  selected key positions s <= t, ascending, -1 padded
 *   scores [T][topk] fp32   I[t, idx] (may be NULL), -inf padded
 * No T x T score matrix is stored: each row first scores one key per 32-key stratum to place
 * a threshold, the full causal score stream then keeps only the (score, index) pairs at or
 * above it, and the top-k is selected exactly from those; a row the threshold cannot decide
 * (too few or too many kept keys) is scored again in full into a bounded scratch row.  The
 * result equals the full sort of each row whatever the data.  The workspace
 * (DSA_IDX_OP_SCORE_TOPK) grows linearly in T: about 3.8 GB at T = 65,536, 4.3 GB at
 * T = 1,048,576.  Its first 32-bit word is the status that dsa_idx_workspace_status() reads.
 * Limit: T <= 16,777,216. */
int dsa_idx_score_topk(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                       int64_t T, int topk, int32_t *idx, float *scores, void *ws,
                       size_t ws_bytes, void *stream);

/* Ragged (varlen) form: B sequences packed back to back.  cu_seqlens (device, int32
 * [B+1], non-decreasing, cu_seqlens[0] = 0, cu_seqlens[B] = total) delimits them;
 * max_seqlen bounds every length.  Scoring is causal inside each sequence and never
 * crosses sequences; returned indices are relative to the sequence start.  q, k, w,
 * idx and scores are the packed [total][...] arrays of dsa_idx_score_topk.
 * A ragged prefill batch runs this call once per MLA layer: each of the 24 MLA layers has an
 * indexer of its own, with its own weights, and no layer reuses another's selection
 * ("Qwen3.5-397B-A17B vs Kimi K3.1 Pro" compare page, component table, sparse/compressed-
 * attention and gated-MLA rows). */
int dsa_idx_score_topk_varlen(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k,
                              const dsa_idx_bf16 *w, const int32_t *cu_seqlens, int B,
                              int max_seqlen, int64_t total, int topk, int32_t *idx,
                              float *scores, void *ws, size_t ws_bytes, void *stream);

/* The causal score rows themselves (32 heads), for callers that want the scores I[t, s] of
 * every key, and a row top-k over them.  cu_seqlens == NULL: one sequence of `total` tokens
 * (B and max_seqlen ignored); else a ragged batch as dsa_idx_score_topk_varlen.  These two
 * calls DO store every causal score: their workspace (DSA_IDX_OP_PREFILL_ROWS) is about
 * 2 total^2 bytes for one sequence (8.6 GB at 65,536 tokens), so they suit inspection and
 * moderate lengths; dsa_idx_score_topk does not need them.
 *
 * dsa_idx_prefill_scores writes into ws: a 256-byte header whose first word is the status
 * (see dsa_idx_workspace_status); B' + 1 int64 (B' = 1 without cu_seqlens, else B) at byte
 * 256, the sequences' float offsets into the row area, padded to H = 256 + 256 *
 * ceil(8 (B' + 1) / 256) bytes; a scratch row of 4 * 128 * ceil(max_len / 128) bytes (rounded
 * up to 256; max_len = total or max_seqlen); then the row area: row t of sequence i starts at
 * float offset
 *     base[i] + 8192 q (q + 1) + 128 r (q + 1),   q = t / 128, r = t % 128,
 * and holds 128 (q + 1) floats, of which the first t + 1 are the scores (the rest are
 * unspecified).
 * dsa_idx_prefill_select reads those rows and writes idx and scores as dsa_idx_score_topk
 * (every row index -2 and score NaN if the status word says the scoring kernel gave up). */
int dsa_idx_prefill_scores(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                           const int32_t *cu_seqlens, int B, int max_seqlen, int64_t total,
                           void *ws, size_t ws_bytes, void *stream);
int dsa_idx_prefill_select(const int32_t *cu_seqlens, int B, int max_seqlen, int64_t total,
                           int topk, int32_t *idx, float *scores, void *ws, size_t ws_bytes,
                           void *stream);

/* Chunked prefill: C new query tokens of one sequence, at positions prefix .. prefix + C - 1,
 * against the whole causal prefix, the long-context mode in which the indexer scores every
 * earlier token of the window ("Kimi K3.1 Pro vs Gemma 4 31B" page, long-context row: a
 * 1,048,576-token window, all of it scored).  Query i scores keys 0 .. prefix + i:
 *   q [C][32][128], w [C][32]      the chunk's projections
 *   k [prefix + C][128]            keys of positions 0 .. prefix + C - 1: the cached prefix
 *                                  followed by the chunk's own keys
 *   idx [C][topk], scores [C][topk] (may be NULL): row i as prefill row prefix + i of
 *                                  dsa_idx_score_topk (absolute positions, ascending,
 *                                  -1 / -inf padded)
 * prefix = 0 is dsa_idx_score_topk, and the method and workspace are that call's: the
 * workspace (DSA_IDX_OP_PREFILL_CHUNK, total_tokens = C, max_seqlen = prefix) is linear in C
 * and in prefix + C (4.3 GB for the last 4,096 queries of a 1,048,576-token window).
 * Limit: prefix + C <= 16,777,216. */
int dsa_idx_prefill_chunk(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                          int64_t C, int64_t prefix, int topk, int32_t *idx, float *scores,
                          void *ws, size_t ws_bytes, void *stream);

/* Decode: one new query per sequence against that sequence's cached keys.
 *   q [B][32][128], w [B][32]      the new tokens' projections (from dsa_idx_project)
 *   k_cache [*][128]               cache rows; sequence b owns rows
 *                                  [start[b], start[b] + seqlens[b]), whose last row is
 *                                  the new token's own key (written by dsa_idx_project
 *                                  through k_slot)
 *   start   (device, int64 [B]), seqlens (device, int32 [B], 1 <= seqlens[b] <= max_seqlen),
 *   max_seqlen <= 16,777,216
 *   idx [B][topk], scores [B][topk] (may be NULL): as for prefill row seqlens[b] - 1,
 *   indices relative to start[b].
 * The cached keys are the per-layer indexer keys that serving engines keep across steps. */
int dsa_idx_decode(const dsa_idx_bf16 *q, const dsa_idx_bf16 *w, const dsa_idx_bf16 *k_cache,
                   const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                   int topk, int32_t *idx, float *scores, void *ws, size_t ws_bytes,
                   void *stream);

/* dsa_idx_decode without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Its
 * scratch is a static array of DSA_IDX_DECODE_NOALLOC_SCRATCH bytes inside the library, one
 * copy per device (held until the process ends); the call allocates nothing and otherwise
 * behaves as dsa_idx_decode (same kernels, same results).  A (B, max_seqlen) whose decode
 * workspace exceeds the array is rejected with DSA_IDX_EUNSUPPORTED (64 sequences of up to
 * 131,072 cached keys fit).  Every call on one device shares that device's array: calls that
 * may overlap on one device (several streams, several host threads) race and must be
 * serialized by the caller. */
#define DSA_IDX_DECODE_NOALLOC_SCRATCH (128u << 20)
int dsa_idx_decode_noalloc(const dsa_idx_bf16 *q, const dsa_idx_bf16 *w, const dsa_idx_bf16 *k_cache,
                           const int64_t *start, const int32_t *seqlens, int B, int max_seqlen, int topk,
                           int32_t *idx, float *scores, void *stream);

/* ---- FP8 key cache ("Kimi K3.1 Pro vs GLM-5" page, low-precision row: the serving engines
 * cache the indexer keys in FP8; the pages give no format or scale).  Format of this library:
 * a cached key is 128 OCP E4M3 codes (bias 7, largest finite value 448, no infinities; one
 * byte per dimension, k8 [*][128]) and one fp32 scale k_scale[*] = 2^e, the smallest power of
 * two with max_j |k_j| <= 448 * 2^e; code_j = E4M3(k_j / 2^e) rounded to nearest even (the
 * division is exact, so this is the only rounding).  Dequantised: k_j ~ 2^e * E4M3 value. */

/* Quantises N bf16 keys k [N][ldk] (ldk >= 128, a multiple of 8; k 16-byte aligned) into cache
 * rows slot[i] (device int64 [N]; NULL: row i) of k8 (16-byte aligned) and k_scale.
 * Asynchronous on `stream`; no workspace. */
int dsa_idx_quantize_keys(const dsa_idx_bf16 *k, int64_t ldk, int64_t N, const int64_t *slot,
                          uint8_t *k8, float *k_scale, void *stream);

/* Decode against an FP8 cache: as dsa_idx_decode, with the cached keys given as k8 / k_scale
 * rows [start[b], start[b] + seqlens[b]).  The new queries are quantised the same way, one
 * scale per head (q_h ~ 2^eq_h * E4M3 codes), and
 *   scores[b][j] = I[s] = 2^e_s * sum_h w[b][h] 2^eq_h max(0, sum_d E4M3(q_h)[d] E4M3(k_s)[d]),
 * the indexer formula on the dequantised vectors, in fp32 (the E4M3 products are exact).
 * Needs dsa_idx_workspace_size(DSA_IDX_OP_DECODE_FP8, 0, B, max_seqlen, topk) bytes. */
int dsa_idx_decode_fp8(const dsa_idx_bf16 *q, const dsa_idx_bf16 *w, const uint8_t *k8,
                       const float *k_scale, const int64_t *start, const int32_t *seqlens, int B,
                       int max_seqlen, int topk, int32_t *idx, float *scores, void *ws,
                       size_t ws_bytes, void *stream);

/* ---- The consumer of the selection: sparse MLA over the selected tokens ("Qwen3.5-397B-A17B
 * vs Kimi K3.1 Pro" page, gated-MLA row: H = 96; a cache row of 512 latent + 64 position-key
 * values = 576 per token; q/k head dim 192, v head dim 128; query t attends to the <= 2,048
 * rows picked for it; no rotary step, RoPE row of the "Kimi K3.1 Pro vs Gemma 4 31B" page).  Queries come in the absorbed
 * latent form (the key up-projection folded into each head's 128 no-position dims, its 64
 * key-slot dims as they are), so for query t and head h over its valid selections j:
 *   z_j = scale * q[t][h] . kv[row0[t] + idx[t][j]]                (576 values)
 *   o[t][h] = sum_j exp(z_j - m) kv[row_j][0:512] / sum_j exp(z_j - m),   m = max_j z_j
 *   lse[t][h] = m + ln(sum_j exp(z_j - m))
 * The value up-projection, the output gate and the output projection that follow are dense
 * products and not part of this call.
 *   q [T][96][576] bf16, kv [*][576] bf16 (16-byte aligned; row 0 must exist: it stands in
 *   for empty slots), idx [T][topk] int32 (-1: no token), row0 (device int64 [T], or NULL for
 *   0), scale > 0 (the pages' q/k head dim 192 gives 1/sqrt(192)),
 *   o [T][96][512] bf16 (rounded to nearest even), lse [T][96] fp32 natural log (may be NULL).
 * A query with no valid selection gets o = 0 and lse = -inf.  Logits and the softmax are fp32;
 * the probabilities enter the weighted sum rounded to bf16.
 * Needs dsa_idx_workspace_size(DSA_IDX_OP_SPARSE_MLA, T, 0, 0, topk) bytes. */
int dsa_idx_sparse_mla(const dsa_idx_bf16 *q, const dsa_idx_bf16 *kv, const int32_t *idx,
                       const int64_t *row0, int64_t T, int topk, float scale, dsa_idx_bf16 *o,
                       float *lse, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- 64-head indexer
 * The DeepSeek-V3.2-shaped indexer: 64 heads ("Qwen3.5-397B-A17B vs Kimi K3.1 Pro" page,
 * sparse-attention row) with a rotary step on 64 of the 128 dims (RoPE row of the "Kimi K3.1
 * Pro vs Gemma 4 31B" page), otherwise the indexer above: q from the 1,536-dim query latent
 * (1,536 -> 8,192 = 64 heads x 128), one LayerNorm key from the hidden state, head weights
 * 7,168 -> 64, I = sum over the 64 heads of w_h ReLU(q_h . k), top-k per query.
 * The rotary step (this library's reading): dims (2i, 2i+1), i < 32, of every query head and
 * of the key (after its LayerNorm) turn by the angle pos * rope_theta^(-2i/64), applied to the
 * fp32 projections, and each result is rounded to bf16 (nearest even) once; dims 64..127 do
 * not turn. */
#define DSA_IDX_V32_HEADS 64
#define DSA_IDX_V32_QOUT 8192

/* Projections and rotary step of T tokens at positions pos0 .. pos0 + T - 1.
 *   wt: W_q [1536][8192], W_k [7168][128], W_w [7168][64] (row-major), LayerNorm gamma,
 *       beta [128], ln_eps > 0; x [T][ldx], c_q [T][ldc] as for dsa_idx_project;
 *   pos0 >= 0, rope_theta > 0 (10000 in the oracle's reading);
 *   q [T][64][128], k [T][128], w [T][64] bf16 out (16-byte aligned).
 * One pass: x is read once for the key and all 64 head weights, and the rotary step runs in
 * the projection epilogues from a (cos, sin) table the call forms first in the workspace.
 * Needs dsa_idx_workspace_size(DSA_IDX_OP_V32_PROJECT, T, ...) bytes of workspace: W_q
 * transposed (25.2 MB) for T > 64 (fp32 split-K partial sums of q for T <= 64), the key /
 * head-weight split-K partial sums for T <= 32,768, then 256 B per token for the table. */
int dsa_idx_v32_project(const dsa_idx_weights *wt, const dsa_idx_bf16 *x, int64_t ldx,
                        const dsa_idx_bf16 *c_q, int64_t ldc, int64_t T, int64_t pos0, float rope_theta,
                        dsa_idx_bf16 *q, dsa_idx_bf16 *k, dsa_idx_bf16 *w, void *ws, size_t ws_bytes,
                        void *stream);

/* Causal scores and top-k of one sequence for the 64-head indexer: as dsa_idx_score_topk,
 * with q [T][64][128] and w [T][64] (the keys [T][128] as before); all 64 heads are summed in
 * one pass (fp32).  Needs dsa_idx_workspace_size(DSA_IDX_OP_V32_SCORE_TOPK, T, 0, 0, topk)
 * bytes. */
int dsa_idx_v32_score_topk(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                           int64_t T, int topk, int32_t *idx, float *scores, void *ws,
                           size_t ws_bytes, void *stream);

/* Ragged prefill for the 64-head indexer: as dsa_idx_score_topk_varlen, with q [total][64][128]
 * and w [total][64].  The rotary positions are each token's position in its own sequence, so
 * project each sequence with its own pos0 (dsa_idx_v32_project).
 * Needs dsa_idx_workspace_size(DSA_IDX_OP_V32_SCORE_TOPK_VARLEN, total, B, max_seqlen, topk)
 * bytes. */
int dsa_idx_v32_score_topk_varlen(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k,
                                  const dsa_idx_bf16 *w, const int32_t *cu_seqlens, int B,
                                  int max_seqlen, int64_t total, int topk, int32_t *idx,
                                  float *scores, void *ws, size_t ws_bytes, void *stream);

/* Chunked prefill for the 64-head indexer: as dsa_idx_prefill_chunk, with q [C][64][128] and
 * w [C][64] (the queries' rotary positions prefix .. prefix + C - 1: project the chunk with
 * pos0 = prefix).  Needs dsa_idx_workspace_size(DSA_IDX_OP_V32_PREFILL_CHUNK, C, 0, prefix, topk)
 * bytes. */
int dsa_idx_v32_prefill_chunk(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                              int64_t C, int64_t prefix, int topk, int32_t *idx, float *scores,
                              void *ws, size_t ws_bytes, void *stream);

/* Decode for the 64-head indexer: as dsa_idx_decode, with q [B][64][128] and w [B][64] (the
 * new tokens' projections at their positions seqlens[b] - 1, from dsa_idx_v32_project, and
 * their rotated keys in the cache).  Needs dsa_idx_workspace_size(DSA_IDX_OP_DECODE, 0, B,
 * max_seqlen, topk) bytes. */
int dsa_idx_v32_decode(const dsa_idx_bf16 *q, const dsa_idx_bf16 *w, const dsa_idx_bf16 *k_cache,
                       const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                       int topk, int32_t *idx, float *scores, void *ws, size_t ws_bytes,
                       void *stream);

/* Decode for the 64-head indexer against the FP8 key cache: as dsa_idx_decode_fp8, with
 * q [B][64][128] and w [B][64] (each head quantised with its own power-of-two scale).  Needs
 * dsa_idx_workspace_size(DSA_IDX_OP_DECODE_FP8, 0, B, max_seqlen, topk) bytes. */
int dsa_idx_v32_decode_fp8(const dsa_idx_bf16 *q, const dsa_idx_bf16 *w, const uint8_t *k8,
                           const float *k_scale, const int64_t *start, const int32_t *seqlens, int B,
                           int max_seqlen, int topk, int32_t *idx, float *scores, void *ws,
                           size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- run-time checks
 * The prefill score kernels order their key ring with per-wave progress counters; every wait
 * on them is bounded (2^20 polls by default).  A wait that runs out of polls (which a correct
 * kernel never does) lets the kernel finish, sets bit 0 of the first 32-bit word of the
 * workspace, and the call's outputs become index -2, score NaN.
 *
 * dsa_idx_workspace_status reads that word after the work queued on `stream` so far: it
 * SYNCHRONIZES the stream, then returns DSA_IDX_OK, or DSA_IDX_ESTALL with a message.  Valid
 * on the workspaces of the prefill top-k ops (SCORE_TOPK, the VARLEN and PREFILL_CHUNK ops and
 * their V32 forms) and of PREFILL_ROWS. */
int dsa_idx_workspace_status(const void *ws, size_t ws_bytes, void *stream);

/* Diagnostic: sets the polls allowed per ring wait of the prefill score kernels for calls
 * launched afterwards (process-wide; values < 0 read as 0, and 0 makes every wait that is not
 * already satisfied give up at once).  Returns the previous value.  For tests of the status
 * report; the default needs no change. */
int dsa_idx_set_wait_budget(int polls);

/* Diagnostic phase timing of the prefill top-k calls (process-wide, off by default).  While it
 * is on, each phase launch of a call is bracketed by two HIP events on the call's stream:
 *   0 sample scores, 1 thresholds, 2 score and filter pass, 3 select, 4 fallback.
 * dsa_idx_phase_timing(1) switches it on and forgets older records, (0) switches it off.
 * dsa_idx_phase_times(ms, count, n) SYNCHRONIZES on the recorded events, writes the summed
 * milliseconds and the number of launches of phases 0 .. n - 1, and forgets the records. */
int dsa_idx_phase_timing(int enable);
int dsa_idx_phase_times(double *ms, int *count, int n);

/* Calibration (not part of the indexer; for measurement only): the sustained bf16 matrix-core
 * rate of the device, against which the score pass and the projections are measured beside the
 * published peak of 2,516.6 TFLOP/s (which assumes the top clock).  Launches, on `stream`, 1,024
 * workgroups of 4 waves; each wave runs `iters` rounds of 16 independent v_mfma_f32_16x16x32_bf16
 * products on register operands (no memory traffic): zero operands (random_operands = 0) or
 * bf16 values with random signs and mantissas in [0.5, 2) in magnitude (1), since the matrix
 * cores' power, and hence the clock, depends on the data.  Each thread writes the sum of its
 * accumulators to sink[thread] (device memory, at least DSA_IDX_CALIB_SINK floats; its values
 * have no meaning beyond keeping the work).  *flop (host) receives the bf16 flop the launch
 * executes: 1,024 x 4 x iters x 16 x 16,384.  Asynchronous; the caller times it with events.
 * iters in [1, 2^32]. */
#define DSA_IDX_CALIB_SINK 262144
int dsa_idx_mfma_calibrate(int64_t iters, int random_operands, float *sink, size_t sink_floats, int64_t *flop,
                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSAIDX_H */
