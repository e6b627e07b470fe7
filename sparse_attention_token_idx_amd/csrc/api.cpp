// C-ABI of libdsaidx: argument validation, workspace sizing, device check, error state and
// dispatch to the HIP kernels.  The contract of every entry point is documented in
// include/dsaidx.h.  Validation runs entirely on the host before any HIP call, so a
// rejected call touches neither the device nor the outputs.
#include "../../include/dsaidx.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() { return DSA_IDX_OK; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_fail(const char *what, hipError_t e) {
    return fail(DSA_IDX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// gfx950 check, cached per device.
int check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    static std::mutex mu;
    static int state[64] = {0};   // 0 unknown, 1 ok, 2 unsupported
    if (dev < 0 || dev >= 64) return fail(DSA_IDX_EUNSUPPORTED, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lk(mu);
    if (state[dev] == 0) {
        hipDeviceProp_t p;
        e = hipGetDeviceProperties(&p, dev);
        if (e != hipSuccess) return hip_fail("hipGetDeviceProperties", e);
        state[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (state[dev] == 2)
            return fail(DSA_IDX_EUNSUPPORTED, "device %d is %s; libdsaidx runs on gfx950 only", dev,
                        p.gcnArchName);
    }
    if (state[dev] == 2) return fail(DSA_IDX_EUNSUPPORTED, "device %d is not gfx950", dev);
    return ok();
}

int check_topk(int topk) {
    if (topk < 1 || topk > DSA_IDX_MAX_TOPK)
        return fail(DSA_IDX_EUNSUPPORTED, "topk=%d outside [1, %d]", topk, DSA_IDX_MAX_TOPK);
    return ok();
}

// Longest sequence the prefill grid can address (row blocks of 32 on grid.y).
constexpr int64_t kMaxSeq = 65535LL * 32;

// Prefill workspace: [sequence bases: int64 x (B + 1)] [dummy row] [triangular score rows],
// each part a multiple of 256 bytes.
size_t round256(size_t b) { return (b + 255u) & ~(size_t)255u; }
size_t ws_hdr(int B) { return round256(8u * (size_t)(B + 1)); }
size_t ws_dummy(int64_t max_len) {
    const int64_t q = dsaidx::kRowQuant;
    return round256(4u * (size_t)(((max_len + q - 1) / q) * q));
}

// Score floats of a ragged batch: sequence i needs tri_row_offset(L_i) <= (L_i + Q)^2 / 2
// floats (Q = kRowQuant), and with sum L_i = total, L_i <= max_len and at most B sequences
// that sum of squares is largest when as many sequences as possible have max_len.
int64_t varlen_score_floats(int64_t total, int B, int64_t max_len) {
    if (total == 0 || B == 0 || max_len == 0) return 0;
    int64_t k = total / max_len;
    if (k > B) k = B;
    const int64_t rem = total - k * max_len;
    const int64_t Q = dsaidx::kRowQuant;
    const int64_t u = max_len + Q;
    int64_t sq = k * u * u;
    if (k < B) sq += (rem + Q) * (rem + Q) + (int64_t)(B - k - 1) * Q * Q;
    return ((sq / 2 + Q - 1) / Q) * Q;
}

size_t ws_score_topk(int64_t T) {
    return ws_hdr(1) + ws_dummy(T) + 4u * (size_t)dsaidx::tri_row_offset(T);
}
// chunk of C query rows at positions prefix .. prefix + C - 1 of one sequence
size_t ws_prefill_chunk(int64_t C, int64_t prefix) {
    return ws_hdr(1) + ws_dummy(prefix + C) +
           4u * (size_t)(dsaidx::tri_row_offset(prefix + C) - dsaidx::tri_row_offset(prefix));
}
// Longest sequence (prefix + chunk) a chunked prefill call accepts.
constexpr int64_t kMaxWindow = 1LL << 24;
size_t ws_score_topk_varlen(int64_t total, int B, int max_seqlen) {
    return ws_hdr(B) + ws_dummy(max_seqlen) + 4u * (size_t)varlen_score_floats(total, B, max_seqlen);
}

size_t ws_decode(int B, int max_seqlen) { return dsaidx::decode_workspace(B, max_seqlen, false); }
size_t ws_decode_fp8(int B, int max_seqlen) { return dsaidx::decode_workspace(B, max_seqlen, true); }

}  // namespace

extern "C" {

const char *dsa_idx_version(void) { return "libdsaidx 0.1.0 (gfx950)"; }

const char *dsa_idx_last_error(void) { return g_err; }

int dsa_idx_workspace_size(int op, int64_t total_tokens, int B, int max_seqlen, int topk,
                           size_t *bytes) {
    if (!bytes) return fail(DSA_IDX_EINVAL, "bytes is NULL");
    switch (op) {
        case DSA_IDX_OP_PROJECT:
            if (total_tokens < 0) return fail(DSA_IDX_EINVAL, "T=%lld < 0", (long long)total_tokens);
            *bytes = dsaidx::project_workspace(total_tokens);
            return ok();
        case DSA_IDX_OP_SCORE_TOPK: {
            if (total_tokens < 0) return fail(DSA_IDX_EINVAL, "T=%lld < 0", (long long)total_tokens);
            int r = check_topk(topk);
            if (r) return r;
            *bytes = ws_score_topk(total_tokens);
            return ok();
        }
        case DSA_IDX_OP_SCORE_TOPK_VARLEN: {
            if (total_tokens < 0 || B < 0 || max_seqlen < 0)
                return fail(DSA_IDX_EINVAL, "total=%lld B=%d max_seqlen=%d must be >= 0",
                            (long long)total_tokens, B, max_seqlen);
            int r = check_topk(topk);
            if (r) return r;
            *bytes = ws_score_topk_varlen(total_tokens, B, max_seqlen);
            return ok();
        }
        case DSA_IDX_OP_PREFILL_CHUNK: {
            if (total_tokens < 0 || max_seqlen < 0)
                return fail(DSA_IDX_EINVAL, "C=%lld prefix=%d must be >= 0", (long long)total_tokens, max_seqlen);
            int r = check_topk(topk);
            if (r) return r;
            *bytes = total_tokens == 0 ? 0 : ws_prefill_chunk(total_tokens, max_seqlen);
            return ok();
        }
        case DSA_IDX_OP_V32_PROJECT:
            if (total_tokens < 0) return fail(DSA_IDX_EINVAL, "T=%lld < 0", (long long)total_tokens);
            *bytes = dsaidx::project_workspace(total_tokens);   // the halves reuse it in turn
            return ok();
        case DSA_IDX_OP_V32_SCORE_TOPK: {
            if (total_tokens < 0) return fail(DSA_IDX_EINVAL, "T=%lld < 0", (long long)total_tokens);
            int r = check_topk(topk);
            if (r) return r;
            *bytes = ws_score_topk(total_tokens);
            return ok();
        }
        case DSA_IDX_OP_SPARSE_MLA: {
            if (total_tokens < 0) return fail(DSA_IDX_EINVAL, "T=%lld < 0", (long long)total_tokens);
            int r = check_topk(topk);
            if (r) return r;
            *bytes = dsaidx::sparse_mla_workspace(total_tokens, topk);
            return ok();
        }
        case DSA_IDX_OP_DECODE:
        case DSA_IDX_OP_DECODE_FP8: {
            if (B < 0 || max_seqlen < 0) return fail(DSA_IDX_EINVAL, "B=%d max_seqlen=%d", B, max_seqlen);
            int r = check_topk(topk);
            if (r) return r;
            *bytes = op == DSA_IDX_OP_DECODE ? ws_decode(B, max_seqlen) : ws_decode_fp8(B, max_seqlen);
            return ok();
        }
        default:
            return fail(DSA_IDX_EINVAL, "unknown op %d", op);
    }
}

int dsa_idx_project(const dsa_idx_weights *wt, const dsa_idx_bf16 *x, int64_t ldx,
                    const dsa_idx_bf16 *c_q, int64_t ldc, int64_t T, dsa_idx_bf16 *q,
                    dsa_idx_bf16 *k_base, const int64_t *k_slot, dsa_idx_bf16 *w, void *ws,
                    size_t ws_bytes, void *stream) {
    if (!wt) return fail(DSA_IDX_EINVAL, "weights is NULL");
    if (T < 0) return fail(DSA_IDX_EINVAL, "T=%lld < 0", (long long)T);
    if (T == 0) return ok();
    if (!wt->W_q || !wt->W_k || !wt->W_w || !wt->ln_gamma || !wt->ln_beta)
        return fail(DSA_IDX_EINVAL, "a weight pointer is NULL");
    if (!x || !c_q || !q || !k_base || !w) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    if (ldx < DSA_IDX_HIDDEN || ldx % 8) return fail(DSA_IDX_EINVAL, "ldx=%lld must be >= 7168 and a multiple of 8", (long long)ldx);
    if (ldc < DSA_IDX_QLAT || ldc % 8) return fail(DSA_IDX_EINVAL, "ldc=%lld must be >= 1536 and a multiple of 8", (long long)ldc);
    if (!(wt->ln_eps > 0.f)) return fail(DSA_IDX_EINVAL, "ln_eps must be > 0");
    const void *ptrs[] = {x, c_q, q, k_base, w, wt->W_q, wt->W_k, wt->W_w};
    for (const void *p : ptrs)
        if (!aligned16(p)) return fail(DSA_IDX_EINVAL, "tensor pointer %p is not 16-byte aligned", p);
    if (T > (int64_t)INT32_MAX * 128) return fail(DSA_IDX_EUNSUPPORTED, "T=%lld too large", (long long)T);
    const size_t need = dsaidx::project_workspace(T);
    if (need && (!ws || ws_bytes < need))
        return fail(DSA_IDX_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
    if (need && !aligned16(ws)) return fail(DSA_IDX_EINVAL, "workspace must be 16-byte aligned");
    int r = check_device();
    if (r) return r;
    hipError_t e = dsaidx::launch_project(x, ldx, c_q, ldc, T, wt->W_q, wt->W_k, wt->W_w, wt->ln_gamma,
                                          wt->ln_beta, wt->ln_eps, q, k_base, k_slot, w,
                                          static_cast<float *>(ws), reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("project launch", e);
    return ok();
}


// Workspace parts of a prefill call.  cu == nullptr: one sequence of `total` tokens.
struct PrefillWs {
    int64_t *base;
    float *dummy;
    float *rows;
};

static int64_t prefill_max_len(const int32_t *cu, int max_seqlen, int64_t total) {
    return cu ? (int64_t)max_seqlen : total;
}

static int prefill_check(const int32_t *cu, int B, int max_seqlen, int64_t total, void *ws,
                         size_t ws_bytes, size_t &need) {
    if (total < 0) return fail(DSA_IDX_EINVAL, "total=%lld < 0", (long long)total);
    if (cu) {
        if (B < 0 || max_seqlen < 0)
            return fail(DSA_IDX_EINVAL, "B=%d max_seqlen=%d must be >= 0", B, max_seqlen);
        if (B > 65535) return fail(DSA_IDX_EUNSUPPORTED, "B=%d above 65535", B);
        if (max_seqlen > kMaxSeq)
            return fail(DSA_IDX_EUNSUPPORTED, "max_seqlen=%d above %lld", max_seqlen, (long long)kMaxSeq);
        if (total > (int64_t)B * max_seqlen)
            return fail(DSA_IDX_EINVAL, "total=%lld above B * max_seqlen", (long long)total);
        need = ws_score_topk_varlen(total, B, max_seqlen);
    } else {
        if (total > kMaxSeq) return fail(DSA_IDX_EUNSUPPORTED, "T=%lld above %lld", (long long)total, (long long)kMaxSeq);
        need = ws_score_topk(total);
    }
    if (total == 0 || (cu && (B == 0 || max_seqlen == 0))) return ok();
    if (!ws || ws_bytes < need)
        return fail(DSA_IDX_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
    if (!aligned16(ws)) return fail(DSA_IDX_EINVAL, "workspace must be 16-byte aligned");
    return ok();
}

static PrefillWs prefill_ws(const int32_t *cu, int B, int max_seqlen, int64_t total, void *ws) {
    const int Bh = cu ? B : 1;
    char *p = static_cast<char *>(ws);
    PrefillWs r;
    r.base = reinterpret_cast<int64_t *>(p);
    r.dummy = reinterpret_cast<float *>(p + ws_hdr(Bh));
    r.rows = reinterpret_cast<float *>(p + ws_hdr(Bh) + ws_dummy(prefill_max_len(cu, max_seqlen, total)));
    return r;
}

static bool prefill_empty(const int32_t *cu, int B, int max_seqlen, int64_t total) {
    return total == 0 || (cu && (B == 0 || max_seqlen == 0));
}

int dsa_idx_prefill_scores(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                           const int32_t *cu_seqlens, int B, int max_seqlen, int64_t total,
                           void *ws, size_t ws_bytes, void *stream) {
    size_t need = 0;
    int r = prefill_check(cu_seqlens, B, max_seqlen, total, ws, ws_bytes, need);
    if (r || prefill_empty(cu_seqlens, B, max_seqlen, total)) return r;
    if (!q || !k || !w) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(w))
        return fail(DSA_IDX_EINVAL, "q, k and w must be 16-byte aligned");
    r = check_device();
    if (r) return r;
    const PrefillWs p = prefill_ws(cu_seqlens, B, max_seqlen, total, ws);
    hipError_t e = dsaidx::launch_scores(q, k, w, cu_seqlens, cu_seqlens ? B : 1,
                                         prefill_max_len(cu_seqlens, max_seqlen, total), total, 0, p.base,
                                         p.rows, p.dummy, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("scores launch", e);
    return ok();
}

int dsa_idx_prefill_select(const int32_t *cu_seqlens, int B, int max_seqlen, int64_t total,
                           int topk, int32_t *idx, float *scores, void *ws, size_t ws_bytes,
                           void *stream) {
    int r = check_topk(topk);
    if (r) return r;
    size_t need = 0;
    r = prefill_check(cu_seqlens, B, max_seqlen, total, ws, ws_bytes, need);
    if (r || prefill_empty(cu_seqlens, B, max_seqlen, total)) return r;
    if (!idx) return fail(DSA_IDX_EINVAL, "idx is NULL");
    r = check_device();
    if (r) return r;
    const PrefillWs p = prefill_ws(cu_seqlens, B, max_seqlen, total, ws);
    hipError_t e = dsaidx::launch_row_topk_prefill(p.rows, cu_seqlens, p.base, cu_seqlens ? B : 1,
                                                   prefill_max_len(cu_seqlens, max_seqlen, total), 0,
                                                   total, topk, idx, scores,
                                                   reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("row top-k launch", e);
    return ok();
}

int dsa_idx_score_topk(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                       int64_t T, int topk, int32_t *idx, float *scores, void *ws,
                       size_t ws_bytes, void *stream) {
    if (T < 0) return fail(DSA_IDX_EINVAL, "T=%lld < 0", (long long)T);
    int r = check_topk(topk);
    if (r) return r;
    if (T > 0 && (!q || !k || !w || !idx)) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    size_t need = 0;
    r = prefill_check(nullptr, 1, 0, T, ws, ws_bytes, need);
    if (r || T == 0) return r;
    r = dsa_idx_prefill_scores(q, k, w, nullptr, 1, 0, T, ws, ws_bytes, stream);
    if (r) return r;
    return dsa_idx_prefill_select(nullptr, 1, 0, T, topk, idx, scores, ws, ws_bytes, stream);
}

int dsa_idx_v32_project(const dsa_idx_weights *wt, const dsa_idx_bf16 *x, int64_t ldx,
                        const dsa_idx_bf16 *c_q, int64_t ldc, int64_t T, int64_t pos0, float rope_theta,
                        dsa_idx_bf16 *q, dsa_idx_bf16 *k, dsa_idx_bf16 *w, void *ws, size_t ws_bytes,
                        void *stream) {
    if (!wt) return fail(DSA_IDX_EINVAL, "weights is NULL");
    if (T < 0 || pos0 < 0) return fail(DSA_IDX_EINVAL, "T=%lld pos0=%lld must be >= 0", (long long)T, (long long)pos0);
    if (!(rope_theta > 0.f)) return fail(DSA_IDX_EINVAL, "rope_theta must be > 0");
    if (T == 0) return ok();
    if (!wt->W_q || !wt->W_k || !wt->W_w || !wt->ln_gamma || !wt->ln_beta)
        return fail(DSA_IDX_EINVAL, "a weight pointer is NULL");
    if (!x || !c_q || !q || !k || !w) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    if (ldx < DSA_IDX_HIDDEN || ldx % 8) return fail(DSA_IDX_EINVAL, "ldx=%lld must be >= 7168 and a multiple of 8", (long long)ldx);
    if (ldc < DSA_IDX_QLAT || ldc % 8) return fail(DSA_IDX_EINVAL, "ldc=%lld must be >= 1536 and a multiple of 8", (long long)ldc);
    if (!(wt->ln_eps > 0.f)) return fail(DSA_IDX_EINVAL, "ln_eps must be > 0");
    const void *ptrs[] = {x, c_q, q, k, w, wt->W_q, wt->W_k, wt->W_w};
    for (const void *p : ptrs)
        if (!aligned16(p)) return fail(DSA_IDX_EINVAL, "tensor pointer %p is not 16-byte aligned", p);
    if (T > (int64_t)INT32_MAX * 128) return fail(DSA_IDX_EUNSUPPORTED, "T=%lld too large", (long long)T);
    const size_t need = dsaidx::project_workspace(T);
    if (need && (!ws || ws_bytes < need))
        return fail(DSA_IDX_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
    if (need && !aligned16(ws)) return fail(DSA_IDX_EINVAL, "workspace must be 16-byte aligned");
    int r = check_device();
    if (r) return r;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    constexpr int64_t kHalf = DSA_IDX_QOUT;   // q columns and w columns of one half: 4,096 and 32
    // first half: q columns 0..4,095, the key, w columns 0..31; second: the rest, no key
    hipError_t e = dsaidx::launch_project_ex(x, ldx, c_q, ldc, T, wt->W_q, DSA_IDX_V32_QOUT, wt->W_k, wt->W_w,
                                             DSA_IDX_V32_HEADS, wt->ln_gamma, wt->ln_beta, wt->ln_eps, q,
                                             DSA_IDX_V32_QOUT, k, nullptr, w, DSA_IDX_V32_HEADS,
                                             static_cast<float *>(ws), st);
    if (e != hipSuccess) return hip_fail("project launch", e);
    e = dsaidx::launch_project_ex(x, ldx, c_q, ldc, T, wt->W_q + kHalf, DSA_IDX_V32_QOUT, wt->W_k,
                                  wt->W_w + DSA_IDX_HEADS, DSA_IDX_V32_HEADS, wt->ln_gamma, wt->ln_beta, wt->ln_eps,
                                  q + kHalf, DSA_IDX_V32_QOUT, nullptr, nullptr, w + DSA_IDX_HEADS,
                                  DSA_IDX_V32_HEADS, static_cast<float *>(ws), st);
    if (e != hipSuccess) return hip_fail("project launch", e);
    e = dsaidx::launch_rope(q, DSA_IDX_V32_QOUT, DSA_IDX_V32_HEADS, k, DSA_IDX_DIM, T, pos0, (double)rope_theta, st);
    if (e != hipSuccess) return hip_fail("rotary launch", e);
    return ok();
}

int dsa_idx_v32_score_topk(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                           int64_t T, int topk, int32_t *idx, float *scores, void *ws,
                           size_t ws_bytes, void *stream) {
    if (T < 0) return fail(DSA_IDX_EINVAL, "T=%lld < 0", (long long)T);
    int r = check_topk(topk);
    if (r) return r;
    if (T > 0 && (!q || !k || !w || !idx)) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    size_t need = 0;
    r = prefill_check(nullptr, 1, 0, T, ws, ws_bytes, need);
    if (r || T == 0) return r;
    if (!aligned16(q) || !aligned16(k) || !aligned16(w))
        return fail(DSA_IDX_EINVAL, "q, k and w must be 16-byte aligned");
    r = check_device();
    if (r) return r;
    const PrefillWs p = prefill_ws(nullptr, 1, 0, T, ws);
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // heads 0..31 write the score rows, heads 32..63 add to them
    for (int half = 0; half < 2; ++half) {
        hipError_t e = dsaidx::launch_scores_ex(q + half * DSA_IDX_QOUT, DSA_IDX_V32_QOUT, k, w + half * DSA_IDX_HEADS,
                                                DSA_IDX_V32_HEADS, half == 1, nullptr, 1, T, T, 0, p.base, p.rows,
                                                p.dummy, st);
        if (e != hipSuccess) return hip_fail("scores launch", e);
    }
    return dsa_idx_prefill_select(nullptr, 1, 0, T, topk, idx, scores, ws, ws_bytes, stream);
}

int dsa_idx_v32_score_topk_varlen(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k,
                                  const dsa_idx_bf16 *w, const int32_t *cu_seqlens, int B,
                                  int max_seqlen, int64_t total, int topk, int32_t *idx,
                                  float *scores, void *ws, size_t ws_bytes, void *stream) {
    if (B < 0 || max_seqlen < 0 || total < 0)
        return fail(DSA_IDX_EINVAL, "B=%d max_seqlen=%d total=%lld must be >= 0", B, max_seqlen, (long long)total);
    if (B > 0 && !cu_seqlens) return fail(DSA_IDX_EINVAL, "cu_seqlens is NULL");
    int r = check_topk(topk);
    if (r) return r;
    if (total > 0 && (!q || !k || !w || !idx)) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    if (B == 0) return total == 0 ? ok() : fail(DSA_IDX_EINVAL, "total=%lld with B=0", (long long)total);
    size_t need = 0;
    r = prefill_check(cu_seqlens, B, max_seqlen, total, ws, ws_bytes, need);
    if (r || prefill_empty(cu_seqlens, B, max_seqlen, total)) return r;
    if (!aligned16(q) || !aligned16(k) || !aligned16(w))
        return fail(DSA_IDX_EINVAL, "q, k and w must be 16-byte aligned");
    r = check_device();
    if (r) return r;
    const PrefillWs p = prefill_ws(cu_seqlens, B, max_seqlen, total, ws);
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // heads 0..31 write the score rows, heads 32..63 add to them
    for (int half = 0; half < 2; ++half) {
        hipError_t e = dsaidx::launch_scores_ex(q + half * DSA_IDX_QOUT, DSA_IDX_V32_QOUT, k, w + half * DSA_IDX_HEADS,
                                                DSA_IDX_V32_HEADS, half == 1, cu_seqlens, B, max_seqlen, total, 0,
                                                p.base, p.rows, p.dummy, st);
        if (e != hipSuccess) return hip_fail("scores launch", e);
    }
    return dsa_idx_prefill_select(cu_seqlens, B, max_seqlen, total, topk, idx, scores, ws, ws_bytes, stream);
}

int dsa_idx_score_topk_varlen(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k,
                              const dsa_idx_bf16 *w, const int32_t *cu_seqlens, int B,
                              int max_seqlen, int64_t total, int topk, int32_t *idx,
                              float *scores, void *ws, size_t ws_bytes, void *stream) {
    if (B < 0 || max_seqlen < 0 || total < 0)
        return fail(DSA_IDX_EINVAL, "B=%d max_seqlen=%d total=%lld must be >= 0", B, max_seqlen, (long long)total);
    if (B > 0 && !cu_seqlens) return fail(DSA_IDX_EINVAL, "cu_seqlens is NULL");
    int r = check_topk(topk);
    if (r) return r;
    if (total > 0 && (!q || !k || !w || !idx)) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    if (B == 0) return total == 0 ? ok() : fail(DSA_IDX_EINVAL, "total=%lld with B=0", (long long)total);
    size_t need = 0;
    r = prefill_check(cu_seqlens, B, max_seqlen, total, ws, ws_bytes, need);
    if (r || prefill_empty(cu_seqlens, B, max_seqlen, total)) return r;
    r = dsa_idx_prefill_scores(q, k, w, cu_seqlens, B, max_seqlen, total, ws, ws_bytes, stream);
    if (r) return r;
    return dsa_idx_prefill_select(cu_seqlens, B, max_seqlen, total, topk, idx, scores, ws, ws_bytes,
                                  stream);
}

// A chunk of C queries against its whole prefix, with heads/32 scoring passes of 32 heads each
// (q rows heads x 128, w rows heads), the later ones adding to the score rows.
static int prefill_chunk_impl(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                              int64_t C, int64_t prefix, int topk, int32_t *idx, float *scores,
                              void *ws, size_t ws_bytes, void *stream, int heads) {
    if (C < 0 || prefix < 0)
        return fail(DSA_IDX_EINVAL, "C=%lld prefix=%lld must be >= 0", (long long)C, (long long)prefix);
    int r = check_topk(topk);
    if (r) return r;
    if (C == 0) return ok();
    if (!q || !k || !w || !idx) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(w))
        return fail(DSA_IDX_EINVAL, "q, k and w must be 16-byte aligned");
    if (C > kMaxSeq) return fail(DSA_IDX_EUNSUPPORTED, "C=%lld above %lld", (long long)C, (long long)kMaxSeq);
    if (prefix + C > kMaxWindow)
        return fail(DSA_IDX_EUNSUPPORTED, "prefix + C = %lld above %lld", (long long)(prefix + C),
                    (long long)kMaxWindow);
    const size_t need = ws_prefill_chunk(C, prefix);
    if (!ws || ws_bytes < need)
        return fail(DSA_IDX_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
    if (!aligned16(ws)) return fail(DSA_IDX_EINVAL, "workspace must be 16-byte aligned");
    r = check_device();
    if (r) return r;
    char *wsb = static_cast<char *>(ws);
    int64_t *base = reinterpret_cast<int64_t *>(wsb);
    float *dummy = reinterpret_cast<float *>(wsb + ws_hdr(1));
    float *rows = reinterpret_cast<float *>(wsb + ws_hdr(1) + ws_dummy(prefix + C));
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    for (int half = 0; half < heads / DSA_IDX_HEADS; ++half) {
        e = dsaidx::launch_scores_ex(q + half * DSA_IDX_QOUT, (int64_t)heads * DSA_IDX_DIM, k, w + half * DSA_IDX_HEADS,
                                     heads, half > 0, nullptr, 1, C, C, prefix, base, rows, dummy, st);
        if (e != hipSuccess) return hip_fail("scores launch", e);
    }
    e = dsaidx::launch_row_topk_prefill(rows, nullptr, base, 1, C, prefix, C, topk, idx, scores, st);
    if (e != hipSuccess) return hip_fail("row top-k launch", e);
    return ok();
}

int dsa_idx_prefill_chunk(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                          int64_t C, int64_t prefix, int topk, int32_t *idx, float *scores,
                          void *ws, size_t ws_bytes, void *stream) {
    return prefill_chunk_impl(q, k, w, C, prefix, topk, idx, scores, ws, ws_bytes, stream, DSA_IDX_HEADS);
}

int dsa_idx_v32_prefill_chunk(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                              int64_t C, int64_t prefix, int topk, int32_t *idx, float *scores,
                              void *ws, size_t ws_bytes, void *stream) {
    return prefill_chunk_impl(q, k, w, C, prefix, topk, idx, scores, ws, ws_bytes, stream, DSA_IDX_V32_HEADS);
}

int dsa_idx_sparse_mla(const dsa_idx_bf16 *q, const dsa_idx_bf16 *kv, const int32_t *idx,
                       const int64_t *row0, int64_t T, int topk, float scale, dsa_idx_bf16 *o,
                       float *lse, void *ws, size_t ws_bytes, void *stream) {
    if (T < 0) return fail(DSA_IDX_EINVAL, "T=%lld < 0", (long long)T);
    int r = check_topk(topk);
    if (r) return r;
    if (T == 0) return ok();
    if (!q || !kv || !idx || !o) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    if (!aligned16(q) || !aligned16(kv) || !aligned16(o)) return fail(DSA_IDX_EINVAL, "q, kv and o must be 16-byte aligned");
    if (!(scale > 0.f) || !(scale < INFINITY)) return fail(DSA_IDX_EINVAL, "scale must be positive and finite");
    if (T > 65535) return fail(DSA_IDX_EUNSUPPORTED, "T=%lld above 65535", (long long)T);
    const size_t need = dsaidx::sparse_mla_workspace(T, topk);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(DSA_IDX_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
    if (need > 0 && !aligned16(ws)) return fail(DSA_IDX_EINVAL, "workspace must be 16-byte aligned");
    r = check_device();
    if (r) return r;
    hipError_t e = dsaidx::launch_sparse_mla(q, kv, idx, row0, T, topk, scale, o, lse, static_cast<float *>(ws),
                                             reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("sparse_mla launch", e);
    return ok();
}

// heads: 32, or 64 for the 64-head indexer
static int decode_impl(const dsa_idx_bf16 *q, const dsa_idx_bf16 *w, const dsa_idx_bf16 *k_cache,
                       const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                       int topk, int32_t *idx, float *scores, void *ws, size_t ws_bytes,
                       void *stream, int heads) {
    if (B < 0 || max_seqlen < 0) return fail(DSA_IDX_EINVAL, "B=%d max_seqlen=%d must be >= 0", B, max_seqlen);
    int r = check_topk(topk);
    if (r) return r;
    if (B == 0) return ok();
    if (max_seqlen < 1) return fail(DSA_IDX_EINVAL, "max_seqlen must be >= 1");
    if (!q || !w || !k_cache || !start || !seqlens || !idx) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    if (!aligned16(q) || !aligned16(w) || !aligned16(k_cache))
        return fail(DSA_IDX_EINVAL, "q, w and k_cache must be 16-byte aligned");
    if (B > 65535) return fail(DSA_IDX_EUNSUPPORTED, "B=%d above 65535", B);
    const size_t need = ws_decode(B, max_seqlen);
    if (!ws || ws_bytes < need)
        return fail(DSA_IDX_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
    if (!aligned16(ws)) return fail(DSA_IDX_EINVAL, "workspace must be 16-byte aligned");
    r = check_device();
    if (r) return r;
    hipError_t e = heads == DSA_IDX_V32_HEADS
                       ? dsaidx::launch_decode_v32(q, w, k_cache, start, seqlens, B, max_seqlen, topk, ws, idx,
                                                   scores, reinterpret_cast<hipStream_t>(stream))
                       : dsaidx::launch_decode(q, w, k_cache, start, seqlens, B, max_seqlen, topk, ws, idx,
                                               scores, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("decode launch", e);
    return ok();
}

int dsa_idx_decode(const dsa_idx_bf16 *q, const dsa_idx_bf16 *w, const dsa_idx_bf16 *k_cache,
                   const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                   int topk, int32_t *idx, float *scores, void *ws, size_t ws_bytes,
                   void *stream) {
    return decode_impl(q, w, k_cache, start, seqlens, B, max_seqlen, topk, idx, scores, ws, ws_bytes, stream,
                       DSA_IDX_HEADS);
}

int dsa_idx_v32_decode(const dsa_idx_bf16 *q, const dsa_idx_bf16 *w, const dsa_idx_bf16 *k_cache,
                       const int64_t *start, const int32_t *seqlens, int B, int max_seqlen,
                       int topk, int32_t *idx, float *scores, void *ws, size_t ws_bytes,
                       void *stream) {
    return decode_impl(q, w, k_cache, start, seqlens, B, max_seqlen, topk, idx, scores, ws, ws_bytes, stream,
                       DSA_IDX_V32_HEADS);
}

int dsa_idx_quantize_keys(const dsa_idx_bf16 *k, int64_t ldk, int64_t N, const int64_t *slot,
                          uint8_t *k8, float *k_scale, void *stream) {
    if (N < 0) return fail(DSA_IDX_EINVAL, "N=%lld < 0", (long long)N);
    if (N == 0) return ok();
    if (!k || !k8 || !k_scale) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    if (ldk < DSA_IDX_DIM || ldk % 8) return fail(DSA_IDX_EINVAL, "ldk=%lld must be >= 128 and a multiple of 8", (long long)ldk);
    if (!aligned16(k) || !aligned16(k8)) return fail(DSA_IDX_EINVAL, "k and k8 must be 16-byte aligned");
    if (N > (int64_t)INT32_MAX * 4) return fail(DSA_IDX_EUNSUPPORTED, "N=%lld too large", (long long)N);
    int r = check_device();
    if (r) return r;
    hipError_t e = dsaidx::launch_quantize_keys(k, ldk, N, slot, k8, k_scale, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("quantize_keys launch", e);
    return ok();
}

static int decode_fp8_impl(const dsa_idx_bf16 *q, const dsa_idx_bf16 *w, const uint8_t *k8,
                           const float *k_scale, const int64_t *start, const int32_t *seqlens, int B,
                           int max_seqlen, int topk, int32_t *idx, float *scores, void *ws,
                           size_t ws_bytes, void *stream, int heads) {
    if (B < 0 || max_seqlen < 0) return fail(DSA_IDX_EINVAL, "B=%d max_seqlen=%d must be >= 0", B, max_seqlen);
    int r = check_topk(topk);
    if (r) return r;
    if (B == 0) return ok();
    if (max_seqlen < 1) return fail(DSA_IDX_EINVAL, "max_seqlen must be >= 1");
    if (!q || !w || !k8 || !k_scale || !start || !seqlens || !idx) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    if (!aligned16(q) || !aligned16(w) || !aligned16(k8))
        return fail(DSA_IDX_EINVAL, "q, w and k8 must be 16-byte aligned");
    if (B > 65535) return fail(DSA_IDX_EUNSUPPORTED, "B=%d above 65535", B);
    const size_t need = ws_decode_fp8(B, max_seqlen);
    if (!ws || ws_bytes < need)
        return fail(DSA_IDX_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
    if (!aligned16(ws)) return fail(DSA_IDX_EINVAL, "workspace must be 16-byte aligned");
    r = check_device();
    if (r) return r;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = heads == DSA_IDX_V32_HEADS
                       ? dsaidx::launch_decode_fp8_v32(q, w, k8, k_scale, start, seqlens, B, max_seqlen, topk, ws,
                                                       idx, scores, st)
                       : dsaidx::launch_decode_fp8(q, w, k8, k_scale, start, seqlens, B, max_seqlen, topk, ws, idx,
                                                   scores, st);
    if (e != hipSuccess) return hip_fail("decode_fp8 launch", e);
    return ok();
}

int dsa_idx_decode_fp8(const dsa_idx_bf16 *q, const dsa_idx_bf16 *w, const uint8_t *k8,
                       const float *k_scale, const int64_t *start, const int32_t *seqlens, int B,
                       int max_seqlen, int topk, int32_t *idx, float *scores, void *ws,
                       size_t ws_bytes, void *stream) {
    return decode_fp8_impl(q, w, k8, k_scale, start, seqlens, B, max_seqlen, topk, idx, scores, ws, ws_bytes,
                           stream, DSA_IDX_HEADS);
}

int dsa_idx_v32_decode_fp8(const dsa_idx_bf16 *q, const dsa_idx_bf16 *w, const uint8_t *k8,
                           const float *k_scale, const int64_t *start, const int32_t *seqlens, int B,
                           int max_seqlen, int topk, int32_t *idx, float *scores, void *ws,
                           size_t ws_bytes, void *stream) {
    return decode_fp8_impl(q, w, k8, k_scale, start, seqlens, B, max_seqlen, topk, idx, scores, ws, ws_bytes,
                           stream, DSA_IDX_V32_HEADS);
}

}  // extern "C"
