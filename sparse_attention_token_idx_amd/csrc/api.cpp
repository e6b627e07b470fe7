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

// The architecture part of a gcnArchName ("gfx950:sramecc+:xnack-" -> "gfx950") must be gfx950.
bool arch_is_gfx950(const char *name) {
    const size_t n = strcspn(name, ":");
    return n == 6 && strncmp(name, "gfx950", 6) == 0;
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
        state[dev] = arch_is_gfx950(p.gcnArchName) ? 1 : 2;
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

// Longest sequence (prefix + chunk, or one sequence) a prefill call accepts: key positions stay
// below 2^24, so 32-bit element offsets within a sequence never wrap.
constexpr int64_t kMaxWindow = 1LL << 24;
// Longest sequence of a ragged batch (its row blocks sit on grid.y, at most 65,535; 16 rows a
// block for 64 heads).
constexpr int64_t kMaxVarlenSeq = 65535LL * 16;

size_t round256(size_t b) { return (b + 255u) & ~(size_t)255u; }

// Raw causal score rows (dsa_idx_prefill_scores / dsa_idx_prefill_select): [status word, 256 B]
// [sequence bases: int64 x (B + 1)] [dummy row] [triangular rows], each part 256-byte aligned.
size_t rows_hdr(int B) { return 256u + round256(8u * (size_t)(B + 1)); }
size_t rows_dummy(int64_t max_len) {
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
size_t ws_rows(const bool varlen, int64_t total, int B, int64_t max_seqlen) {
    if (!varlen) return rows_hdr(1) + rows_dummy(total) + 4u * (size_t)dsaidx::tri_row_offset(total);
    return rows_hdr(B) + rows_dummy(max_seqlen) + 4u * (size_t)varlen_score_floats(total, B, max_seqlen);
}

// Top-k workspace of a prefill call (see prefill_plan): linear in the rows.
size_t ws_topk(int heads, bool varlen, int64_t rows, int B, int64_t max_len, int64_t pos0) {
    if (rows == 0) return 0;
    return dsaidx::prefill_plan(heads, varlen, rows, B, max_len, pos0).bytes;
}

size_t ws_decode(int B, int max_seqlen) { return dsaidx::decode_workspace(B, max_seqlen, false); }
size_t ws_decode_fp8(int B, int max_seqlen) { return dsaidx::decode_workspace(B, max_seqlen, true); }

}  // namespace

extern "C" {

const char *dsa_idx_version(void) { return "libdsaidx 0.1.0 (gfx950)"; }

int dsa_idx_arch_supported(const char *arch_name) {
    if (!arch_name) return fail(DSA_IDX_EINVAL, "arch_name is null");
    if (!arch_is_gfx950(arch_name))
        return fail(DSA_IDX_EUNSUPPORTED, "architecture %.64s; libdsaidx runs on gfx950 only", arch_name);
    return ok();
}

const char *dsa_idx_last_error(void) { return g_err; }

int dsa_idx_workspace_size(int op, int64_t total_tokens, int B, int max_seqlen, int topk,
                           size_t *bytes) {
    if (!bytes) return fail(DSA_IDX_EINVAL, "bytes is NULL");
    switch (op) {
        case DSA_IDX_OP_PROJECT:
            if (total_tokens < 0) return fail(DSA_IDX_EINVAL, "T=%lld < 0", (long long)total_tokens);
            *bytes = dsaidx::project_workspace(total_tokens);
            return ok();
        case DSA_IDX_OP_SCORE_TOPK:
        case DSA_IDX_OP_V32_SCORE_TOPK: {
            if (total_tokens < 0) return fail(DSA_IDX_EINVAL, "T=%lld < 0", (long long)total_tokens);
            int r = check_topk(topk);
            if (r) return r;
            *bytes = ws_topk(op == DSA_IDX_OP_SCORE_TOPK ? 32 : 64, false, total_tokens, 1, total_tokens, 0);
            return ok();
        }
        case DSA_IDX_OP_SCORE_TOPK_VARLEN:
        case DSA_IDX_OP_V32_SCORE_TOPK_VARLEN: {
            if (total_tokens < 0 || B < 0 || max_seqlen < 0)
                return fail(DSA_IDX_EINVAL, "total=%lld B=%d max_seqlen=%d must be >= 0",
                            (long long)total_tokens, B, max_seqlen);
            int r = check_topk(topk);
            if (r) return r;
            *bytes = B == 0 || max_seqlen == 0
                         ? 0
                         : ws_topk(op == DSA_IDX_OP_SCORE_TOPK_VARLEN ? 32 : 64, true, total_tokens, B, max_seqlen, 0);
            return ok();
        }
        case DSA_IDX_OP_PREFILL_CHUNK:
        case DSA_IDX_OP_V32_PREFILL_CHUNK: {
            if (total_tokens < 0 || max_seqlen < 0)
                return fail(DSA_IDX_EINVAL, "C=%lld prefix=%d must be >= 0", (long long)total_tokens, max_seqlen);
            int r = check_topk(topk);
            if (r) return r;
            *bytes = ws_topk(op == DSA_IDX_OP_PREFILL_CHUNK ? 32 : 64, false, total_tokens, 1, total_tokens, max_seqlen);
            return ok();
        }
        case DSA_IDX_OP_PREFILL_ROWS: {
            if (total_tokens < 0 || B < 0 || max_seqlen < 0)
                return fail(DSA_IDX_EINVAL, "total=%lld B=%d max_seqlen=%d must be >= 0",
                            (long long)total_tokens, B, max_seqlen);
            *bytes = total_tokens == 0 ? 0 : ws_rows(B > 0, total_tokens, B, max_seqlen);
            return ok();
        }
        case DSA_IDX_OP_V32_PROJECT:
            if (total_tokens < 0) return fail(DSA_IDX_EINVAL, "T=%lld < 0", (long long)total_tokens);
            *bytes = dsaidx::project_workspace(total_tokens, DSA_IDX_V32_QOUT, DSA_IDX_V32_HEADS, true);
            return ok();
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


// ---------------------------------------------------------------- prefill
// Shape checks shared by the prefill entries.  varlen: B sequences packed back to back
// (longest max_seqlen); else one sequence of `rows` tokens at positions pos0 ...
static int prefill_args(bool varlen, const int32_t *cu, int B, int max_seqlen, int64_t rows, int64_t pos0) {
    if (rows < 0 || pos0 < 0) return fail(DSA_IDX_EINVAL, "rows=%lld pos0=%lld must be >= 0", (long long)rows, (long long)pos0);
    if (varlen) {
        if (B < 0 || max_seqlen < 0)
            return fail(DSA_IDX_EINVAL, "B=%d max_seqlen=%d must be >= 0", B, max_seqlen);
        if (B > 0 && !cu) return fail(DSA_IDX_EINVAL, "cu_seqlens is NULL");
        if (B == 0 && rows > 0) return fail(DSA_IDX_EINVAL, "total=%lld with B=0", (long long)rows);
        if (B > 65535) return fail(DSA_IDX_EUNSUPPORTED, "B=%d above 65535", B);
        if (max_seqlen > kMaxVarlenSeq)
            return fail(DSA_IDX_EUNSUPPORTED, "max_seqlen=%d above %lld", max_seqlen, (long long)kMaxVarlenSeq);
        if (rows > (int64_t)B * max_seqlen)
            return fail(DSA_IDX_EINVAL, "total=%lld above B * max_seqlen", (long long)rows);
    } else if (pos0 + rows > kMaxWindow) {
        return fail(DSA_IDX_EUNSUPPORTED, "sequence of %lld keys above %lld", (long long)(pos0 + rows),
                    (long long)kMaxWindow);
    }
    return ok();
}

static bool prefill_empty(bool varlen, int B, int max_seqlen, int64_t rows) {
    return rows == 0 || (varlen && (B == 0 || max_seqlen == 0));
}

// Scores and top-k of every row, workspace linear in the rows (heads: 32, or 64).
static int prefill_topk_impl(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w, bool varlen,
                             const int32_t *cu, int B, int max_seqlen, int64_t rows, int64_t pos0, int topk,
                             int32_t *idx, float *scores, void *ws, size_t ws_bytes, void *stream, int heads) {
    int r = check_topk(topk);
    if (r) return r;
    r = prefill_args(varlen, cu, B, max_seqlen, rows, pos0);
    if (r || prefill_empty(varlen, B, max_seqlen, rows)) return r;
    if (!q || !k || !w || !idx) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(w))
        return fail(DSA_IDX_EINVAL, "q, k and w must be 16-byte aligned");
    const dsaidx::PrefillPlan plan =
        dsaidx::prefill_plan(heads, varlen, rows, varlen ? B : 1, varlen ? max_seqlen : rows, pos0);
    if (!ws || ws_bytes < plan.bytes)
        return fail(DSA_IDX_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, plan.bytes);
    if (!aligned16(ws)) return fail(DSA_IDX_EINVAL, "workspace must be 16-byte aligned");
    r = check_device();
    if (r) return r;
    hipError_t e = dsaidx::launch_prefill_topk(plan, q, k, w, varlen ? cu : nullptr, topk, idx, scores, ws,
                                               reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("prefill launch", e);
    return ok();
}

int dsa_idx_score_topk(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                       int64_t T, int topk, int32_t *idx, float *scores, void *ws,
                       size_t ws_bytes, void *stream) {
    return prefill_topk_impl(q, k, w, false, nullptr, 1, 0, T, 0, topk, idx, scores, ws, ws_bytes, stream,
                             DSA_IDX_HEADS);
}

int dsa_idx_score_topk_varlen(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k,
                              const dsa_idx_bf16 *w, const int32_t *cu_seqlens, int B,
                              int max_seqlen, int64_t total, int topk, int32_t *idx,
                              float *scores, void *ws, size_t ws_bytes, void *stream) {
    return prefill_topk_impl(q, k, w, true, cu_seqlens, B, max_seqlen, total, 0, topk, idx, scores, ws, ws_bytes,
                             stream, DSA_IDX_HEADS);
}

int dsa_idx_prefill_chunk(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                          int64_t C, int64_t prefix, int topk, int32_t *idx, float *scores,
                          void *ws, size_t ws_bytes, void *stream) {
    return prefill_topk_impl(q, k, w, false, nullptr, 1, 0, C, prefix, topk, idx, scores, ws, ws_bytes, stream,
                             DSA_IDX_HEADS);
}

int dsa_idx_v32_score_topk(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                           int64_t T, int topk, int32_t *idx, float *scores, void *ws,
                           size_t ws_bytes, void *stream) {
    return prefill_topk_impl(q, k, w, false, nullptr, 1, 0, T, 0, topk, idx, scores, ws, ws_bytes, stream,
                             DSA_IDX_V32_HEADS);
}

int dsa_idx_v32_score_topk_varlen(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k,
                                  const dsa_idx_bf16 *w, const int32_t *cu_seqlens, int B,
                                  int max_seqlen, int64_t total, int topk, int32_t *idx,
                                  float *scores, void *ws, size_t ws_bytes, void *stream) {
    return prefill_topk_impl(q, k, w, true, cu_seqlens, B, max_seqlen, total, 0, topk, idx, scores, ws, ws_bytes,
                             stream, DSA_IDX_V32_HEADS);
}

int dsa_idx_v32_prefill_chunk(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                              int64_t C, int64_t prefix, int topk, int32_t *idx, float *scores,
                              void *ws, size_t ws_bytes, void *stream) {
    return prefill_topk_impl(q, k, w, false, nullptr, 1, 0, C, prefix, topk, idx, scores, ws, ws_bytes, stream,
                             DSA_IDX_V32_HEADS);
}

// ---- raw causal score rows (32 heads) and the row top-k over them
struct RowsWs {
    uint32_t *status;
    int64_t *base;
    float *dummy;
    float *rows;
};

static RowsWs rows_ws(bool varlen, int B, int max_seqlen, int64_t total, void *ws) {
    const int Bh = varlen ? B : 1;
    char *p = static_cast<char *>(ws);
    RowsWs r;
    r.status = reinterpret_cast<uint32_t *>(p);
    r.base = reinterpret_cast<int64_t *>(p + 256);
    r.dummy = reinterpret_cast<float *>(p + rows_hdr(Bh));
    r.rows = reinterpret_cast<float *>(p + rows_hdr(Bh) + rows_dummy(varlen ? max_seqlen : total));
    return r;
}

static int rows_check(bool varlen, const int32_t *cu, int B, int max_seqlen, int64_t total, void *ws,
                      size_t ws_bytes) {
    int r = prefill_args(varlen, cu, B, max_seqlen, total, 0);
    if (r || prefill_empty(varlen, B, max_seqlen, total)) return r;
    if (varlen && max_seqlen > 65535LL * 32)
        return fail(DSA_IDX_EUNSUPPORTED, "max_seqlen=%d above %lld", max_seqlen, 65535LL * 32);
    const size_t need = ws_rows(varlen, total, B, max_seqlen);
    if (!ws || ws_bytes < need)
        return fail(DSA_IDX_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
    if (!aligned16(ws)) return fail(DSA_IDX_EINVAL, "workspace must be 16-byte aligned");
    return ok();
}

int dsa_idx_prefill_scores(const dsa_idx_bf16 *q, const dsa_idx_bf16 *k, const dsa_idx_bf16 *w,
                           const int32_t *cu_seqlens, int B, int max_seqlen, int64_t total,
                           void *ws, size_t ws_bytes, void *stream) {
    const bool varlen = cu_seqlens != nullptr;
    int r = rows_check(varlen, cu_seqlens, B, max_seqlen, total, ws, ws_bytes);
    if (r || prefill_empty(varlen, B, max_seqlen, total)) return r;
    if (!q || !k || !w) return fail(DSA_IDX_EINVAL, "a tensor pointer is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(w))
        return fail(DSA_IDX_EINVAL, "q, k and w must be 16-byte aligned");
    r = check_device();
    if (r) return r;
    const RowsWs p = rows_ws(varlen, B, max_seqlen, total, ws);
    hipError_t e = dsaidx::launch_scores(q, k, w, cu_seqlens, varlen ? B : 1, varlen ? max_seqlen : total, total, 0,
                                         p.base, p.rows, p.dummy, p.status, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("scores launch", e);
    return ok();
}

int dsa_idx_prefill_select(const int32_t *cu_seqlens, int B, int max_seqlen, int64_t total,
                           int topk, int32_t *idx, float *scores, void *ws, size_t ws_bytes,
                           void *stream) {
    int r = check_topk(topk);
    if (r) return r;
    const bool varlen = cu_seqlens != nullptr;
    r = rows_check(varlen, cu_seqlens, B, max_seqlen, total, ws, ws_bytes);
    if (r || prefill_empty(varlen, B, max_seqlen, total)) return r;
    if (!idx) return fail(DSA_IDX_EINVAL, "idx is NULL");
    r = check_device();
    if (r) return r;
    const RowsWs p = rows_ws(varlen, B, max_seqlen, total, ws);
    hipError_t e = dsaidx::launch_row_topk_prefill(p.rows, cu_seqlens, p.base, varlen ? B : 1,
                                                   varlen ? max_seqlen : total, 0, total, topk, idx, scores,
                                                   p.status, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("row top-k launch", e);
    return ok();
}

int dsa_idx_workspace_status(const void *ws, size_t ws_bytes, void *stream) {
    if (!ws || ws_bytes < 4) return fail(DSA_IDX_EINVAL, "workspace is NULL or smaller than its status word");
    uint32_t st = 0;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(&st, ws, sizeof(st), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail("status copy", e);
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail("stream synchronize", e);
    if (st & 1u)
        return fail(DSA_IDX_ESTALL,
                    "a score kernel's wait on its key ring ran out of polls; that call's outputs are invalid "
                    "(indices -2, scores NaN)");
    return ok();
}

int dsa_idx_phase_timing(int enable) {
    if (enable) {
        double ms[dsaidx::kPhases];
        int cnt[dsaidx::kPhases];
        (void)dsaidx::prefill_phase_times(ms, cnt, dsaidx::kPhases);   // forget older records
    }
    dsaidx::prefill_phase_timing(enable != 0);
    return ok();
}

int dsa_idx_phase_times(double *ms, int *count, int n) {
    if (!ms || !count || n < 0) return fail(DSA_IDX_EINVAL, "ms and count must be non-NULL, n >= 0");
    hipError_t e = dsaidx::prefill_phase_times(ms, count, n);
    if (e != hipSuccess) return hip_fail("phase events", e);
    return ok();
}

static_assert(DSA_IDX_CALIB_SINK == dsaidx::kCalibBlocks * 256, "calibration sink size");

int dsa_idx_mfma_calibrate(int64_t iters, int random_operands, float *sink, size_t sink_floats, int64_t *flop,
                           void *stream) {
    if (iters < 1 || iters > (int64_t)1 << 32) return fail(DSA_IDX_EINVAL, "iters=%lld must be in [1, 2^32]", (long long)iters);
    if (!sink || !flop) return fail(DSA_IDX_EINVAL, "sink and flop must be non-NULL");
    if (sink_floats < (size_t)DSA_IDX_CALIB_SINK) return fail(DSA_IDX_EINVAL, "sink_floats=%zu below %d", sink_floats, DSA_IDX_CALIB_SINK);
    const int r = check_device();
    if (r != DSA_IDX_OK) return r;
    *flop = dsaidx::mfma_calibrate_flop(iters);
    const hipError_t e = dsaidx::launch_mfma_calibrate(iters, random_operands ? 1 : 0, sink,
                                                       reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail("mfma_calibrate_kernel launch", e);
    return ok();
}

int dsa_idx_set_wait_budget(int polls) {
    const int prev = dsaidx::prefill_wait_budget();
    dsaidx::prefill_set_wait_budget(polls);
    return prev;
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
    const size_t need = dsaidx::project_workspace(T, DSA_IDX_V32_QOUT, DSA_IDX_V32_HEADS, true);
    if (!ws || ws_bytes < need)
        return fail(DSA_IDX_EWORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
    if (!aligned16(ws)) return fail(DSA_IDX_EINVAL, "workspace must be 16-byte aligned");
    int r = check_device();
    if (r) return r;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // one pass: all 8,192 q columns, the key and all 64 w columns, the rotary step in the epilogues
    hipError_t e = dsaidx::launch_project_ex(x, ldx, c_q, ldc, T, wt->W_q, DSA_IDX_V32_QOUT, DSA_IDX_V32_QOUT,
                                             wt->W_k, wt->W_w, DSA_IDX_V32_HEADS, DSA_IDX_V32_HEADS, wt->ln_gamma,
                                             wt->ln_beta, wt->ln_eps, q, DSA_IDX_V32_QOUT, k, nullptr, w,
                                             DSA_IDX_V32_HEADS, pos0, (double)rope_theta, static_cast<float *>(ws), st);
    if (e != hipSuccess) return hip_fail("project launch", e);
    return ok();
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
    if (max_seqlen > kMaxWindow)
        return fail(DSA_IDX_EUNSUPPORTED, "max_seqlen=%d above %lld", max_seqlen, (long long)kMaxWindow);
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

}  // extern "C"

// ---- The decode entry that allocates nothing: its scratch is this array.  Each device the
// library runs on holds its own copy until the process ends; host code never passes the array's
// name to a kernel (on the host it is only a stand-in), but the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[DSA_IDX_DECODE_NOALLOC_SCRATCH];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[dsaidx::kMaxDevices] = {};

int static_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev < 0 || dev >= dsaidx::kMaxDevices) return fail(DSA_IDX_EUNSUPPORTED, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
        if (!p) return fail(DSA_IDX_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ok();
}
}  // namespace

extern "C" {

int dsa_idx_decode_noalloc(const dsa_idx_bf16 *q, const dsa_idx_bf16 *w, const dsa_idx_bf16 *k_cache,
                           const int64_t *start, const int32_t *seqlens, int B, int max_seqlen, int topk,
                           int32_t *idx, float *scores, void *stream) {
    if (B < 0 || max_seqlen < 0) return fail(DSA_IDX_EINVAL, "B=%d max_seqlen=%d must be >= 0", B, max_seqlen);
    int r = check_topk(topk);
    if (r) return r;
    if (B == 0) return ok();
    if (max_seqlen > kMaxWindow)
        return fail(DSA_IDX_EUNSUPPORTED, "max_seqlen=%d above %lld", max_seqlen, (long long)kMaxWindow);
    const size_t need = ws_decode(B, max_seqlen);
    if (need > (size_t)DSA_IDX_DECODE_NOALLOC_SCRATCH)
        return fail(DSA_IDX_EUNSUPPORTED,
                    "B=%d, max_seqlen=%d need %zu bytes of scratch, above the %zu bytes this entry holds; "
                    "use dsa_idx_decode with a workspace",
                    B, max_seqlen, need, (size_t)DSA_IDX_DECODE_NOALLOC_SCRATCH);
    r = check_device();
    if (r) return r;
    void *ws = nullptr;
    r = static_scratch(&ws);
    if (r) return r;
    return decode_impl(q, w, k_cache, start, seqlens, B, max_seqlen, topk, idx, scores, ws,
                       (size_t)DSA_IDX_DECODE_NOALLOC_SCRATCH, stream, DSA_IDX_HEADS);
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
    if (max_seqlen > kMaxWindow)
        return fail(DSA_IDX_EUNSUPPORTED, "max_seqlen=%d above %lld", max_seqlen, (long long)kMaxWindow);
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
