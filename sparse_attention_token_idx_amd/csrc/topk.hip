// Row top-k kernels (prefill rows and decode rows); the selection itself is in topk_impl.hpp.
#include "topk_impl.hpp"

namespace dsaidx {
namespace {
using namespace topk_impl;

// One workgroup per row.
template <int W>
__global__ __launch_bounds__(64 * W, W == 4 ? 5 : 16 / W) void row_topk_kernel(TopkArgs a) {
    __shared__ TopkSmem<W> sm;
    const int64_t g = a.g0 + (int64_t)blockIdx.x;
    if (a.status && (*a.status & 1u)) {
        // the scoring kernel's ring wait gave up: its rows are not to be trusted
        for (int i = (int)threadIdx.x; i < a.topk; i += 64 * W) {
            a.out_idx[g * a.topk + i] = -2;
            if (a.out_score) a.out_score[g * a.topk + i] = __builtin_nanf("");
        }
        return;
    }
    row_topk_row<W>(a, g, sm);
}

}  // namespace

hipError_t launch_row_topk_prefill(const float *scores, const int32_t *cu_seqlens,
                                   const int64_t *seq_base, int B, int64_t max_len, int64_t pos0,
                                   int64_t rows, int topk, int32_t *idx, float *out_scores,
                                   const uint32_t *status, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    TopkArgs a{};
    a.scores = scores;
    a.mode = 0;
    a.cu_seqlens = cu_seqlens;
    a.seq_base = seq_base;
    a.pos0 = cu_seqlens ? 0 : pos0;
    a.B = B;
    a.topk = topk;
    a.out_idx = idx;
    a.out_score = out_scores;
    a.status = status;
    // rows of up to kLongRow scores: 4-wave workgroups; longer rows: the 16-wave variant
    // (ragged batches take one variant for all rows, from the longest sequence)
    int64_t g1 = rows;
    if (cu_seqlens) {
        g1 = max_len > kLongRow ? 0 : rows;
    } else {
        g1 = kLongRow - a.pos0;
        g1 = g1 < 0 ? 0 : (g1 > rows ? rows : g1);
    }
    if (g1 > 0) {
        a.g0 = 0;
        hipLaunchKernelGGL(row_topk_kernel<4>, dim3((unsigned)g1), dim3(256), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (g1 < rows) {
        a.g0 = g1;
        hipLaunchKernelGGL(row_topk_kernel<16>, dim3((unsigned)(rows - g1)), dim3(1024), 0, stream, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_row_topk_decode(const float *scores, const int32_t *seqlens, int B, int64_t ld,
                                  int64_t nmax, int topk, int32_t *idx, float *out_scores,
                                  hipStream_t stream) {
    if (B == 0) return hipSuccess;
    TopkArgs a{};
    a.scores = scores;
    a.mode = 1;
    a.seqlens = seqlens;
    a.ld = ld;
    a.nmax = nmax;
    a.B = B;
    a.topk = topk;
    a.out_idx = idx;
    a.out_score = out_scores;
    hipLaunchKernelGGL(row_topk_kernel<16>, dim3((unsigned)B), dim3(1024), 0, stream, a);
    return hipGetLastError();
}

}  // namespace dsaidx
