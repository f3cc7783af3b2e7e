// k_gate.hip -- the low-rank forget gate written out as log_g.
//
// GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"), Method §1: the
// key-side forget gate is generated from the input by a light low-rank
// projection with a temperature.  For token n (b L + grid position) and column
// j = h dk + c of the H dk gate channels:
//     x = sum_r feat[n][r] gate_w[r][j] + gate_b[j],   log_g[n][j] = logsigmoid(x) / tau
// This kernel serves the paths whose kernels read log_g from memory; the
// matrix-core path for rank 16, dk = dv = 64, chunk 64 forms the gate inside
// its own kernels instead.
//
// Workgroup = (16 tokens, 256 consecutive gate channels); thread = one channel.
// The weight column is read once per workgroup and the 16 tokens' features are
// workgroup-uniform loads; each channel's sum runs over r in order (fp32).
#include "gtr_internal.hpp"

namespace gtr {
namespace {

constexpr int GT_THREADS = 256;
constexpr int GT_TOKENS = 16;

template <int DT>
__global__ __launch_bounds__(GT_THREADS) void k_gate_proj(const void *__restrict__ feat,
                                                          const void *__restrict__ gw,
                                                          const float *__restrict__ gb,
                                                          float inv_tau, int rank, int hd,
                                                          int64_t n_tok, float *__restrict__ out) {
    const int j = blockIdx.y * GT_THREADS + threadIdx.x;
    if (j >= hd) return;  // no barriers below
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * GT_TOKENS;
    const int nt = static_cast<int>(n_tok - t0 < GT_TOKENS ? n_tok - t0 : GT_TOKENS);
    const float bias = gb[j];
    float acc[GT_TOKENS];
#pragma unroll
    for (int t = 0; t < GT_TOKENS; ++t) acc[t] = bias;
    for (int r = 0; r < rank; ++r) {
        const float w = ld<DT>(gw, static_cast<int64_t>(r) * hd + j);
#pragma unroll
        for (int t = 0; t < GT_TOKENS; ++t) {
            const int64_t tok = t0 + (t < nt ? t : nt - 1);  // in bounds; unused past nt
            acc[t] = fmaf(ld<DT>(feat, tok * rank + r), w, acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < GT_TOKENS; ++t)
        if (t < nt) out[(t0 + t) * hd + j] = log_sigmoid(acc[t]) * inv_tau;
}

}  // namespace

hipError_t gate_materialize(const GlaArgs &a, float *log_g, hipStream_t s) {
    const int64_t n_tok = static_cast<int64_t>(a.B) * a.L;
    const int hd = a.H * a.dk;
    const int64_t bx = (n_tok + GT_TOKENS - 1) / GT_TOKENS;
    if (bx > 0x7fffffff || a.rank <= 0) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(bx), static_cast<unsigned>((hd + GT_THREADS - 1) / GT_THREADS));
    switch (a.dtype) {
    case DT_F32:
        hipLaunchKernelGGL(k_gate_proj<DT_F32>, grid, dim3(GT_THREADS), 0, s, a.feat, a.gate_w,
                           a.gate_b, a.inv_tau, a.rank, hd, n_tok, log_g);
        break;
    case DT_F16:
        hipLaunchKernelGGL(k_gate_proj<DT_F16>, grid, dim3(GT_THREADS), 0, s, a.feat, a.gate_w,
                           a.gate_b, a.inv_tau, a.rank, hd, n_tok, log_g);
        break;
    case DT_BF16:
        hipLaunchKernelGGL(k_gate_proj<DT_BF16>, grid, dim3(GT_THREADS), 0, s, a.feat, a.gate_w,
                           a.gate_b, a.inv_tau, a.rank, hd, n_tok, log_g);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gtr
