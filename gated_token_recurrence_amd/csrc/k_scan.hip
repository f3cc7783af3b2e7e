// k_scan.hip -- boundary-state scan between chunks (or segments of chunks).
//
// GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"), Method §4: the
// states passed between chunks are cheap to compute and are carried forward
// sequentially over contiguous, coalesced memory.  For unit n of a sequence,
// with summary U_n (dk x dv) and summed log-gate Gamma_n (dk):
//     S_before(0) = 0,   S_before(n+1) = Diag(exp(Gamma_n)) S_before(n) + U_n.
// The kernel overwrites U_n with S_before(n) in place.  One thread owns one
// state element of one sequence; neighbouring threads own neighbouring
// elements, so every step is a coalesced read and write of the unit's state.
#include "gtr_internal.hpp"

namespace gtr {
namespace {

constexpr int NT = 256;
constexpr int PF = 8;  // units fetched ahead of the dependent chain

__global__ __launch_bounds__(NT) void k_state_scan(float *__restrict__ U,
                                                   const float *__restrict__ G, int64_t n_elem,
                                                   int n_units, int dk, int dv) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x;
    if (e >= n_elem) return;
    const int64_t dd = static_cast<int64_t>(dk) * dv;
    const int64_t seq = e / dd;
    const int64_t el = e - seq * dd;
    const int c = static_cast<int>(el / dv);
    float *u = U + seq * n_units * dd + el;
    const float *g = G + seq * n_units * dk + c;
    float s = 0.f;
    for (int n0 = 0; n0 < n_units; n0 += PF) {
        float x[PF], gg[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const bool ok = n0 + i < n_units;
            x[i] = ok ? u[static_cast<int64_t>(n0 + i) * dd] : 0.f;
            gg[i] = ok ? g[static_cast<int64_t>(n0 + i) * dk] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            if (n0 + i < n_units) {
                u[static_cast<int64_t>(n0 + i) * dd] = s;
                s = expf(gg[i]) * s + x[i];
            }
        }
    }
}

}  // namespace

hipError_t state_scan(float *U, const float *G, int n_seq, int n_units, int dk, int dv,
                      hipStream_t s) {
    const int64_t n_elem = static_cast<int64_t>(n_seq) * dk * dv;
    const dim3 grid(static_cast<unsigned>((n_elem + NT - 1) / NT));
    hipLaunchKernelGGL(k_state_scan, grid, dim3(NT), 0, s, U, G, n_elem, n_units, dk, dv);
    return hipGetLastError();
}

}  // namespace gtr
