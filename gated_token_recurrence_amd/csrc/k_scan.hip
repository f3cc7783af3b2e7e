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

// The same recurrence over the segments of an MFMA plan: thread = (sequence,
// state element); the sequence's segments are seg_id(seq N) .. seg_id((seq+1) N) - 1.
__global__ __launch_bounds__(NT) void k_state_scan_plan(float *__restrict__ U,
                                                        const float *__restrict__ G,
                                                        MfmaPlan pl, int64_t n_elem, int dk,
                                                        int dv) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x;
    if (e >= n_elem) return;
    const int64_t dd = static_cast<int64_t>(dk) * dv;
    const int64_t seq = e / dd;
    const int64_t el = e - seq * dd;
    const int c = static_cast<int>(el / dv);
    const int64_t s0 = seg_id(seq * pl.N, pl), s1 = seg_id((seq + 1) * pl.N, pl);
    float s = 0.f;
    constexpr int PF2 = 16;
    for (int64_t k0 = s0; k0 < s1; k0 += PF2) {
        float x[PF2], gg[PF2];
#pragma unroll
        for (int i = 0; i < PF2; ++i) {
            const bool ok = k0 + i < s1;
            x[i] = ok ? U[(k0 + i) * dd + el] : 0.f;
            gg[i] = ok ? G[(k0 + i) * dk + c] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < PF2; ++i) {
            if (k0 + i < s1) {
                U[(k0 + i) * dd + el] = s;
                s = expf(gg[i]) * s + x[i];
            }
        }
    }
}

}  // namespace

hipError_t state_scan_plan(float *U, const float *G, const MfmaPlan &pl, int n_seq, int dk,
                           int dv, hipStream_t s) {
    const int64_t n_elem = static_cast<int64_t>(n_seq) * dk * dv;
    const dim3 grid(static_cast<unsigned>((n_elem + NT - 1) / NT));
    hipLaunchKernelGGL(k_state_scan_plan, grid, dim3(NT), 0, s, U, G, pl, n_elem, dk, dv);
    return hipGetLastError();
}

hipError_t state_scan(float *U, const float *G, int n_seq, int n_units, int dk, int dv,
                      hipStream_t s) {
    const int64_t n_elem = static_cast<int64_t>(n_seq) * dk * dv;
    const dim3 grid(static_cast<unsigned>((n_elem + NT - 1) / NT));
    hipLaunchKernelGGL(k_state_scan, grid, dim3(NT), 0, s, U, G, n_elem, n_units, dk, dv);
    return hipGetLastError();
}

}  // namespace gtr
