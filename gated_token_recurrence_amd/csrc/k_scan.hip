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

// The same recurrence over the segments of an MFMA plan (summed gates in log2
// units).  Workgroup = (sequence, slice of 256 state elements); its segments
// are seg_id(seq N) .. seg_id((seq + 1) N) - 1.  Segments are fetched in
// batches, the next batch's loads issued before the current batch's stores, so
// the dependent chain waits on memory about once per batch.  Loads past the
// last segment re-read the last one (in bounds, unused).
constexpr int SB = 16;

__global__ __launch_bounds__(NT) void k_state_scan_plan(float *__restrict__ U,
                                                        const float *__restrict__ G,
                                                        MfmaPlan pl, int dk, int dv) {
    const int64_t dd = static_cast<int64_t>(dk) * dv;
    const int slices = static_cast<int>(dd / NT);
    const int64_t seq = blockIdx.x / slices;
    const int64_t el = static_cast<int64_t>(blockIdx.x % slices) * NT + threadIdx.x;
    // channel of this wave's 64 consecutive elements (dv >= 64): wave-uniform
    const int c = __builtin_amdgcn_readfirstlane(static_cast<int>(el / dv));
    const int64_t s0 = seg_id(seq * pl.N, pl), s1 = seg_id((seq + 1) * pl.N, pl);
    float *u = U + el;
    const float *gp = G + c;
    // batch starting at segment kb: values of segments kb .. kb + SB - 1; past the
    // last segment the pointers stop advancing (in bounds, values unused)
    auto fetch = [&](int64_t kb, float *xo, float *go) {
        const int64_t base = (kb < s1) ? kb : s1 - 1;
        const int nb = (s1 - base < SB) ? static_cast<int>(s1 - base) : SB;
        const float *up = u + base * dd;
        const float *gq = gp + base * dk;
#pragma unroll
        for (int i = 0; i < SB; ++i) {
            xo[i] = *up;
            go[i] = *gq;
            const bool adv = i + 1 < nb;
            up += adv ? dd : 0;
            gq += adv ? dk : 0;
        }
    };
    float x[SB], gg[SB];
    fetch(s0, x, gg);
    float s = 0.f;
    for (int64_t k0 = s0; k0 < s1; k0 += SB) {
        float xn[SB], gn[SB];
        fetch(k0 + SB, xn, gn);
        const int n = (s1 - k0 < SB) ? static_cast<int>(s1 - k0) : SB;
        float *ub = u + k0 * dd;
#pragma unroll
        for (int i = 0; i < SB; ++i) {
            if (i < n) {
                *ub = s;
                s = __builtin_amdgcn_exp2f(gg[i]) * s + x[i];
                ub += dd;
            }
        }
#pragma unroll
        for (int i = 0; i < SB; ++i) {
            x[i] = xn[i];
            gg[i] = gn[i];
        }
    }
}

// The same recurrence with each element's chain of segments cut into P parts
// of at most M segments, so that memory latency is paid about once: a part
// loads all its segments at once and folds them into its own (decay product,
// partial state); the parts' folds are combined through LDS; each part then
// writes its exclusive prefixes.  Workgroup: NT / P consecutive state elements
// of one sequence x P parts.
template <int P, int M>
__global__ __launch_bounds__(NT) void k_scan_parts(float *__restrict__ U,
                                                   const float *__restrict__ G, MfmaPlan pl,
                                                   int dk, int dv) {
    constexpr int EPW = NT / P;
    __shared__ float sA[P][EPW], sB[P][EPW];
    const int64_t dd = static_cast<int64_t>(dk) * dv;
    const int part = threadIdx.x / EPW, le = threadIdx.x % EPW;
    const int64_t ge = static_cast<int64_t>(blockIdx.x) * EPW + le;  // dd % EPW == 0
    const int64_t seq = ge / dd, el = ge - seq * dd;
    const int c = static_cast<int>(el / dv);
    const int64_t s0 = seg_id(seq * pl.N, pl), s1 = seg_id((seq + 1) * pl.N, pl);
    const int64_t len = (s1 - s0 + P - 1) / P;  // <= M (checked by the host)
    const int64_t kb = s0 + part * len;
    const int64_t ke = (kb + len < s1) ? kb + len : s1;
    float x[M], e[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int64_t k = kb + i;
        const bool ok = k < ke;
        x[i] = ok ? U[k * dd + el] : 0.f;
        e[i] = ok ? __builtin_amdgcn_exp2f(G[k * dk + c]) : 1.f;
    }
    float A = 1.f, B = 0.f;
#pragma unroll
    for (int i = 0; i < M; ++i) {
        B = e[i] * B + x[i];
        A *= e[i];
    }
    sA[part][le] = A;
    sB[part][le] = B;
    __syncthreads();
    float s = 0.f;  // state before this part's first segment
    for (int q = 0; q < part; ++q) s = sA[q][le] * s + sB[q][le];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int64_t k = kb + i;
        if (k < ke) {
            U[k * dd + el] = s;
            s = e[i] * s + x[i];
        }
    }
}

}  // namespace

hipError_t state_scan_plan(float *U, const float *G, const MfmaPlan &pl, int n_seq, int dk,
                           int dv, hipStream_t s) {
    const int64_t dd = static_cast<int64_t>(dk) * dv;
    if (dd % NT != 0 || dv < 64) return hipErrorInvalidValue;
    const int64_t n_el = static_cast<int64_t>(n_seq) * dd;
    const int64_t most = (pl.N + pl.Q - 1) / pl.Q + 1;  // segments of one sequence, at most
    if (most <= 8 * 16) {
        hipLaunchKernelGGL((k_scan_parts<8, 16>), dim3(static_cast<unsigned>(n_el / (NT / 8))),
                           dim3(NT), 0, s, U, G, pl, dk, dv);
    } else if (most <= 32 * 16) {
        hipLaunchKernelGGL((k_scan_parts<32, 16>), dim3(static_cast<unsigned>(n_el / (NT / 32))),
                           dim3(NT), 0, s, U, G, pl, dk, dv);
    } else {
        hipLaunchKernelGGL(k_state_scan_plan, dim3(static_cast<unsigned>(n_el / NT)), dim3(NT), 0,
                           s, U, G, pl, dk, dv);
    }
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
