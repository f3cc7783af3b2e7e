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
                                                   int n_units, int dk, int dv, bool log2_gates) {
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
                s = (log2_gates ? __builtin_amdgcn_exp2f(gg[i]) : expf(gg[i])) * s + x[i];
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

// The same recurrence with each element's chain of segments cut into P parts,
// one per wave, so that memory latency is paid about once: a wave loads all the
// segments of its part at once (64 consecutive state elements of one key
// channel: one 256-byte row per segment, and the decay as a wave-uniform value)
// and folds them into its own (decay product, partial state); the parts' folds
// are combined through LDS; each wave then writes its exclusive prefixes.
// Workgroup: (sequence, 64-element slice of the state).
template <int M, int P>
__global__ __launch_bounds__(64 * P) void k_scan_rows(float *__restrict__ U,
                                                      const float *__restrict__ G, MfmaPlan pl,
                                                      int dk, int dv) {
    __shared__ float sA[P][64], sB[P][64];
    const int64_t dd = static_cast<int64_t>(dk) * dv;
    const uint32_t slices = static_cast<uint32_t>(dk * dv / 64);  // 32-bit: no long division
    const uint32_t seq32 = blockIdx.x / slices;
    const int64_t seq = seq32;
    const int lane = threadIdx.x & 63;
    const int part = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const uint32_t el0 = (blockIdx.x - seq32 * slices) * 64;
    const int64_t el = el0 + lane;
    const int c = static_cast<int>(el0 / static_cast<uint32_t>(dv));  // the slice's key channel
    const int64_t s0 = seg_id(seq * pl.N, pl), s1 = seg_id((seq + 1) * pl.N, pl);
    const int64_t len = (s1 - s0 + P - 1) / P;  // <= M (checked by the host)
    const int64_t kb = s0 + part * len;
    const int n = static_cast<int>(kb < s1 ? (kb + len < s1 ? len : s1 - kb) : 0);
    float x[M], e[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int64_t k = (i < n) ? kb + i : s1 - 1;  // in bounds; unused past n
        const float xv = U[k * dd + el];
        const float gv = G[k * dk + c];
        x[i] = (i < n) ? xv : 0.f;
        e[i] = (i < n) ? __builtin_amdgcn_exp2f(gv) : 1.f;
    }
    float A = 1.f, B = 0.f;
#pragma unroll
    for (int i = 0; i < M; ++i) {
        B = e[i] * B + x[i];
        A *= e[i];
    }
    sA[part][lane] = A;
    sB[part][lane] = B;
    __syncthreads();
    float s = 0.f;  // state before this part's first segment
    for (int q = 0; q < part; ++q) s = sA[q][lane] * s + sB[q][lane];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        if (i < n) {
            U[(kb + i) * dd + el] = s;
            s = e[i] * s + x[i];
        }
    }
}

// k_scan_rows with four consecutive elements per lane (one 16-byte load per
// segment instead of four 4-byte ones): workgroup = (sequence, 256-element
// slice), four times fewer workgroups.  The four elements of a lane share one key
// channel (dv >= 64), and each element's fold is k_scan_rows' (the same results).
template <int M, int P>
__global__ __launch_bounds__(64 * P) void k_scan_rows4(float *__restrict__ U,
                                                       const float *__restrict__ G, MfmaPlan pl,
                                                       int dk, int dv) {
    __shared__ float sA[P][64];
    __shared__ float4 sB[P][64];
    const int64_t dd = static_cast<int64_t>(dk) * dv;
    const uint32_t slices = static_cast<uint32_t>(dk * dv / 256);
    const uint32_t seq32 = blockIdx.x / slices;
    const int64_t seq = seq32;
    const int lane = threadIdx.x & 63;
    const int part = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const uint32_t el0 = (blockIdx.x - seq32 * slices) * 256;
    const int64_t el = el0 + 4 * lane;
    const int c = static_cast<int>(static_cast<uint32_t>(el) / static_cast<uint32_t>(dv));
    const int64_t s0 = seg_id(seq * pl.N, pl), s1 = seg_id((seq + 1) * pl.N, pl);
    const int64_t len = (s1 - s0 + P - 1) / P;  // <= M (checked by the host)
    const int64_t kb = s0 + part * len;
    const int n = static_cast<int>(kb < s1 ? (kb + len < s1 ? len : s1 - kb) : 0);
    float4 x[M];
    float e[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int64_t k = (i < n) ? kb + i : s1 - 1;  // in bounds; unused past n
        const float4 xv = *reinterpret_cast<const float4 *>(U + k * dd + el);
        const float gv = G[k * dk + c];
        x[i] = (i < n) ? xv : make_float4(0.f, 0.f, 0.f, 0.f);
        e[i] = (i < n) ? __builtin_amdgcn_exp2f(gv) : 1.f;
    }
    float A = 1.f;
    float4 B = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < M; ++i) {
        B.x = e[i] * B.x + x[i].x;
        B.y = e[i] * B.y + x[i].y;
        B.z = e[i] * B.z + x[i].z;
        B.w = e[i] * B.w + x[i].w;
        A *= e[i];
    }
    sA[part][lane] = A;
    sB[part][lane] = B;
    __syncthreads();
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);  // state before this part's first segment
    for (int q = 0; q < part; ++q) {
        const float a = sA[q][lane];
        const float4 b = sB[q][lane];
        s.x = a * s.x + b.x;
        s.y = a * s.y + b.y;
        s.z = a * s.z + b.z;
        s.w = a * s.w + b.w;
    }
#pragma unroll
    for (int i = 0; i < M; ++i) {
        if (i < n) {
            *reinterpret_cast<float4 *>(U + (kb + i) * dd + el) = s;
            s.x = e[i] * s.x + x[i].x;
            s.y = e[i] * s.y + x[i].y;
            s.z = e[i] * s.z + x[i].z;
            s.w = e[i] * s.w + x[i].w;
        }
    }
}

// Few segments per sequence (at most M): one wave per (sequence, 64-element
// slice), W of them per workgroup, each lane loading its element of every
// segment at once and folding them in order.  With several slices per workgroup
// the launch has W times fewer workgroups than k_scan_rows (whose workgroups
// then carry a segment or two per wave, and dispatch, not memory, bounds it).
template <int M, int W>
__global__ __launch_bounds__(64 * W) void k_scan_slices(float *__restrict__ U,
                                                        const float *__restrict__ G, MfmaPlan pl,
                                                        int dk, int dv) {
    const int64_t dd = static_cast<int64_t>(dk) * dv;
    const uint32_t slices = static_cast<uint32_t>(dk * dv / 64);
    const uint32_t wv = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(threadIdx.x >> 6));
    const uint32_t sl = blockIdx.x * W + wv;  // global slice (the host sizes the grid exactly)
    const uint32_t seq32 = sl / slices;
    const int64_t seq = seq32;
    const int lane = threadIdx.x & 63;
    const uint32_t el0 = (sl - seq32 * slices) * 64;
    const int64_t el = el0 + lane;
    const int c = static_cast<int>(el0 / static_cast<uint32_t>(dv));
    const int64_t s0 = seg_id(seq * pl.N, pl), s1 = seg_id((seq + 1) * pl.N, pl);
    const int n = static_cast<int>(s1 - s0);  // <= M (checked by the host)
    float x[M], e[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int64_t k = (i < n) ? s0 + i : s1 - 1;  // in bounds; unused past n
        x[i] = U[k * dd + el];
        e[i] = __builtin_amdgcn_exp2f(G[k * dk + c]);
    }
    float st = 0.f;
#pragma unroll
    for (int i = 0; i < M; ++i) {
        if (i < n) {
            U[(s0 + i) * dd + el] = st;
            st = e[i] * st + x[i];
        }
    }
}

// The same fold in P parts (one wave each) for plain sequences of n_units units each (unit k of
// sequence seq at index seq n_units + k), any dv: each lane takes its own key
// channel.  Workgroup = (sequence, 64 consecutive state elements).  LOG2: the
// unit gate totals G are in log2 units (else natural).
template <int M, bool LOG2, int P>
__global__ __launch_bounds__(64 * P) void k_scan_rows_seq(float *__restrict__ U,
                                                          const float *__restrict__ G, int n_units,
                                                          int dk, int dv) {
    __shared__ float sA[P][64], sB[P][64];
    const int64_t dd = static_cast<int64_t>(dk) * dv;
    const uint32_t slices = static_cast<uint32_t>(dk * dv / 64);
    const uint32_t seq32 = blockIdx.x / slices;
    const int64_t seq = seq32;
    const int lane = threadIdx.x & 63;
    const int part = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t el = static_cast<int64_t>(blockIdx.x - seq32 * slices) * 64 + lane;
    const int c = static_cast<int>(el / dv);
    const int64_t s0 = seq * n_units, s1 = s0 + n_units;
    const int64_t len = (n_units + P - 1) / P;  // <= M (checked by the host)
    const int64_t kb = s0 + part * len;
    const int n = static_cast<int>(kb < s1 ? (kb + len < s1 ? len : s1 - kb) : 0);
    float x[M], e[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int64_t k = (i < n) ? kb + i : s1 - 1;  // in bounds; unused past n
        const float xv = U[k * dd + el];
        const float gv = G[k * dk + c];
        x[i] = (i < n) ? xv : 0.f;
        e[i] = (i < n) ? (LOG2 ? __builtin_amdgcn_exp2f(gv) : expf(gv)) : 1.f;
    }
    float A = 1.f, B = 0.f;
#pragma unroll
    for (int i = 0; i < M; ++i) {
        B = e[i] * B + x[i];
        A *= e[i];
    }
    sA[part][lane] = A;
    sB[part][lane] = B;
    __syncthreads();
    float st = 0.f;
    for (int q = 0; q < part; ++q) st = sA[q][lane] * st + sB[q][lane];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        if (i < n) {
            U[(kb + i) * dd + el] = st;
            st = e[i] * st + x[i];
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
    const dim3 rows_grid(static_cast<unsigned>(n_el / 64));
    const int64_t n_slices = n_el / 64;
    if (most <= 8 && n_slices % 16 == 0 && n_slices / 16 <= 0x7fffffff) {
        hipLaunchKernelGGL((k_scan_slices<8, 16>), dim3(static_cast<unsigned>(n_slices / 16)),
                           dim3(64 * 16), 0, s, U, G, pl, dk, dv);
    } else if (most <= 4 * 16 && (dk * dv) % 256 == 0) {
        // four parts (more parts measured no faster at 16.4K tokens: 44 segments per
        // sequence), four elements per lane (10.3 -> 8.4 us there)
        hipLaunchKernelGGL((k_scan_rows4<16, 4>), dim3(static_cast<unsigned>(n_el / 256)), dim3(NT),
                           0, s, U, G, pl, dk, dv);
    } else if (most <= 4 * 16) {
        hipLaunchKernelGGL((k_scan_rows<16, 4>), rows_grid, dim3(NT), 0, s, U, G, pl, dk, dv);
    } else if (most <= 4 * 32) {
        hipLaunchKernelGGL((k_scan_rows<32, 4>), rows_grid, dim3(NT), 0, s, U, G, pl, dk, dv);
    } else {
        hipLaunchKernelGGL(k_state_scan_plan, dim3(static_cast<unsigned>(n_el / NT)), dim3(NT), 0,
                           s, U, G, pl, dk, dv);
    }
    return hipGetLastError();
}

namespace {
template <int M, int P>
void launch_rows_seq(float *U, const float *G, int n_units, int dk, int dv, bool log2_gates,
                     dim3 grid, hipStream_t s) {
    if (log2_gates)
        hipLaunchKernelGGL((k_scan_rows_seq<M, true, P>), grid, dim3(64 * P), 0, s, U, G, n_units,
                           dk, dv);
    else
        hipLaunchKernelGGL((k_scan_rows_seq<M, false, P>), grid, dim3(64 * P), 0, s, U, G, n_units,
                           dk, dv);
}
}  // namespace

hipError_t state_scan(float *U, const float *G, int n_seq, int n_units, int dk, int dv,
                      hipStream_t s, bool log2_gates) {
    const int64_t n_elem = static_cast<int64_t>(n_seq) * dk * dv;
    if ((static_cast<int64_t>(dk) * dv) % 64 == 0 && n_units <= 16 * 16) {
        // the folds in parts: memory latency paid about once per sequence
        const dim3 grid(static_cast<unsigned>(n_elem / 64));
        if (n_units <= 4 * 16)
            launch_rows_seq<16, 4>(U, G, n_units, dk, dv, log2_gates, grid, s);
        else if (n_units <= 8 * 16)
            launch_rows_seq<16, 8>(U, G, n_units, dk, dv, log2_gates, grid, s);
        else
            launch_rows_seq<16, 16>(U, G, n_units, dk, dv, log2_gates, grid, s);
        return hipGetLastError();
    }
    const dim3 grid(static_cast<unsigned>((n_elem + NT - 1) / NT));
    hipLaunchKernelGGL(k_state_scan, grid, dim3(NT), 0, s, U, G, n_elem, n_units, dk, dv, log2_gates);
    return hipGetLastError();
}

}  // namespace gtr
