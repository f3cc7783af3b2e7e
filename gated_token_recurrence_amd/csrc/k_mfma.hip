// k_mfma.hip -- chunkwise Key-only GLA on gfx950 matrix cores (16-bit I/O, dk = 64).
//
// GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"), Method §4
// "硬件感知分块推理算子": chunk summaries on the matrix units, a light boundary-state
// scan, and per-chunk outputs whose score tile stays in on-chip memory, with the
// output gate fused into the epilogue.  The recurrence, readout, RMSNorm and
// SiLU(z) gate are those of Method §1.
//
// Work split.  The T = B * H * N chunks of C tokens (N per sequence) are taken
// in sequence-major order and cut into equal ranges of Q chunks, one range per
// workgroup.  A range may run into the next sequence; the pieces of a range
// inside one sequence are its segments.  Two kernels run over the same ranges:
//   k_chunk<..., true>  (summary): per segment, U = sum_t k~_t v_t^T with
//       k~_t = k_t * prod_{r > t in segment} g_r, and the segment's summed log-gate;
//   k_chunk<..., false> (output):  per segment, from the incoming state the scan
//       produced, the chunks in order: readout, RMSNorm * rms_w * SiLU(z), store at
//       the token's grid position.
//
// Per chunk (a_i = in-chunk inclusive cumulative log2-gate, G = a at the chunk's
// last token):
//   o_i   = (q_i 2^a_i)^T S + sum_{j <= i} (sum_c (q_ic 2^a_ic)(k_jc 2^-a_jc)) v_j
//   S_new = Diag(2^G) S + sum_j (k_j 2^(G - a_j)) v_j^T
// q 2^a and k 2^(G - a) never exceed |q|, |k|; k 2^-a grows with the chunk's
// decay span, so a chunk whose span exceeds kSpanMax (log2 units) is instead
// run token by token in fp32 (S_t = Diag(g_t) S + k_t v_t^T, o_t = S_t^T q_t).
//
// The per-chunk steps (operand staging, matrix products, token-serial fallback,
// epilogue) live in mfma_common.hpp.  The next chunk's inputs are loaded into
// registers while the current one is computed: log_g and v as soon as phase 1
// has consumed the current ones, q and k after phase 2, z after the epilogue.
#include "mfma_common.hpp"

namespace gtr {
namespace {

using namespace mf;

template <int DT, int DV, int NB, bool SUM>
__global__ __launch_bounds__(NT, SUM ? (DV == 128 ? 2 : 4) : (DV == 128 ? 1 : 2)) void k_chunk(
    GlaArgs a, float *__restrict__ U, float *__restrict__ Gs, const float *__restrict__ Sx,
    MfmaPlan pl, MfmaPlan ps) {
    using T = Tile<DT, DV, NB, SUM>;
    __shared__ __attribute__((aligned(16))) char smem[T::K::BYTES];
    T t;
    t.init(a, smem);
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * pl.Q;
    const int64_t p1 = (p0 + pl.Q < pl.T) ? p0 + pl.Q : pl.T;
    if (p0 >= p1) return;  // the whole workgroup

    int64_t bh = p0 / pl.N;  // current sequence and chunk, advanced incrementally
    int64_t ch = p0 - bh * pl.N;
    t.rows_of(bh, ch, 0);
    __syncthreads();
    t.prefetch_main(0);
    t.prefetch_z(0);
    float gam = 0.f;  // summary: summed log2-gate of the current segment, channel l

    for (int64_t p = p0; p < p1; ++p) {
        const int cur = static_cast<int>((p - p0) & 1);
        const bool last_in_seq = (ch == pl.N - 1);
        if (p == p0 || ch == 0) {  // segment start: incoming state
            if (SUM)
                t.zero_state();
            else
                t.load_state(Sx + seg_id(p, ps) * DK * DV);
            gam = 0.f;
        }
        t.phase1();
        if (p + 1 < p1) t.rows_of(last_in_seq ? bh + 1 : bh, last_in_seq ? 0 : ch + 1, cur ^ 1);
        __syncthreads();  // B1: block totals, V, the next chunk's rows
        if (p + 1 < p1) t.prefetch_gv(cur ^ 1);  // phase 1 consumed log_g and v
        const bool slow = t.phase2(&gam);
        if (p + 1 < p1) t.prefetch_qk(cur ^ 1);  // phase 2 consumed q and k
        __syncthreads();  // B2: operand matrices

        if (SUM) {
            t.s_update();
            __syncthreads();  // LDS is rewritten by the next chunk
            if (p == p1 - 1 || last_in_seq) {  // segment end
                const int64_t sid = seg_id((p - ch > p0) ? p - ch : p0, pl);
                t.store_state(U + sid * DK * DV);
                if (t.w == 0) Gs[sid * DK + t.l] = gam;  // log2 units
            }
        } else {
            if (!slow) {
                t.inter();
                t.scores();
                t.s_update();
                __syncthreads();  // B3: score tiles
                t.intra();
            } else {
                __syncthreads();  // pairs with B3
                t.serial();
            }
            t.out_stage();
            __syncthreads();  // B4: output tile
            t.epilogue();
            if (p + 1 < p1) t.prefetch_z(cur ^ 1);
        }
        if (last_in_seq) {
            ch = 0;
            ++bh;
        } else {
            ++ch;
        }
    }
}

template <bool SUM, int DT, int DV, int NB>
hipError_t launch_t(const GlaArgs &a, float *U, float *G, const float *Sx, const MfmaPlan &pl,
                    const MfmaPlan &ps, hipStream_t st) {
    hipLaunchKernelGGL((k_chunk<DT, DV, NB, SUM>), dim3(static_cast<unsigned>(pl.n_wg)), dim3(NT),
                       0, st, a, U, G, Sx, pl, ps);
    return hipGetLastError();
}

template <bool SUM, int DT>
hipError_t launch_dt(const GlaArgs &a, float *U, float *G, const float *Sx, const MfmaPlan &pl,
                     const MfmaPlan &ps, hipStream_t st) {
    if (a.dv == 64) {
        if (a.chunk == 32) return launch_t<SUM, DT, 64, 2>(a, U, G, Sx, pl, ps, st);
        if (a.chunk == 64) return launch_t<SUM, DT, 64, 4>(a, U, G, Sx, pl, ps, st);
    } else if (a.dv == 128) {
        if (a.chunk == 32) return launch_t<SUM, DT, 128, 2>(a, U, G, Sx, pl, ps, st);
        if (a.chunk == 64) return launch_t<SUM, DT, 128, 4>(a, U, G, Sx, pl, ps, st);
    }
    return hipErrorInvalidValue;
}

template <bool SUM>
hipError_t launch(const GlaArgs &a, float *U, float *G, const float *Sx, const MfmaPlan &pl,
                  const MfmaPlan &ps, hipStream_t st) {
    if (a.dtype == DT_F16) return launch_dt<SUM, DT_F16>(a, U, G, Sx, pl, ps, st);
    if (a.dtype == DT_BF16) return launch_dt<SUM, DT_BF16>(a, U, G, Sx, pl, ps, st);
    return hipErrorInvalidValue;
}

int64_t gcd64(int64_t x, int64_t y) {
    while (y) {
        const int64_t t = x % y;
        x = y;
        y = t;
    }
    return x;
}

}  // namespace

bool mfma_supported(const GlaArgs &a) {
    return (a.dtype == DT_F16 || a.dtype == DT_BF16) && a.dk == DK && (a.dv == 64 || a.dv == 128) &&
           (a.chunk == 32 || a.chunk == 64);
}

MfmaPlan mfma_plan(const GlaArgs &a, int64_t chunks_per_wg) {
    MfmaPlan pl;
    pl.N = (a.L + a.chunk - 1) / a.chunk;
    pl.T = static_cast<int64_t>(a.B) * a.H * pl.N;
    pl.Q = chunks_per_wg;
    pl.n_wg = (pl.T + pl.Q - 1) / pl.Q;
    pl.lcm = pl.N / gcd64(pl.N, pl.Q) * pl.Q;
    pl.n_seg = seg_id(pl.T, pl);  // index of the (virtual) segment starting at T
    return pl;
}

void mfma_plans(const GlaArgs &a, int64_t chunks_per_wg, MfmaPlan *ps, MfmaPlan *po) {
    const int64_t N = (a.L + a.chunk - 1) / a.chunk;
    const int64_t T = static_cast<int64_t>(a.B) * a.H * N;
    int64_t q1 = chunks_per_wg, q2 = chunks_per_wg;
    if (chunks_per_wg <= 0) {
        // dv = 128 summary workgroups (eight waves at chunk 64) also take a whole CU
        const int64_t most1 = (a.dv == 128 && a.chunk == 64) ? kSummaryWorkgroups / 2 : kSummaryWorkgroups;
        const int64_t t1 = most1 < T ? most1 : T;
        q1 = (T + t1 - 1) / t1;
        // dv = 128 output workgroups take a whole CU (eight waves, or four at one wave
        // per SIMD): one per CU
        const int64_t most = a.dv == 128 ? kMfmaWorkgroups / 2 : kMfmaWorkgroups;
        const int64_t t2 = most < T ? most : T;
        const int64_t want = (T + t2 - 1) / t2;
        const int64_t m = (want + q1 / 2) / q1;
        q2 = q1 * (m > 1 ? m : 1);
    }
    *ps = mfma_plan(a, q1);
    *po = mfma_plan(a, q2);
}

hipError_t mfma_summary(const GlaArgs &a, const MfmaPlan &ps, float *U, float *G,
                        hipStream_t s) {
    return launch<true>(a, U, G, nullptr, ps, ps, s);
}

hipError_t mfma_output(const GlaArgs &a, const MfmaPlan &po, const MfmaPlan &ps, const float *Sx,
                       hipStream_t s) {
    return launch<false>(a, nullptr, nullptr, Sx, po, ps, s);
}

}  // namespace gtr
