// k_fast.hip -- single-launch chunkwise mixer for short sequences (16-bit I/O, dk = 64).
//
// GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"), Method §4
// "硬件感知分块推理算子": chunk summaries, a light boundary-state scan and
// per-chunk outputs.  The page benchmarks its operator with graph launch at
// about 1.6K tokens, where launch overhead is a large share of the time; this
// kernel runs all three phases in one cooperative launch, one workgroup per
// chunk, with two grid-wide barriers between them:
//   1. every workgroup stages its chunk (operands stay in LDS), computes the
//      chunk summary U_n = sum_t (k_t 2^(G - a_t)) v_t^T from a zero state and
//      writes U_n and the chunk's summed log2-gate G_n;
//   2. the summaries are scanned over the chunks of each sequence, spread over
//      all threads of the grid: U_n <- S before chunk n;
//   3. every workgroup reads its incoming state and produces its outputs from
//      the operands still in LDS.
// The launch needs every workgroup resident at once; the host only takes this
// path when the grid fits.
#include <hip/hip_cooperative_groups.h>

#include "mfma_common.hpp"

namespace gtr {
namespace {

using namespace mf;
namespace cg = cooperative_groups;

template <int DT, int DV, int NB>
__global__ __launch_bounds__(NT, DV == 128 ? 1 : 2) void k_fast(GlaArgs a, float *__restrict__ U,
                                                                 float *__restrict__ Gs,
                                                                 int64_t N) {
    using T = Tile<DT, DV, NB, false>;
    __shared__ __attribute__((aligned(16))) char smem[T::K::BYTES];
    T t;
    t.init(a, smem);
    const int64_t p = blockIdx.x;  // this workgroup's chunk
    const int64_t bh = p / N, ch = p - bh * N;
    constexpr int64_t dd = static_cast<int64_t>(DK) * DV;

    // ---- 1. stage the chunk; its summary from a zero state
    t.rows_of(bh, ch, 0);
    __syncthreads();
    t.prefetch_main(0);
    t.prefetch_z(0);
    float gam = 0.f;
    t.phase1();
    __syncthreads();
    const bool slow = t.phase2(&gam);
    __syncthreads();
    t.zero_state();
    if (!slow)
        t.s_update();
    else
        t.serial();  // token by token from zero: the final state is the summary
    t.store_state(U + p * dd);
    if (t.w == 0) Gs[p * DK + t.l] = gam;

    cg::this_grid().sync();

    // ---- 2. exclusive scan of the summaries over each sequence's chunks
    {
        const int64_t n_seq = static_cast<int64_t>(gridDim.x) / N;
        const int64_t total = n_seq * dd;
        const int64_t stride = static_cast<int64_t>(gridDim.x) * NT;
        for (int64_t e = p * NT + t.tid; e < total; e += stride) {
            const int64_t seq = e / dd, el = e - seq * dd;
            const int c = static_cast<int>(el / DV);
            float *u = U + seq * N * dd + el;
            const float *gp = Gs + seq * N * DK + c;
            float s = 0.f;
            constexpr int SB = 16;
            for (int64_t n0 = 0; n0 < N; n0 += SB) {
                float x[SB], gg[SB];
#pragma unroll
                for (int i = 0; i < SB; ++i) {
                    const int64_t n = (n0 + i < N) ? n0 + i : N - 1;
                    x[i] = u[n * dd];
                    gg[i] = gp[n * DK];
                }
#pragma unroll
                for (int i = 0; i < SB; ++i) {
                    if (n0 + i < N) {
                        u[(n0 + i) * dd] = s;
                        s = fexp2(gg[i]) * s + x[i];
                    }
                }
            }
        }
    }

    cg::this_grid().sync();

    // ---- 3. outputs from the incoming state and the staged operands
    t.load_state(U + p * dd);
    if (!slow) {
        t.inter();
        t.scores();
        __syncthreads();  // score tiles
        t.intra();
    } else {
        __syncthreads();
        t.serial();
    }
    t.sum_squares();
    __syncthreads();
    t.epilogue();
}

template <int DT, int DV, int NB>
const void *kernel_ptr() {
    return reinterpret_cast<const void *>(&k_fast<DT, DV, NB>);
}

const void *pick(const GlaArgs &a) {
    const bool f16 = a.dtype == DT_F16;
    if (a.dv == 64 && a.chunk == 32) return f16 ? kernel_ptr<DT_F16, 64, 2>() : kernel_ptr<DT_BF16, 64, 2>();
    if (a.dv == 64 && a.chunk == 64) return f16 ? kernel_ptr<DT_F16, 64, 4>() : kernel_ptr<DT_BF16, 64, 4>();
    if (a.dv == 128 && a.chunk == 32) return f16 ? kernel_ptr<DT_F16, 128, 2>() : kernel_ptr<DT_BF16, 128, 2>();
    if (a.dv == 128 && a.chunk == 64) return f16 ? kernel_ptr<DT_F16, 128, 4>() : kernel_ptr<DT_BF16, 128, 4>();
    return nullptr;
}

}  // namespace

int64_t fast_chunks(const GlaArgs &a) {
    const int64_t N = (a.L + a.chunk - 1) / a.chunk;
    return static_cast<int64_t>(a.B) * a.H * N;
}

// Workgroups of this variant that can be resident at once on the current
// device (0 if cooperative launch is unavailable).
int64_t fast_capacity(const GlaArgs &a) {
    if (!mfma_supported(a)) return 0;
    const void *k = pick(a);
    if (!k) return 0;
    int dev = 0, coop = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop)
        return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, NT, 0) != hipSuccess) return 0;
    return static_cast<int64_t>(cus) * per_cu;
}

hipError_t fast_launch(const GlaArgs &a, float *U, float *G, hipStream_t s) {
    const void *k = pick(a);
    if (!k) return hipErrorInvalidValue;
    GlaArgs args = a;
    int64_t N = (a.L + a.chunk - 1) / a.chunk;
    void *params[] = {&args, &U, &G, &N};
    return hipLaunchCooperativeKernel(k, dim3(static_cast<unsigned>(fast_chunks(a))), dim3(NT),
                                      params, 0, s);
}

}  // namespace gtr
