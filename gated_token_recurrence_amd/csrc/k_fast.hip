// k_fast.hip -- single-launch chunkwise mixer for short sequences (16-bit I/O, dk = 64).
//
// GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"), Method §4
// "硬件感知分块推理算子": chunk summaries, a light boundary-state scan and
// per-chunk outputs.  The page benchmarks its operator with graph launch at
// about 1.6K tokens, where launch overhead is a large share of the time; this
// kernel runs the phases in one launch, one workgroup per chunk:
//   1. a workgroup takes the next chunk from a ticket counter, stages it
//      (operands stay in LDS), computes the chunk summary
//      U_n = sum_t (k_t 2^(G - a_t)) v_t^T from a zero state, writes U_n and the
//      chunk's decay 2^(G_n) per key channel, and raises the chunk's ready flag;
//   2. it forms the chunk's intra-chunk products (scores and P V), which need no
//      incoming state, while the chunks before it finish their summaries;
//   3. it waits for the ready flags of the chunks before it in its sequence and
//      builds its incoming state S_n = sum_{m < n} Diag(2^(G_{m+1} + ... +
//      G_{n-1})) U_m directly in the registers that hold the state, in order,
//      S <- Diag(2^G_m) S + U_m; the decays come from an LDS table that the whole
//      workgroup fills first, so the registers in flight hold only summaries
//      (eight predecessors' at dv = 64);
//   4. it adds the readout of that state, Q~ S, and finishes the outputs.
// Chunks are handed out in ticket order, so a workgroup only waits for
// workgroups that took their tickets earlier and are running; those wait only
// for earlier ones in turn, so every wait ends whatever the grid size and
// whatever else runs on the device (the waits are also bounded).  The last
// workgroup of a sequence to finish clears that sequence's flags, and the last
// workgroup of the launch clears the ticket counters, so the next launch (or
// graph replay) starts from zero.  A wait that gives up (after far longer than
// any real wait) makes the chunk's incoming state NaN, so its outputs show it
// instead of being silently wrong.
#include "mfma_common.hpp"

namespace gtr {
namespace {

using namespace mf;

// Counter block: [0] ticket, [1] finished workgroups, then per sequence one
// finished-workgroup count, then one ready flag per chunk.
template <int DT, int DV, int NB>
__global__ __launch_bounds__(NT, DV == 128 ? 1 : 2) void k_fast(GlaArgs a, float *__restrict__ U,
                                                                 float *__restrict__ Gs,
                                                                 unsigned *__restrict__ cnt,
                                                                 int N, unsigned spin_limit) {
    using T = Tile<DT, DV, NB, false>;
    __shared__ __attribute__((aligned(16))) char smem[T::K::BYTES];
    T t;
    t.init(a, smem);
    const int n_seq = a.B * a.H, T_all = n_seq * N;
    unsigned *ticket = cnt, *finished = cnt + 1, *seq_done = cnt + 2, *ready = cnt + 2 + n_seq;
    // the ticket is passed through the first LDS word (Q~ tile, first written in phase 2)
    int *s_ticket = reinterpret_cast<int *>(smem);
    __shared__ int s_gave_up;
    if (t.tid == 0)
        *s_ticket = static_cast<int>(
            __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    __syncthreads();
    const int p = *s_ticket;  // this workgroup's chunk
    const int bh = p / N, ch = p - bh * N;
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
    if (ch + 1 < N) {  // the last chunk's summary is never read
        if (!slow)
            t.s_update();
        else
            t.serial();  // token by token from zero: the final state is the summary
        // agent-coherent stores (no cache write-back needed), each thread waits for
        // its own to complete, then one flag for the workgroup
        t.store_state_coherent(U + p * dd);
        if (t.w == 0)
            __hip_atomic_store(Gs + static_cast<int64_t>(p) * DK + t.l, fexp2(gam), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t.tid == 0)
            __hip_atomic_store(ready + p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    t.zero_state();

    // ---- 2. the intra-chunk products, which do not need the incoming state, while
    // the chunks before this one finish theirs
    if (!slow) {
        t.zero_out();
        t.scores();
        __syncthreads();  // score tiles
        t.intra();
    }

    // ---- 3. wait for the chunks before this one (lane m of wave 0 polls chunk m's
    // flag with cache-bypassing loads); the summaries are then read the same way
    if (ch > 0) {
        if (t.w == 0) {
            const unsigned *fl = ready + static_cast<int64_t>(bh) * N;
            unsigned spins = 0;
            bool mine = t.l >= ch;  // lanes past the predecessors are done
            while (true) {
                if (!mine)
                    mine = __hip_atomic_load(fl + t.l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
                if (__builtin_amdgcn_read_exec() == __ballot(mine)) break;
                if (++spins >= spin_limit) break;
                __builtin_amdgcn_s_sleep(2);
            }
            if (t.l == 0) s_gave_up = spins >= spin_limit;
        }
        __syncthreads();  // (also: every wave is past its intra-chunk products)

        // S <- Diag(2^G_m) S + U_m over the chunks m before this one, in order
        const float *ub = U + static_cast<int64_t>(bh) * N * dd, *eb = Gs + static_cast<int64_t>(bh) * N * DK;
        if (!slow && ch * DK * 4 <= T::K::KN) {
            // the predecessors' decays into an LDS table first (the K^ area: scores
            // and the state update are done with it), every thread loading a few
            float *etab = reinterpret_cast<float *>(smem + T::K::O_KN);
            constexpr int PER = 64 * DK / NT;  // table entries per thread, 64 predecessors at most
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int x = t.tid + NT * i;  // entry: predecessor x / DK, channel x % DK
                if (x < ch * DK)
                    etab[x] = __hip_atomic_load(eb + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            constexpr int MB = DV == 64 ? 8 : 4;  // summaries in flight together
            for (int m0 = 0; m0 < ch; m0 += MB) {
                typename T::UIn in[MB];
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const int m = (m0 + i < ch) ? m0 + i : ch - 1;  // clamped, then skipped
                    t.state_u_load(in[i], ub + m * dd);
                }
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    if (m0 + i < ch) t.state_u_apply(in[i], etab + (m0 + i) * DK);
            }
        } else {
            constexpr int MB = DV == 64 ? 4 : 2;  // chunks whose loads are in flight together
            for (int m0 = 0; m0 < ch; m0 += MB) {
                typename T::StateIn in[MB];
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const int m = (m0 + i < ch) ? m0 + i : ch - 1;  // clamped, then skipped
                    t.state_in_load(in[i], ub + m * dd, eb + static_cast<int64_t>(m) * DK);
                }
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    if (m0 + i < ch) t.state_in_apply(in[i]);
            }
        }
        if (s_gave_up) t.poison_state();
    }

    // ---- 4. outputs: the readout of the incoming state added to the intra-chunk
    // products (token by token instead for a chunk past the matrix path's span)
    if (!slow) {
        t.template inter<true>();
    } else {
        __syncthreads();
        t.serial();
    }
    t.out_stage();
    __syncthreads();
    t.epilogue();

    // ---- counters back to zero: a sequence's flags once all its chunks have
    // passed their waits, the tickets once every workgroup has finished
    if (t.tid == 0) {
        if (__hip_atomic_fetch_add(seq_done + bh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            static_cast<unsigned>(N) - 1) {
            for (int m = 0; m < N; ++m)
                __hip_atomic_store(ready + static_cast<int64_t>(bh) * N + m, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(seq_done + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (__hip_atomic_fetch_add(finished, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            static_cast<unsigned>(T_all) - 1) {
            __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(finished, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
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

int64_t fast_counters(const GlaArgs &a) {
    return 2 + static_cast<int64_t>(a.B) * a.H + fast_chunks(a);
}

bool fast_supported(const GlaArgs &a) {
    return mfma_supported(a) && pick(a) != nullptr && (a.L + a.chunk - 1) / a.chunk <= 64;
}

hipError_t fast_launch(const GlaArgs &a, float *U, float *G, unsigned *cnt, unsigned spin_limit,
                       hipStream_t s) {
    const void *k = pick(a);
    const int64_t N = (a.L + a.chunk - 1) / a.chunk;
    if (!k || N > 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL(reinterpret_cast<void (*)(GlaArgs, float *, float *, unsigned *, int, unsigned)>(
                           const_cast<void *>(k)),
                       dim3(static_cast<unsigned>(fast_chunks(a))), dim3(NT), 0, s, a, U, G, cnt,
                       static_cast<int>(N), spin_limit);
    return hipGetLastError();
}

}  // namespace gtr
