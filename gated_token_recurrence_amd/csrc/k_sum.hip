// k_sum.hip -- segment summaries with per-wave partial sums (16-bit I/O, dk = 64,
// dv = 64, chunk 64).
//
// GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"), Method §4
// "硬件感知分块推理算子": the chunk summaries that the boundary-state scan
// combines, formed on the matrix units.  For a segment (consecutive chunks of
// one sequence) the summary is the state its tokens build from zero,
//   U = sum_t (prod_{s > t in segment} g_s) k_t v_t^T,
// and its summed log2-gate.  A workgroup walks its chunks last to first, so the
// decay from a token to the segment's end is known when the token is reached:
// with R the summed log2-gate of the segment's later chunks, G the chunk's and
// a_t the in-chunk inclusive cumulative one, token t enters as
//   k_t 2^(R + G - a_t) v_t^T,
// and the factor never exceeds 1, so k 2^(...) is held as hi + lo of the I/O
// type (fp16 or bf16), v enters the products as stored, and the sums need no
// rescaling.
//
// The sum over a chunk's tokens is split by token: wave w takes tokens
// [16 w, 16 w + 16) of every chunk and keeps its own partial U (all dk x dv
// entries, in MFMA accumulators).  Its operands K~^T and V (16 tokens each) go
// through a wave-private LDS area and come back with the transposing load as
// 16x16x16 MFMA operands, so the only cross-wave exchange per chunk is the
// sub-block gate totals (one barrier).  At a segment's end the four partials
// are added through LDS.
//
// dv = 128 runs eight waves in two value halves: waves w and w + 4 take the same
// 16 tokens, and wave w keeps the partial of value columns [64 (w / 4),
// 64 (w / 4) + 64) (a full-width partial would need twice the accumulators).
// The pair splits the key channels instead: wave w reads k and log_g of
// channels [32 (w / 4), 32 (w / 4) + 32) only, forms their gates and K~, and
// writes K~ into an LDS area the pair shares; a second barrier per chunk then
// lets both read all 64 channels.  So k and log_g are read once, and each wave
// stages only its half of V.
//
// Low-rank gate variant (LRG): the gates come from the tokens' rank-16
// features (Method §1: a light low-rank projection with a temperature), four
// 16x16x16 products against the head's projection held in registers, then
// logsigmoid / tau; log_g is not read.
#include <type_traits>

#include "mfma_common.hpp"

namespace gtr {
namespace {

using namespace mf;

template <int DT, int DV, bool RES, bool LRG>
struct SumTile {
    static constexpr bool F16 = DT == DT_F16;
    static constexpr int C = 64, NB = 4;
    static constexpr int CS = DV / 64;   // value halves (dv = 128: two groups of four waves)
    static constexpr int NW = 4 * CS;    // waves
    static constexpr int NTH = 64 * NW;  // threads
    static constexpr int ND = 4;         // value tiles of a wave's partial (its 64 columns)
    static constexpr int NE = 2;         // 16-byte value pieces per lane
    static constexpr int SUB = 16 * 64;  // elements of one [16 tokens][64 columns] matrix
    static constexpr int NK = 2 / CS;    // 32-channel key blocks a wave forms (dv = 128: one)
    // LDS (bytes): per token group K~ hi, lo ([16][64] each, shared by the group's
    // waves); per wave V ([16][64]); gate totals (two chunk buffers); per-wave
    // tables.  The segment-end reduction reuses the start of the area for four
    // [64][64] fp32 partials (one value half at a time).
    static constexpr int O_K = 0;                            // [4 groups][hi, lo][SUB]
    static constexpr int O_V = O_K + 4 * 2 * SUB * 2;        // [NW][SUB]
    static constexpr int O_TOT = O_V + NW * SUB * 2;         // float [2][NB][DK]
    static constexpr int O_TAB = O_TOT + 2 * NB * DK * 4;    // float [NW waves][2][DK]
    static constexpr int BYTES_MAIN = O_TAB + NW * 2 * DK * 4;
    static constexpr int RED_BYTES = 4 * 64 * 68 * 4;        // one 64-column half at a time
    static constexpr int BYTES = BYTES_MAIN > RED_BYTES ? BYTES_MAIN : RED_BYTES;

    GlaArgs a;
    char *smem;
    uint16_t *sKh, *sKl, *sV;
    float *sTab;
    int w, tw, hv, l, lr, g;  // wave, its token rows [16 tw, 16 tw + 16), its value half
    // inputs of the next two chunks (register sets alternate by chunk); pr: the
    // previous block's output, added to v where v is consumed
    uint4 pk[2][NK], pv[2][NE], pr[2][RES ? NE : 1];
    float4 pg[2][LRG ? 1 : 2 * NK];  // log_g (LRG: the gate features pf instead)
    uint2 pf[2];
    LowRankGate<DT> lg;
    float cs[8 * NK];  // cumulative gates of the wave's channels: 32 kap + 8 g + s, kap of its blocks
    int kap0;          // first 32-channel key block of the wave
    f32x4 U[4][ND];  // U[ct][dt][r] = partial U[16 ct + 4 g + r][64 hv + 16 dt + lr]
    float R;         // summed log2-gate of the segment's chunks after this one, channel l

    __device__ __forceinline__ void init(const GlaArgs &args, char *sm) {
        a = args;
        smem = sm;
        const int tid = threadIdx.x;
        w = __builtin_amdgcn_readfirstlane(tid >> 6);
        tw = w & 3;
        hv = w >> 2;
        l = tid & 63;
        lr = l & 15;
        g = l >> 4;
        kap0 = CS == 1 ? 0 : hv;
        sKh = reinterpret_cast<uint16_t *>(sm + O_K) + tw * 2 * SUB;
        sKl = sKh + SUB;
        sV = reinterpret_cast<uint16_t *>(sm + O_V) + w * SUB;
        sTab = reinterpret_cast<float *>(sm + O_TAB) + w * 2 * DK;
    }

    // row ((b L + grid position) H + h) of this lane's token of chunk ch of
    // sequence (b, h); a token past the end of the sequence takes the last token's
    // row (its values reach only the sequence's final state, which is never used)
    __device__ __forceinline__ int64_t row_of(uint32_t b, uint32_t h, int64_t ch, int64_t &tok) const {
        const uint32_t L32 = static_cast<uint32_t>(a.L);
        const uint32_t t0 = static_cast<uint32_t>(ch) * C + 16 * tw + lr;
        uint32_t t = t0 < L32 ? t0 : L32 - 1;
        if (a.direction & 1) t = L32 - 1 - t;
        uint32_t pos = t;
        if (a.direction >= 2) {
            const uint32_t gh = static_cast<uint32_t>(a.gh);
            const uint32_t c = t / gh;
            pos = (t - c * gh) * static_cast<uint32_t>(a.gw) + c;
        }
        tok = static_cast<int64_t>(b) * a.L + pos;
        return tok * a.H + h;
    }

    template <int S>
    __device__ __forceinline__ void prefetch_g(int64_t row, int64_t tok) {
        if constexpr (LRG) {
            pf[S] = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(a.feat) +
                                                     tok * kFusedGateRank + 4 * g);
        } else {
#pragma unroll
            for (int j = 0; j < NK; ++j) {
                const int c0 = 32 * (kap0 + j) + 8 * g;
                pg[S][2 * j] = *reinterpret_cast<const float4 *>(a.log_g + row * DK + c0);
                pg[S][2 * j + 1] = *reinterpret_cast<const float4 *>(a.log_g + row * DK + c0 + 4);
            }
        }
    }

    template <int S>
    __device__ __forceinline__ void prefetch_kv(int64_t row) {
#pragma unroll
        for (int j = 0; j < NK; ++j)
            pk[S][j] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) + row * DK +
                                                     32 * (kap0 + j) + 8 * g);
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int d0 = 64 * hv + 32 * e + 8 * g;
            pv[S][e] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) + row * DV + d0);
            if constexpr (RES)
                pr[S][e] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.resid) + row * DV + d0);
        }
    }

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) U[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        R = 0.f;
    }

    // cumulative gates of the wave's tokens (natural-log units) and the sub-block
    // totals into buffer buf
    template <int buf>
    __device__ __forceinline__ void gates() {
        if constexpr (LRG) {
            lg.gates(pf[buf], cs);
        } else {
#pragma unroll
            for (int q4 = 0; q4 < 2 * NK; ++q4) {
                cs[4 * q4] = pg[buf][q4].x; cs[4 * q4 + 1] = pg[buf][q4].y;
                cs[4 * q4 + 2] = pg[buf][q4].z; cs[4 * q4 + 3] = pg[buf][q4].w;
            }
        }
        row_scan(cs);
        if (lr == 15) {
            float *tot = reinterpret_cast<float *>(smem + O_TOT) + (buf * NB + tw) * DK;
#pragma unroll
            for (int j = 0; j < NK; ++j) {
                float *dst = tot + 32 * (kap0 + j) + 8 * g;
                *reinterpret_cast<float4 *>(dst) =
                    make_float4(cs[8 * j], cs[8 * j + 1], cs[8 * j + 2], cs[8 * j + 3]);
                *reinterpret_cast<float4 *>(dst + 4) =
                    make_float4(cs[8 * j + 4], cs[8 * j + 5], cs[8 * j + 6], cs[8 * j + 7]);
            }
        }
    }

    // (after the barrier) the table, K~ = k 2^(R + G - a) and V into the wave's LDS area
    template <int buf>
    __device__ __forceinline__ void stage() {
        const float *tot = reinterpret_cast<const float *>(smem + O_TOT) + buf * NB * DK;
        float r_l = 0.f, tot_l = 0.f;
#pragma unroll
        for (int J = 0; J < NB; ++J) {
            const float t = tot[J * DK + l];
            if (J < tw) r_l += t;
            tot_l += t;
        }
        tot_l *= kLog2e;
        sTab[l] = R + tot_l - r_l * kLog2e;  // R + G - r (log2), channel l
        R += tot_l;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int c0 = 32 * (kap0 + j) + 8 * g;
            float gr[8], kt[8];
#pragma unroll
            for (int h4 = 0; h4 < 2; ++h4) {
                const float4 x = *reinterpret_cast<const float4 *>(sTab + c0 + 4 * h4);
                gr[4 * h4] = x.x; gr[4 * h4 + 1] = x.y; gr[4 * h4 + 2] = x.z; gr[4 * h4 + 3] = x.w;
            }
            unpack8<DT>(pk[buf][j], kt);
#pragma unroll
            for (int s = 0; s < 8; ++s) kt[s] *= fexp2(fmaf(-cs[8 * j + s], kLog2e, gr[s]));
            uint32_t hi[4], lo[4];
            split_pk<F16>(kt, hi, lo);
            const int off = swn(lr, c0);
            *reinterpret_cast<uint4 *>(sKh + off) = u4(hi);
            *reinterpret_cast<uint4 *>(sKl + off) = u4(lo);
        }
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int d0 = 32 * e + 8 * g;  // column within the wave's half
            uint4 x = pv[buf][e];
            if constexpr (RES) x = add_io<DT>(x, pr[buf][e]);  // stack residual
            *reinterpret_cast<uint4 *>(sV + swn(lr, d0)) = x;
        }
    }

    // transposing read of a [16 tokens][64] matrix: lane column cb + lr, tokens
    // 4 g .. 4 g + 3 (the k slots of a 16x16x16 operand)
    __device__ __forceinline__ s16x4 op16(const uint16_t *m, int cb) const {
        return ld_tr(m + swn(4 * g + (lr >> 2), cb + 4 * (lr & 3)));
    }

    // U += K~^T V over the wave's 16 tokens
    __device__ __forceinline__ void accumulate() {
        s16x4 bv[ND];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) bv[dt] = op16(sV, 16 * dt);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const s16x4 ah = op16(sKh, 16 * ct);
            const s16x4 al = op16(sKl, 16 * ct);
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                U[ct][dt] = mma16<F16>(ah, bv[dt], U[ct][dt]);
                U[ct][dt] = mma16<F16>(al, bv[dt], U[ct][dt]);
            }
        }
    }

    // segment end: the four token partials of each value half added through LDS,
    // one half at a time ([token group][column][channel], rows padded to 68
    // floats); every wave then sums 64 / NW channels for every column of that half
    // (lane = column) and stores them as whole 256-byte rows
    __device__ __forceinline__ void finish(float *dst, float *gdst) {
        constexpr int RS = 68;
        constexpr int CH = 64 / NW;  // channels summed per wave
        float *red = reinterpret_cast<float *>(smem);  // [4][64 columns][RS]
#pragma unroll
        for (int h = 0; h < CS; ++h) {
            __syncthreads();  // the LDS area is free (operands, previous half)
            if (hv == h) {
                float *m = red + tw * 64 * RS + lr * RS + 4 * g;
#pragma unroll
                for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        *reinterpret_cast<f32x4 *>(m + 16 * d4 * RS + 16 * ct) = U[ct][d4];
            }
            __syncthreads();
            const float *m = red + l * RS + CH * w;
            float sum[CH];
#pragma unroll
            for (int j4 = 0; j4 < CH / 4; ++j4) {
                f32x4 x = *reinterpret_cast<const f32x4 *>(m + 4 * j4);
#pragma unroll
                for (int q = 1; q < 4; ++q) {
                    const f32x4 y = *reinterpret_cast<const f32x4 *>(m + q * 64 * RS + 4 * j4);
                    x[0] += y[0]; x[1] += y[1]; x[2] += y[2]; x[3] += y[3];
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) sum[4 * j4 + r] = x[r];
            }
            float *o = dst + (CH * w) * DV + 64 * h + l;
#pragma unroll
            for (int j = 0; j < CH; ++j) o[j * DV] = sum[j];
        }
        if (w == 0) gdst[l] = R;
        __syncthreads();  // the LDS area is rewritten by the next chunk
    }
};

template <int DT, int DV, bool RES, bool LRG>
__global__ __launch_bounds__(64 * 4 * (DV / 64), DV == 64 ? 2 : 1) void k_sum(GlaArgs a, float *__restrict__ Uo,
                                                                             float *__restrict__ Gs, MfmaPlan pl) {
    using T = SumTile<DT, DV, RES, LRG>;
    static_assert(T::NTH == 64 * 4 * (DV / 64), "launch bounds");
    __shared__ __attribute__((aligned(16))) char smem[T::BYTES];
    T t;
    t.init(a, smem);
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * pl.Q;
    const int64_t p1 = (p0 + pl.Q < pl.T) ? p0 + pl.Q : pl.T;
    if (p0 >= p1) return;  // the whole workgroup

    // Chunks last to first.  Cursors (b, h, ch): the current chunk's image, head and
    // index in its sequence; (fb, fh, fch): the chunk two before it, whose inputs
    // are loaded while the current one is worked on (register set = chunk parity,
    // which also picks the gate-total buffer).  Tracked incrementally: no divisions
    // in the loop.
    struct Cur {
        uint32_t b, h;
        int64_t ch;
    };
    const int64_t bh1 = (p1 - 1) / pl.N;
    Cur cur{static_cast<uint32_t>(bh1 / a.H), static_cast<uint32_t>(bh1 % a.H), (p1 - 1) - bh1 * pl.N};
    Cur far = cur;
    auto back = [&](Cur &c) {
        if (c.ch == 0) {
            c.ch = pl.N - 1;
            if (c.h == 0) {
                c.h = static_cast<uint32_t>(a.H) - 1;
                --c.b;
            } else {
                --c.h;
            }
        } else {
            --c.ch;
        }
    };
    {
        int64_t tok, tok1;
        const int64_t row = t.row_of(far.b, far.h, far.ch, tok);
        t.template prefetch_g<0>(row, tok);
        t.template prefetch_kv<0>(row);
        back(far);
        tok1 = tok;
        const int64_t row1 = (p1 - 2 >= p0) ? t.row_of(far.b, far.h, far.ch, tok1) : row;
        t.template prefetch_g<1>(row1, tok1);
        t.template prefetch_kv<1>(row1);
        back(far);  // now two before the current chunk
    }
    if constexpr (LRG) {  // weights of the last chunk's head
        t.lg.load(a, cur.h, t.lr, t.g);
        t.lg.ready();
    }
    t.zero();
    auto step = [&](auto S_, int64_t p) {
        constexpr int S = decltype(S_)::value;
        // Loads are issued every step (past the range's first chunk they re-read
        // the current chunk's rows, unused), so that the wait-count bookkeeping
        // sees the same load sequence each time and never has to drain the queue.
        const bool ahead = p - 2 >= p0;
        int64_t tok;
        const int64_t row = ahead ? t.row_of(far.b, far.h, far.ch, tok) : t.row_of(cur.b, cur.h, cur.ch, tok);
        // the gates and the K~ staging (vector work the next barrier and the products
        // wait on) at raised wave priority, the products at the normal one
        __builtin_amdgcn_s_setprio(1);
        t.template gates<S>();
        t.template prefetch_g<S>(row, tok);  // the gates are consumed
        __syncthreads();  // the chunk's sub-block totals
        t.template stage<S>();
        t.template prefetch_kv<S>(row);  // k and v are consumed
        if constexpr (T::CS == 2) __syncthreads();  // the pair's two halves of K~
        __builtin_amdgcn_s_setprio(0);
        t.accumulate();
        const bool seg_start = p == p0 || cur.ch == 0;
        if (seg_start) {  // the segment's first chunk: its summary is complete
            const int64_t sid = seg_id(p, pl);
            t.finish(Uo + sid * DK * DV, Gs + sid * DK);
            t.zero();
        }
        back(cur);
        if (ahead) back(far);
        if constexpr (LRG) {
            if (seg_start && p > p0) {  // the next chunk belongs to the previous head
                t.lg.load(a, cur.h, t.lr, t.g);
                t.lg.ready();
            }
        }
    };
    for (int64_t p = p1 - 1; p >= p0; p -= 2) {
        step(std::integral_constant<int, 0>{}, p);
        if (p - 1 < p0) break;
        step(std::integral_constant<int, 1>{}, p - 1);
    }
}

template <int DT, int DV>
hipError_t launch_sum(const GlaArgs &a, const MfmaPlan &ps, float *U, float *G, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(ps.n_wg));
    const dim3 block(64 * 4 * (DV / 64));
    if (a.feat) {  // gates from rank-16 features, dv = 64, no residual
        if constexpr (DV == 64) {
            if (a.resid || a.rank != kFusedGateRank) return hipErrorInvalidValue;
            hipLaunchKernelGGL((k_sum<DT, DV, false, true>), grid, block, 0, st, a, U, G, ps);
        } else {
            return hipErrorInvalidValue;
        }
    } else if (a.resid) {
        hipLaunchKernelGGL((k_sum<DT, DV, true, false>), grid, block, 0, st, a, U, G, ps);
    } else {
        hipLaunchKernelGGL((k_sum<DT, DV, false, false>), grid, block, 0, st, a, U, G, ps);
    }
    return hipGetLastError();
}

}  // namespace

bool sum_supported(const GlaArgs &a) {
    return (a.dtype == DT_F16 || a.dtype == DT_BF16) && a.dk == DK && (a.dv == 64 || a.dv == 128) &&
           a.chunk == 64;
}

hipError_t sum_launch(const GlaArgs &a, const MfmaPlan &ps, float *U, float *G, hipStream_t s) {
    if (a.dtype == DT_F16) return a.dv == 64 ? launch_sum<DT_F16, 64>(a, ps, U, G, s)
                                             : launch_sum<DT_F16, 128>(a, ps, U, G, s);
    if (a.dtype == DT_BF16) return a.dv == 64 ? launch_sum<DT_BF16, 64>(a, ps, U, G, s)
                                              : launch_sum<DT_BF16, 128>(a, ps, U, G, s);
    return hipErrorInvalidValue;
}

// The segment summaries of plan ps.  Short segments go to the shared-tile summary
// kernel of k_mfma.hip, which has no reduction of four per-wave partials at a segment's
// end: up to 5 chunks at dv = 64, one chunk at dv = 128 (measured on MI355X, fp16:
// 1.6K tokens 20.2 -> 19.0 us with 6 heads, 24.6 -> 24.3 us with 16; 64x64 grid, 12
// heads (2 chunks) 32.9 -> 31.4 us; 3 to 5 chunks 0.4-0.7 us faster; 6 chunks, the
// 16.4K-token workload, alike; dv = 128 with 6 heads 25.4 -> 23.5 us).  Longer segments,
// and calls whose gate is formed from features (the shared-tile kernel reads log_g),
// go to the per-wave-partial kernel above.
constexpr int64_t kSharedTileChunks64 = 5, kSharedTileChunks128 = 1;

hipError_t segment_summaries(const GlaArgs &a, const MfmaPlan &ps, float *U, float *G, hipStream_t s) {
    const int64_t most = a.dv == 64 ? kSharedTileChunks64 : kSharedTileChunks128;
    if (sum_supported(a) && (ps.Q > most || a.feat)) return sum_launch(a, ps, U, G, s);
    return mfma_summary(a, ps, U, G, s);
}

}  // namespace gtr
