// k_rows.hip -- chunk-output kernel with token-row ownership (16-bit I/O, dk = 64,
// chunk 64, dv in {64, 128}).
//
// GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"), Method §4
// "硬件感知分块推理算子": per-chunk outputs whose score tile stays on chip, with
// the output gate fused into the epilogue; Method §1 gives the recurrence, the
// readout, RMSNorm and the SiLU(z) gate.  With a_i the in-chunk inclusive
// cumulative log2-gate and G = a at the chunk's last token:
//   o_i   = (q_i 2^a_i)^T S + sum_{j <= i} (sum_c (q_ic 2^a_ic)(k_jc 2^-a_jc)) v_j
//   S_new = Diag(2^G) (S + sum_j (k_j 2^-a_j) v_j^T)
// A chunk whose decay span exceeds kSpanMax (log2 units) runs token by token in
// fp32 instead (S_t = Diag(g_t) S + k_t v_t^T, o_t = S_t^T q_t).
//
// Work split inside a workgroup of four waves: wave w owns the chunk's tokens
// [16 u, 16 u + 16) of its token group u (a rotation of the wave index, see
// init) -- it loads them, forms their operands, computes all of their output
// columns and runs their epilogue -- and the state columns of value tiles
// NS w .. NS w + NS - 1.  So:
//   * Q~ = q 2^a of a wave's own tokens is already in the MFMA operand layout
//     where it is formed and never goes through LDS;
//   * a wave's score tiles P^T_J = K^_J Q~_u^T (J <= u) stay in registers and
//     feed the intra-chunk product directly (their register order is the k-slot
//     order of the V^T operand);
//   * every output column of a token is in one wave, so RMSNorm needs only
//     cross-lane sums and the epilogue stores whole 64-byte half rows.
// What the waves share through LDS: K^ (hi, lo) for the scores and the state
// update, V for the intra product and the state update, and the state S^T
// (hi, lo) that every wave reads for Q~ S.  Three barriers per chunk.
//
// Incoming state of a range: the scanned state of its segment, or, for
// sequences of few segments, the boundary recurrence folded in the prologue
// from the segment summaries (the scan launch is then left out).
//
// dv = 128 runs eight waves in two value halves: two waves, one per half, own
// the same 16 tokens, wave w takes the value columns [64 (w / 4), 64 (w / 4) + 64) of
// them and state tile w, so each wave holds what a dv = 64 wave holds (the
// four-wave form would need about 450 registers per lane, one wave per SIMD).
// The pair splits the key channels: wave w reads q, k and log_g of channels
// [32 (w / 4), 32 (w / 4) + 32) only and forms their gates, Q~ and K^; its half
// of Q~ goes to an LDS area the pair shares, from which each wave takes the
// other half after the second barrier.  Both halves form the score tiles.  The
// RMSNorm sum over all 128 columns is completed through LDS: each half puts its
// tokens' partial sums before the end-of-chunk barrier and both add the two in
// the same order.
//
// Low-rank gate variant (LRG): instead of reading log_g, each wave forms its
// tokens' gates from their rank-16 features (Method §1: a light low-rank
// projection with a temperature) with four 16x16x16 products against the
// segment head's projection, kept in LDS, and logsigmoid / tau.
//
// Value-column map.  MFMA tile dd of the output O^T (16 value columns) holds in
// its row m the value column dcol(dd, m) = colB(dd, m / 4) + m % 4 with
// colB(dd, k) = 32 (dd / 2) + 8 k + 4 ((dd & 1) ^ (k & 1)).  Then lane group g
// of a token holds the columns [32 e + 8 g, 32 e + 8 g + 8) of tiles 2e, 2e + 1
// (the first four from tile 2e + (g & 1)), i.e. whole 16-byte pieces, and the
// transposing V reads that produce this order are free of bank conflicts under
// the swizzle swv.  The state tiles use the same map for their columns.
#include "mfma_common.hpp"

namespace gtr {
namespace {

using namespace mf;

// Token-major V matrix [token][64 columns]: 16-byte pieces XORed by
// fv(row) = r1 | r3 << 1 | r2 << 2 (bit i of the row = ri).
__device__ __forceinline__ int swv(int row, int col) {
    const int f = ((row >> 1) & 1) | (((row >> 3) & 1) << 1) | (((row >> 2) & 1) << 2);
    return row * 64 + ((((col >> 3) ^ f) << 3) | (col & 7));
}

// S^T matrix [value column][64 key channels]: pieces XORed by r1 | (r4 r3) << 1.
__device__ __forceinline__ int sws(int row, int col) {
    const int f = ((row >> 1) & 1) | (((row >> 3) & 3) << 1);
    return row * 64 + ((((col >> 3) ^ f) << 3) | (col & 7));
}

__device__ __forceinline__ int colB(int dd, int k) {
    return 32 * (dd >> 1) + 8 * k + 4 * ((dd & 1) ^ (k & 1));
}
__device__ __forceinline__ int dcol(int dd, int m) { return colB(dd, m >> 2) + (m & 3); }

template <int DT, int DV, bool RES, bool LRG>
struct RowTile {
    static constexpr int C = 64, NB = 4;
    static constexpr int CS = DV / 64;  // value halves (dv = 128: two groups of four waves)
    static constexpr int NW = 4 * CS;   // waves
    static constexpr int NTH = 64 * NW; // threads
    static constexpr int ND = DV / 16;  // value tiles
    static constexpr int NDW = 4;       // value tiles of a wave's outputs (its half)
    static constexpr int NS = ND / NW;  // state tiles per wave (one)
    static constexpr int VP = DV / 64;  // 64-column planes of V
    static constexpr int NV = (DT == DT_F16) ? 2 : 1;  // V as bf16 hi (+ lo for fp16)
    static constexpr int NE = 2;        // 16-byte value pieces per lane of its half (epilogue, V loads)
    static constexpr int NK = 2 / CS;   // 32-channel key blocks whose q, k, gates a wave forms
    static constexpr int MAT = C * 64;
    // LDS carve-up (bytes).  Token-serial chunks reuse K (raw q, k) and S (fp32
    // gates, then the output exchange).
    static constexpr int O_K = 0;                           // K^ hi, lo
    static constexpr int O_V = O_K + 2 * MAT * 2;           // V [part][plane][64][64]
    static constexpr int O_S = O_V + NV * VP * MAT * 2;     // S^T hi, lo [2][DV][64]
    static constexpr int O_TOT = O_S + 2 * DV * 64 * 2;     // float [NB][DK]
    static constexpr int O_TAB = O_TOT + NB * DK * 4;       // float [NW waves][2][DK]
    static constexpr int O_RW = O_TAB + NW * 2 * DK * 4;    // float [DV]
    static constexpr int O_SS = O_RW + DV * 4;              // float [CS][C]: halves' sums of squares
    static constexpr int O_QP = O_SS + CS * C * 4;          // Q~ hi, lo per token group (dv = 128)
    static constexpr int O_GATE = O_QP + (CS == 2 ? 4 * 2 * 16 * 64 * 2 : 0);  // low-rank gate weights (LRG)
    static constexpr int BYTES = O_GATE + (LRG ? LowRankGate<DT>::LDS_BYTES : 0);
    static_assert(C * DK * 4 <= 2 * DV * 64 * 2, "fp32 gates must fit the state area");
    static_assert(ND * 4 * 64 * 16 <= 2 * DV * 64 * 2, "output exchange must fit the state area");

    GlaArgs a;
    uint16_t *sK, *sV, *sS, *sQ;
    float *sTot, *sTab, *sRw, *sSS;
    char *sGate;
    int w, tw, hv, l, lr, g;  // wave, its token rows [16 tw, 16 tw + 16), its value half
    int kap0;                 // first 32-channel key block of the wave (0 at dv = 64)

    // register-array element i, i uniform across the wave but not a compile-time
    // constant: selected by branches, so the array stays in registers
    __device__ __forceinline__ static void put2(s16x8 (&x)[2], int i, s16x8 v) {
        if (i == 0)
            x[0] = v;
        else
            x[1] = v;
    }

    // this lane's token: rows (negative = past the end, ~row of the last token) and
    // token indices b L + grid position (of the row read)
    int64_t rowC, rowN, tokC, tokN;
    // next chunk's inputs of this lane's token
    uint4 pq[NK], pk[NK], pv[NE], pz[NE];
    uint4 pr[RES ? NE : 1];  // previous block's output, added to v where v is consumed
    float4 pg[LRG ? 1 : 2 * NK];  // log_g (LRG: the gate features pf instead)
    uint2 pf;
    float cs[8 * NK];  // cumulative gates of channels 32 kap + 8 g + s for the wave's blocks
    // state tiles (S[s][ct][r] = S[16 ct + 4 g + r][dcol(NS w + s, lr)]) and the
    // output tiles of this wave's tokens in its half (O[e][r] = O^T[dcol(NDW hv + e, 4 g + r)][token lr])
    f32x4 S[NS][4];
    f32x4 O[NDW];
    s16x8 qh[2], ql[2];  // Q~ of this wave's tokens, B-operand layout

    __device__ __forceinline__ static int hv_of(int wave) { return CS == 1 ? 0 : wave >> 2; }

    __device__ __forceinline__ void init(const GlaArgs &args, char *smem) {
        a = args;
        sK = reinterpret_cast<uint16_t *>(smem + O_K);
        sV = reinterpret_cast<uint16_t *>(smem + O_V);
        sS = reinterpret_cast<uint16_t *>(smem + O_S);
        sTot = reinterpret_cast<float *>(smem + O_TOT);
        sRw = reinterpret_cast<float *>(smem + O_RW);
        sSS = reinterpret_cast<float *>(smem + O_SS);
        sGate = smem + O_GATE;
        const int tid = threadIdx.x;
        w = __builtin_amdgcn_readfirstlane(tid >> 6);
        // Wave w's token group.  A group's causal share of the score and intra-chunk
        // products grows with its index, and waves w and w + 4 (and the same wave of the
        // two workgroups that share a CU, launched 256 apart) run on one SIMD: the groups
        // are spread so that no SIMD takes the last group twice.
        tw = CS == 1 ? ((w + 2 * ((blockIdx.x >> 8) & 1)) & 3) : ((w + 2 * hv_of(w)) & 3);
        hv = hv_of(w);
        kap0 = CS == 1 ? 0 : hv;
        sQ = reinterpret_cast<uint16_t *>(smem + O_QP) + tw * 2 * 16 * 64;
        l = tid & 63;
        lr = l & 15;
        g = l >> 4;
        sTab = reinterpret_cast<float *>(smem + O_TAB) + w * 2 * DK;
        if (tid < DV) sRw[tid] = a.rms_w[tid];  // read after later barriers
    }

    // Row index ((b L + grid position) H + h) of this lane's token of chunk ch of
    // sequence bh.  A token past the end of the sequence reads the last token's
    // row (finite values that reach only masked scores, its own unstored output
    // and the state after the sequence's last chunk, which is never used).
    __device__ __forceinline__ int64_t row_of(uint32_t b, uint32_t h, int64_t ch, int64_t &tok) const {
        const uint32_t L32 = static_cast<uint32_t>(a.L);
        const uint32_t t0 = static_cast<uint32_t>(ch) * C + 16 * tw + lr;
        uint32_t t = t0 < L32 ? t0 : L32 - 1;
        if (a.direction & 1) t = L32 - 1 - t;  // RL, BT: reversed sequence
        uint32_t pos = t;
        if (a.direction >= 2) {                // TB, BT: column-major raster
            const uint32_t gh = static_cast<uint32_t>(a.gh);
            const uint32_t c = t / gh;
            pos = (t - c * gh) * static_cast<uint32_t>(a.gw) + c;
        }
        tok = static_cast<int64_t>(b) * a.L + pos;
        const int64_t row = tok * a.H + h;
        return t0 < L32 ? row : ~row;
    }
    __device__ __forceinline__ static int64_t live(int64_t row) { return row < 0 ? ~row : row; }

    __device__ __forceinline__ void prefetch_gv(int64_t rw, int64_t tok) {
        const int64_t row = live(rw);
        if constexpr (LRG) {
            pf = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(a.feat) +
                                                  tok * kFusedGateRank + 4 * g);
        } else {
#pragma unroll
            for (int j = 0; j < NK; ++j) {
                const int c0 = 32 * (kap0 + j) + 8 * g;
                pg[2 * j] = *reinterpret_cast<const float4 *>(a.log_g + row * DK + c0);
                pg[2 * j + 1] = *reinterpret_cast<const float4 *>(a.log_g + row * DK + c0 + 4);
            }
        }
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int d0 = 64 * hv + 32 * e + 8 * g;
            pv[e] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) + row * DV + d0);
            if constexpr (RES)
                pr[e] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.resid) + row * DV + d0);
        }
    }

    __device__ __forceinline__ void prefetch_qk(int64_t rw) {
        const int64_t row = live(rw);
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int c0 = 32 * (kap0 + j) + 8 * g;
            pq[j] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + row * DK + c0);
            pk[j] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) + row * DK + c0);
        }
    }

    __device__ __forceinline__ void prefetch_z(int64_t rw) {
        const int64_t row = live(rw);
#pragma unroll
        for (int e = 0; e < NE; ++e)
            pz[e] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.z) + row * DV +
                                                     64 * hv + 32 * e + 8 * g);
    }

    // incoming state (fp32 [DK][DV]) of the owned tiles
    __device__ __forceinline__ void load_state(const float *src) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int d = dcol(NS * w + s, lr);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[s][ct][r] = src[(16 * ct + 4 * g + r) * DV + d];
        }
    }

    __device__ __forceinline__ void zero_state() {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) S[s][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Incoming state of the owned tiles folded from the segment summaries U (fp32
    // [segment][DK][DV]) and summed log2-gates Gs ([segment][DK]) of the sequence's
    // segments s0 .. sj - 1, in order: the boundary recurrence
    // S <- Diag(2^(G_m)) S + U_m, the same arithmetic as the scan kernels.
    __device__ __forceinline__ void fold_state(const float *U, const float *Gs, int64_t s0,
                                               int64_t sj) {
        zero_state();
        for (int64_t m = s0; m < sj; ++m) {
            const float *src = U + m * DK * DV;
            float4 gm[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                gm[ct] = *reinterpret_cast<const float4 *>(Gs + m * DK + 16 * ct + 4 * g);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int d = dcol(NS * w + s, lr);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const float e[4] = {fexp2(gm[ct].x), fexp2(gm[ct].y), fexp2(gm[ct].z),
                                        fexp2(gm[ct].w)};
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        S[s][ct][r] = e[r] * S[s][ct][r] + src[(16 * ct + 4 * g + r) * DV + d];
                }
            }
        }
    }

    // Waits for the incoming state here, at the segment start: the chunk loop then
    // never holds a load that is outstanding on one path into it and not the other.
    __device__ __forceinline__ void state_ready() {
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) asm volatile("" ::"v"(S[s][ct]));
    }

    // ---- phase 1: the state S^T (hi, lo) of the owned tiles into LDS; cumulative
    // gates of the wave's tokens (registers, natural-log units) and their totals;
    // V into LDS.
    __device__ __forceinline__ void phase1() {
        uint16_t *sh = sS, *sl = sS + DV * 64;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int d = dcol(NS * w + s, lr);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const float x[4] = {S[s][ct][0], S[s][ct][1], S[s][ct][2], S[s][ct][3]};
                uint32_t hi[2], lo[2];
                split_pk<false>(x, hi, lo);
                const int off = sws(d, 16 * ct + 4 * g);
                *reinterpret_cast<uint2 *>(sh + off) = make_uint2(hi[0], hi[1]);
                *reinterpret_cast<uint2 *>(sl + off) = make_uint2(lo[0], lo[1]);
            }
        }
        if constexpr (LRG) {
            LowRankGate<DT>::gates_lds(sGate, l, g, a.inv_tau, pf, cs);
        } else {
#pragma unroll
            for (int q4 = 0; q4 < 2 * NK; ++q4) {
                cs[4 * q4] = pg[q4].x; cs[4 * q4 + 1] = pg[q4].y;
                cs[4 * q4 + 2] = pg[q4].z; cs[4 * q4 + 3] = pg[q4].w;
            }
        }
        row_scan(cs);
        if (lr == 15) {
#pragma unroll
            for (int j = 0; j < NK; ++j) {
                float *dst = sTot + tw * DK + 32 * (kap0 + j) + 8 * g;
                *reinterpret_cast<float4 *>(dst) =
                    make_float4(cs[8 * j], cs[8 * j + 1], cs[8 * j + 2], cs[8 * j + 3]);
                *reinterpret_cast<float4 *>(dst + 4) =
                    make_float4(cs[8 * j + 4], cs[8 * j + 5], cs[8 * j + 6], cs[8 * j + 7]);
            }
        }
        const int i = 16 * tw + lr;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int d0 = 64 * hv + 32 * e + 8 * g;
            uint16_t *m = sV + (d0 >> 6) * MAT + swv(i, d0 & 63);
            uint4 vx = pv[e];
            if constexpr (RES) vx = add_io<DT>(vx, pr[e]);  // stack residual
            if (NV == 1) {
                *reinterpret_cast<uint4 *>(m) = vx;
            } else {  // fp16 values as bf16 hi + lo (exact)
                float x[8];
                unpack8<DT>(vx, x);
                uint32_t hi[4], lo[4];
                split_pk<false>(x, hi, lo);
                *reinterpret_cast<uint4 *>(m) = u4(hi);
                *reinterpret_cast<uint4 *>(m + VP * MAT) = u4(lo);
            }
        }
    }

    // ---- phase 2 (after phase 1 everywhere): chunk totals, span check, operands.
    // Lane l computes for channel l the sum r of the sub-block totals before the
    // wave's tokens and the chunk's decay 2^G; Q~ stays in registers, K^ (hi, lo)
    // goes to LDS.  Returns whether the chunk runs token by token (the same in
    // every wave).
    __device__ __forceinline__ bool phase2() {
        float r_l = 0.f, tot_l = 0.f;
#pragma unroll
        for (int J = 0; J < NB; ++J) {
            const float t = sTot[J * DK + l];
            if (J < tw) r_l += t;
            tot_l += t;
        }
        r_l *= kLog2e;
        tot_l *= kLog2e;
        const bool slow = __ballot(-tot_l > kSpanMax) != 0;  // any channel's span
        sTab[l] = r_l;
        sTab[DK + l] = fexp2(tot_l);
        __builtin_amdgcn_wave_barrier();
        const int i = 16 * tw + lr;
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int kap = CS == 1 ? j : kap0;
            const int c0 = 32 * kap + 8 * g;
            // the two halves of a dv = 128 workgroup share Q~, K^ and the token-serial
            // operands: half hv forms those of the channels [32 hv, 32 hv + 32)
            constexpr bool mine = true;
            if (!slow) {
                float rI[8];
#pragma unroll
                for (int h4 = 0; h4 < 2; ++h4) {
                    const float4 x = *reinterpret_cast<const float4 *>(sTab + c0 + 4 * h4);
                    rI[4 * h4] = x.x; rI[4 * h4 + 1] = x.y; rI[4 * h4 + 2] = x.z; rI[4 * h4 + 3] = x.w;
                }
                float qt[8], aa[8];
                unpack8<DT>(pq[j], qt);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    aa[s] = fmaf(cs[8 * j + s], kLog2e, rI[s]);
                    qt[s] *= fexp2(aa[s]);  // q 2^a
                }
                uint32_t qhi[4], qlo[4];
                split_pk<false>(qt, qhi, qlo);
                if constexpr (CS == 1) {
                    qh[kap] = __builtin_bit_cast(s16x8, u4(qhi));
                    ql[kap] = __builtin_bit_cast(s16x8, u4(qlo));
                } else {
                    put2(qh, kap, __builtin_bit_cast(s16x8, u4(qhi)));
                    put2(ql, kap, __builtin_bit_cast(s16x8, u4(qlo)));
                }
                if constexpr (CS == 2) {  // the pair's other half reads it after the barrier
                    const int off = lr * 64 + (((4 * kap + g) ^ (lr & 7)) << 3);
                    *reinterpret_cast<uint4 *>(sQ + off) = u4(qhi);
                    *reinterpret_cast<uint4 *>(sQ + 16 * 64 + off) = u4(qlo);
                }
                if (mine) {
                    float kh[8];
                    unpack8<DT>(pk[j], kh);
#pragma unroll
                    for (int s = 0; s < 8; ++s) kh[s] *= fexp2(-aa[s]);  // k 2^-a
                    uint32_t khi[4], klo[4];
                    split_pk<false>(kh, khi, klo);
                    const int off = swn(i, c0);
                    *reinterpret_cast<uint4 *>(sK + off) = u4(khi);
                    *reinterpret_cast<uint4 *>(sK + MAT + off) = u4(klo);
                }
            } else if (mine) {
                // token-serial operands, [token][channel] without swizzle: q and k as
                // stored (K area), g = 2^(a_i - a_{i-1}) in fp32 (state area)
                *reinterpret_cast<uint4 *>(sK + i * DK + c0) = pq[j];
                *reinterpret_cast<uint4 *>(sK + MAT + i * DK + c0) = pk[j];
                float *fG = reinterpret_cast<float *>(sS);
                float gg[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float up = __shfl_up(cs[8 * j + s], 1, 16);
                    const float prev = (lr == 0) ? 0.f : up;
                    gg[s] = fexp2((cs[8 * j + s] - prev) * kLog2e);
                }
                *reinterpret_cast<float4 *>(fG + i * DK + c0) = make_float4(gg[0], gg[1], gg[2], gg[3]);
                *reinterpret_cast<float4 *>(fG + i * DK + c0 + 4) = make_float4(gg[4], gg[5], gg[6], gg[7]);
            }
        }
        return slow;
    }

    // dv = 128 (after the second barrier): the other half of Q~ from the pair's area
    __device__ __forceinline__ void partner_q() {
        if constexpr (CS == 2) {
            const int kap = 1 - hv;
            const int off = lr * 64 + (((4 * kap + g) ^ (lr & 7)) << 3);
            put2(qh, kap, *reinterpret_cast<const s16x8 *>(sQ + off));
            put2(ql, kap, *reinterpret_cast<const s16x8 *>(sQ + 16 * 64 + off));
        }
    }

    // V^T operand of value tile dd, V part p: lane row / column dcol(dd, lr), k
    // slots = tokens rb + 4 g + s (s < 4) and rb + 16 + 4 g + (s - 4), by two
    // transposing reads (lane i's slot j comes from source lane 4 j + i / 4).
    __device__ __forceinline__ s16x8 op_v(int p, int dd, int rb) const {
        const uint16_t *m = sV + (p * VP + (dd >> 2)) * MAT;
        const int r = rb + 4 * g + (lr >> 2);
        const int c = colB(dd, lr & 3) & 63;
        const s16x4 x0 = ld_tr(m + swv(r, c));
        const s16x4 x1 = ld_tr(m + swv(r + 16, c));
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }

    // K^T operand (A rows = channels cb + lr), same token slots
    __device__ __forceinline__ s16x8 op_k(const uint16_t *m, int rb, int cb) const {
        const int r = rb + 4 * g + (lr >> 2);
        const int c = cb + 4 * (lr & 3);
        const s16x4 x0 = ld_tr(m + swn(r, c));
        const s16x4 x1 = ld_tr(m + swn(r + 16, c));
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }

    // ---- products of a chunk (after phase 2 everywhere).  upd: the state after the
    // chunk is used (the chunk is not the last of its piece of a sequence); otherwise
    // the state update is left out (a one-chunk range's whole third of the products).
    __device__ __forceinline__ void compute(bool upd) {
        // inter-chunk readout O^T = S^T Q~_w^T, the value tiles' products interleaved
        const uint16_t *sh = sS, *sl = sS + DV * 64;
#pragma unroll
        for (int e = 0; e < NDW; ++e) O[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kap = 0; kap < 2; ++kap) {
            s16x8 ah[NDW], al[NDW];
#pragma unroll
            for (int e = 0; e < NDW; ++e) {
                const int off = sws(dcol(NDW * hv + e, lr), 32 * kap + 8 * g);
                ah[e] = *reinterpret_cast<const s16x8 *>(sh + off);
                al[e] = *reinterpret_cast<const s16x8 *>(sl + off);
            }
#pragma unroll
            for (int e = 0; e < NDW; ++e) O[e] = mma<false>(ah[e], qh[kap], O[e]);
#pragma unroll
            for (int e = 0; e < NDW; ++e) O[e] = mma<false>(ah[e], ql[kap], O[e]);
#pragma unroll
            for (int e = 0; e < NDW; ++e) O[e] = mma<false>(al[e], qh[kap], O[e]);
        }
        __builtin_amdgcn_sched_barrier(0);  // keeps the operand loads of each step near it
        // causal score tiles P^T_J[j][i] = K^_J Q~_w^T (hi + lo), two at a time, each
        // pair feeding the intra-chunk readout O^T += V^T P^T (32 tokens per step) at
        // once.  A wave takes the pairs that reach its own tokens; a tile past them
        // (J > w) is formed and zeroed by the mask like the causal part of J = w.
#pragma unroll
        for (int kt = 0; kt < NB / 2; ++kt) {
            if (2 * kt <= tw) {
                uint32_t bh[4], bl[4];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int J = 2 * kt + u;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kap = 0; kap < 2; ++kap) {
                        const int off = swn(16 * J + lr, 32 * kap + 8 * g);
                        const s16x8 kh = *reinterpret_cast<const s16x8 *>(sK + off);
                        const s16x8 kl = *reinterpret_cast<const s16x8 *>(sK + MAT + off);
                        acc = mma<false>(kh, qh[kap], acc);
                        acc = mma<false>(kh, ql[kap], acc);
                        acc = mma<false>(kl, qh[kap], acc);
                    }
                    float x[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        x[r] = (J > tw || (J == tw && 4 * g + r > lr)) ? 0.f : acc[r];  // j <= i
                    uint32_t h2[2], l2[2];
                    split_pk<false>(x, h2, l2);
                    bh[2 * u] = h2[0]; bh[2 * u + 1] = h2[1];
                    bl[2 * u] = l2[0]; bl[2 * u + 1] = l2[1];
                }
                const s16x8 ph = __builtin_bit_cast(s16x8, make_uint4(bh[0], bh[1], bh[2], bh[3]));
                const s16x8 pl = __builtin_bit_cast(s16x8, make_uint4(bl[0], bl[1], bl[2], bl[3]));
#pragma unroll
                for (int e = 0; e < NDW; ++e) {
                    const s16x8 av = op_v(0, NDW * hv + e, 32 * kt);
                    O[e] = mma<false>(av, ph, O[e]);
                    O[e] = mma<false>(av, pl, O[e]);
                    if (NV == 2) O[e] = mma<false>(op_v(NV - 1, NDW * hv + e, 32 * kt), ph, O[e]);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!upd) return;
        // state update of the owned tiles: S = Diag(2^G) (S + K^^T V)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int dd = NS * w + s;
#pragma unroll
            for (int kt = 0; kt < NB / 2; ++kt) {
                s16x8 bv[NV];
#pragma unroll
                for (int p = 0; p < NV; ++p) bv[p] = op_v(p, dd, 32 * kt);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    __builtin_amdgcn_sched_barrier(0);
                    const s16x8 akh = op_k(sK, 32 * kt, 16 * ct);
                    const s16x8 akl = op_k(sK + MAT, 32 * kt, 16 * ct);
                    S[s][ct] = mma<false>(akh, bv[0], S[s][ct]);
                    S[s][ct] = mma<false>(akl, bv[0], S[s][ct]);
                    if (NV == 2) S[s][ct] = mma<false>(akh, bv[NV - 1], S[s][ct]);
                }
            }
        }
        decay();
    }

    __device__ __forceinline__ void decay() {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const float4 e4 = *reinterpret_cast<const float4 *>(sTab + DK + 16 * ct + 4 * g);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                S[s][ct][0] *= e4.x; S[s][ct][1] *= e4.y; S[s][ct][2] *= e4.z; S[s][ct][3] *= e4.w;
            }
        }
    }

    // ---- token-serial chunk: S and o from the fp32 operands of phase 2, for the
    // owned tiles and every token; the tiles are then exchanged through LDS so
    // that each wave holds all columns of its own tokens.
    __device__ __forceinline__ void serial() {
        const uint16_t *fQ = sK, *fK = sK + MAT;
        const float *fG = reinterpret_cast<const float *>(sS);
        f32x4 Os[NS][NB];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) Os[s][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int t = 0; t < C; ++t) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int d = dcol(NS * w + s, lr);
                const uint16_t *vm = sV + (d >> 6) * MAT + swv(t, d & 63);
                float vd;
                if (NV == 2)
                    vd = __uint_as_float(static_cast<uint32_t>(vm[0]) << 16) +
                         __uint_as_float(static_cast<uint32_t>(vm[VP * MAT]) << 16);
                else
                    vd = h2f<DT>(vm[0]);
                float part = 0.f;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const int c = 16 * ct + 4 * g;
                    const float4 gq = *reinterpret_cast<const float4 *>(fG + t * DK + c);
                    const uint2 kq = *reinterpret_cast<const uint2 *>(fK + t * DK + c);
                    const uint2 qq = *reinterpret_cast<const uint2 *>(fQ + t * DK + c);
                    const float gg[4] = {gq.x, gq.y, gq.z, gq.w};
                    const float kk[4] = {h2f<DT>(kq.x & 0xffffu), h2f<DT>(kq.x >> 16),
                                         h2f<DT>(kq.y & 0xffffu), h2f<DT>(kq.y >> 16)};
                    const float q4[4] = {h2f<DT>(qq.x & 0xffffu), h2f<DT>(qq.x >> 16),
                                         h2f<DT>(qq.y & 0xffffu), h2f<DT>(qq.y >> 16)};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        S[s][ct][r] = gg[r] * S[s][ct][r] + kk[r] * vd;
                        part += S[s][ct][r] * q4[r];
                    }
                }
                part += __shfl_xor(part, 16);
                part += __shfl_xor(part, 32);
                // o_t at column dcol(dd, lr) is now in every lane group; lane (t % 16, g)
                // takes the columns dcol(dd, 4 g + r) = colB(dd, g) + r
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = __shfl(part, 4 * g + r);
                    if (lr == (t & 15)) {
#pragma unroll
                        for (int tb = 0; tb < NB; ++tb)
                            if (tb == (t >> 4)) Os[s][tb][r] = x;
                    }
                }
            }
        }
        __syncthreads();  // every wave is done with the gates in the state area
        f32x4 *X = reinterpret_cast<f32x4 *>(sS);  // [dd][tb][lane]
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) X[((NS * w + s) * NB + tb) * 64 + l] = Os[s][tb];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < NDW; ++e) O[e] = X[((NDW * hv + e) * NB + tw) * 64 + l];
    }

    // ---- epilogue: y = o / sqrt(mean_j o_j^2 + eps) * rms_w * z * sigmoid(z) for the
    // wave's tokens, stored at the token's grid position (pairs rounded to nearest
    // even by the packed conversion; streaming stores)
    __device__ __forceinline__ float half_ss() const {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < NDW; ++e)
#pragma unroll
            for (int r = 0; r < 4; ++r) ss += O[e][r] * O[e][r];
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        return ss;
    }
    // two halves: each puts its tokens' sum before a barrier, and the epilogue adds
    // both in half order (the same sum in both).  One buffer is enough: the next
    // chunk's sums are written after that chunk's first two barriers, which no wave
    // passes before it has read this chunk's.
    __device__ __forceinline__ void put_ss() {
        const float ss = half_ss();
        if (g == 0) sSS[hv * C + 16 * tw + lr] = ss;
    }
    __device__ __forceinline__ void epilogue() {
        float ss;
        if constexpr (CS == 1) {
            ss = half_ss();
        } else {
            ss = sSS[16 * tw + lr] + sSS[C + 16 * tw + lr];
        }
        const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / DV) + GTR_RMS_EPS);
        const bool odd = g & 1;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int d0 = 64 * hv + 32 * e + 8 * g;
            const f32x4 lo4 = odd ? O[2 * e + 1] : O[2 * e];
            const f32x4 hi4 = odd ? O[2 * e] : O[2 * e + 1];
            const float o[8] = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
            const float4 w0 = *reinterpret_cast<const float4 *>(sRw + d0);
            const float4 w1 = *reinterpret_cast<const float4 *>(sRw + d0 + 4);
            const float rw[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            float zz[8];
            unpack8<DT>(pz[e], zz);
            float y[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float silu = zz[k] * frcp(1.0f + fexp2(-zz[k] * kLog2e));
                y[k] = (o[k] * inv) * (rw[k] * silu);
            }
            const uint4 yb = make_uint4(pk2<DT == DT_F16>(y[0], y[1]), pk2<DT == DT_F16>(y[2], y[3]),
                                        pk2<DT == DT_F16>(y[4], y[5]), pk2<DT == DT_F16>(y[6], y[7]));
            if (rowC >= 0)
                store_stream16(static_cast<uint16_t *>(a.out) + rowC * DV + d0, yb);
        }
    }
};

template <int DT, int DV, bool RES, bool LRG>
__global__ __launch_bounds__(64 * 4 * (DV / 64), DV == 64 ? 2 : 1) void k_rows(GlaArgs a, const float *__restrict__ Sx,
                                                               const float *__restrict__ Gf,
                                                               MfmaPlan pl, MfmaPlan ps) {
    using R = RowTile<DT, DV, RES, LRG>;
    static_assert(R::NTH == 64 * 4 * (DV / 64), "launch bounds");
    __shared__ __attribute__((aligned(16))) char smem[R::BYTES];
    R t;
    t.init(a, smem);
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * pl.Q;
    const int64_t p1 = (p0 + pl.Q < pl.T) ? p0 + pl.Q : pl.T;
    if (p0 >= p1) return;  // the whole workgroup

    // current image b, head h and chunk ch, advanced incrementally (no divisions
    // in the loop)
    const int64_t bh0 = p0 / pl.N;
    int64_t ch = p0 - bh0 * pl.N;
    uint32_t b = static_cast<uint32_t>(bh0 / a.H), h = static_cast<uint32_t>(bh0 % a.H);
    t.rowC = t.row_of(b, h, ch, t.tokC);
    t.prefetch_gv(t.rowC, t.tokC);
    t.prefetch_qk(t.rowC);
    t.prefetch_z(t.rowC);

    // Segments (the range's pieces within one sequence) in an outer loop, so that
    // the incoming state is loaded outside the chunk loop: the chunk loop then
    // issues the same loads every time and the wait-count bookkeeping never has to
    // drain the load queue.
    // With Gf, Sx holds the segment summaries and the state entering the range is
    // folded from those of its sequence's earlier segments (every later piece of the
    // range starts a sequence, from zero); without, Sx holds each segment's state.
    if (Gf) t.fold_state(Sx, Gf, seg_id(p0 - ch, ps), seg_id(p0, ps));
    for (int64_t p = p0; p < p1;) {
        const int64_t pe = (p - ch + pl.N < p1) ? p - ch + pl.N : p1;  // segment end
        if (!Gf)
            t.load_state(Sx + seg_id(p, ps) * DK * DV);
        else if (p != p0)
            t.zero_state();
        LowRankGate<DT> lg;
        if constexpr (LRG) lg.load(a, h, t.lr, t.g);  // the segment's head
        t.state_ready();
        // (every wave is past the previous chunk's last barrier: the old copy is unused)
        if constexpr (LRG) lg.put(t.sGate, t.l, t.g);
        for (; p < pe; ++p) {
            const bool last_in_seq = (ch == pl.N - 1);
            const bool more = p + 1 < p1;
            // Phases 1 and 2 (the state's hi/lo split, the gate scan, the operands'
            // exponentials and splits: vector instructions the next barrier waits on) run
            // at raised wave priority, so a SIMD issues them ahead of the other
            // workgroup's wave in its matrix products (16.4K tokens: 68.9 -> 66.6 us per
            // call on MI355X).
            __builtin_amdgcn_s_setprio(1);
            t.phase1();
            __syncthreads();  // B1: state, gate totals, V
            // The next chunk's loads are issued on every chunk (on the range's last
            // one they re-read its own rows, unused).
            uint32_t nb = b, nh = h;
            if (last_in_seq && ++nh == static_cast<uint32_t>(a.H)) {
                nh = 0;
                ++nb;
            }
            t.tokN = t.tokC;
            t.rowN = more ? t.row_of(nb, nh, last_in_seq ? 0 : ch + 1, t.tokN) : t.rowC;
            t.prefetch_gv(t.rowN, t.tokN);  // phase 1 consumed the gates and v
            const bool slow = t.phase2();
            __builtin_amdgcn_s_setprio(0);
            t.prefetch_qk(t.rowN);  // phase 2 consumed q and k
            __syncthreads();  // B2: K^ (and the pair's halves of Q~)
            if (!slow) {
                t.partner_q();
                t.compute(p + 1 < pe);
            } else {
                t.serial();
            }
            if constexpr (R::CS == 1) {
                t.epilogue();
                t.prefetch_z(t.rowN);
                __syncthreads();  // B3: LDS is rewritten by the next chunk
            } else {
                t.put_ss();
                __syncthreads();  // B3: as above; both halves' sums of squares
                t.epilogue();
                t.prefetch_z(t.rowN);
            }
            t.rowC = t.rowN;
            t.tokC = t.tokN;
            ch = last_in_seq ? 0 : ch + 1;
            b = nb;
            h = nh;
        }
    }
}

template <int DT, int DV>
hipError_t launch_rows(const GlaArgs &a, const float *Sx, const float *Gf, const MfmaPlan &po,
                       const MfmaPlan &ps, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(po.n_wg));
    if (a.feat) {  // gates from rank-16 features: dv = 64, no residual
        if constexpr (DV == 64) {
            if (a.resid || a.rank != kFusedGateRank) return hipErrorInvalidValue;
            hipLaunchKernelGGL((k_rows<DT, DV, false, true>), grid, dim3(RowTile<DT, DV, false, true>::NTH), 0, st, a, Sx, Gf, po, ps);
        } else {
            return hipErrorInvalidValue;
        }
    } else if (a.resid) {
        hipLaunchKernelGGL((k_rows<DT, DV, true, false>), grid, dim3(RowTile<DT, DV, true, false>::NTH), 0, st, a, Sx, Gf, po, ps);
    } else {
        hipLaunchKernelGGL((k_rows<DT, DV, false, false>), grid, dim3(RowTile<DT, DV, false, false>::NTH), 0, st, a, Sx, Gf, po, ps);
    }
    return hipGetLastError();
}

}  // namespace

bool rows_supported(const GlaArgs &a) {
    return (a.dtype == DT_F16 || a.dtype == DT_BF16) && a.dk == DK && (a.dv == 64 || a.dv == 128) &&
           a.chunk == 64;
}

hipError_t rows_output(const GlaArgs &a, const MfmaPlan &po, const MfmaPlan &ps, const float *Sx,
                       const float *Gf, hipStream_t s) {
    if (a.dtype == DT_F16) {
        if (a.dv == 64) return launch_rows<DT_F16, 64>(a, Sx, Gf, po, ps, s);
        if (a.dv == 128) return launch_rows<DT_F16, 128>(a, Sx, Gf, po, ps, s);
    } else if (a.dtype == DT_BF16) {
        if (a.dv == 64) return launch_rows<DT_BF16, 64>(a, Sx, Gf, po, ps, s);
        if (a.dv == 128) return launch_rows<DT_BF16, 128>(a, Sx, Gf, po, ps, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gtr
