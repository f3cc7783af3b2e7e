// k_mfma.hip -- chunkwise Key-only GLA on gfx950 matrix cores (16-bit I/O, dk = 64).
//
// GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"), Method §4
// "硬件感知分块推理算子": chunk summaries on the matrix units, a light boundary-state
// scan, and per-chunk outputs whose score tile never leaves on-chip memory, with
// the output gate fused into the epilogue.  The recurrence, readout, RMSNorm and
// SiLU(z) gate are those of Method §1.  Two kernels live here:
//
//   k_chunk<..., true>  :  per (b, h, segment of chunks) U_seg = sum_t k~_t v_t^T
//                           (k~_t = k_t * prod_{r>t in segment} g_r) and the
//                           segment's summed log-gate.
//   k_chunk<..., false> :  per (b, h, segment) re-runs the segment chunk by chunk
//                           from the incoming state the scan produced, emitting
//                           y_t = RMSNorm(S_t^T q_t) * rms_w * SiLU(z_t) at the
//                           token's grid position.
//
// Per chunk of C = 16 * NB tokens (a_i = in-chunk inclusive cumulative log2-gate,
// G = a at the chunk's last token; sub-block I covers tokens [16I, 16I + 16) and
// r_I is a just before it):
//   o_i   = (q_i * 2^a_i)^T S_prev + sum_{j <= i} (sum_c q_ic k_jc 2^(a_ic - a_jc)) v_j
//   S_new = Diag(2^G) S_prev + sum_j (k_j * 2^(G - a_j)) v_j^T
// Scores of sub-block pair (J < I) are factored as
//   (q_i 2^(a_i - r_I)) * 2^(r_I - r_{J+1}) * (k_j 2^(r_{J+1} - a_j)),
// every factor <= 1.  The diagonal pair uses 2^(r_I - r_{I+1}) >= 1 (the
// sub-block's decay span), which stays finite while the span is at most
// kSpanMax (log2 units); beyond that the diagonal tile is computed pair by pair.
//
// Matrix products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
// Every fp32 operand is split into bf16 hi + lo (x = hi + lo to ~16 bits);
// the product of two split operands takes hi*hi + hi*lo + lo*hi, of a split
// and an exact operand two products.  fp16 inputs are exact as bf16 hi + lo.
//
// Workgroup: 4 waves.  Wave w owns value columns [16 w DPW, 16 (w+1) DPW) of
// the fp32 state S (held in MFMA accumulators) and the token sub-blocks
// I = w, w + 4, ... of each chunk.  Lane l: lr = l % 16, g = l / 16.
#include "gtr_internal.hpp"

namespace gtr {
namespace {

using bf16 = __bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int NT = 256;
constexpr int DK = 64;
constexpr int KP = DK + 8;  // pitch (elements) of [token][channel] bf16 rows
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kSpanMax = 64.f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two 4-element runs of a bf16 row, 16 elements apart, as one MFMA operand.
__device__ __forceinline__ bf16x8 ld_pair4(const bf16 *p) {
    const bf16x4 x0 = *reinterpret_cast<const bf16x4 *>(p);
    const bf16x4 x1 = *reinterpret_cast<const bf16x4 *>(p + 16);
    return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void split(float x, bf16 &hi, bf16 &lo) {
    hi = static_cast<bf16>(x);
    lo = static_cast<bf16>(x - static_cast<float>(hi));
}

// Inclusive prefix sum over the 16 lanes of a DPP row (lanes with equal lane / 16).
__device__ __forceinline__ float row_scan(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
    return x;
}

template <int DT> __device__ __forceinline__ float h2f(uint32_t bits16);
template <> __device__ __forceinline__ float h2f<DT_F16>(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}
template <> __device__ __forceinline__ float h2f<DT_BF16>(uint32_t b) {
    return __uint_as_float(b << 16);
}

// 8 consecutive 16-bit elements starting at element index idx (16-byte aligned).
template <int DT>
__device__ __forceinline__ void ld8(const void *base, int64_t idx, float *o) {
    const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + idx);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int s = 0; s < 8; ++s) o[s] = h2f<DT>((w[s >> 1] >> (16 * (s & 1))) & 0xffffu);
}

template <int DT> __device__ __forceinline__ uint16_t f2h(float x);
template <> __device__ __forceinline__ uint16_t f2h<DT_F16>(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
template <> __device__ __forceinline__ uint16_t f2h<DT_BF16>(float x) { return f32_to_bf16(x); }

template <int DT, int DV, int NB, bool SUM>
struct Cfg {
    static constexpr int C = 16 * NB;         // chunk length
    static constexpr int CP = C + 8;          // pitch of [row][token] bf16 rows
    static constexpr int NDB = DV / 16;       // value-column blocks
    static constexpr int DPW = NDB / 4;       // value-column blocks per wave
    static constexpr int BPW = (NB + 3) / 4;  // token sub-blocks per wave (max)
    static constexpr int NV = (DT == DT_F16) ? 2 : 1;  // bf16 parts of v
    static constexpr int NTRI = NB * (NB + 1) / 2;
    // LDS carve-up (bytes).  sQt and sKp are reused for the intra-chunk
    // exchange sX; sKt for the output staging sY.
    static constexpr int QT = SUM ? 0 : 2 * C * KP * 2;      // Q~ hi, lo   [i][c]
    static constexpr int KPB = SUM ? 0 : 2 * C * KP * 2;     // K'' hi, lo  [j][c]
    static constexpr int KT = 2 * DK * CP * 2;               // K~^T hi, lo [c][j]
    static constexpr int VT = NV * DV * CP * 2;              // V^T parts   [d][j]
    static constexpr int XP = C + 4;                         // pitch of sX rows (floats)
    static constexpr int X = SUM ? 0 : DV * XP * 4;
    static constexpr int YP = DV + 8;
    static constexpr int Y = SUM ? 0 : C * YP * 2;
    static_assert(X <= QT + KPB, "exchange buffer must fit in the Q~/K'' region");
    static_assert(Y <= KT, "output staging must fit in the K~ region");
    static constexpr int O_QT = 0;
    static constexpr int O_KP = O_QT + QT;
    static constexpr int O_KT = O_KP + KPB;
    static constexpr int O_VT = O_KT + KT;
    static constexpr int O_TOT = O_VT + VT;                  // float [NB][DK]
    static constexpr int O_ERI = O_TOT + NB * DK * 4;        // float [NB][DK] 2^r_I
    static constexpr int O_EG = O_ERI + NB * DK * 4;         // float [NB][DK] 2^(G - r_{I+1})
    static constexpr int O_F = O_EG + NB * DK * 4;           // float [NTRI][DK] 2^(r_I - r_{J+1})
    static constexpr int O_EGC = O_F + (SUM ? 0 : NTRI * DK * 4);  // float [DK] 2^G
    static constexpr int O_SS = O_EGC + DK * 4;              // float [4][C]
    static constexpr int O_ROW = O_SS + (SUM ? 0 : 4 * C * 4);     // int64 [C]
    static constexpr int BYTES = O_ROW + C * 8;
};

template <int DT, int DV, int NB, bool SUM>
__global__ __launch_bounds__(NT, (DV == 128 || NB == 8) ? 1 : 2) void k_chunk(
    GlaArgs a, float *__restrict__ U, float *__restrict__ G, const float *__restrict__ Sx,
    int n_seg, int seg_chunks) {
    using K = Cfg<DT, DV, NB, SUM>;
    constexpr int C = K::C, CP = K::CP, NDB = K::NDB, DPW = K::DPW, BPW = K::BPW, NV = K::NV;
    __shared__ __attribute__((aligned(16))) char smem[K::BYTES];
    bf16 *sQt = reinterpret_cast<bf16 *>(smem + K::O_QT);  // [2][C][KP]
    bf16 *sKp = reinterpret_cast<bf16 *>(smem + K::O_KP);  // [2][C][KP]
    bf16 *sKt = reinterpret_cast<bf16 *>(smem + K::O_KT);  // [2][DK][CP]
    bf16 *sVt = reinterpret_cast<bf16 *>(smem + K::O_VT);  // [NV][DV][CP]
    float *sTot = reinterpret_cast<float *>(smem + K::O_TOT);
    float *sErI = reinterpret_cast<float *>(smem + K::O_ERI);
    float *sEg = reinterpret_cast<float *>(smem + K::O_EG);
    float *sF = reinterpret_cast<float *>(smem + K::O_F);
    float *sEGc = reinterpret_cast<float *>(smem + K::O_EGC);
    float *sSS = reinterpret_cast<float *>(smem + K::O_SS);
    int64_t *sRow = reinterpret_cast<int64_t *>(smem + K::O_ROW);
    float *sX = reinterpret_cast<float *>(smem + K::O_QT);     // [DV][XP]
    uint16_t *sY = reinterpret_cast<uint16_t *>(smem + K::O_KT);  // [C][YP]

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, lr = l & 15, g = l >> 4;
    const int seg = blockIdx.x % n_seg;
    const int bh = blockIdx.x / n_seg;
    const int b = bh / a.H, h = bh % a.H;
    const int64_t n_chunks = (a.L + C - 1) / C;
    const int64_t ch0 = static_cast<int64_t>(seg) * seg_chunks;
    const int64_t ch1 = (ch0 + seg_chunks < n_chunks) ? ch0 + seg_chunks : n_chunks;
    const size_t soff = (static_cast<size_t>(bh) * n_seg + seg) * DK * DV;

    // fp32 state, accumulator layout: S[dd][ct][r] = S[16 ct + 4 g + r][16 (w DPW + dd) + lr]
    f32x4 S[DPW][4];
#pragma unroll
    for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[dd][ct][r] = SUM ? 0.f
                                   : Sx[soff + static_cast<size_t>(16 * ct + 4 * g + r) * DV +
                                        16 * (w * DPW + dd) + lr];
    float gam_run = 0.f;  // summed log2-gate of the segment, channel l (wave 0)

    for (int64_t ch = ch0; ch < ch1; ++ch) {
        const int64_t t0 = ch * C;
        if (tid < C) sRow[tid] = (t0 + tid < a.L) ? scan_row(a, b, h, t0 + tid) : -1;
        __syncthreads();

        // ---- staging 1: gates (cumulative within sub-blocks), q, k, and V^T
        float qv[BPW][16], kv[BPW][16], cs[BPW][16];
#pragma unroll
        for (int m = 0; m < BPW; ++m) {
            const int I = w + 4 * m;
            if (I >= NB) break;
            const int64_t row = sRow[16 * I + lr];
#pragma unroll
            for (int kap = 0; kap < 2; ++kap) {
                const int c0 = 32 * kap + 8 * g;
                float lg[8];
                if (row >= 0) {
                    ld8<DT>(a.k, row * DK + c0, &kv[m][8 * kap]);
                    if (!SUM) ld8<DT>(a.q, row * DK + c0, &qv[m][8 * kap]);
                    const float4 g0 = *reinterpret_cast<const float4 *>(a.log_g + row * DK + c0);
                    const float4 g1 = *reinterpret_cast<const float4 *>(a.log_g + row * DK + c0 + 4);
                    lg[0] = g0.x; lg[1] = g0.y; lg[2] = g0.z; lg[3] = g0.w;
                    lg[4] = g1.x; lg[5] = g1.y; lg[6] = g1.z; lg[7] = g1.w;
                } else {
#pragma unroll
                    for (int s = 0; s < 8; ++s) { kv[m][8 * kap + s] = 0.f; qv[m][8 * kap + s] = 0.f; lg[s] = 0.f; }
                }
#pragma unroll
                for (int s = 0; s < 8; ++s) cs[m][8 * kap + s] = row_scan(lg[s] * kLog2e);
            }
            if (lr == 15) {
#pragma unroll
                for (int kap = 0; kap < 2; ++kap)
#pragma unroll
                    for (int s = 0; s < 8; ++s) sTot[I * DK + 32 * kap + 8 * g + s] = cs[m][8 * kap + s];
            }
            // V^T[d][16 I + ii] for d = l + 64 dm (value input, residual added in a stack)
#pragma unroll
            for (int dm = 0; dm < DV / 64; ++dm) {
                const int d = l + 64 * dm;
                float vv[16];
#pragma unroll
                for (int ii = 0; ii < 16; ++ii) {
                    const int64_t rr = sRow[16 * I + ii];
                    vv[ii] = rr >= 0 ? ld_v<DT>(a, rr * DV + d) : 0.f;
                }
                bf16x8 p0[NV], p1[NV];
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) {
                    if (NV == 2) {
                        bf16 hi, lo;
                        split(vv[ii], hi, lo); p0[0][ii] = hi; p0[NV - 1][ii] = lo;
                        split(vv[ii + 8], hi, lo); p1[0][ii] = hi; p1[NV - 1][ii] = lo;
                    } else {
                        p0[0][ii] = static_cast<bf16>(vv[ii]);
                        p1[0][ii] = static_cast<bf16>(vv[ii + 8]);
                    }
                }
#pragma unroll
                for (int pv = 0; pv < NV; ++pv) {
                    bf16 *dst = sVt + (pv * DV + d) * CP + 16 * I;
                    *reinterpret_cast<bf16x8 *>(dst) = p0[pv];
                    *reinterpret_cast<bf16x8 *>(dst + 8) = p1[pv];
                }
            }
        }
        __syncthreads();

        // ---- tables: per channel l, for the sub-blocks this wave owns
        bool span_bad[BPW];
#pragma unroll
        for (int m = 0; m < BPW; ++m) {
            span_bad[m] = false;
            const int I = w + 4 * m;
            if (I >= NB) break;
            float pre[NB + 1];
            pre[0] = 0.f;
#pragma unroll
            for (int J = 0; J < NB; ++J) pre[J + 1] = pre[J] + sTot[J * DK + l];
            const float rI = pre[I], tI = sTot[I * DK + l], gm = pre[NB];
            sErI[I * DK + l] = fexp2(rI);
            sEg[I * DK + l] = fexp2(gm - rI - tI);
            if (!SUM) {
#pragma unroll
                for (int J = 0; J <= I; ++J)
                    sF[(I * (I + 1) / 2 + J) * DK + l] = fexp2(fminf(rI - pre[J + 1], kSpanMax));
                // the diagonal factor 2^(-t_I) must stay finite: wave-wide span check
                float sp = -tI;
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) sp = fmaxf(sp, __shfl_xor(sp, off));
                span_bad[m] = sp > kSpanMax;
            }
            if (w == 0 && m == 0) {
                sEGc[l] = fexp2(gm);
                gam_run += gm;
            }
        }
        __syncthreads();

        // ---- staging 2: operand matrices in LDS; q' kept in registers
        float qp[BPW][16];
#pragma unroll
        for (int m = 0; m < BPW; ++m) {
            const int I = w + 4 * m;
            if (I >= NB) break;
            const int i = 16 * I + lr;
#pragma unroll
            for (int kap = 0; kap < 2; ++kap) {
                const int c0 = 32 * kap + 8 * g;
                bf16x8 qh, ql, kh, kl;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int c = c0 + s;
                    const float tI = sTot[I * DK + c];
                    const float a_loc = cs[m][8 * kap + s];         // a_i - r_I
                    const float kpp = kv[m][8 * kap + s] * fexp2(tI - a_loc);  // k 2^(r_{I+1} - a)
                    const float kt = kpp * sEg[I * DK + c];                     // k 2^(G - a)
                    bf16 hi, lo;
                    split(kt, hi, lo);
                    sKt[c * CP + i] = hi;
                    sKt[(DK + c) * CP + i] = lo;
                    if (!SUM) {
                        const float q1 = qv[m][8 * kap + s] * fexp2(a_loc);  // q 2^(a - r_I)
                        qp[m][8 * kap + s] = q1;
                        split(q1 * sErI[I * DK + c], hi, lo);               // q 2^a
                        qh[s] = hi; ql[s] = lo;
                        split(kpp, hi, lo);
                        kh[s] = hi; kl[s] = lo;
                    }
                }
                if (!SUM) {
                    *reinterpret_cast<bf16x8 *>(sQt + i * KP + c0) = qh;
                    *reinterpret_cast<bf16x8 *>(sQt + (C + i) * KP + c0) = ql;
                    *reinterpret_cast<bf16x8 *>(sKp + i * KP + c0) = kh;
                    *reinterpret_cast<bf16x8 *>(sKp + (C + i) * KP + c0) = kl;
                }
            }
        }
        __syncthreads();

        f32x4 O[DPW][NB];        // inter-chunk readout, later the whole output
        f32x4 Oi[BPW][NDB];      // intra-chunk readout of the own sub-blocks
        if (!SUM) {
            // ---- O^T[d][i] = S^T Q~^T  (A = S from the accumulators, B = Q~^T)
#pragma unroll
            for (int dd = 0; dd < DPW; ++dd) {
                bf16x8 ah[2], al[2];
#pragma unroll
                for (int kap = 0; kap < 2; ++kap)
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        bf16 hi, lo;
                        split(S[dd][2 * kap + (s >> 2)][s & 3], hi, lo);
                        ah[kap][s] = hi; al[kap][s] = lo;
                    }
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    const int i = 16 * tb + lr;
#pragma unroll
                    for (int kap = 0; kap < 2; ++kap) {
                        const bf16x8 bh = ld_pair4(sQt + i * KP + 32 * kap + 4 * g);
                        const bf16x8 bl = ld_pair4(sQt + (C + i) * KP + 32 * kap + 4 * g);
                        acc = mfma(ah[kap], bh, acc);
                        acc = mfma(ah[kap], bl, acc);
                        acc = mfma(al[kap], bh, acc);
                    }
                    O[dd][tb] = acc;
                }
            }

            // ---- scores P^T[j][i] for the own sub-blocks, then O_intra^T = V^T P^T
#pragma unroll
            for (int m = 0; m < BPW; ++m) {
                const int I = w + 4 * m;
                if (I >= NB) break;
                f32x4 P[NB];
#pragma unroll
                for (int J = 0; J < NB; ++J) {
                    P[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (J > I) continue;
                    if (J == I && span_bad[m]) continue;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kap = 0; kap < 2; ++kap) {
                        const int c0 = 32 * kap + 8 * g;
                        const bf16x8 akh = *reinterpret_cast<const bf16x8 *>(sKp + (16 * J + lr) * KP + c0);
                        const bf16x8 akl = *reinterpret_cast<const bf16x8 *>(sKp + (C + 16 * J + lr) * KP + c0);
                        const float *f = sF + (I * (I + 1) / 2 + J) * DK + c0;
                        bf16x8 bh, bl;
#pragma unroll
                        for (int s = 0; s < 8; ++s) {
                            bf16 hi, lo;
                            split(qp[m][8 * kap + s] * f[s], hi, lo);
                            bh[s] = hi; bl[s] = lo;
                        }
                        acc = mfma(akh, bh, acc);
                        acc = mfma(akh, bl, acc);
                        acc = mfma(akl, bh, acc);
                    }
                    if (J == I) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (4 * g + r > lr) acc[r] = 0.f;  // causal: keep j <= i
                    }
                    P[J] = acc;
                }
                if (span_bad[m]) {
                    // Diagonal tile pair by pair: sum_c q_ic k_jc 2^(a_ic - a_jc), j <= i.
                    const int64_t rowi = sRow[16 * I + lr];
                    float q16[16], k16[16], a16[16];
#pragma unroll
                    for (int kap = 0; kap < 2; ++kap) {
                        const int c0 = 32 * kap + 8 * g;
                        if (rowi >= 0) {
                            ld8<DT>(a.q, rowi * DK + c0, &q16[8 * kap]);
                            ld8<DT>(a.k, rowi * DK + c0, &k16[8 * kap]);
                        } else {
#pragma unroll
                            for (int s = 0; s < 8; ++s) { q16[8 * kap + s] = 0.f; k16[8 * kap + s] = 0.f; }
                        }
#pragma unroll
                        for (int s = 0; s < 8; ++s) a16[8 * kap + s] = cs[m][8 * kap + s];
                    }
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    for (int jl = 0; jl < 16; ++jl) {
                        const int src = 16 * g + jl;
                        float part = 0.f;
#pragma unroll
                        for (int s = 0; s < 16; ++s) {
                            const float kj = __shfl(k16[s], src);
                            const float aj = __shfl(a16[s], src);
                            if (jl <= lr) part += q16[s] * kj * fexp2(a16[s] - aj);
                        }
                        part += __shfl_xor(part, 16);
                        part += __shfl_xor(part, 32);
                        if ((jl >> 2) == g) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if ((jl & 3) == r) acc[r] = part;
                        }
                    }
                    P[I] = acc;
                }
                // O_intra^T[d][i] for i in sub-block I, all value columns
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kap = 0; kap < (NB + 1) / 2; ++kap) {
                        if (2 * kap > I) break;
                        bf16x8 bh, bl;
#pragma unroll
                        for (int s = 0; s < 8; ++s) {
                            const int J = 2 * kap + (s >> 2);
                            const float x = (J <= I) ? P[J][s & 3] : 0.f;
                            bf16 hi, lo;
                            split(x, hi, lo);
                            bh[s] = hi; bl[s] = lo;
                        }
                        const int d = 16 * db + lr;
                        bf16x8 av[NV];
#pragma unroll
                        for (int pv = 0; pv < NV; ++pv)
                            av[pv] = ld_pair4(sVt + (pv * DV + d) * CP + 32 * kap + 4 * g);
                        acc = mfma(av[0], bh, acc);
                        acc = mfma(av[0], bl, acc);
                        if (NV == 2) acc = mfma(av[NV - 1], bh, acc);
                    }
                    Oi[m][db] = acc;
                }
            }
        }

        // ---- state update: S = Diag(2^G) S + K~^T V  (own value columns)
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd) {
            const int d = 16 * (w * DPW + dd) + lr;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                f32x4 acc = S[dd][ct];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= sEGc[16 * ct + 4 * g + r];
#pragma unroll
                for (int kt = 0; kt < C / 32; ++kt) {
                    const int j0 = 32 * kt + 8 * g;
                    const bf16x8 akh = *reinterpret_cast<const bf16x8 *>(sKt + (16 * ct + lr) * CP + j0);
                    const bf16x8 akl = *reinterpret_cast<const bf16x8 *>(sKt + (DK + 16 * ct + lr) * CP + j0);
                    const bf16x8 bv0 = *reinterpret_cast<const bf16x8 *>(sVt + d * CP + j0);
                    acc = mfma(akh, bv0, acc);
                    acc = mfma(akl, bv0, acc);
                    if (NV == 2) {
                        const bf16x8 bv1 = *reinterpret_cast<const bf16x8 *>(sVt + (DV + d) * CP + j0);
                        acc = mfma(akh, bv1, acc);
                    }
                }
                S[dd][ct] = acc;
            }
        }

        if (!SUM) {
            __syncthreads();  // every wave is done with sQt / sKp / sKt
            // ---- exchange O_intra^T through sX[d][i]
#pragma unroll
            for (int m = 0; m < BPW; ++m) {
                const int I = w + 4 * m;
                if (I >= NB) break;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sX[(16 * db + 4 * g + r) * K::XP + 16 * I + lr] = Oi[m][db][r];
            }
            __syncthreads();
            // ---- add, then per-token sums of squares for the RMSNorm
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                float ss = 0.f;
#pragma unroll
                for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float o = O[dd][tb][r] +
                                        sX[(16 * (w * DPW + dd) + 4 * g + r) * K::XP + 16 * tb + lr];
                        O[dd][tb][r] = o;
                        ss += o * o;
                    }
                ss += __shfl_xor(ss, 16);
                ss += __shfl_xor(ss, 32);
                if (g == 0) sSS[w * C + 16 * tb + lr] = ss;
            }
            __syncthreads();
            // ---- epilogue: y = o / sqrt(mean o^2 + eps) * rms_w * z * sigmoid(z) -> sY[i][d]
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                const int i = 16 * tb + lr;
                const float ss = sSS[i] + sSS[C + i] + sSS[2 * C + i] + sSS[3 * C + i];
                const float inv = 1.0f / sqrtf(ss * (1.0f / DV) + GTR_RMS_EPS);
                const int64_t row = sRow[i];
#pragma unroll
                for (int dd = 0; dd < DPW; ++dd) {
                    const int d0 = 16 * (w * DPW + dd) + 4 * g;
                    float zz[4] = {0.f, 0.f, 0.f, 0.f};
                    if (row >= 0) {
                        const uint2 zu = *reinterpret_cast<const uint2 *>(
                            static_cast<const uint16_t *>(a.z) + row * DV + d0);
                        zz[0] = h2f<DT>(zu.x & 0xffffu); zz[1] = h2f<DT>(zu.x >> 16);
                        zz[2] = h2f<DT>(zu.y & 0xffffu); zz[3] = h2f<DT>(zu.y >> 16);
                    }
                    const float4 wv = *reinterpret_cast<const float4 *>(a.rms_w + d0);
                    const float ww[4] = {wv.x, wv.y, wv.z, wv.w};
                    uint16_t yb[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float silu = zz[r] / (1.0f + fexp2(-zz[r] * kLog2e));
                        yb[r] = f2h<DT>(O[dd][tb][r] * inv * ww[r] * silu);
                    }
                    uint2 yu;
                    yu.x = static_cast<uint32_t>(yb[0]) | (static_cast<uint32_t>(yb[1]) << 16);
                    yu.y = static_cast<uint32_t>(yb[2]) | (static_cast<uint32_t>(yb[3]) << 16);
                    *reinterpret_cast<uint2 *>(sY + i * K::YP + d0) = yu;
                }
            }
            __syncthreads();
            // ---- grid-order store, 16 bytes per thread per step
            constexpr int PIECES = DV / 8;
            for (int idx = tid; idx < C * PIECES; idx += NT) {
                const int i = idx / PIECES, pc = idx % PIECES;
                const int64_t row = sRow[i];
                if (row >= 0)
                    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.out) + row * DV + 8 * pc) =
                        *reinterpret_cast<const uint4 *>(sY + i * K::YP + 8 * pc);
            }
        }
        __syncthreads();  // LDS is rewritten by the next chunk
    }

    if (SUM) {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    U[soff + static_cast<size_t>(16 * ct + 4 * g + r) * DV + 16 * (w * DPW + dd) + lr] =
                        S[dd][ct][r];
        if (w == 0) G[(static_cast<size_t>(bh) * n_seg + seg) * DK + l] = gam_run * kLn2;
    }
}

template <bool SUM, int DT, int DV, int NB>
hipError_t launch_t(const GlaArgs &a, float *U, float *G, const float *Sx, int n_seg, int sc,
                    hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.H * n_seg));
    hipLaunchKernelGGL((k_chunk<DT, DV, NB, SUM>), grid, dim3(NT), 0, st, a, U, G, Sx, n_seg, sc);
    return hipGetLastError();
}

template <bool SUM, int DT>
hipError_t launch_dt(const GlaArgs &a, float *U, float *G, const float *Sx, int n_seg, int sc,
                     hipStream_t st) {
    if (a.dv == 64) {
        if (a.chunk == 32) return launch_t<SUM, DT, 64, 2>(a, U, G, Sx, n_seg, sc, st);
        if (a.chunk == 64) return launch_t<SUM, DT, 64, 4>(a, U, G, Sx, n_seg, sc, st);
        if (a.chunk == 128) return launch_t<SUM, DT, 64, 8>(a, U, G, Sx, n_seg, sc, st);
    } else if (a.dv == 128) {
        if (a.chunk == 32) return launch_t<SUM, DT, 128, 2>(a, U, G, Sx, n_seg, sc, st);
        if (a.chunk == 64) return launch_t<SUM, DT, 128, 4>(a, U, G, Sx, n_seg, sc, st);
    }
    return hipErrorInvalidValue;
}

template <bool SUM>
hipError_t launch(const GlaArgs &a, float *U, float *G, const float *Sx, int n_seg, int sc,
                  hipStream_t st) {
    if (a.dtype == DT_F16) return launch_dt<SUM, DT_F16>(a, U, G, Sx, n_seg, sc, st);
    if (a.dtype == DT_BF16) return launch_dt<SUM, DT_BF16>(a, U, G, Sx, n_seg, sc, st);
    return hipErrorInvalidValue;
}

}  // namespace

bool mfma_supported(const GlaArgs &a) {
    // chunk 128 with dv 128 would need more LDS than a CU has
    return (a.dtype == DT_F16 || a.dtype == DT_BF16) && a.dk == DK &&
           ((a.dv == 64 && (a.chunk == 32 || a.chunk == 64 || a.chunk == 128)) ||
            (a.dv == 128 && (a.chunk == 32 || a.chunk == 64)));
}

hipError_t mfma_summary(const GlaArgs &a, float *U, float *G, int n_seg, int seg_chunks,
                        hipStream_t s) {
    return launch<true>(a, U, G, nullptr, n_seg, seg_chunks, s);
}

hipError_t mfma_output(const GlaArgs &a, const float *Sx, int n_seg, int seg_chunks,
                       hipStream_t s) {
    return launch<false>(a, nullptr, nullptr, Sx, n_seg, seg_chunks, s);
}

}  // namespace gtr
