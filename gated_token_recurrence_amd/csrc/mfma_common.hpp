// mfma_common.hpp -- per-chunk building blocks of the matrix-core kernels
// (k_mfma.hip: summary and output kernels; k_fast.hip: single-launch kernel).
//
// One chunk of C = 16 NB tokens of one (b, h) sequence, 16-bit I/O, dk = 64
// (GTR write-up "端侧实时感知新标杆！通用线性骨干网络GTR开源": Method §1 gives the
// recurrence, readout, RMSNorm and SiLU(z) gate; Method §4 the chunkwise
// evaluation with on-chip score tiles and an epilogue-fused output gate).
// With a_i the in-chunk inclusive cumulative log2-gate and G = a at the last token:
//   o_i   = (q_i 2^a_i)^T S + sum_{j <= i} (sum_c (q_ic 2^a_ic)(k_jc 2^-a_jc)) v_j
//   S_new = Diag(2^G) S + sum_j (k_j 2^(G - a_j)) v_j^T
// q 2^a and k 2^(G - a) never exceed |q|, |k|; k 2^-a grows with the chunk's
// decay span, so a chunk whose span exceeds kSpanMax (log2 units) is run token
// by token in fp32 instead (S_t = Diag(g_t) S + k_t v_t^T, o_t = S_t^T q_t).
//
// Products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  An fp32
// operand is split into bf16 hi + lo; two split operands take
// hi*hi + hi*lo + lo*hi, a split and an exact operand two products.  fp16
// values are exact as bf16 hi + lo.
//
// Workgroup of 4 waves.  Wave w owns value columns [16 w DPW, 16 (w + 1) DPW)
// of the fp32 state S (MFMA accumulators: S[dd][ct][r] = S[16 ct + 4 g + r]
// [16 (w DPW + dd) + lr]), stages token sub-block w (tokens [16 w, 16 w + 16))
// and computes every fourth causal score tile.  Lane l: lr = l % 16, g = l / 16.
// LDS rows of 16-bit elements keep their 16-byte pieces XOR-swizzled by row,
// so row-parallel 8- and 16-byte accesses spread over the banks.
#pragma once

#include "gtr_internal.hpp"

namespace gtr {
namespace mf {

using bf16 = __bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int NT = 256;
constexpr int DK = 64;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kSpanMax = 64.f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x = hi + lo, hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split(float x, bf16 &hi, bf16 &lo) {
    hi = static_cast<bf16>(x);
    lo = static_cast<bf16>(x - static_cast<float>(hi));
}

// Element offset of (row, col) in an LDS matrix of 16-bit elements with rows of
// W elements (W a multiple of 64): the 8-element pieces of a row are swizzled.
template <int W>
__device__ __forceinline__ int sw(int row, int col) {
    return row * W + ((((col >> 3) ^ (row & 7)) << 3) | (col & 7));
}

// Inclusive prefix sum over the 16 lanes of a DPP row.
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
template <int DT> __device__ __forceinline__ uint32_t f2h(float x);
template <> __device__ __forceinline__ uint32_t f2h<DT_F16>(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
template <> __device__ __forceinline__ uint32_t f2h<DT_BF16>(float x) { return f32_to_bf16(x); }

__device__ __forceinline__ uint32_t half16(const uint4 &u, int s) {
    const uint32_t w = (s < 2) ? u.x : (s < 4) ? u.y : (s < 6) ? u.z : u.w;
    return (s & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int DT, int DV, int NB, bool SUM>
struct Cfg {
    static constexpr int C = 16 * NB;
    static constexpr int NDB = DV / 16;
    static constexpr int DPW = NDB / 4;
    static constexpr int NV = (DT == DT_F16) ? 2 : 1;
    static constexpr int NTRI = NB * (NB + 1) / 2;
    static constexpr int TPW = (NTRI + 3) / 4;
    static constexpr int CW = (C < 64) ? 64 : C;  // row width of [row][token] matrices
    // LDS carve-up (bytes)
    static constexpr int QT = SUM ? 0 : 2 * C * DK * 2;  // Q~ hi, lo [i][c]   (fallback: q fp32)
    static constexpr int KH = SUM ? 0 : 2 * C * DK * 2;  // K^ hi, lo [j][c]   (fallback: k fp32)
    static constexpr int KT = 2 * DK * CW * 2;           // K~^T hi, lo [c][j] (fallback: g fp32)
    static constexpr int VT = NV * DV * CW * 2;          // V^T parts [d][j]
    static constexpr int PB = SUM ? 0 : NTRI * 1024;     // score tiles: [tile][hi, lo][lane][4]
    static constexpr int O_QT = 0;
    static constexpr int O_KH = O_QT + QT;
    static constexpr int O_KT = O_KH + KH;
    static constexpr int O_VT = O_KT + KT;
    static constexpr int O_P = O_VT + VT;
    static constexpr int O_TOT = O_P + PB;                      // float [NB][DK]
    static constexpr int O_TAB = O_TOT + NB * DK * 4;           // float [4 waves][3][DK]
    static constexpr int O_SS = O_TAB + 4 * 3 * DK * 4;         // float [4][C]
    static constexpr int O_ROW = O_SS + (SUM ? 0 : 4 * C * 4);  // int64 [2][C]
    static constexpr int BYTES = O_ROW + 2 * C * 8;
    static_assert(NB == 2 || NB == 4, "chunks of 32 or 64 tokens");
    static_assert(SUM || C * DK * 4 <= QT, "fallback q must fit");
    static_assert(C * DK * 4 <= KT, "fallback g must fit");
};

// State of one workgroup working through chunks.  Everything is inlined; the
// arrays live in registers.
template <int DT, int DV, int NB, bool SUM>
struct Tile {
    using K = Cfg<DT, DV, NB, SUM>;
    static constexpr int C = K::C, DPW = K::DPW, NV = K::NV, NTRI = K::NTRI, CW = K::CW;

    GlaArgs a;
    bf16 *sQt, *sKh, *sKt, *sVt, *sP;
    float *sTot, *sTab, *sSS, *fQ, *fK, *fG;
    int64_t *sRow;
    int tid, w, l, lr, g;
    bool own;  // this wave stages a token sub-block (w < NB)

    // next chunk's inputs (registers)
    uint4 pq[2], pk[2], pv[DV / 32];
    float4 pg[4];
    uint2 pz[DPW][NB];
    int64_t rowE[NB];
    float rw[DPW][4];
    // chunk state
    f32x4 S[DPW][4];
    f32x4 O[DPW][NB];
    float cs[16];

    __device__ __forceinline__ void init(const GlaArgs &args, char *smem) {
        a = args;
        sQt = reinterpret_cast<bf16 *>(smem + K::O_QT);
        sKh = reinterpret_cast<bf16 *>(smem + K::O_KH);
        sKt = reinterpret_cast<bf16 *>(smem + K::O_KT);
        sVt = reinterpret_cast<bf16 *>(smem + K::O_VT);
        sP = reinterpret_cast<bf16 *>(smem + K::O_P);
        sTot = reinterpret_cast<float *>(smem + K::O_TOT);
        sSS = reinterpret_cast<float *>(smem + K::O_SS);
        sRow = reinterpret_cast<int64_t *>(smem + K::O_ROW);
        fQ = reinterpret_cast<float *>(smem + K::O_QT);
        fK = reinterpret_cast<float *>(smem + K::O_KH);
        fG = reinterpret_cast<float *>(smem + K::O_KT);
        tid = threadIdx.x;
        w = tid >> 6;
        l = tid & 63;
        lr = l & 15;
        g = l >> 4;
        own = w < NB;
        sTab = reinterpret_cast<float *>(smem + K::O_TAB) + w * 3 * DK;
        if (!SUM) {
#pragma unroll
            for (int dd = 0; dd < DPW; ++dd) {
                const float4 t =
                    *reinterpret_cast<const float4 *>(a.rms_w + 16 * (w * DPW + dd) + 4 * g);
                rw[dd][0] = t.x; rw[dd][1] = t.y; rw[dd][2] = t.z; rw[dd][3] = t.w;
            }
        }
    }

    // Row index ((b L + grid position) H + h) of every token of chunk ch of sequence bh.
    __device__ __forceinline__ void rows_of(int64_t bh, int64_t ch, int buf) {
        if (tid < C) {
            const uint32_t L32 = static_cast<uint32_t>(a.L);
            uint32_t t = static_cast<uint32_t>(ch) * C + tid;
            int64_t row = -1;
            if (t < L32) {
                if (a.direction & 1) t = L32 - 1 - t;  // RL, BT: reversed sequence
                uint32_t pos = t;
                if (a.direction >= 2) {                // TB, BT: column-major raster
                    const uint32_t gh = static_cast<uint32_t>(a.gh);
                    const uint32_t c = t / gh;
                    pos = (t - c * gh) * static_cast<uint32_t>(a.gw) + c;
                }
                const uint32_t b = static_cast<uint32_t>(bh) / static_cast<uint32_t>(a.H);
                const uint32_t h = static_cast<uint32_t>(bh) - b * static_cast<uint32_t>(a.H);
                row = (static_cast<int64_t>(b) * a.L + pos) * a.H + h;
            }
            sRow[buf * C + tid] = row;
        }
    }

    __device__ __forceinline__ void prefetch_main(int buf) {
        if (!own) return;
        const int64_t row = sRow[buf * C + 16 * w + lr];
#pragma unroll
        for (int kap = 0; kap < 2; ++kap) {
            const int c0 = 32 * kap + 8 * g;
            if (row >= 0) {
                if (!SUM)
                    pq[kap] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) +
                                                               row * DK + c0);
                pk[kap] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) +
                                                           row * DK + c0);
                pg[2 * kap] = *reinterpret_cast<const float4 *>(a.log_g + row * DK + c0);
                pg[2 * kap + 1] = *reinterpret_cast<const float4 *>(a.log_g + row * DK + c0 + 4);
            } else {
                pq[kap] = make_uint4(0, 0, 0, 0);
                pk[kap] = make_uint4(0, 0, 0, 0);
                pg[2 * kap] = make_float4(0.f, 0.f, 0.f, 0.f);
                pg[2 * kap + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int vm = 0; vm < DV / 32; ++vm) {
            const int d0 = 8 * (g + 4 * vm);
            uint4 x = make_uint4(0, 0, 0, 0);
            if (row >= 0) {
                x = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) + row * DV +
                                                     d0);
                if (a.resid) {  // stack residual: v + out_prev, rounded to the I/O type
                    const uint4 y = *reinterpret_cast<const uint4 *>(
                        static_cast<const uint16_t *>(a.resid) + row * DV + d0);
                    uint32_t xs[4] = {x.x, x.y, x.z, x.w};
                    const uint32_t ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo = f2h<DT>(h2f<DT>(xs[e] & 0xffffu) + h2f<DT>(ys[e] & 0xffffu));
                        const uint32_t hi = f2h<DT>(h2f<DT>(xs[e] >> 16) + h2f<DT>(ys[e] >> 16));
                        xs[e] = lo | (hi << 16);
                    }
                    x = make_uint4(xs[0], xs[1], xs[2], xs[3]);
                }
            }
            pv[vm] = x;
        }
    }

    __device__ __forceinline__ void prefetch_z(int buf) {
        if (SUM) return;
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            const int64_t row = sRow[buf * C + 16 * tb + lr];
            rowE[tb] = row;
#pragma unroll
            for (int dd = 0; dd < DPW; ++dd) {
                const int d0 = 16 * (w * DPW + dd) + 4 * g;
                pz[dd][tb] = row >= 0 ? *reinterpret_cast<const uint2 *>(
                                            static_cast<const uint16_t *>(a.z) + row * DV + d0)
                                      : make_uint2(0, 0);
            }
        }
    }

    __device__ __forceinline__ void zero_state() {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) S[dd][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // state [DK][DV] fp32 at src
    __device__ __forceinline__ void load_state(const float *src) {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[dd][ct][r] = src[(16 * ct + 4 * g + r) * DV + 16 * (w * DPW + dd) + lr];
    }

    __device__ __forceinline__ void store_state(float *dst) const {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(16 * ct + 4 * g + r) * DV + 16 * (w * DPW + dd) + lr] = S[dd][ct][r];
    }

    // One step of a scan over chunk summaries, in the state's register layout:
    // S <- Diag(e) S + u, with u a [DK][DV] summary and e the per-channel decay.
    struct StateIn {
        f32x4 e[4];
        float u[DPW][4][4];
    };
    __device__ __forceinline__ void state_in_load(StateIn &x, const float *u, const float *e) const {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const float4 d = *reinterpret_cast<const float4 *>(e + 16 * ct + 4 * g);
            x.e[ct] = f32x4{d.x, d.y, d.z, d.w};
        }
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    x.u[dd][ct][r] = u[(16 * ct + 4 * g + r) * DV + 16 * (w * DPW + dd) + lr];
    }
    __device__ __forceinline__ void state_in_apply(const StateIn &x) {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[dd][ct][r] = fmaf(S[dd][ct][r], x.e[ct][r], x.u[dd][ct][r]);
    }

    // ---- phase 1: cumulative gates within the sub-block (registers), block totals,
    // V^T into LDS.  Consumes the prefetched inputs except q and k.
    __device__ __forceinline__ void phase1() {
        if (!own) return;
        const int i = 16 * w + lr;
#pragma unroll
        for (int kap = 0; kap < 2; ++kap) {
            const float gl[8] = {pg[2 * kap].x, pg[2 * kap].y, pg[2 * kap].z, pg[2 * kap].w,
                                 pg[2 * kap + 1].x, pg[2 * kap + 1].y, pg[2 * kap + 1].z,
                                 pg[2 * kap + 1].w};
#pragma unroll
            for (int s = 0; s < 8; ++s) cs[8 * kap + s] = row_scan(gl[s] * kLog2e);
        }
        if (lr == 15) {
#pragma unroll
            for (int kap = 0; kap < 2; ++kap) {
                float *dst = sTot + w * DK + 32 * kap + 8 * g;
                *reinterpret_cast<float4 *>(dst) =
                    make_float4(cs[8 * kap], cs[8 * kap + 1], cs[8 * kap + 2], cs[8 * kap + 3]);
                *reinterpret_cast<float4 *>(dst + 4) =
                    make_float4(cs[8 * kap + 4], cs[8 * kap + 5], cs[8 * kap + 6], cs[8 * kap + 7]);
            }
        }
#pragma unroll
        for (int vm = 0; vm < DV / 32; ++vm) {
            const int d0 = 8 * (g + 4 * vm);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const uint32_t bits = half16(pv[vm], s);
                if (NV == 2) {
                    bf16 hi, lo;
                    split(h2f<DT>(bits), hi, lo);
                    sVt[sw<CW>(d0 + s, i)] = hi;
                    sVt[DV * CW + sw<CW>(d0 + s, i)] = lo;
                } else {
                    sVt[sw<CW>(d0 + s, i)] = __builtin_bit_cast(bf16, static_cast<uint16_t>(bits));
                }
            }
        }
    }

    // ---- phase 2 (after phase 1 everywhere): chunk totals, span check, operands.
    // Lane l computes for channel l the sum r of the sub-block totals before the
    // wave's own sub-block and the chunk total G; the wave's table holds r, G
    // and 2^G (G, in log2 units, is added to *gam).  Returns whether the chunk
    // must be run token by token (the same in every wave).
    __device__ __forceinline__ bool phase2(float *gam) {
        const int Iown = own ? w : 0;
        float r_l = 0.f, tot_l = 0.f;
#pragma unroll
        for (int J = 0; J < NB; ++J) {
            const float t = sTot[J * DK + l];
            if (J < Iown) r_l += t;
            tot_l += t;
        }
        bool slow = false;
        if (!SUM) {
            float sp2 = -tot_l;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) sp2 = fmaxf(sp2, __shfl_xor(sp2, off));
            slow = sp2 > kSpanMax;
        }
        *gam += tot_l;
        sTab[l] = r_l;
        sTab[DK + l] = tot_l;
        sTab[2 * DK + l] = fexp2(tot_l);
        __builtin_amdgcn_wave_barrier();
        if (!own) return slow;
        const int i = 16 * w + lr;
#pragma unroll
        for (int kap = 0; kap < 2; ++kap) {
            const int c0 = 32 * kap + 8 * g;
            float rI[8], gC[8], eG[8], kv[8], qv[8];
#pragma unroll
            for (int h4 = 0; h4 < 2; ++h4) {
                const float4 x = *reinterpret_cast<const float4 *>(sTab + c0 + 4 * h4);
                const float4 y = *reinterpret_cast<const float4 *>(sTab + DK + c0 + 4 * h4);
                const float4 z = *reinterpret_cast<const float4 *>(sTab + 2 * DK + c0 + 4 * h4);
                rI[4 * h4] = x.x; rI[4 * h4 + 1] = x.y; rI[4 * h4 + 2] = x.z; rI[4 * h4 + 3] = x.w;
                gC[4 * h4] = y.x; gC[4 * h4 + 1] = y.y; gC[4 * h4 + 2] = y.z; gC[4 * h4 + 3] = y.w;
                eG[4 * h4] = z.x; eG[4 * h4 + 1] = z.y; eG[4 * h4 + 2] = z.z; eG[4 * h4 + 3] = z.w;
            }
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                kv[s] = h2f<DT>(half16(pk[kap], s));
                qv[s] = SUM ? 0.f : h2f<DT>(half16(pq[kap], s));
            }
            if (SUM) {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float kt = kv[s] * fexp2(gC[s] - rI[s] - cs[8 * kap + s]);  // k 2^(G - a)
                    bf16 hi, lo;
                    split(kt, hi, lo);
                    sKt[sw<CW>(c0 + s, i)] = hi;
                    sKt[DK * CW + sw<CW>(c0 + s, i)] = lo;
                }
            } else if (!slow) {
                bf16x8 qh, ql, kh, kl;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float aa = rI[s] + cs[8 * kap + s];
                    const float kh_f = kv[s] * fexp2(-aa);  // k 2^-a
                    bf16 hi, lo;
                    split(qv[s] * fexp2(aa), hi, lo);       // q 2^a
                    qh[s] = hi; ql[s] = lo;
                    split(kh_f, hi, lo);
                    kh[s] = hi; kl[s] = lo;
                    split(kh_f * eG[s], hi, lo);            // k 2^(G - a)
                    sKt[sw<CW>(c0 + s, i)] = hi;
                    sKt[DK * CW + sw<CW>(c0 + s, i)] = lo;
                }
                *reinterpret_cast<bf16x8 *>(sQt + sw<DK>(i, c0)) = qh;
                *reinterpret_cast<bf16x8 *>(sQt + C * DK + sw<DK>(i, c0)) = ql;
                *reinterpret_cast<bf16x8 *>(sKh + sw<DK>(i, c0)) = kh;
                *reinterpret_cast<bf16x8 *>(sKh + C * DK + sw<DK>(i, c0)) = kl;
            } else {
                // token-serial operands: q, k and g = 2^(a_i - a_{i-1}) in fp32 [token][channel],
                // plus k 2^(G - a) for a summary of the chunk
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    fQ[i * DK + c0 + s] = qv[s];
                    fK[i * DK + c0 + s] = kv[s];
                    const float up = __shfl_up(cs[8 * kap + s], 1, 16);
                    const float prev = (lr == 0) ? 0.f : up;
                    fG[i * DK + c0 + s] = fexp2(cs[8 * kap + s] - prev);
                }
            }
        }
        return slow;
    }

    // ---- inter-chunk readout O^T[d][i] = S^T (Q~)^T (the state before the chunk)
    __device__ __forceinline__ void inter() {
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
            for (int tb = 0; tb < NB; ++tb) O[dd][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kap = 0; kap < 2; ++kap) {
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) {
                    const int i = 16 * tb + lr;
                    const int c0 = 32 * kap + 4 * g;
                    const bf16x4 h0 = *reinterpret_cast<const bf16x4 *>(sQt + sw<DK>(i, c0));
                    const bf16x4 h1 = *reinterpret_cast<const bf16x4 *>(sQt + sw<DK>(i, c0 + 16));
                    const bf16x4 l0 = *reinterpret_cast<const bf16x4 *>(sQt + C * DK + sw<DK>(i, c0));
                    const bf16x4 l1 = *reinterpret_cast<const bf16x4 *>(sQt + C * DK + sw<DK>(i, c0 + 16));
                    const bf16x8 bh = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
                    const bf16x8 bl = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
                    O[dd][tb] = mfma(ah[kap], bh, O[dd][tb]);
                    O[dd][tb] = mfma(ah[kap], bl, O[dd][tb]);
                    O[dd][tb] = mfma(al[kap], bh, O[dd][tb]);
                }
            }
        }
    }

    // ---- causal score tiles P^T[j][i] = K^_J (Q~_I)^T, every fourth tile, into sP
    __device__ __forceinline__ void scores() {
#pragma unroll
        for (int tt = 0; tt < K::TPW; ++tt) {
            const int t = w + 4 * tt;
            if (t >= NTRI) break;
            int I = 0;
            while ((I + 1) * (I + 2) / 2 <= t) ++I;
            const int J = t - I * (I + 1) / 2;
            bf16x8 ak[2][2], bq[2][2];
#pragma unroll
            for (int kap = 0; kap < 2; ++kap) {
                const int c0 = 32 * kap + 8 * g;
#pragma unroll
                for (int hl = 0; hl < 2; ++hl) {
                    ak[kap][hl] = *reinterpret_cast<const bf16x8 *>(sKh + hl * C * DK + sw<DK>(16 * J + lr, c0));
                    bq[kap][hl] = *reinterpret_cast<const bf16x8 *>(sQt + hl * C * DK + sw<DK>(16 * I + lr, c0));
                }
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kap = 0; kap < 2; ++kap) {
                acc = mfma(ak[kap][0], bq[kap][0], acc);
                acc = mfma(ak[kap][0], bq[kap][1], acc);
                acc = mfma(ak[kap][1], bq[kap][0], acc);
            }
            bf16x4 ph, plo;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = (J == I && 4 * g + r > lr) ? 0.f : acc[r];  // keep j <= i
                bf16 hi, lo;
                split(x, hi, lo);
                ph[r] = hi; plo[r] = lo;
            }
            *reinterpret_cast<bf16x4 *>(sP + (2 * t) * 256 + 4 * l) = ph;
            *reinterpret_cast<bf16x4 *>(sP + (2 * t + 1) * 256 + 4 * l) = plo;
        }
    }

    // ---- state update S = Diag(2^G) S + K~^T V
    __device__ __forceinline__ void s_update() {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd) {
            const int d = 16 * (w * DPW + dd) + lr;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const float4 e4 = *reinterpret_cast<const float4 *>(sTab + 2 * DK + 16 * ct + 4 * g);
                S[dd][ct][0] *= e4.x; S[dd][ct][1] *= e4.y; S[dd][ct][2] *= e4.z; S[dd][ct][3] *= e4.w;
            }
#pragma unroll
            for (int kt = 0; kt < C / 32; ++kt) {
                const int j0 = 32 * kt + 8 * g;
                const bf16x8 bv0 = *reinterpret_cast<const bf16x8 *>(sVt + sw<CW>(d, j0));
                bf16x8 bv1 = bv0;
                if (NV == 2) bv1 = *reinterpret_cast<const bf16x8 *>(sVt + DV * CW + sw<CW>(d, j0));
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const bf16x8 akh = *reinterpret_cast<const bf16x8 *>(sKt + sw<CW>(16 * ct + lr, j0));
                    const bf16x8 akl = *reinterpret_cast<const bf16x8 *>(sKt + DK * CW + sw<CW>(16 * ct + lr, j0));
                    S[dd][ct] = mfma(akh, bv0, S[dd][ct]);
                    S[dd][ct] = mfma(akl, bv0, S[dd][ct]);
                    if (NV == 2) S[dd][ct] = mfma(akh, bv1, S[dd][ct]);
                }
            }
        }
    }

    // ---- intra-chunk readout O^T[d][i] += V^T P^T (score tiles from sP)
    __device__ __forceinline__ void intra() {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd) {
            const int d = 16 * (w * DPW + dd) + lr;
#pragma unroll
            for (int kap = 0; kap < NB / 2; ++kap) {
                const int j0 = 32 * kap + 4 * g;
                bf16x8 av[NV];
#pragma unroll
                for (int pp = 0; pp < NV; ++pp) {
                    const bf16x4 x0 = *reinterpret_cast<const bf16x4 *>(sVt + pp * DV * CW + sw<CW>(d, j0));
                    const bf16x4 x1 = *reinterpret_cast<const bf16x4 *>(sVt + pp * DV * CW + sw<CW>(d, j0 + 16));
                    av[pp] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
                }
#pragma unroll
                for (int I = 2 * kap; I < NB; ++I) {
                    const int t0 = I * (I + 1) / 2 + 2 * kap;
                    const bf16x4 zero = {};
                    const bool two = 2 * kap + 1 <= I;
                    const bf16x4 h0 = *reinterpret_cast<const bf16x4 *>(sP + (2 * t0) * 256 + 4 * l);
                    const bf16x4 l0 = *reinterpret_cast<const bf16x4 *>(sP + (2 * t0 + 1) * 256 + 4 * l);
                    const bf16x4 h1 = two ? *reinterpret_cast<const bf16x4 *>(sP + (2 * t0 + 2) * 256 + 4 * l) : zero;
                    const bf16x4 l1 = two ? *reinterpret_cast<const bf16x4 *>(sP + (2 * t0 + 3) * 256 + 4 * l) : zero;
                    const bf16x8 bh = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
                    const bf16x8 bl = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
                    O[dd][I] = mfma(av[0], bh, O[dd][I]);
                    O[dd][I] = mfma(av[0], bl, O[dd][I]);
                    if (NV == 2) O[dd][I] = mfma(av[NV - 1], bh, O[dd][I]);
                }
            }
        }
    }

    // ---- token-serial chunk: S and O from the fp32 operands of phase 2
    __device__ __forceinline__ void serial() {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) O[dd][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int t = 0; t < C; ++t) {
#pragma unroll
            for (int dd = 0; dd < DPW; ++dd) {
                const int d = 16 * (w * DPW + dd) + lr;
                float vd = static_cast<float>(sVt[sw<CW>(d, t)]);
                if (NV == 2) vd += static_cast<float>(sVt[DV * CW + sw<CW>(d, t)]);
                float part = 0.f;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const float4 gq = *reinterpret_cast<const float4 *>(fG + t * DK + 16 * ct + 4 * g);
                    const float4 kq = *reinterpret_cast<const float4 *>(fK + t * DK + 16 * ct + 4 * g);
                    const float4 qq = *reinterpret_cast<const float4 *>(fQ + t * DK + 16 * ct + 4 * g);
                    const float gg[4] = {gq.x, gq.y, gq.z, gq.w};
                    const float kk[4] = {kq.x, kq.y, kq.z, kq.w};
                    const float q4[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        S[dd][ct][r] = gg[r] * S[dd][ct][r] + kk[r] * vd;
                        part += S[dd][ct][r] * q4[r];
                    }
                }
                part += __shfl_xor(part, 16);
                part += __shfl_xor(part, 32);
                // o_t at value column 16 (w DPW + dd) + lr is now in every lane group
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = __shfl(part, 4 * g + r);
                    if (lr == (t & 15)) {
#pragma unroll
                        for (int tb = 0; tb < NB; ++tb)
                            if (tb == (t >> 4)) O[dd][tb][r] = x;
                    }
                }
            }
        }
    }

    // ---- per-token sums of squares of this wave's value columns into sSS
    __device__ __forceinline__ void sum_squares() {
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            float ss = 0.f;
#pragma unroll
            for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
                for (int r = 0; r < 4; ++r) ss += O[dd][tb][r] * O[dd][tb][r];
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            if (g == 0) sSS[w * C + 16 * tb + lr] = ss;
        }
    }

    // ---- epilogue (after sum_squares everywhere):
    // y = o / sqrt(mean_j o_j^2 + eps) * rms_w * z * sigmoid(z), stored at the grid position
    __device__ __forceinline__ void epilogue() {
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            const int i = 16 * tb + lr;
            const float ss = sSS[i] + sSS[C + i] + sSS[2 * C + i] + sSS[3 * C + i];
            const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / DV) + GTR_RMS_EPS);
            const int64_t row = rowE[tb];
#pragma unroll
            for (int dd = 0; dd < DPW; ++dd) {
                const float zz[4] = {h2f<DT>(pz[dd][tb].x & 0xffffu), h2f<DT>(pz[dd][tb].x >> 16),
                                     h2f<DT>(pz[dd][tb].y & 0xffffu), h2f<DT>(pz[dd][tb].y >> 16)};
                uint32_t yb[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float silu = zz[r] * frcp(1.0f + fexp2(-zz[r] * kLog2e));
                    yb[r] = f2h<DT>(O[dd][tb][r] * inv * rw[dd][r] * silu);
                }
                if (row >= 0)
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + row * DV +
                                               16 * (w * DPW + dd) + 4 * g) =
                        make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
            }
        }
    }
};

}  // namespace mf
}  // namespace gtr
