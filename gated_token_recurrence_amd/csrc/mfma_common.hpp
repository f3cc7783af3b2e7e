// mfma_common.hpp -- per-chunk building blocks of the matrix-core kernels
// (k_mfma.hip: summary and output kernels; k_fast.hip: single-launch kernel).
//
// One chunk of C = 16 NB tokens of one (b, h) sequence, 16-bit I/O, dk = 64
// (GTR write-up "端侧实时感知新标杆！通用线性骨干网络GTR开源": Method §1 gives the
// recurrence, readout, RMSNorm and SiLU(z) gate; Method §4 the chunkwise
// evaluation with on-chip score tiles and an epilogue-fused output gate).
// With a_i the in-chunk inclusive cumulative log2-gate and G = a at the last token:
//   o_i   = (q_i 2^a_i)^T S + sum_{j <= i} (sum_c (q_ic 2^a_ic)(k_jc 2^-a_jc)) v_j
//   S_new = Diag(2^G) (S + sum_j (k_j 2^-a_j) v_j^T)            (output kernel)
//         = Diag(2^G) S + sum_j (k_j 2^(G - a_j)) v_j^T         (summary kernel)
// q 2^a and k 2^(G - a) never exceed |q|, |k|; k 2^-a grows with the chunk's
// decay span, so a chunk whose span exceeds kSpanMax (log2 units) is run token
// by token in fp32 instead (S_t = Diag(g_t) S + k_t v_t^T, o_t = S_t^T q_t).
//
// Products run on v_mfma_f32_16x16x32_{bf16,f16} with fp32 accumulation.  An
// fp32 operand is split into hi + lo of the 16-bit type; two split operands take
// hi*hi + hi*lo + lo*hi, a split and an exact operand two products.  fp16 values
// are exact as bf16 hi + lo.  The summary kernel takes k 2^(G - a), which never
// exceeds |k|, in the I/O type's own format (fp16 hi + lo for fp16 I/O), so v
// enters its products as stored.
//
// LDS matrices are token-major ([token][64 columns] of 16-bit elements, as the
// inputs are stored); the operands that run along tokens (K^T, V, V^T) are read
// with the transposing LDS load ds_read_b64_tr_b16.  The 16-byte pieces of a row
// are XOR-swizzled by a function of the row chosen so that both row-parallel
// 16-byte accesses and the transposing reads are free of bank conflicts.
//
// Workgroup of 4 waves.  Wave w owns value columns [16 w DPW, 16 (w + 1) DPW)
// of the fp32 state S (MFMA accumulators: S[dd][ct][r] = S[16 ct + 4 g + r]
// [16 (w DPW + dd) + lr]), stages token sub-block w (tokens [16 w, 16 w + 16))
// and computes every fourth causal score tile.  Lane l: lr = l % 16, g = l / 16.
#pragma once

#include "gtr_internal.hpp"

namespace gtr {
namespace mf {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef short s16x4 __attribute__((ext_vector_type(4)));  // raw 16-bit elements
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int NT = 256;
constexpr int DK = 64;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kSpanMax = 64.f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }

// D += A B on raw 16-bit operands, fp16 (F16) or bf16 elements.
template <bool F16>
__device__ __forceinline__ f32x4 mma(s16x8 a, s16x8 b, f32x4 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// (a, b) rounded to a packed pair of the 16-bit type, and back to floats
template <bool F16>
__device__ __forceinline__ uint32_t pk2(float a, float b) {
    const f32x2_t v = {a, b};
    if constexpr (F16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
template <bool F16>
__device__ __forceinline__ void unpk2(uint32_t u, float &a, float &b) {
    if constexpr (F16) {
        const f16x2_t h = __builtin_bit_cast(f16x2_t, u);
        a = static_cast<float>(h[0]);
        b = static_cast<float>(h[1]);
    } else {
        a = __uint_as_float(u << 16);
        b = __uint_as_float(u & 0xffff0000u);
    }
}

// x = hi + lo element-wise, hi and lo as packed pairs of the 16-bit type
template <bool F16, int N>
__device__ __forceinline__ void split_pk(const float (&x)[N], uint32_t (&hi)[N / 2],
                                         uint32_t (&lo)[N / 2]) {
#pragma unroll
    for (int e = 0; e < N / 2; ++e) {
        hi[e] = pk2<F16>(x[2 * e], x[2 * e + 1]);
        float h0, h1;
        unpk2<F16>(hi[e], h0, h1);
        lo[e] = pk2<F16>(x[2 * e] - h0, x[2 * e + 1] - h1);
    }
}

__device__ __forceinline__ uint4 u4(const uint32_t (&x)[4]) { return make_uint4(x[0], x[1], x[2], x[3]); }

// 16-byte store with the streaming (non-temporal) hint: for outputs nothing in the
// same call reads again.  Measured on MI355X, it keeps them from lingering dirty in
// the caches, whose later write-back otherwise slows the next call's first reads.
__device__ __forceinline__ void store_stream16(void *p, const uint4 &v) {
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t *>(p));
}

// the eight 16-bit values of u as floats (I/O type DT)
template <int DT>
__device__ __forceinline__ void unpack8(const uint4 &u, float (&x)[8]) {
    unpk2<DT == DT_F16>(u.x, x[0], x[1]);
    unpk2<DT == DT_F16>(u.y, x[2], x[3]);
    unpk2<DT == DT_F16>(u.z, x[4], x[5]);
    unpk2<DT == DT_F16>(u.w, x[6], x[7]);
}

// Element offset of (row, col) in a token-major LDS matrix of 16-bit elements
// with 64 columns.  The eight 16-byte pieces of a row are XOR-swizzled by
// f(row) = 2 ((row >> 1) & 3) + ((row >> 3) & 1): sixteen consecutive rows at
// one column piece, and the 4-row x 16-column blocks of a transposing read,
// then spread over all banks.
__device__ __forceinline__ int swn(int row, int col) {
    const int f = (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
    return row * 64 + ((((col >> 3) ^ f) << 3) | (col & 7));
}

__device__ __forceinline__ s16x4 ld_tr(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
}

// Inclusive prefix sums over the 16 lanes of a DPP row, of N values at once
// (one shift step for all values before the next, so no step waits on the last).
template <int N>
__device__ __forceinline__ void row_scan(float (&x)[N]) {
#pragma unroll
    for (int s = 0; s < N; ++s)
        x[s] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[s]), 0x111, 0xf, 0xf, true));
#pragma unroll
    for (int s = 0; s < N; ++s)
        x[s] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[s]), 0x112, 0xf, 0xf, true));
#pragma unroll
    for (int s = 0; s < N; ++s)
        x[s] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[s]), 0x114, 0xf, 0xf, true));
#pragma unroll
    for (int s = 0; s < N; ++s)
        x[s] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[s]), 0x118, 0xf, 0xf, true));
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

// x + y element-wise on eight 16-bit values of the I/O type, each sum formed in
// float32 and rounded to nearest even to the I/O type (the stack residual
// v + out_prev), two values per packed conversion
template <int DT>
__device__ __forceinline__ uint4 add_io(const uint4 &x, const uint4 &y) {
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
    const uint32_t ys[4] = {y.x, y.y, y.z, y.w};
    uint32_t o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        float x0, x1, y0, y1;
        unpk2<DT == DT_F16>(xs[u], x0, x1);
        unpk2<DT == DT_F16>(ys[u], y0, y1);
        o[u] = pk2<DT == DT_F16>(x0 + y0, x1 + y1);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ uint32_t half16(const uint4 &u, int s) {
    const uint32_t w = (s < 2) ? u.x : (s < 4) ? u.y : (s < 6) ? u.z : u.w;
    return (s & 1) ? (w >> 16) : (w & 0xffffu);
}

typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;

// D += A B, 16x16x16, raw 16-bit operands (4 per lane): lane i holds A[i % 16]
// [4 (i / 16) ..], B[4 (i / 16) ..][i % 16] and D[4 (i / 16) + r][i % 16].
template <bool F16>
__device__ __forceinline__ f32x4 mma16(s16x4 a, s16x4 b, f32x4 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Forget gate of one token from its rank-16 features (GTR write-up, Method §1:
// a light low-rank projection of the input with a temperature), for the 16 key
// channels a lane holds in the token-row layout: lane (lr, g) of a wave holds
// token lr and cs[8 kap + s] is channel 32 kap + 8 g + s.  The projection runs
// as four 16x16x16 products with M = 16 channels, K = the 16 ranks, N = 16
// tokens; tile ct puts in its row m the channel
//     chan(ct, m) = 32 (ct / 2) + 8 (m / 4) + 4 (ct % 2) + m % 4,
// so that output element r of tile ct (row 4 g + r) is cs[4 ct + r].
template <int DT>
struct LowRankGate {
    s16x4 wa[4];    // A operands: gate_w[4 g + j][h dk + chan(ct, lr)], j < 4
    f32x4 bias[4];  // gate_b of the lane's output channels (the accumulator start)
    float inv_tau;

    __device__ __forceinline__ static int chan(int ct, int m) {
        return 32 * (ct >> 1) + 8 * (m >> 2) + 4 * (ct & 1) + (m & 3);
    }
    // weights of head h (loads; the caller waits for them before the chunk loop)
    __device__ __forceinline__ void load(const GlaArgs &a, uint32_t h, int lr, int g) {
        const uint16_t *wp = static_cast<const uint16_t *>(a.gate_w);
        const int64_t hd = static_cast<int64_t>(a.H) * DK;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int64_t col = static_cast<int64_t>(h) * DK + chan(ct, lr);
#pragma unroll
            for (int j = 0; j < 4; ++j) wa[ct][j] = static_cast<short>(wp[(4 * g + j) * hd + col]);
            const float4 b4 = *reinterpret_cast<const float4 *>(a.gate_b + h * DK + chan(ct, 4 * g));
            bias[ct] = f32x4{b4.x, b4.y, b4.z, b4.w};
        }
        inv_tau = a.inv_tau;
    }
    __device__ __forceinline__ void ready() const {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) asm volatile("" ::"v"(wa[ct]), "v"(bias[ct]));
    }
    // cs (natural-log units) from this lane's features f = feat[token lr][4 g .. 4 g + 3]
    __device__ __forceinline__ void gates(uint2 f, float (&cs)[16]) const {
        const s16x4 fb = __builtin_bit_cast(s16x4, f);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const f32x4 x = mma16<DT == DT_F16>(wa[ct], fb, bias[ct]);
#pragma unroll
            for (int r = 0; r < 4; ++r) cs[4 * ct + r] = log_sigmoid(x[r]) * inv_tau;
        }
    }

    // LDS copy for kernels short of registers: the A operands [4][64 lanes] and
    // the 64 biases of the head.  Every wave of a workgroup works on the same head
    // and writes the whole copy (the same values), so a wave's own writes are all
    // it needs before reading; callers write only after every wave is done with
    // the previous head's copy.
    static constexpr int LDS_BYTES = 4 * 64 * 8 + 64 * 4;
    __device__ __forceinline__ void put(char *m, int l, int g) const {
        s16x4 *wm = reinterpret_cast<s16x4 *>(m);
        float *bm = reinterpret_cast<float *>(m + 4 * 64 * 8);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            wm[ct * 64 + l] = wa[ct];
            *reinterpret_cast<f32x4 *>(bm + chan(ct, 4 * g)) = bias[ct];
        }
    }
    __device__ __forceinline__ static void gates_lds(const char *m, int l, int g, float itau,
                                                     uint2 f, float (&cs)[16]) {
        const s16x4 *wm = reinterpret_cast<const s16x4 *>(m);
        const float *bm = reinterpret_cast<const float *>(m + 4 * 64 * 8);
        const s16x4 fb = __builtin_bit_cast(s16x4, f);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const f32x4 b = *reinterpret_cast<const f32x4 *>(bm + chan(ct, 4 * g));
            const f32x4 x = mma16<DT == DT_F16>(wm[ct * 64 + l], fb, b);
#pragma unroll
            for (int r = 0; r < 4; ++r) cs[4 * ct + r] = log_sigmoid(x[r]) * itau;
        }
    }
};

template <int DT, int DV, int NB, bool SUM>
struct Cfg {
    static constexpr int C = 16 * NB;
    static constexpr int NDB = DV / 16;
    static constexpr int DPW = NDB / 4;
    static constexpr int VP = DV / 64;  // 64-column planes of V
    // V in LDS: as stored (summary; bf16 output), or bf16 hi + lo of fp16 (output)
    static constexpr int NV = (!SUM && DT == DT_F16) ? 2 : 1;
    static constexpr int NTRI = NB * (NB + 1) / 2;
    static constexpr int TPW = (NTRI + 3) / 4;
    static constexpr int MAT = C * 64;  // elements of one [C][64] matrix
    // LDS carve-up (bytes)
    static constexpr int QT = SUM ? 0 : 2 * MAT * 2;  // Q~ hi, lo          (fallback: g fp32 [C][64])
    static constexpr int KN = 2 * MAT * 2;            // K^ or K~ hi, lo    (fallback: raw q, k)
    static constexpr int VN = NV * VP * MAT * 2;      // V [part][plane][C][64]
    static constexpr int PB = SUM ? 0 : NTRI * 1024;  // score tiles: [tile][hi, lo][lane][4]
    static constexpr int OT = SUM ? 0 : C * DV * 4;   // fp32 output tile [token][column]
    // epilogue: wave w finishes tokens [EPW w, EPW (w + 1)), LPT lanes per token,
    // CPL consecutive columns per lane
    static constexpr int EPW = C / 4;
    static constexpr int LPT = 64 / EPW;
    static constexpr int CPL = DV / LPT;
    static constexpr int O_QT = 0;
    static constexpr int O_KN = O_QT + QT;
    static constexpr int O_VN = O_KN + KN;
    static constexpr int O_P = O_VN + VN;
    static constexpr int O_OT = O_P + PB;
    static constexpr int O_RW = O_OT + OT;                       // float [DV]
    static constexpr int O_TOT = O_RW + (SUM ? 0 : DV * 4);      // float [NB][DK]
    static constexpr int O_TAB = O_TOT + NB * DK * 4;            // float [4 waves][3][DK]
    static constexpr int O_ROW = O_TAB + 4 * 3 * DK * 4;         // int64 [2][C]
    static constexpr int BYTES = O_ROW + 2 * C * 8;
    static_assert(NB == 2 || NB == 4, "chunks of 32 or 64 tokens");
    static_assert(SUM || C * DK * 4 <= QT, "fallback g must fit");
    static_assert(2 * C * DK * 2 <= KN, "fallback q, k must fit");
};

// State of one workgroup working through chunks.  Everything is inlined; the
// arrays live in registers.
template <int DT, int DV, int NB, bool SUM>
struct Tile {
    using K = Cfg<DT, DV, NB, SUM>;
    static constexpr int C = K::C, DPW = K::DPW, NV = K::NV, NTRI = K::NTRI, VP = K::VP,
                         MAT = K::MAT, EPW = K::EPW, LPT = K::LPT, CPL = K::CPL;
    static constexpr bool SF16 = SUM && DT == DT_F16;  // summary products in fp16

    GlaArgs a;
    uint16_t *sQ, *sK, *sV, *sP, *fQr, *fKr;
    float *sTot, *sTab, *sOt, *sRw, *fG;
    int64_t *sRow;
    int tid, w, l, lr, g;
    bool own;  // this wave stages a token sub-block (w < NB)

    // next chunk's inputs (registers)
    uint4 pq[2], pk[2], pv[DV / 32];
    float4 pg[4];
    uint4 pz[CPL / 8];  // z of this lane's token and columns (epilogue layout)
    int64_t rowE;       // grid row of this lane's epilogue token
    // chunk state
    f32x4 S[DPW][4];
    f32x4 O[DPW][NB];
    float cs[16];

    __device__ __forceinline__ void init(const GlaArgs &args, char *smem) {
        a = args;
        sQ = reinterpret_cast<uint16_t *>(smem + K::O_QT);
        sK = reinterpret_cast<uint16_t *>(smem + K::O_KN);
        sV = reinterpret_cast<uint16_t *>(smem + K::O_VN);
        sP = reinterpret_cast<uint16_t *>(smem + K::O_P);
        sTot = reinterpret_cast<float *>(smem + K::O_TOT);
        sOt = reinterpret_cast<float *>(smem + K::O_OT);
        sRw = reinterpret_cast<float *>(smem + K::O_RW);
        sRow = reinterpret_cast<int64_t *>(smem + K::O_ROW);
        fG = reinterpret_cast<float *>(smem + K::O_QT);
        fQr = sK;
        fKr = sK + MAT;
        tid = threadIdx.x;
        w = tid >> 6;
        l = tid & 63;
        lr = l & 15;
        g = l >> 4;
        own = w < NB;
        sTab = reinterpret_cast<float *>(smem + K::O_TAB) + w * 3 * DK;
        if (!SUM && tid < DV) sRw[tid] = a.rms_w[tid];  // read after later barriers
    }

    // epilogue layout: this lane's token in the chunk and first column
    __device__ __forceinline__ int ep_token() const { return EPW * w + l / LPT; }
    __device__ __forceinline__ int ep_col() const { return (l % LPT) * CPL; }

    // Offset of the 4-column piece starting at column col of token i in the fp32
    // output tile: pieces XOR-swizzled by token, so the tile's writes (16 tokens
    // at one piece) and the epilogue's row reads spread over all banks.
    __device__ __forceinline__ int ot_off(int i, int col) const {
        return i * DV + ((((col >> 2) ^ (i & 15))) << 2);
    }

    // the [C][64] matrix of V part p that holds value column d
    __device__ __forceinline__ uint16_t *vmat(int p, int d) const {
        return sV + (p * VP + (d >> 6)) * MAT;
    }

    // MFMA operand whose lane holds column cb + lr of a token-major matrix at
    // tokens rb + 4 g + s (slots s = 0..3) and rb + 16 + 4 g + (s - 4) (slots
    // 4..7), by two transposing reads.  Slot order matches the score tiles'
    // register layout, so the same slots serve both operands of a product.
    __device__ __forceinline__ s16x8 op_tr(const uint16_t *m, int rb, int cb) const {
        const int r = rb + 4 * g + (lr >> 2);
        const int c = cb + 4 * (lr & 3);
        const s16x4 x0 = ld_tr(m + swn(r, c));
        const s16x4 x1 = ld_tr(m + swn(r + 16, c));
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }

    // Row index ((b L + grid position) H + h) of every token of chunk ch of sequence bh.
    // A token past the end of the sequence (tail chunk) gets ~row of the last token:
    // its loads read that row (finite values; they reach only masked scores and the
    // state after the sequence's last chunk, which is never used) and its output is
    // not stored.
    __device__ __forceinline__ void rows_of(int64_t bh, int64_t ch, int buf) {
        if (tid < C) {
            const uint32_t L32 = static_cast<uint32_t>(a.L);
            const uint32_t t0 = static_cast<uint32_t>(ch) * C + tid;
            uint32_t t = t0 < L32 ? t0 : L32 - 1;  // past the end: the last token's row
            if (a.direction & 1) t = L32 - 1 - t;  // RL, BT: reversed sequence
            uint32_t pos = t;
            if (a.direction >= 2) {                // TB, BT: column-major raster
                const uint32_t gh = static_cast<uint32_t>(a.gh);
                const uint32_t c = t / gh;
                pos = (t - c * gh) * static_cast<uint32_t>(a.gw) + c;
            }
            const uint32_t b = static_cast<uint32_t>(bh) / static_cast<uint32_t>(a.H);
            const uint32_t h = static_cast<uint32_t>(bh) - b * static_cast<uint32_t>(a.H);
            const int64_t row = (static_cast<int64_t>(b) * a.L + pos) * a.H + h;
            sRow[buf * C + tid] = t0 < L32 ? row : ~row;
        }
    }

    __device__ __forceinline__ int64_t own_row(int buf) const {
        const int64_t row = sRow[buf * C + 16 * w + lr];
        return row < 0 ? ~row : row;
    }

    // next chunk's inputs, in two parts: log_g and v (consumed by phase 1), then
    // q and k (consumed by phase 2)
    __device__ __forceinline__ void prefetch_gv(int buf) {
        if (!own) return;
        const int64_t row = own_row(buf);
#pragma unroll
        for (int kap = 0; kap < 2; ++kap) {
            const int c0 = 32 * kap + 8 * g;
            pg[2 * kap] = *reinterpret_cast<const float4 *>(a.log_g + row * DK + c0);
            pg[2 * kap + 1] = *reinterpret_cast<const float4 *>(a.log_g + row * DK + c0 + 4);
        }
#pragma unroll
        for (int vm = 0; vm < DV / 32; ++vm) {
            const int d0 = 8 * (g + 4 * vm);
            uint4 x = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) + row * DV + d0);
            if (a.resid) {  // stack residual: v + out_prev, rounded to the I/O type
                const uint4 y = *reinterpret_cast<const uint4 *>(
                    static_cast<const uint16_t *>(a.resid) + row * DV + d0);
                x = add_io<DT>(x, y);
            }
            pv[vm] = x;
        }
    }

    __device__ __forceinline__ void prefetch_qk(int buf) {
        if (!own) return;
        const int64_t row = own_row(buf);
#pragma unroll
        for (int kap = 0; kap < 2; ++kap) {
            const int c0 = 32 * kap + 8 * g;
            if (!SUM)
                pq[kap] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) +
                                                           row * DK + c0);
            pk[kap] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) +
                                                       row * DK + c0);
        }
    }

    __device__ __forceinline__ void prefetch_main(int buf) {
        prefetch_gv(buf);
        prefetch_qk(buf);
    }

    __device__ __forceinline__ void prefetch_z(int buf) {
        if (SUM) return;
        const int64_t row = sRow[buf * C + ep_token()];
        rowE = row;
        const uint16_t *zp = static_cast<const uint16_t *>(a.z) + (row < 0 ? ~row : row) * DV + ep_col();
#pragma unroll
        for (int e = 0; e < CPL / 8; ++e) pz[e] = *reinterpret_cast<const uint4 *>(zp + 8 * e);
    }

    // the incoming state could not be formed (a bounded wait gave up): NaN, so the
    // chunk's outputs show it
    __device__ __forceinline__ void poison_state() {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) S[dd][ct] = f32x4{__builtin_nanf(""), __builtin_nanf(""),
                                                          __builtin_nanf(""), __builtin_nanf("")};
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

    // store_state with agent-coherent stores: visible to other workgroups (any XCD)
    // that read it with agent-coherent loads, with no cache write-back
    __device__ __forceinline__ void store_state_coherent(float *dst) const {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __hip_atomic_store(dst + (16 * ct + 4 * g + r) * DV + 16 * (w * DPW + dd) + lr,
                                       S[dd][ct][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // One step of a scan over chunk summaries, in the state's register layout:
    // S <- Diag(e) S + u, with u a [DK][DV] summary and e the per-channel decay.
    struct StateIn {
        f32x4 e[4];
        float u[DPW][4][4];
    };
    // (agent-coherent loads: the summaries come from other workgroups of this launch)
    __device__ __forceinline__ void state_in_load(StateIn &x, const float *u, const float *e) const {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                x.e[ct][r] = __hip_atomic_load(e + 16 * ct + 4 * g + r, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    x.u[dd][ct][r] = __hip_atomic_load(
                        u + (16 * ct + 4 * g + r) * DV + 16 * (w * DPW + dd) + lr, __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT);
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

    // The same step with the decay read from an LDS table ([predecessor][DK] fp32,
    // filled once per workgroup), so that only the summaries are loaded per
    // predecessor and twice as many of them can be in flight.
    struct UIn {
        float u[DPW][4][4];
    };
    __device__ __forceinline__ void state_u_load(UIn &x, const float *u) const {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    x.u[dd][ct][r] = __hip_atomic_load(
                        u + (16 * ct + 4 * g + r) * DV + 16 * (w * DPW + dd) + lr, __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ __forceinline__ void state_u_apply(const UIn &x, const float *etab) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const f32x4 e = *reinterpret_cast<const f32x4 *>(etab + 16 * ct + 4 * g);
#pragma unroll
            for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[dd][ct][r] = fmaf(S[dd][ct][r], e[r], x.u[dd][ct][r]);
        }
    }

    __device__ __forceinline__ void zero_out() {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) O[dd][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- phase 1: cumulative gates within the sub-block (registers, natural-log
    // units), block totals, V into LDS.  Consumes the prefetched inputs except q, k.
    __device__ __forceinline__ void phase1() {
        if (!own) return;
        const int i = 16 * w + lr;
        // natural-log units; scaled to log2 where the exponentials are taken
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            cs[4 * q4] = pg[q4].x; cs[4 * q4 + 1] = pg[q4].y;
            cs[4 * q4 + 2] = pg[q4].z; cs[4 * q4 + 3] = pg[q4].w;
        }
        row_scan(cs);
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
            const int off = swn(i, d0 & 63);
            if (NV == 1) {
                *reinterpret_cast<uint4 *>(vmat(0, d0) + off) = pv[vm];
            } else {  // fp16 values as bf16 hi + lo (exact)
                float x[8];
                unpack8<DT>(pv[vm], x);
                uint32_t hi[4], lo[4];
                split_pk<false>(x, hi, lo);
                *reinterpret_cast<uint4 *>(vmat(0, d0) + off) = u4(hi);
                *reinterpret_cast<uint4 *>(vmat(1, d0) + off) = u4(lo);
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
        r_l *= kLog2e;
        tot_l *= kLog2e;
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
            const int off = swn(i, c0);
            float rI[8], gC[8];
#pragma unroll
            for (int h4 = 0; h4 < 2; ++h4) {
                const float4 x = *reinterpret_cast<const float4 *>(sTab + c0 + 4 * h4);
                const float4 y = *reinterpret_cast<const float4 *>(sTab + DK + c0 + 4 * h4);
                rI[4 * h4] = x.x; rI[4 * h4 + 1] = x.y; rI[4 * h4 + 2] = x.z; rI[4 * h4 + 3] = x.w;
                gC[4 * h4] = y.x; gC[4 * h4 + 1] = y.y; gC[4 * h4 + 2] = y.z; gC[4 * h4 + 3] = y.w;
            }
            if (SUM) {
                float kt[8];
                unpack8<DT>(pk[kap], kt);
#pragma unroll
                for (int s = 0; s < 8; ++s)  // k 2^(G - a)
                    kt[s] *= fexp2(fmaf(-cs[8 * kap + s], kLog2e, gC[s] - rI[s]));
                uint32_t hi[4], lo[4];
                split_pk<SF16>(kt, hi, lo);
                *reinterpret_cast<uint4 *>(sK + off) = u4(hi);
                *reinterpret_cast<uint4 *>(sK + MAT + off) = u4(lo);
            } else if (!slow) {
                float qt[8], kh[8];
                unpack8<DT>(pq[kap], qt);
                unpack8<DT>(pk[kap], kh);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float aa = fmaf(cs[8 * kap + s], kLog2e, rI[s]);
                    qt[s] *= fexp2(aa);   // q 2^a
                    kh[s] *= fexp2(-aa);  // k 2^-a
                }
                uint32_t qh[4], ql[4], khh[4], khl[4];
                split_pk<false>(qt, qh, ql);
                split_pk<false>(kh, khh, khl);
                *reinterpret_cast<uint4 *>(sQ + off) = u4(qh);
                *reinterpret_cast<uint4 *>(sQ + MAT + off) = u4(ql);
                *reinterpret_cast<uint4 *>(sK + off) = u4(khh);
                *reinterpret_cast<uint4 *>(sK + MAT + off) = u4(khl);
            } else {
                // token-serial operands: q and k as stored, g = 2^(a_i - a_{i-1}) in fp32,
                // all [token][channel] without swizzle
                *reinterpret_cast<uint4 *>(fQr + i * DK + c0) = pq[kap];
                *reinterpret_cast<uint4 *>(fKr + i * DK + c0) = pk[kap];
                float gg[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float up = __shfl_up(cs[8 * kap + s], 1, 16);
                    const float prev = (lr == 0) ? 0.f : up;
                    gg[s] = fexp2((cs[8 * kap + s] - prev) * kLog2e);
                }
                *reinterpret_cast<float4 *>(fG + i * DK + c0) = make_float4(gg[0], gg[1], gg[2], gg[3]);
                *reinterpret_cast<float4 *>(fG + i * DK + c0 + 4) = make_float4(gg[4], gg[5], gg[6], gg[7]);
            }
        }
        return slow;
    }

    // ---- inter-chunk readout O^T[d][i] = S^T (Q~)^T (the state before the chunk);
    // ACC: added to what O holds (the intra-chunk products formed first)
    template <bool ACC = false>
    __device__ __forceinline__ void inter() {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd) {
            s16x8 ah[2], al[2];
#pragma unroll
            for (int kap = 0; kap < 2; ++kap) {
                float x[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) x[s] = S[dd][2 * kap + (s >> 2)][s & 3];
                uint32_t hi[4], lo[4];
                split_pk<false>(x, hi, lo);
                ah[kap] = __builtin_bit_cast(s16x8, u4(hi));
                al[kap] = __builtin_bit_cast(s16x8, u4(lo));
            }
            if (!ACC) {
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) O[dd][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int kap = 0; kap < 2; ++kap) {
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) {
                    const int i = 16 * tb + lr;
                    const int c0 = 32 * kap + 4 * g;
                    const s16x4 h0 = *reinterpret_cast<const s16x4 *>(sQ + swn(i, c0));
                    const s16x4 h1 = *reinterpret_cast<const s16x4 *>(sQ + swn(i, c0 + 16));
                    const s16x4 l0 = *reinterpret_cast<const s16x4 *>(sQ + MAT + swn(i, c0));
                    const s16x4 l1 = *reinterpret_cast<const s16x4 *>(sQ + MAT + swn(i, c0 + 16));
                    const s16x8 bh = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
                    const s16x8 bl = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
                    O[dd][tb] = mma<false>(ah[kap], bh, O[dd][tb]);
                    O[dd][tb] = mma<false>(ah[kap], bl, O[dd][tb]);
                    O[dd][tb] = mma<false>(al[kap], bh, O[dd][tb]);
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
            const int I = (t >= 1) + (t >= 3) + (t >= 6);  // tile t = I (I + 1) / 2 + J
            const int J = t - I * (I + 1) / 2;
            s16x8 ak[2][2], bq[2][2];
#pragma unroll
            for (int kap = 0; kap < 2; ++kap) {
                const int c0 = 32 * kap + 8 * g;
#pragma unroll
                for (int hl = 0; hl < 2; ++hl) {
                    ak[kap][hl] = *reinterpret_cast<const s16x8 *>(sK + hl * MAT + swn(16 * J + lr, c0));
                    bq[kap][hl] = *reinterpret_cast<const s16x8 *>(sQ + hl * MAT + swn(16 * I + lr, c0));
                }
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kap = 0; kap < 2; ++kap) {
                acc = mma<false>(ak[kap][0], bq[kap][0], acc);
                acc = mma<false>(ak[kap][0], bq[kap][1], acc);
                acc = mma<false>(ak[kap][1], bq[kap][0], acc);
            }
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = (J == I && 4 * g + r > lr) ? 0.f : acc[r];  // j <= i
            uint32_t hi[2], lo[2];
            split_pk<false>(x, hi, lo);
            *reinterpret_cast<uint2 *>(sP + (2 * t) * 256 + 4 * l) = make_uint2(hi[0], hi[1]);
            *reinterpret_cast<uint2 *>(sP + (2 * t + 1) * 256 + 4 * l) = make_uint2(lo[0], lo[1]);
        }
    }

    // ---- state update.  Output kernel: S = Diag(2^G) (S + K^^T V).  Summary
    // kernel: S = Diag(2^G) S + K~^T V, with K~ in the I/O type's format.
    __device__ __forceinline__ void s_update() {
        if (SUM) decay();
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd) {
            const int dt = w * DPW + dd;
            const int cb = 16 * (dt & 3);
#pragma unroll
            for (int kt = 0; kt < C / 32; ++kt) {
                s16x8 bv[NV];
#pragma unroll
                for (int p = 0; p < NV; ++p) bv[p] = op_tr(vmat(p, 16 * dt), 32 * kt, cb);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const s16x8 akh = op_tr(sK, 32 * kt, 16 * ct);
                    const s16x8 akl = op_tr(sK + MAT, 32 * kt, 16 * ct);
                    S[dd][ct] = mma<SF16>(akh, bv[0], S[dd][ct]);
                    S[dd][ct] = mma<SF16>(akl, bv[0], S[dd][ct]);
                    if (NV == 2) S[dd][ct] = mma<false>(akh, bv[NV - 1], S[dd][ct]);
                }
            }
        }
        if (!SUM) decay();
    }

    __device__ __forceinline__ void decay() {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const float4 e4 = *reinterpret_cast<const float4 *>(sTab + 2 * DK + 16 * ct + 4 * g);
#pragma unroll
            for (int dd = 0; dd < DPW; ++dd) {
                S[dd][ct][0] *= e4.x; S[dd][ct][1] *= e4.y; S[dd][ct][2] *= e4.z; S[dd][ct][3] *= e4.w;
            }
        }
    }

    // ---- intra-chunk readout O^T[d][i] += V^T P^T (score tiles from sP)
    __device__ __forceinline__ void intra() {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd) {
            const int dt = w * DPW + dd;
            const int cb = 16 * (dt & 3);
#pragma unroll
            for (int kap = 0; kap < NB / 2; ++kap) {
                s16x8 av[NV];
#pragma unroll
                for (int p = 0; p < NV; ++p) av[p] = op_tr(vmat(p, 16 * dt), 32 * kap, cb);
#pragma unroll
                for (int I = 2 * kap; I < NB; ++I) {
                    const int t0 = I * (I + 1) / 2 + 2 * kap;
                    const s16x4 zero = {0, 0, 0, 0};
                    const bool two = 2 * kap + 1 <= I;
                    const s16x4 h0 = *reinterpret_cast<const s16x4 *>(sP + (2 * t0) * 256 + 4 * l);
                    const s16x4 l0 = *reinterpret_cast<const s16x4 *>(sP + (2 * t0 + 1) * 256 + 4 * l);
                    const s16x4 h1 = two ? *reinterpret_cast<const s16x4 *>(sP + (2 * t0 + 2) * 256 + 4 * l) : zero;
                    const s16x4 l1 = two ? *reinterpret_cast<const s16x4 *>(sP + (2 * t0 + 3) * 256 + 4 * l) : zero;
                    const s16x8 bh = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
                    const s16x8 bl = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
                    O[dd][I] = mma<false>(av[0], bh, O[dd][I]);
                    O[dd][I] = mma<false>(av[0], bl, O[dd][I]);
                    if (NV == 2) O[dd][I] = mma<false>(av[NV - 1], bh, O[dd][I]);
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
                const int off = swn(t, d & 63);
                float vd;
                if (NV == 2)
                    vd = __uint_as_float(static_cast<uint32_t>(vmat(0, d)[off]) << 16) +
                         __uint_as_float(static_cast<uint32_t>(vmat(1, d)[off]) << 16);
                else
                    vd = h2f<DT>(vmat(0, d)[off]);
                float part = 0.f;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const int c = 16 * ct + 4 * g;
                    const float4 gq = *reinterpret_cast<const float4 *>(fG + t * DK + c);
                    const uint2 kq = *reinterpret_cast<const uint2 *>(fKr + t * DK + c);
                    const uint2 qq = *reinterpret_cast<const uint2 *>(fQr + t * DK + c);
                    const float gg[4] = {gq.x, gq.y, gq.z, gq.w};
                    const float kk[4] = {h2f<DT>(kq.x & 0xffffu), h2f<DT>(kq.x >> 16),
                                         h2f<DT>(kq.y & 0xffffu), h2f<DT>(kq.y >> 16)};
                    const float q4[4] = {h2f<DT>(qq.x & 0xffffu), h2f<DT>(qq.x >> 16),
                                         h2f<DT>(qq.y & 0xffffu), h2f<DT>(qq.y >> 16)};
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

    // ---- the chunk's output tile O (fp32) into LDS, [token][column]
    __device__ __forceinline__ void out_stage() {
#pragma unroll
        for (int dd = 0; dd < DPW; ++dd)
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                const int i = 16 * tb + lr;
                const int col = 16 * (w * DPW + dd) + 4 * g;
                *reinterpret_cast<f32x4 *>(sOt + ot_off(i, col)) = O[dd][tb];
            }
    }

    // ---- epilogue (after out_stage everywhere), one token per LPT lanes:
    // y = o / sqrt(mean_j o_j^2 + eps) * rms_w * z * sigmoid(z), whole rows stored
    // at the token's grid position
    __device__ __forceinline__ void epilogue() {
        const int i = ep_token(), c0 = ep_col();
        float o[CPL];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < CPL / 4; ++e) {
            const f32x4 x = *reinterpret_cast<const f32x4 *>(sOt + ot_off(i, c0 + 4 * e));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                o[4 * e + r] = x[r];
                ss += x[r] * x[r];
            }
        }
#pragma unroll
        for (int m = 1; m < LPT; m <<= 1) ss += __shfl_xor(ss, m);
        const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / DV) + GTR_RMS_EPS);
        uint32_t yb[CPL / 2];
#pragma unroll
        for (int e = 0; e < CPL / 4; ++e) {
            const float4 wr = *reinterpret_cast<const float4 *>(sRw + c0 + 4 * e);
            const float rwv[4] = {wr.x, wr.y, wr.z, wr.w};
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                uint32_t h[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int k = 4 * e + r + u;
                    const float zz = h2f<DT>(half16(pz[k / 8], k % 8));
                    const float silu = zz * frcp(1.0f + fexp2(-zz * kLog2e));
                    h[u] = f2h<DT>(o[k] * inv * rwv[r + u] * silu);
                }
                yb[(4 * e + r) / 2] = h[0] | (h[1] << 16);
            }
        }
        if (rowE >= 0) {
            uint16_t *op = static_cast<uint16_t *>(a.out) + rowE * DV + c0;
#pragma unroll
            for (int e = 0; e < CPL / 8; ++e)
                *reinterpret_cast<uint4 *>(op + 8 * e) =
                    make_uint4(yb[4 * e], yb[4 * e + 1], yb[4 * e + 2], yb[4 * e + 3]);
        }
    }
};

}  // namespace mf
}  // namespace gtr
