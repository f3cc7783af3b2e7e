// k_sswiglu.hip -- the fused middle of the Spatial SwiGLU feed-forward block.
//
// GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"), Method §2: in the
// channel expansion of the SwiGLU block the value branch is reshaped to the
// 2-D token grid and mixed by a depthwise convolution before the gated
// product.  From the expanded projection u = [gate | value] ([B, gh, gw, 2F],
// channels last) this kernel writes
//     m[b, y, x, f] = SiLU(gate[b, y, x, f]) *
//                     (bias[f] + sum_{i,j < K} w[f, i, j] value[b, y + i - K/2, x + j - K/2, f])
// with zero padding (cross-correlation), fp32 arithmetic, m rounded to the I/O
// type.  It moves 3F elements per token and does K^2 FMAs per element: HBM
// bound, so it is built for coalesced, cache-friendly reads rather than for
// the matrix units.
//
// Work split.  A thread owns CPL consecutive channels (one 16-, 8- or 4-byte
// piece: the wider the kernel the narrower the piece, so that the K^2 CPL taps
// stay in registers) of RY grid rows times a strip of at most 64 consecutive
// columns; a workgroup's threads take consecutive channel pieces, so every
// load of a wave is one contiguous run of memory.  Along the strip the thread
// walks the input columns once: each column's RY + K - 1 rows are loaded (two
// columns ahead of their use), converted and added into the K output columns
// that still need them (input-stationary), and an output is finished when its
// last input column has arrived.  Rows shared by neighbouring row blocks are
// re-read from L2: the strips are numbered row by row, and workgroup n, which
// the dispatcher places on XCD n mod 8, is given strip number
// (n mod 8) * ceil(N / 8) + n / 8 (adjusted for a remainder), so that each XCD
// works through a contiguous band of rows and its own L2 holds the rows the
// band shares.
#include "gtr_internal.hpp"

namespace gtr {
namespace {

constexpr int SW_THREADS = 256;

template <int BYTES> struct Piece;
template <> struct Piece<16> { using T = uint4; };
template <> struct Piece<8> { using T = uint2; };
template <> struct Piece<4> { using T = uint32_t; };

// the CPL values of a piece as floats
template <int DT, int CPL, typename P>
__device__ __forceinline__ void unpack(const P &p, float (&x)[CPL]) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(&p);
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) x[c] = __uint_as_float(w[c]);
    } else {
#pragma unroll
        for (int c = 0; c < CPL; c += 2) {
            const uint32_t u = w[c / 2];
            if constexpr (DT == DT_F16) {
                x[c] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u & 0xffffu)));
                x[c + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u >> 16)));
            } else {
                x[c] = __uint_as_float(u << 16);
                x[c + 1] = __uint_as_float(u & 0xffff0000u);
            }
        }
    }
}

template <int DT, int CPL, typename P>
__device__ __forceinline__ P pack(const float (&y)[CPL]) {
    P p;
    uint32_t *w = reinterpret_cast<uint32_t *>(&p);
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) w[c] = __float_as_uint(y[c]);
    } else {
#pragma unroll
        for (int c = 0; c < CPL; c += 2) {
            // a pair per packed round-to-nearest-even conversion
            typedef float f2_t __attribute__((ext_vector_type(2)));
            const f2_t v = {y[c], y[c + 1]};
            if constexpr (DT == DT_F16) {
                typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
                w[c / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2_t));
            } else {
                typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
                w[c / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2_t));
            }
        }
    }
    return p;
}

// Per kernel size: bytes of a thread's channel piece, output rows per thread.
template <int K> struct SwCfg;
template <> struct SwCfg<1> { static constexpr int PB = 16, RY = 1; };
template <> struct SwCfg<3> { static constexpr int PB = 8, RY = 2; };
template <> struct SwCfg<5> { static constexpr int PB = 8, RY = 1; };
template <> struct SwCfg<7> { static constexpr int PB = 4, RY = 1; };
constexpr int SW_D = 2;  // input columns loaded ahead of the one being used

template <int DT, int K, int TX>
__global__ __launch_bounds__(SW_THREADS) void k_sswiglu(const void *__restrict__ u,
                                                        const float *__restrict__ wc,
                                                        const float *__restrict__ bc,
                                                        void *__restrict__ m, int gh, int gw,
                                                        int F, int strips_x, int strips_y,
                                                        uint32_t n_items) {
    using E = typename Elem<DT>::T;
    constexpr int PB = SwCfg<K>::PB, RY = SwCfg<K>::RY, D = SW_D;
    constexpr int CPL = PB / static_cast<int>(sizeof(E));  // channels per thread
    constexpr int R = K / 2;
    constexpr int NR = RY + 2 * R;  // input rows per column
    constexpr int NC = TX + 2 * R;  // input columns x0 - R .. x0 + TX - 1 + R
    using P = typename Piece<PB>::T;

    const int groups = F / CPL;
    const int cg = blockIdx.y * SW_THREADS + threadIdx.x;
    if (cg >= groups) return;  // no barriers below
    const int c0 = cg * CPL;

    // XCD-aware strip number (see the header)
    const uint32_t n = blockIdx.x, nb = gridDim.x;
    const uint32_t per = nb / 8, rem = nb % 8, xcd = n % 8, j = n / 8;
    const uint32_t item = (xcd < rem) ? xcd * (per + 1) + j : rem * (per + 1) + (xcd - rem) * per + j;
    if (item >= n_items) return;
    const uint32_t xs = item % static_cast<uint32_t>(strips_x);
    const uint32_t rowi = item / static_cast<uint32_t>(strips_x);
    const int y0 = static_cast<int>(rowi % static_cast<uint32_t>(strips_y)) * RY;
    const int64_t b = rowi / static_cast<uint32_t>(strips_y);
    const int x0 = static_cast<int>(xs) * TX;

    const E *ue = static_cast<const E *>(u);
    E *me = static_cast<E *>(m);
    const int64_t rowbase = b * gh * gw;  // token index of (b, 0, 0)

    // Column t's value pieces (rows y0 - R .. y0 + RY - 1 + R) and the gate pieces of
    // output column x0 + t - 2R, loaded D columns ahead; positions off the grid read
    // a clamped in-grid position and are zeroed (values) or not stored (outputs).
    P raw[D][NR], graw[D][RY];
    auto issue = [&](int t, P (&dst)[NR], P (&gdst)[RY]) {
        const int cx = x0 - R + t;
        const int cxc = cx < 0 ? 0 : (cx >= gw ? gw - 1 : cx);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int yy = y0 + i - R;
            const int yc = yy < 0 ? 0 : (yy >= gh ? gh - 1 : yy);
            dst[i] = *reinterpret_cast<const P *>(ue + (rowbase + static_cast<int64_t>(yc) * gw + cxc) * 2 * F + F + c0);
        }
        const int xo = cx - R;
        const int xoc = xo < 0 ? 0 : (xo >= gw ? gw - 1 : xo);
#pragma unroll
        for (int ry = 0; ry < RY; ++ry) {
            const int yo = y0 + ry < gh ? y0 + ry : gh - 1;
            gdst[ry] = *reinterpret_cast<const P *>(ue + (rowbase + static_cast<int64_t>(yo) * gw + xoc) * 2 * F + c0);
        }
    };
#pragma unroll
    for (int s = 0; s < D; ++s)
        if (s < NC) issue(s, raw[s], graw[s]);

    float w[K][K][CPL], bias[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        bias[c] = bc[c0 + c];
#pragma unroll
        for (int i = 0; i < K; ++i)
#pragma unroll
            for (int jj = 0; jj < K; ++jj) w[i][jj][c] = wc[(static_cast<int64_t>(c0 + c) * K + i) * K + jj];
    }
    // acc[o][ry]: output (x0 + t - 2R + o, y0 + ry) at column t; input column t feeds
    // it through kernel column K - 1 - o, and acc[0] is complete after column t
    float acc[K][RY][CPL];
#pragma unroll
    for (int o = 0; o < K; ++o)
#pragma unroll
        for (int ry = 0; ry < RY; ++ry)
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[o][ry][c] = bias[c];

    // (the strip is fully unrolled: every load is issued unconditionally, so the
    // wait counts never depend on a branch)
#pragma unroll
    for (int t = 0; t < NC; ++t) {
        const int s = t % D;
        const int cx = x0 - R + t;
        const bool col_ok = cx >= 0 && cx < gw;
        float v[NR][CPL];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int yy = y0 + i - R;
            const bool ok = col_ok && yy >= 0 && yy < gh;
            unpack<DT, CPL>(raw[s][i], v[i]);
#pragma unroll
            for (int c = 0; c < CPL; ++c) v[i][c] = ok ? v[i][c] : 0.f;
        }
        P gcur[RY];
#pragma unroll
        for (int ry = 0; ry < RY; ++ry) gcur[ry] = graw[s][ry];
        if (t + D < NC) issue(t + D, raw[s], graw[s]);
#pragma unroll
        for (int o = 0; o < K; ++o)
#pragma unroll
            for (int ry = 0; ry < RY; ++ry)
#pragma unroll
                for (int i = 0; i < K; ++i)
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
                        acc[o][ry][c] = fmaf(w[i][K - 1 - o][c], v[ry + i][c], acc[o][ry][c]);
        const int xo = x0 + t - 2 * R;
        if (t >= 2 * R && xo < gw) {
#pragma unroll
            for (int ry = 0; ry < RY; ++ry) {
                if (y0 + ry < gh) {
                    const int64_t tok = rowbase + static_cast<int64_t>(y0 + ry) * gw + xo;
                    float gv[CPL], out[CPL];
                    unpack<DT, CPL>(gcur[ry], gv);
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        const float silu = gv[c] * __builtin_amdgcn_rcpf(
                            1.f + __builtin_amdgcn_exp2f(-gv[c] * 1.44269504088896340736f));
                        out[c] = silu * acc[0][ry][c];
                    }
                    *reinterpret_cast<P *>(me + tok * F + c0) = pack<DT, CPL, P>(out);
                }
            }
        }
#pragma unroll
        for (int o = 0; o + 1 < K; ++o)
#pragma unroll
            for (int ry = 0; ry < RY; ++ry)
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[o][ry][c] = acc[o + 1][ry][c];
#pragma unroll
        for (int ry = 0; ry < RY; ++ry)
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[K - 1][ry][c] = bias[c];
    }
}

template <int DT, int K, int TX>
hipError_t launch_tx(const void *u, const float *w, const float *b, void *m, int B, int gh, int gw,
                     int F, int strips_y, int gy, hipStream_t s) {
    const int strips_x = (gw + TX - 1) / TX;
    const int64_t items = static_cast<int64_t>(B) * strips_y * strips_x;
    if (items > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_sswiglu<DT, K, TX>), dim3(static_cast<unsigned>(items), gy), dim3(SW_THREADS),
                       0, s, u, w, b, m, gh, gw, F, strips_x, strips_y, static_cast<uint32_t>(items));
    return hipGetLastError();
}

// Strips of 64 columns where the grid is wide and there are enough of them for
// the GPU (>= 512 workgroups, two per CU); 8-column strips otherwise (small grids, where
// parallelism matters more than the re-read of 2R columns per strip).
template <int DT, int K>
hipError_t launch_k(const void *u, const float *w, const float *b, void *m, int B, int gh, int gw,
                    int F, hipStream_t s) {
    constexpr int CPL = SwCfg<K>::PB / static_cast<int>(sizeof(typename Elem<DT>::T));
    const int strips_y = (gh + SwCfg<K>::RY - 1) / SwCfg<K>::RY;
    const int gy = (F / CPL + SW_THREADS - 1) / SW_THREADS;
    const int64_t wide = static_cast<int64_t>(B) * strips_y * ((gw + 63) / 64) * gy;
    if (gw >= 48 && wide >= 512) return launch_tx<DT, K, 64>(u, w, b, m, B, gh, gw, F, strips_y, gy, s);
    return launch_tx<DT, K, 8>(u, w, b, m, B, gh, gw, F, strips_y, gy, s);
}

template <int DT>
hipError_t launch_dt(const void *u, const float *w, const float *b, void *m, int B, int gh, int gw,
                     int F, int k, hipStream_t s) {
    switch (k) {
    case 1: return launch_k<DT, 1>(u, w, b, m, B, gh, gw, F, s);
    case 3: return launch_k<DT, 3>(u, w, b, m, B, gh, gw, F, s);
    case 5: return launch_k<DT, 5>(u, w, b, m, B, gh, gw, F, s);
    case 7: return launch_k<DT, 7>(u, w, b, m, B, gh, gw, F, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t sswiglu_launch(const void *u, const float *w, const float *b, void *m, int B, int gh,
                          int gw, int F, int k, int dtype, hipStream_t s) {
    switch (dtype) {
    case DT_F32: return launch_dt<DT_F32>(u, w, b, m, B, gh, gw, F, k, s);
    case DT_F16: return launch_dt<DT_F16>(u, w, b, m, B, gh, gw, F, k, s);
    case DT_BF16: return launch_dt<DT_BF16>(u, w, b, m, B, gh, gw, F, k, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gtr
