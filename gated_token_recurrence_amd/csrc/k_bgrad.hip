// k_bgrad.hip -- matrix-core kernels of the backward pass (16-bit I/O, dk = dv = 64,
// chunk <= 64): the epilogue backward with the reverse chunk summaries (k_bdo)
// and the gradients of q, k, v and the gates per chunk (k_bgrad).
//
// GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"): Method §1 gives the
// recurrence S_t = Diag(g_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t; Method §4 its
// chunkwise evaluation.  Differentiating the chunkwise form of a chunk with
// incoming state S (from the earlier chunks), incoming gradient state E (from the
// later chunks, already carrying the next chunk's first gate), a the in-chunk
// inclusive cumulative log2-gate and G = a at the chunk's last token:
//   Q~ = q 2^a,  K^ = k 2^-a,  K~ = k 2^(G - a),  M = [j <= i]
//   D = (dO V^T) . M            (gradient of the scores, no gate on the v . do sum)
//   P = (Q~ K^^T) . M           (the forward scores)
//   dQ = 2^a . (dO S^T + D K^)
//   dK = 2^-a . (D^T Q~) + 2^(G - a) . (V E^T)
//   dV = P^T dO + K~ E
// The gate gradient's per-token term q . dq - k . dk is summed in reverse over
// the chunk and offset by the sum over all later tokens of the sequence, which
// equals sum_d E[c][d] S_out[c][d] (the gate gradient at the next chunk's first
// token, g S_prev . dS there: E carries that token's gate, S_out = 2^G . (S + K^^T V)
// is the state after this chunk's last token), so dlog_g is complete here.
// 2^-a grows with the chunk's decay span: a chunk whose span exceeds kSpanMax
// (log2 units) in any channel is only flagged here, and the fp32 token-serial
// kernels produce its gradients.
//
// Persistent workgroups of eight waves, one chunk at a time; the next chunk's
// inputs are requested while the current chunk is computed.  Every product is a
// 64 x 64 x 64 product on v_mfma_f32_16x16x32_bf16 with each operand split into
// bf16 hi + lo (three products per pair), wave w computing output rows
// [16 (w % 4), + 16) and columns [32 (w / 4), + 32) (two waves per SIMD, so one
// wave's waits overlap the other's work).  Operands are split once, when written
// to LDS, into hi and lo planes of 64 x 64 16-bit elements (rows XOR-swizzled
// by 16-byte piece); a
// product reads rows of a plane (16- or 8-byte pieces) or columns of it (the
// transposing ds_read_b64_tr_b16).  D and P are stored transposed, so that a
// lane's four results per tile are one 8-byte piece.  E enters pre-scaled by
// 2^G (E' = 2^G . E), which merges dK's two terms under one factor 2^-a and
// makes dV = P^T dO + K^ E'.  dq, dk and dv pass through an fp32 staging
// matrix on their way out (16-byte global stores), where the gate gradient's
// per-token term q dq - k dk is formed from the exact q and k.
#include "mfma_common.hpp"

namespace gtr {
namespace {

using namespace mf;

constexpr int BC = 64;         // chunk tokens (rows of every matrix) and channels
constexpr int LS = BC + 4;     // fp32 LDS row stride
constexpr int MAT = BC * BC;   // elements of one 16-bit plane

struct BgArgs {
    GlaArgs a;
    const float *dO;    // [rows][64]
    const float *Sseg;  // forward incoming state of each segment of pl [seg][64][64]
    const float *Sx;    // forward incoming state per chunk, for the flagged chunks' successors
    const float *Er;    // reverse incoming gradient state per chunk, reversed chunk order
    void *dq, *dk, *dv;
    float *dlog_g;      // complete gate gradient
    const int *flags;   // per chunk: 1 = left to the token-serial kernels
    int n_chunks;
    MfmaPlan pl;        // segments of the incoming states Sseg
    int64_t R;          // workgroup b takes chunks [b R, b R + R) in order (R: a multiple of pl.Q)
};

__device__ __forceinline__ void st4(float *dst, float4 x) { *reinterpret_cast<float4 *>(dst) = x; }
__device__ __forceinline__ float4 ld4(const float *src) { return *reinterpret_cast<const float4 *>(src); }

// hi and lo planes (X, X + MAT) of N consecutive elements of row `row` from `col`
template <int N>
__device__ __forceinline__ void put(uint16_t *X, int row, int col, const float (&x)[N]) {
    uint32_t h[N / 2], l[N / 2];
    split_pk<false>(x, h, l);
    const int off = swn(row, col);
    if constexpr (N == 8) {
        *reinterpret_cast<uint4 *>(X + off) = u4(h);
        *reinterpret_cast<uint4 *>(X + MAT + off) = u4(l);
    } else {
        static_assert(N == 4, "4 or 8 elements");
        *reinterpret_cast<uint2 *>(X + off) = make_uint2(h[0], h[1]);
        *reinterpret_cast<uint2 *>(X + MAT + off) = make_uint2(l[0], l[1]);
    }
}

// Operand fetch of lane (lr, g), k block kap.  NAT: row m, k slots
// 32 kap + 8 g + s.  PERM: row m, k slots 32 kap + 16 (s / 4) + 4 g + s % 4.
// TRN: column m (= a multiple of 16 + lr), the same k slots as PERM, which are
// what the transposing read delivers (lane lr's slot j of one read comes from
// the 8-byte piece of lane 4 j + lr / 4).  Both operands of a product use NAT,
// or both use PERM / TRN.
enum { NAT = 0, PERM = 1, TRN = 2 };
template <int MODE>
__device__ __forceinline__ void fetch(const uint16_t *X, int m, int lr, int g, int kap, s16x8 &hi,
                                      s16x8 &lo) {
    if constexpr (MODE == NAT) {
        const int off = swn(m, 32 * kap + 8 * g);
        hi = *reinterpret_cast<const s16x8 *>(X + off);
        lo = *reinterpret_cast<const s16x8 *>(X + MAT + off);
    } else if constexpr (MODE == PERM) {
        const int o0 = swn(m, 32 * kap + 4 * g), o1 = swn(m, 32 * kap + 16 + 4 * g);
        const s16x4 h0 = *reinterpret_cast<const s16x4 *>(X + o0);
        const s16x4 h1 = *reinterpret_cast<const s16x4 *>(X + o1);
        const s16x4 l0 = *reinterpret_cast<const s16x4 *>(X + MAT + o0);
        const s16x4 l1 = *reinterpret_cast<const s16x4 *>(X + MAT + o1);
        hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        const int r = 32 * kap + 4 * g + (lr >> 2), c = (m & ~15) + 4 * (lr & 3);
        const int o0 = swn(r, c), o1 = swn(r + 16, c);
        const s16x4 h0 = ld_tr(X + o0), h1 = ld_tr(X + o1);
        const s16x4 l0 = ld_tr(X + MAT + o0), l1 = ld_tr(X + MAT + o1);
        hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// Position of chunk c (of B H N, sequence-major) and its token count
struct ChunkAt {
    int n, bh, b, h, nt;
    int64_t t0;
    size_t cidx, ridx;
    __device__ ChunkAt(const GlaArgs &a, int n_chunks, int64_t c) {
        n = static_cast<int>(c % n_chunks);
        bh = static_cast<int>(c / n_chunks);
        b = bh / a.H;
        h = bh % a.H;
        t0 = static_cast<int64_t>(n) * a.chunk;
        nt = static_cast<int>((t0 + a.chunk < a.L) ? a.chunk : a.L - t0);
        cidx = static_cast<size_t>(c);
        ridx = static_cast<size_t>(bh) * n_chunks + (n_chunks - 1 - n);
    }
    // global row of token t; rows past the chunk's end repeat its last row
    __device__ int64_t row(const GlaArgs &a, int t) const {
        return scan_row(a, b, h, t0 + (t < nt ? t : nt - 1));
    }
};

template <int DT>
__device__ __forceinline__ uint4 pack8(const float *x) {
    uint32_t u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = pk2<DT == DT_F16>(x[2 * e], x[2 * e + 1]);
    return u4(u);
}

// ---- The epilogue backward and the reverse chunk summary (they precede the
// gradients): per chunk, with S the forward incoming state,
//   O = Q~ S + P V                      (the forward outputs before RMSNorm)
//   r = (mean(o^2) + eps)^-1/2, n = r o, dn = dy w silu(z)
//   dO = r (dn - n mean(dn n)),  dz = dy n w silu'(z),  drms_w partial = sum dy n silu(z)
//   Ur = Q~^T dO = sum_i 2^(a_i) q_i dO_i^T   (the chunk's gradient state from zero,
//                                              times its first gate), with G (log2)
// Same workgroup layout as the gradient kernel; the epilogue runs in the load
// layout (a thread holds 8 columns of a row; the 8 lanes of a row reduce together)
// through an fp32 staging matrix.
struct BdArgs {
    GlaArgs a;
    const void *dy;     // gradient of out, I/O type
    const float *Sseg;  // forward incoming state of each segment of pl [seg][64][64]
    float *Sx;          // out: forward incoming state of each flagged chunk and of its successor
    float *dO;          // [rows][64]
    void *dz;
    float *wr;          // [workgroup][64] drms_w sums over the range's unflagged chunks
    float *Ur, *Gr;     // reverse summaries and chunk gates (log2), reversed chunk order
    int *flags;         // per chunk: 1 = left to the token-serial kernels
    int n_chunks;
    MfmaPlan pl;        // segments of the incoming states Sseg
    int64_t R;          // workgroup b takes chunks [b R, b R + R) in order (R: a multiple of pl.Q)
};

// Eight waves (two per SIMD, so that one wave's LDS, matrix-unit and memory
// waits overlap the other's work): wave w computes rows [16 (w % 4), + 16) and
// columns [32 (w / 4), + 32) of every product.
constexpr int NW = 8;
constexpr int NTB = 64 * NW;

// acc[tt] += A[16 rs + .., :] B[:, 16 (2 ch + tt) + ..], tt = 0, 1.  Row modes: A
// stored [m][k], B stored [n][k]; TRN: A stored [k][m], B stored [k][n].  Lane l:
// output rows 16 rs + 4 (l / 16) + r, column 16 (2 ch + tt) + l % 16 (acc[tt][r]).
template <int MA, int MB>
__device__ __forceinline__ void gemm2(f32x4 (&acc)[2], const uint16_t *A, const uint16_t *B, int rs,
                                      int ch, int lr, int g) {
    static_assert((MA == NAT) == (MB == NAT), "both operands must use one k slot order");
#pragma unroll
    for (int kap = 0; kap < 2; ++kap) {
        s16x8 ah, al;
        fetch<MA>(A, 16 * rs + lr, lr, g, kap, ah, al);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            s16x8 bh, bl;
            fetch<MB>(B, 16 * (2 * ch + tt) + lr, lr, g, kap, bh, bl);
            acc[tt] = mma<false>(ah, bh, acc[tt]);
            acc[tt] = mma<false>(ah, bl, acc[tt]);
            acc[tt] = mma<false>(al, bh, acc[tt]);
        }
    }
}

__device__ __forceinline__ void zero2(f32x4 (&acc)[2]) {
    acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Cumulative gates of a chunk from its log_g pieces (fp32 pieces i = tid + 512 u,
// u < 2): A2[t][c] = 2^a (a: in-chunk inclusive cumulative log2-gate, rows past
// nt add nothing; LOG: a itself, and Gl[c] = G), G2[c] = 2^G; returns G of
// channel tid % 64 (log2).  Wave w
// scans tokens [8 w, 8 w + 8).  Ends before a barrier the caller places.
template <bool LOG = false>
__device__ __forceinline__ float chunk_gates8(const float4 (&xg)[2], float (*A2)[LS], float *G2,
                                              float (*tot8)[BC], int nt, int tid,
                                              float *Gl = nullptr) {
    const int w = tid >> 6, l = tid & 63;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + NTB * u, t = i >> 4, c = (i & 15) * 4;
        const bool ok = t < nt;
        const float4 x = xg[u];
        st4(&A2[t][c], make_float4(ok ? x.x * kLog2e : 0.f, ok ? x.y * kLog2e : 0.f,
                                   ok ? x.z * kLog2e : 0.f, ok ? x.w * kLog2e : 0.f));
    }
    __syncthreads();
    float cum[8];
    {
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            acc += A2[8 * w + s][l];
            cum[s] = acc;
        }
        tot8[w][l] = acc;
    }
    __syncthreads();
    float off = 0.f, tot = 0.f;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
        const float x = tot8[u][l];
        off += (u < w) ? x : 0.f;
        tot += x;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) A2[8 * w + s][l] = LOG ? cum[s] + off : fexp2(cum[s] + off);
    if (w == 0) {
        G2[l] = fexp2(tot);
        if (LOG) Gl[l] = tot;
    }
    return tot;
}

// Per-token inputs of the epilogue kernel: fp32 pieces i = tid + 512 u (u < 2),
// rows i / 16, columns 4 (i % 16); 16-bit pieces: row tid / 8, columns 8 (tid % 8).
struct DoIn {
    float4 g[2];
    uint4 q, k, v, z, dy;
};

__device__ __forceinline__ void request_do(DoIn &in, const BdArgs &p, const int64_t *rows, int tid) {
    const GlaArgs &a = p.a;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + NTB * u, t = i >> 4, c = (i & 15) * 4;
        in.g[u] = ld4(a.log_g + rows[t] * DK + c);
    }
    const int t = tid >> 3, c = (tid & 7) * 8;
    const int64_t rk = rows[t] * DK + c, rv = rows[t] * BC + c;
    in.q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + rk);
    in.k = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) + rk);
    in.v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) + rv);
    in.z = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.z) + rv);
    in.dy = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.dy) + rv);
}

template <int DT>
__global__ __launch_bounds__(NTB, 1) void k_bdo(BdArgs p) {
    const GlaArgs &a = p.a;
    // hi + lo planes: Q~; K^, then P^T; K~; V; S^T, then dO
    __shared__ __attribute__((aligned(16))) uint16_t sQT[2 * MAT], sKP[2 * MAT], sKT[2 * MAT];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2 * MAT], sSD[2 * MAT];
    __shared__ __attribute__((aligned(16))) float sX[BC][LS];  // a (log2), then O, then Ur (staging)
    __shared__ float sG[BC], sGl[BC], sTot[NW][BC], sW[NW][BC];
    __shared__ int64_t srow[2][BC];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, g = l >> 4;
    const int rs = w & 3, ch2 = w >> 2;  // row stripe, column half
    const int64_t total = static_cast<int64_t>(a.B) * a.H * p.n_chunks;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * p.R;
    const int64_t c1 = (c0 + p.R < total) ? c0 + p.R : total;
    const int et = tid >> 3, ec = (tid & 7) * 8;  // load-layout row and columns of this thread
    float rw[8];                                  // rms_w of those columns
    {
        const float4 w0 = ld4(a.rms_w + ec), w1 = ld4(a.rms_w + ec + 4);
        rw[0] = w0.x; rw[1] = w0.y; rw[2] = w0.z; rw[3] = w0.w;
        rw[4] = w1.x; rw[5] = w1.y; rw[6] = w1.z; rw[7] = w1.w;
    }
    // carried forward state, MFMA layout: sreg[tt][r] = S[16 rs + 4 g + r][16 (2 ch2 + tt) + lr];
    // a range's first chunk starts from its segment's incoming state (none at a
    // sequence's first chunk)
    float sreg[2][4];
    {
        const bool first = ChunkAt(a, p.n_chunks, c0).n == 0;
        const float *src = p.Sseg + seg_id(c0, p.pl) * MAT;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sreg[tt][r] = first ? 0.f : src[(16 * rs + 4 * g + r) * BC + 16 * (2 * ch2 + tt) + lr];
    }

    float wsum = 0.f;  // wave 0, lane l: drms_w partials of the range's unflagged chunks, in order
    int buf = 0;
    if (tid < BC) srow[0][tid] = ChunkAt(a, p.n_chunks, c0).row(a, tid);
    __syncthreads();
    DoIn in;
    request_do(in, p, srow[0], tid);

    for (int64_t chk = c0; chk < c1; ++chk, buf ^= 1) {
        const ChunkAt at(a, p.n_chunks, chk);
        const int64_t *rows = srow[buf];
        const int nt = at.nt;
        const int64_t cn = chk + 1;
        if (at.n == 0) {  // a new sequence
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r) sreg[tt][r] = 0.f;
        }

        const float tot = chunk_gates8<true>(in.g, sX, sG, sTot, nt, tid, sGl);
        const bool slow = __syncthreads_or(-tot > kSpanMax);
        if (tid == 0) p.flags[at.cidx] = slow ? 1 : 0;

        // ---- the chunk's incoming state as S^T planes; a flagged chunk's also to Sx
        // (the token-serial kernels read it, and the state after it)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int d = 16 * (2 * ch2 + tt) + lr;
            if (slow) {
#pragma unroll
                for (int r = 0; r < 4; ++r) p.Sx[at.cidx * MAT + (16 * rs + 4 * g + r) * BC + d] = sreg[tt][r];
            }
            put<4>(sSD, d, 16 * rs + 4 * g, sreg[tt]);
        }
        // ---- operands (rows past the chunk's end are zero): K~ = k 2^(G - a) and V
        // always (the state carry); Q~ = q 2^a and K^ = k 2^-a for the matrix path
        uint4 zk, yk;  // z and dy, kept for the epilogue
        {
            const bool ok = et < nt;
            float q8[8], k8[8], v8[8], kt[8];
            unpack8<DT>(in.q, q8);
            unpack8<DT>(in.k, k8);
            unpack8<DT>(in.v, v8);
            zk = in.z;
            yk = in.dy;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const float av = sX[et][ec + s];
                kt[s] = ok ? k8[s] * fexp2(sGl[ec + s] - av) : 0.f;
                q8[s] = ok ? q8[s] * fexp2(av) : 0.f;
                k8[s] = ok ? k8[s] * fexp2(-av) : 0.f;
                v8[s] = ok ? v8[s] : 0.f;
            }
            put<8>(sKT, et, ec, kt);
            put<8>(sV, et, ec, v8);
            if (!slow) {
                put<8>(sQT, et, ec, q8);
                put<8>(sKP, et, ec, k8);
            }
        }
        if (cn < c1 && tid < BC) srow[buf ^ 1][tid] = ChunkAt(a, p.n_chunks, cn).row(a, tid);
        __syncthreads();
        if (cn < c1) request_do(in, p, srow[buf ^ 1], tid);

        f32x4 acc[2];
        // ---- the state after the chunk: S <- 2^G . S + K~^T V
        zero2(acc);
        gemm2<TRN, TRN>(acc, sKT, sV, rs, ch2, lr, g);    // A(m=c, k=j) = K~[j][c], B(k=j, n=d) = V[j][d]
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sreg[tt][r] = sG[16 * rs + 4 * g + r] * sreg[tt][r] + acc[tt][r];
        if (slow) {  // the whole workgroup; the token-serial kernels take the chunk
            if (at.n + 1 < p.n_chunks) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        p.Sx[(at.cidx + 1) * MAT + (16 * rs + 4 * g + r) * BC + 16 * (2 * ch2 + tt) + lr] =
                            sreg[tt][r];
            }
            __syncthreads();
            continue;
        }

        // ---- P = (Q~ K^^T) . M; P^T replaces K^
        zero2(acc);
        gemm2<NAT, NAT>(acc, sQT, sKP, rs, ch2, lr, g);   // B(k=c, n=j) = K^[j][c]
        __syncthreads();  // K^ is read
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = 2 * ch2 + tt;
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = (16 * t + lr <= 16 * rs + 4 * g + r) ? acc[tt][r] : 0.f;
            put<4>(sKP, 16 * t + lr, 16 * rs + 4 * g, x);
        }
        __syncthreads();
        // ---- O = Q~ S + P V, staged
        zero2(acc);
        gemm2<NAT, NAT>(acc, sQT, sSD, rs, ch2, lr, g);   // B(k=c, n=d) = S[c][d] = S^T[d][c]
        gemm2<TRN, TRN>(acc, sKP, sV, rs, ch2, lr, g);    // A(m=i, k=j) = P[i][j], B(k=j, n=d) = V[j][d]
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sX[16 * rs + 4 * g + r][16 * (2 * ch2 + tt) + lr] = acc[tt][r];
        __syncthreads();  // O staged; S is read

        // ---- epilogue backward in the load layout: row et, columns ec .. ec + 7
        {
            const bool ok = et < nt;
            float o[8], z8[8], dy8[8];
            const float4 o0 = ld4(&sX[et][ec]), o1 = ld4(&sX[et][ec + 4]);
            o[0] = o0.x; o[1] = o0.y; o[2] = o0.z; o[3] = o0.w;
            o[4] = o1.x; o[5] = o1.y; o[6] = o1.z; o[7] = o1.w;
            unpack8<DT>(zk, z8);
            unpack8<DT>(yk, dy8);
            float ss = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s) ss += o[s] * o[s];
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            ss += __shfl_xor(ss, 4);
            const float r = 1.0f / sqrtf(ss / BC + GTR_RMS_EPS);
            float nn[8], dn[8], sg[8], md = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                nn[s] = o[s] * r;
                sg[s] = frcp(1.0f + fexp2(-z8[s] * kLog2e));
                dn[s] = dy8[s] * rw[s] * (z8[s] * sg[s]);
                md += dn[s] * nn[s];
            }
            md += __shfl_xor(md, 1);
            md += __shfl_xor(md, 2);
            md += __shfl_xor(md, 4);
            md *= 1.0f / BC;
            float dov[8], dzv[8], wp[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                dov[s] = ok ? r * (dn[s] - nn[s] * md) : 0.f;
                dzv[s] = dy8[s] * nn[s] * rw[s] * sg[s] * (1.0f + z8[s] * (1.0f - sg[s]));
                wp[s] = ok ? dy8[s] * nn[s] * (z8[s] * sg[s]) : 0.f;
            }
            put<8>(sSD, et, ec, dov);
            if (ok) {
                float *dst = p.dO + rows[et] * BC + ec;
                st4(dst, make_float4(dov[0], dov[1], dov[2], dov[3]));
                st4(dst + 4, make_float4(dov[4], dov[5], dov[6], dov[7]));
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.dz) + rows[et] * BC + ec) = pack8<DT>(dzv);
            }
            // drms_w partial: the 8 rows of this wave that share the columns
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                float x = wp[s];
                x += __shfl_xor(x, 8);
                x += __shfl_xor(x, 16);
                x += __shfl_xor(x, 32);
                wp[s] = x;
            }
            if (l < 8) {
#pragma unroll
                for (int s = 0; s < 8; ++s) sW[w][8 * l + s] = wp[s];
            }
        }
        __syncthreads();  // dO in LDS; O is read

        // ---- Ur = Q~^T dO (rows c), staged; G and the drms_w partial (waves in order)
        zero2(acc);
        gemm2<TRN, TRN>(acc, sQT, sSD, rs, ch2, lr, g);   // A(m=c, k=i) = Q~[i][c], B(k=i, n=d) = dO[i][d]
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sX[16 * rs + 4 * g + r][16 * (2 * ch2 + tt) + lr] = acc[tt][r];
        if (w == 0) {
            float x = 0.f;
#pragma unroll
            for (int u = 0; u < NW; ++u) x += sW[u][l];
            p.Gr[at.ridx * BC + l] = tot;
            wsum += x;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = tid + NTB * u, t = i >> 4, c = (i & 15) * 4;
            st4(p.Ur + at.ridx * MAT + t * BC + c, ld4(&sX[t][c]));
        }
        __syncthreads();  // LDS is rewritten by the next chunk
    }
    if (w == 0) p.wr[static_cast<int64_t>(blockIdx.x) * BC + l] = wsum;
}

// ---- The gradients (see the top of the file), eight waves.
// Per-token inputs: fp32 pieces i = tid + 512 u (u < 2), rows i / 16, columns
// 4 (i % 16); 16-bit pieces: row tid / 8, columns 8 (tid % 8).
struct TokIn {
    float4 g[2], dO[2];
    uint4 q, k, v;
    int flag;  // the chunk's flag (same address in every lane)
};
struct StateIn {  // the chunk's reverse state, requested once the last is used
    float4 E[2];
};

__device__ __forceinline__ void request_tok(TokIn &in, const BgArgs &p, const int64_t *rows,
                                            int64_t chunk, int tid) {
    const GlaArgs &a = p.a;
    in.flag = p.flags[chunk];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + NTB * u, t = i >> 4, c = (i & 15) * 4;
        in.g[u] = ld4(a.log_g + rows[t] * DK + c);
    }
    {
        const int t = tid >> 3, c = (tid & 7) * 8;
        in.q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + rows[t] * DK + c);
        in.k = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) + rows[t] * DK + c);
        in.v = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) + rows[t] * BC + c);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + NTB * u, t = i >> 4, c = (i & 15) * 4;
        in.dO[u] = ld4(p.dO + rows[t] * BC + c);
    }
}

__device__ __forceinline__ void request_state(StateIn &in, const BgArgs &p, const ChunkAt &at, int tid) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = tid + NTB * u, t = i >> 4, c = (i & 15) * 4;
        in.E[u] = ld4(p.Er + at.ridx * MAT + t * BC + c);  // E[c'][d]: row c' = t, column d = c
    }
}

__device__ __forceinline__ void ld8(const float *src, float (&x)[8]) {
    const float4 a = ld4(src), b = ld4(src + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <int DT>
__global__ __launch_bounds__(NTB, 1) void k_bgrad(BgArgs p) {
    const GlaArgs &a = p.a;
    // hi + lo planes; SE holds S, then E'
    __shared__ __attribute__((aligned(16))) uint16_t sDO[2 * MAT], sQT[2 * MAT], sKH[2 * MAT], sV[2 * MAT];
    __shared__ __attribute__((aligned(16))) uint16_t sSE[2 * MAT], sDT[2 * MAT], sPT[2 * MAT];
    __shared__ __attribute__((aligned(16))) float sA2[BC][LS];  // 2^a, later q dq - k dk
    __shared__ __attribute__((aligned(16))) float sX[BC][LS];   // fp32 staging: T, dq, dk, dv
    __shared__ float sG[BC], sOff[BC], sTot[NW][BC];
    __shared__ int64_t srow[2][BC];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, g = l >> 4;
    const int rs = w & 3, ch2 = w >> 2;           // row stripe, column half
    const int et = tid >> 3, ec = (tid & 7) * 8;  // load-layout row and columns (16-bit pieces)
    const int64_t total = static_cast<int64_t>(a.B) * a.H * p.n_chunks;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * p.R;
    const int64_t c1 = (c0 + p.R < total) ? c0 + p.R : total;
    // carried forward state, transposed in the MFMA layout: sreg[tt][r] =
    // S[16 (2 ch2 + tt) + lr][16 rs + 4 g + r] (four consecutive columns of a row of S),
    // from the segment's incoming state (none at a sequence's first chunk)
    float sreg[2][4];
    auto load_state = [&](const float *src) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const float4 x = ld4(src + (16 * (2 * ch2 + tt) + lr) * BC + 16 * rs + 4 * g);
            sreg[tt][0] = x.x; sreg[tt][1] = x.y; sreg[tt][2] = x.z; sreg[tt][3] = x.w;
        }
    };
    auto zero_state = [&]() {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sreg[tt][r] = 0.f;
    };
    if (ChunkAt(a, p.n_chunks, c0).n == 0)
        zero_state();
    else
        load_state(p.Sseg + seg_id(c0, p.pl) * MAT);

    int buf = 0;
    if (tid < BC) srow[0][tid] = ChunkAt(a, p.n_chunks, c0).row(a, tid);
    __syncthreads();
    TokIn in;
    StateIn st_in;
    request_tok(in, p, srow[0], c0, tid);
    request_state(st_in, p, ChunkAt(a, p.n_chunks, c0), tid);

    for (int64_t chk = c0; chk < c1; ++chk, buf ^= 1) {
        const ChunkAt at(a, p.n_chunks, chk);
        const int64_t *rows = srow[buf];
        const int nt = at.nt;
        const int64_t cn = chk + 1;  // next chunk of this workgroup (if below c1)
        if (at.n == 0) zero_state();  // a new sequence

        chunk_gates8(in.g, sA2, sG, sTot, nt, tid);
        const bool slow = in.flag != 0;  // the epilogue kernel's decision; uniform
        __syncthreads();

        // ---- operands (rows past the chunk's end are zero); exact q and k kept
        uint4 qkeep, kkeep;
        if (!slow) {
            const bool ok = et < nt;
            float q8[8], k8[8], v8[8];
            unpack8<DT>(in.q, q8);
            unpack8<DT>(in.k, k8);
            unpack8<DT>(in.v, v8);
            qkeep = in.q;
            kkeep = in.k;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const float e = sA2[et][ec + s];
                q8[s] = ok ? q8[s] * e : 0.f;
                k8[s] = ok ? k8[s] * frcp(e) : 0.f;
                v8[s] = ok ? v8[s] : 0.f;
            }
            put<8>(sQT, et, ec, q8);
            put<8>(sKH, et, ec, k8);
            put<8>(sV, et, ec, v8);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int i = tid + NTB * u, t = i >> 4, c = (i & 15) * 4;
                const float4 d = in.dO[u];
                const bool okr = t < nt;
                const float dd[4] = {okr ? d.x : 0.f, okr ? d.y : 0.f, okr ? d.z : 0.f, okr ? d.w : 0.f};
                put<4>(sDO, t, c, dd);
            }
            // the incoming state as S planes (row c, columns d)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) put<4>(sSE, 16 * (2 * ch2 + tt) + lr, 16 * rs + 4 * g, sreg[tt]);
        }
        // ---- the next chunk's rows, then its per-token inputs (those registers are free)
        if (cn < c1 && tid < BC) srow[buf ^ 1][tid] = ChunkAt(a, p.n_chunks, cn).row(a, tid);
        __syncthreads();
        if (cn < c1) request_tok(in, p, srow[buf ^ 1], cn, tid);
        if (slow) {  // the whole workgroup; its gradients come from the token-serial kernels
            if (cn < c1) request_state(st_in, p, ChunkAt(a, p.n_chunks, cn), tid);
            // the state after the chunk, as the epilogue kernel wrote it; waited for
            // here (an empty asm reads the registers), so that no load into them is
            // outstanding where the other path reuses registers
            if (at.n + 1 < p.n_chunks)
                load_state(p.Sx + (at.cidx + 1) * MAT);
            else
                zero_state();
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                asm volatile("" ::"v"(sreg[tt][0]), "v"(sreg[tt][1]), "v"(sreg[tt][2]), "v"(sreg[tt][3]));
            continue;
        }

        f32x4 acc[2];
        // ---- D = (dO V^T) . M and P = (Q~ K^^T) . M, stored transposed
        zero2(acc);
        gemm2<NAT, NAT>(acc, sDO, sV, rs, ch2, lr, g);    // B(k=d, n=j) = V[j][d]
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = 2 * ch2 + tt;
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = (16 * t + lr <= 16 * rs + 4 * g + r) ? acc[tt][r] : 0.f;
            put<4>(sDT, 16 * t + lr, 16 * rs + 4 * g, x);
        }
        zero2(acc);
        gemm2<NAT, NAT>(acc, sQT, sKH, rs, ch2, lr, g);   // B(k=c, n=j) = K^[j][c]
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = 2 * ch2 + tt;
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = (16 * t + lr <= 16 * rs + 4 * g + r) ? acc[tt][r] : 0.f;
            put<4>(sPT, 16 * t + lr, 16 * rs + 4 * g, x);
        }
        // ---- the state after the chunk, S_out^T = (S^T + V^T K^) . 2^G (columns c),
        // carried and staged as S_out
        zero2(acc);
        gemm2<TRN, TRN>(acc, sV, sKH, rs, ch2, lr, g);    // A(m=d, k=j) = V[j][d], B(k=j, n=c) = K^[j][c]
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int c = 16 * (2 * ch2 + tt) + lr;
            const float gc = sG[c];
#pragma unroll
            for (int r = 0; r < 4; ++r) sreg[tt][r] = gc * (sreg[tt][r] + acc[tt][r]);
            st4(&sX[c][16 * rs + 4 * g], make_float4(sreg[tt][0], sreg[tt][1], sreg[tt][2], sreg[tt][3]));
        }
        __syncthreads();

        // ---- offset of the gate gradient: sum_d E[c][d] S_out[c][d]; the 16 lanes
        // of a channel row reduce together
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = tid + NTB * u, t = i >> 4, c = (i & 15) * 4;
            const float4 ev = st_in.E[u], sv = ld4(&sX[t][c]);
            float x = ev.x * sv.x + ev.y * sv.y + ev.z * sv.z + ev.w * sv.w;
            x += __shfl_xor(x, 1);
            x += __shfl_xor(x, 2);
            x += __shfl_xor(x, 4);
            x += __shfl_xor(x, 8);
            if ((tid & 15) == 0) sOff[t] = x;
        }

        // ---- dQ = 2^a . (dO S^T + D K^)
        zero2(acc);
        gemm2<NAT, NAT>(acc, sDO, sSE, rs, ch2, lr, g);   // B(k=d, n=c) = S[c][d]
        gemm2<TRN, TRN>(acc, sDT, sKH, rs, ch2, lr, g);   // A(m=i, k=j) = D[i][j], B(k=j, n=c) = K^[j][c]
        __syncthreads();  // S and T are read
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * rs + 4 * g + r, c = 16 * (2 * ch2 + tt) + lr;
                sX[i][c] = sA2[i][c] * acc[tt][r];
            }
        // E' = 2^G . E (rows c scaled), then the next chunk's states
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = tid + NTB * u, t = i >> 4, c = (i & 15) * 4;
            const float4 ev = st_in.E[u];
            const float gt = sG[t];
            const float ee[4] = {gt * ev.x, gt * ev.y, gt * ev.z, gt * ev.w};
            put<4>(sSE, t, c, ee);
        }
        if (cn < c1) request_state(st_in, p, ChunkAt(a, p.n_chunks, cn), tid);
        __syncthreads();
        // dq out; q . dq of this thread's piece
        float qdq[8];
        {
            float x[8], q8[8];
            ld8(&sX[et][ec], x);
            unpack8<DT>(qkeep, q8);
#pragma unroll
            for (int s = 0; s < 8; ++s) qdq[s] = q8[s] * x[s];
            if (et < nt)
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.dq) + rows[et] * DK + ec) = pack8<DT>(x);
        }

        // ---- dK = 2^-a . (D^T Q~ + V E'^T)
        zero2(acc);
        gemm2<PERM, TRN>(acc, sDT, sQT, rs, ch2, lr, g);  // A(m=j, k=i) = D[i][j], B(k=i, n=c) = Q~[i][c]
        gemm2<NAT, NAT>(acc, sV, sSE, rs, ch2, lr, g);    // B(k=d, n=c) = E'[c][d]
        __syncthreads();  // dq is read
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * rs + 4 * g + r, c = 16 * (2 * ch2 + tt) + lr;
                sX[j][c] = acc[tt][r] * frcp(sA2[j][c]);
            }
        __syncthreads();
        // dk out; the gate gradient's terms q dq - k dk replace 2^a
        {
            float x[8], k8[8], y[8];
            ld8(&sX[et][ec], x);
            unpack8<DT>(kkeep, k8);
            const bool ok = et < nt;
#pragma unroll
            for (int s = 0; s < 8; ++s) y[s] = ok ? qdq[s] - k8[s] * x[s] : 0.f;
            st4(&sA2[et][ec], make_float4(y[0], y[1], y[2], y[3]));
            st4(&sA2[et][ec + 4], make_float4(y[4], y[5], y[6], y[7]));
            if (ok)
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.dk) + rows[et] * DK + ec) = pack8<DT>(x);
        }

        // ---- dV = P^T dO + K^ E'
        zero2(acc);
        gemm2<PERM, TRN>(acc, sPT, sDO, rs, ch2, lr, g);  // A(m=j, k=i) = P[i][j], B(k=i, n=d) = dO[i][d]
        gemm2<PERM, TRN>(acc, sKH, sSE, rs, ch2, lr, g);  // A(m=j, k=c) = K^[j][c], B(k=c, n=d) = E'[c][d]
        __syncthreads();  // dk and the gate terms are through LDS
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sX[16 * rs + 4 * g + r][16 * (2 * ch2 + tt) + lr] = acc[tt][r];
        // dlog_g, part 1: wave w takes tokens [8 w, 8 w + 8) of channel l
        float x8[8];
        {
            float s = 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                x8[u] = sA2[8 * w + u][l];
                s += x8[u];
            }
            sTot[w][l] = s;
        }
        __syncthreads();
        // dv out
        {
            float x[8];
            ld8(&sX[et][ec], x);
            if (et < nt)
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.dv) + rows[et] * BC + ec) = pack8<DT>(x);
        }
        // dlog_g, part 2: reverse cumulative sum from the offset and the later segments
        float s = sOff[l];
#pragma unroll
        for (int u = NW - 1; u > 0; --u) s += (u > w) ? sTot[u][l] : 0.f;
#pragma unroll
        for (int u = 7; u >= 0; --u) {
            const int t = 8 * w + u;
            s += x8[u];
            if (t < nt) p.dlog_g[rows[t] * DK + l] = s;
        }
        __syncthreads();  // LDS is rewritten by the next chunk
    }
}

}  // namespace

bool bgrad_supported(const GlaArgs &a) {
    auto al16 = [](const void *x) { return (reinterpret_cast<uintptr_t>(x) & 15) == 0; };
    return (a.dtype == DT_F16 || a.dtype == DT_BF16) && a.dk == 64 && a.dv == 64 && a.chunk <= 64 &&
           !a.resid && al16(a.q) && al16(a.k) && al16(a.v) && al16(a.log_g);
}

hipError_t bdo_launch(const GlaArgs &a, const MfmaPlan &pl, int64_t R, const void *dy,
                      const float *Sseg, float *Sx, float *dO, void *dz, float *wr, float *Ur,
                      float *Gr, int *flags, int n_chunks, hipStream_t s) {
    const BdArgs p{a, dy, Sseg, Sx, dO, dz, wr, Ur, Gr, flags, n_chunks, pl, R};
    const dim3 grid(static_cast<unsigned>((pl.T + R - 1) / R));
    if (a.dtype == DT_F16)
        hipLaunchKernelGGL((k_bdo<DT_F16>), grid, dim3(NTB), 0, s, p);
    else if (a.dtype == DT_BF16)
        hipLaunchKernelGGL((k_bdo<DT_BF16>), grid, dim3(NTB), 0, s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t bgrad_launch(const GlaArgs &a, const MfmaPlan &pl, int64_t R, const float *dO,
                        const float *Sseg, const float *Sx, const float *Er, void *dq, void *dk,
                        void *dv, float *dlog_g, const int *flags, int n_chunks, hipStream_t s) {
    const BgArgs p{a, dO, Sseg, Sx, Er, dq, dk, dv, dlog_g, flags, n_chunks, pl, R};
    const dim3 grid(static_cast<unsigned>((pl.T + R - 1) / R));
    if (a.dtype == DT_F16)
        hipLaunchKernelGGL((k_bgrad<DT_F16>), grid, dim3(NTB), 0, s, p);
    else if (a.dtype == DT_BF16)
        hipLaunchKernelGGL((k_bgrad<DT_BF16>), grid, dim3(NTB), 0, s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gtr
