// k_bwd.hip -- backward pass of one mixer call, fp32, chunk-parallel.
//
// GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"), Method §1 gives the
// forward: S_t = Diag(g_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, then RMSNorm,
// the rms_w weight and the SiLU(z) gate; Method §4 its chunkwise evaluation
// (chunk summaries, a boundary-state scan, per-chunk outputs), which the
// backward mirrors in both directions.  With dy the gradient of the output:
//   epilogue   r = (mean(o^2) + eps)^-1/2, n = r o:  dn = dy w silu(z),
//              do = r (dn - n mean(dn n)),  dz = dy n w silu'(z),  drms_w = sum dy n silu(z)
//   forward    dq_t = S_t do_t                         (S_t from the chunk's incoming state)
//   reverse    dS_t = q_t do_t^T + Diag(g_{t+1}) dS_{t+1},  dk_t = dS_t v_t,  dv_t = dS_t^T k_t
//   gate       dlog_g_t = sum_{s >= t} (q_s dq_s - k_s dk_s)   (reverse cumulative sum; the
//              derivative of the loss with respect to the cumulative log-gate at step s is
//              q_s dq_s - k_s dk_s, and log g_t enters every cumulative sum from t on)
// The reverse recurrence has the same form as the forward one read backwards:
// a chunk's dS summary from zero, E = Diag(g_first) dS_first, chains across chunks
// as E_{n-1} = Diag(exp(Gamma_n)) E_n + (summary of chunk n), so the forward scan
// kernel runs it over the chunks in reversed order.
//
// Every kernel is token-serial inside a chunk, one workgroup per (b, h, chunk),
// with the dk x dv state (or its gradient) in registers.  Two thread->state maps:
//   A: column j = tid % DV, channels c0 + CSTEP m (c0 = tid / DV): sums over
//      channels (o_t, dv_t) are per-thread partials added across CSTEP groups;
//   B: channel c = tid % DK, columns j0 + JSTEP m (j0 = tid / DK): sums over columns
//      (dq_t, dk_t) likewise.
// Where a chunk needs sums along both axes it is walked twice, once per map.
#include "gtr_internal.hpp"

namespace gtr {
namespace {

constexpr int NT = 256;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int64_t kBwdWorkgroups = 256;  // matrix-core backward kernels: one per CU

template <int DK, int DV> struct BwdShape {
    static constexpr int PER = DK * DV / NT;      // state elements per thread
    static constexpr int CSTEP = NT / DV;         // map A: channel stride
    static constexpr int JSTEP = NT / DK;         // map B: column stride
    static constexpr int TILE = (DK + DV > 128) ? 8 : 16;
    static constexpr int RG = CSTEP > JSTEP ? CSTEP : JSTEP;
    static constexpr int RW = DK > DV ? DK : DV;
    // LDS order of the per-token channel and column vectors: the PER channels a
    // map-A thread walks (c0 + CSTEP m) and the PER columns a map-B thread walks
    // (j0 + JSTEP m) are contiguous, so each thread reads them as 16-byte pieces
    __device__ static int pc(int c) { return (c % CSTEP) * PER + c / CSTEP; }
    __device__ static int pj(int j) { return (j % JSTEP) * PER + j / JSTEP; }
};

// PER floats of an LDS row starting at a 16-byte aligned offset
template <int PER>
__device__ __forceinline__ void lds_vec(const float *src, float (&dst)[PER]) {
#pragma unroll
    for (int i = 0; i < PER / 4; ++i) {
        const float4 x = reinterpret_cast<const float4 *>(src)[i];
        dst[4 * i] = x.x; dst[4 * i + 1] = x.y; dst[4 * i + 2] = x.z; dst[4 * i + 3] = x.w;
    }
}

struct BwdArgs {
    GlaArgs a;
    const void *dy;      // gradient of out, I/O type
    const float *Sx;     // forward incoming state per chunk [bh N + n][DK][DV]
    const float *Er;     // reverse incoming gradient state per chunk, reversed order
    float *dO;           // [rows][DV]
    float *qdq;          // [rows][DK]
    float *Ur, *Gr;      // reverse summaries and chunk gates, reversed chunk order
    float *Tn;           // [bh N + n][DK] chunk totals of q dq - k dk
    float *dWp;          // [bh N + n][DV] drms_w partials
    void *dq, *dk, *dv, *dz;
    float *dlog_g, *drms_w;
    const int *flags;    // chunks left to the token-serial gradients (matrix-core path)
    int n_chunks;
    float *part2;        // [WS_BLOCKS][DV] drms_w block sums
    unsigned *ctr;       // zero between calls
};

// Chunk c (of B H N, sequence-major) and its token range
struct ChunkPos {
    int n, bh, b, h;
    int64_t t0, t1, c;
    __device__ ChunkPos(const GlaArgs &a, int n_chunks, int64_t c_) : c(c_) {
        n = static_cast<int>(c % n_chunks);
        bh = static_cast<int>(c / n_chunks);
        b = bh / a.H;
        h = bh % a.H;
        t0 = static_cast<int64_t>(n) * a.chunk;
        t1 = (t0 + a.chunk < a.L) ? t0 + a.chunk : a.L;
    }
    __device__ size_t cid() const { return static_cast<size_t>(c); }
};

// ---- B1: forward walk.  Pass 1 (map A): o_t, epilogue backward -> do_t (global),
// dz_t, drms_w partials.  Pass 2 (map B): dq_t = S_t do_t, q dq (fp32, global).
// MODE 0: both passes; 1: pass 1 only; 2: pass 2 only.
template <int DT, int DK, int DV, int MODE>
__device__ __forceinline__ void fwdwalk_body(const BwdArgs &p, const ChunkPos &cp) {
    using Sh = BwdShape<DK, DV>;
    constexpr int PER = Sh::PER, CSTEP = Sh::CSTEP, JSTEP = Sh::JSTEP, TILE = Sh::TILE;
    const GlaArgs &a = p.a;
    __shared__ __attribute__((aligned(16))) float sq[TILE][DK], sk[TILE][DK], sg[TILE][DK];
    __shared__ __attribute__((aligned(16))) float sv[TILE][DV], sz[TILE][DV], sdy[TILE][DV], so[TILE][DV], sdn[TILE][DV];
    __shared__ __attribute__((aligned(16))) float red[TILE][Sh::RG][Sh::RW];
    __shared__ __attribute__((aligned(16))) float swp[NT];
    __shared__ __attribute__((aligned(16))) float sinv[TILE], smdn[TILE];  // per token: RMSNorm factor, mean(dn n)
    __shared__ int64_t srow[TILE];
    const int tid = threadIdx.x;
    const size_t soff = cp.cid() * DK * DV;

    // ---- pass 1, map A
    if constexpr (MODE != 2) {
        const int j = tid % DV, c0 = tid / DV;
        float s[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) s[m] = p.Sx[soff + static_cast<size_t>(c0 + CSTEP * m) * DV + j];
        float wacc = 0.f;  // drms_w partial of column tid % DV
        for (int64_t tb = cp.t0; tb < cp.t1; tb += TILE) {
            const int nt = static_cast<int>((cp.t1 - tb < TILE) ? cp.t1 - tb : TILE);
            __syncthreads();
            if (tid < TILE) srow[tid] = tid < nt ? scan_row(a, cp.b, cp.h, tb + tid) : 0;
            __syncthreads();
            for (int i = tid; i < TILE * DK; i += NT) {
                const int tt = i / DK, c = i % DK;
                float kk = 0.f, lg = 0.f, qq = 0.f;
                if (tt < nt) {
                    const int64_t r = srow[tt] * DK + c;
                    kk = ld<DT>(a.k, r);
                    lg = a.log_g[r];
                    qq = ld<DT>(a.q, r);
                }
                sk[tt][Sh::pc(c)] = kk;
                sg[tt][Sh::pc(c)] = expf(lg);
                sq[tt][Sh::pc(c)] = qq;
            }
            for (int i = tid; i < TILE * DV; i += NT) {
                const int tt = i / DV, jj = i % DV;
                float vv = 0.f, zz = 0.f, gy = 0.f;
                if (tt < nt) {
                    const int64_t r = srow[tt] * DV + jj;
                    vv = ld<DT>(a.v, r);
                    zz = ld<DT>(a.z, r);
                    gy = ld<DT>(p.dy, r);
                }
                sv[tt][jj] = vv;
                sz[tt][jj] = zz;
                sdy[tt][jj] = gy;
            }
            __syncthreads();
            for (int tt = 0; tt < nt; ++tt) {
                const float vj = sv[tt][j];
                float gg[PER], kk[PER], qq[PER];
                lds_vec<PER>(&sg[tt][c0 * PER], gg);
                lds_vec<PER>(&sk[tt][c0 * PER], kk);
                lds_vec<PER>(&sq[tt][c0 * PER], qq);
                float part = 0.f;
#pragma unroll
                for (int m = 0; m < PER; ++m) {
                    s[m] = gg[m] * s[m] + kk[m] * vj;
                    part += s[m] * qq[m];
                }
                red[tt][c0][j] = part;
            }
            __syncthreads();
            for (int i = tid; i < TILE * DV; i += NT) {
                const int tt = i / DV, jj = i % DV;
                float o = 0.f;
#pragma unroll
                for (int r = 0; r < CSTEP; ++r) o += red[tt][r][jj];
                so[tt][jj] = o;
            }
            __syncthreads();
            if (tid < nt) {  // one thread per token: the RMSNorm factor
                float ss = 0.f;
                for (int x = 0; x < DV; ++x) ss += so[tid][x] * so[tid][x];
                sinv[tid] = 1.0f / sqrtf(ss / DV + GTR_RMS_EPS);
            }
            __syncthreads();
            // epilogue backward, element (tt, jj) = (i / DV, i % DV), i = tid + u NT; jj is
            // tid % DV for every u (NT is a multiple of DV)
            constexpr int ITER = TILE * DV / NT;
            float nn[ITER], inv_t[ITER];
#pragma unroll
            for (int u = 0; u < ITER; ++u) {
                const int i = tid + u * NT;
                nn[u] = inv_t[u] = 0.f;
                if (i < nt * DV) {
                    const int tt = i / DV, jj = i % DV;
                    const float inv = sinv[tt];
                    const float n = so[tt][jj] * inv;
                    const float zz = sz[tt][jj];
                    const float sig = 1.0f / (1.0f + expf(-zz));
                    const float silu = zz * sig;
                    const float gy = sdy[tt][jj];
                    const float w = a.rms_w[jj];
                    sdn[tt][jj] = gy * w * silu * n;  // dn * n, for the projection term
                    wacc += gy * n * silu;
                    st<DT>(p.dz, srow[tt] * DV + jj, gy * n * w * sig * (1.0f + zz * (1.0f - sig)));
                    nn[u] = n;
                    inv_t[u] = inv;
                }
            }
            __syncthreads();
            if (tid < nt) {
                float mdn = 0.f;
                for (int x = 0; x < DV; ++x) mdn += sdn[tid][x];
                smdn[tid] = mdn * (1.0f / DV);
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < ITER; ++u) {
                const int i = tid + u * NT;
                if (i < nt * DV) {
                    const int tt = i / DV, jj = i % DV;
                    const float mdn = smdn[tt];
                    const float zz = sz[tt][jj];
                    const float silu = zz / (1.0f + expf(-zz));
                    const float dn = sdy[tt][jj] * a.rms_w[jj] * silu;
                    p.dO[srow[tt] * DV + jj] = inv_t[u] * (dn - nn[u] * mdn);
                }
            }
        }
        swp[tid] = wacc;
        __syncthreads();
        if (tid < DV) {
            float w = 0.f;
            for (int r = tid; r < NT; r += DV) w += swp[r];
            p.dWp[cp.cid() * DV + tid] = w;
        }
    }
    if constexpr (MODE == 1) return;
    __syncthreads();  // this workgroup's do_t writes are visible to its own reads below

    // ---- pass 2, map B: dq_t = S_t do_t
    {
        const int c = tid % DK, j0 = tid / DK;
        float s[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) s[m] = p.Sx[soff + static_cast<size_t>(c) * DV + j0 + JSTEP * m];
        for (int64_t tb = cp.t0; tb < cp.t1; tb += TILE) {
            const int nt = static_cast<int>((cp.t1 - tb < TILE) ? cp.t1 - tb : TILE);
            __syncthreads();
            if (tid < TILE) srow[tid] = tid < nt ? scan_row(a, cp.b, cp.h, tb + tid) : 0;
            __syncthreads();
            for (int i = tid; i < TILE * DK; i += NT) {
                const int tt = i / DK, cc = i % DK;
                float kk = 0.f, lg = 0.f, qq = 0.f;
                if (tt < nt) {
                    const int64_t r = srow[tt] * DK + cc;
                    kk = ld<DT>(a.k, r);
                    lg = a.log_g[r];
                    qq = ld<DT>(a.q, r);
                }
                sk[tt][Sh::pc(cc)] = kk;
                sg[tt][Sh::pc(cc)] = expf(lg);
                sq[tt][Sh::pc(cc)] = qq;
            }
            for (int i = tid; i < TILE * DV; i += NT) {
                const int tt = i / DV, jj = i % DV;
                float vv = 0.f, dd = 0.f;
                if (tt < nt) {
                    const int64_t r = srow[tt] * DV + jj;
                    vv = ld<DT>(a.v, r);
                    dd = p.dO[r];
                }
                sv[tt][Sh::pj(jj)] = vv;
                so[tt][Sh::pj(jj)] = dd;  // do_t
            }
            __syncthreads();
            for (int tt = 0; tt < nt; ++tt) {
                const float g = sg[tt][Sh::pc(c)], kc = sk[tt][Sh::pc(c)];
                float vv[PER], dd[PER];
                lds_vec<PER>(&sv[tt][j0 * PER], vv);
                lds_vec<PER>(&so[tt][j0 * PER], dd);
                float part = 0.f;
#pragma unroll
                for (int m = 0; m < PER; ++m) {
                    s[m] = g * s[m] + kc * vv[m];
                    part += s[m] * dd[m];
                }
                red[tt][j0][c] = part;
            }
            __syncthreads();
            for (int i = tid; i < nt * DK; i += NT) {
                const int tt = i / DK, cc = i % DK;
                float d = 0.f;
#pragma unroll
                for (int r = 0; r < JSTEP; ++r) d += red[tt][r][cc];
                const int64_t r = srow[tt] * DK + cc;
                st<DT>(p.dq, r, d);
                p.qdq[r] = sq[tt][Sh::pc(cc)] * d;
            }
        }
    }
}

// ---- B2: reverse summary of each chunk (map A; no sums): dS walked from the
// chunk's last token to its first from zero, then Diag(g_first) dS; written with
// the chunk's summed gate (log2 units) at the reversed chunk index.
template <int DT, int DK, int DV>
__device__ __forceinline__ void revsum_body(const BwdArgs &p, const ChunkPos &cp) {
    using Sh = BwdShape<DK, DV>;
    constexpr int PER = Sh::PER, CSTEP = Sh::CSTEP, TILE = Sh::TILE;
    const GlaArgs &a = p.a;
    __shared__ __attribute__((aligned(16))) float sq[TILE][DK], sg[TILE][DK], sdo[TILE][DV];
    __shared__ __attribute__((aligned(16))) float gpart[NT];
    __shared__ int64_t srow[TILE];
    const int tid = threadIdx.x;
    const int j = tid % DV, c0 = tid / DV;
    float s[PER], gnext[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) s[m] = 0.f, gnext[m] = 0.f;  // no decay before the last token
    float gacc = 0.f;
    const int64_t len = cp.t1 - cp.t0;
    const int64_t ntiles = (len + TILE - 1) / TILE;
    for (int64_t ti = ntiles - 1; ti >= 0; --ti) {
        const int64_t tb = cp.t0 + ti * TILE;
        const int nt = static_cast<int>((cp.t1 - tb < TILE) ? cp.t1 - tb : TILE);
        __syncthreads();
        if (tid < TILE) srow[tid] = tid < nt ? scan_row(a, cp.b, cp.h, tb + tid) : 0;
        __syncthreads();
        for (int i = tid; i < TILE * DK; i += NT) {
            const int tt = i / DK, c = i % DK;
            float lg = 0.f, qq = 0.f;
            if (tt < nt) {
                const int64_t r = srow[tt] * DK + c;
                lg = a.log_g[r];
                qq = ld<DT>(a.q, r);
            }
            sg[tt][Sh::pc(c)] = expf(lg);
            sq[tt][Sh::pc(c)] = qq;
            gacc += lg;
        }
        for (int i = tid; i < TILE * DV; i += NT) {
            const int tt = i / DV, jj = i % DV;
            sdo[tt][jj] = tt < nt ? p.dO[srow[tt] * DV + jj] : 0.f;
        }
        __syncthreads();
        for (int tt = nt - 1; tt >= 0; --tt) {
            const float dj = sdo[tt][j];
            float qq[PER];
            lds_vec<PER>(&sq[tt][c0 * PER], qq);
#pragma unroll
            for (int m = 0; m < PER; ++m) s[m] = gnext[m] * s[m] + qq[m] * dj;
            lds_vec<PER>(&sg[tt][c0 * PER], gnext);
        }
    }
    // E contribution: Diag(g of the chunk's first token) dS_first
    const size_t ridx = static_cast<size_t>(cp.bh) * p.n_chunks + (p.n_chunks - 1 - cp.n);
#pragma unroll
    for (int m = 0; m < PER; ++m)
        p.Ur[ridx * DK * DV + static_cast<size_t>(c0 + CSTEP * m) * DV + j] = gnext[m] * s[m];
    gpart[tid] = gacc;
    __syncthreads();
    if (tid < DK) {
        float gsum = 0.f;
        for (int r = tid; r < NT; r += DK) gsum += gpart[r];
        p.Gr[ridx * DK + tid] = gsum * kLog2e;
    }
}

// ---- B3: reverse walk from the incoming gradient state E.  Pass A (map B):
// dk_t = dS_t v_t, then q dq - k dk, its reverse cumulative sum inside the chunk
// (written as dlog_g, completed by B4) and the chunk total.  Pass B (map A):
// dv_t = dS_t^T k_t.  OFFSET: dlog_g is completed here (the matrix-core path's
// fallback, which has no offset pass).
template <int DT, int DK, int DV, bool OFFSET>
__device__ __forceinline__ void revwalk_body(const BwdArgs &p, const ChunkPos &cp) {
    using Sh = BwdShape<DK, DV>;
    constexpr int PER = Sh::PER, CSTEP = Sh::CSTEP, JSTEP = Sh::JSTEP, TILE = Sh::TILE;
    const GlaArgs &a = p.a;
    __shared__ __attribute__((aligned(16))) float sq[TILE][DK], sk[TILE][DK], sg[TILE][DK];
    __shared__ __attribute__((aligned(16))) float sv[TILE][DV], sdo[TILE][DV];
    __shared__ __attribute__((aligned(16))) float red[TILE][Sh::RG][Sh::RW];
    __shared__ __attribute__((aligned(16))) float sacc[DK];
    __shared__ int64_t srow[TILE];
    const int tid = threadIdx.x;
    const size_t eoff = (static_cast<size_t>(cp.bh) * p.n_chunks + (p.n_chunks - 1 - cp.n)) * DK * DV;
    const int64_t len = cp.t1 - cp.t0;
    const int64_t ntiles = (len + TILE - 1) / TILE;

    auto load_tile = [&](int64_t tb, int nt) {
        __syncthreads();
        if (tid < TILE) srow[tid] = tid < nt ? scan_row(a, cp.b, cp.h, tb + tid) : 0;
        __syncthreads();
        for (int i = tid; i < TILE * DK; i += NT) {
            const int tt = i / DK, c = i % DK;
            float kk = 0.f, lg = 0.f, qq = 0.f;
            if (tt < nt) {
                const int64_t r = srow[tt] * DK + c;
                kk = ld<DT>(a.k, r);
                lg = a.log_g[r];
                qq = ld<DT>(a.q, r);
            }
            sk[tt][Sh::pc(c)] = kk;
            sg[tt][Sh::pc(c)] = expf(lg);
            sq[tt][Sh::pc(c)] = qq;
        }
        for (int i = tid; i < TILE * DV; i += NT) {
            const int tt = i / DV, jj = i % DV;
            float vv = 0.f, dd = 0.f;
            if (tt < nt) {
                const int64_t r = srow[tt] * DV + jj;
                vv = ld<DT>(a.v, r);
                dd = p.dO[r];
            }
            sv[tt][Sh::pj(jj)] = vv;
            sdo[tt][Sh::pj(jj)] = dd;
        }
        __syncthreads();
    };

    // ---- pass A, map B
    {
        const int c = tid % DK, j0 = tid / DK;
        float s[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) s[m] = p.Er[eoff + static_cast<size_t>(c) * DV + j0 + JSTEP * m];
        float gnext = 1.f;  // E already carries the next chunk's first gate
        if (tid < DK) {
            // complete dlog_g for a flagged chunk (the matrix-core path has no offset
            // pass): the sum over the later tokens of the sequence is the gate
            // gradient at the next chunk's first token, sum_d E[c][d] S_out[c][d],
            // with S_out the next chunk's incoming state (none after the last chunk)
            float o = 0.f;
            if (OFFSET && cp.n + 1 < p.n_chunks) {
                const float *sn = p.Sx + (cp.cid() + 1) * DK * DV + static_cast<size_t>(tid) * DV;
                const float *en = p.Er + eoff + static_cast<size_t>(tid) * DV;
#pragma unroll 16
                for (int d = 0; d < DV; ++d) o += en[d] * sn[d];
            }
            sacc[tid] = o;
        }
        for (int64_t ti = ntiles - 1; ti >= 0; --ti) {
            const int64_t tb = cp.t0 + ti * TILE;
            const int nt = static_cast<int>((cp.t1 - tb < TILE) ? cp.t1 - tb : TILE);
            load_tile(tb, nt);
            for (int tt = nt - 1; tt >= 0; --tt) {
                const float qc = sq[tt][Sh::pc(c)];
                float dd[PER], vv[PER];
                lds_vec<PER>(&sdo[tt][j0 * PER], dd);
                lds_vec<PER>(&sv[tt][j0 * PER], vv);
                float part = 0.f;
#pragma unroll
                for (int m = 0; m < PER; ++m) {
                    s[m] = gnext * s[m] + qc * dd[m];
                    part += s[m] * vv[m];
                }
                gnext = sg[tt][Sh::pc(c)];
                red[tt][j0][c] = part;
            }
            __syncthreads();
            // dk, then the in-chunk reverse cumulative sum of q dq - k dk (thread c < DK
            // walks the tile's tokens last to first)
            for (int i = tid; i < nt * DK; i += NT) {
                const int tt = i / DK, cc = i % DK;
                float d = 0.f;
#pragma unroll
                for (int r = 0; r < JSTEP; ++r) d += red[tt][r][cc];
                st<DT>(p.dk, srow[tt] * DK + cc, d);
                red[tt][0][cc] = d;  // reuse: dk of (tt, cc)
            }
            __syncthreads();
            if (tid < DK) {
                float acc = sacc[tid];
                for (int tt = nt - 1; tt >= 0; --tt) {
                    const int64_t r = srow[tt] * DK + tid;
                    acc += p.qdq[r] - sk[tt][Sh::pc(tid)] * red[tt][0][tid];
                    p.dlog_g[r] = acc;
                }
                sacc[tid] = acc;
            }
        }
        __syncthreads();
        // chunk totals for the fp32 path's offset pass (the OFFSET path has none, and
        // there Tn holds the ranges' drms_w sums)
        if (!OFFSET && tid < DK) p.Tn[cp.cid() * DK + tid] = sacc[tid];
    }

    // ---- pass B, map A: dv_t = dS_t^T k_t
    {
        const int j = tid % DV, c0 = tid / DV;
        float s[PER], gnext[PER];
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            s[m] = p.Er[eoff + static_cast<size_t>(c0 + CSTEP * m) * DV + j];
            gnext[m] = 1.f;
        }
        for (int64_t ti = ntiles - 1; ti >= 0; --ti) {
            const int64_t tb = cp.t0 + ti * TILE;
            const int nt = static_cast<int>((cp.t1 - tb < TILE) ? cp.t1 - tb : TILE);
            load_tile(tb, nt);
            for (int tt = nt - 1; tt >= 0; --tt) {
                const float dj = sdo[tt][Sh::pj(j)];
                float qq[PER], kk[PER];
                lds_vec<PER>(&sq[tt][c0 * PER], qq);
                lds_vec<PER>(&sk[tt][c0 * PER], kk);
                float part = 0.f;
#pragma unroll
                for (int m = 0; m < PER; ++m) {
                    s[m] = gnext[m] * s[m] + qq[m] * dj;
                    part += s[m] * kk[m];
                }
                lds_vec<PER>(&sg[tt][c0 * PER], gnext);
                red[tt][c0][j] = part;
            }
            __syncthreads();
            for (int i = tid; i < nt * DV; i += NT) {
                const int tt = i / DV, jj = i % DV;
                float d = 0.f;
#pragma unroll
                for (int r = 0; r < CSTEP; ++r) d += red[tt][r][jj];
                st<DT>(p.dv, srow[tt] * DV + jj, d);
            }
        }
    }
}

// Kernels of the fp32 path: one workgroup per chunk.
template <int DT, int DK, int DV>
__global__ __launch_bounds__(NT) void k_bwd_fwdwalk(BwdArgs p) {
    fwdwalk_body<DT, DK, DV, 0>(p, ChunkPos(p.a, p.n_chunks, blockIdx.x));
}
template <int DT, int DK, int DV>
__global__ __launch_bounds__(NT) void k_bwd_revsum(BwdArgs p) {
    revsum_body<DT, DK, DV>(p, ChunkPos(p.a, p.n_chunks, blockIdx.x));
}
template <int DT, int DK, int DV>
__global__ __launch_bounds__(NT) void k_bwd_revwalk(BwdArgs p) {
    revwalk_body<DT, DK, DV, false>(p, ChunkPos(p.a, p.n_chunks, blockIdx.x));
}

// Token-serial fallback of the matrix-core path for the chunks it flagged, by the
// matrix-core kernels' ranges (workgroup b: chunks [b R, b R + R), in order).
// PHASE 1 (after the epilogue kernel): dO, dz, drms_w partials, then the reverse
// summary (from the dO just written); range b's drms_w sum (the epilogue
// kernel's, over its unflagged chunks, in wr[b]) gains its flagged chunks'
// partials in order.  PHASE 2 (after the gradient kernel): dq and q dq, then dk,
// dv and the complete dlog_g; workgroup 0 also adds the ranges' sums in order
// into drms_w.
template <int DT, int DK, int DV, int PHASE>
__global__ __launch_bounds__(NT) void k_bwd_fallback(BwdArgs p, int64_t R, float *wr) {
    __shared__ int sflag[64];
    const int tid = threadIdx.x;
    const int64_t total = static_cast<int64_t>(p.a.B) * p.a.H * p.n_chunks;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * R;
    const int64_t c1 = (c0 + R < total) ? c0 + R : total;
    float wacc = 0.f;  // PHASE 1, thread tid < DV: the flagged chunks' drms_w partials
    for (int64_t b0 = c0; b0 < c1; b0 += 64) {
        __syncthreads();
        if (tid < 64) sflag[tid] = (b0 + tid < c1) ? p.flags[b0 + tid] : 0;
        __syncthreads();
        for (int k = 0; k < 64 && b0 + k < c1; ++k) {
            if (sflag[k] == 0) continue;  // uniform: one LDS value
            const ChunkPos cp(p.a, p.n_chunks, b0 + k);
            if constexpr (PHASE == 1) {
                fwdwalk_body<DT, DK, DV, 1>(p, cp);
                __syncthreads();  // dO and the drms_w partial of this chunk are in global memory
                revsum_body<DT, DK, DV>(p, cp);
                if (tid < DV) wacc += p.dWp[cp.cid() * DV + tid];
            } else {
                fwdwalk_body<DT, DK, DV, 2>(p, cp);
                __syncthreads();  // q dq of this chunk is in global memory
                revwalk_body<DT, DK, DV, true>(p, cp);
            }
            __syncthreads();
        }
    }
    if constexpr (PHASE == 1) {
        if (tid < DV && wacc != 0.f) wr[static_cast<int64_t>(blockIdx.x) * DV + tid] += wacc;
    } else if (blockIdx.x == 0) {
        // drms_w = the ranges' sums in order (complete: phase 1 ran before); NT / DV
        // groups of threads take consecutive parts (16 loads in flight each), then
        // the groups' sums in order
        __shared__ float part[NT];
        constexpr int GS = NT / DV;
        const int j = tid % DV, gq = tid / DV;
        const int64_t nr = (total + R - 1) / R;
        const int64_t per = (nr + GS - 1) / GS;
        const int64_t r0 = gq * per, r1 = (r0 + per < nr) ? r0 + per : nr;
        float w = 0.f;
        for (int64_t b0 = r0; b0 < r1; b0 += 16) {
            float x[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) x[u] = (b0 + u < r1) ? wr[(b0 + u) * DV + j] : 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) w += x[u];
        }
        __syncthreads();
        part[tid] = w;
        __syncthreads();
        if (tid < DV) {
            float x = 0.f;
            for (int r = 0; r < GS; ++r) x += part[r * DV + tid];
            p.drms_w[tid] = x;
        }
    }
}

// ---- B4a: Tn[n] <- sum of the totals of the sequence's later chunks (exclusive
// reverse scan, in place).  Thread = (sequence, channel); the loads of 16 chunks
// are issued before their sums.
__global__ __launch_bounds__(NT) void k_bwd_gatescan(float *__restrict__ Tn, int n_seq,
                                                     int n_chunks, int dk) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x;
    if (i >= static_cast<int64_t>(n_seq) * dk) return;
    const int64_t seq = i / dk;
    const int c = static_cast<int>(i % dk);
    float *t = Tn + seq * n_chunks * dk + c;
    float acc = 0.f;
    for (int n1 = n_chunks; n1 > 0; n1 -= 16) {
        const int n0 = n1 - 16 > 0 ? n1 - 16 : 0;
        float x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) x[u] = (n0 + u < n1) ? t[static_cast<int64_t>(n0 + u) * dk] : 0.f;
#pragma unroll
        for (int u = 15; u >= 0; --u) {
            if (n0 + u < n1) {
                t[static_cast<int64_t>(n0 + u) * dk] = acc;
                acc += x[u];
            }
        }
    }
}

// ---- B4b: dlog_g of chunk n += the scanned totals of the later chunks.
template <int DK>
__global__ __launch_bounds__(NT) void k_bwd_gateoff(BwdArgs p) {
    const GlaArgs &a = p.a;
    __shared__ __attribute__((aligned(16))) float soff[DK];
    const int tid = threadIdx.x;
    const ChunkPos cp(a, p.n_chunks, blockIdx.x);
    if (tid < DK) soff[tid] = p.Tn[cp.cid() * DK + tid];
    __syncthreads();
    const int64_t len = cp.t1 - cp.t0;
    for (int64_t i = tid; i < len * DK; i += NT) {
        const int64_t tt = i / DK;
        const int c = static_cast<int>(i % DK);
        const int64_t r = scan_row(a, cp.b, cp.h, cp.t0 + tt) * DK + c;
        p.dlog_g[r] += soff[c];
    }
}

// ---- B5: drms_w = sum of the per-chunk partials in a fixed order, two levels:
// block b sums parts [b R, (b + 1) R) (256 threads: 256 / DV row groups of each
// column, 8 loads in flight each, then the groups in order) into part2[b]; the
// block that finishes last (device counter) adds part2[0 ..] in order and resets
// the counter to zero for the next call.
constexpr int WS_BLOCKS = 64;
template <int DV>
__global__ __launch_bounds__(NT) void k_bwd_wsum(BwdArgs p, int64_t n_parts, float *part2,
                                                 unsigned *ctr) {
    __shared__ float part[NT];
    __shared__ bool last;
    const int tid = threadIdx.x;
    const int j = tid % DV, g = tid / DV;
    constexpr int GS = NT / DV;
    const int64_t R = (n_parts + gridDim.x - 1) / gridDim.x;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * R;
    const int64_t r1 = (r0 + R < n_parts) ? r0 + R : n_parts;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t rb = r0 + g; rb < r1; rb += 8 * GS) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t r = rb + static_cast<int64_t>(u) * GS;
            acc[u] += (r < r1) ? p.dWp[r * DV + j] : 0.f;
        }
    }
    part[tid] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    __syncthreads();
    if (tid < DV) {
        float w = 0.f;
        for (int r = 0; r < GS; ++r) w += part[r * DV + tid];
        part2[static_cast<int64_t>(blockIdx.x) * DV + tid] = w;
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) last = atomicAdd(ctr, 1u) == gridDim.x - 1;
    __syncthreads();
    if (!last) return;
    __threadfence();
    if (tid < DV) {  // in block order, 16 loads in flight
        float w = 0.f;
        for (unsigned b0 = 0; b0 < gridDim.x; b0 += 16) {
            float x[16];
#pragma unroll
            for (unsigned u = 0; u < 16; ++u)
                x[u] = (b0 + u < gridDim.x) ? part2[static_cast<int64_t>(b0 + u) * DV + tid] : 0.f;
#pragma unroll
            for (unsigned u = 0; u < 16; ++u) w += x[u];
        }
        p.drms_w[tid] = w;
    }
    if (tid == 0) atomicExch(ctr, 0u);
}

template <int DT, int DK, int DV>
hipError_t run_shape(const BwdArgs &p, bool mfma, const MfmaPlan &ps, const float *Useg,
                     hipStream_t st, const BwdLaunchHooks &hooks, int *flags) {
    const int64_t ncb = static_cast<int64_t>(p.a.B) * p.a.H * p.n_chunks;
    const dim3 grid(static_cast<unsigned>(ncb));
    // chunks per workgroup of the matrix-core kernels: whole segments of ps, about
    // one workgroup per CU (their LDS allows one)
    const int64_t per = (ps.n_wg + kBwdWorkgroups / 2) / kBwdWorkgroups;
    const int64_t R = ps.Q * (per > 1 ? per : 1);
    const dim3 ranges(static_cast<unsigned>(mfma ? (ncb + R - 1) / R : 1));
    auto done = [&]() {
        const hipError_t e = hipGetLastError();
        return e != hipSuccess ? e : hooks.after(st);
    };
    BwdArgs q = p;
    q.flags = flags;
    hipError_t e;
    if (mfma) {
        // the epilogue backward and the reverse summaries, the forward state carried
        // through each segment of ps from Useg (stored for the flagged chunks only)
        // (p.Tn, unused on this path, holds the ranges' drms_w sums)
        e = bdo_launch(p.a, ps, R, p.dy, Useg, const_cast<float *>(p.Sx), p.dO, p.dz, p.Tn, p.Ur,
                       p.Gr, flags, p.n_chunks, st);
        if (e != hipSuccess || (e = hooks.after(st)) != hipSuccess) return e;
        // chunks out of the matrix path's exponent range: token-serial dO and summaries
        hipLaunchKernelGGL((k_bwd_fallback<DT, DK, DV, 1>), ranges, dim3(NT), 0, st, q, R, p.Tn);
    } else {
        hipLaunchKernelGGL((k_bwd_fwdwalk<DT, DK, DV>), grid, dim3(NT), 0, st, p);
        if ((e = done()) != hipSuccess) return e;
        hipLaunchKernelGGL((k_bwd_revsum<DT, DK, DV>), grid, dim3(NT), 0, st, p);
    }
    if ((e = done()) != hipSuccess) return e;
    e = state_scan(p.Ur, p.Gr, static_cast<int>(p.a.B * p.a.H), p.n_chunks, DK, DV, st, true);
    if (e != hipSuccess || (e = hooks.after(st)) != hipSuccess) return e;
    q.Er = p.Ur;  // scanned in place
    if (mfma) {
        e = bgrad_launch(p.a, ps, R, p.dO, Useg, p.Sx, q.Er, p.dq, p.dk, p.dv, p.dlog_g, flags,
                         p.n_chunks, st);
        if (e != hipSuccess || (e = hooks.after(st)) != hipSuccess) return e;
        // chunks out of the matrix path's exponent range: token-serial gradients; drms_w
        hipLaunchKernelGGL((k_bwd_fallback<DT, DK, DV, 2>), ranges, dim3(NT), 0, st, q, R, p.Tn);
        return done();
    }
    hipLaunchKernelGGL((k_bwd_revwalk<DT, DK, DV>), grid, dim3(NT), 0, st, q);
    if ((e = done()) != hipSuccess) return e;
    // fp32 path: gate offsets across chunks, then drms_w
    const int64_t nsc = static_cast<int64_t>(p.a.B) * p.a.H * DK;
    hipLaunchKernelGGL(k_bwd_gatescan, dim3(static_cast<unsigned>((nsc + NT - 1) / NT)), dim3(NT), 0,
                       st, p.Tn, static_cast<int>(p.a.B * p.a.H), p.n_chunks, DK);
    if ((e = done()) != hipSuccess) return e;
    hipLaunchKernelGGL((k_bwd_gateoff<DK>), grid, dim3(NT), 0, st, q);
    if ((e = done()) != hipSuccess) return e;
    const int64_t nb = ncb < WS_BLOCKS ? ncb : WS_BLOCKS;
    hipLaunchKernelGGL((k_bwd_wsum<DV>), dim3(static_cast<unsigned>(nb)), dim3(NT), 0, st, q, ncb,
                       p.part2, p.ctr);
    return done();
}

template <int DT>
hipError_t run_dt(const BwdArgs &p, bool mfma, const MfmaPlan &ps, const float *Useg, hipStream_t st,
                  const BwdLaunchHooks &hooks, int *flags) {
#define GTR_BWD_CASE(DK_, DV_) \
    if (p.a.dk == DK_ && p.a.dv == DV_)                                      \
        return run_shape<DT, DK_, DV_>(p, mfma, ps, Useg, st, hooks, flags);
    GTR_BWD_CASE(32, 32) GTR_BWD_CASE(32, 64) GTR_BWD_CASE(32, 128)
    GTR_BWD_CASE(64, 32) GTR_BWD_CASE(64, 64) GTR_BWD_CASE(64, 128)
    GTR_BWD_CASE(128, 32) GTR_BWD_CASE(128, 64) GTR_BWD_CASE(128, 128)
#undef GTR_BWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace

size_t bwd_workspace_bytes(const GlaArgs &a, int n_chunks) {
    const size_t ncb = static_cast<size_t>(a.B) * a.H * n_chunks;
    const size_t rows = static_cast<size_t>(a.B) * a.L * a.H;
    return 4 * (2 * ncb * (static_cast<size_t>(a.dk) * a.dv + a.dk)  // forward and reverse states
                + rows * (a.dv + a.dk)                                // do, q dq
                + ncb * (a.dk + a.dv)                                 // chunk totals, drms_w parts
                + ncb                                                 // chunk flags
                + static_cast<size_t>(WS_BLOCKS) * a.dv               // drms_w block sums
                + ncb * (static_cast<size_t>(a.dk) * a.dv + a.dk));   // segment states (<= chunks)
}

hipError_t bwd_launch(const GlaArgs &a, const void *dy, void *dq, void *dk, void *dv,
                      float *dlog_g, void *dz, float *drms_w, void *ws, unsigned *ctr,
                      int n_chunks, int64_t chunks_per_wg, const float *fwd_states, hipStream_t st,
                      const BwdLaunchHooks &hooks) {
    const size_t ncb = static_cast<size_t>(a.B) * a.H * n_chunks;
    const size_t rows = static_cast<size_t>(a.B) * a.L * a.H;
    const size_t dd = static_cast<size_t>(a.dk) * a.dv;
    float *f = static_cast<float *>(ws);
    float *Uf = f, *Gf = Uf + ncb * dd, *Ur = Gf + ncb * a.dk, *Gr = Ur + ncb * dd;
    float *dO = Gr + ncb * a.dk, *qdq = dO + rows * a.dv, *Tn = qdq + rows * a.dk;
    float *dWp = Tn + ncb * a.dk;
    int *flags = reinterpret_cast<int *>(dWp + ncb * a.dv);
    float *part2 = reinterpret_cast<float *>(flags + ncb);
    float *Useg = part2 + static_cast<size_t>(WS_BLOCKS) * a.dv, *Gseg = Useg + ncb * dd;
    auto al16 = [](const void *x) { return (reinterpret_cast<uintptr_t>(x) & 15) == 0; };
    // matrix-core path where the shape allows (16-bit I/O, dk = dv = 64, chunk <= 64)
    const bool mfma = a.dtype != DT_F32 && a.dk == 64 && a.dv == 64 && bgrad_supported(a) &&
                      al16(dq) && al16(dk) && al16(dv) && al16(dz) && al16(dy) && al16(a.z) &&
                      al16(a.rms_w);
    // forward incoming states.  Matrix-core path: the forward path's segment
    // summaries (log2 gate totals) and scan where its kernel applies, else
    // per-chunk (one-chunk segments); the epilogue kernel carries the state
    // through each segment and writes every chunk's.  fp32 path: per-chunk
    // summaries and scan.
    MfmaPlan ps{};
    hipError_t e = hipSuccess;
    if (mfma) {
        const bool msum = sum_supported(a) && !a.feat && !a.resid && al16(a.k) && al16(a.v) &&
                          al16(a.log_g);
        if (msum) {
            MfmaPlan po;
            mfma_plans(a, chunks_per_wg, &ps, &po);  // the forward's segments
        } else {
            ps = mfma_plan(a, 1);
        }
        if (msum && fwd_states) {
            // the forward's segment states, given (gtr_gla_fwd_states): two launches fewer
            Useg = const_cast<float *>(fwd_states);
        } else {
            e = msum ? segment_summaries(a, ps, Useg, Gseg, st) : serial_summary(a, Useg, Gseg, n_chunks, st);
            if (e != hipSuccess || (e = hooks.after(st)) != hipSuccess) return e;
            e = msum ? state_scan_plan(Useg, Gseg, ps, static_cast<int>(a.B * a.H), a.dk, a.dv, st)
                     : state_scan(Useg, Gseg, static_cast<int>(a.B * a.H), n_chunks, a.dk, a.dv, st);
            if (e != hipSuccess || (e = hooks.after(st)) != hipSuccess) return e;
        }
    } else {
        e = serial_summary(a, Uf, Gf, n_chunks, st);
        if (e != hipSuccess || (e = hooks.after(st)) != hipSuccess) return e;
        e = state_scan(Uf, Gf, static_cast<int>(a.B * a.H), n_chunks, a.dk, a.dv, st);
        if (e != hipSuccess || (e = hooks.after(st)) != hipSuccess) return e;
    }
    BwdArgs p{a, dy, Uf, nullptr, dO, qdq, Ur, Gr, Tn, dWp, dq, dk, dv, dz, dlog_g, drms_w,
              nullptr, n_chunks, part2, ctr};
    switch (a.dtype) {
    case DT_F32: return run_dt<DT_F32>(p, false, ps, Useg, st, hooks, flags);
    case DT_F16: return run_dt<DT_F16>(p, mfma, ps, Useg, st, hooks, flags);
    case DT_BF16: return run_dt<DT_BF16>(p, mfma, ps, Useg, st, hooks, flags);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gtr
