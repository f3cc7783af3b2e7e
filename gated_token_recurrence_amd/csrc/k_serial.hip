// k_serial.hip -- fp32 chunk path: token-serial recurrence inside each chunk.
//
// Three phases as in the GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源",
// Method §4 "硬件感知分块推理算子"): (1) every chunk's summary, computed here by
// running the recurrence U = Diag(g_t) U + k_t v_t^T from U = 0 over the chunk,
// together with the chunk's total log-gate; (2) the boundary-state scan
// (k_scan.hip); (3) every chunk's outputs, re-running the recurrence from the
// chunk's incoming state and reading o_t = S_t^T q_t after each token, with
// RMSNorm, the SiLU(z) gate and the grid-order store fused after it
// (Method §1 gives the recurrence, the readout and the gating).
//
// All arithmetic is fp32; this path serves float32 I/O (where results must be
// fp32-accurate) and shapes the MFMA path does not cover.  The dk x dv state
// lives in registers: thread tid owns column j = tid % dv and channels
// c = tid / dv + (256 / dv) * m.  Tokens are staged through LDS in tiles.
#include "gtr_internal.hpp"

namespace gtr {
namespace {

constexpr int NT = 256;

template <int DT, int DK, int DV, bool OUTPUT>
__global__ __launch_bounds__(NT) void k_serial(GlaArgs a, float *__restrict__ U,
                                               float *__restrict__ G,
                                               const float *__restrict__ Sx, int n_chunks) {
    static_assert(NT % DV == 0 && NT % DK == 0, "head widths must divide the block");
    constexpr int PER = DK * DV / NT;     // state elements per thread
    constexpr int CSTEP = NT / DV;        // channel stride between them
    constexpr int TILE = (DK + DV > 128) ? 8 : 16;

    __shared__ float sk[TILE][DK], sg[TILE][DK], sv[TILE][DV];
    __shared__ float sq[OUTPUT ? TILE : 1][DK], sz[OUTPUT ? TILE : 1][DV];
    __shared__ float red[OUTPUT ? TILE : 1][CSTEP][DV];
    __shared__ float so[OUTPUT ? TILE : 1][DV];
    __shared__ float gpart[NT];
    __shared__ int64_t srow[TILE];

    const int tid = threadIdx.x;
    const int n = blockIdx.x % n_chunks;
    const int bh = blockIdx.x / n_chunks;
    const int b = bh / a.H, h = bh % a.H;
    const int j = tid % DV, c0 = tid / DV;
    const size_t soff = (static_cast<size_t>(bh) * n_chunks + n) * DK * DV;

    float s[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m)
        s[m] = OUTPUT ? Sx[soff + static_cast<size_t>(c0 + CSTEP * m) * DV + j] : 0.f;
    float gacc = 0.f;  // this thread's share of the chunk's summed log-gate, channel tid % DK

    const int64_t t0 = static_cast<int64_t>(n) * a.chunk;
    const int64_t t1 = (t0 + a.chunk < a.L) ? t0 + a.chunk : a.L;
    for (int64_t tb = t0; tb < t1; tb += TILE) {
        const int nt = static_cast<int>((t1 - tb < TILE) ? t1 - tb : TILE);
        __syncthreads();  // the previous tile is consumed
        if (tid < TILE) srow[tid] = tid < nt ? scan_row(a, b, h, tb + tid) : 0;
        __syncthreads();
        for (int i = tid; i < TILE * DK; i += NT) {
            const int tt = i / DK, c = i % DK;
            float kk = 0.f, lg = 0.f, qq = 0.f;
            if (tt < nt) {
                const int64_t r = srow[tt] * DK + c;
                kk = ld<DT>(a.k, r);
                lg = a.log_g[r];
                if (OUTPUT) qq = ld<DT>(a.q, r);
            }
            sk[tt][c] = kk;
            sg[tt][c] = expf(lg);
            gacc += lg;
            if (OUTPUT) sq[tt][c] = qq;
        }
        for (int i = tid; i < TILE * DV; i += NT) {
            const int tt = i / DV, jj = i % DV;
            float vv = 0.f, zz = 0.f;
            if (tt < nt) {
                const int64_t r = srow[tt] * DV + jj;
                vv = ld_v<DT>(a, r);
                if (OUTPUT) zz = ld<DT>(a.z, r);
            }
            sv[tt][jj] = vv;
            if (OUTPUT) sz[tt][jj] = zz;
        }
        __syncthreads();
        for (int tt = 0; tt < nt; ++tt) {
            const float vj = sv[tt][j];
            float part = 0.f;
#pragma unroll
            for (int m = 0; m < PER; ++m) {
                const int c = c0 + CSTEP * m;
                s[m] = sg[tt][c] * s[m] + sk[tt][c] * vj;   // S_t = Diag(g_t) S_{t-1} + k_t v_t^T
                if (OUTPUT) part += s[m] * sq[tt][c];       // o_t = S_t^T q_t (partial)
            }
            if (OUTPUT) red[tt][c0][j] = part;
        }
        if (OUTPUT) {
            __syncthreads();
            for (int i = tid; i < TILE * DV; i += NT) {
                const int tt = i / DV, jj = i % DV;
                float o = 0.f;
#pragma unroll
                for (int r = 0; r < CSTEP; ++r) o += red[tt][r][jj];
                so[tt][jj] = o;
            }
            __syncthreads();
            for (int i = tid; i < nt * DV; i += NT) {
                const int tt = i / DV, jj = i % DV;
                float ss = 0.f;
                for (int x = 0; x < DV; ++x) ss += so[tt][x] * so[tt][x];
                const float inv = 1.0f / sqrtf(ss / DV + GTR_RMS_EPS);
                const float zz = sz[tt][jj];
                const float y = so[tt][jj] * inv * a.rms_w[jj] * (zz / (1.0f + expf(-zz)));
                st<DT>(a.out, srow[tt] * DV + jj, y);
            }
        }
    }
    if (!OUTPUT) {
#pragma unroll
        for (int m = 0; m < PER; ++m) U[soff + static_cast<size_t>(c0 + CSTEP * m) * DV + j] = s[m];
        gpart[tid] = gacc;
        __syncthreads();
        if (tid < DK) {
            float g = 0.f;
            for (int r = tid; r < NT; r += DK) g += gpart[r];
            G[(static_cast<size_t>(bh) * n_chunks + n) * DK + tid] = g;
        }
    }
}

template <int DT, bool OUTPUT>
hipError_t launch(const GlaArgs &a, float *U, float *G, const float *Sx, int n_chunks,
                  hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.H * n_chunks));
#define GTR_SERIAL_CASE(DK_, DV_)                                                        \
    if (a.dk == DK_ && a.dv == DV_) {                                                    \
        hipLaunchKernelGGL((k_serial<DT, DK_, DV_, OUTPUT>), grid, dim3(NT), 0, st, a, U, G, \
                           Sx, n_chunks);                                               \
        return hipGetLastError();                                                        \
    }
    GTR_SERIAL_CASE(32, 32) GTR_SERIAL_CASE(32, 64) GTR_SERIAL_CASE(32, 128)
    GTR_SERIAL_CASE(64, 32) GTR_SERIAL_CASE(64, 64) GTR_SERIAL_CASE(64, 128)
    GTR_SERIAL_CASE(128, 32) GTR_SERIAL_CASE(128, 64) GTR_SERIAL_CASE(128, 128)
#undef GTR_SERIAL_CASE
    return hipErrorInvalidValue;
}

template <bool OUTPUT>
hipError_t dispatch(const GlaArgs &a, float *U, float *G, const float *Sx, int n_chunks,
                    hipStream_t st) {
    switch (a.dtype) {
    case DT_F32: return launch<DT_F32, OUTPUT>(a, U, G, Sx, n_chunks, st);
    case DT_F16: return launch<DT_F16, OUTPUT>(a, U, G, Sx, n_chunks, st);
    case DT_BF16: return launch<DT_BF16, OUTPUT>(a, U, G, Sx, n_chunks, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t serial_summary(const GlaArgs &a, float *U, float *G, int n_chunks, hipStream_t s) {
    return dispatch<false>(a, U, G, nullptr, n_chunks, s);
}

hipError_t serial_output(const GlaArgs &a, const float *Sx, int n_chunks, hipStream_t s) {
    return dispatch<true>(a, nullptr, nullptr, Sx, n_chunks, s);
}

}  // namespace gtr
