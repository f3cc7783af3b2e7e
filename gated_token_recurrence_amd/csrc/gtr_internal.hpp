// gtr_internal.hpp -- shared declarations of libgtrscan's kernels and launchers.
//
// Device helpers here: I/O element loads and round-to-nearest-even stores,
// and the scan-order map of the four directions (GTR write-up
// "端侧实时感知新标杆！通用线性骨干网络GTR开源", Method §1: LR, RL, TB, BT, grid
// order restored after each block's scan).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gtrscan.h"

namespace gtr {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

struct GlaArgs {
    const void *q, *k, *v;
    const float *log_g;
    const void *z;
    const float *rms_w;
    void *out;
    const void *resid;  // previous block's output (stack residual) or nullptr
    int B, H, gh, gw, dk, dv, direction, chunk, dtype;
    int64_t L;
    // Low-rank gate (kernels that form log_g themselves; log_g is then unused):
    // feat [B L][rank] and gate_w [rank][H dk] of the I/O type, gate_b [H dk]
    // float32, log g = logsigmoid(feat . gate_w + gate_b) / tau.
    const void *feat = nullptr;
    const void *gate_w = nullptr;
    const float *gate_b = nullptr;
    float inv_tau = 1.f;
    int rank = 0;
};

// log(sigmoid(x)) = min(x, 0) - log(1 + exp(-|x|)) with the native base-2
// exponential and logarithm (1 + exp(-|x|) lies in [1, 2]: no overflow for
// either sign of x).
__device__ __forceinline__ float log_sigmoid(float x) {
    const float u = __builtin_amdgcn_exp2f(-fabsf(x) * 1.44269504088896340736f);
    return fminf(x, 0.f) - 0.69314718055994530942f * __builtin_amdgcn_logf(1.f + u);
}

// ------------------------------------------------------------ element I/O --
template <int DT> struct Elem;
template <> struct Elem<DT_F32> { using T = float; };
template <> struct Elem<DT_F16> { using T = _Float16; };
template <> struct Elem<DT_BF16> { using T = uint16_t; };  // bf16 bit pattern

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <int DT> __device__ __forceinline__ float ld(const void *p, int64_t i);
template <> __device__ __forceinline__ float ld<DT_F32>(const void *p, int64_t i) {
    return static_cast<const float *>(p)[i];
}
template <> __device__ __forceinline__ float ld<DT_F16>(const void *p, int64_t i) {
    return static_cast<float>(static_cast<const _Float16 *>(p)[i]);
}
template <> __device__ __forceinline__ float ld<DT_BF16>(const void *p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
}

template <int DT> __device__ __forceinline__ void st(void *p, int64_t i, float x);
template <> __device__ __forceinline__ void st<DT_F32>(void *p, int64_t i, float x) {
    static_cast<float *>(p)[i] = x;
}
template <> __device__ __forceinline__ void st<DT_F16>(void *p, int64_t i, float x) {
    static_cast<_Float16 *>(p)[i] = static_cast<_Float16>(x);  // RNE conversion
}
template <> __device__ __forceinline__ void st<DT_BF16>(void *p, int64_t i, float x) {
    static_cast<uint16_t *>(p)[i] = f32_to_bf16(x);
}

// Round a float to the I/O type and back (the stack residual add is rounded
// to the I/O type before use, as a stored tensor would be).
template <int DT> __device__ __forceinline__ float round_io(float x);
template <> __device__ __forceinline__ float round_io<DT_F32>(float x) { return x; }
template <> __device__ __forceinline__ float round_io<DT_F16>(float x) {
    return static_cast<float>(static_cast<_Float16>(x));
}
template <> __device__ __forceinline__ float round_io<DT_BF16>(float x) {
    return bf16_to_f32(f32_to_bf16(x));
}

// value input of one element: v, or round_io(v + resid) inside a stack
template <int DT>
__device__ __forceinline__ float ld_v(const GlaArgs &a, int64_t i) {
    float x = ld<DT>(a.v, i);
    if (a.resid) x = round_io<DT>(x + ld<DT>(a.resid, i));
    return x;
}

// ------------------------------------------------------------- scan order --
// Grid index p of scan step t (p = r * gw + c).
__device__ __forceinline__ int64_t scan_to_grid(int64_t t, int64_t L, int gh, int gw, int dir) {
    if (dir & 1) t = L - 1 - t;          // RL, BT: the reversed sequence
    if (dir < 2) return t;               // LR, RL: row-major raster
    int64_t c = t / gh, r = t - c * gh;  // TB, BT: column-major raster
    return r * gw + c;
}

// Row (token-head) index of scan step t for sequence (b, h).
__device__ __forceinline__ int64_t scan_row(const GlaArgs &a, int b, int h, int64_t t) {
    return (static_cast<int64_t>(b) * a.L + scan_to_grid(t, a.L, a.gh, a.gw, a.direction)) * a.H + h;
}

// --------------------------------------------------------------- launchers --
// Token-serial fp32 chunk path.
hipError_t serial_summary(const GlaArgs &a, float *U, float *G, int n_chunks, hipStream_t s);
hipError_t serial_output(const GlaArgs &a, const float *Sx, int n_chunks, hipStream_t s);
// Inter-chunk (or inter-segment) state scan, in place: U[n] <- S before unit n.
// G: summed gates of each unit, natural log (log2_gates: log2 units).
hipError_t state_scan(float *U, const float *G, int n_seq, int n_units, int dk, int dv,
                      hipStream_t s, bool log2_gates = false);
// MFMA chunk path.  The B*H*N chunks (N per sequence, sequence-major) are cut
// into ranges of Q chunks, one per workgroup; segments are the pieces of those
// ranges within one sequence.  Segment k starts at the k-th element of the
// sorted union of the multiples of N and of Q below T.
struct MfmaPlan {
    int64_t N;      // chunks per sequence
    int64_t T;      // chunks in total
    int64_t Q;      // chunks per workgroup range
    int64_t n_wg;   // workgroups
    int64_t lcm;    // lcm(N, Q)
    int64_t n_seg;  // segments
};
constexpr int64_t kMfmaWorkgroups = 512;      // output kernel: two per CU on 256 CUs
constexpr int64_t kSummaryWorkgroups = 512;   // summary kernel (finer ranges only lengthen the scan)

__host__ __device__ __forceinline__ int64_t seg_id(int64_t p, const MfmaPlan &pl) {
    if (p < (int64_t{1} << 31) && pl.lcm < (int64_t{1} << 31)) {  // every sum below 2^32
        const uint32_t u = static_cast<uint32_t>(p), n = static_cast<uint32_t>(pl.N),
                       q = static_cast<uint32_t>(pl.Q), m = static_cast<uint32_t>(pl.lcm);
        return static_cast<int64_t>((u + n - 1) / n + (u + q - 1) / q) - (u + m - 1) / m;
    }
    return (p + pl.N - 1) / pl.N + (p + pl.Q - 1) / pl.Q - (p + pl.lcm - 1) / pl.lcm;
}

bool mfma_supported(const GlaArgs &a);
MfmaPlan mfma_plan(const GlaArgs &a, int64_t chunks_per_wg);
// Plans of the summary kernel (ps: its ranges are the scan's segments) and of the
// output kernel (po: ranges of a whole number of ps ranges, so every po segment
// starts where a ps segment does).  chunks_per_wg > 0 forces both to that size.
void mfma_plans(const GlaArgs &a, int64_t chunks_per_wg, MfmaPlan *ps, MfmaPlan *po);
hipError_t mfma_summary(const GlaArgs &a, const MfmaPlan &ps, float *U, float *G, hipStream_t s);
// Sx: incoming state of every ps segment
hipError_t mfma_output(const GlaArgs &a, const MfmaPlan &po, const MfmaPlan &ps, const float *Sx,
                       hipStream_t s);
// Segment summaries with per-wave partial sums (k_sum.hip): 16-bit I/O, dk = 64,
// dv = 64, chunk 64.  Same plan and outputs as mfma_summary.
bool sum_supported(const GlaArgs &a);
hipError_t sum_launch(const GlaArgs &a, const MfmaPlan &ps, float *U, float *G, hipStream_t s);
// The segment summaries of plan ps on the matrix-core path (mfma_supported): the
// kernel above, or mfma_summary for short segments (same outputs).
hipError_t segment_summaries(const GlaArgs &a, const MfmaPlan &ps, float *U, float *G, hipStream_t s);
// Chunk outputs with token-row ownership per wave (k_rows.hip): 16-bit I/O,
// dk = 64, dv in {64, 128}, chunk 64.  Same plans and incoming states as mfma_output;
// or, with Gf (the summaries' summed log2-gates), Sx holds the segment summaries
// themselves and each workgroup folds its segment's incoming state from them.
bool rows_supported(const GlaArgs &a);
hipError_t rows_output(const GlaArgs &a, const MfmaPlan &po, const MfmaPlan &ps, const float *Sx,
                       const float *Gf, hipStream_t s);
// Single-launch path (one workgroup per chunk, chunks handed out by ticket).
int64_t fast_chunks(const GlaArgs &a);    // workgroups the launch needs
int64_t fast_counters(const GlaArgs &a);  // 32-bit counters the launch needs
bool fast_supported(const GlaArgs &a);    // shape has a kernel and <= 64 chunks per sequence
// U: [chunks][dk][dv] fp32; G: [chunks][dk]; cnt: fast_counters() words, zero before
// the first launch (each launch leaves them zero).
// spin_limit: polls of a wait for earlier chunks before it gives up (the chunk's
// incoming state is then NaN).
constexpr unsigned kFastSpinLimit = 1u << 24;  // far beyond any real wait
hipError_t fast_launch(const GlaArgs &a, float *U, float *G, unsigned *cnt, unsigned spin_limit,
                       hipStream_t s);
// Low-rank gate written out: log_g [B L][H dk] (float32) from a.feat, a.gate_w,
// a.gate_b, a.inv_tau, a.rank (k_gate.hip).
hipError_t gate_materialize(const GlaArgs &a, float *log_g, hipStream_t s);
// The summary and output kernels that form the gate from rank-16 features
// themselves (sum_launch / rows_output with a.feat set).
constexpr int kFusedGateRank = 16;
bool lowrank_fused_supported(const GlaArgs &a);
// Spatial SwiGLU middle (k_sswiglu.hip): m = SiLU(gate) * (depthwise k x k conv of
// value + bias) from u = [gate | value].
hipError_t sswiglu_launch(const void *u, const float *w, const float *b, void *m, int B, int gh,
                          int gw, int F, int k, int dtype, hipStream_t s);
// Backward pass (k_bwd.hip: pipeline and the fp32 token-serial kernels; k_bgrad.hip:
// the matrix-core kernels).  hooks.after() runs after every launch (event
// recording).  ws: bwd_workspace_bytes(a, n_chunks) bytes.
struct BwdLaunchHooks {
    hipError_t (*fn)(void *ctx, hipStream_t st) = nullptr;
    void *ctx = nullptr;
    hipError_t after(hipStream_t st) const { return fn ? fn(ctx, st) : hipSuccess; }
};
size_t bwd_workspace_bytes(const GlaArgs &a, int n_chunks);
// The matrix-core backward kernels' shape: 16-bit I/O, dk = dv = 64, chunk <= 64,
// 16-byte aligned q, k, v, log_g.
bool bgrad_supported(const GlaArgs &a);
// Matrix-core epilogue backward and reverse chunk summaries: workgroup b walks
// chunks [b R, b R + R) in order (R a multiple of pl.Q, so b R starts a segment
// of pl), carrying the forward state from that segment's incoming state
// (Sseg[seg_id(b R)]).  It writes dO, dz, Ur and Gr (log2), the drms_w sum over
// the range's unflagged chunks (wr[b]), the per-chunk flags (1: the decay span
// exceeds the matrix path's range; the token-serial kernels take the chunk), and
// the incoming state of each flagged chunk and of its successor to Sx.
hipError_t bdo_launch(const GlaArgs &a, const MfmaPlan &pl, int64_t R, const void *dy,
                      const float *Sseg, float *Sx, float *dO, void *dz, float *wr, float *Ur,
                      float *Gr, int *flags, int n_chunks, hipStream_t s);
// Matrix-core gradients (dq, dk, dv, complete dlog_g) of the chunks bdo_launch did
// not flag, the same walk with the same plan; Er: the scanned reverse states.
hipError_t bgrad_launch(const GlaArgs &a, const MfmaPlan &pl, int64_t R, const float *dO,
                        const float *Sseg, const float *Sx, const float *Er, void *dq, void *dk,
                        void *dv, float *dlog_g, const int *flags, int n_chunks, hipStream_t s);
hipError_t bwd_launch(const GlaArgs &a, const void *dy, void *dq, void *dk, void *dv,
                      float *dlog_g, void *dz, float *drms_w, void *ws, unsigned *ctr,
                      int n_chunks, int64_t chunks_per_wg, const float *fwd_states, hipStream_t st,
                      const BwdLaunchHooks &hooks);
// State scan over the segments of a plan, in place: U[k] <- state before segment k.
hipError_t state_scan_plan(float *U, const float *G, const MfmaPlan &pl, int n_seq, int dk,
                           int dv, hipStream_t s);

}  // namespace gtr
