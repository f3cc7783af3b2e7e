// api.cpp -- libgtrscan's C ABI: argument checks, path choice, workspace, launches.
//
// The operation and the layouts are documented in include/gtrscan.h.  Every
// check runs on the host before anything is enqueued; device data (NaN, Inf,
// positive log-gates) is not inspected.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "gtr_internal.hpp"
#include "gtrscan.h"

using namespace gtr;

namespace {

thread_local std::string g_err;

gtr_status fail(gtr_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

gtr_status hip_fail(hipError_t e, const char *what) {
    return fail(GTR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------- workspace --
// Grow-only device buffer per (device, stream).  Growing synchronises the
// stream first, because queued kernels may still use the old buffer.
struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
// log_g written out by the low-rank gate kernel (kept apart from the states)
std::map<std::pair<int, hipStream_t>, Workspace> g_gws;

// A stream under graph capture cannot synchronise, free or allocate: a buffer that
// would have to be created or grown then is refused with a clear error instead of
// invalidating the capture.  (Work captured into a graph keeps the buffer's address,
// so the buffer must not change while such a graph may still be replayed.)
gtr_status no_growth_while_capturing(hipStream_t stream, const char *what) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
        return fail(GTR_ERR_UNSUPPORTED,
                    "the %s would have to grow while the stream is being captured; make the same "
                    "call once on this stream before capturing",
                    what);
    return GTR_OK;
}

gtr_status workspace(hipStream_t stream, size_t bytes, void **out,
                     std::map<std::pair<int, hipStream_t>, Workspace> &pool = g_ws) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_ws_mu);
    Workspace &w = pool[std::make_pair(dev, stream)];
    if (w.bytes < bytes) {
        gtr_status cs = no_growth_while_capturing(stream, "workspace");
        if (cs != GTR_OK) return cs;
        if (w.ptr) {
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
            e = hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
            if (e != hipSuccess) return hip_fail(e, "hipFree");
        }
        size_t want = bytes + bytes / 4;  // headroom against repeated small growth
        e = hipMalloc(&w.ptr, want);
        if (e != hipSuccess) {
            w.ptr = nullptr;
            return hip_fail(e, "hipMalloc(workspace)");
        }
        w.bytes = want;
    }
    *out = w.ptr;
    return GTR_OK;
}

// Zero-initialised counters of the single-launch path, per (device, stream).
// Every launch leaves them zero; growing synchronises the stream first.
std::map<std::pair<int, hipStream_t>, Workspace> g_ctr;

gtr_status counters(hipStream_t stream, size_t n, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_ws_mu);
    Workspace &w = g_ctr[std::make_pair(dev, stream)];
    const size_t bytes = n * sizeof(unsigned);
    if (w.bytes < bytes) {
        gtr_status cs = no_growth_while_capturing(stream, "counter block");
        if (cs != GTR_OK) return cs;
        if (w.ptr) {
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
            e = hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
            if (e != hipSuccess) return hip_fail(e, "hipFree");
        }
        e = hipMalloc(&w.ptr, bytes);
        if (e != hipSuccess) {
            w.ptr = nullptr;
            return hip_fail(e, "hipMalloc(counters)");
        }
        e = hipMemset(w.ptr, 0, bytes);
        if (e != hipSuccess) return hip_fail(e, "hipMemset(counters)");
        w.bytes = bytes;
    }
    *out = w.ptr;
    return GTR_OK;
}

// --------------------------------------------------------------- validation --
bool head_width_ok(int d) { return d == 32 || d == 64 || d == 128; }

gtr_status check(const void *q, const void *k, const void *v, const float *log_g,
                 const void *z, const float *rms_w, const void *out, int B, int H, int gh,
                 int gw, int dk, int dv, int direction, int chunk, int dtype, int path) {
    if (!q || !k || !v || !log_g || !z || !rms_w || !out)
        return fail(GTR_ERR_ARG, "null tensor pointer");
    if (B <= 0 || H <= 0 || gh <= 0 || gw <= 0)
        return fail(GTR_ERR_ARG, "B, H, grid_h, grid_w must be positive (got %d, %d, %d, %d)",
                    B, H, gh, gw);
    if (direction < 0 || direction > 3)
        return fail(GTR_ERR_ARG, "direction must be 0..3 (LR, RL, TB, BT), got %d", direction);
    if (!(chunk == 0 || chunk == 16 || chunk == 32 || chunk == 64 || chunk == 128))
        return fail(GTR_ERR_ARG, "chunk must be 0, 16, 32, 64 or 128, got %d", chunk);
    if (static_cast<int64_t>(gh) * gw >= (static_cast<int64_t>(1) << 31))
        return fail(GTR_ERR_UNSUPPORTED, "grid_h * grid_w must be below 2^31 tokens");
    if (dtype < GTR_F32 || dtype > GTR_BF16)
        return fail(GTR_ERR_ARG, "unknown dtype %d", dtype);
    if (path < GTR_PATH_AUTO || path > GTR_PATH_SERIAL)
        return fail(GTR_ERR_ARG, "unknown path %d", path);
    if (!head_width_ok(dk) || !head_width_ok(dv))
        return fail(GTR_ERR_UNSUPPORTED, "dk and dv must be 32, 64 or 128 (got %d, %d)", dk, dv);
    const uintptr_t eb = dtype == GTR_F32 ? 4 : 2;
    for (const void *p : {q, k, v, z, static_cast<const void *>(out)})
        if (reinterpret_cast<uintptr_t>(p) % eb != 0)
            return fail(GTR_ERR_ARG, "q, k, v, z and out must be aligned to their element size");
    if (reinterpret_cast<uintptr_t>(log_g) % 4 != 0 || reinterpret_cast<uintptr_t>(rms_w) % 4 != 0)
        return fail(GTR_ERR_ARG, "log_g and rms_w must be 4-byte aligned");
    const __int128 rows = static_cast<__int128>(B) * gh * gw * H;
    if (rows * (dk > dv ? dk : dv) * 4 > (static_cast<__int128>(1) << 62) ||
        static_cast<int64_t>(gh) * gw > (static_cast<int64_t>(1) << 40))
        return fail(GTR_ERR_UNSUPPORTED, "tensor sizes overflow 64-bit offsets");
    return GTR_OK;
}

gtr_status check_aliasing(const void *out, size_t out_bytes, const void *const *ins,
                          const size_t *in_bytes, int n) {
    const char *o0 = static_cast<const char *>(out), *o1 = o0 + out_bytes;
    for (int i = 0; i < n; ++i) {
        const char *a0 = static_cast<const char *>(ins[i]), *a1 = a0 + in_bytes[i];
        if (a0 < o1 && o0 < a1) return fail(GTR_ERR_ARG, "out overlaps input %d", i);
    }
    return GTR_OK;
}

size_t elem_bytes(int dtype) { return dtype == GTR_F32 ? 4 : 2; }

// Records events around launches when the caller asked for them.
struct Marks {
    hipEvent_t *ev = nullptr;
    int n = 0;
    int launches = 0;
    hipError_t record(hipStream_t st, int i) {
        return (ev && i < n) ? hipEventRecord(ev[i], st) : hipSuccess;
    }
    hipError_t after_launch(hipStream_t st) { return record(st, ++launches); }
    // event 0, unless an earlier launch of the call already recorded it
    hipError_t start(hipStream_t st) { return launches == 0 ? record(st, 0) : hipSuccess; }
};

// Where a run's workspace comes from: the library's grow-only buffer (ptr null) or
// a fixed region that must already be large enough (the no-allocation entry point).
struct WsSource {
    void *ptr = nullptr;
    size_t bytes = 0;
};

gtr_status take_workspace(hipStream_t st, size_t need, const WsSource *src, void **out) {
    if (!src || !src->ptr) return workspace(st, need, out);
    if (need > src->bytes)
        return fail(GTR_ERR_UNSUPPORTED,
                    "this call needs %zu bytes of scratch; the fixed scratch holds %zu", need,
                    src->bytes);
    *out = src->ptr;
    return GTR_OK;
}

constexpr int kDefaultChunk = 64;
constexpr int kFastMaxTokens = 2048;
// Sequences of at most this many segments skip the scan launch: their output kernel
// folds the incoming states itself (the scan then costs a launch and its drain, ~11 us
// on MI355X for the 12-block stack's blocks, against a few loads per workgroup).
constexpr int64_t kFoldSegments = 8;

int g_chunks_per_wg = 0;  // 0: automatic (gtr_set_segment_chunks)
unsigned g_fast_spin_limit = kFastSpinLimit;  // gtr_set_wait_limit

gtr_status run_serial(const GlaArgs &a, hipStream_t st, Marks &mk, const WsSource *src = nullptr) {
    const int64_t n_chunks = (a.L + a.chunk - 1) / a.chunk;
    const int64_t n_seq = static_cast<int64_t>(a.B) * a.H;
    if (n_seq * n_chunks > 0x7fffffff) return fail(GTR_ERR_UNSUPPORTED, "too many chunks");
    const size_t ubytes = static_cast<size_t>(n_seq * n_chunks) * a.dk * a.dv * 4;
    const size_t gbytes = static_cast<size_t>(n_seq * n_chunks) * a.dk * 4;
    void *ws = nullptr;
    gtr_status s = take_workspace(st, ubytes + gbytes, src, &ws);
    if (s != GTR_OK) return s;
    float *U = static_cast<float *>(ws);
    float *G = reinterpret_cast<float *>(static_cast<char *>(ws) + ubytes);
    hipError_t e = mk.start(st);
    if (e == hipSuccess) e = serial_summary(a, U, G, static_cast<int>(n_chunks), st);
    if (e == hipSuccess) e = mk.after_launch(st);
    if (e != hipSuccess) return hip_fail(e, "chunk summary launch");
    e = state_scan(U, G, static_cast<int>(n_seq), static_cast<int>(n_chunks), a.dk, a.dv, st);
    if (e == hipSuccess) e = mk.after_launch(st);
    if (e != hipSuccess) return hip_fail(e, "state scan launch");
    e = serial_output(a, U, static_cast<int>(n_chunks), st);
    if (e == hipSuccess) e = mk.after_launch(st);
    if (e != hipSuccess) return hip_fail(e, "chunk output launch");
    return GTR_OK;
}

// states_out: where the segment states go (the caller's buffer of gtr_gla_fwd_states),
// else the workspace
gtr_status run_mfma(const GlaArgs &a, hipStream_t st, Marks &mk, float *states_out = nullptr,
                    const WsSource *src = nullptr) {
    MfmaPlan pl, po;
    mfma_plans(a, g_chunks_per_wg, &pl, &po);
    const int64_t n_seq = static_cast<int64_t>(a.B) * a.H;
    if (pl.n_wg > 0x7fffffff || n_seq * a.dk * a.dv > 0x7fffffff)
        return fail(GTR_ERR_UNSUPPORTED, "too many chunks");
    const size_t ubytes = states_out ? 0 : static_cast<size_t>(pl.n_seg) * a.dk * a.dv * 4;
    const size_t gbytes = static_cast<size_t>(pl.n_seg) * a.dk * 4;
    void *ws = nullptr;
    gtr_status s = take_workspace(st, ubytes + gbytes, src, &ws);
    if (s != GTR_OK) return s;
    float *U = states_out ? states_out : static_cast<float *>(ws);
    float *G = reinterpret_cast<float *>(static_cast<char *>(ws) + ubytes);
    hipError_t e = mk.start(st);
    if (e == hipSuccess) e = segment_summaries(a, pl, U, G, st);
    if (e == hipSuccess) e = mk.after_launch(st);
    if (e != hipSuccess) return hip_fail(e, "segment summary launch");
    // With few segments per sequence the output kernel folds each segment's incoming
    // state from the summaries itself (at most kFoldSegments - 1 of them, the same
    // arithmetic in the same order as the scan) and the scan launch is left out; the
    // caller's states buffer always gets the scanned states.
    const int64_t most = (pl.N + pl.Q - 1) / pl.Q + 1;  // segments of one sequence, at most
    const bool fold = !states_out && rows_supported(a) && most <= kFoldSegments;
    if (!fold) {
        e = state_scan_plan(U, G, pl, static_cast<int>(n_seq), a.dk, a.dv, st);
        if (e == hipSuccess) e = mk.after_launch(st);
        if (e != hipSuccess) return hip_fail(e, "state scan launch");
    }
    e = rows_supported(a) ? rows_output(a, po, pl, U, fold ? G : nullptr, st)
                          : mfma_output(a, po, pl, U, st);
    if (e == hipSuccess) e = mk.after_launch(st);
    if (e != hipSuccess) return hip_fail(e, "chunk output launch");
    return GTR_OK;
}

}  // namespace

// The summary and output kernels form the gate themselves for rank-16 features
// at their one shape (16-bit I/O, dk = dv = 64, chunk 64), without a residual.
bool gtr::lowrank_fused_supported(const GlaArgs &a) {
    return a.feat && a.rank == kFusedGateRank && !a.resid && a.dtype != GTR_F32 &&
           mfma_supported(a) && sum_supported(a) && rows_supported(a) && a.dv == 64;
}

namespace {

// The matrix-core and single-launch kernels move token rows in 16-byte pieces:
// every row pointer they touch must be 16-byte aligned (a contiguous view with a
// storage offset may not be).  Null pointers (log_g of a low-rank call, no
// residual) do not count.
bool vec16(const GlaArgs &a) {
    for (const void *p : {a.q, a.k, a.v, static_cast<const void *>(a.log_g), a.z,
                          static_cast<const void *>(a.out), a.resid})
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return false;
    return true;
}

bool mfma_ok(const GlaArgs &a) { return a.dtype != GTR_F32 && mfma_supported(a) && vec16(a); }

// The single-launch path: batch one, at most kFastMaxTokens tokens.
bool fast_ok(const GlaArgs &a) {
    if (!mfma_ok(a) || !fast_supported(a)) return false;
    return a.B == 1 && a.L <= kFastMaxTokens;
}

// AUTO takes the single-launch path for batch-one calls of at most kFastAutoChunks
// chunks per sequence (measured on MI355X with warmed-up calls, 6 and 16 heads: at
// chunk 64 it wins by 5-7 us at one chunk and by 1-3 us at 13 to 16, ties at 20 with
// 6 heads and loses from about 17 chunks with 16; at chunk 32 it wins by 1.5-3 us up
// to 8 chunks, about ties at 12 and loses at 16: each chunk's fold of every earlier
// chunk's summary dominates), the matrix-core path for the other 16-bit calls at its
// shapes with 16-byte aligned rows, and the token-serial path otherwise.
constexpr int64_t kFastAutoChunks = 16;    // chunk 64
constexpr int64_t kFastAutoChunks32 = 12;  // chunk 32

int auto_path(const GlaArgs &a) {
    const int64_t n_chunks = (a.L + a.chunk - 1) / a.chunk;
    const int64_t most = a.chunk == 32 ? kFastAutoChunks32 : kFastAutoChunks;
    if (!a.feat && !a.resid && fast_ok(a) && n_chunks <= most) return GTR_PATH_FAST;
    return mfma_ok(a) ? GTR_PATH_MFMA : GTR_PATH_SERIAL;
}

// Resolves AUTO and checks that an explicit path can take the arguments (before
// anything touches the device).
gtr_status resolve_path(const GlaArgs &a, int path, int *out) {
    if (path == GTR_PATH_AUTO) path = auto_path(a);
    if (path == GTR_PATH_MFMA && !mfma_ok(a))
        return fail(GTR_ERR_UNSUPPORTED,
                    "MFMA path needs 16-bit I/O, dk = 64, dv in {64, 128}, chunk in {32, 64} and "
                    "16-byte aligned tensors");
    if (path == GTR_PATH_FAST && !fast_ok(a))
        return fail(GTR_ERR_UNSUPPORTED,
                    "single-launch path needs 16-bit I/O, dk = 64, dv in {64, 128}, chunk in "
                    "{32, 64}, 16-byte aligned tensors, B = 1 and at most %d tokens",
                    kFastMaxTokens);
    *out = path;
    return GTR_OK;
}

gtr_status run_fast(const GlaArgs &a, hipStream_t st, Marks &mk) {
    const size_t T = static_cast<size_t>(fast_chunks(a));
    void *ws = nullptr, *ctr = nullptr;
    gtr_status s = workspace(st, T * a.dk * a.dv * 4 + T * a.dk * 4, &ws);
    if (s == GTR_OK) s = counters(st, static_cast<size_t>(fast_counters(a)), &ctr);
    if (s != GTR_OK) return s;
    float *U = static_cast<float *>(ws);
    float *G = U + T * a.dk * a.dv;
    hipError_t e = mk.start(st);
    if (e == hipSuccess) e = fast_launch(a, U, G, static_cast<unsigned *>(ctr), g_fast_spin_limit, st);
    if (e == hipSuccess) e = mk.after_launch(st);
    if (e != hipSuccess) return hip_fail(e, "single-launch kernel");
    return GTR_OK;
}

gtr_status run(const GlaArgs &a0, int path, hipStream_t st, Marks &mk) {
    GlaArgs a = a0;
    if (a.chunk == 0) a.chunk = kDefaultChunk;
    gtr_status s = resolve_path(a, path, &path);
    if (s != GTR_OK) return s;
    switch (path) {
    case GTR_PATH_SERIAL: return run_serial(a, st, mk);
    case GTR_PATH_MFMA: return run_mfma(a, st, mk);
    case GTR_PATH_FAST: return run_fast(a, st, mk);
    default: return fail(GTR_ERR_ARG, "unknown path %d", path);
    }
}

// Workspace bytes a run() of these arguments on this path needs (so that a caller
// issuing several runs can size it once, before the first launch).
size_t run_workspace_bytes(const GlaArgs &a0, int path) {
    GlaArgs a = a0;
    if (a.chunk == 0) a.chunk = kDefaultChunk;
    if (path == GTR_PATH_AUTO) path = auto_path(a);
    if (path == GTR_PATH_MFMA) {
        MfmaPlan pl, po;
        mfma_plans(a, g_chunks_per_wg, &pl, &po);
        return static_cast<size_t>(pl.n_seg) * a.dk * a.dv * 4 + static_cast<size_t>(pl.n_seg) * a.dk * 4;
    }
    if (path == GTR_PATH_FAST) {
        const size_t T = static_cast<size_t>(fast_chunks(a));
        return T * a.dk * a.dv * 4 + T * a.dk * 4;
    }
    const size_t n = static_cast<size_t>(a.B) * a.H * ((a.L + a.chunk - 1) / a.chunk);
    return n * a.dk * a.dv * 4 + n * a.dk * 4;
}

int device_ok() {
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n <= 0) {
        fail(GTR_ERR_HIP, "no HIP device available (%s)",
             e != hipSuccess ? hipGetErrorString(e) : "device count is 0");
        return 0;
    }
    return 1;
}

gtr_status lowrank_impl(const void *q, const void *k, const void *v, const void *feat,
                        const void *gate_w, const float *gate_b, float tau, int rank,
                        const void *z, const float *rms_w, void *out, int B, int H, int gh,
                        int gw, int dk, int dv, int direction, int chunk, int dtype, int path,
                        hipStream_t stream, Marks &mk) {
    g_err.clear();
    if (!feat || !gate_w || !gate_b) return fail(GTR_ERR_ARG, "null gate pointer");
    gtr_status s = check(q, k, v, gate_b, z, rms_w, out, B, H, gh, gw, dk, dv, direction, chunk,
                         dtype, path);
    if (s != GTR_OK) return s;
    if (rank < 1 || rank > 256) return fail(GTR_ERR_ARG, "rank must be 1..256, got %d", rank);
    if (!(std::isfinite(tau) && tau > 0.f))
        return fail(GTR_ERR_ARG, "tau must be finite and positive, got %g", static_cast<double>(tau));
    for (const void *p : {feat, gate_w, static_cast<const void *>(gate_b)})
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(GTR_ERR_ARG, "feat, gate_w and gate_b must be 16-byte aligned");
    const size_t tokens = static_cast<size_t>(B) * gh * gw;
    const size_t rows = tokens * H;
    const size_t eb = elem_bytes(dtype);
    const size_t hd = static_cast<size_t>(H) * dk;
    const void *ins[] = {q, k, v, feat, gate_w, gate_b, z, rms_w};
    const size_t nb[] = {rows * dk * eb, rows * dk * eb, rows * dv * eb, tokens * rank * eb,
                         static_cast<size_t>(rank) * hd * eb, hd * 4, rows * dv * eb,
                         static_cast<size_t>(dv) * 4};
    s = check_aliasing(out, rows * dv * eb, ins, nb, 8);
    if (s != GTR_OK) return s;
    GlaArgs a{q, k, v, nullptr, z, rms_w, out, nullptr, B, H, gh, gw, dk, dv, direction,
              chunk ? chunk : kDefaultChunk, dtype, static_cast<int64_t>(gh) * gw};
    a.feat = feat;
    a.gate_w = gate_w;
    a.gate_b = gate_b;
    a.inv_tau = 1.f / tau;
    a.rank = rank;
    int p = path;
    s = resolve_path(a, path, &p);  // log_g is null here: the gate buffer is aligned
    if (s != GTR_OK) return s;
    if (!device_ok()) return GTR_ERR_HIP;
    if (p == GTR_PATH_MFMA && lowrank_fused_supported(a)) return run_mfma(a, stream, mk);
    // every other path reads log_g: write it out first
    void *lg = nullptr;
    s = workspace(stream, rows * dk * 4, &lg, g_gws);
    if (s != GTR_OK) return s;
    hipError_t e = mk.start(stream);
    if (e == hipSuccess) e = gate_materialize(a, static_cast<float *>(lg), stream);
    if (e == hipSuccess) e = mk.after_launch(stream);
    if (e != hipSuccess) return hip_fail(e, "gate projection launch");
    a.log_g = static_cast<const float *>(lg);
    a.feat = nullptr;
    return run(a, p, stream, mk);
}

gtr_status fwd_impl(const void *q, const void *k, const void *v, const float *log_g,
                    const void *z, const float *rms_w, void *out, const void *resid, int B,
                    int H, int gh, int gw, int dk, int dv, int direction, int chunk, int dtype,
                    int path, hipStream_t stream, Marks &mk) {
    g_err.clear();
    gtr_status s = check(q, k, v, log_g, z, rms_w, out, B, H, gh, gw, dk, dv, direction, chunk,
                         dtype, path);
    if (s != GTR_OK) return s;
    const size_t rows = static_cast<size_t>(B) * gh * gw * H;
    const size_t eb = elem_bytes(dtype);
    const void *ins[] = {q, k, v, log_g, z, rms_w, resid ? resid : q};
    const size_t nb[] = {rows * dk * eb, rows * dk * eb, rows * dv * eb, rows * dk * 4,
                         rows * dv * eb, static_cast<size_t>(dv) * 4, rows * dv * eb};
    s = check_aliasing(out, rows * dv * eb, ins, nb, 7);
    if (s != GTR_OK) return s;
    GlaArgs a{q, k, v, log_g, z, rms_w, out, resid, B, H, gh, gw, dk, dv, direction,
              chunk ? chunk : kDefaultChunk, dtype, static_cast<int64_t>(gh) * gw};
    int resolved = path;
    s = resolve_path(a, path, &resolved);
    if (s != GTR_OK) return s;
    if (!device_ok()) return GTR_ERR_HIP;
    return run(a, resolved, stream, mk);
}

// Forward segment states shared by gtr_gla_fwd_states and gtr_gla_bwd_states: the
// shapes whose backward takes the matrix-core path with the segment summaries (16-bit
// I/O, dk = dv = 64, chunk 64).  0 bytes where there are none.
size_t states_bytes_of(const GlaArgs &a) {
    if ((a.dtype != GTR_F16 && a.dtype != GTR_BF16) || a.dk != 64 || a.dv != 64 || a.chunk != 64 ||
        !sum_supported(a) || !mfma_supported(a))
        return 0;
    MfmaPlan pl, po;
    mfma_plans(a, g_chunks_per_wg, &pl, &po);
    return static_cast<size_t>(pl.n_seg) * a.dk * a.dv * 4;
}

GlaArgs shape_args(int B, int H, int gh, int gw, int dk, int dv, int direction, int chunk,
                   int dtype) {
    return GlaArgs{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, B, H,
                   gh, gw, dk, dv, direction, chunk ? chunk : kDefaultChunk, dtype,
                   static_cast<int64_t>(gh) * gw};
}

// ------------------------------------------------------ fixed device scratch --
// For callers that cannot allocate: the segment states (matrix-core path) or chunk
// states (token-serial path) of gtr_gla_fwd_noalloc live in this array, one copy per
// device, held from module load to process end.  Host code must never take the
// array's name as a device address: it only names the symbol.  The address on a
// device comes from hipGetSymbolAddress, made once per device with that device
// current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t{32} << 20;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_ptr;  // device -> address of its copy of `scratch`

gtr_status scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it == g_scratch_ptr.end()) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(GTR_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
        it = g_scratch_ptr.emplace(dev, ptr).first;
    }
    *out = it->second;
    return GTR_OK;
}

}  // namespace

extern "C" {

gtr_status gtr_gla_fwd(const void *q, const void *k, const void *v, const float *log_g,
                       const void *z, const float *rms_w, void *out, int B, int H, int grid_h,
                       int grid_w, int dk, int dv, int direction, int chunk, gtr_dtype dtype,
                       hipStream_t stream) {
    Marks mk;
    return fwd_impl(q, k, v, log_g, z, rms_w, out, nullptr, B, H, grid_h, grid_w, dk, dv,
                    direction, chunk, dtype, GTR_PATH_AUTO, stream, mk);
}

gtr_status gtr_gla_fwd_path(const void *q, const void *k, const void *v, const float *log_g,
                            const void *z, const float *rms_w, void *out, int B, int H,
                            int grid_h, int grid_w, int dk, int dv, int direction, int chunk,
                            gtr_dtype dtype, int path, hipStream_t stream) {
    Marks mk;
    return fwd_impl(q, k, v, log_g, z, rms_w, out, nullptr, B, H, grid_h, grid_w, dk, dv,
                    direction, chunk, dtype, path, stream, mk);
}

gtr_status gtr_gla_fwd_events(const void *q, const void *k, const void *v, const float *log_g,
                              const void *z, const float *rms_w, void *out, int B, int H,
                              int grid_h, int grid_w, int dk, int dv, int direction, int chunk,
                              gtr_dtype dtype, int path, hipEvent_t *events, int n_events,
                              int *n_launches, hipStream_t stream) {
    if (n_events < 0 || (n_events > 0 && !events))
        return fail(GTR_ERR_ARG, "events: need n_events >= 0 and a non-null array");
    Marks mk;
    mk.ev = events;
    mk.n = n_events;
    gtr_status s = fwd_impl(q, k, v, log_g, z, rms_w, out, nullptr, B, H, grid_h, grid_w, dk,
                            dv, direction, chunk, dtype, path, stream, mk);
    if (n_launches) *n_launches = mk.launches;
    return s;
}

gtr_status gtr_gla_fwd_noalloc(const void *q, const void *k, const void *v, const float *log_g,
                               const void *z, const float *rms_w, void *out, int B, int H,
                               int grid_h, int grid_w, int dk, int dv, int direction, int chunk,
                               gtr_dtype dtype, hipStream_t stream) {
    g_err.clear();
    gtr_status s = check(q, k, v, log_g, z, rms_w, out, B, H, grid_h, grid_w, dk, dv, direction,
                         chunk, dtype, GTR_PATH_AUTO);
    if (s != GTR_OK) return s;
    const size_t rows = static_cast<size_t>(B) * grid_h * grid_w * H;
    const size_t eb = elem_bytes(dtype);
    const void *ins[] = {q, k, v, log_g, z, rms_w};
    const size_t nb[] = {rows * dk * eb, rows * dk * eb, rows * dv * eb, rows * dk * 4,
                         rows * dv * eb, static_cast<size_t>(dv) * 4};
    s = check_aliasing(out, rows * dv * eb, ins, nb, 6);
    if (s != GTR_OK) return s;
    GlaArgs a{q, k, v, log_g, z, rms_w, out, nullptr, B, H, grid_h, grid_w, dk, dv, direction,
              chunk ? chunk : kDefaultChunk, dtype, static_cast<int64_t>(grid_h) * grid_w};
    // matrix-core or token-serial (the single-launch path needs the library's counters)
    const int path = mfma_ok(a) ? GTR_PATH_MFMA : GTR_PATH_SERIAL;
    const size_t need = run_workspace_bytes(a, path);
    if (need > kScratchBytes)
        return fail(GTR_ERR_UNSUPPORTED,
                    "this call needs %zu bytes of scratch; the fixed scratch holds %zu (use "
                    "gtr_gla_fwd)",
                    need, kScratchBytes);
    if (!device_ok()) return GTR_ERR_HIP;
    WsSource src;
    s = scratch_address(&src.ptr);
    if (s != GTR_OK) return s;
    src.bytes = kScratchBytes;
    Marks mk;
    return path == GTR_PATH_MFMA ? run_mfma(a, stream, mk, nullptr, &src)
                                 : run_serial(a, stream, mk, &src);
}

size_t gtr_gla_states_bytes(int B, int H, int grid_h, int grid_w, int dk, int dv, int chunk,
                            gtr_dtype dtype) {
    if (B <= 0 || H <= 0 || grid_h <= 0 || grid_w <= 0) return 0;
    return states_bytes_of(shape_args(B, H, grid_h, grid_w, dk, dv, 0, chunk, dtype));
}

gtr_status gtr_gla_fwd_states(const void *q, const void *k, const void *v, const float *log_g,
                              const void *z, const float *rms_w, void *out, int B, int H,
                              int grid_h, int grid_w, int dk, int dv, int direction, int chunk,
                              gtr_dtype dtype, float *states, size_t states_bytes,
                              hipStream_t stream) {
    g_err.clear();
    gtr_status s = check(q, k, v, log_g, z, rms_w, out, B, H, grid_h, grid_w, dk, dv, direction,
                         chunk, dtype, GTR_PATH_MFMA);
    if (s != GTR_OK) return s;
    if (!states) return fail(GTR_ERR_ARG, "null states pointer");
    GlaArgs a{q, k, v, log_g, z, rms_w, out, nullptr, B, H, grid_h, grid_w, dk, dv, direction,
              chunk ? chunk : kDefaultChunk, dtype, static_cast<int64_t>(grid_h) * grid_w};
    const size_t need = states_bytes_of(a);
    if (need == 0)
        return fail(GTR_ERR_UNSUPPORTED,
                    "forward states need 16-bit I/O, dk = dv = 64 and chunk 64");
    if (states_bytes < need)
        return fail(GTR_ERR_ARG, "states buffer of %zu bytes, need %zu", states_bytes, need);
    if (!vec16(a) || reinterpret_cast<uintptr_t>(states) % 16 != 0)
        return fail(GTR_ERR_UNSUPPORTED, "forward states need 16-byte aligned tensors");
    const size_t rows = static_cast<size_t>(B) * grid_h * grid_w * H;
    const size_t eb = elem_bytes(dtype);
    const void *ins[] = {q, k, v, log_g, z, rms_w, out};
    const size_t nb[] = {rows * dk * eb, rows * dk * eb, rows * dv * eb, rows * dk * 4,
                         rows * dv * eb, static_cast<size_t>(dv) * 4, rows * dv * eb};
    s = check_aliasing(out, rows * dv * eb, ins, nb, 6);
    if (s == GTR_OK) s = check_aliasing(states, need, ins, nb, 7);
    if (s != GTR_OK) return s;
    if (!device_ok()) return GTR_ERR_HIP;
    Marks mk;
    return run_mfma(a, stream, mk, states);
}

gtr_status gtr_gla_stack_fwd(const void *q, const void *k, const void *v, const float *log_g,
                             const void *z, const float *rms_w, void *out, int n_blocks, int B,
                             int H, int grid_h, int grid_w, int dk, int dv, int first_direction,
                             int chunk, gtr_dtype dtype, hipStream_t stream) {
    g_err.clear();
    if (n_blocks <= 0) return fail(GTR_ERR_ARG, "n_blocks must be positive, got %d", n_blocks);
    if (first_direction < 0 || first_direction > 3)
        return fail(GTR_ERR_ARG, "first_direction must be 0..3, got %d", first_direction);
    gtr_status s = check(q, k, v, log_g, z, rms_w, out, B, H, grid_h, grid_w, dk, dv,
                         first_direction, chunk, dtype, GTR_PATH_AUTO);
    if (s != GTR_OK) return s;
    const size_t rows = static_cast<size_t>(B) * grid_h * grid_w * H;
    const size_t eb = elem_bytes(dtype);
    const size_t qk_b = rows * dk * eb, v_b = rows * dv * eb, g_b = rows * dk * 4;
    const void *ins[] = {q, k, v, log_g, z, rms_w};
    const size_t nb[] = {qk_b * n_blocks, qk_b * n_blocks, v_b * n_blocks, g_b * n_blocks,
                         v_b * n_blocks, static_cast<size_t>(dv) * 4 * n_blocks};
    s = check_aliasing(out, v_b * n_blocks, ins, nb, 6);
    if (s != GTR_OK) return s;
    // Every block has the same shape; block i's pointers are block 0's plus whole
    // tensors, so their alignment is block 0's (rows of 16-bit elements are 64 B or
    // more).  The path and the workspace are settled here, so that an argument or
    // workspace error leaves nothing enqueued.
    GlaArgs a0{q, k, v, log_g, z, rms_w, out, n_blocks > 1 ? out : nullptr, B, H, grid_h, grid_w,
               dk, dv, first_direction, chunk ? chunk : kDefaultChunk, dtype,
               static_cast<int64_t>(grid_h) * grid_w};
    int path = GTR_PATH_AUTO;
    s = resolve_path(a0, GTR_PATH_AUTO, &path);
    if (s != GTR_OK) return s;
    if (!device_ok()) return GTR_ERR_HIP;
    {
        void *ws = nullptr;
        s = workspace(stream, run_workspace_bytes(a0, path), &ws);
        if (s != GTR_OK) return s;
    }
    for (int i = 0; i < n_blocks; ++i) {
        const char *qi = static_cast<const char *>(q) + qk_b * i;
        const char *ki = static_cast<const char *>(k) + qk_b * i;
        const char *vi = static_cast<const char *>(v) + v_b * i;
        const char *zi = static_cast<const char *>(z) + v_b * i;
        const float *gi = reinterpret_cast<const float *>(
            reinterpret_cast<const char *>(log_g) + g_b * i);
        const float *wi = rms_w + static_cast<size_t>(dv) * i;
        char *oi = static_cast<char *>(out) + v_b * i;
        const void *resid = i > 0 ? static_cast<const void *>(oi - v_b) : nullptr;
        GlaArgs a{qi, ki, vi, gi, zi, wi, oi, resid, B, H, grid_h, grid_w, dk, dv,
                  (first_direction + i) % 4, chunk, dtype, static_cast<int64_t>(grid_h) * grid_w};
        Marks mk;
        s = run(a, path, stream, mk);
        if (s != GTR_OK) {  // a launch failure: blocks 0 .. i-1 are enqueued
            std::string msg = g_err;
            return fail(s, "block %d: %s", i, msg.c_str());
        }
    }
    return GTR_OK;
}

int gtr_gla_auto_path(int B, int H, int grid_h, int grid_w, int dk, int dv, int chunk,
                      gtr_dtype dtype) {
    g_err.clear();
    const int fake = 1;
    gtr_status s = check(&fake, &fake, &fake, reinterpret_cast<const float *>(&fake), &fake,
                         reinterpret_cast<const float *>(&fake), &fake, B, H, grid_h, grid_w, dk,
                         dv, 0, chunk, dtype, GTR_PATH_AUTO);
    if (s != GTR_OK) return s;
    GlaArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, B, H,
              grid_h, grid_w, dk, dv, 0, chunk ? chunk : kDefaultChunk, dtype,
              static_cast<int64_t>(grid_h) * grid_w};
    return auto_path(a);
}

gtr_status gtr_gla_lowrank_fwd(const void *q, const void *k, const void *v, const void *feat,
                               const void *gate_w, const float *gate_b, float tau, int rank,
                               const void *z, const float *rms_w, void *out, int B, int H,
                               int grid_h, int grid_w, int dk, int dv, int direction, int chunk,
                               gtr_dtype dtype, int path, hipEvent_t *events, int n_events,
                               int *n_launches, hipStream_t stream) {
    if (n_events < 0 || (n_events > 0 && !events)) {
        g_err.clear();
        return fail(GTR_ERR_ARG, "events: need n_events >= 0 and a non-null array");
    }
    Marks mk;
    mk.ev = events;
    mk.n = n_events;
    gtr_status s = lowrank_impl(q, k, v, feat, gate_w, gate_b, tau, rank, z, rms_w, out, B, H,
                                grid_h, grid_w, dk, dv, direction, chunk, dtype, path, stream, mk);
    if (n_launches) *n_launches = mk.launches;
    return s;
}

static hipError_t mark_after(void *ctx, hipStream_t st) {
    return static_cast<Marks *>(ctx)->after_launch(st);
}

gtr_status gtr_gla_bwd(const void *q, const void *k, const void *v, const float *log_g,
                       const void *z, const float *rms_w, const void *dout, void *dq, void *dk,
                       void *dv, float *dlog_g, void *dz, float *drms_w, int B, int H,
                       int grid_h, int grid_w, int dk_, int dv_, int direction, int chunk,
                       gtr_dtype dtype, hipEvent_t *events, int n_events, int *n_launches,
                       hipStream_t stream) {
    return gtr_gla_bwd_states(q, k, v, log_g, z, rms_w, dout, dq, dk, dv, dlog_g, dz, drms_w, B, H,
                              grid_h, grid_w, dk_, dv_, direction, chunk, dtype, nullptr, 0, events,
                              n_events, n_launches, stream);
}

gtr_status gtr_gla_bwd_states(const void *q, const void *k, const void *v, const float *log_g,
                              const void *z, const float *rms_w, const void *dout, void *dq,
                              void *dk, void *dv, float *dlog_g, void *dz, float *drms_w, int B,
                              int H, int grid_h, int grid_w, int dk_, int dv_, int direction,
                              int chunk, gtr_dtype dtype, const float *states,
                              size_t states_bytes, hipEvent_t *events, int n_events,
                              int *n_launches, hipStream_t stream) {
    g_err.clear();
    if (n_launches) *n_launches = 0;
    if (n_events < 0 || (n_events > 0 && !events))
        return fail(GTR_ERR_ARG, "events: need n_events >= 0 and a non-null array");
    if (!dout || !dq || !dk || !dv || !dlog_g || !dz || !drms_w)
        return fail(GTR_ERR_ARG, "null gradient pointer");
    gtr_status s = check(q, k, v, log_g, z, rms_w, dq, B, H, grid_h, grid_w, dk_, dv_, direction,
                         chunk, dtype, GTR_PATH_AUTO);
    if (s != GTR_OK) return s;
    const size_t rows = static_cast<size_t>(B) * grid_h * grid_w * H;
    const size_t eb = elem_bytes(dtype);
    const void *bufs[] = {q, k, v, log_g, z, rms_w, dout, dq, dk, dv, dlog_g, dz, drms_w};
    const size_t nb[] = {rows * dk_ * eb, rows * dk_ * eb, rows * dv_ * eb, rows * dk_ * 4,
                         rows * dv_ * eb, static_cast<size_t>(dv_) * 4, rows * dv_ * eb,
                         rows * dk_ * eb, rows * dk_ * eb, rows * dv_ * eb, rows * dk_ * 4,
                         rows * dv_ * eb, static_cast<size_t>(dv_) * 4};
    for (int o = 7; o < 13; ++o) {  // every gradient against every other buffer
        for (int i = 0; i < 13; ++i) {
            if (i == o) continue;
            const char *a0 = static_cast<const char *>(bufs[i]), *a1 = a0 + nb[i];
            const char *o0 = static_cast<const char *>(bufs[o]), *o1 = o0 + nb[o];
            if (a0 < o1 && o0 < a1) return fail(GTR_ERR_ARG, "gradient %d overlaps buffer %d", o - 7, i);
        }
    }
    GlaArgs a{q, k, v, log_g, z, rms_w, nullptr, nullptr, B, H, grid_h, grid_w, dk_, dv_,
              direction, chunk ? chunk : kDefaultChunk, dtype,
              static_cast<int64_t>(grid_h) * grid_w};
    if (states) {  // the forward's segment states (gtr_gla_fwd_states with the same arguments)
        const size_t need = states_bytes_of(a);
        if (need == 0)
            return fail(GTR_ERR_UNSUPPORTED,
                        "forward states need 16-bit I/O, dk = dv = 64 and chunk 64");
        if (states_bytes < need)
            return fail(GTR_ERR_ARG, "states buffer of %zu bytes, need %zu", states_bytes, need);
        for (int o = 7; o < 13; ++o) {
            const char *a0 = reinterpret_cast<const char *>(states), *a1 = a0 + need;
            const char *o0 = static_cast<const char *>(bufs[o]), *o1 = o0 + nb[o];
            if (a0 < o1 && o0 < a1) return fail(GTR_ERR_ARG, "gradient %d overlaps the states", o - 7);
        }
    }
    if (!device_ok()) return GTR_ERR_HIP;
    const int64_t n_chunks = (a.L + a.chunk - 1) / a.chunk;
    if (static_cast<int64_t>(B) * H * n_chunks > 0x7fffffff)
        return fail(GTR_ERR_UNSUPPORTED, "too many chunks");
    void *ws = nullptr;
    s = workspace(stream, bwd_workspace_bytes(a, static_cast<int>(n_chunks)), &ws);
    if (s != GTR_OK) return s;
    void *ctr = nullptr;  // the drms_w reduction's block counter (left zero)
    s = counters(stream, 1, &ctr);
    if (s != GTR_OK) return s;
    Marks mk;
    mk.ev = events;
    mk.n = n_events;
    BwdLaunchHooks hooks;
    hooks.fn = mark_after;
    hooks.ctx = &mk;
    hipError_t e = mk.start(stream);
    if (e == hipSuccess)
        e = bwd_launch(a, dout, dq, dk, dv, dlog_g, dz, drms_w, ws, static_cast<unsigned *>(ctr),
                       static_cast<int>(n_chunks), g_chunks_per_wg, states, stream, hooks);
    if (n_launches) *n_launches = mk.launches;
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return GTR_OK;
}

gtr_status gtr_sswiglu_mix(const void *u, const float *w_conv, const float *b_conv, void *m,
                           int B, int grid_h, int grid_w, int F, int k, gtr_dtype dtype,
                           hipStream_t stream) {
    g_err.clear();
    if (!u || !w_conv || !b_conv || !m) return fail(GTR_ERR_ARG, "null tensor pointer");
    if (B <= 0 || grid_h <= 0 || grid_w <= 0 || F <= 0)
        return fail(GTR_ERR_ARG, "B, grid_h, grid_w, F must be positive (got %d, %d, %d, %d)", B,
                    grid_h, grid_w, F);
    if (F % 8 != 0) return fail(GTR_ERR_ARG, "F must be a multiple of 8, got %d", F);
    if (!(k == 1 || k == 3 || k == 5 || k == 7))
        return fail(GTR_ERR_ARG, "kernel size must be 1, 3, 5 or 7, got %d", k);
    if (dtype < GTR_F32 || dtype > GTR_BF16) return fail(GTR_ERR_ARG, "unknown dtype %d", dtype);
    if (reinterpret_cast<uintptr_t>(u) % 16 != 0 || reinterpret_cast<uintptr_t>(m) % 16 != 0)
        return fail(GTR_ERR_ARG, "u and m must be 16-byte aligned");
    const __int128 toks = static_cast<__int128>(B) * grid_h * grid_w;
    if (toks * 2 * F * 4 > (static_cast<__int128>(1) << 62) || toks > 0x7fffffff)
        return fail(GTR_ERR_UNSUPPORTED, "tensor sizes overflow the supported range");
    const size_t eb = elem_bytes(dtype), nt = static_cast<size_t>(toks);
    const void *ins[] = {u, w_conv, b_conv};
    const size_t nb[] = {nt * 2 * F * eb, static_cast<size_t>(F) * k * k * 4,
                         static_cast<size_t>(F) * 4};
    gtr_status s = check_aliasing(m, nt * F * eb, ins, nb, 3);
    if (s != GTR_OK) return s;
    if (!device_ok()) return GTR_ERR_HIP;
    hipError_t e = sswiglu_launch(u, w_conv, b_conv, m, B, grid_h, grid_w, F, k, dtype, stream);
    if (e != hipSuccess) return hip_fail(e, "S-SwiGLU launch");
    return GTR_OK;
}

const char *gtr_last_error(void) { return g_err.c_str(); }

int gtr_version(void) { return GTR_VERSION; }

void gtr_set_segment_chunks(int chunks) { g_chunks_per_wg = chunks > 0 ? chunks : 0; }

void gtr_set_wait_limit(unsigned polls) { g_fast_spin_limit = polls > 0 ? polls : kFastSpinLimit; }

void gtr_release_workspace(void) {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    int cur = 0;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (auto *m : {&g_ws, &g_ctr, &g_gws}) {
        for (auto &kv : *m) {
            if (!kv.second.ptr) continue;
            if (hipSetDevice(kv.first.first) == hipSuccess) {
                (void)hipDeviceSynchronize();
                (void)hipFree(kv.second.ptr);
            }
        }
        m->clear();
    }
    if (have_cur) (void)hipSetDevice(cur);
}

}  // extern "C"
