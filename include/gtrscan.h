/*
 * gtrscan.h -- C ABI of libgtrscan, the Key-only gated-linear-attention token
 * mixer of GTR (Gated Token Recurrence) for AMD Instinct MI355X (gfx950).
 *
 * Operation (GTR write-up "端侧实时感知新标杆！通用线性骨干网络GTR开源",
 * Method §1 "骨干架构：Key-only 门控递归与四向交替扫描"; the page's formulas were
 * lost, the prose fixes their form): for every batch image b and head h the
 * tokens of a grid_h x grid_w patch grid are visited in one scan order, and a
 * dk x dv state is carried with the value-side decay fixed at 1 and a
 * data-dependent key-side forget gate g_t = exp(log_g_t):
 *
 *     S_0 = 0,   S_t = Diag(g_t) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t
 *     out_t = o_t / sqrt(mean_j(o_t[j]^2) + GTR_RMS_EPS) * rms_w * z_t * sigmoid(z_t)
 *
 * (RMSNorm, then the SiLU output gate, same section), and out_t is written at
 * token t's own grid position, so grid order is restored after the scan.  The
 * evaluation is chunkwise (Method §4 "硬件感知分块推理算子": chunk summaries,
 * a boundary-state scan, per-chunk outputs with the gate fused in the
 * epilogue); the chunk size changes rounding only.
 *
 * Tensor layout (all contiguous, row-major, token-major grid order):
 *   q, k   : [B, grid_h, grid_w, H, dk]  I/O type
 *   v, z   : [B, grid_h, grid_w, H, dv]  I/O type
 *   out    : [B, grid_h, grid_w, H, dv]  I/O type, rounded to nearest even
 *   log_g  : [B, grid_h, grid_w, H, dk]  float32, must be <= 0 (not checked)
 *   rms_w  : [dv]                        float32, shared by all heads
 * Grid index of row r, column c is p = r * grid_w + c.
 *
 * Scan orders (directions): LR p(t) = t; RL p(t) = L-1-t (whole raster
 * reversed); TB visits the columns left to right, each top to bottom;
 * BT is TB reversed.  L = grid_h * grid_w.
 *
 * Alignment: every tensor must be aligned to its element size (GTR_ERR_ARG
 * otherwise).  The matrix-core and single-launch paths move rows in 16-byte
 * pieces and need q, k, v, log_g, z and out (and a stack's residual) 16-byte
 * aligned: an explicit request for them with a misaligned pointer returns
 * GTR_ERR_UNSUPPORTED, and AUTO then takes the token-serial path.
 *
 * Ownership: every tensor pointer is DEVICE memory owned by the caller; the
 * library never frees it.  out must not overlap any input.  The library keeps
 * a grow-only workspace per (device, stream), released by
 * gtr_release_workspace().
 *
 * Asynchrony: work is enqueued on `stream` (0 = the null stream) and the call
 * returns without waiting for it.  The current HIP device must own the
 * pointers and the stream.
 *
 * Graph capture: a call may be captured into a HIP graph once the same call
 * (same shape and path) has run on that stream outside capture, so that the
 * workspace already has its size; a call that would have to create or grow the
 * workspace while its stream is capturing returns GTR_ERR_UNSUPPORTED and does
 * not disturb the capture.  A captured graph holds the workspace's address:
 * while it may still be replayed, make no larger call on that stream and do
 * not call gtr_release_workspace().
 *
 * Errors: argument, path and workspace errors are found before anything is
 * enqueued; a message is available from gtr_last_error() (thread-local).
 * Data errors on the device (NaN, Inf, log_g > 0) are not checked; they
 * propagate.
 */
#ifndef GTRSCAN_H
#define GTRSCAN_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GTR_VERSION 100
#define GTR_RMS_EPS 1e-5f

typedef enum {
    GTR_OK = 0,
    GTR_ERR_ARG = -1,          /* null pointer, non-positive size, bad enum or chunk */
    GTR_ERR_UNSUPPORTED = -2,  /* dk/dv outside {32, 64, 128}, size overflow, path not available */
    GTR_ERR_HIP = -3           /* no device, allocation or launch failure */
} gtr_status;

typedef enum { GTR_F32 = 0, GTR_F16 = 1, GTR_BF16 = 2 } gtr_dtype;

typedef enum { GTR_LR = 0, GTR_RL = 1, GTR_TB = 2, GTR_BT = 3 } gtr_direction;

/* Kernel path.  AUTO picks, for 16-bit I/O with dk = 64, dv in {64, 128},
 * chunk in {32, 64} and 16-byte aligned tensors: the single-launch path for
 * B == 1 with at most 16 chunks per sequence (12 at chunk 32) and no residual or gate
 * projection, the MFMA chunk path otherwise; and the fp32 token-serial chunk
 * path for everything else (float32 I/O, other dk/dv or chunk, unaligned
 * views).  gtr_gla_auto_path reports the choice. */
typedef enum {
    GTR_PATH_AUTO = 0,
    GTR_PATH_MFMA = 1,    /* segment summaries, state scan, chunk outputs (the scan left out
                             at chunk 64 when every sequence has at most 8 segments: the
                             output kernel then folds the incoming states itself) */
    GTR_PATH_FAST = 2,    /* one launch; B == 1, L <= 2048, 16-bit I/O, MFMA shapes */
    GTR_PATH_SERIAL = 3   /* fp32 arithmetic, token-serial inside each chunk */
} gtr_path;

/*
 * One mixer call (one block's token mixing).
 *   direction : gtr_direction
 *   chunk     : 0 (library default, 64) or one of 16, 32, 64, 128
 *   dtype     : I/O type of q, k, v, z, out
 * Returns GTR_OK or an error status.
 */
gtr_status gtr_gla_fwd(const void *q, const void *k, const void *v, const float *log_g,
                       const void *z, const float *rms_w, void *out,
                       int B, int H, int grid_h, int grid_w, int dk, int dv,
                       int direction, int chunk, gtr_dtype dtype, hipStream_t stream);

/* gtr_gla_fwd with an explicit kernel path (gtr_path); a path that cannot take
 * the arguments returns GTR_ERR_UNSUPPORTED.  Used to check paths against
 * each other. */
gtr_status gtr_gla_fwd_path(const void *q, const void *k, const void *v, const float *log_g,
                            const void *z, const float *rms_w, void *out,
                            int B, int H, int grid_h, int grid_w, int dk, int dv,
                            int direction, int chunk, gtr_dtype dtype, int path,
                            hipStream_t stream);

/* gtr_gla_fwd_path that also records `events` (hipEvent_t handles created by
 * the caller) on `stream`: events[0] before the first kernel launch and
 * events[i] after launch i, for as many as n_events allows.  The launches of a
 * call are, in order: MFMA path -- segment summaries, state scan (absent where
 * the output kernel folds the states, see GTR_PATH_MFMA), chunk outputs;
 * serial path -- chunk summaries, state scan, chunk outputs; fast path -- one
 * kernel.  For timing single kernels.  *n_launches (nullable)
 * receives the number of launches of the call. */
gtr_status gtr_gla_fwd_events(const void *q, const void *k, const void *v, const float *log_g,
                              const void *z, const float *rms_w, void *out,
                              int B, int H, int grid_h, int grid_w, int dk, int dv,
                              int direction, int chunk, gtr_dtype dtype, int path,
                              hipEvent_t *events, int n_events, int *n_launches,
                              hipStream_t stream);

/*
 * gtr_gla_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops that forbid allocation after start-up,
 * harnesses without an allocator.  Same arguments and operation as
 * gtr_gla_fwd; it takes the MFMA path where gtr_gla_fwd's AUTO takes the MFMA
 * or the single-launch path, and the token-serial path otherwise, with results
 * equal bit for bit to gtr_gla_fwd_path on that path.  It calls no hipMalloc,
 * hipFree or other allocating routine: the per-call segment (or chunk) states
 * live in a fixed device array of the library, 32 MiB on each device, held from
 * the library's load until the process ends.  A call whose states would not fit
 * (more than 32 MiB: e.g. beyond about 2000 segments at dk = dv = 64) returns
 * GTR_ERR_UNSUPPORTED before anything is enqueued.  Nothing in the array has to
 * start at zero: every word a call reads was written earlier in the same call.
 * All calls on one device share the array, so calls that may overlap in time on
 * one device (different streams without ordering between them) race and must
 * not be issued; calls ordered on one stream are safe.
 */
gtr_status gtr_gla_fwd_noalloc(const void *q, const void *k, const void *v, const float *log_g,
                               const void *z, const float *rms_w, void *out,
                               int B, int H, int grid_h, int grid_w, int dk, int dv,
                               int direction, int chunk, gtr_dtype dtype, hipStream_t stream);

/*
 * A stack of n_blocks mixer calls (Method §1: the scan direction cycles
 * LR, RL, TB, BT with depth and grid order is restored after every block).
 * Every tensor gains a leading [n_blocks] dimension: q, k, log_g, v, z as
 * above per block, rms_w is [n_blocks, dv], and out is [n_blocks, B, grid_h,
 * grid_w, H, dv] and receives every block's output.  Block i scans direction
 * (first_direction + i) mod 4 and uses the value input
 *     v_eff_i = round_io(v_i + out_{i-1})   (i > 0; float32 add),  v_eff_0 = v_0,
 * the previous block's output fed forward as a residual.  Blocks are ordered
 * on `stream`; there is no host synchronisation between them.  The path and the
 * workspace are settled for all blocks before block 0 is enqueued, so argument
 * and workspace errors leave nothing enqueued; a kernel launch that fails in
 * block i (i > 0) leaves blocks 0 .. i-1 enqueued.
 */
gtr_status gtr_gla_stack_fwd(const void *q, const void *k, const void *v, const float *log_g,
                             const void *z, const float *rms_w, void *out, int n_blocks,
                             int B, int H, int grid_h, int grid_w, int dk, int dv,
                             int first_direction, int chunk, gtr_dtype dtype,
                             hipStream_t stream);

/*
 * One mixer call whose forget gate is formed inside the library from rank-r
 * gate features (GTR write-up "端侧实时感知新标杆！通用线性骨干网络GTR开源",
 * Method §1: the gate is generated from the input by a light low-rank
 * projection with a temperature; the page's rank and temperature were lost,
 * so both are arguments):
 *     x[b, p, h, c]     = sum_j feat[b, p, j] * gate_w[j, h*dk + c] + gate_b[h*dk + c]
 *     log_g[b, p, h, c] = logsigmoid(x) / tau         (g = sigmoid(x)^(1/tau))
 * and then exactly the operation of gtr_gla_fwd with that log_g.
 *   feat   : [B, grid_h, grid_w, rank]  I/O type; one vector per token, shared by
 *            all heads (the input already projected to rank r)
 *   gate_w : [rank, H*dk]               I/O type
 *   gate_b : [H*dk]                     float32
 *   rank   : 1 .. 256;   tau: finite and > 0 (the usual GLA choice is 16)
 * feat, gate_w and gate_b must be 16-byte aligned.  The other tensors, dtype,
 * direction and chunk are as for gtr_gla_fwd; path as gtr_gla_fwd_path, and
 * AUTO picks the path gtr_gla_fwd would.  With 16-bit I/O, dk = dv = 64,
 * chunk 64 and rank 16 the MFMA path forms the gate inside its summary and
 * output kernels and log_g never reaches memory; every other case first
 * writes log_g (float32) to a library workspace with one extra launch.
 * events / n_events / n_launches as gtr_gla_fwd_events (that extra launch,
 * when there is one, is the first); events may be NULL when n_events is 0, and
 * n_launches may be NULL.  Errors as gtr_gla_fwd.
 */
gtr_status gtr_gla_lowrank_fwd(const void *q, const void *k, const void *v, const void *feat,
                               const void *gate_w, const float *gate_b, float tau, int rank,
                               const void *z, const float *rms_w, void *out,
                               int B, int H, int grid_h, int grid_w, int dk, int dv,
                               int direction, int chunk, gtr_dtype dtype, int path,
                               hipEvent_t *events, int n_events, int *n_launches,
                               hipStream_t stream);

/*
 * Backward pass of one mixer call (gtr_gla_fwd's operation, Method §1 of the
 * GTR write-up "端侧实时感知新标杆！通用线性骨干网络GTR开源", evaluated chunkwise as
 * in Method §4 in both scan directions): given dout = dL/dout, writes
 *   dq, dk : [B, grid_h, grid_w, H, dk]  I/O type
 *   dv, dz : [B, grid_h, grid_w, H, dv]  I/O type
 *   dlog_g : [B, grid_h, grid_w, H, dk]  float32
 *   drms_w : [dv]                        float32 (summed over every token and head)
 * Inputs q, k, v, log_g, z, rms_w, dims, direction and chunk as gtr_gla_fwd
 * (no stack residual); dout has out's shape and type.  Accumulation is fp32
 * (16-bit I/O at dk = dv = 64, chunk <= 64: products on the matrix cores with
 * bf16 hi + lo operands; the forward states are recomputed, not stored);
 * gradients of 16-bit I/O are rounded to nearest even; results do not depend
 * on timing (no atomics).  No gradient buffer may overlap another buffer.
 * events / n_events / n_launches as gtr_gla_fwd_events (NULL / 0 allowed).
 * Errors, ownership and asynchrony as gtr_gla_fwd.
 */
gtr_status gtr_gla_bwd(const void *q, const void *k, const void *v, const float *log_g,
                       const void *z, const float *rms_w, const void *dout, void *dq, void *dk,
                       void *dv, float *dlog_g, void *dz, float *drms_w,
                       int B, int H, int grid_h, int grid_w, int dk_, int dv_, int direction,
                       int chunk, gtr_dtype dtype, hipEvent_t *events, int n_events,
                       int *n_launches, hipStream_t stream);

/*
 * Forward states kept for the backward (GTR write-up "端侧实时感知新标杆！通用线性骨干网络GTR开源",
 * Method §4: the chunk summaries and the boundary-state scan, whose result is
 * the state entering each piece of the scan).  A forward call on the
 * matrix-core path can leave the incoming state of every segment (run of
 * chunks one workgroup summarises) in a caller buffer; a backward call with the
 * same inputs and arguments then takes them instead of recomputing them.
 *
 * gtr_gla_states_bytes: the buffer size for this shape, or 0 where the shape
 * has no such states (they exist for 16-bit I/O with dk = dv = 64 and chunk 64
 * or 0).  Pure host computation; the size depends on gtr_set_segment_chunks,
 * which must not change between the two calls.
 *
 * gtr_gla_fwd_states: gtr_gla_fwd on the matrix-core path that also writes the
 * segment states, float32 [segment][dk][dv], to `states` (device memory owned
 * by the caller, states_bytes >= gtr_gla_states_bytes(...), overlapping no
 * other buffer).  out is bit for bit gtr_gla_fwd's on that path.
 * GTR_ERR_UNSUPPORTED for other shapes; GTR_ERR_ARG for a null or short buffer;
 * otherwise errors as gtr_gla_fwd.
 *
 * gtr_gla_bwd_states: gtr_gla_bwd given those states (NULL: recomputed, as
 * gtr_gla_bwd).  The states must come from gtr_gla_fwd_states with the same q,
 * k, v, log_g, shape, direction, chunk and dtype; the library cannot check
 * their content.  Where the backward does not take the matrix-core path (the
 * gradient or input pointers not 16-byte aligned) they are not used.  The
 * gradients are bit for bit gtr_gla_bwd's; two launches fewer.
 */
size_t gtr_gla_states_bytes(int B, int H, int grid_h, int grid_w, int dk, int dv, int chunk,
                            gtr_dtype dtype);
gtr_status gtr_gla_fwd_states(const void *q, const void *k, const void *v, const float *log_g,
                              const void *z, const float *rms_w, void *out, int B, int H,
                              int grid_h, int grid_w, int dk, int dv, int direction, int chunk,
                              gtr_dtype dtype, float *states, size_t states_bytes,
                              hipStream_t stream);
gtr_status gtr_gla_bwd_states(const void *q, const void *k, const void *v, const float *log_g,
                              const void *z, const float *rms_w, const void *dout, void *dq,
                              void *dk, void *dv, float *dlog_g, void *dz, float *drms_w, int B,
                              int H, int grid_h, int grid_w, int dk_, int dv_, int direction,
                              int chunk, gtr_dtype dtype, const float *states,
                              size_t states_bytes, hipEvent_t *events, int n_events,
                              int *n_launches, hipStream_t stream);

/*
 * The fused middle of the Spatial SwiGLU feed-forward block (GTR write-up
 * "端侧实时感知新标杆！通用线性骨干网络GTR开源", Method §2 "Spatial SwiGLU": in the
 * channel expansion the value branch is reshaped to the 2-D token grid and
 * mixed by a depthwise convolution; the page's kernel size was lost, so it is
 * an argument):
 *     m[b, y, x, f] = SiLU(gate[b, y, x, f]) * (b_conv[f] + sum_{i, j < k}
 *                     w_conv[f, i, j] * value[b, y + i - k/2, x + j - k/2, f])
 * with gate = u[..., :F] and value = u[..., F:] (one expanded projection),
 * zero padding outside the grid (cross-correlation, as deep-learning
 * frameworks define convolution), fp32 arithmetic, m rounded to nearest even.
 *   u      : [B, grid_h, grid_w, 2F]  I/O type
 *   w_conv : [F, k, k]                float32
 *   b_conv : [F]                      float32
 *   m      : [B, grid_h, grid_w, F]   I/O type; must not overlap any input
 *   k      : 1, 3, 5 or 7;  F: a positive multiple of 8
 * u and m must be 16-byte aligned.  The projections around it (x W_in before,
 * m W_out after) are plain GEMMs left to the caller's BLAS.  Ownership,
 * asynchrony and errors as gtr_gla_fwd.
 */
gtr_status gtr_sswiglu_mix(const void *u, const float *w_conv, const float *b_conv, void *m,
                           int B, int grid_h, int grid_w, int F, int k, gtr_dtype dtype,
                           hipStream_t stream);

/* The gtr_path that GTR_PATH_AUTO selects for a gtr_gla_fwd call with these
 * arguments and 16-byte aligned tensors, or a negative gtr_status if the
 * arguments are invalid (no device access).  (Unaligned views take the
 * token-serial path; a stack of more than one block, whose blocks all take one
 * path and add a residual after the first, and the low-rank gate calls never
 * take the single-launch path.) */
int gtr_gla_auto_path(int B, int H, int grid_h, int grid_w, int dk, int dv, int chunk,
                      gtr_dtype dtype);

/* Message of the calling thread's last error ("" if none).  Never NULL. */
const char *gtr_last_error(void);

/* GTR_VERSION of the built library. */
int gtr_version(void);

/* Tuning hook: number of chunks each workgroup of the MFMA path processes (its
 * range of the sequence-major chunk list); 0 restores the automatic choice
 * (about 512 workgroups).  Process-wide; results depend on it only through
 * rounding. */
void gtr_set_segment_chunks(int chunks);

/* Test hook: how many times a single-launch (GTR_PATH_FAST) workgroup polls the
 * ready flags of its sequence's earlier chunks before its bounded wait gives up;
 * 0 restores the default (2^24 polls, far beyond any real wait).  A wait that
 * gives up makes that chunk's incoming state NaN, so every output of the chunk
 * is NaN instead of silently wrong; the launch still finishes and leaves its
 * counters ready for the next call.  A small limit lets a test force give-ups
 * from the host.  Process-wide; read when a call is enqueued. */
void gtr_set_wait_limit(unsigned polls);

/* Frees every cached workspace after synchronising the device that owns it. */
void gtr_release_workspace(void);

#ifdef __cplusplus
}
#endif

#endif /* GTRSCAN_H */
