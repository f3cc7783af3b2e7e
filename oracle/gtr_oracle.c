/*
 * gtr_oracle.c -- fp64 reference for the Key-only gated linear attention
 * token mixer of GTR.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may call it; the library's
 * product path never does.  It shares no code, header or constant with the
 * HIP path.
 *
 * What it computes (GTR write-up "端侧实时感知新标杆！通用线性骨干网络GTR开源",
 * Method §1 "骨干架构：Key-only 门控递归与四向交替扫描"; the formulas did not
 * survive on the page, the prose fixes their form):
 *   per batch b and head h, with the value-side decay fixed at 1 and a
 *   key-side forget gate g_t = exp(log_g_t) in (0, 1]^dk,
 *       S_0 = 0,   S_t = Diag(g_t) S_{t-1} + k_t v_t^T      (dk x dv)
 *       o_t = S_t^T q_t                                      (dv)
 *   then RMSNorm of o_t over its dv entries, times the weight rms_w, times
 *   the SiLU output gate z_t * sigmoid(z_t)  (same section: RMSNorm, then a
 *   data-dependent SiLU gate).  The scan visits the grid in one of four
 *   orders (same section: LR, RL, TB, BT per block) and every output is
 *   written back at its own grid position (grid order restored).
 *
 * Readings where the page is silent (see the design notes): no scaling of q;
 * S_0 = 0; RMSNorm mean over dv with eps as passed; grid index p = r*gw + c;
 * LR p(t) = t; RL p(t) = L-1-t; TB visits columns left to right, each top to
 * bottom; BT is TB with t -> L-1-t.
 *
 * The step recurrence is evaluated exactly as written, one token at a time, in
 * double precision.  Work is split over (b, h, block of value columns): the
 * columns of S evolve independently, so this is the same arithmetic in any
 * split.  Compile with -ffp-contract=off, no fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_COLS 8 /* value columns per work item */

static int64_t scan_to_grid(int64_t t, int64_t L, int gh, int gw, int direction)
{
    /* Direction names from Method §1; the index maps are this oracle's reading. */
    switch (direction) {
    case 0: /* LR: row-major raster */
        return t;
    case 1: /* RL: the whole raster reversed */
        return L - 1 - t;
    case 2: { /* TB: column-major raster, each column top to bottom */
        int64_t c = t / gh, r = t % gh;
        return r * gw + c;
    }
    case 3: { /* BT: TB reversed */
        int64_t u = L - 1 - t;
        int64_t c = u / gh, r = u % gh;
        return r * gw + c;
    }
    default:
        return -1;
    }
}

int gtr_oracle_version(void) { return 1; }

/*
 * Single mixer call.  All arrays are float64, token-major grid order:
 *   q, k, log_g: [B, gh, gw, H, dk];  v, z, out: [B, gh, gw, H, dv];
 *   rms_w: [dv].
 * apply_epilogue = 0 stores the raw readout o_t instead of the gated RMSNorm.
 * bh_list (nullable, n_bh entries) restricts the work to those b*H + h
 * sequences; other outputs are left untouched.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int gtr_oracle_fwd(const double *q, const double *k, const double *v, const double *log_g,
                   const double *z, const double *rms_w, double *out,
                   int B, int H, int gh, int gw, int dk, int dv, int direction,
                   double eps, int apply_epilogue, const int64_t *bh_list, int64_t n_bh)
{
    if (!q || !k || !v || !log_g || !out || B <= 0 || H <= 0 || gh <= 0 || gw <= 0 ||
        dk <= 0 || dv <= 0 || direction < 0 || direction > 3)
        return -1;
    if (apply_epilogue && (!z || !rms_w))
        return -1;
    const int64_t L = (int64_t)gh * gw;
    const int64_t nbh = bh_list ? n_bh : (int64_t)B * H;
    const int ncb = (dv + ORACLE_COLS - 1) / ORACLE_COLS;
    const int64_t items = nbh * ncb;
    int failed = 0;

#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * ORACLE_COLS);
        double *g = (double *)malloc(sizeof(double) * (size_t)dk);
        if (!S || !g) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < items; ++it) {
            if (!S || !g)
                continue;
            const int64_t bh = bh_list ? bh_list[it / ncb] : it / ncb;
            const int64_t b = bh / H, h = bh % H;
            const int j0 = (int)(it % ncb) * ORACLE_COLS;
            const int nj = (dv - j0) < ORACLE_COLS ? (dv - j0) : ORACLE_COLS;
            memset(S, 0, sizeof(double) * (size_t)dk * ORACLE_COLS);
            for (int64_t t = 0; t < L; ++t) {
                const int64_t p = scan_to_grid(t, L, gh, gw, direction);
                const int64_t row = (b * L + p) * H + h;
                const double *qt = q + row * dk, *kt = k + row * dk, *lg = log_g + row * dk;
                const double *vt = v + row * dv + j0;
                for (int c = 0; c < dk; ++c)
                    g[c] = exp(lg[c]);
                /* S_t = Diag(g_t) S_{t-1} + k_t v_t^T  (this column block) */
                for (int c = 0; c < dk; ++c)
                    for (int j = 0; j < nj; ++j)
                        S[c * ORACLE_COLS + j] = g[c] * S[c * ORACLE_COLS + j] + kt[c] * vt[j];
                /* o_t = S_t^T q_t */
                double *ot = out + row * dv + j0;
                for (int j = 0; j < nj; ++j) {
                    double acc = 0.0;
                    for (int c = 0; c < dk; ++c)
                        acc += S[c * ORACLE_COLS + j] * qt[c];
                    ot[j] = acc;
                }
            }
        }
        free(S);
        free(g);
    }
    if (failed)
        return -1;
    if (!apply_epilogue)
        return 0;

    /* y = o / sqrt(mean(o^2) + eps) * rms_w * z * sigmoid(z)   (Method §1: RMSNorm, SiLU gate) */
    const int64_t rows = nbh * L;
#pragma omp parallel for schedule(static)
    for (int64_t it = 0; it < rows; ++it) {
        const int64_t bh = bh_list ? bh_list[it / L] : it / L;
        const int64_t b = bh / H, h = bh % H, p = it % L;
        const int64_t row = (b * L + p) * H + h;
        double *ot = out + row * dv;
        const double *zt = z + row * dv;
        double ss = 0.0;
        for (int j = 0; j < dv; ++j)
            ss += ot[j] * ot[j];
        const double inv = 1.0 / sqrt(ss / dv + eps);
        for (int j = 0; j < dv; ++j) {
            const double silu = zt[j] / (1.0 + exp(-zt[j]));
            ot[j] = ot[j] * inv * rms_w[j] * silu;
        }
    }
    return 0;
}

/* Threads the OpenMP runtime would use; reported beside the CPU timing. */
int gtr_oracle_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads of later calls (timing at one thread and at all of them). */
void gtr_oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
