/*
 * fp64 CPU oracle for the 2DMamba 2D selective scan (forward and backward).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no source with the GPU kernels.
 *
 * What it computes, per batch b, channel d, state n and cell (i, j) of an
 * H x W map (row-major, j fastest):
 *
 *   discretisation      Abar = exp(delta * A[d,n]),  Bx = delta * B[b,n,i,j] * x
 *       (the pages name Abar and Bbar without defining them; this is the
 *        zero-order-hold A / Euler B reading used by Mamba)
 *   horizontal scan     hh[i,j] = Abar[i,j] * hh[i,j-1] + Bx[i,j],  hh[i,-1] = 0
 *       (juejin.cn "2DMamba 精读", part 四 section 5, 横向扫描)
 *   vertical scan       h[i,j]  = Abar[i,j] * h[i-1,j]  + hh[i,j],  h[-1,j] = 0
 *       (same page, section 5(2) 纵向扫描; it scans the horizontal results,
 *        papernotes.org "2DMamba", 关键设计: 2D选择性SSM架构)
 *   output              y[i,j]  = sum_n C[b,n,i,j] * h[i,j] + D[d] * x[i,j]
 *       (juejin.cn "2DMamba 精读", part 四 section 5, 最终输出 y = C h; the D x skip term is the
 *        Mamba convention and is added here)
 *
 * Every step is executed literally, in the order written, in double precision,
 * one state map at a time. There is no blocking, fusion or reordering.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* The two recurrences on one (b, d, n) state map.
 * abar, bx: [H][W] inputs; h: [H][W] output. hh_row: scratch of length W. */
static void scan_state_map(const double *abar, const double *bx, double *h,
                           double *hh_row, int64_t H, int64_t W)
{
    for (int64_t i = 0; i < H; ++i) {
        /* horizontal recurrence along row i, left to right, zero start */
        double carry = 0.0;
        for (int64_t j = 0; j < W; ++j) {
            carry = abar[i * W + j] * carry + bx[i * W + j];
            hh_row[j] = carry;
        }
        /* vertical recurrence down each column, over the horizontal results */
        for (int64_t j = 0; j < W; ++j) {
            double up = (i > 0) ? h[(i - 1) * W + j] : 0.0;
            h[i * W + j] = abar[i * W + j] * up + hh_row[j];
        }
    }
}

/* The same two recurrences in another scan direction or order.
 *
 * The pages' scan runs left to right, then top to bottom, and leaves both
 * the reverse scans and the vertical-then-horizontal order as variants: the
 * papernotes.org page (消融实验要点) finds the two orders nearly equal, its
 * 局限与展望 notes that the upper-left scan needs a reverse scan for full
 * context, and the juejin.cn page (part 七, section 4) lists bidirectional and
 * four-quadrant 2D propagation. Read plainly, a flipped axis scans from the
 * other end, with zero state before the first cell in scan order; the
 * vertical-first order runs the column recurrence on Bx and the row
 * recurrence over its results.
 *
 *   flip_h: rows bottom to top; flip_w: columns right to left;
 *   vfirst: v[i,j] = Abar[i,j] v[i-1,j] + Bx[i,j] (column scan first),
 *           h[i,j] = Abar[i,j] h[i,j-1] + v[i,j]  (row scan of the results)
 * ("i-1", "j-1" meaning the previous cell in scan order). tmp: H*W scratch. */
static void scan_state_map_dir(const double *abar, const double *bx, double *h, double *tmp,
                               int64_t H, int64_t W, int flip_h, int flip_w, int vfirst,
                               const double *h0, double *hl, const double *g0, double *gl)
{
    /* h0 (may be NULL: zeros): the carried vertical state before the first
     * row in scan order, by column (h for the horizontal-first order, v for
     * vertical-first); hl (may be NULL): the same state after the last row.
     * Scanning a map in bands of rows, each band's h0 the previous band's hl,
     * gives the scan of the whole map.
     * g0 (may be NULL: zeros): the carried horizontal state before the first
     * column in scan order, by row (the row recurrence's carry: hh for the
     * horizontal-first order, h for vertical-first); gl (may be NULL): the
     * same state after the last column. Bands of columns compose the same
     * way, and tiles with both carries too. */
    for (int64_t si = 0; si < H; ++si) {
        const int64_t i = flip_h ? H - 1 - si : si;      /* row in scan order */
        const int64_t ip = flip_h ? i + 1 : i - 1;        /* previous row in scan order */
        if (!vfirst) {
            double carry = g0 ? g0[i] : 0.0;              /* row recurrence first */
            for (int64_t sj = 0; sj < W; ++sj) {
                const int64_t j = flip_w ? W - 1 - sj : sj;
                carry = abar[i * W + j] * carry + bx[i * W + j];
                tmp[i * W + j] = carry;
            }
            if (gl) gl[i] = carry;
            for (int64_t j = 0; j < W; ++j) {
                const double prev = (si > 0) ? h[ip * W + j] : (h0 ? h0[j] : 0.0);
                h[i * W + j] = abar[i * W + j] * prev + tmp[i * W + j];
            }
        } else {
            for (int64_t j = 0; j < W; ++j) {             /* column recurrence first */
                const double prev = (si > 0) ? tmp[ip * W + j] : (h0 ? h0[j] : 0.0);
                tmp[i * W + j] = abar[i * W + j] * prev + bx[i * W + j];
            }
            double carry = g0 ? g0[i] : 0.0;
            for (int64_t sj = 0; sj < W; ++sj) {
                const int64_t j = flip_w ? W - 1 - sj : sj;
                carry = abar[i * W + j] * carry + tmp[i * W + j];
                h[i * W + j] = carry;
            }
            if (gl) gl[i] = carry;
        }
    }
    if (hl) {
        const int64_t last = flip_h ? 0 : H - 1;  /* last row in scan order */
        for (int64_t j = 0; j < W; ++j) hl[j] = vfirst ? tmp[last * W + j] : h[last * W + j];
    }
}

/* Direction / order flags of the variant entries (bit values). */
#define ORACLE_FLIP_H 1
#define ORACLE_FLIP_W 2
#define ORACLE_VFIRST 4

/* Internal entry: the recurrences in the direction and order `flags` selects,
 * on caller-supplied Abar and Bx ([H][W] doubles). Returns 0, 2 or 6. */
int oracle_ssm2d_states_ex_f64(const double *abar, const double *bx, double *h,
                               int64_t H, int64_t W, int flags)
{
    if (H < 0 || W < 0) return 2;
    if (H == 0 || W == 0) return 0;
    double *tmp = (double *)malloc((size_t)(H * W) * sizeof(double));
    if (!tmp) return 6;
    scan_state_map_dir(abar, bx, h, tmp, H, W, (flags & ORACLE_FLIP_H) != 0,
                       (flags & ORACLE_FLIP_W) != 0, (flags & ORACLE_VFIRST) != 0, NULL, NULL, NULL, NULL);
    free(tmp);
    return 0;
}

/* Internal entry: the recurrences alone, on caller-supplied Abar and Bx.
 * abar, bx, h: [H][W] doubles. Returns 0, or 2 on a bad size. */
int oracle_ssm2d_states_f64(const double *abar, const double *bx, double *h,
                            int64_t H, int64_t W)
{
    if (H < 0 || W < 0) return 2;
    if (H == 0 || W == 0) return 0;
    double *hh_row = (double *)malloc((size_t)W * sizeof(double));
    if (!hh_row) return 6;
    scan_state_map(abar, bx, h, hh_row, H, W);
    free(hh_row);
    return 0;
}

/* One (b, d) map: y_map[H][W]. */
static int forward_one_map(const double *x, const double *delta, const double *A,
                           const double *B, const double *C, const double *D,
                           double *y_map, int64_t b, int64_t d, int64_t d_inner,
                           int64_t d_state, int64_t H, int64_t W, int flags,
                           const double *h0m, double *hlm, const double *g0m, double *glm)
{
    /* h0m, hlm (may be NULL): carried vertical states [d_state][W] of this map;
     * g0m, glm (may be NULL): carried horizontal states [d_state][H] */
    const int carries = (h0m != NULL) || (hlm != NULL) || (g0m != NULL) || (glm != NULL);
    const int64_t L = H * W;
    const double *xm = x + (b * d_inner + d) * L;
    const double *dm = delta + (b * d_inner + d) * L;
    double *abar = (double *)malloc((size_t)L * sizeof(double));
    double *bx = (double *)malloc((size_t)L * sizeof(double));
    double *h = (double *)malloc((size_t)L * sizeof(double));
    double *hh_row = (double *)malloc((size_t)((flags || carries) ? L : W) * sizeof(double));
    if (!abar || !bx || !h || !hh_row) {
        free(abar); free(bx); free(h); free(hh_row);
        return 6;
    }
    for (int64_t p = 0; p < L; ++p) y_map[p] = 0.0;
    for (int64_t n = 0; n < d_state; ++n) {
        const double a = A[d * d_state + n];
        const double *Bn = B + (b * d_state + n) * L;
        const double *Cn = C + (b * d_state + n) * L;
        for (int64_t p = 0; p < L; ++p) {
            abar[p] = exp(dm[p] * a);
            bx[p] = dm[p] * Bn[p] * xm[p];
        }
        if (flags == 0 && !carries) scan_state_map(abar, bx, h, hh_row, H, W);
        else scan_state_map_dir(abar, bx, h, hh_row, H, W, (flags & ORACLE_FLIP_H) != 0,
                                (flags & ORACLE_FLIP_W) != 0, (flags & ORACLE_VFIRST) != 0,
                                h0m ? h0m + n * W : NULL, hlm ? hlm + n * W : NULL,
                                g0m ? g0m + n * H : NULL, glm ? glm + n * H : NULL);
        for (int64_t p = 0; p < L; ++p) y_map[p] += Cn[p] * h[p];
    }
    for (int64_t p = 0; p < L; ++p) y_map[p] += D[d] * xm[p];
    free(abar); free(bx); free(h); free(hh_row);
    return 0;
}

/* Forward pass over a list of (b, d) maps.
 *
 * x, delta: [batch][d_inner][H][W]; A: [d_inner][d_state]; B, C:
 * [batch][d_state][H][W]; D: [d_inner]. maps: n_maps flat indices
 * m = b * d_inner + d (NULL = all maps in order). y: [n_maps][H][W].
 * nthreads: OpenMP threads (<= 0: runtime default).
 * Returns 0 on success, 2 on a bad size or map index, 6 on allocation failure.
 */
static int fwd_maps(const double *x, const double *delta, const double *A, const double *B,
                    const double *C, const double *D, double *y, int64_t batch, int64_t d_inner,
                    int64_t d_state, int64_t H, int64_t W, const int64_t *maps, int64_t n_maps,
                    int nthreads, int flags, const double *h0, double *hl, const double *g0,
                    double *gl)
{
    if (batch < 0 || d_inner < 0 || d_state < 0 || H < 0 || W < 0) return 2;
    const int64_t total = batch * d_inner;
    if (maps == NULL) n_maps = total;
    if (n_maps < 0) return 2;
    for (int64_t k = 0; maps != NULL && k < n_maps; ++k)
        if (maps[k] < 0 || maps[k] >= total) return 2;
    if (n_maps == 0 || H == 0 || W == 0) return 0;
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t k = 0; k < n_maps; ++k) {
        const int64_t m = maps ? maps[k] : k;
        int s = forward_one_map(x, delta, A, B, C, D, y + k * H * W, m / d_inner,
                                m % d_inner, d_inner, d_state, H, W, flags,
                                h0 ? h0 + m * d_state * W : NULL, hl ? hl + m * d_state * W : NULL,
                                g0 ? g0 + m * d_state * H : NULL, gl ? gl + m * d_state * H : NULL);
        if (s != 0) {
#pragma omp atomic write
            status = s;
        }
    }
    return status;
}

int oracle_ssm2d_fwd_maps_f64(const double *x, const double *delta, const double *A,
                              const double *B, const double *C, const double *D,
                              double *y, int64_t batch, int64_t d_inner, int64_t d_state,
                              int64_t H, int64_t W, const int64_t *maps, int64_t n_maps,
                              int nthreads)
{
    return fwd_maps(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, maps, n_maps,
                    nthreads, 0, NULL, NULL, NULL, NULL);
}

/* The forward pass in the direction / order `flags` selects (ORACLE_FLIP_H,
 * ORACLE_FLIP_W, ORACLE_VFIRST); otherwise as oracle_ssm2d_fwd_maps_f64. */
int oracle_ssm2d_fwd_ex_f64(const double *x, const double *delta, const double *A,
                            const double *B, const double *C, const double *D,
                            double *y, int64_t batch, int64_t d_inner, int64_t d_state,
                            int64_t H, int64_t W, const int64_t *maps, int64_t n_maps,
                            int nthreads, int flags)
{
    if (flags < 0 || flags > 7) return 2;
    return fwd_maps(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, maps, n_maps,
                    nthreads, flags, NULL, NULL, NULL, NULL);
}

/* The forward pass with carried vertical states (all maps): h0 (may be NULL)
 * holds, per (b, d, n) and column, the state before the first row in scan
 * order, hl (may be NULL) receives the state after the last row; both
 * [batch][d_inner][d_state][W]. Otherwise as oracle_ssm2d_fwd_ex_f64. */
int oracle_ssm2d_fwd_carry_f64(const double *x, const double *delta, const double *A,
                               const double *B, const double *C, const double *D,
                               double *y, const double *h0, double *hl, int64_t batch,
                               int64_t d_inner, int64_t d_state, int64_t H, int64_t W,
                               int nthreads, int flags)
{
    if (flags < 0 || flags > 7) return 2;
    return fwd_maps(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, NULL, 0,
                    nthreads, flags, h0, hl, NULL, NULL);
}

/* The forward pass of one tile of a larger map (all maps): h0 / hl as in
 * oracle_ssm2d_fwd_carry_f64 ([batch][d_inner][d_state][W], the vertical
 * state before the first / after the last row in scan order), g0 / gl
 * ([batch][d_inner][d_state][H], the horizontal state before the first /
 * after the last column in scan order, by row); any may be NULL (zeros in,
 * nothing out). Scanning a map tile by tile in scan order, each tile taking
 * the carries its upper and left neighbours (in scan order) hand out, gives
 * the scan of the whole map. */
int oracle_ssm2d_fwd_tile_f64(const double *x, const double *delta, const double *A,
                              const double *B, const double *C, const double *D,
                              double *y, const double *h0, double *hl, const double *g0,
                              double *gl, int64_t batch, int64_t d_inner, int64_t d_state,
                              int64_t H, int64_t W, int nthreads, int flags)
{
    if (flags < 0 || flags > 7) return 2;
    return fwd_maps(x, delta, A, B, C, D, y, batch, d_inner, d_state, H, W, NULL, 0,
                    nthreads, flags, h0, hl, g0, gl);
}

/* ---------------------------------------------------------------- backward
 *
 * Gradients of a scalar loss L through the forward pass above, given
 * dy = dL/dy. The pages describe training but not the backward pass; this is
 * reverse-mode differentiation of the forward steps, taken in reverse order,
 * in fp64 (pinned against finite differences of the forward pass). Per
 * (b, d, n) map, with a = Abar, u = Bx:
 *
 *   y  <- h  : g_h[i,j]  = dy[i,j] C[i,j] + a[i+1,j] g_h[i+1,j]   (h[i,j] also feeds h[i+1,j])
 *   h  <- hh : g_hh[i,j] = g_h[i,j] + a[i,j+1] g_hh[i,j+1]        (hh[i,j] also feeds hh[i,j+1])
 *   a        : g_a[i,j]  = g_hh[i,j] hh[i,j-1] + g_h[i,j] h[i-1,j]
 *   u        : g_u[i,j]  = g_hh[i,j]
 *   a = exp(delta A), u = delta B x:
 *     d delta += g_a A a + g_u B x      dA[d,n] += g_a delta a
 *     dB[b,n] += g_u delta x            dx      += g_u delta B
 *     dC[b,n] += dy h
 *   skip term: dx += dy D[d],  dD[d] += dy x
 * (terms with index -1 or beyond the map are zero). */
static void backward_one_map(const double *xm, const double *dm, double a_dn, const double *Bn,
                             const double *Cn, const double *dym, double *dxm, double *ddm,
                             double *dBn, double *dCn, double *dA_dn, int64_t H, int64_t W,
                             double *a, double *u, double *hh, double *h, double *gh, double *ghh,
                             const double *h0, const double *gl, double *dh0,
                             const double *g0, const double *ggl, double *dg0)
{
    /* g0, ggl, dg0 (may be NULL): the same for the carried row state ([H]):
     * g0 the state left of column 0, ggl dL/dhh of the state after the last
     * column (hh of column W-1), dg0 receives dL/dg0 = a[i,0] g_hh[i,0]. */
    /* h0 (may be NULL: zeros): the carried vertical state above row 0 ([W]);
     * gl (may be NULL: zeros): dL/dh of the state after the last row, which
     * the forward hands out (h of row H-1); dh0 (may be NULL): receives
     * dL/dh0 = a[0,j] g_h[0,j], h0 entering row 0 through its decay. */
    const int64_t L = H * W;
    for (int64_t p = 0; p < L; ++p) {
        a[p] = exp(dm[p] * a_dn);
        u[p] = dm[p] * Bn[p] * xm[p];
    }
    /* forward states, kept whole */
    for (int64_t i = 0; i < H; ++i) {
        for (int64_t j = 0; j < W; ++j) {
            const double left = (j > 0) ? hh[i * W + j - 1] : (g0 ? g0[i] : 0.0);
            hh[i * W + j] = a[i * W + j] * left + u[i * W + j];
        }
        for (int64_t j = 0; j < W; ++j) {
            const double up = (i > 0) ? h[(i - 1) * W + j] : (h0 ? h0[j] : 0.0);
            h[i * W + j] = a[i * W + j] * up + hh[i * W + j];
        }
    }
    /* adjoint of the vertical scan: bottom to top (the last row also feeds
     * the handed-out state) */
    for (int64_t i = H - 1; i >= 0; --i)
        for (int64_t j = 0; j < W; ++j) {
            const double below = (i + 1 < H) ? a[(i + 1) * W + j] * gh[(i + 1) * W + j] : (gl ? gl[j] : 0.0);
            gh[i * W + j] = dym[i * W + j] * Cn[i * W + j] + below;
        }
    if (dh0)
        for (int64_t j = 0; j < W; ++j) dh0[j] = (H > 0) ? a[j] * gh[j] : (gl ? gl[j] : 0.0);
    /* adjoint of the horizontal scan: right to left along each row (the last
     * column also feeds the handed-out row state) */
    for (int64_t i = 0; i < H; ++i) {
        for (int64_t j = W - 1; j >= 0; --j) {
            const double right = (j + 1 < W) ? a[i * W + j + 1] * ghh[i * W + j + 1] : (ggl ? ggl[i] : 0.0);
            ghh[i * W + j] = gh[i * W + j] + right;
        }
        if (dg0) dg0[i] = (W > 0) ? a[i * W] * ghh[i * W] : (ggl ? ggl[i] : 0.0);
    }
    /* local derivatives */
    double dA_sum = 0.0;
    for (int64_t i = 0; i < H; ++i)
        for (int64_t j = 0; j < W; ++j) {
            const int64_t p = i * W + j;
            const double left = (j > 0) ? hh[p - 1] : (g0 ? g0[i] : 0.0);
            const double up = (i > 0) ? h[p - W] : (h0 ? h0[j] : 0.0);
            const double g_a = ghh[p] * left + gh[p] * up;
            const double g_u = ghh[p];
            ddm[p] += g_a * a_dn * a[p] + g_u * Bn[p] * xm[p];
            dA_sum += g_a * dm[p] * a[p];
            dBn[p] += g_u * dm[p] * xm[p];
            dxm[p] += g_u * dm[p] * Bn[p];
            dCn[p] += dym[p] * h[p];
        }
    *dA_dn += dA_sum;
}

/* Internal entry: gradients of the forward pass. Inputs as for the forward
 * (x, delta, dy: [batch][d_inner][H][W]; A: [d_inner][d_state]; B, C:
 * [batch][d_state][H][W]; D: [d_inner]); outputs dx, ddelta, dA, dB, dC, dD
 * of the same shapes, overwritten. OpenMP over batch entries; the per-entry
 * dA and dD parts are added in batch order, so results do not depend on the
 * thread count. Returns 0, 2 on a bad size, 6 on allocation failure. */
static int bwd_maps(const double *x, const double *delta, const double *A, const double *B,
                    const double *C, const double *D, const double *dy, double *dx,
                    double *ddelta, double *dA, double *dB, double *dC, double *dD,
                    int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W,
                    int nthreads, const double *h0, const double *gl, double *dh0, const double *g0,
                    const double *ggl, double *dg0)
{
    if (batch < 0 || d_inner < 0 || d_state < 0 || H < 0 || W < 0) return 2;
    const int64_t L = H * W;
    memset(dx, 0, (size_t)(batch * d_inner * L) * sizeof(double));
    memset(ddelta, 0, (size_t)(batch * d_inner * L) * sizeof(double));
    memset(dA, 0, (size_t)(d_inner * d_state) * sizeof(double));
    memset(dB, 0, (size_t)(batch * d_state * L) * sizeof(double));
    memset(dC, 0, (size_t)(batch * d_state * L) * sizeof(double));
    memset(dD, 0, (size_t)d_inner * sizeof(double));
    if (batch == 0 || d_inner == 0 || L == 0) return 0;
    /* per batch entry: dA and dD parts, added in order at the end */
    double *dA_b = (double *)calloc((size_t)(batch * d_inner * d_state) + 1, sizeof(double));
    double *dD_b = (double *)calloc((size_t)(batch * d_inner) + 1, sizeof(double));
    if (!dA_b || !dD_b) {
        free(dA_b); free(dD_b);
        return 6;
    }
    int status = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t b = 0; b < batch; ++b) {
        double *buf = (double *)malloc((size_t)(6 * L) * sizeof(double));
        if (!buf) {
#pragma omp atomic write
            status = 6;
            continue;
        }
        for (int64_t d = 0; d < d_inner; ++d) {
            const int64_t m = (b * d_inner + d) * L;
            for (int64_t n = 0; n < d_state; ++n) {
                const int64_t q = (b * d_state + n) * L;
                const int64_t c = ((b * d_inner + d) * d_state + n) * W;  /* carried-state rows */
                const int64_t cr = ((b * d_inner + d) * d_state + n) * H;
                backward_one_map(x + m, delta + m, A[d * d_state + n], B + q, C + q, dy + m,
                                 dx + m, ddelta + m, dB + q, dC + q,
                                 dA_b + (b * d_inner + d) * d_state + n, H, W,
                                 buf, buf + L, buf + 2 * L, buf + 3 * L, buf + 4 * L, buf + 5 * L,
                                 h0 ? h0 + c : NULL, gl ? gl + c : NULL, dh0 ? dh0 + c : NULL,
                                 g0 ? g0 + cr : NULL, ggl ? ggl + cr : NULL, dg0 ? dg0 + cr : NULL);
            }
            double s = 0.0;
            for (int64_t p = 0; p < L; ++p) {
                dx[m + p] += dy[m + p] * D[d];
                s += dy[m + p] * x[m + p];
            }
            dD_b[b * d_inner + d] = s;
        }
        free(buf);
    }
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t d = 0; d < d_inner; ++d) {
            dD[d] += dD_b[b * d_inner + d];
            for (int64_t n = 0; n < d_state; ++n)
                dA[d * d_state + n] += dA_b[(b * d_inner + d) * d_state + n];
        }
    free(dA_b);
    free(dD_b);
    return status;
}

int oracle_ssm2d_bwd_f64(const double *x, const double *delta, const double *A, const double *B,
                         const double *C, const double *D, const double *dy, double *dx,
                         double *ddelta, double *dA, double *dB, double *dC, double *dD,
                         int64_t batch, int64_t d_inner, int64_t d_state, int64_t H, int64_t W,
                         int nthreads)
{
    return bwd_maps(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W,
                    nthreads, NULL, NULL, NULL, NULL, NULL, NULL);
}

/* The backward pass of the forward with carried vertical states: h0 (may be
 * NULL) the state above row 0 the forward started from, gl (may be NULL)
 * dL/dh_last for the state it handed out after the last row, dh0 (may be
 * NULL) receives dL/dh0; all [batch][d_inner][d_state][W]. Otherwise as
 * oracle_ssm2d_bwd_f64. */
int oracle_ssm2d_bwd_carry_f64(const double *x, const double *delta, const double *A, const double *B,
                               const double *C, const double *D, const double *dy, const double *h0,
                               const double *gl, double *dx, double *ddelta, double *dA, double *dB,
                               double *dC, double *dD, double *dh0, int64_t batch, int64_t d_inner,
                               int64_t d_state, int64_t H, int64_t W, int nthreads)
{
    if (dh0 && batch >= 0 && d_inner >= 0 && d_state >= 0 && W >= 0 && H == 0) {
        /* no rows: the handed-out state is h0 itself */
        for (int64_t k = 0; k < batch * d_inner * d_state * W; ++k) dh0[k] = gl ? gl[k] : 0.0;
    }
    return bwd_maps(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W,
                    nthreads, h0, gl, dh0, NULL, NULL, NULL);
}

/* The backward pass of a tile: carried vertical states as in
 * oracle_ssm2d_bwd_carry_f64, and carried row states g0 (the state left of
 * column 0 the forward started each row from), ggl (dL/dhh_last for the row
 * state it handed out after the last column) and dg0 (receives dL/dg0), all
 * three [batch][d_inner][d_state][H]; any may be NULL. */
int oracle_ssm2d_bwd_tile_f64(const double *x, const double *delta, const double *A, const double *B,
                              const double *C, const double *D, const double *dy, const double *h0,
                              const double *gl, const double *g0, const double *ggl, double *dx,
                              double *ddelta, double *dA, double *dB, double *dC, double *dD, double *dh0,
                              double *dg0, int64_t batch, int64_t d_inner, int64_t d_state, int64_t H,
                              int64_t W, int nthreads)
{
    if (batch >= 0 && d_inner >= 0 && d_state >= 0 && W >= 0 && H >= 0) {
        /* no rows (or no columns): a handed-out state is the carried one itself */
        if (dh0 && H == 0)
            for (int64_t k = 0; k < batch * d_inner * d_state * W; ++k) dh0[k] = gl ? gl[k] : 0.0;
        if (dg0 && W == 0)
            for (int64_t k = 0; k < batch * d_inner * d_state * H; ++k) dg0[k] = ggl ? ggl[k] : 0.0;
    }
    return bwd_maps(x, delta, A, B, C, D, dy, dx, ddelta, dA, dB, dC, dD, batch, d_inner, d_state, H, W,
                    nthreads, h0, gl, dh0, g0, ggl, dg0);
}

/* Number of threads the OpenMP runtime would use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
