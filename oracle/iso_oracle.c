/*
 * Test infrastructure: the CPU oracle for the weighted isotonic fit.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * this code.  The GPU library never links, includes or calls it, and it shares
 * no code with the GPU library.
 *
 * What it computes (paper "Merge Hulls Without Copying Vertices: GPU Isotonic
 * Regression", section 2.1, equation (1)):
 *
 *     z* = argmin  sum_i w_i (z_i - y_i)^2   subject to  z_1 <= z_2 <= ... <= z_n,
 *
 * with all w_i > 0.  The solution is unique and piecewise constant; on each block
 * of consecutive indices it equals the weighted mean of y over the block
 * (same section).  The oracle reaches it with pool adjacent violators (the
 * sequential algorithm named in the same section and restated on the blog note
 * "Isotonic Regression on GPU", section "A curve that is only allowed to go up",
 * and on the Mova groupant card for isotonic_regression/mod.rs, "Forward"):
 * every element starts as its own block; while the block before the last has a
 * mean that is not below the last block's mean, the two are pooled.
 *
 * Readings taken where the pages leave a step open:
 *  - Equal adjacent means are pooled (the paper's convention that a point on the
 *    segment between its neighbours is not a hull vertex, section 2.1), so the
 *    oracle's blocks have strictly increasing means.  The fit itself does not
 *    depend on this choice.
 *  - Means are compared by cross-multiplication in f64, valid because every
 *    block weight is positive.
 *  - Everything is accumulated in f64 (double), one pass, left to right.
 *
 * Also here, as independent checks of the PAVA routine (tests only):
 *  - oracle_brute_force: minimum weighted squared error over all 2^(n-1)
 *    contiguous partitions whose block means do not decrease (the Mova
 *    groupant card's "kkt_prefix" entry names enumeration of contiguous
 *    partitions as an independent check of the least-squares optimum).
 *  - oracle_hull_fit: the slope sequence of the lower convex hull of the
 *    cumulative sum diagram (paper section 2.1, equations (2) and (3)), built
 *    with a monotone chain that drops points on or above a chord.
 *
 * Also here: oracle_vjp_f64, the vector-Jacobian product of the fit (block
 * averaging of the incoming gradient, paper section 6, "Gradient").
 *
 * Compile-time switch ORACLE_MUTANT=k (k >= 1) plants one deliberate mistake:
 * k = 1..6 in the PAVA routine, k = 7..10 in the vector-Jacobian product.  It
 * exists only so that the test suite can show that its pins catch each planted
 * mistake; the default build (no switch) has none.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* One block of pool adjacent violators: total weight, weighted sum of y, and
 * the index of its first element. */
typedef struct {
    double sw;
    double swy;
    int64_t start;
} oracle_block;

/*
 * Weighted PAVA over one row.
 *   y[n], w[n] (w == NULL means unit weights), all finite, w > 0.
 *   z[n]       receives the f64 fit.
 *   block_id   (may be NULL) receives the 0-based index of each element's block.
 * Returns the number of blocks, or -1 when the scratch allocation fails.
 */
int64_t oracle_pava_f64(const double* y, const double* w, int64_t n, double* z,
                        int32_t* block_id) {
    if (n <= 0) return 0;
    oracle_block* st = (oracle_block*)malloc((size_t)n * sizeof(oracle_block));
    if (!st) return -1;
    int64_t top = 0; /* number of blocks on the stack */
    for (int64_t i = 0; i < n; ++i) {
        double wi = w ? w[i] : 1.0;
#if ORACLE_MUTANT == 1 /* mistake: weights ignored when pooling */
        wi = 1.0;
#endif
        st[top].sw = wi;
#if ORACLE_MUTANT == 2 /* mistake: the weighted sum drops the weight */
        st[top].swy = y[i];
#else
        st[top].swy = wi * y[i];
#endif
        st[top].start = i;
        ++top;
#if ORACLE_MUTANT == 3 /* mistake: pools at most once per element */
        if (top >= 2) {
#else
        while (top >= 2) {
#endif
            oracle_block* a = &st[top - 2];
            oracle_block* b = &st[top - 1];
            /* mean(a) >= mean(b)  <=>  swy_a * sw_b >= swy_b * sw_a  (sw > 0) */
#if ORACLE_MUTANT == 4 /* mistake: comparison reversed */
            int violated = a->swy * b->sw <= b->swy * a->sw;
#else
            int violated = a->swy * b->sw >= b->swy * a->sw;
#endif
            if (!violated) break;
            a->sw += b->sw;
            a->swy += b->swy;
            --top;
        }
    }
    for (int64_t b = 0; b < top; ++b) {
        int64_t end = (b + 1 < top) ? st[b + 1].start : n;
#if ORACLE_MUTANT == 5 /* mistake: mean divided by the element count */
        double mean = st[b].swy / (double)(end - st[b].start);
#else
        double mean = st[b].swy / st[b].sw;
#endif
        for (int64_t i = st[b].start; i < end; ++i) {
            z[i] = mean;
            if (block_id) block_id[i] = (int32_t)b;
        }
#if ORACLE_MUTANT == 6 /* mistake: a block's first element keeps the previous mean */
        if (b > 0) z[st[b].start] = z[st[b].start - 1];
#endif
    }
    free(st);
    return top;
}

/*
 * Rows of one common length, row-major; f32 inputs widened exactly to f64,
 * f32 output rounded once (round to nearest even) from the f64 fit, as the
 * paper's section 6 ("Output") asks of the working type.
 *   out64 (may be NULL) receives the f64 fit as well.
 * Returns 0, or -1 on allocation failure.
 */
int oracle_fit_rows_f32(const float* y, const float* w, int64_t rows, int64_t n,
                        float* out, double* out64, int32_t* block_id) {
    if (rows <= 0 || n <= 0) return 0;
    double* yd = (double*)malloc((size_t)n * sizeof(double));
    double* wd = w ? (double*)malloc((size_t)n * sizeof(double)) : NULL;
    double* zd = (double*)malloc((size_t)n * sizeof(double));
    if (!yd || !zd || (w && !wd)) {
        free(yd); free(wd); free(zd);
        return -1;
    }
    int rc = 0;
    for (int64_t r = 0; r < rows; ++r) {
        const float* yr = y + r * n;
        for (int64_t i = 0; i < n; ++i) yd[i] = (double)yr[i];
        if (w) {
            const float* wr = w + r * n;
            for (int64_t i = 0; i < n; ++i) wd[i] = (double)wr[i];
        }
        if (oracle_pava_f64(yd, wd, n, zd, block_id ? block_id + r * n : NULL) < 0) {
            rc = -1;
            break;
        }
        float* o = out + r * n;
        for (int64_t i = 0; i < n; ++i) o[i] = (float)zd[i];
        if (out64) memcpy(out64 + r * n, zd, (size_t)n * sizeof(double));
    }
    free(yd); free(wd); free(zd);
    return rc;
}

/*
 * Brute force over all contiguous partitions (n <= 24).  A partition is
 * feasible when its block means do not decrease; among feasible partitions the
 * one of least weighted squared error gives z.  Returns that error, or -1.0 if
 * n is out of range.
 */
double oracle_brute_force(const double* y, const double* w, int n, double* z) {
    if (n <= 0 || n > 24) return -1.0;
    double best = INFINITY;
    double mean[24];
    int first[24];
    uint32_t ncut = 1u << (n - 1);
    for (uint32_t cuts = 0; cuts < ncut; ++cuts) {
        /* bit k of cuts set: a block ends after element k */
        int nb = 0;
        int s = 0;
        int feasible = 1;
        double err = 0.0;
        for (int i = 0; i < n; ++i) {
            int ends = (i == n - 1) || ((cuts >> i) & 1u);
            if (!ends) continue;
            double sw = 0.0, swy = 0.0;
            for (int k = s; k <= i; ++k) {
                double wk = w ? w[k] : 1.0;
                sw += wk;
                swy += wk * y[k];
            }
            double m = swy / sw;
            if (nb > 0 && m < mean[nb - 1]) {
                feasible = 0;
                break;
            }
            for (int k = s; k <= i; ++k) {
                double wk = w ? w[k] : 1.0;
                err += wk * (y[k] - m) * (y[k] - m);
            }
            mean[nb] = m;
            first[nb] = s;
            ++nb;
            s = i + 1;
        }
        if (!feasible || !(err < best)) continue;
        best = err;
        for (int b = 0; b < nb; ++b) {
            int e = (b + 1 < nb) ? first[b + 1] : n;
            for (int k = first[b]; k < e; ++k) z[k] = mean[b];
        }
    }
    return best;
}

/*
 * The fit as slopes of the lower convex hull of the cumulative sum diagram
 * P_k = (W_k, S_k), P_0 = (0, 0) (paper section 2.1, equations (2)-(3)).
 * Monotone chain: a point is dropped while it lies on or above the segment
 * from the point under it to the new point.  z_i is the slope of the hull
 * edge above [W_{i-1}, W_i].  Returns the number of hull vertices, or -1.
 */
int64_t oracle_hull_fit(const double* y, const double* w, int64_t n, double* z) {
    if (n <= 0) return 0;
    double* W = (double*)malloc((size_t)(n + 1) * sizeof(double));
    double* S = (double*)malloc((size_t)(n + 1) * sizeof(double));
    int64_t* h = (int64_t*)malloc((size_t)(n + 1) * sizeof(int64_t));
    if (!W || !S || !h) {
        free(W); free(S); free(h);
        return -1;
    }
    W[0] = 0.0;
    S[0] = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double wi = w ? w[i] : 1.0;
        W[i + 1] = W[i] + wi;
        S[i + 1] = S[i] + wi * y[i];
    }
    int64_t top = 0;
    for (int64_t k = 0; k <= n; ++k) {
        while (top >= 2) {
            int64_t a = h[top - 2], b = h[top - 1];
            /* cross product of (b - a) and (k - a): <= 0 means b is on or above
             * the chord from a to k */
            double cross = (W[b] - W[a]) * (S[k] - S[a]) - (S[b] - S[a]) * (W[k] - W[a]);
            if (cross > 0.0) break;
            --top;
        }
        h[top++] = k;
    }
    for (int64_t v = 0; v + 1 < top; ++v) {
        int64_t a = h[v], b = h[v + 1];
        double slope = (S[b] - S[a]) / (W[b] - W[a]);
        for (int64_t i = a; i < b; ++i) z[i] = slope;
    }
    free(W); free(S); free(h);
    return top;
}

/*
 * Vector-Jacobian product of the fit (paper "Merge Hulls Without Copying
 * Vertices: GPU Isotonic Regression", section 6, paragraph "Gradient").  The
 * fit is constant on blocks, each block's value the weighted mean z of y over
 * it, so its Jacobian averages over blocks.  With g the gradient with respect
 * to the fit and, over an element's block, G the sum of g and W the sum of w:
 *     d/dy_i = w_i G / W,        d/dw_i = (y_i - z) G / W,
 * wherever the blocks do not change.
 *   y[n], w[n] (NULL: unit weights), g[n]   f64.
 *   block_id   the blocks to differentiate over (a block starts at element 0
 *              and wherever the id changes), or NULL for this oracle's own
 *              PAVA blocks.  A row whose first id is negative (a non-finite
 *              row of the fit) gets NaN.
 *   gy, gw     (either may be NULL) receive the gradients in f64.
 * Every sum is formed left to right over the block in f64.
 * Returns 0, or -1 when a scratch allocation fails.
 */
int oracle_vjp_f64(const double* y, const double* w, const double* g, const int32_t* block_id,
                   int64_t n, double* gy, double* gw) {
    if (n <= 0) return 0;
    int32_t* own = NULL;
    const int32_t* bid = block_id;
    if (!bid) {
        double* z = (double*)malloc((size_t)n * sizeof(double));
        own = (int32_t*)malloc((size_t)n * sizeof(int32_t));
        if (!z || !own) {
            free(z); free(own);
            return -1;
        }
        if (oracle_pava_f64(y, w, n, z, own) < 0) {
            free(z); free(own);
            return -1;
        }
        free(z);
        bid = own;
    }
    if (bid[0] < 0) {
        for (int64_t i = 0; i < n; ++i) {
            if (gy) gy[i] = NAN;
            if (gw) gw[i] = NAN;
        }
        free(own);
        return 0;
    }
    int64_t a = 0;
    while (a < n) {
        int64_t b = a + 1; /* the block is [a, b) */
        while (b < n && bid[b] == bid[a]) ++b;
#if ORACLE_MUTANT == 10 /* mistake: the block's sums run one element too far */
        int64_t bs = b < n ? b + 1 : b;
#else
        int64_t bs = b;
#endif
        double G = 0.0, W = 0.0, S = 0.0;
        for (int64_t i = a; i < bs; ++i) {
            double wi = w ? w[i] : 1.0;
            G += g[i];
            W += wi;
            S += wi * y[i];
        }
#if ORACLE_MUTANT == 9 /* mistake: G divided by the element count, not by W */
        double r = G / (double)(bs - a);
#else
        double r = G / W;
#endif
        double z = S / W;
        for (int64_t i = a; i < b; ++i) {
            double wi = w ? w[i] : 1.0;
#if ORACLE_MUTANT == 7 /* mistake: the weight factor of d/dy dropped */
            if (gy) gy[i] = r;
#else
            if (gy) gy[i] = wi * r;
#endif
#if ORACLE_MUTANT == 8 /* mistake: d/dw with its sign reversed */
            if (gw) gw[i] = (z - y[i]) * r;
#else
            if (gw) gw[i] = (y[i] - z) * r;
#endif
        }
        a = b;
    }
    free(own);
    return 0;
}

/*
 * Rows of one common length, row-major, f32 inputs widened exactly to f64:
 * the vector-Jacobian product of each row's fit (oracle_vjp_f64 per row).
 *   w may be NULL (unit weights); block_id may be NULL (own blocks).
 *   gy64, gw64 (either may be NULL) receive the f64 gradients.
 * Returns 0, or -1 on allocation failure.
 */
int oracle_vjp_rows_f32(const float* y, const float* w, const float* g, const int32_t* block_id,
                        int64_t rows, int64_t n, double* gy64, double* gw64) {
    if (rows <= 0 || n <= 0) return 0;
    double* yd = (double*)malloc((size_t)n * sizeof(double));
    double* wd = w ? (double*)malloc((size_t)n * sizeof(double)) : NULL;
    double* gd = (double*)malloc((size_t)n * sizeof(double));
    if (!yd || !gd || (w && !wd)) {
        free(yd); free(wd); free(gd);
        return -1;
    }
    int rc = 0;
    for (int64_t r = 0; r < rows && rc == 0; ++r) {
        for (int64_t i = 0; i < n; ++i) {
            yd[i] = (double)y[r * n + i];
            gd[i] = (double)g[r * n + i];
            if (w) wd[i] = (double)w[r * n + i];
        }
        rc = oracle_vjp_f64(yd, wd, gd, block_id ? block_id + r * n : NULL, n,
                            gy64 ? gy64 + r * n : NULL, gw64 ? gw64 + r * n : NULL);
    }
    free(yd); free(wd); free(gd);
    return rc;
}
