/*
 * Test infrastructure: a driver that runs every oracle routine on seeded
 * inputs (sizes 0 to 3000, ties, constant and strictly monotone rows, tiny
 * brute-force cases, block ids given and own, non-finite rows of the block
 * ids) so that the oracle can be built and run under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitized.py).  It checks
 * nothing of the results itself; the sanitizers end the run on any invalid
 * access or undefined operation.  Exit status 0 when every call returned.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int64_t oracle_pava_f64(const double* y, const double* w, int64_t n, double* z, int32_t* block_id);
int oracle_fit_rows_f32(const float* y, const float* w, int64_t rows, int64_t n, float* out,
                        double* out64, int32_t* block_id);
double oracle_brute_force(const double* y, const double* w, int n, double* z);
int64_t oracle_hull_fit(const double* y, const double* w, int64_t n, double* z);
int oracle_vjp_f64(const double* y, const double* w, const double* g, const int32_t* block_id,
                   int64_t n, double* gy, double* gw);
int oracle_vjp_rows_f32(const float* y, const float* w, const float* g, const int32_t* block_id,
                        int64_t rows, int64_t n, double* gy64, double* gw64);

static uint64_t rng_state = 88172645463325252ull;
static double next_unit(void) { /* xorshift64 */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}

int main(void) {
    const int64_t sizes[] = {0, 1, 2, 3, 7, 64, 65, 1000, 3000};
    for (int si = 0; si < (int)(sizeof(sizes) / sizeof(sizes[0])); ++si) {
        const int64_t n = sizes[si];
        const size_t nn = n > 0 ? (size_t)n : 1;
        for (int kind = 0; kind < 5; ++kind) {
            double* y = malloc(nn * sizeof(double));
            double* w = malloc(nn * sizeof(double));
            double* g = malloc(nn * sizeof(double));
            double* z = malloc(nn * sizeof(double));
            double* gy = malloc(nn * sizeof(double));
            double* gw = malloc(nn * sizeof(double));
            int32_t* b = malloc(nn * sizeof(int32_t));
            for (int64_t i = 0; i < n; ++i) {
                if (kind == 0) y[i] = next_unit();
                else if (kind == 1) y[i] = (double)(int)(4 * next_unit());  /* ties */
                else if (kind == 2) y[i] = 0.5;                              /* constant */
                else if (kind == 3) y[i] = (double)i;                        /* increasing */
                else y[i] = -(double)i;                                      /* decreasing */
                w[i] = 0.1 + next_unit();
                g[i] = next_unit() - 0.5;
            }
            int64_t nb = oracle_pava_f64(y, kind % 2 ? w : NULL, n, z, b);
            (void)oracle_hull_fit(y, kind % 2 ? NULL : w, n, z);
            (void)oracle_vjp_f64(y, w, g, NULL, n, gy, gw);
            (void)oracle_vjp_f64(y, NULL, g, n > 0 ? b : NULL, n, gy, NULL);
            if (n > 0 && nb > 0) {
                b[0] = -1; /* a non-finite row's ids */
                for (int64_t i = 1; i < n; ++i) b[i] = -1;
                (void)oracle_vjp_f64(y, w, g, b, n, gy, gw);
            }
            if (n >= 1 && n <= 12) (void)oracle_brute_force(y, kind % 2 ? w : NULL, (int)n, z);
            free(y); free(w); free(g); free(z); free(gy); free(gw); free(b);
        }
    }
    /* rows of f32 */
    const int64_t rows = 5, n = 777;
    float* yf = malloc(rows * n * sizeof(float));
    float* wf = malloc(rows * n * sizeof(float));
    float* gf = malloc(rows * n * sizeof(float));
    float* of = malloc(rows * n * sizeof(float));
    double* o64 = malloc(rows * n * sizeof(double));
    double* gy64 = malloc(rows * n * sizeof(double));
    double* gw64 = malloc(rows * n * sizeof(double));
    int32_t* bid = malloc(rows * n * sizeof(int32_t));
    for (int64_t i = 0; i < rows * n; ++i) {
        yf[i] = (float)next_unit();
        wf[i] = (float)(0.5 + next_unit());
        gf[i] = (float)(next_unit() - 0.5);
    }
    if (oracle_fit_rows_f32(yf, wf, rows, n, of, o64, bid) != 0) return 1;
    if (oracle_fit_rows_f32(yf, NULL, rows, n, of, NULL, NULL) != 0) return 1;
    if (oracle_vjp_rows_f32(yf, wf, gf, bid, rows, n, gy64, gw64) != 0) return 1;
    if (oracle_vjp_rows_f32(yf, NULL, gf, NULL, rows, n, gy64, NULL) != 0) return 1;
    free(yf); free(wf); free(gf); free(of); free(o64); free(gy64); free(gw64); free(bid);
    printf("oracle sanitized run: ok\n");
    return 0;
}
