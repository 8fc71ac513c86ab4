/* Driver of the sanitizer build of the C oracle (oracle/ssd_oracle.c): runs
 * the fp64 recurrence on small random problems -- one token, ragged lengths,
 * grouped B/C, document resets, initial states, no D -- and checks identities
 * that hold exactly in the recurrence (B = 0 gives y = D x; one token from a
 * zero state gives y = dt (C.B) x + D x; a reset at every token gives the
 * same per-token result).  AddressSanitizer / UndefinedBehaviorSanitizer
 * abort on a finding; exit status 1 on a failed identity. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ssd_oracle_fwd_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                       int64_t ngroups, const double *x, const double *dt, const double *A,
                       const double *B, const double *C, const double *D, const int32_t *seq_idx,
                       const double *init_states, double *y, double *final_states, int nthreads);

static uint64_t g_rng = 88172645463325252ull;
static double urand(void) {
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 7;
    g_rng ^= g_rng << 17;
    return (double)(g_rng >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double *arr(size_t n, double scale) {
    double *p = malloc((n ? n : 1) * sizeof(double));
    for (size_t k = 0; k < n; ++k) p[k] = urand() * scale;
    return p;
}

static int g_fail = 0;

static void one(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int with_seq, int with_h0,
                int with_D) {
    const size_t nx = (size_t)(b * L * H * P), nbc = (size_t)(b * L * G * N), nst = (size_t)(b * H * P * N);
    double *x = arr(nx, 1.0), *dt = arr((size_t)(b * L * H), 0.5), *A = arr((size_t)H, 2.0);
    double *B = arr(nbc, 0.3), *C = arr(nbc, 0.3), *D = with_D ? arr((size_t)H, 1.0) : NULL;
    double *h0 = with_h0 ? arr(nst, 1.0) : NULL;
    for (size_t k = 0; k < (size_t)(b * L * H); ++k) dt[k] = fabs(dt[k]) + 1e-3;
    for (int64_t h = 0; h < H; ++h) A[h] = -fabs(A[h]);
    int32_t *seq = NULL;
    if (with_seq) {
        seq = malloc((size_t)(b * L) * sizeof(int32_t));
        for (int64_t r = 0; r < b; ++r) {
            int32_t id = 0;
            for (int64_t t = 0; t < L; ++t) {
                if (t > 0 && urand() > 0.8) ++id;
                seq[r * L + t] = id;
            }
        }
    }
    double *y = malloc(nx * sizeof(double)), *fs = malloc(nst * sizeof(double));
    if (ssd_oracle_fwd_f64(b, L, H, P, N, G, x, dt, A, B, C, D, seq, h0, y, fs, 2) != 0) {
        fprintf(stderr, "FAIL: oracle rejected b%lld L%lld\n", (long long)b, (long long)L);
        g_fail = 1;
    }
    /* B = 0 and no initial state: y = D x exactly */
    if (!with_h0) {
        double *B0 = calloc(nbc ? nbc : 1, sizeof(double));
        ssd_oracle_fwd_f64(b, L, H, P, N, G, x, dt, A, B0, C, D, seq, NULL, y, fs, 1);
        for (int64_t r = 0; r < b; ++r)
            for (int64_t t = 0; t < L; ++t)
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t p = 0; p < P; ++p) {
                        const size_t i = (size_t)(((r * L + t) * H + h) * P + p);
                        const double want = D ? D[h] * x[i] : 0.0;
                        if (y[i] != want) {
                            fprintf(stderr, "FAIL: B = 0 gives y %g, want %g\n", y[i], want);
                            g_fail = 1;
                            goto out0;
                        }
                    }
    out0:
        free(B0);
    }
    /* one token from a zero state: y = dt (C.B) x + D x */
    {
        double *y1 = malloc((size_t)(b * H * P) * sizeof(double)), *fs1 = malloc(nst * sizeof(double));
        double *x1 = malloc((size_t)(b * H * P) * sizeof(double)), *dt1 = malloc((size_t)(b * H) * sizeof(double));
        double *B1 = malloc((size_t)(b * G * N) * sizeof(double)), *C1 = malloc((size_t)(b * G * N) * sizeof(double));
        for (int64_t r = 0; r < b; ++r) {
            memcpy(x1 + r * H * P, x + (size_t)(r * L * H * P), (size_t)(H * P) * sizeof(double));
            memcpy(dt1 + r * H, dt + (size_t)(r * L * H), (size_t)H * sizeof(double));
            memcpy(B1 + r * G * N, B + (size_t)(r * L * G * N), (size_t)(G * N) * sizeof(double));
            memcpy(C1 + r * G * N, C + (size_t)(r * L * G * N), (size_t)(G * N) * sizeof(double));
        }
        ssd_oracle_fwd_f64(b, 1, H, P, N, G, x1, dt1, A, B1, C1, D, NULL, NULL, y1, fs1, 1);
        for (int64_t r = 0; r < b; ++r)
            for (int64_t h = 0; h < H; ++h) {
                const int64_t g = h / (H / G);
                double cb = 0.0;
                for (int64_t n = 0; n < N; ++n) cb += C1[(r * G + g) * N + n] * B1[(r * G + g) * N + n];
                for (int64_t p = 0; p < P; ++p) {
                    const double xv = x1[(r * H + h) * P + p];
                    const double want = dt1[r * H + h] * cb * xv + (D ? D[h] * xv : 0.0);
                    const double got = y1[(r * H + h) * P + p];
                    if (fabs(got - want) > 1e-12 * (1.0 + fabs(want))) {
                        fprintf(stderr, "FAIL: one token y %g, want %g\n", got, want);
                        g_fail = 1;
                    }
                }
            }
        free(y1); free(fs1); free(x1); free(dt1); free(B1); free(C1);
    }
    free(x); free(dt); free(A); free(B); free(C); free(D); free(h0); free(seq); free(y); free(fs);
}

int main(void) {
    one(1, 1, 1, 1, 1, 1, 0, 0, 1);
    one(2, 37, 4, 8, 5, 2, 1, 1, 1);
    one(1, 130, 2, 16, 16, 1, 1, 0, 0);
    one(3, 64, 6, 4, 8, 3, 0, 1, 0);
    one(2, 200, 2, 3, 7, 1, 1, 0, 1);
    if (g_fail) return 1;
    printf("oracle driver: all checks passed\n");
    return 0;
}
