/*
 * Plain fp64 CPU oracle for the SSD (Mamba-2) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark do.
 *
 * What it computes is the plain definition, not the chunked algorithm:
 * the selective state-space recurrence with a scalar-times-identity
 * transition (page "State Space Duality and Mamba-2", section "The
 * Mathematical Bridge": h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t, with
 * A_t = a_t I), discretised by the step size dt as on page "NVIDIA
 * Accelerates Mamba-2 Forward Kernel with CUDA Tile" (section "What CUDA
 * Tile Is", dt sets A_bar and B_bar):
 *
 *     a_t      = exp(dt_t * A_h)
 *     h_t      = a_t * h_{t-1} + dt_t * x_t B_t^T        (P x N per head)
 *     y_t      = h_t C_t + D_h * x_t
 *
 * Document packing (page "Parallel Scan and Hardware-Aware SSM Kernels",
 * section "When it breaks"): where seq_idx changes between t-1 and t the
 * state is reset, i.e. a_t is masked to zero, so no information crosses a
 * document boundary.  init_states feeds only the first document of a row;
 * final_states is the state after the row's last token.
 *
 * Grouped B/C (page "State Space Duality and Mamba-2", section
 * "Architectural Scaling", grouped-query SSM): head h reads group
 * g = h / (nheads / ngroups).
 *
 * Layouts (dense, row-major): x, y [b, L, H, P]; dt [b, L, H]; A, D [H];
 * B, C [b, L, G, N]; seq_idx [b, L]; init/final states [b, H, P, N].
 * Everything is double; the caller widens fp32/bf16 values exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Returns 0 on success, 1 on bad arguments, 2 on allocation failure. */
int ssd_oracle_fwd_f64(int64_t batch, int64_t seqlen, int64_t nheads,
                       int64_t headdim, int64_t dstate, int64_t ngroups,
                       const double *x, const double *dt, const double *A,
                       const double *B, const double *C,
                       const double *D,            /* nullable: no skip */
                       const int32_t *seq_idx,     /* nullable: one document */
                       const double *init_states,  /* nullable: zero */
                       double *y,
                       double *final_states,       /* nullable */
                       int nthreads)
{
    if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 ||
        dstate <= 0 || ngroups <= 0 || nheads % ngroups != 0)
        return 1;
    if (!x || !dt || !A || !B || !C || !y)
        return 1;
    const int64_t H = nheads, P = headdim, N = dstate, G = ngroups;
    const int64_t heads_per_group = H / G;
    const int64_t units = batch * H;
    int failed = 0;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int64_t b = u / H, h = u % H;
        const int64_t g = h / heads_per_group;
        double *S = (double *)malloc((size_t)(P * N) * sizeof(double));
        if (!S) {
            failed |= 1;
            continue;
        }
        if (init_states)
            memcpy(S, init_states + (b * H + h) * P * N,
                   (size_t)(P * N) * sizeof(double));
        else
            memset(S, 0, (size_t)(P * N) * sizeof(double));
        const double Ah = A[h];
        const double Dh = D ? D[h] : 0.0;
        for (int64_t t = 0; t < seqlen; ++t) {
            if (seq_idx && t > 0 && seq_idx[b * seqlen + t] != seq_idx[b * seqlen + t - 1])
                memset(S, 0, (size_t)(P * N) * sizeof(double));
            const double dtv = dt[(b * seqlen + t) * H + h];
            const double a = exp(dtv * Ah);
            const double *xt = x + ((b * seqlen + t) * H + h) * P;
            const double *Bt = B + ((b * seqlen + t) * G + g) * N;
            const double *Ct = C + ((b * seqlen + t) * G + g) * N;
            double *yt = y + ((b * seqlen + t) * H + h) * P;
            for (int64_t p = 0; p < P; ++p) {
                double *Sp = S + p * N;
                const double ux = dtv * xt[p];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    Sp[n] = a * Sp[n] + ux * Bt[n];
                    acc += Ct[n] * Sp[n];
                }
                yt[p] = acc + Dh * xt[p];
            }
        }
        if (final_states)
            memcpy(final_states + (b * H + h) * P * N, S,
                   (size_t)(P * N) * sizeof(double));
        free(S);
    }
    return failed ? 2 : 0;
}

/* Number of threads an OpenMP parallel region would use. */
int ssd_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
