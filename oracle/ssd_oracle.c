/*
 * ssd_oracle.c -- float64 CPU oracle for the SSD (structured state space
 * duality) layer forward.  TEST INFRASTRUCTURE ONLY: it is linked by the test
 * suite, the smoke check and the benchmark's CPU-baseline leg, never by the
 * product library, and it shares no code with the HIP path.
 *
 * What it computes is the plain definition of the layer, the linear
 * (recurrent) mode of a scalar-identity SSM:
 *   - "Transformers are SSMs" (paper summary page), section 2.4 "SSD layer
 *     overview": A_t is a scalar times the identity, head dimension P > 1;
 *   - same page, section 3.4.1 "linear (recurrent) mode": expand x by B, run
 *     the scalar recurrence, contract by C;
 *   - same page, section 5.1: A_t = a_t I, so every one of the P*N state
 *     entries obeys one shared scalar recurrence.
 * Per head (head h reads group g = h / (H/G), section 7.2 grouped-input heads):
 *     S   = a_t * S + x_t (outer) B_t         S is P x N, S[p][n]
 *     y_t = S C_t                             y_t[p] = sum_n S[p][n] C_t[n]
 * with a_t = exp(logA_t).  The state before the first token is init (zeros
 * when absent), so token 0 sees S = a_0 * init + x_0 B_0^T; the state after
 * the last token is returned as the final state.  With seq_offsets the packed
 * batch is a list of independent sequences (section 8.3 variable length):
 * no state crosses a sequence boundary and each sequence starts from its own
 * init.
 *
 * Layouts (row-major, float64):
 *   X [batch, T, H, P]; logA [batch, T, H]; B, C [batch, T, G, N];
 *   init, final [nseq, H, P, N]; seq_offsets [nseq + 1] (batch must be 1).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int ssd_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Returns 0 on success, -1 on a malformed argument, -2 on allocation failure. */
int ssd_oracle_recurrence(int64_t batch, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G,
                          const double* X, const double* logA, const double* B, const double* C,
                          const double* init, const int64_t* seq_offsets, int64_t nseq,
                          double* Y, double* final_state, int nthreads) {
    if (batch < 1 || T < 0 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0) return -1;
    if (seq_offsets) {
        if (batch != 1 || nseq < 1 || seq_offsets[0] != 0 || seq_offsets[nseq] != T) return -1;
        for (int64_t s = 0; s < nseq; ++s)
            if (seq_offsets[s + 1] < seq_offsets[s]) return -1;
    } else {
        nseq = batch;
    }
    const int64_t heads_per_group = H / G;
    const int64_t ntask = nseq * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t task = 0; task < ntask; ++task) {
        const int64_t s = task / H, h = task % H;
        const int64_t g = h / heads_per_group;
        /* token rows of this sequence, as indices into the flattened [batch*T] axis */
        int64_t row0, row1;
        if (seq_offsets) { row0 = seq_offsets[s]; row1 = seq_offsets[s + 1]; }
        else { row0 = s * T; row1 = (s + 1) * T; }
        double* S = (double*)malloc((size_t)(P * N) * sizeof(double));
        if (!S) { failed = 1; continue; }
        if (init) memcpy(S, init + (s * H + h) * P * N, (size_t)(P * N) * sizeof(double));
        else memset(S, 0, (size_t)(P * N) * sizeof(double));
        for (int64_t r = row0; r < row1; ++r) {
            const double a = exp(logA[r * H + h]);
            const double* x = X + (r * H + h) * P;
            const double* b = B + (r * G + g) * N;
            const double* c = C + (r * G + g) * N;
            double* y = Y + (r * H + h) * P;
            for (int64_t p = 0; p < P; ++p) {
                double* Sp = S + p * N;
                const double xp = x[p];
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    Sp[n] = a * Sp[n] + xp * b[n];
                    acc += Sp[n] * c[n];
                }
                y[p] = acc;
            }
        }
        if (final_state) memcpy(final_state + (s * H + h) * P * N, S, (size_t)(P * N) * sizeof(double));
        free(S);
    }
    return failed ? -2 : 0;
}
