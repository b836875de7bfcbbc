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

/*
 * Reverse-mode derivative of ssd_oracle_recurrence: the adjoint recurrence.
 * For L = <dY, Y> + <dfinal, final> (dfinal NULL means zero), it returns dL
 * with respect to every input.  Let G be the adjoint of the state S.  Walking
 * the tokens of a sequence backwards from G = dfinal:
 *     G       += dy_t C_t^T             y_t = S_t C_t
 *     dC_t    += S_t^T dy_t             (summed over the heads of the group)
 *     dx_t     = G B_t                  S_t = a_t S_{t-1} + x_t B_t^T
 *     dB_t    += G^T x_t                (summed over the heads of the group)
 *     dlogA_t  = a_t <G, S_{t-1}>       a_t = exp(logA_t)
 *     G        = a_t G                  (the adjoint of S_{t-1})
 * and dinit = G after the first token (= dfinal for an empty sequence).
 * S_{t-1} comes from the forward recurrence: the state is stored every
 * kCheckpoint tokens and each stretch is recomputed from its checkpoint during
 * the backward walk.  One task per (sequence, group); the heads of a group are
 * walked one after the other, so dB and dC accumulate without races.
 * dX [rows, H, P], dlogA [rows, H], dB, dC [rows, G, N], dinit [nseq, H, P, N]
 * (dinit may be NULL).
 */
enum { kCheckpoint = 64 };

int ssd_oracle_backward(int64_t batch, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G,
                        const double* X, const double* logA, const double* B, const double* C,
                        const double* init, const int64_t* seq_offsets, int64_t nseq,
                        const double* dY, const double* dfinal,
                        double* dX, double* dlogA, double* dB, double* dC, double* dinit,
                        int nthreads) {
    if (batch < 1 || T < 0 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0) return -1;
    if (seq_offsets) {
        if (batch != 1 || nseq < 1 || seq_offsets[0] != 0 || seq_offsets[nseq] != T) return -1;
        for (int64_t s = 0; s < nseq; ++s)
            if (seq_offsets[s + 1] < seq_offsets[s]) return -1;
    } else {
        nseq = batch;
    }
    const int64_t rows = batch * T, PN = P * N;
    memset(dB, 0, (size_t)(rows * G * N) * sizeof(double));
    memset(dC, 0, (size_t)(rows * G * N) * sizeof(double));
    const int64_t heads_per_group = H / G;
    const int64_t ntask = nseq * G;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t task = 0; task < ntask; ++task) {
        const int64_t s = task / G, g = task % G;
        int64_t row0, row1;
        if (seq_offsets) { row0 = seq_offsets[s]; row1 = seq_offsets[s + 1]; }
        else { row0 = s * T; row1 = (s + 1) * T; }
        const int64_t len = row1 - row0;
        const int64_t nck = (len + kCheckpoint - 1) / kCheckpoint;
        double* ck = (double*)malloc((size_t)((nck > 0 ? nck : 1) * PN) * sizeof(double));
        double* St = (double*)malloc((size_t)(kCheckpoint * PN) * sizeof(double));
        double* Gm = (double*)malloc((size_t)PN * sizeof(double));
        if (!ck || !St || !Gm) { failed = 1; free(ck); free(St); free(Gm); continue; }
        for (int64_t h = g * heads_per_group; h < (g + 1) * heads_per_group; ++h) {
            /* forward: ck[j] = the state before token row0 + j * kCheckpoint */
            double* S = Gm;   /* scratch for the forward walk */
            if (init) memcpy(S, init + (s * H + h) * PN, (size_t)PN * sizeof(double));
            else memset(S, 0, (size_t)PN * sizeof(double));
            for (int64_t r = row0; r < row1; ++r) {
                if ((r - row0) % kCheckpoint == 0)
                    memcpy(ck + ((r - row0) / kCheckpoint) * PN, S, (size_t)PN * sizeof(double));
                const double a = exp(logA[r * H + h]);
                const double* x = X + (r * H + h) * P;
                const double* b = B + (r * G + g) * N;
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n) S[p * N + n] = a * S[p * N + n] + x[p] * b[n];
            }
            /* backward */
            if (dfinal) memcpy(Gm, dfinal + (s * H + h) * PN, (size_t)PN * sizeof(double));
            else memset(Gm, 0, (size_t)PN * sizeof(double));
            for (int64_t j = nck - 1; j >= 0; --j) {
                const int64_t t0 = row0 + j * kCheckpoint;
                const int64_t t1 = t0 + kCheckpoint < row1 ? t0 + kCheckpoint : row1;
                /* St[i] = the state after token t0 + i */
                for (int64_t r = t0; r < t1; ++r) {
                    const double* prev = r == t0 ? ck + j * PN : St + (r - 1 - t0) * PN;
                    double* cur = St + (r - t0) * PN;
                    const double a = exp(logA[r * H + h]);
                    const double* x = X + (r * H + h) * P;
                    const double* b = B + (r * G + g) * N;
                    for (int64_t p = 0; p < P; ++p)
                        for (int64_t n = 0; n < N; ++n) cur[p * N + n] = a * prev[p * N + n] + x[p] * b[n];
                }
                for (int64_t r = t1 - 1; r >= t0; --r) {
                    const double* Scur = St + (r - t0) * PN;
                    const double* Sprev = r == t0 ? ck + j * PN : St + (r - 1 - t0) * PN;
                    const double a = exp(logA[r * H + h]);
                    const double* x = X + (r * H + h) * P;
                    const double* b = B + (r * G + g) * N;
                    const double* c = C + (r * G + g) * N;
                    const double* dy = dY + (r * H + h) * P;
                    double* dx = dX + (r * H + h) * P;
                    double* db = dB + (r * G + g) * N;
                    double* dc = dC + (r * G + g) * N;
                    double da = 0.0;
                    for (int64_t p = 0; p < P; ++p) {
                        double acc = 0.0;
                        for (int64_t n = 0; n < N; ++n) {
                            double* gpn = Gm + p * N + n;
                            *gpn += dy[p] * c[n];
                            dc[n] += Scur[p * N + n] * dy[p];
                            acc += *gpn * b[n];
                            db[n] += *gpn * x[p];
                            da += *gpn * Sprev[p * N + n];
                            *gpn *= a;
                        }
                        dx[p] = acc;
                    }
                    dlogA[r * H + h] = a * da;
                }
            }
            if (dinit) memcpy(dinit + (s * H + h) * PN, Gm, (size_t)PN * sizeof(double));
        }
        free(ck);
        free(St);
        free(Gm);
    }
    return failed ? -2 : 0;
}
