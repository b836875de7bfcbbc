/* sanitize_check.c -- runs the float64 oracle (ssd_oracle.c) on small seeded problems,
 * built with AddressSanitizer and UndefinedBehaviorSanitizer: plain and packed batches
 * (empty and length-1 sequences among them), with and without an initial state, one and
 * several groups, the backward pass with and without its optional gradients, and
 * malformed arguments.  Test infrastructure, like the oracle itself.
 *
 * Besides memory safety it checks two facts that hold for any input:
 *   - with every decay a_t = 0 (logA = -inf) the state forgets everything before t, so
 *     y_t[p] = x_t[p] (B_t . C_t) exactly as the recurrence S_t = a_t S_{t-1} + x_t B_t^T,
 *     y_t = S_t C_t defines it ("Transformers are SSMs" paper summary page, section 2.4);
 *   - splitting a batch of one sequence into two packed sequences at a token restarts the
 *     state there: the second part's outputs equal those of that part walked alone.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ssd_oracle_recurrence(int64_t batch, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G,
                          const double* X, const double* logA, const double* B, const double* C,
                          const double* init, const int64_t* seq_offsets, int64_t nseq,
                          double* Y, double* final_state, int nthreads);
int ssd_oracle_backward(int64_t batch, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G,
                        const double* X, const double* logA, const double* B, const double* C,
                        const double* init, const int64_t* seq_offsets, int64_t nseq,
                        const double* dY, const double* dfinal,
                        double* dX, double* dlogA, double* dB, double* dC, double* dinit,
                        int nthreads);

static int failures = 0;
#define EXPECT(c, what)                                                        \
    do {                                                                       \
        if (!(c)) {                                                            \
            ++failures;                                                        \
            fprintf(stderr, "FAIL %s (line %d)\n", what, __LINE__);            \
        }                                                                      \
    } while (0)

/* splitmix64 */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) / 9007199254740992.0;
}
static double* filled(size_t n, double lo, double hi) {
    double* a = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * urand();
    return a;
}

static void run_case(int64_t b, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G, const int64_t* off,
                     int64_t nseq, int with_init, int with_dfinal) {
    const int64_t rows = b * T, ns = off ? nseq : b;
    double* X = filled((size_t)(rows * H * P), -1, 1);
    double* la = filled((size_t)(rows * H), -0.5, 0);
    double* B = filled((size_t)(rows * G * N), -1, 1);
    double* C = filled((size_t)(rows * G * N), -1, 1);
    double* init = with_init ? filled((size_t)(ns * H * P * N), -1, 1) : NULL;
    double* Y = filled((size_t)(rows * H * P), 0, 0);
    double* F = filled((size_t)(ns * H * P * N), 0, 0);
    EXPECT(ssd_oracle_recurrence(b, T, H, P, N, G, X, la, B, C, init, off, nseq, Y, F, 2) == 0, "recurrence");
    double* dY = filled((size_t)(rows * H * P), -1, 1);
    double* dF = with_dfinal ? filled((size_t)(ns * H * P * N), -1, 1) : NULL;
    double* dX = filled((size_t)(rows * H * P), 0, 0);
    double* dla = filled((size_t)(rows * H), 0, 0);
    double* dB = filled((size_t)(rows * G * N), 0, 0);
    double* dC = filled((size_t)(rows * G * N), 0, 0);
    double* di = with_init ? filled((size_t)(ns * H * P * N), 0, 0) : NULL;
    EXPECT(ssd_oracle_backward(b, T, H, P, N, G, X, la, B, C, init, off, nseq, dY, dF, dX, dla, dB, dC, di, 2) == 0,
           "backward");
    for (int64_t i = 0; i < rows * H * P; ++i) EXPECT(isfinite(Y[i]) && isfinite(dX[i]), "finite outputs");
    free(X), free(la), free(B), free(C), free(init), free(Y), free(F);
    free(dY), free(dF), free(dX), free(dla), free(dB), free(dC), free(di);
}

/* every decay zero: y_t[p] = x_t[p] (B_t . C_t) */
static void zero_decay_case(void) {
    const int64_t T = 37, H = 4, P = 5, N = 6, G = 2;
    double* X = filled((size_t)(T * H * P), -1, 1);
    double* la = filled((size_t)(T * H), 0, 0);
    for (int64_t i = 0; i < T * H; ++i) la[i] = -INFINITY;
    double* B = filled((size_t)(T * G * N), -1, 1);
    double* C = filled((size_t)(T * G * N), -1, 1);
    double* init = filled((size_t)(H * P * N), -1, 1);
    double* Y = filled((size_t)(T * H * P), 0, 0);
    double* F = filled((size_t)(H * P * N), 0, 0);
    EXPECT(ssd_oracle_recurrence(1, T, H, P, N, G, X, la, B, C, init, NULL, 0, Y, F, 1) == 0, "zero-decay run");
    double worst = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            const int64_t g = h / (H / G);
            double bc = 0;
            for (int64_t n = 0; n < N; ++n) bc += B[(t * G + g) * N + n] * C[(t * G + g) * N + n];
            for (int64_t p = 0; p < P; ++p) {
                const double d = fabs(Y[(t * H + h) * P + p] - X[(t * H + h) * P + p] * bc);
                if (d > worst) worst = d;
            }
        }
    EXPECT(worst < 1e-12, "zero decay: y_t = x_t (B_t . C_t)");
    free(X), free(la), free(B), free(C), free(init), free(Y), free(F);
}

/* a packed split restarts the state: the second part matches that part alone */
static void split_case(void) {
    const int64_t T = 50, cut = 19, H = 2, P = 3, N = 4, G = 1;
    double* X = filled((size_t)(T * H * P), -1, 1);
    double* la = filled((size_t)(T * H), -0.3, 0);
    double* B = filled((size_t)(T * G * N), -1, 1);
    double* C = filled((size_t)(T * G * N), -1, 1);
    double* Y = filled((size_t)(T * H * P), 0, 0);
    double* F = filled((size_t)(2 * H * P * N), 0, 0);
    const int64_t off[3] = {0, cut, T};
    EXPECT(ssd_oracle_recurrence(1, T, H, P, N, G, X, la, B, C, NULL, off, 2, Y, F, 1) == 0, "split run");
    double* Y2 = filled((size_t)((T - cut) * H * P), 0, 0);
    double* F2 = filled((size_t)(H * P * N), 0, 0);
    EXPECT(ssd_oracle_recurrence(1, T - cut, H, P, N, G, X + cut * H * P, la + cut * H, B + cut * G * N,
                                 C + cut * G * N, NULL, NULL, 0, Y2, F2, 1) == 0,
           "second part alone");
    int same = memcmp(Y + cut * H * P, Y2, (size_t)((T - cut) * H * P) * sizeof(double)) == 0 &&
               memcmp(F + H * P * N, F2, (size_t)(H * P * N) * sizeof(double)) == 0;
    EXPECT(same, "packed split restarts the state");
    free(X), free(la), free(B), free(C), free(Y), free(F), free(Y2), free(F2);
}

int main(void) {
    run_case(2, 70, 4, 8, 16, 2, NULL, 0, 1, 1);
    run_case(1, 1, 1, 1, 1, 1, NULL, 0, 0, 0);
    run_case(3, 5, 6, 3, 7, 3, NULL, 0, 0, 1);
    {
        const int64_t off[7] = {0, 0, 1, 66, 66, 67, 130};   /* empty and length-1 sequences */
        run_case(1, 130, 4, 8, 16, 2, off, 6, 1, 1);
        run_case(1, 130, 4, 8, 16, 4, off, 6, 0, 0);
    }
    {
        const int64_t off[3] = {0, 0, 0};   /* no tokens at all: two empty sequences */
        run_case(1, 0, 2, 4, 4, 1, off, 2, 1, 1);
    }
    zero_decay_case();
    split_case();
    /* malformed arguments: rejected before any memory is touched */
    double one = 0;
    const int64_t bad_off[3] = {0, 5, 3};
    EXPECT(ssd_oracle_recurrence(0, 4, 1, 1, 1, 1, &one, &one, &one, &one, NULL, NULL, 0, &one, &one, 1) == -1,
           "batch 0");
    EXPECT(ssd_oracle_recurrence(1, 4, 3, 1, 1, 2, &one, &one, &one, &one, NULL, NULL, 0, &one, &one, 1) == -1,
           "H % G != 0");
    EXPECT(ssd_oracle_recurrence(1, 3, 1, 1, 1, 1, &one, &one, &one, &one, NULL, bad_off, 2, &one, &one, 1) == -1,
           "decreasing offsets");
    EXPECT(ssd_oracle_backward(2, 4, 1, 1, 1, 1, &one, &one, &one, &one, NULL, bad_off, 2, &one, NULL, &one, &one,
                               &one, &one, NULL, 1) == -1,
           "offsets with batch 2");
    printf("oracle sanitize check: %d failures\n", failures);
    return failures ? 1 : 0;
}
