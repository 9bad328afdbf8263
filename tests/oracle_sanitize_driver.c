// Driver that runs the fp64 oracle's whole-layer forward under the host
// sanitizers (tests/test_oracle_sanitizers.py builds it with gcc): every
// buffer is a heap block of exactly the size the interface documents, so an
// access past an end is reported; the shapes cover ragged batches with empty
// and one-token sequences, dk != dv, three value heads per key head, a batch
// of empty sequences, N = 0, NULL states and one to eight threads.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
typedef struct { int Hk, Hv, dk, dv, K; double scale, eps_l2, eps_rms; } oracle_dims;
int oracle_gdn_forward(const oracle_dims* d, int N, const int64_t* cu, const double* q, const double* k,
                       const double* v, const double* z, const double* a, const double* b,
                       const double* conv_w, const double* A_log, const double* dt_bias,
                       const double* norm_w, const double* state_in, const double* conv_in, double* out,
                       double* core_out, double* state_out, double* conv_out, int nthreads);
static double* rnd(size_t n, unsigned* s) {
    double* p = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) { *s = *s * 1664525u + 1013904223u; p[i] = ((*s >> 8) & 0xFFFF) / 32768.0 - 1.0; }
    return p;
}
static int run(int Hk, int Hv, int dk, int dv, const int* lens, int N, int with_states, int nthreads) {
    oracle_dims d = {Hk, Hv, dk, dv, 4, 0.177, 1e-6, 1e-6};
    int64_t* cu = malloc((N + 1) * sizeof(int64_t));
    cu[0] = 0;
    for (int n = 0; n < N; ++n) cu[n + 1] = cu[n] + lens[n];
    const int64_t T = cu[N];
    const int Cc = 2 * Hk * dk + Hv * dv;
    unsigned s = 7u + N;
    double *q = rnd(T * Hk * dk, &s), *k = rnd(T * Hk * dk, &s), *v = rnd(T * Hv * dv, &s), *z = rnd(T * Hv * dv, &s);
    double *a = rnd(T * Hv, &s), *b = rnd(T * Hv, &s), *cw = rnd((size_t)Cc * 4, &s);
    double *Al = rnd(Hv, &s), *dtb = rnd(Hv, &s), *nw = rnd(dv, &s);
    double* si = with_states ? rnd((size_t)N * Hv * dk * dv, &s) : NULL;
    double* ci = with_states ? rnd((size_t)N * 3 * Cc, &s) : NULL;
    double *out = malloc((T * Hv * dv + 1) * sizeof(double)), *core = malloc((T * Hv * dv + 1) * sizeof(double));
    double *so = malloc(((size_t)N * Hv * dk * dv + 1) * sizeof(double)), *co = malloc(((size_t)N * 3 * Cc + 1) * sizeof(double));
    const int rc = oracle_gdn_forward(&d, N, cu, q, k, v, z, a, b, cw, Al, dtb, nw, si, ci, out, core, so, co, nthreads);
    printf("Hk %d Hv %d dk %d dv %d N %d T %ld states %d threads %d: rc %d\n", Hk, Hv, dk, dv, N, (long)T, with_states, nthreads, rc);
    free(cu); free(q); free(k); free(v); free(z); free(a); free(b); free(cw); free(Al); free(dtb); free(nw);
    free(si); free(ci); free(out); free(core); free(so); free(co);
    return rc;
}
int main(void) {
    const int l1[] = {37, 0, 27, 1, 16, 3, 2};
    const int l2[] = {0, 0, 0};
    const int l3[] = {130, 5};
    int bad = 0;
    bad |= run(2, 4, 32, 32, l1, 7, 1, 1);
    bad |= run(2, 4, 32, 32, l1, 7, 1, 4);
    bad |= run(2, 4, 32, 64, l1, 7, 0, 3);
    bad |= run(1, 3, 16, 8, l3, 2, 1, 2);
    bad |= run(2, 4, 32, 32, l2, 3, 1, 2);
    bad |= run(2, 4, 32, 32, l1, 0, 0, 1);
    bad |= run(16, 32, 128, 128, l3, 2, 1, 8);
    return bad ? 1 : 0;
}
