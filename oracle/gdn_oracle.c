/*
 * gdn_oracle.c -- plain, slow, fp64 CPU oracle for one Gated DeltaNet layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source
 * with the HIP path and nothing in the product path may call it.
 *
 * What it computes, token by token and in double precision, for every
 * sequence of a packed batch and every value head:
 *
 *   1. causal depthwise conv1d over the concatenated q|k|v channels, taps
 *      w[c][0..K-1] with w[c][K-1] on the current token, history before the
 *      sequence start taken from the carried conv state (zeros if none),
 *      followed by SiLU(x) = x / (1 + e^-x);
 *   2. per-head L2 normalisation of q and k over the key dimension,
 *      q^ = s * q~ / sqrt(|q~|^2 + eps1), k^ = k~ / sqrt(|k~|^2 + eps1);
 *   3. gates g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b);
 *   4. the gated delta rule (Yang, Kautz, Hatamizadeh, "Gated Delta
 *      Networks: Improving Mamba2 with Delta Rule", ICLR 2025, the gated
 *      delta rule recurrence):
 *          S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *          o_t = S_t q_t,           S in R^{dv x dk};
 *   5. the output gate y = w (.) o / sqrt(mean(o^2) + eps2) (.) SiLU(z).
 *
 * The layer is the recurrent block of the hybrid Qwen3.x models that the
 * engines on the pages serve (llmxabe README, "Status" and the model section:
 * three of every four layers are Gated DeltaNet with a fixed-size state per
 * sequence; skindeep.ai "Our own inference runtime", "What it is": 36 of 48
 * layers are gated delta net).  The pages give no formula; the recurrence is
 * the published one above, written out as a plain matrix product here.
 *
 * Storage conventions (shared with the C ABI only as a documented layout,
 * not as code):
 *   q, k   [T][Hk][dk]     v, z [T][Hv][dv]     a, b [T][Hv]
 *   conv_w [Cc][K], channel c: q channels (head-major), then k, then v,
 *          Cc = 2*Hk*dk + Hv*dv
 *   state  [N][Hv][dk][dv] holding S^T, i.e. state[n][h][i][j] = S[j][i]
 *   conv state [N][K-1][Cc], oldest tap first
 *   value head h reads key head h / (Hv/Hk) (contiguous groups).
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int Hk, Hv, dk, dv, K;
    double scale, eps_l2, eps_rms;
} oracle_dims;

/* ---- scalar pieces ----------------------------------------------------- */

double oracle_silu(double x) { return x / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + e^x), written in the overflow-free form
 * max(x,0) + log1p(e^-|x|). */
double oracle_softplus(double x) {
    double m = x > 0.0 ? x : 0.0;
    return m + log1p(exp(-fabs(x)));
}

double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b). */
void oracle_gates(double a, double b, double A_log, double dt_bias,
                  double* g, double* beta) {
    *g = -exp(A_log) * oracle_softplus(a + dt_bias);
    *beta = oracle_sigmoid(b);
}

/* y = s * x / sqrt(sum(x^2) + eps) over n entries. */
void oracle_l2norm(int n, const double* x, double eps, double s, double* y) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[i] * x[i];
    double r = s / sqrt(ss + eps);
    for (int i = 0; i < n; ++i) y[i] = x[i] * r;
}

/* y = w (.) o / sqrt(mean(o^2) + eps) (.) SiLU(z) over n entries. */
void oracle_rmsnorm_gate(int n, const double* o, const double* z,
                         const double* w, double eps, double* y) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += o[i] * o[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (int i = 0; i < n; ++i) y[i] = w[i] * o[i] * r * oracle_silu(z[i]);
}

/* One step of the gated delta rule on S [dv][dk] (row-major, S[j][i]).
 *   S <- exp(g) * S * (I - beta k k^T) + beta v k^T ;  o = S q.
 * S (I - beta k k^T) = S - beta (S k) k^T is the matrix product expanded
 * by distributivity; nothing is reordered across tokens. */
void oracle_delta_step(int dk, int dv, double* S, const double* q,
                       const double* k, const double* v, double g,
                       double beta, double* o) {
    double eg = exp(g);
    for (int j = 0; j < dv; ++j) {
        double* row = S + (size_t)j * dk;
        double sk = 0.0;                      /* (S k)_j */
        for (int i = 0; i < dk; ++i) sk += row[i] * k[i];
        for (int i = 0; i < dk; ++i)
            row[i] = eg * (row[i] - beta * sk * k[i]) + beta * v[j] * k[i];
    }
    for (int j = 0; j < dv; ++j) {
        const double* row = S + (size_t)j * dk;
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += row[i] * q[i];
        o[j] = acc;
    }
}

/* The bare recurrence over T tokens for one head, on already-normalised
 * inputs: q, k [T][dk], v [T][dv], g, beta [T]; S [dv][dk] in/out;
 * o [T][dv]. */
void oracle_delta_rule(int T, int dk, int dv, const double* q,
                       const double* k, const double* v, const double* g,
                       const double* beta, double* S, double* o) {
    for (int t = 0; t < T; ++t)
        oracle_delta_step(dk, dv, S, q + (size_t)t * dk, k + (size_t)t * dk,
                          v + (size_t)t * dv, g[t], beta[t],
                          o + (size_t)t * dv);
}

/* ---- the whole layer ---------------------------------------------------- */

typedef struct {
    const oracle_dims* d;
    int N;
    const int64_t* cu;
    const double *q, *k, *v, *z, *a, *b;
    const double *conv_w, *A_log, *dt_bias, *norm_w;
    const double *state_in, *conv_in;
    double *out, *core_out, *state_out, *conv_out;
    int ntasks;
    int next;                 /* next task, under lock */
    pthread_mutex_t lock;
} job_t;

/* raw input of channel c at absolute token position pos of sequence n whose
 * first token is `start`; positions before the start read the conv state. */
static double raw_channel(const job_t* J, int n, int64_t start, int64_t pos,
                          int c) {
    const oracle_dims* d = J->d;
    int Cc = 2 * d->Hk * d->dk + d->Hv * d->dv;
    if (pos < start) {
        int64_t r = (d->K - 1) + (pos - start);          /* 0 = oldest tap */
        if (r < 0 || !J->conv_in) return 0.0;
        return J->conv_in[((size_t)n * (d->K - 1) + (size_t)r) * Cc + c];
    }
    int qk = d->Hk * d->dk;
    if (c < qk) return J->q[(size_t)pos * qk + c];
    if (c < 2 * qk) return J->k[(size_t)pos * qk + (c - qk)];
    return J->v[(size_t)pos * d->Hv * d->dv + (c - 2 * qk)];
}

/* conv1d + SiLU of channel c at token pos. */
static double conv_silu(const job_t* J, int n, int64_t start, int64_t pos,
                        int c) {
    int K = J->d->K;
    double acc = 0.0;
    for (int j = 0; j < K; ++j)
        acc += J->conv_w[(size_t)c * K + j] *
               raw_channel(J, n, start, pos - (K - 1) + j, c);
    return oracle_silu(acc);
}

static void run_task(job_t* J, int task) {
    const oracle_dims* d = J->d;
    int n = task / d->Hv, h = task % d->Hv;
    int G = d->Hv / d->Hk, hk = h / G;
    int dk = d->dk, dv = d->dv;
    int qk = d->Hk * dk;
    int Cc = 2 * qk + d->Hv * dv;
    int64_t start = J->cu[n], end = J->cu[n + 1];

    double* S = (double*)calloc((size_t)dv * dk, sizeof(double));
    double* xq = (double*)malloc(sizeof(double) * dk);
    double* xk = (double*)malloc(sizeof(double) * dk);
    double* qh = (double*)malloc(sizeof(double) * dk);
    double* kh = (double*)malloc(sizeof(double) * dk);
    double* vh = (double*)malloc(sizeof(double) * dv);
    double* o = (double*)malloc(sizeof(double) * dv);
    double* y = (double*)malloc(sizeof(double) * dv);

    size_t sbase = ((size_t)n * d->Hv + h) * dk * dv;
    if (J->state_in)
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(size_t)j * dk + i] = J->state_in[sbase + (size_t)i * dv + j];

    for (int64_t t = start; t < end; ++t) {
        for (int i = 0; i < dk; ++i) {
            xq[i] = conv_silu(J, n, start, t, hk * dk + i);
            xk[i] = conv_silu(J, n, start, t, qk + hk * dk + i);
        }
        for (int j = 0; j < dv; ++j)
            vh[j] = conv_silu(J, n, start, t, 2 * qk + h * dv + j);
        oracle_l2norm(dk, xq, d->eps_l2, d->scale, qh);
        oracle_l2norm(dk, xk, d->eps_l2, 1.0, kh);
        double g, beta;
        oracle_gates(J->a[(size_t)t * d->Hv + h], J->b[(size_t)t * d->Hv + h],
                     J->A_log[h], J->dt_bias[h], &g, &beta);
        oracle_delta_step(dk, dv, S, qh, kh, vh, g, beta, o);
        size_t obase = ((size_t)t * d->Hv + h) * dv;
        if (J->core_out) memcpy(J->core_out + obase, o, sizeof(double) * dv);
        if (J->out) {
            oracle_rmsnorm_gate(dv, o, J->z + obase, J->norm_w, d->eps_rms, y);
            memcpy(J->out + obase, y, sizeof(double) * dv);
        }
    }

    if (J->state_out)
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                J->state_out[sbase + (size_t)i * dv + j] = S[(size_t)j * dk + i];

    /* new conv state: the last K-1 raw rows of (old state ++ inputs), for
     * this value head's v channels and, once per key head, its q/k ones. */
    if (J->conv_out) {
        for (int r = 0; r < d->K - 1; ++r) {
            int64_t pos = end - (d->K - 1) + r;
            double* dst = J->conv_out + ((size_t)n * (d->K - 1) + r) * Cc;
            for (int j = 0; j < dv; ++j) {
                int c = 2 * qk + h * dv + j;
                dst[c] = raw_channel(J, n, start, pos, c);
            }
            if (h % G == 0)
                for (int i = 0; i < dk; ++i) {
                    int cq = hk * dk + i, ck = qk + hk * dk + i;
                    dst[cq] = raw_channel(J, n, start, pos, cq);
                    dst[ck] = raw_channel(J, n, start, pos, ck);
                }
        }
    }
    free(S); free(xq); free(xk); free(qh); free(kh); free(vh); free(o); free(y);
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int t = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (t >= J->ntasks) break;
        run_task(J, t);
    }
    return NULL;
}

/* Whole layer over N packed sequences; cu [N+1] token offsets.  Any of out,
 * core_out, state_out, conv_out may be NULL (not produced); state_in and
 * conv_in may be NULL (zeros).  Returns 0, or -1 on bad dimensions. */
int oracle_gdn_forward(const oracle_dims* d, int N, const int64_t* cu,
                       const double* q, const double* k, const double* v,
                       const double* z, const double* a, const double* b,
                       const double* conv_w, const double* A_log,
                       const double* dt_bias, const double* norm_w,
                       const double* state_in, const double* conv_in,
                       double* out, double* core_out, double* state_out,
                       double* conv_out, int nthreads) {
    if (!d || d->Hk <= 0 || d->Hv <= 0 || d->Hv % d->Hk || d->dk <= 0 ||
        d->dv <= 0 || d->K <= 0 || N < 0)
        return -1;
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n]) return -1;
    job_t J;
    memset(&J, 0, sizeof J);
    J.d = d; J.N = N; J.cu = cu;
    J.q = q; J.k = k; J.v = v; J.z = z; J.a = a; J.b = b;
    J.conv_w = conv_w; J.A_log = A_log; J.dt_bias = dt_bias; J.norm_w = norm_w;
    J.state_in = state_in; J.conv_in = conv_in;
    J.out = out; J.core_out = core_out; J.state_out = state_out;
    J.conv_out = conv_out;
    J.ntasks = N * d->Hv;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads <= 1) {
        worker(&J);
    } else {
        pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
        for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
        for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&J.lock);
    return 0;
}
