/*
 * kda_oracle.c -- fp64 CPU oracle for the forward pass of gated delta-rule
 * linear attention (KDA with per-channel decay, GDN with one scalar decay per
 * head).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; it exists so that tests, the smoke check and the benchmark's
 * CPU baseline can check the GPU library against an obviously correct,
 * slow, token-by-token recurrence.  It shares no code with the HIP library.
 *
 * What it computes (one (sequence, head) at a time, tokens in order):
 *
 *   q^_t = q_t / sqrt(sum_c q_tc^2 + eps),  k^_t likewise          (eps = 1e-6)
 *   KDA:  log a_tc = max(lb, -exp(A_log[h]) * softplus(g_tc + dt_bias[h,c]))
 *         beta_t   = sigmoid(beta_logit_t)
 *   GDN:  log a_tc = g_t[h]  (the same for every channel c),  beta_t as given
 *   S_t  = (I - beta_t k^_t k^_t^T) Diag(a_t) S_{t-1} + beta_t k^_t v_t^T
 *   o_t  = scale * S_t^T q^_t        (S in [K,V] layout; token t sees itself)
 *
 * Sources on the pages:
 *  - "FlashKDA: MoonshotAI ... Kimi Delta Attention ..." (discuss.pytorch.kr),
 *    section "FlashKDA의 KDA 연산 구조" (the flash_kda.fwd parameter table):
 *    q,k [B,T,H,K], v [B,T,H,V], g = pre-activation gate [B,T,H,K], beta =
 *    logits with the sigmoid taken inside, A_log [H] log-gate parameter,
 *    dt_bias [H,K] gate bias, lower_bound in [-5, 0], optional initial and
 *    final recurrent state; L2 normalisation of q and k and the gate
 *    activation are fused into the kernel.
 *  - Same page, section "커널 퓨전(Kernel Fusion) 전략의 분리": the operations are
 *    gate activation, L2 norm, decay, matrix inverse, chunked delta-rule
 *    recurrence and output projection.
 *  - "cuLA -- CUDA Linear Attention" (README mirror), section "KDA (Kimi Delta
 *    Attention) -- Blackwell (SM10X)" and its Notes: the state is fp32
 *    [B,H,K,V]; cu_seqlens is int32.
 * The pages print no equation.  The formulas above are the plain reading of
 * those parameter roles (gate = -exp(A_log) * softplus(g + dt_bias) floored at
 * lower_bound; delta rule with decay applied before the rank-one correction;
 * output read from the updated state); every such reading is listed with the
 * design notes.  The chunked form used on the GPU is algebraically identical
 * to this recurrence, so the oracle is the recurrence itself.
 *
 * Inputs are fp64 (the caller up-casts bf16/fp32 bytes exactly).  Layouts are
 * contiguous row-major: q,k,(KDA g) [B,T,H,K]; v,o [B,T,H,V]; beta [B,T,H];
 * GDN g [B,T,H]; A_log [H]; dt_bias [H,K]; states [N,H,K,V] where N = B, or
 * N = n_seqs when cu (int64 offsets, B must be 1) is given.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_NORM_EPS 1e-6

static double softplus(double x) {
    /* log(1 + e^x), evaluated without overflow. */
    return fmax(x, 0.0) + log1p(exp(-fabs(x)));
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static void l2_normalise(const double* x, double* out, int64_t n) {
    double ss = 0.0;
    for (int64_t c = 0; c < n; ++c) ss += x[c] * x[c];
    double inv = 1.0 / sqrt(ss + ORACLE_NORM_EPS);
    for (int64_t c = 0; c < n; ++c) out[c] = x[c] * inv;
}

/* Runs tokens [t0, t1) of one (batch row, head).  Row pointers are already
 * offset to the batch row.  S (K*V) holds the incoming state and receives the
 * outgoing one.  work holds 3*K + V doubles. */
static void run_sequence(int gdn, const double* q, const double* k, const double* v,
                         const double* g, const double* beta, double decay_rate,
                         const double* dt_bias_h, double lower_bound, double scale,
                         int64_t t0, int64_t t1, int64_t H, int64_t h, int64_t K, int64_t V,
                         double* S, double* o, double* work) {
    double* qn = work;
    double* kn = work + K;
    double* log_a = work + 2 * K;
    double* r = work + 3 * K;
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t row = t * H + h;
        l2_normalise(q + row * K, qn, K);
        l2_normalise(k + row * K, kn, K);
        double b;
        if (gdn) {
            for (int64_t c = 0; c < K; ++c) log_a[c] = g[row];
            b = beta[row];
        } else {
            for (int64_t c = 0; c < K; ++c) {
                double a = -decay_rate * softplus(g[row * K + c] + dt_bias_h[c]);
                log_a[c] = fmax(lower_bound, a);
            }
            b = sigmoid(beta[row]);
        }
        /* S <- Diag(a_t) S */
        for (int64_t c = 0; c < K; ++c) {
            double a = exp(log_a[c]);
            for (int64_t j = 0; j < V; ++j) S[c * V + j] *= a;
        }
        /* r = S^T k^_t (what the decayed state predicts for this key) */
        for (int64_t j = 0; j < V; ++j) r[j] = 0.0;
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j) r[j] += S[c * V + j] * kn[c];
        /* S <- S + beta_t k^_t (v_t - r)^T */
        const double* vt = v + row * V;
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j) S[c * V + j] += b * kn[c] * (vt[j] - r[j]);
        /* o_t = scale * S^T q^_t */
        double* ot = o + row * V;
        for (int64_t j = 0; j < V; ++j) ot[j] = 0.0;
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j) ot[j] += S[c * V + j] * qn[c];
        for (int64_t j = 0; j < V; ++j) ot[j] *= scale;
    }
}

/*
 * gdn: 0 = KDA (g pre-activation [B,T,H,K], beta logits, A_log, dt_bias used),
 *      1 = GDN (g log-decay [B,T,H], beta probabilities, A_log/dt_bias unused).
 * h0 may be NULL (zero state); hT may be NULL (not written).
 * cu may be NULL (fixed length, N = B); else cu[0..n_seqs] with B == 1.
 * threads <= 0 uses the OpenMP default.
 * Returns 0 on success, -1 on a bad argument.
 */
int kda_oracle_forward(int gdn, const double* q, const double* k, const double* v,
                       const double* g, const double* beta, const double* A_log,
                       const double* dt_bias, double lower_bound, double scale,
                       const double* h0, double* hT, const int64_t* cu, int64_t n_seqs,
                       int64_t B, int64_t T, int64_t H, int64_t K, int64_t V, double* o,
                       int threads) {
    if (!q || !k || !v || !g || !beta || !o || B < 1 || T < 0 || H < 1 || K < 1 || V < 1)
        return -1;
    if (!gdn && (!A_log || !dt_bias)) return -1;
    if (cu && B != 1) return -1;
    const int64_t N = cu ? n_seqs : B;
    if (N < 1) return -1;
    const int64_t units = N * H;
    int failed = 0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int64_t n = u / H, h = u % H;
        const int64_t b = cu ? 0 : n;
        const int64_t t0 = cu ? cu[n] : 0;
        const int64_t t1 = cu ? cu[n + 1] : T;
        double* S = (double*)malloc(sizeof(double) * (size_t)(K * V));
        double* work = (double*)malloc(sizeof(double) * (size_t)(3 * K + V));
        if (!S || !work) {
            free(S);
            free(work);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
            continue;
        }
        if (h0)
            memcpy(S, h0 + (n * H + h) * K * V, sizeof(double) * (size_t)(K * V));
        else
            memset(S, 0, sizeof(double) * (size_t)(K * V));
        const int64_t off = b * T * H;
        run_sequence(gdn, q + off * K, k + off * K, v + off * V, gdn ? g + off : g + off * K,
                     beta + off, gdn ? 0.0 : exp(A_log[h]), gdn ? NULL : dt_bias + h * K,
                     lower_bound, scale, t0, t1, H, h, K, V, S, o + off * V, work);
        if (hT) memcpy(hT + (n * H + h) * K * V, S, sizeof(double) * (size_t)(K * V));
        free(S);
        free(work);
    }
    return failed ? -1 : 0;
}

int kda_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
