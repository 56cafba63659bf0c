/*
 * KDA forward oracle: token-by-token fp64 recurrence on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP
 * path.
 *
 * What it computes (Kimi Delta Attention, the gated delta rule with
 * per-channel decay).  "Autoresearch on Kimi Delta Attention", section
 * "KDA in one minute", describes the operator in words: a fixed-size matrix
 * memory per head; each token reads what the memory predicts for its key and
 * writes only the correction; a learned gate lets each memory channel forget
 * at its own rate; the state does not grow with the sequence.  Written as a
 * formula, per head and per sequence, with S a dk x dv matrix:
 *
 *     S_t = (I - beta_t khat_t khat_t^T) Diag(alpha_t) S_{t-1} + beta_t khat_t v_t^T
 *     o_t = scale * S_t^T qhat_t
 *
 * with alpha_t = exp(g_t) (g is a natural-log gate, one value per key channel,
 * so the gate scales the ROWS of S), qhat = q/||q||_2 and khat = k/||k||_2
 * (the L2 normalisation of Q and K that "Kernel Design Agents (KDA) optimize
 * Kimi Delta Attention (KDA)", section "03 - Reward hacking", says the kernel
 * must compute for real), and a zero vector normalised to zero.  The output
 * of token t is read after token t's own update.
 *
 * The same page, section "01 - Results", names a token-by-token fp64
 * recurrence as the accuracy reference; this is that reference.  Each
 * (sequence, head) chain is independent; sequences come from token offsets
 * cu[0..N] (fixed-length batches are offsets 0, T, 2T, ...).  A NULL h0 means
 * a zero initial state; an empty sequence returns ht = h0.
 *
 * Expanding the formula, one token is: decay the rows of S, predict
 * u = S^T khat, write S += beta * khat (v - u)^T, read o = scale * S^T qhat.
 * That expansion is exact algebra of the formula above (no reordering of the
 * recurrence), done here in fp64 with the straightforward loops.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* L2-normalise x (length d) into out; zero vector -> zero. */
static void l2_normalise(const double* x, int64_t d, double* out) {
    double ss = 0.0;
    for (int64_t c = 0; c < d; ++c) ss += x[c] * x[c];
    double n = sqrt(ss);
    for (int64_t c = 0; c < d; ++c) out[c] = (n > 0.0) ? x[c] / n : 0.0;
}

/*
 * Layouts (row-major, contiguous):
 *   q, k, g  [T_total, H, dk]      v, out  [T_total, H, dv]
 *   beta     [T_total, H]          h0, ht  [N, H, dk, dv]
 *   cu       [N + 1] token offsets, cu[0] = 0, non-decreasing, cu[N] = T_total
 * h0 and ht may be NULL.  Returns 0, or -1 on a bad argument.
 */
int kda_oracle_fwd(int64_t num_seqs, const int64_t* cu, int64_t H, int64_t dk, int64_t dv,
                   const double* q, const double* k, const double* v, const double* g,
                   const double* beta, const double* h0, double scale, double* out, double* ht,
                   int nthreads) {
    if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu) return -1;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (cu[n + 1] < cu[n]) return -1;
    int64_t chains = num_seqs * H;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)(dk * dv));
        double* qh = (double*)malloc(sizeof(double) * (size_t)dk);
        double* kh = (double*)malloc(sizeof(double) * (size_t)dk);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!S || !qh || !kh || !u) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t ch = 0; ch < chains; ++ch) {
                int64_t n = ch / H, h = ch % H;
                if (h0)
                    memcpy(S, h0 + ch * dk * dv, sizeof(double) * (size_t)(dk * dv));
                else
                    memset(S, 0, sizeof(double) * (size_t)(dk * dv));
                for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
                    const double* qt = q + (t * H + h) * dk;
                    const double* kt = k + (t * H + h) * dk;
                    const double* gt = g + (t * H + h) * dk;
                    const double* vt = v + (t * H + h) * dv;
                    double bt = beta[t * H + h];
                    l2_normalise(qt, dk, qh);
                    l2_normalise(kt, dk, kh);
                    /* Diag(alpha_t) S: each key channel (row) forgets at its own rate */
                    for (int64_t c = 0; c < dk; ++c) {
                        double a = exp(gt[c]);
                        for (int64_t j = 0; j < dv; ++j) S[c * dv + j] *= a;
                    }
                    /* prediction u = S^T khat (what the memory currently returns for k) */
                    for (int64_t j = 0; j < dv; ++j) u[j] = 0.0;
                    for (int64_t c = 0; c < dk; ++c)
                        for (int64_t j = 0; j < dv; ++j) u[j] += S[c * dv + j] * kh[c];
                    /* write only the correction: S += beta khat (v - u)^T */
                    for (int64_t c = 0; c < dk; ++c) {
                        double w = bt * kh[c];
                        for (int64_t j = 0; j < dv; ++j) S[c * dv + j] += w * (vt[j] - u[j]);
                    }
                    /* read after the update: o_t = scale S^T qhat */
                    double* ot = out + (t * H + h) * dv;
                    for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
                    for (int64_t c = 0; c < dk; ++c)
                        for (int64_t j = 0; j < dv; ++j) ot[j] += S[c * dv + j] * qh[c];
                    for (int64_t j = 0; j < dv; ++j) ot[j] *= scale;
                }
                if (ht) memcpy(ht + ch * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
            }
        }
        free(S);
        free(qh);
        free(kh);
        free(u);
    }
    return err ? -1 : 0;
}

/* Threads an OpenMP region would use (reported next to the CPU baseline). */
int kda_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
