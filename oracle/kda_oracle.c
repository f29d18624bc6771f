/*
 * CPU oracle for the Kimi Delta Attention (KDA) forward pass -- TEST
 * INFRASTRUCTURE ONLY.  Nothing in the product path may link or call it.
 *
 * Plain fp64 sequential recurrence, one (batch, head) chain per OpenMP task.
 * Kimi K3 technical report summary (page "Kimi K3 Technical Report - Open
 * Frontier Intelligence"), "Key claims" and "Method", section 2.1: KDA is a
 * delta-rule attention with a fixed-size per-head state and channel-wise
 * (per key channel) decay.  Per head and token t, with S in R^{dk x dv}:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t                      (scale = 1/sqrt(dk))
 *
 * written here in the exactly equivalent form
 *     S' = Diag(exp(g_t)) S_{t-1}
 *     u  = beta_t (v_t - S'^T k_t)
 *     S_t = S' + k_t u^T .
 *
 * Inputs are the exact values the device receives (fp32 or bf16 upcast to
 * fp32 by the caller); every operation is done in fp64.
 *
 * Layouts (row-major, contiguous):
 *   q, k, g : [B, T, H, dk]     v, o : [B, T, H, dv]     beta : [B, T, H]
 *   h0, ht  : [B, H, dk, dv] (fp64; h0 may be NULL = zero state; ht may be NULL)
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int kda_oracle_version(void) { return 1; }

int kda_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int kda_oracle_seq(const float* q, const float* k, const float* v, const float* g,
                   const float* beta, const double* h0, double scale,
                   long B, long T, long H, long dk, long dv,
                   double* o, double* ht, int nthreads)
{
    if (B <= 0 || H <= 0 || dk <= 0 || dv <= 0 || T < 0) return 1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1) reduction(| : failed)
#endif
    for (long bh = 0; bh < B * H; ++bh) {
        const long b = bh / H, h = bh % H;
        double* S = (double*)malloc(sizeof(double) * dk * dv);
        double* u = (double*)malloc(sizeof(double) * dv);
        double* dec = (double*)malloc(sizeof(double) * dk);
        if (!S || !u || !dec) { failed |= 1; free(S); free(u); free(dec); continue; }

        if (h0) memcpy(S, h0 + bh * dk * dv, sizeof(double) * dk * dv);
        else memset(S, 0, sizeof(double) * dk * dv);

        for (long t = 0; t < T; ++t) {
            const long row = (b * T + t) * H + h;
            const float* qt = q + row * dk;
            const float* kt = k + row * dk;
            const float* gt = g + row * dk;
            const float* vt = v + row * dv;
            const double bt = (double)beta[row];
            double* ot = o + row * dv;

            /* S' = Diag(exp(g_t)) S : decay scales the key rows */
            for (long c = 0; c < dk; ++c) dec[c] = exp((double)gt[c]);
            for (long c = 0; c < dk; ++c)
                for (long j = 0; j < dv; ++j) S[c * dv + j] *= dec[c];

            /* u = beta (v - S'^T k) */
            for (long j = 0; j < dv; ++j) u[j] = 0.0;
            for (long c = 0; c < dk; ++c) {
                const double kc = (double)kt[c];
                for (long j = 0; j < dv; ++j) u[j] += kc * S[c * dv + j];
            }
            for (long j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - u[j]);

            /* S = S' + k u^T */
            for (long c = 0; c < dk; ++c) {
                const double kc = (double)kt[c];
                for (long j = 0; j < dv; ++j) S[c * dv + j] += kc * u[j];
            }

            /* o = scale * S^T q  (reads the state after token t's own write) */
            for (long j = 0; j < dv; ++j) ot[j] = 0.0;
            for (long c = 0; c < dk; ++c) {
                const double qc = (double)qt[c];
                for (long j = 0; j < dv; ++j) ot[j] += qc * S[c * dv + j];
            }
            for (long j = 0; j < dv; ++j) ot[j] *= scale;
        }
        if (ht) memcpy(ht + bh * dk * dv, S, sizeof(double) * dk * dv);
        free(S); free(u); free(dec);
    }
    return failed ? 2 : 0;
}
