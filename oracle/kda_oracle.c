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
 *
 * kda_oracle_seq_bwd is the gradient of that recurrence (reverse-mode chain
 * rule through the four steps above, token by token from the last one):
 * given do = dL/do and dht = dL/dS_T it returns dq, dk, dv, dg, dbeta and
 * dh0 = dL/dS_0.  The states it needs are recomputed forward from states
 * kept every `seg` tokens (the same arithmetic as the forward, repeated).
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

/*
 * Adjoint of one token, with dS = dL/dS_t on entry (the output's own term
 * included by the caller) and dL/dS_{t-1} on exit.  Sp = S' = Diag(e^g) S_{t-1},
 * u and p = S'^T k as in the forward.
 *   S_t = S' + k u^T       : dk += dS u,  du = dS^T k,  dS' = dS
 *   u = beta (v - p)       : dbeta = du . (v - p),  dv = beta du,  dp = -beta du
 *   p = S'^T k             : dk += S' dp,  dS' += k dp^T
 *   S' = Diag(e^g) S_{t-1} : dg_c = sum_j dS'[c,j] S'[c,j],  dS_{t-1} = Diag(e^g) dS'
 */
int kda_oracle_seq_bwd(const float* q, const float* k, const float* v, const float* g,
                       const float* beta, const double* h0, const double* dout, const double* dht,
                       double scale, long B, long T, long H, long dk, long dv, long seg,
                       double* dq, double* dk_, double* dv_, double* dg, double* dbeta, double* dh0,
                       int nthreads)
{
    if (B <= 0 || H <= 0 || dk <= 0 || dv <= 0 || T < 0 || seg <= 0) return 1;
    const long nseg = (T + seg - 1) / seg;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1) reduction(| : failed)
#endif
    for (long bh = 0; bh < B * H; ++bh) {
        const long b = bh / H, h = bh % H;
        const long SZ = dk * dv;
        double* ck = (double*)malloc(sizeof(double) * SZ * (nseg + 1));  /* state entering each segment */
        double* st = (double*)malloc(sizeof(double) * SZ * (seg + 1));   /* states inside one segment */
        double* dS = (double*)malloc(sizeof(double) * SZ);
        double* Sp = (double*)malloc(sizeof(double) * SZ);
        double* u = (double*)malloc(sizeof(double) * dv);
        double* p = (double*)malloc(sizeof(double) * dv);
        double* du = (double*)malloc(sizeof(double) * dv);
        double* dec = (double*)malloc(sizeof(double) * dk);
        if (!ck || !st || !dS || !Sp || !u || !p || !du || !dec) {
            failed |= 1;
            free(ck); free(st); free(dS); free(Sp); free(u); free(p); free(du); free(dec);
            continue;
        }
        /* one forward step from S (SZ values) into Snew; also returns S', u, p */
#define ROW(t) ((b * T + (t)) * H + h)
#define STEP(S, Snew, t)                                                          \
        do {                                                                      \
            const float* kt = k + ROW(t) * dk;                                    \
            const float* gt = g + ROW(t) * dk;                                    \
            const float* vt = v + ROW(t) * dv;                                    \
            const double bt = (double)beta[ROW(t)];                               \
            for (long c = 0; c < dk; ++c) dec[c] = exp((double)gt[c]);            \
            for (long c = 0; c < dk; ++c)                                         \
                for (long j = 0; j < dv; ++j) Sp[c * dv + j] = dec[c] * (S)[c * dv + j]; \
            for (long j = 0; j < dv; ++j) p[j] = 0.0;                             \
            for (long c = 0; c < dk; ++c)                                         \
                for (long j = 0; j < dv; ++j) p[j] += (double)kt[c] * Sp[c * dv + j]; \
            for (long j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - p[j]);     \
            for (long c = 0; c < dk; ++c)                                         \
                for (long j = 0; j < dv; ++j)                                     \
                    (Snew)[c * dv + j] = Sp[c * dv + j] + (double)kt[c] * u[j];   \
        } while (0)

        if (h0) memcpy(ck, h0 + bh * SZ, sizeof(double) * SZ);
        else memset(ck, 0, sizeof(double) * SZ);
        for (long sgi = 0; sgi < nseg; ++sgi) {      /* forward: keep segment-entry states */
            memcpy(st, ck + sgi * SZ, sizeof(double) * SZ);
            const long t1 = (sgi + 1) * seg < T ? (sgi + 1) * seg : T;
            for (long t = sgi * seg; t < t1; ++t) {
                STEP(st, st + SZ, t);
                memcpy(st, st + SZ, sizeof(double) * SZ);
            }
            memcpy(ck + (sgi + 1) * SZ, st, sizeof(double) * SZ);
        }

        if (dht) memcpy(dS, dht + bh * SZ, sizeof(double) * SZ);
        else memset(dS, 0, sizeof(double) * SZ);
        for (long sgi = nseg - 1; sgi >= 0; --sgi) {
            const long t0 = sgi * seg, t1 = (sgi + 1) * seg < T ? (sgi + 1) * seg : T;
            memcpy(st, ck + sgi * SZ, sizeof(double) * SZ);
            for (long t = t0; t < t1; ++t) STEP(st + (t - t0) * SZ, st + (t - t0 + 1) * SZ, t);
            for (long t = t1 - 1; t >= t0; --t) {
                const double* Sprev = st + (t - t0) * SZ;
                const double* St = st + (t - t0 + 1) * SZ;
                STEP(Sprev, st + (t - t0 + 1) * SZ, t);   /* recompute S', u, p (S_t rewritten unchanged) */
                const float* qt = q + ROW(t) * dk;
                const float* kt = k + ROW(t) * dk;
                const float* vt = v + ROW(t) * dv;
                const double bt = (double)beta[ROW(t)];
                const double* dot = dout + ROW(t) * dv;
                double* dqt = dq + ROW(t) * dk;
                double* dkt = dk_ + ROW(t) * dk;
                double* dvt = dv_ + ROW(t) * dv;
                double* dgt = dg + ROW(t) * dk;

                /* o = scale S_t^T q */
                for (long c = 0; c < dk; ++c) {
                    double a = 0.0;
                    for (long j = 0; j < dv; ++j) a += St[c * dv + j] * dot[j];
                    dqt[c] = scale * a;
                }
                for (long c = 0; c < dk; ++c)
                    for (long j = 0; j < dv; ++j) dS[c * dv + j] += scale * (double)qt[c] * dot[j];
                /* S_t = S' + k u^T */
                for (long c = 0; c < dk; ++c) {
                    double a = 0.0;
                    for (long j = 0; j < dv; ++j) a += dS[c * dv + j] * u[j];
                    dkt[c] = a;
                }
                for (long j = 0; j < dv; ++j) du[j] = 0.0;
                for (long c = 0; c < dk; ++c)
                    for (long j = 0; j < dv; ++j) du[j] += (double)kt[c] * dS[c * dv + j];
                /* u = beta (v - p) */
                double db = 0.0;
                for (long j = 0; j < dv; ++j) db += du[j] * ((double)vt[j] - p[j]);
                dbeta[ROW(t)] = db;
                for (long j = 0; j < dv; ++j) { dvt[j] = bt * du[j]; du[j] = -bt * du[j]; }  /* du now holds dp */
                /* p = S'^T k */
                for (long c = 0; c < dk; ++c) {
                    double a = 0.0;
                    for (long j = 0; j < dv; ++j) a += Sp[c * dv + j] * du[j];
                    dkt[c] += a;
                }
                for (long c = 0; c < dk; ++c)
                    for (long j = 0; j < dv; ++j) dS[c * dv + j] += (double)kt[c] * du[j];
                /* S' = Diag(e^g) S_{t-1} */
                for (long c = 0; c < dk; ++c) {
                    double a = 0.0;
                    for (long j = 0; j < dv; ++j) a += dS[c * dv + j] * Sp[c * dv + j];
                    dgt[c] = a;
                }
                for (long c = 0; c < dk; ++c)
                    for (long j = 0; j < dv; ++j) dS[c * dv + j] *= dec[c];
            }
        }
        memcpy(dh0 + bh * SZ, dS, sizeof(double) * SZ);
#undef STEP
#undef ROW
        free(ck); free(st); free(dS); free(Sp); free(u); free(p); free(du); free(dec);
    }
    return failed ? 2 : 0;
}
