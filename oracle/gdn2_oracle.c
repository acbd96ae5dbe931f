/*
 * gdn2_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, token-by-token fp64 CPU implementation of the gated
 * delta-rule-2 recurrence.  It exists to check the GPU library; the
 * product path never links, loads or calls it.  It shares no code,
 * header, table or helper with the HIP library (it does not even include
 * the library's public header): only tests/, the smoke check and the
 * bench's cpu_baseline leg may use it.
 *
 * What it computes, per (batch b, head h), with the state S in R^{dk x dv}
 * held in key-by-value orientation (rows = key channels, cols = value
 * channels), for t = 0 .. T-1:
 *
 *   1. decay:  Sbar = Diag(a_t) S,  a_t = exp(log_decay_t)      (scalar
 *      per head, or one factor per key channel).  Decay comes first and the
 *      read below sees the decayed state ("Gated DeltaNet" page, section
 *      "Decay first, then compute the write error"; course slides, "Worked
 *      case -- full trace", parts B and D).
 *   2. read:   m_t = Sbar^T k_t   (the key read of the decayed state).
 *   3. erase along the key with the erase gate, write with the write gate
 *      ("Gated DeltaNet-2" blog summary, "Core Mechanism": separate
 *      channel-wise erase gate b_t and write gate w_t; key-axis reading of
 *      both gates):
 *         S_t = Sbar - (b_t .* k_t) m_t^T + (w_t .* k_t) v_t^T
 *      (w := b when the write gate is tied to the erase gate).
 *   4. output: o_t = S_t^T (q_scale * q_t)   (read after the update, as the
 *      course slides' worked trace reads [5.30, 5.70] from S_1).
 *
 * Setting b = w = beta (scalar) gives Gated DeltaNet; per-channel decay with
 * tied scalar beta gives KDA; a = 1 gives the plain delta rule (gist.science
 * summary, "Technische Samenvatting", section 1).
 *
 * value_write_form != 0 selects the update as the gist.science summary
 * writes it ("Methodologie", 1. "Gated Delta-regel-2"): the write gate has
 * one factor per VALUE channel and the erase gate weights the read,
 *         m_t = Sbar^T (b_t .* k_t),   S_t = Sbar - k_t m_t^T + k_t (w_t .* v_t)^T
 * i.e. S_t = (I - k_t (b_t .* k_t)^T) Sbar + k_t (w_t .* v_t)^T; the write
 * gate is then [B, T, H, dv] (per channel) or [B, T, H], and must be given.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   q, k        [B, T, H, dk]
 *   v, o        [B, T, H, dv]
 *   gates       [B, T, H, dk] when *_per_key != 0, else [B, T, H]
 *               (the write gate of the value-write form: [B, T, H, dv])
 *   S0, S_T     [B, H, dk, dv]   (S0 may be NULL: zero initial state;
 *                                  S_T may be NULL: not written)
 *   w           may be NULL: tied to b.
 *
 * Returns 0 on success, -1 on a NULL required pointer or a bad size.
 * Chains (b, h) are independent and run in parallel with OpenMP when
 * nthreads > 1; within a chain the order of operations is exactly 1..4.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int gdn2_oracle_fwd(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                    const double *q, const double *k, const double *v,
                    const double *log_decay, int decay_per_key,
                    const double *erase, int erase_per_key,
                    const double *write, int write_per_key,
                    const double *S0, double q_scale,
                    double *o, double *S_T, int value_write_form, int nthreads)
{
    if (B < 0 || T < 0 || H < 1 || dk < 1 || dv < 1) return -1;
    if (B * T > 0 && (!q || !k || !v || !log_decay || !erase || !o)) return -1;
    if (value_write_form && B * T > 0 && !write) return -1;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        double *S = (double *)malloc((size_t)(dk * dv) * sizeof(double));
        double *m = (double *)malloc((size_t)dv * sizeof(double));
        if (!S || !m) {
            free(S);
            free(m);
#pragma omp atomic write
            bad = 1;
            continue;
        }
        if (S0)
            memcpy(S, S0 + bh * dk * dv, (size_t)(dk * dv) * sizeof(double));
        else
            memset(S, 0, (size_t)(dk * dv) * sizeof(double));

        for (int64_t t = 0; t < T; ++t) {
            const int64_t row = (b * T + t) * H + h; /* token-head index */
            const double *kt = k + row * dk;
            const double *qt = q + row * dk;
            const double *vt = v + row * dv;
            double *ot = o + row * dv;

            /* 1. decay each key row of the state */
            for (int64_t i = 0; i < dk; ++i) {
                const double la = decay_per_key ? log_decay[row * dk + i] : log_decay[row];
                const double a = exp(la);
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= a;
            }
            /* 2. read the decayed state along the key: m = Sbar^T k */
            for (int64_t j = 0; j < dv; ++j) m[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) m[j] += S[i * dv + j] * kt[i];
            if (value_write_form) {
                /* 2'. read along the erase-weighted key instead: m = Sbar^T (b .* k) */
                for (int64_t j = 0; j < dv; ++j) m[j] = 0.0;
                for (int64_t i = 0; i < dk; ++i) {
                    const double bi = erase_per_key ? erase[row * dk + i] : erase[row];
                    for (int64_t j = 0; j < dv; ++j) m[j] += S[i * dv + j] * bi * kt[i];
                }
                /* 3'. erase k m^T, write k (w .* v)^T */
                for (int64_t i = 0; i < dk; ++i)
                    for (int64_t j = 0; j < dv; ++j) {
                        const double wj = write_per_key ? write[row * dv + j] : write[row];
                        S[i * dv + j] = S[i * dv + j] - kt[i] * m[j] + kt[i] * wj * vt[j];
                    }
                goto query_read;
            }
            /* 3. erase (b .* k) m^T, write (w .* k) v^T */
            for (int64_t i = 0; i < dk; ++i) {
                const double bi = erase_per_key ? erase[row * dk + i] : erase[row];
                double wi;
                if (write)
                    wi = write_per_key ? write[row * dk + i] : write[row];
                else
                    wi = bi;
                const double ei = bi * kt[i];
                const double ui = wi * kt[i];
                for (int64_t j = 0; j < dv; ++j)
                    S[i * dv + j] = S[i * dv + j] - ei * m[j] + ui * vt[j];
            }
        query_read:;
            /* 4. read the updated state with the query */
            for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
                const double qi = q_scale * qt[i];
                for (int64_t j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * qi;
            }
        }
        if (S_T) memcpy(S_T + bh * dk * dv, S, (size_t)(dk * dv) * sizeof(double));
        free(S);
        free(m);
    }
    return bad ? -1 : 0;
}

int gdn2_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
