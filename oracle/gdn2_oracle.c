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

/*
 * gdn2_oracle_bwd -- TEST INFRASTRUCTURE ONLY.
 *
 * The gradients of L = <d_o, o> + <d_ST, S_T> with respect to every input of
 * gdn2_oracle_fwd (key form: erase (b .* k) m^T, write (w .* k) v^T), as the
 * reverse-mode derivative of steps 1..4 above written out by hand, token by
 * token, in fp64.  With S the state entering token t, a = exp(log_decay_t),
 * e = b .* k, u = w .* k, q~ = q_scale q and dS the gradient of the state
 * leaving token t (d_ST for the last one):
 *
 *   forward again:  Sbar = a .* S (rows),  m = Sbar^T k,
 *                   S' = Sbar - e m^T + u v^T,   o = S'^T q~
 *   4. read         dS  += q~ do^T,          dq = q_scale S' do
 *   3. erase/write  dm   = -dS^T e,          de = -dS m,   du = dS v,
 *                   dv   = dS^T u
 *   2. key read     dk   = Sbar dm + de .* b + du .* w,    dSbar = dS + k dm^T
 *                   (e = b .* k and u = w .* k give db = de .* k, dw = du .* k;
 *                   tied, w := b, the erase gate collects both)
 *   1. decay        d log_decay = a .* rowsum(dSbar .* S),   dS <- a .* dSbar
 *
 * and d_S0 is the dS left after token 0.  A gate given per token-head takes
 * the sum of its per-channel gradients.  The states entering every token are
 * recomputed per segment of SEG tokens from checkpoints taken on a first
 * forward pass.  Chains run in parallel (OpenMP); each writes only its own
 * rows, so there are no races.  The value-write form is not covered here
 * (returns -2).  Returns 0, or -1 on a NULL required pointer, a bad size or
 * a failed allocation.
 */
#define GDN2_ORACLE_SEG 64

int gdn2_oracle_bwd(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                    const double *q, const double *k, const double *v,
                    const double *log_decay, int decay_per_key,
                    const double *erase, int erase_per_key,
                    const double *write, int write_per_key,
                    const double *S0, double q_scale,
                    const double *d_o, const double *d_ST,
                    double *dq, double *dk_out, double *dv_out,
                    double *d_log_decay, double *d_erase, double *d_write,
                    double *d_S0, int value_write_form, int nthreads)
{
    if (value_write_form) return -2;
    if (B < 0 || T < 0 || H < 1 || dk < 1 || dv < 1) return -1;
    if (B * T > 0 && (!q || !k || !v || !log_decay || !erase || !dq || !dk_out || !dv_out ||
                      !d_log_decay || !d_erase))
        return -1;
    if (B * T > 0 && write && !d_write) return -1;
    if (nthreads < 1) nthreads = 1;
    const int64_t L = GDN2_ORACLE_SEG;
    const int64_t nseg = (T + L - 1) / L;
    const int64_t n2 = dk * dv;
    int bad = 0;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        double *ck = (double *)malloc((size_t)((nseg > 0 ? nseg : 1) * n2) * sizeof(double));
        double *st = (double *)malloc((size_t)(L * n2) * sizeof(double));
        double *S = (double *)malloc((size_t)n2 * sizeof(double));
        double *Sb = (double *)malloc((size_t)n2 * sizeof(double));
        double *Sn = (double *)malloc((size_t)n2 * sizeof(double));
        double *dS = (double *)malloc((size_t)n2 * sizeof(double));
        double *vec = (double *)malloc((size_t)(6 * dk + 3 * dv) * sizeof(double));
        if (!ck || !st || !S || !Sb || !Sn || !dS || !vec) {
            free(ck); free(st); free(S); free(Sb); free(Sn); free(dS); free(vec);
#pragma omp atomic write
            bad = 1;
            continue;
        }
        double *a = vec, *bt = vec + dk, *wt = vec + 2 * dk, *de = vec + 3 * dk, *du = vec + 4 * dk,
               *dla = vec + 5 * dk;
        double *m = vec + 6 * dk, *dm = m + dv, *tmp = dm + dv;
        (void)tmp;

        /* the gates of token-head `row`, per channel */
        #define GDN2_GATES(row)                                                              \
            for (int64_t c = 0; c < dk; ++c) {                                               \
                a[c] = exp(decay_per_key ? log_decay[(row) * dk + c] : log_decay[(row)]);    \
                bt[c] = erase_per_key ? erase[(row) * dk + c] : erase[(row)];                \
                wt[c] = write ? (write_per_key ? write[(row) * dk + c] : write[(row)]) : bt[c]; \
            }
        /* one forward token from S (entering) into Sn (leaving); also
           leaves Sbar in Sb and m */
        #define GDN2_STEP(row)                                                               \
            do {                                                                             \
                const double *kt_ = k + (row) * dk, *vt_ = v + (row) * dv;                   \
                for (int64_t c = 0; c < dk; ++c)                                             \
                    for (int64_t j = 0; j < dv; ++j) Sb[c * dv + j] = a[c] * S[c * dv + j];  \
                for (int64_t j = 0; j < dv; ++j) m[j] = 0.0;                                 \
                for (int64_t c = 0; c < dk; ++c)                                             \
                    for (int64_t j = 0; j < dv; ++j) m[j] += Sb[c * dv + j] * kt_[c];        \
                for (int64_t c = 0; c < dk; ++c) {                                           \
                    const double ec = bt[c] * kt_[c], uc = wt[c] * kt_[c];                   \
                    for (int64_t j = 0; j < dv; ++j)                                         \
                        Sn[c * dv + j] = Sb[c * dv + j] - ec * m[j] + uc * vt_[j];           \
                }                                                                            \
            } while (0)

        /* forward pass: checkpoint the state entering every segment */
        if (S0) memcpy(S, S0 + bh * n2, (size_t)n2 * sizeof(double));
        else memset(S, 0, (size_t)n2 * sizeof(double));
        for (int64_t t = 0; t < T; ++t) {
            if (t % L == 0) memcpy(ck + (t / L) * n2, S, (size_t)n2 * sizeof(double));
            const int64_t row = (b * T + t) * H + h;
            GDN2_GATES(row);
            GDN2_STEP(row);
            memcpy(S, Sn, (size_t)n2 * sizeof(double));
        }

        /* reverse pass */
        if (d_ST) memcpy(dS, d_ST + bh * n2, (size_t)n2 * sizeof(double));
        else memset(dS, 0, (size_t)n2 * sizeof(double));
        for (int64_t s = nseg - 1; s >= 0; --s) {
            const int64_t t0 = s * L, t1 = (t0 + L < T) ? t0 + L : T;
            /* the states entering tokens t0 .. t1-1 */
            memcpy(S, ck + s * n2, (size_t)n2 * sizeof(double));
            for (int64_t t = t0; t < t1; ++t) {
                memcpy(st + (t - t0) * n2, S, (size_t)n2 * sizeof(double));
                if (t + 1 < t1) {
                    const int64_t row = (b * T + t) * H + h;
                    GDN2_GATES(row);
                    GDN2_STEP(row);
                    memcpy(S, Sn, (size_t)n2 * sizeof(double));
                }
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const int64_t row = (b * T + t) * H + h;
                const double *kt = k + row * dk, *vt = v + row * dv, *qt = q + row * dk;
                memcpy(S, st + (t - t0) * n2, (size_t)n2 * sizeof(double));
                GDN2_GATES(row);
                GDN2_STEP(row);
                /* 4. the query read o = S'^T (q_scale q) */
                const double *dot = d_o ? d_o + row * dv : NULL;
                for (int64_t c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    if (dot)
                        for (int64_t j = 0; j < dv; ++j) {
                            acc += Sn[c * dv + j] * dot[j];
                            dS[c * dv + j] += q_scale * qt[c] * dot[j];
                        }
                    dq[row * dk + c] = q_scale * acc;
                }
                /* 3. erase and write: S' = Sbar - e m^T + u v^T */
                for (int64_t j = 0; j < dv; ++j) {
                    double am = 0.0, av = 0.0;
                    for (int64_t c = 0; c < dk; ++c) {
                        am -= dS[c * dv + j] * bt[c] * kt[c];
                        av += dS[c * dv + j] * wt[c] * kt[c];
                    }
                    dm[j] = am;
                    dv_out[row * dv + j] = av;
                }
                for (int64_t c = 0; c < dk; ++c) {
                    double ae = 0.0, au = 0.0;
                    for (int64_t j = 0; j < dv; ++j) {
                        ae -= dS[c * dv + j] * m[j];
                        au += dS[c * dv + j] * vt[j];
                    }
                    de[c] = ae;
                    du[c] = au;
                }
                /* 2. the key read m = Sbar^T k; dSbar = dS + k dm^T (in dS) */
                for (int64_t c = 0; c < dk; ++c) {
                    double ak = 0.0;
                    for (int64_t j = 0; j < dv; ++j) {
                        ak += Sb[c * dv + j] * dm[j];
                        dS[c * dv + j] += kt[c] * dm[j];
                    }
                    dk_out[row * dk + c] = ak + de[c] * bt[c] + du[c] * wt[c];
                }
                /* 1. decay: Sbar = a .* S (S is the state entering token t) */
                for (int64_t c = 0; c < dk; ++c) {
                    double ad = 0.0;
                    for (int64_t j = 0; j < dv; ++j) ad += dS[c * dv + j] * S[c * dv + j];
                    dla[c] = a[c] * ad;
                    for (int64_t j = 0; j < dv; ++j) dS[c * dv + j] *= a[c];
                }
                /* the gates' gradients, summed over channels when per head */
                double sla = 0.0, sb = 0.0, sw = 0.0;
                for (int64_t c = 0; c < dk; ++c) {
                    const double gb = de[c] * kt[c] + (write ? 0.0 : du[c] * kt[c]);
                    const double gw = du[c] * kt[c];
                    if (decay_per_key) d_log_decay[row * dk + c] = dla[c];
                    if (erase_per_key) d_erase[row * dk + c] = gb;
                    if (write && write_per_key) d_write[row * dk + c] = gw;
                    sla += dla[c];
                    sb += gb;
                    sw += gw;
                }
                if (!decay_per_key) d_log_decay[row] = sla;
                if (!erase_per_key) d_erase[row] = sb;
                if (write && !write_per_key) d_write[row] = sw;
            }
        }
        if (d_S0) memcpy(d_S0 + bh * n2, dS, (size_t)n2 * sizeof(double));
        #undef GDN2_GATES
        #undef GDN2_STEP
        free(ck); free(st); free(S); free(Sb); free(Sn); free(dS); free(vec);
    }
    return bad ? -1 : 0;
}
