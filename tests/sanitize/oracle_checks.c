/*
 * The fp64 oracle (oracle/gdn2_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every entry point on small inputs of every
 * gate kind and both forms, serial and threaded, with checks that need no
 * stored values -- a split sequence resumed from its final state equals one
 * call bit for bit, decay alone multiplies the state by the decays, scalar
 * gates make the two forms agree, T = 0 returns the initial state, and the
 * reverse pass equals central differences of L = <d_o, o> + <d_ST, S_T>.
 * Prints one line per failed check and exits with their count.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdn2_oracle_fwd(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, const double *q, const double *k,
                    const double *v, const double *log_decay, int decay_per_key, const double *erase,
                    int erase_per_key, const double *write, int write_per_key, const double *S0, double q_scale,
                    double *o, double *S_T, int value_write_form, int nthreads);
int gdn2_oracle_bwd(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, const double *q, const double *k,
                    const double *v, const double *log_decay, int decay_per_key, const double *erase,
                    int erase_per_key, const double *write, int write_per_key, const double *S0, double q_scale,
                    const double *d_o, const double *d_ST, double *dq, double *dk_out, double *dv_out,
                    double *d_log_decay, double *d_erase, double *d_write, double *d_S0, int value_write_form,
                    int nthreads);

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            printf("FAIL line %d: ", __LINE__);            \
            printf(__VA_ARGS__);                           \
            printf("\n");                                  \
            ++failures;                                    \
        }                                                  \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double unif(void) { /* xorshift64*, uniform in (0, 1) */
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return ((rng * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0) + 1e-300;
}
static double *fill(size_t n, double lo, double hi) {
    double *p = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * unif();
    return p;
}

typedef struct {
    int64_t B, T, H, dk, dv;
    int la_key, eb_key, wr_key, tied, vw;
    double *q, *k, *v, *la, *eb, *wr, *S0;
} Case;

static Case make(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int la_key, int eb_key, int wr_key,
                 int tied, int vw) {
    Case c = {B, T, H, dk, dv, la_key, eb_key, wr_key, tied, vw, 0, 0, 0, 0, 0, 0, 0};
    const size_t tok = (size_t)(B * T * H);
    c.q = fill(tok * dk, -1, 1);
    c.k = fill(tok * dk, -0.5, 0.5);
    c.v = fill(tok * dv, -1, 1);
    c.la = fill(tok * (la_key ? dk : 1), -0.7, -0.01);
    c.eb = fill(tok * (eb_key ? dk : 1), 0, 1);
    c.wr = tied ? NULL : fill(tok * (wr_key ? (vw ? dv : dk) : 1), 0, 1);
    c.S0 = fill((size_t)(B * H * dk * dv), -0.5, 0.5);
    return c;
}

static void drop(Case *c) {
    free(c->q); free(c->k); free(c->v); free(c->la); free(c->eb); free(c->wr); free(c->S0);
}

static int run(const Case *c, int64_t t0, int64_t t1, const double *S0, double *o, double *ST, int nthreads) {
    /* tokens t0 .. t1-1 of a B = 1 case (rows of [T, H, ...] are contiguous in t) */
    const int64_t H = c->H, dk = c->dk, dv = c->dv;
    const int64_t gl = c->la_key ? dk : 1, ge = c->eb_key ? dk : 1, gw = c->wr_key ? (c->vw ? dv : dk) : 1;
    return gdn2_oracle_fwd(c->B, t1 - t0, H, dk, dv, c->q + t0 * H * dk, c->k + t0 * H * dk, c->v + t0 * H * dv,
                           c->la + t0 * H * gl, c->la_key, c->eb + t0 * H * ge, c->eb_key,
                           c->wr ? c->wr + t0 * H * gw : NULL, c->wr_key, S0, 0.75, o, ST, c->vw, nthreads);
}

static double loss(const Case *c, const double *d_o, const double *d_ST) {
    const size_t no = (size_t)(c->T * c->H * c->dv), ns = (size_t)(c->H * c->dk * c->dv);
    double *o = malloc(no * sizeof(double)), *ST = malloc(ns * sizeof(double));
    run(c, 0, c->T, c->S0, o, ST, 1);
    double L = 0;
    for (size_t i = 0; i < no; ++i) L += d_o[i] * o[i];
    for (size_t i = 0; i < ns; ++i) L += d_ST[i] * ST[i];
    free(o); free(ST);
    return L;
}

/* central difference of L along element i of x, against the analytic gradient g */
static void fd_check(const Case *c, double *x, size_t i, double g, const double *d_o, const double *d_ST,
                     const char *what) {
    const double h = 1e-6, x0 = x[i];
    x[i] = x0 + h; const double lp = loss(c, d_o, d_ST);
    x[i] = x0 - h; const double lm = loss(c, d_o, d_ST);
    x[i] = x0;
    const double fd = (lp - lm) / (2 * h);
    CHECK(fabs(fd - g) <= 1e-6 * (1 + fabs(fd)), "%s[%zu]: reverse pass %.12g, central difference %.12g", what, i,
          g, fd);
}

static void forward_checks(int la_key, int eb_key, int wr_key, int tied, int vw, int nthreads) {
    Case c = make(1, 37, 3, 5, 7, la_key, eb_key, wr_key, tied, vw);
    const size_t no = (size_t)(c.T * c.H * c.dv), ns = (size_t)(c.H * c.dk * c.dv);
    double *o = calloc(no, sizeof(double)), *ST = calloc(ns, sizeof(double));
    double *o2 = calloc(no, sizeof(double)), *mid = calloc(ns, sizeof(double)), *ST2 = calloc(ns, sizeof(double));
    CHECK(run(&c, 0, c.T, c.S0, o, ST, nthreads) == 0, "forward failed");
    /* split at t = 11, resume from the state there */
    CHECK(run(&c, 0, 11, c.S0, o2, mid, nthreads) == 0, "first part failed");
    CHECK(run(&c, 11, c.T, mid, o2 + 11 * c.H * c.dv, ST2, nthreads) == 0, "second part failed");
    CHECK(memcmp(o, o2, no * sizeof(double)) == 0 && memcmp(ST, ST2, ns * sizeof(double)) == 0,
          "split and resume differs from one call (kinds %d%d%d tied %d vw %d)", la_key, eb_key, wr_key, tied, vw);
    /* T = 0 returns the initial state */
    CHECK(run(&c, 0, 0, c.S0, NULL, ST2, nthreads) == 0 && memcmp(ST2, c.S0, ns * sizeof(double)) == 0,
          "T = 0 changed the state");
    free(o); free(ST); free(o2); free(mid); free(ST2);
    drop(&c);
}

static void decay_only(void) {
    Case c = make(1, 13, 2, 4, 3, 1, 1, 1, 0, 0);
    const size_t tok = (size_t)(c.T * c.H * c.dk), ns = (size_t)(c.H * c.dk * c.dv);
    memset(c.eb, 0, tok * sizeof(double));
    memset(c.wr, 0, tok * sizeof(double));
    double *o = calloc((size_t)(c.T * c.H * c.dv), sizeof(double)), *ST = calloc(ns, sizeof(double));
    run(&c, 0, c.T, c.S0, o, ST, 1);
    for (int64_t h = 0; h < c.H; ++h)
        for (int64_t i = 0; i < c.dk; ++i) {
            double g = 0;
            for (int64_t t = 0; t < c.T; ++t) g += c.la[(t * c.H + h) * c.dk + i];
            for (int64_t j = 0; j < c.dv; ++j) {
                const size_t e = (size_t)((h * c.dk + i) * c.dv + j);
                CHECK(fabs(ST[e] - exp(g) * c.S0[e]) <= 1e-13 * fabs(c.S0[e]), "decay-only state wrong at %zu", e);
            }
        }
    free(o); free(ST);
    drop(&c);
}

static void scalar_gates_forms_agree(void) {
    Case c = make(1, 21, 2, 4, 6, 1, 0, 0, 0, 1);
    const size_t no = (size_t)(c.T * c.H * c.dv), ns = (size_t)(c.H * c.dk * c.dv);
    double *o = calloc(no, sizeof(double)), *ST = calloc(ns, sizeof(double));
    double *o2 = calloc(no, sizeof(double)), *ST2 = calloc(ns, sizeof(double));
    run(&c, 0, c.T, c.S0, o, ST, 1);
    c.vw = 0;
    run(&c, 0, c.T, c.S0, o2, ST2, 1);
    double e = 0, n = 0;
    for (size_t i = 0; i < no; ++i) { e += (o[i] - o2[i]) * (o[i] - o2[i]); n += o[i] * o[i]; }
    for (size_t i = 0; i < ns; ++i) { e += (ST[i] - ST2[i]) * (ST[i] - ST2[i]); n += ST[i] * ST[i]; }
    CHECK(sqrt(e / n) < 1e-13, "scalar gates: the two forms differ by %.3g", sqrt(e / n));
    free(o); free(ST); free(o2); free(ST2);
    drop(&c);
}

static void reverse_pass(int la_key, int eb_key, int wr_key, int tied, int nthreads) {
    Case c = make(1, 9, 2, 3, 2, la_key, eb_key, wr_key, tied, 0);
    const int64_t H = c.H, dk = c.dk, dv = c.dv, T = c.T;
    const size_t no = (size_t)(T * H * dv), ns = (size_t)(H * dk * dv), nq = (size_t)(T * H * dk);
    const size_t nl = (size_t)(T * H * (la_key ? dk : 1)), ne = (size_t)(T * H * (eb_key ? dk : 1));
    const size_t nw = tied ? 0 : (size_t)(T * H * (wr_key ? dk : 1));
    double *d_o = fill(no, -1, 1), *d_ST = fill(ns, -1, 1);
    double *dq = calloc(nq, 8), *dk_ = calloc(nq, 8), *dv_ = calloc(no, 8), *dl = calloc(nl, 8);
    double *de = calloc(ne, 8), *dw = calloc(nw ? nw : 1, 8), *dS0 = calloc(ns, 8);
    CHECK(gdn2_oracle_bwd(1, T, H, dk, dv, c.q, c.k, c.v, c.la, la_key, c.eb, eb_key, c.wr, wr_key, c.S0, 0.75, d_o,
                          d_ST, dq, dk_, dv_, dl, de, tied ? NULL : dw, dS0, 0, nthreads) == 0,
          "reverse pass failed");
    const size_t picks[] = {0, 5, 11, 17};
    for (int p = 0; p < 4; ++p) {
        fd_check(&c, c.q, picks[p] % nq, dq[picks[p] % nq], d_o, d_ST, "q");
        fd_check(&c, c.k, picks[p] % nq, dk_[picks[p] % nq], d_o, d_ST, "k");
        fd_check(&c, c.v, picks[p] % no, dv_[picks[p] % no], d_o, d_ST, "v");
        fd_check(&c, c.la, picks[p] % nl, dl[picks[p] % nl], d_o, d_ST, "log_decay");
        fd_check(&c, c.eb, picks[p] % ne, de[picks[p] % ne], d_o, d_ST, "erase");
        if (!tied) fd_check(&c, c.wr, picks[p] % nw, dw[picks[p] % nw], d_o, d_ST, "write");
        fd_check(&c, c.S0, picks[p] % ns, dS0[picks[p] % ns], d_o, d_ST, "S0");
    }
    free(d_o); free(d_ST); free(dq); free(dk_); free(dv_); free(dl); free(de); free(dw); free(dS0);
    drop(&c);
}

int main(void) {
    for (int threads = 1; threads <= 3; threads += 2) {
        forward_checks(1, 1, 1, 0, 0, threads);
        forward_checks(0, 0, 0, 1, 0, threads);
        forward_checks(1, 0, 0, 1, 0, threads);
        forward_checks(1, 1, 0, 0, 0, threads);
        forward_checks(1, 1, 1, 0, 1, threads);
        forward_checks(0, 0, 0, 0, 1, threads);
        reverse_pass(1, 1, 1, 0, threads);
        reverse_pass(0, 0, 0, 1, threads);
        reverse_pass(1, 0, 0, 1, threads);
    }
    decay_only();
    scalar_gates_forms_agree();
    printf("%d failures\n", failures);
    return failures;
}
