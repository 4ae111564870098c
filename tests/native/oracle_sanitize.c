/* Host-side memory and undefined-behaviour check of the fp64 oracle:
 * compiled together with oracle/kron_delta_oracle.c under
 * -fsanitize=address,undefined by tests/test_oracle_sanitized.py, it runs the
 * oracle's entry points on small seeded inputs, including the edge cases the
 * parity tests use (T = 0, one token, a ragged 64-token tail, gates at 0 and 1,
 * S0 given and not, dS_T given and not).  Exit status 0 when every call
 * returns success and produces finite values; the sanitizers abort on any
 * out-of-bounds access, leak or undefined operation. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int kdo_fwd(int B, int T, int H, int dk, int dv, const double *q, const double *k, const double *v,
            const double *f, const double *beta, const double *c, const double *S0, double *o, double *ST,
            double *r_out);
int kdo_bwd(int B, int T, int H, int dk, int dv, const double *q, const double *k, const double *v,
            const double *f, const double *beta, const double *c, const double *S0, const double *dO,
            const double *dST, double *dq, double *dk_out, double *dv_out, double *df, double *dbeta,
            double *dc, double *dS0);
int gdo_fwd(int B, int T, int H, int dk, int dv, const double *q, const double *k, const double *v,
            const double *alpha, const double *b, const double *w, const double *S0, double *o, double *ST);

static unsigned long long rng = 0x9E3779B97F4A7C15ull;
static double uni(void) {   /* xorshift64*, uniform in [0, 1) */
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (double)((rng * 2685821657736338717ull) >> 11) / 9007199254740992.0;
}
static double *arr(size_t n, double lo, double hi) {
    double *p = (double *)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uni();
    return p;
}
static int finite_all(const double *p, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static int run(int B, int T, int H, int d, int with_s0, int with_dst, int gate_edges) {
    const size_t nt = (size_t)B * T * H, nx = nt * d, ns = (size_t)B * H * d * d;
    double *q = arr(nx, -1, 1), *k = arr(nx, -1, 1), *v = arr(nx, -1, 1), *f = arr(nx, 0, 1);
    double *beta = arr(nt, 0, 2), *c = arr(nt, 0, 1), *dO = arr(nx, -1, 1);
    double *S0 = with_s0 ? arr(ns, -0.1, 0.1) : NULL, *dST = with_dst ? arr(ns, -0.1, 0.1) : NULL;
    if (gate_edges)
        for (size_t i = 0; i < nx; i += 7) f[i] = (i / 7) % 2 ? 0.0 : 1.0;
    double *o = arr(nx, 0, 0), *ST = arr(ns, 0, 0), *r = arr(nt, 0, 0);
    double *dq = arr(nx, 0, 0), *dk = arr(nx, 0, 0), *dv = arr(nx, 0, 0), *df = arr(nx, 0, 0);
    double *db = arr(nt, 0, 0), *dc = arr(nt, 0, 0), *dS0 = arr(ns, 0, 0);
    int bad = 0;
    bad |= kdo_fwd(B, T, H, d, d, q, k, v, f, beta, c, S0, o, ST, r) != 0;
    bad |= !finite_all(o, nx) || !finite_all(ST, ns) || !finite_all(r, nt);
    bad |= kdo_bwd(B, T, H, d, d, q, k, v, f, beta, c, S0, dO, dST, dq, dk, dv, df, db, dc, dS0) != 0;
    bad |= !finite_all(dq, nx) || !finite_all(dk, nx) || !finite_all(dv, nx) || !finite_all(df, nx);
    bad |= !finite_all(db, nt) || !finite_all(dc, nt) || !finite_all(dS0, ns);
    {   /* Gated Delta Rule-2: per-channel decay alpha and erase b (dk), write w (dv) */
        double *al = arr(nx, 0, 1), *bb = arr(nx, 0, 1), *ww = arr(nx, 0, 1);
        bad |= gdo_fwd(B, T, H, d, d, q, k, v, al, bb, ww, S0, o, ST) != 0;
        bad |= !finite_all(o, nx) || !finite_all(ST, ns);
        free(al); free(bb); free(ww);
    }
    free(q); free(k); free(v); free(f); free(beta); free(c); free(dO); free(S0); free(dST);
    free(o); free(ST); free(r); free(dq); free(dk); free(dv); free(df); free(db); free(dc); free(dS0);
    if (bad) fprintf(stderr, "case B=%d T=%d H=%d d=%d s0=%d dst=%d edges=%d failed\n", B, T, H, d, with_s0, with_dst,
                     gate_edges);
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= run(1, 0, 2, 8, 1, 1, 0);     /* empty sequence */
    bad |= run(2, 1, 1, 8, 0, 0, 0);     /* one token */
    bad |= run(1, 67, 2, 8, 1, 0, 1);    /* ragged tail past one 64-token chunk; f in {0, 1} */
    bad |= run(1, 130, 1, 16, 0, 1, 0);  /* several recompute checkpoints */
    bad |= run(2, 33, 3, 4, 1, 1, 1);
    return bad;
}
