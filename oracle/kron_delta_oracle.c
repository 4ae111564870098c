/*
 * kron_delta_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, sequential fp64 CPU reference of the Kronecker delta rule
 * mixer and of its reverse-mode gradient.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load or call this file.  It
 * shares no code, header, table or helper with the GPU library; the GPU
 * library never loads it.
 *
 * Sources (web pages; cited by title and section):
 *   [KS] onedev.kr paper summary "KronLSTM이 스칼라 보정으로 긴 문맥 선형 어텐션의
 *        기억 간섭을 줄인다" -- sections "어떻게 동작하나" (how it works),
 *        "무엇과 다른가" (how it differs), "어떻게 쓰나" (how it is used).
 *   [KR] blog review "[논문리뷰] Kronecker Delta Rule for Long Context Linear
 *        Attention" -- section 3 (Method & Key Results).
 *
 * The recurrence, per batch element b and head h, state S in R^{dv x dk}
 * (row index i over the value dimension, column index j over the key
 * dimension), for t = 1..T:
 *   (R1) Sbar = S_{t-1} diag(f_t)          key-channel forget gate applied from
 *                                           the right ([KS] how it is used)
 *   (R2) r_t  = v_t^T Sbar k_t             scalar association strength that the
 *                                           rule corrects ([KS] how it works)
 *   (R3) S_t  = Sbar + (c_t - beta_t r_t) v_t k_t^T
 *                                           correction along the outer product of
 *                                           the input pair; beta erases, c writes
 *                                           ([KS] how it works)
 *   (R4) o_t  = S_t q_t                    readout of the post-update state
 * Nothing but S is carried between steps ([KS] how it is used).  The gates
 * f, beta, c are inputs: they are computed upstream of the mixer.
 *
 * Layouts (all row-major, fp64, host memory owned by the caller):
 *   q, k, f : [B, T, H, dk]     v, o, dO : [B, T, H, dv]
 *   beta, c : [B, T, H]         S0, ST   : [B, H, dv, dk]  (S[i][j] at i*dk+j)
 * Parallelism: OpenMP over the B*H independent (b, h) recurrences only; the
 * time loop of each is strictly sequential.
 */
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDO_OK 0
#define KDO_ERR_ARG (-1)
#define KDO_ERR_MEM (-2)

static size_t tok_index(int b, int t, int h, int T, int H)
{
    return ((size_t)b * (size_t)T + (size_t)t) * (size_t)H + (size_t)h;
}

int kdo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void kdo_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* One step of R1..R4 on state S (dv x dk) in place.  Returns r_t and writes
 * o_t when o is non-null. */
static double kdo_step(double *S, int dk, int dv, const double *qt,
                       const double *kt, const double *vt, const double *ft,
                       double bt, double ct, double *ot)
{
    int i, j;
    double r = 0.0, u;
    /* R1: decay every key column j by f_t[j]. */
    for (i = 0; i < dv; ++i)
        for (j = 0; j < dk; ++j)
            S[(size_t)i * dk + j] *= ft[j];
    /* R2: r = v^T Sbar k. */
    for (i = 0; i < dv; ++i) {
        double row = 0.0;
        for (j = 0; j < dk; ++j)
            row += S[(size_t)i * dk + j] * kt[j];
        r += vt[i] * row;
    }
    /* R3: rank-one correction along v k^T with scalar weight c - beta r. */
    u = ct - bt * r;
    for (i = 0; i < dv; ++i)
        for (j = 0; j < dk; ++j)
            S[(size_t)i * dk + j] += u * vt[i] * kt[j];
    /* R4: o = S_t q. */
    if (ot) {
        for (i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (j = 0; j < dk; ++j)
                acc += S[(size_t)i * dk + j] * qt[j];
            ot[i] = acc;
        }
    }
    return r;
}

/*
 * Forward.  S0 may be NULL (zero initial state); ST may be NULL (not
 * returned).  r_out, when non-null, receives r_t as [B, T, H].
 */
int kdo_fwd(int B, int T, int H, int dk, int dv,
            const double *q, const double *k, const double *v,
            const double *f, const double *beta, const double *c,
            const double *S0, double *o, double *ST, double *r_out)
{
    int bh, fail = 0;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return KDO_ERR_ARG;
    if (B * H == 0) return KDO_OK;
    if (T > 0 && (!q || !k || !v || !f || !beta || !c || !o)) return KDO_ERR_ARG;

#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < B * H; ++bh) {
        int b = bh / H, h = bh % H, t;
        size_t sz = (size_t)dv * dk;
        double *S = (double *)malloc(sz * sizeof(double));
        if (!S) {
#pragma omp atomic write
            fail = 1;
            continue;
        }
        if (S0) memcpy(S, S0 + (size_t)bh * sz, sz * sizeof(double));
        else memset(S, 0, sz * sizeof(double));
        for (t = 0; t < T; ++t) {
            size_t n = tok_index(b, t, h, T, H);
            double r = kdo_step(S, dk, dv, q + n * dk, k + n * dk, v + n * dv,
                                f + n * dk, beta[n], c[n], o + n * dv);
            if (r_out) r_out[n] = r;
        }
        if (ST) memcpy(ST + (size_t)bh * sz, S, sz * sizeof(double));
        free(S);
    }
    return fail ? KDO_ERR_MEM : KDO_OK;
}

/*
 * Reverse-mode gradient of L = sum_t <dO_t, o_t> + <dST, S_T> with respect to
 * q, k, v, f, beta, c and S0, derived by hand from R1..R4 (chain rule applied
 * to each statement of the step, last statement first).  With G = dL/dS_t:
 *   R4:  G += dO_t q_t^T ;  dq_t = S_t^T dO_t
 *   R3:  du = v_t^T G k_t ;  dv_t = u G k_t ;  dk_t = u G^T v_t ;
 *        dc_t = du ;  dbeta_t = -r_t du ;  dr = -beta_t du
 *   R2:  dv_t += dr Sbar k_t ;  dk_t += dr Sbar^T v_t ;  Gbar = G + dr v_t k_t^T
 *   R1:  df_t[j] = sum_i S_{t-1}[i][j] Gbar[i][j] ;  G <- Gbar diag(f_t)
 * and dS0 = G after step 1.  States are recomputed segment by segment from
 * checkpoints taken every KDO_SEG steps of a forward sweep (a memory strategy
 * only: the arithmetic is the sequential step above).
 * dST may be NULL (zero); dS0 may be NULL (not returned).
 */
#define KDO_SEG 64
int kdo_bwd(int B, int T, int H, int dk, int dv,
            const double *q, const double *k, const double *v,
            const double *f, const double *beta, const double *c,
            const double *S0, const double *dO, const double *dST,
            double *dq, double *dk_out, double *dv_out, double *df,
            double *dbeta, double *dc, double *dS0)
{
    int bh, fail = 0;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return KDO_ERR_ARG;
    if (B * H == 0) return KDO_OK;
    if (T > 0 && (!q || !k || !v || !f || !beta || !c || !dO || !dq || !dk_out ||
                  !dv_out || !df || !dbeta || !dc))
        return KDO_ERR_ARG;

#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < B * H; ++bh) {
        int b = bh / H, h = bh % H;
        int nseg = (T + KDO_SEG - 1) / KDO_SEG, seg, i, j, s;
        size_t sz = (size_t)dv * dk;
        double *ckpt = (double *)malloc(((size_t)(nseg > 0 ? nseg : 1)) * sz * sizeof(double));
        double *states = (double *)malloc((size_t)(KDO_SEG + 1) * sz * sizeof(double));
        double *rseg = (double *)malloc(KDO_SEG * sizeof(double));
        double *G = (double *)malloc(sz * sizeof(double));
        double *Gk = (double *)malloc((size_t)dv * sizeof(double));
        double *Gtv = (double *)malloc((size_t)dk * sizeof(double));
        if (!ckpt || !states || !rseg || !G || !Gk || !Gtv) {
            free(ckpt); free(states); free(rseg); free(G); free(Gk); free(Gtv);
#pragma omp atomic write
            fail = 1;
            continue;
        }
        /* Forward sweep: checkpoint the state entering each segment. */
        {
            double *S = states; /* scratch */
            int t;
            if (S0) memcpy(S, S0 + (size_t)bh * sz, sz * sizeof(double));
            else memset(S, 0, sz * sizeof(double));
            for (t = 0; t < T; ++t) {
                size_t n = tok_index(b, t, h, T, H);
                if (t % KDO_SEG == 0)
                    memcpy(ckpt + (size_t)(t / KDO_SEG) * sz, S, sz * sizeof(double));
                kdo_step(S, dk, dv, q + n * dk, k + n * dk, v + n * dv, f + n * dk,
                         beta[n], c[n], NULL);
            }
        }
        if (dST) memcpy(G, dST + (size_t)bh * sz, sz * sizeof(double));
        else memset(G, 0, sz * sizeof(double));

        for (seg = nseg - 1; seg >= 0; --seg) {
            int t0 = seg * KDO_SEG;
            int L = (T - t0 < KDO_SEG) ? (T - t0) : KDO_SEG;
            /* states[s] = S_{t0+s-1} (state entering step t0+s); states[s+1] = S_{t0+s}. */
            memcpy(states, ckpt + (size_t)seg * sz, sz * sizeof(double));
            for (s = 0; s < L; ++s) {
                size_t n = tok_index(b, t0 + s, h, T, H);
                double *nxt = states + (size_t)(s + 1) * sz;
                memcpy(nxt, states + (size_t)s * sz, sz * sizeof(double));
                rseg[s] = kdo_step(nxt, dk, dv, q + n * dk, k + n * dk, v + n * dv,
                                   f + n * dk, beta[n], c[n], NULL);
            }
            for (s = L - 1; s >= 0; --s) {
                size_t n = tok_index(b, t0 + s, h, T, H);
                const double *qt = q + n * dk, *kt = k + n * dk, *vt = v + n * dv;
                const double *ft = f + n * dk, *dot = dO + n * dv;
                const double *Sprev = states + (size_t)s * sz;
                const double *Scur = states + (size_t)(s + 1) * sz;
                double *dqt = dq + n * dk, *dkt = dk_out + n * dk, *dvt = dv_out + n * dv;
                double *dft = df + n * dk;
                double r = rseg[s], u = c[n] - beta[n] * r, du = 0.0, dr;

                /* R4 */
                for (j = 0; j < dk; ++j) {
                    double acc = 0.0;
                    for (i = 0; i < dv; ++i) acc += Scur[(size_t)i * dk + j] * dot[i];
                    dqt[j] = acc;
                }
                for (i = 0; i < dv; ++i)
                    for (j = 0; j < dk; ++j)
                        G[(size_t)i * dk + j] += dot[i] * qt[j];
                /* R3 */
                for (i = 0; i < dv; ++i) {
                    double acc = 0.0;
                    for (j = 0; j < dk; ++j) acc += G[(size_t)i * dk + j] * kt[j];
                    Gk[i] = acc;
                    du += vt[i] * acc;
                }
                for (j = 0; j < dk; ++j) {
                    double acc = 0.0;
                    for (i = 0; i < dv; ++i) acc += G[(size_t)i * dk + j] * vt[i];
                    Gtv[j] = acc;
                }
                dc[n] = du;
                dbeta[n] = -r * du;
                dr = -beta[n] * du;
                /* R2, with Sbar = Sprev diag(f_t) */
                for (i = 0; i < dv; ++i) {
                    double acc = 0.0;
                    for (j = 0; j < dk; ++j) acc += Sprev[(size_t)i * dk + j] * ft[j] * kt[j];
                    dvt[i] = u * Gk[i] + dr * acc;
                }
                for (j = 0; j < dk; ++j) {
                    double acc = 0.0;
                    for (i = 0; i < dv; ++i) acc += Sprev[(size_t)i * dk + j] * vt[i];
                    dkt[j] = u * Gtv[j] + dr * ft[j] * acc;
                }
                for (i = 0; i < dv; ++i)
                    for (j = 0; j < dk; ++j)
                        G[(size_t)i * dk + j] += dr * vt[i] * kt[j];
                /* R1 */
                for (j = 0; j < dk; ++j) {
                    double acc = 0.0;
                    for (i = 0; i < dv; ++i) acc += Sprev[(size_t)i * dk + j] * G[(size_t)i * dk + j];
                    dft[j] = acc;
                }
                for (i = 0; i < dv; ++i)
                    for (j = 0; j < dk; ++j)
                        G[(size_t)i * dk + j] *= ft[j];
            }
        }
        if (dS0) memcpy(dS0 + (size_t)bh * sz, G, sz * sizeof(double));
        free(ckpt); free(states); free(rseg); free(G); free(Gk); free(Gtv);
    }
    return fail ? KDO_ERR_MEM : KDO_OK;
}

/* ======================================================================
 * Gated Delta Rule-2 (decoupled erase and write), forward only.
 *
 * Source: aitrends.kr summary of Gated DeltaNet-2 -- sections 핵심 기여
 * (decoupled erase and write; the update S_t = (I - k_t e_t^T) D_t S_{t-1}
 * + k_t z_t^T with e_t = b_t * k_t, z_t = w_t * v_t) and 방법론 steps 1, 2
 * and 4 (channel decay absorbed first, Sbar_t = D_t S_{t-1}, then
 * S_t = Sbar_t + k_t (z_t - Sbar_t^T e_t)^T; readout o_t = S_t^T q_t).
 *
 * State S in R^{dk x dv} (row j over keys, column i over values), per
 * (b, h), for t = 1..T:
 *   (G1) Sbar = diag(alpha_t) S_{t-1}       key-channel decay D_t
 *   (G2) u_t  = w_t * v_t - Sbar^T (b_t * k_t)
 *                                            what the erase leaves to write
 *   (G3) S_t  = Sbar + k_t u_t^T
 *   (G4) o_t  = S_t^T q_t
 * Layouts: q, k, alpha, b : [B, T, H, dk];  v, w, o : [B, T, H, dv];
 *          S0, ST : [B, H, dk, dv]  (S[j][i] at j*dv + i).
 * ====================================================================== */
static void gdo_step(double *S, int dk, int dv, const double *qt, const double *kt,
                     const double *vt, const double *at, const double *bt,
                     const double *wt, double *u, double *ot)
{
    int i, j;
    /* G1 */
    for (j = 0; j < dk; ++j)
        for (i = 0; i < dv; ++i)
            S[(size_t)j * dv + i] *= at[j];
    /* G2: u = z - Sbar^T e, e = b * k, z = w * v */
    for (i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (j = 0; j < dk; ++j)
            acc += S[(size_t)j * dv + i] * (bt[j] * kt[j]);
        u[i] = wt[i] * vt[i] - acc;
    }
    /* G3 */
    for (j = 0; j < dk; ++j)
        for (i = 0; i < dv; ++i)
            S[(size_t)j * dv + i] += kt[j] * u[i];
    /* G4 */
    for (i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (j = 0; j < dk; ++j)
            acc += S[(size_t)j * dv + i] * qt[j];
        ot[i] = acc;
    }
}

int gdo_fwd(int B, int T, int H, int dk, int dv,
            const double *q, const double *k, const double *v,
            const double *alpha, const double *b, const double *w,
            const double *S0, double *o, double *ST)
{
    int bh, fail = 0;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return KDO_ERR_ARG;
    if (B * H == 0) return KDO_OK;
    if (T > 0 && (!q || !k || !v || !alpha || !b || !w || !o)) return KDO_ERR_ARG;

#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < B * H; ++bh) {
        int bb = bh / H, h = bh % H, t;
        size_t sz = (size_t)dk * dv;
        double *S = (double *)malloc((sz + (size_t)dv) * sizeof(double));
        if (!S) {
#pragma omp atomic write
            fail = 1;
            continue;
        }
        double *u = S + sz;
        if (S0) memcpy(S, S0 + (size_t)bh * sz, sz * sizeof(double));
        else memset(S, 0, sz * sizeof(double));
        for (t = 0; t < T; ++t) {
            size_t n = tok_index(bb, t, h, T, H);
            gdo_step(S, dk, dv, q + n * dk, k + n * dk, v + n * dv, alpha + n * dk,
                     b + n * dk, w + n * dv, u, o + n * dv);
        }
        if (ST) memcpy(ST + (size_t)bh * sz, S, sz * sizeof(double));
        free(S);
    }
    return fail ? KDO_ERR_MEM : KDO_OK;
}
