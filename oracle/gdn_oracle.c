/*
 * gdn_oracle.c -- token-serial CPU oracle of the gated delta rule, float64.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE LIBRARY.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load this code.
 * It shares no source, header, table or helper with the HIP library; the two
 * meet only in the seeded input generator.
 *
 * What it computes (gated-deltanet card, "Method"): for every (batch, head)
 * the state S [Dk x Dv] starts at h0 (zeros when absent, as new_state gives)
 * and each token t applies, in this order,
 *     S <- diag(exp(g_t)) S          decay; g_t is one value per key channel
 *                                    (GDN-2, Marin note "Background") or one
 *                                    scalar per head broadcast over channels
 *     m <- S^T k_t                   what the state already returns for k_t
 *     d <- beta_t (v_t - m)          delta scaled by the write gate
 *     S <- S + k_t d^T               rank-one write
 *     o_t <- scale * S^T q_t         read after the write (scale as passed in
 *                                    the atomic_ops card's API, d^-0.5 there)
 * and the final S is h_final.  Everything is float64; the inputs are the
 * exact float64 values of the device's float32 / bf16 bits.
 *
 * The backward pass is the exact adjoint of that loop, run token by token in
 * reverse.  The states it needs are recomputed segment by segment from
 * float64 checkpoints taken every CKPT tokens.
 *
 * Optional prologue (gated-deltanet card, "Usage": use_qk_l2norm, the in-kernel
 * L2 normalisation of queries and keys): every q_t and k_t row (Dk values of one
 * token and head) is replaced by x / sqrt(sum(x^2) + eps) before the loop; its
 * adjoint maps the gradient g_hat of the normalised row back to the raw row as
 * r (g_hat - x_hat (x_hat . g_hat)), r = 1 / sqrt(sum(x^2) + eps).  The pages
 * name the option but not eps; 1e-6 is this oracle's reading.
 *
 * Element type: `real`, float64 unless the file is compiled with
 * -DORACLE_REAL=float, which gives the float32 instantiation of the same code
 * (timed only, as a second CPU baseline; the float64 build is the reference).
 * <tgmath.h> makes exp and sqrt follow the element type.
 *
 * Layouts (row-major, contiguous):
 *   q, k [B,T,H,Dk]; v, o, dO [B,T,H,Dv]; beta [B,T,H];
 *   g [B,T,H,Dk] (per channel) or [B,T,H] (per head);
 *   h0, hT, dhT, dh0 [B,H,Dk,Dv].
 */
#include <stdlib.h>
#include <tgmath.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define CKPT 64

#ifndef ORACLE_REAL
#define ORACLE_REAL double
#endif
typedef ORACLE_REAL real;

typedef struct {
    int B, T, H, Dk, Dv, per_channel;
    real scale;
} dims;

static size_t tok(const dims *d, int b, int t, int h) { return ((size_t)b * d->T + t) * d->H + h; }

/* exp(g) for one token of one head into a[Dk] */
static void decay_factors(const dims *d, const real *g, int b, int t, int h, real *a)
{
    if (d->per_channel) {
        const real *gp = g + tok(d, b, t, h) * d->Dk;
        for (int i = 0; i < d->Dk; ++i) a[i] = exp(gp[i]);
    } else {
        real e = exp(g[tok(d, b, t, h)]);
        for (int i = 0; i < d->Dk; ++i) a[i] = e;
    }
}

/* One token of the recurrence on S in place.  Optionally returns m and d. */
static void step(const dims *d, real *S, const real *a, const real *kt, const real *vt,
                 real bt, real *m, real *dd)
{
    const int Dk = d->Dk, Dv = d->Dv;
    for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) S[i * Dv + j] *= a[i];
    for (int j = 0; j < Dv; ++j) {
        real s = 0.0;
        for (int i = 0; i < Dk; ++i) s += kt[i] * S[i * Dv + j];
        m[j] = s;
    }
    for (int j = 0; j < Dv; ++j) dd[j] = bt * (vt[j] - m[j]);
    for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) S[i * Dv + j] += kt[i] * dd[j];
}

static void read_out(const dims *d, const real *S, const real *qt, real *ot)
{
    for (int j = 0; j < d->Dv; ++j) {
        real s = 0.0;
        for (int i = 0; i < d->Dk; ++i) s += qt[i] * S[i * d->Dv + j];
        ot[j] = d->scale * s;
    }
}

static void head_forward(const dims *d, int b, int h, const real *q, const real *k,
                         const real *v, const real *g, const real *beta,
                         const real *h0, real *o, real *hT)
{
    const int Dk = d->Dk, Dv = d->Dv;
    real *S = calloc((size_t)Dk * Dv, sizeof(real));
    real *a = malloc(sizeof(real) * Dk), *m = malloc(sizeof(real) * Dv),
           *dd = malloc(sizeof(real) * Dv);
    const size_t sidx = ((size_t)b * d->H + h) * Dk * Dv;
    if (h0) memcpy(S, h0 + sidx, sizeof(real) * Dk * Dv);
    for (int t = 0; t < d->T; ++t) {
        const size_t r = tok(d, b, t, h);
        decay_factors(d, g, b, t, h, a);
        step(d, S, a, k + r * Dk, v + r * Dv, beta[r], m, dd);
        read_out(d, S, q + r * Dk, o + r * Dv);
    }
    if (hT) memcpy(hT + sidx, S, sizeof(real) * Dk * Dv);
    free(S); free(a); free(m); free(dd);
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Forward over all (b, h).  h0 and hT may be NULL.  Returns 0, or -1 on bad dims. */
int oracle_forward(int B, int T, int H, int Dk, int Dv, int per_channel, real scale,
                   const real *q, const real *k, const real *v, const real *g,
                   const real *beta, const real *h0, real *o, real *hT, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    dims d = {B, T, H, Dk, Dv, per_channel != 0, scale};
    set_threads(nthreads);
    const int n = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < n; ++bh)
        head_forward(&d, bh / H, bh % H, q, k, v, g, beta, h0, o, hT);
    return 0;
}

/* Reverse pass of one (b, h).  dhT may be NULL (zero); dh0 may be NULL. */
static void head_backward(const dims *d, int b, int h, const real *q, const real *k,
                          const real *v, const real *g, const real *beta,
                          const real *h0, const real *dO, const real *dhT, real *dq,
                          real *dk, real *dv, real *dg, real *dbeta, real *dh0)
{
    const int Dk = d->Dk, Dv = d->Dv, T = d->T;
    const size_t SS = (size_t)Dk * Dv;
    const size_t sidx = ((size_t)b * d->H + h) * SS;
    const int nseg = (T + CKPT - 1) / CKPT;
    /* ck[s] = state before token s*CKPT */
    real *ck = malloc(sizeof(real) * SS * (nseg > 0 ? nseg : 1));
    real *S = calloc(SS, sizeof(real));
    real *prev = malloc(sizeof(real) * SS * CKPT); /* S_{t-1} for each t of a segment */
    real *a = malloc(sizeof(real) * Dk), *m = malloc(sizeof(real) * Dv),
           *dd = malloc(sizeof(real) * Dv);
    real *dS = calloc(SS, sizeof(real)), *Sp = malloc(sizeof(real) * SS),
           *St = malloc(sizeof(real) * SS);
    real *ddv = malloc(sizeof(real) * Dv), *dm = malloc(sizeof(real) * Dv),
           *dgc = malloc(sizeof(real) * Dk);

    if (h0) memcpy(S, h0 + sidx, sizeof(real) * SS);
    for (int t = 0; t < T; ++t) {
        if (t % CKPT == 0) memcpy(ck + (size_t)(t / CKPT) * SS, S, sizeof(real) * SS);
        const size_t r = tok(d, b, t, h);
        decay_factors(d, g, b, t, h, a);
        step(d, S, a, k + r * Dk, v + r * Dv, beta[r], m, dd);
    }
    if (dhT) memcpy(dS, dhT + sidx, sizeof(real) * SS);

    for (int s = nseg - 1; s >= 0; --s) {
        const int t0 = s * CKPT, t1 = (t0 + CKPT < T) ? t0 + CKPT : T;
        memcpy(S, ck + (size_t)s * SS, sizeof(real) * SS);
        for (int t = t0; t < t1; ++t) {
            memcpy(prev + (size_t)(t - t0) * SS, S, sizeof(real) * SS);
            const size_t r = tok(d, b, t, h);
            decay_factors(d, g, b, t, h, a);
            step(d, S, a, k + r * Dk, v + r * Dv, beta[r], m, dd);
        }
        for (int t = t1 - 1; t >= t0; --t) {
            const size_t r = tok(d, b, t, h);
            const real *qt = q + r * Dk, *kt = k + r * Dk, *vt = v + r * Dv, *dot = dO + r * Dv;
            const real bt = beta[r];
            /* rebuild S'_t, m_t, d_t and S_t from S_{t-1} */
            decay_factors(d, g, b, t, h, a);
            const real *Sm1 = prev + (size_t)(t - t0) * SS;
            for (int i = 0; i < Dk; ++i)
                for (int j = 0; j < Dv; ++j) Sp[i * Dv + j] = a[i] * Sm1[i * Dv + j];
            memcpy(St, Sm1, sizeof(real) * SS);
            step(d, St, a, kt, vt, bt, m, dd);

            /* o_t = scale S_t^T q_t */
            for (int i = 0; i < Dk; ++i)
                for (int j = 0; j < Dv; ++j) dS[i * Dv + j] += d->scale * qt[i] * dot[j];
            for (int i = 0; i < Dk; ++i) {
                real s2 = 0.0;
                for (int j = 0; j < Dv; ++j) s2 += St[i * Dv + j] * dot[j];
                dq[r * Dk + i] = d->scale * s2;
            }
            /* S_t = S'_t + k_t d_t^T */
            for (int j = 0; j < Dv; ++j) {
                real s2 = 0.0;
                for (int i = 0; i < Dk; ++i) s2 += dS[i * Dv + j] * kt[i];
                ddv[j] = s2;
            }
            for (int i = 0; i < Dk; ++i) {
                real s2 = 0.0;
                for (int j = 0; j < Dv; ++j) s2 += dS[i * Dv + j] * dd[j];
                dk[r * Dk + i] = s2;
            }
            /* d_t = beta_t (v_t - m_t) */
            real db = 0.0;
            for (int j = 0; j < Dv; ++j) {
                dv[r * Dv + j] = bt * ddv[j];
                db += ddv[j] * (vt[j] - m[j]);
                dm[j] = -bt * ddv[j];
            }
            dbeta[r] = db;
            /* m_t = S'_t^T k_t: dS' = dS + k_t dm^T, dk_t += S'_t dm */
            for (int i = 0; i < Dk; ++i) {
                real s2 = 0.0;
                for (int j = 0; j < Dv; ++j) {
                    dS[i * Dv + j] += kt[i] * dm[j];
                    s2 += Sp[i * Dv + j] * dm[j];
                }
                dk[r * Dk + i] += s2;
            }
            /* S'_t = diag(exp g_t) S_{t-1}: dg_i = sum_j dS'_ij S'_ij; dS_{t-1} = a dS' */
            for (int i = 0; i < Dk; ++i) {
                real s2 = 0.0;
                for (int j = 0; j < Dv; ++j) s2 += dS[i * Dv + j] * Sp[i * Dv + j];
                dgc[i] = s2;
                for (int j = 0; j < Dv; ++j) dS[i * Dv + j] *= a[i];
            }
            if (d->per_channel) {
                for (int i = 0; i < Dk; ++i) dg[r * Dk + i] = dgc[i];
            } else {
                real s2 = 0.0;
                for (int i = 0; i < Dk; ++i) s2 += dgc[i];
                dg[r] = s2;
            }
        }
    }
    if (dh0) memcpy(dh0 + sidx, dS, sizeof(real) * SS);
    free(ck); free(S); free(prev); free(a); free(m); free(dd); free(dS); free(Sp); free(St);
    free(ddv); free(dm); free(dgc);
}

/* Gradients of sum(o * dO) + sum(hT * dhT) with respect to q, k, v, g, beta, h0. */
int oracle_backward(int B, int T, int H, int Dk, int Dv, int per_channel, real scale,
                    const real *q, const real *k, const real *v, const real *g,
                    const real *beta, const real *h0, const real *dO, const real *dhT,
                    real *dq, real *dk, real *dv, real *dg, real *dbeta, real *dh0,
                    int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    dims d = {B, T, H, Dk, Dv, per_channel != 0, scale};
    set_threads(nthreads);
    const int n = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < n; ++bh)
        head_backward(&d, bh / H, bh % H, q, k, v, g, beta, h0, dO, dhT, dq, dk, dv, dg, dbeta,
                      dh0);
    return 0;
}

/* x_hat = x / sqrt(sum(x^2) + eps), row by row over the last dimension D. */
int oracle_l2norm_forward(long rows, int D, real eps, const real *x, real *xhat)
{
    if (rows < 0 || D <= 0) return -1;
    for (long r = 0; r < rows; ++r) {
        real s = 0.0;
        for (int c = 0; c < D; ++c) s += x[r * D + c] * x[r * D + c];
        const real inv = 1.0 / sqrt(s + eps);
        for (int c = 0; c < D; ++c) xhat[r * D + c] = x[r * D + c] * inv;
    }
    return 0;
}

/* Adjoint of oracle_l2norm_forward: dx = r (dxhat - xhat (xhat . dxhat)). */
int oracle_l2norm_backward(long rows, int D, real eps, const real *x, const real *dxhat,
                           real *dx)
{
    if (rows < 0 || D <= 0) return -1;
    for (long r = 0; r < rows; ++r) {
        real s = 0.0;
        for (int c = 0; c < D; ++c) s += x[r * D + c] * x[r * D + c];
        const real inv = 1.0 / sqrt(s + eps);
        real dot = 0.0;
        for (int c = 0; c < D; ++c) dot += x[r * D + c] * inv * dxhat[r * D + c];
        for (int c = 0; c < D; ++c)
            dx[r * D + c] = inv * (dxhat[r * D + c] - x[r * D + c] * inv * dot);
    }
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
