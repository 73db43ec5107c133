/*
 * gdr_ref.c -- fp64 CPU oracle for the gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the bench's CPU
 * baseline may load this library.  It shares no code, header, table or helper
 * with the GPU library; the two never include or link each other.
 *
 * What it computes: the plain sequential recurrence, one token at a time, in
 * double precision, with no chunking and no reordering.  The state S of one
 * (batch, head) is a dk x dv matrix (row i = key channel, column j = value
 * channel), stored row-major, and the read-out is o_t = S_t^T q_t.  The pages
 * write the transposed state (dv x dk) with prediction S k; every formula
 * below is that formula transposed.
 *
 * Variants, each written in the form its page gives:
 *
 *  beta_mode 0 (scalar beta): gated delta rule.
 *     X = Diag(alpha_t) S_{t-1}              forget gate, scalar alpha (Gated
 *                                            DeltaNet) or one alpha per key
 *                                            channel (Kimi Delta Attention);
 *                                            [FG2-GDN page, section 1];
 *                                            [SDM page, Mecanismo Central, item 3]
 *     S_t = X + beta_t kw_t (v_t - X^T k_t)^T
 *        kw = k: the DeltaNet online-gradient step on 1/2 |S k - v|^2
 *                [OSDN page, section 1, update rule], gated.
 *        kw = d (.) k: the diagonally right-preconditioned step; the page shows
 *                that preconditioning the gradient equals scaling the write key
 *                [OSDN page, section 2.1, both update equations].  The gate is
 *                applied first, as for the other backbones the page uses.
 *
 *  beta_mode 1 (one beta vector in R^dk, needs dk == dv) and
 *  beta_mode 2 (separate beta^k in R^dk and beta^v in R^dv):
 *     kt = sqrt(beta^k) (.) k,  vt = sqrt(beta^v) (.) v   (beta^v = beta^k in mode 1)
 *     S_t = (I - kt kt^T) Diag(alpha_t) S_{t-1} + kt vt^T
 *        [FG2-GDN page, section 2.A, absorption and state update;
 *         section 2.B, separate erase and write strengths].
 *     When a separate write key kw is given, the left factor kt becomes
 *     wt = sqrt(beta^k) (.) kw in both places (same rank-1 structure).
 *
 * Inputs are fp64 arrays holding the exact values the GPU path receives
 * (bf16 or fp32 upcast), in the layouts
 *     q, k, kw: [B, T, H, dk]   v: [B, T, H, dv]
 *     alpha: [B, T, H] (mode 0) or [B, T, H, dk] (mode 1)
 *     beta_k: [B, T, H] (beta mode 0) or [B, T, H, dk] (modes 1, 2)
 *     beta_v: [B, T, H, dv] (beta mode 2 only)
 *     S0, ST: [B, H, dk, dv];   o: [B, T, H, dv]
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define REF_OK 0
#define REF_EINVAL (-1)

/* One recurrence step on the state of one (batch, head).
 * a: alpha (1 or dk values), bk: beta^k (1 or dk values), bv: beta^v (dv values or NULL). */
static void ref_step(int dk, int dv, double *S, const double *a, int channel_alpha,
                     int beta_mode, const double *bk, const double *bv,
                     const double *k, const double *kw, const double *v,
                     double *scratch /* >= 2*dk + 2*dv */)
{
    int i, j;
    /* forget gate */
    for (i = 0; i < dk; ++i) {
        const double ai = channel_alpha ? a[i] : a[0];
        for (j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] *= ai;
    }
    if (beta_mode == 0) {
        /* prediction of v from the decayed state, then the rank-1 correction */
        double *pred = scratch;
        const double b = bk[0];
        for (j = 0; j < dv; ++j) {
            double s = 0.0;
            for (i = 0; i < dk; ++i)
                s += S[(size_t)i * dv + j] * k[i];
            pred[j] = s;
        }
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] += b * kw[i] * (v[j] - pred[j]);
    } else {
        /* (I - wt kt^T) X + wt vt^T with kt = sqrt(beta^k) k, wt = sqrt(beta^k) kw,
         * vt = sqrt(beta^v) v */
        double *kt = scratch, *wt = scratch + dk, *vt = scratch + 2 * dk, *r = vt + dv;
        const double *bvv = (beta_mode == 1) ? bk : bv;
        for (i = 0; i < dk; ++i) {
            kt[i] = sqrt(bk[i]) * k[i];
            wt[i] = sqrt(bk[i]) * kw[i];
        }
        for (j = 0; j < dv; ++j)
            vt[j] = sqrt(bvv[j]) * v[j];
        for (j = 0; j < dv; ++j) { /* r = kt^T X */
            double s = 0.0;
            for (i = 0; i < dk; ++i)
                s += kt[i] * S[(size_t)i * dv + j];
            r[j] = s;
        }
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] += wt[i] * (vt[j] - r[j]);
    }
}

/* o = S^T q */
static void ref_readout(int dk, int dv, const double *S, const double *q, double *o)
{
    int i, j;
    for (j = 0; j < dv; ++j) {
        double s = 0.0;
        for (i = 0; i < dk; ++i)
            s += S[(size_t)i * dv + j] * q[i];
        o[j] = s;
    }
}

static int ref_check(int B, int T, int H, int dk, int dv, int alpha_mode, int beta_mode)
{
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1) return REF_EINVAL;
    if (alpha_mode != 0 && alpha_mode != 1) return REF_EINVAL;
    if (beta_mode < 0 || beta_mode > 2) return REF_EINVAL;
    if (beta_mode == 1 && dk != dv) return REF_EINVAL;
    return REF_OK;
}

/*
 * Sequential forward over T tokens for the (batch, head) pairs listed in
 * `heads` (indices b*H + h), or all of them when heads == NULL.  o rows and
 * ST blocks of unlisted pairs are left untouched.  S0 == NULL starts from the
 * zero state; ST == NULL skips the final-state store.  nthreads <= 0 uses the
 * OpenMP default.
 */
int gdr_ref_forward(int B, int T, int H, int dk, int dv, int alpha_mode, int beta_mode,
                    const double *q, const double *k, const double *kw, const double *v,
                    const double *alpha, const double *beta_k, const double *beta_v,
                    const double *S0, double *o, double *ST,
                    const int *heads, int n_heads, int nthreads)
{
    int rc = ref_check(B, T, H, dk, dv, alpha_mode, beta_mode);
    if (rc) return rc;
    if (beta_mode == 2 && !beta_v) return REF_EINVAL;
    if (!q || !k || !v || !alpha || !beta_k || !o) return REF_EINVAL;
    const int total = heads ? n_heads : B * H;
    const size_t sdim = (size_t)dk * dv;
    const int a_n = alpha_mode ? dk : 1;
    const int b_n = beta_mode ? dk : 1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int idx = 0; idx < total; ++idx) {
        const int bh = heads ? heads[idx] : idx;
        if (bh < 0 || bh >= B * H) { failed = 1; continue; }
        const int b = bh / H, h = bh % H;
        double *S = (double *)malloc(sizeof(double) * (sdim + 2 * (size_t)dk + 2 * (size_t)dv));
        if (!S) { failed = 1; continue; }
        double *scratch = S + sdim;
        if (S0) memcpy(S, S0 + (size_t)bh * sdim, sizeof(double) * sdim);
        else memset(S, 0, sizeof(double) * sdim);
        for (int t = 0; t < T; ++t) {
            const size_t tok = ((size_t)b * T + t) * H + h;
            const double *kt = k + tok * dk;
            ref_step(dk, dv, S, alpha + tok * a_n, alpha_mode, beta_mode, beta_k + tok * b_n,
                     beta_mode == 2 ? beta_v + tok * dv : NULL, kt, kw ? kw + tok * dk : kt,
                     v + tok * dv, scratch);
            ref_readout(dk, dv, S, q + tok * dk, o + tok * dv);
        }
        if (ST) memcpy(ST + (size_t)bh * sdim, S, sizeof(double) * sdim);
        free(S);
    }
    return failed ? REF_EINVAL : REF_OK;
}

/*
 * One decode step for every (batch, head): the same recurrence step applied
 * to a caller-held state S [B, H, dk, dv] (updated in place), followed by the
 * read-out o [B, H, dv].  Per-token inputs have the prefill layouts with T
 * removed: q, k, kw [B, H, dk], v [B, H, dv], alpha [B, H] or [B, H, dk], ...
 */
int gdr_ref_decode_step_f64(int B, int H, int dk, int dv, int alpha_mode, int beta_mode,
                            const double *q, const double *k, const double *kw, const double *v,
                            const double *alpha, const double *beta_k, const double *beta_v,
                            double *S, double *o, int nthreads)
{
    int rc = ref_check(B, 1, H, dk, dv, alpha_mode, beta_mode);
    if (rc) return rc;
    if (beta_mode == 2 && !beta_v) return REF_EINVAL;
    if (!q || !k || !v || !alpha || !beta_k || !S || !o) return REF_EINVAL;
    const size_t sdim = (size_t)dk * dv;
    const int a_n = alpha_mode ? dk : 1;
    const int b_n = beta_mode ? dk : 1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int bh = 0; bh < B * H; ++bh) {
        double scratch[4 * 1024];
        if (2 * dk + 2 * dv > 4 * 1024) { failed = 1; continue; }
        const double *kt = k + (size_t)bh * dk;
        ref_step(dk, dv, S + (size_t)bh * sdim, alpha + (size_t)bh * a_n, alpha_mode, beta_mode,
                 beta_k + (size_t)bh * b_n, beta_mode == 2 ? beta_v + (size_t)bh * dv : NULL, kt,
                 kw ? kw + (size_t)bh * dk : kt, v + (size_t)bh * dv, scratch);
        ref_readout(dk, dv, S + (size_t)bh * sdim, q + (size_t)bh * dk, o + (size_t)bh * dv);
    }
    return failed ? REF_EINVAL : REF_OK;
}

/*
 * delta-mem step, in the page's own form and orientation [delta-mem page,
 * section 2.A update rule; section 2.C read]: the memory M (dv x dk, stored
 * [B, H, dv, dk] row-major) predicts a value from a key as M k.  With forget
 * gate lambda and write gate beta (one each per (batch, head)):
 *     r_t = M_{t-1} q_t                                   read, before the write
 *     M_t = lambda_t M_{t-1} + beta_t (v_t - M_{t-1} k_t) k_t^T
 * The prediction M_{t-1} k_t uses the state before the forget gate.  M is
 * updated in place; r is [B, H, dv].
 */
int gdr_ref_dmem_step(int B, int H, int dk, int dv, const double *q, const double *k, const double *v,
                      const double *lam, const double *beta, double *M, double *r, int nthreads)
{
    if (B < 0 || H < 0 || dk < 1 || dv < 1) return REF_EINVAL;
    if (!q || !k || !v || !lam || !beta || !M || !r) return REF_EINVAL;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int bh = 0; bh < B * H; ++bh) {
        double pred[1024];
        if (dv > 1024) { failed = 1; continue; }
        double *Mh = M + (size_t)bh * dv * dk;
        const double *qh = q + (size_t)bh * dk, *kh = k + (size_t)bh * dk, *vh = v + (size_t)bh * dv;
        for (int a = 0; a < dv; ++a) {            /* read and prediction from M_{t-1} */
            double sr = 0.0, sp = 0.0;
            for (int c = 0; c < dk; ++c) {
                sr += Mh[(size_t)a * dk + c] * qh[c];
                sp += Mh[(size_t)a * dk + c] * kh[c];
            }
            r[(size_t)bh * dv + a] = sr;
            pred[a] = sp;
        }
        for (int a = 0; a < dv; ++a)              /* M_t = lambda M + beta (v - M k) k^T */
            for (int c = 0; c < dk; ++c)
                Mh[(size_t)a * dk + c] = lam[bh] * Mh[(size_t)a * dk + c] + beta[bh] * (vh[a] - pred[a]) * kh[c];
    }
    return failed ? REF_EINVAL : REF_OK;
}

/*
 * OSDN phase 1: the scan over the key stream that produces the preconditioned
 * write keys of phase 2 [OSDN page, section 2.2 (hypergradient feedback, the
 * closed-form surrogate, the two phases) and section 2.3 (retention gate of the
 * preconditioner, APF)].  For one (batch, head), with d the diagonal
 * preconditioner (d_0 given, all ones when NULL) and, per token t,
 *     kw_t = d_t (.) k_t                            write key used at token t
 *     h_t(d) = ((1 - beta_t <d, k_t^2>)^2 - 1) / (2 |k_t|^2)   surrogate
 *     grad_t = dh_t/dd at d_t = -beta_t (1 - beta_t <d_t, k_t^2>) k_t^2 / |k_t|^2
 *     d_{t+1} = r_t d_t - eta grad_t                online gradient descent on
 *                                                   h_t, retention r_t (1 = OSDN)
 * (the page prints the APF step with "+ eta grad"; it is read as the descent
 * step of the online gradient method the section names).  A zero key has no
 * gradient (0/0 in the formula): d is only multiplied by r_t then.
 * The per-token loss ratio f_t(S_t) / f_t(S_{t-1}) of phase 2 is
 * (1 - beta_t <d_t, k_t^2>)^2 (the residual along k_t shrinks by that factor
 * in one step [OSDN page, section 2.2 surrogate; section 4.2 q_geo]); q_geo is
 * its geometric mean over the T tokens, exp(mean_t log ratio_t).
 * Layouts: k, kw [B, T, H, dk]; beta, r [B, T, H] (r may be NULL: all ones);
 * d0, dT [B, H, dk] (d0 may be NULL: ones; dT may be NULL); qgeo [B, H] (may
 * be NULL; 1 when T == 0).
 */
int gdr_ref_osdn_precond(int B, int T, int H, int dk, const double *k, const double *beta, const double *r,
                         double eta, const double *d0, double *kw, double *dT, double *qgeo, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dk > 1024) return REF_EINVAL;
    if (!k || !beta || !kw) return REF_EINVAL;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        double d[1024];
        for (int i = 0; i < dk; ++i) d[i] = d0 ? d0[(size_t)bh * dk + i] : 1.0;
        double logsum = 0.0;
        for (int t = 0; t < T; ++t) {
            const size_t tok = ((size_t)b * T + t) * H + h;
            const double *kt = k + tok * dk;
            const double bt = beta[tok], rt = r ? r[tok] : 1.0;
            double nk = 0.0, s = 0.0;
            for (int i = 0; i < dk; ++i) {
                nk += kt[i] * kt[i];
                s += d[i] * kt[i] * kt[i];
                kw[tok * dk + i] = d[i] * kt[i];
            }
            const double u = 1.0 - bt * s;          /* residual factor of this step */
            logsum += log(u * u);
            for (int i = 0; i < dk; ++i) {
                const double grad = nk > 0.0 ? -bt * u * kt[i] * kt[i] / nk : 0.0;
                d[i] = rt * d[i] - eta * grad;
            }
        }
        if (dT)
            for (int i = 0; i < dk; ++i) dT[(size_t)bh * dk + i] = d[i];
        if (qgeo) qgeo[bh] = T > 0 ? exp(logsum / T) : 1.0;
    }
    return REF_OK;
}

/*
 * Mirrors of the GPU library's two entry points, with its argument list: a
 * descriptor laid out field for field like the library's (declared here, not
 * shared), HOST pointers to inputs in their stored dtypes (dtype 0: bf16 bit
 * patterns, 1: fp32), the fp64 recurrence above inside, o written in the io
 * dtype and the states in fp32 -- each output rounded the way the input generator
 * stores values (fp64 -> fp32 round-to-nearest-even -> bf16 round-to-nearest-even).
 * The chunk size, workspace and stream are accepted and not used (the recurrence is
 * sequential); flags must be 0.  S0 == NULL starts from 0, ST == NULL skips it;
 * S0 == ST is allowed.
 */
typedef struct {
    int B, T, H, dk, dv, chunk, io_dtype, gate_dtype, alpha_mode, beta_mode, flags;
} gdr_ref_desc;

static double ref_ld(const void *p, size_t i, int dtype)
{
    if (dtype == 0) {
        const unsigned int u = (unsigned int)((const unsigned short *)p)[i] << 16;
        float f;
        memcpy(&f, &u, 4);
        return f;
    }
    return ((const float *)p)[i];
}

static void ref_st(void *p, size_t i, double x, int dtype)
{
    const float f = (float)x;
    if (dtype != 0) {
        ((float *)p)[i] = f;
        return;
    }
    unsigned int u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) u = 0x7fc00000u;   /* NaN */
    else u += 0x7fffu + ((u >> 16) & 1u);                   /* nearest, ties to even */
    ((unsigned short *)p)[i] = (unsigned short)(u >> 16);
}

/* fp64 copy of n stored values (NULL in, NULL out); *bad set on allocation failure */
static double *ref_up(const void *p, size_t n, int dtype, int *bad)
{
    if (!p) return NULL;
    double *x = (double *)malloc(sizeof(double) * (n ? n : 1));
    if (!x) { *bad = 1; return NULL; }
    for (size_t i = 0; i < n; ++i) x[i] = ref_ld(p, i, dtype);
    return x;
}

static int ref_desc_ok(const gdr_ref_desc *d)
{
    if (!d || d->flags != 0) return 0;
    if ((d->io_dtype != 0 && d->io_dtype != 1) || (d->gate_dtype != 0 && d->gate_dtype != 1)) return 0;
    return ref_check(d->B, d->T < 0 ? -1 : (d->T ? d->T : 1), d->H, d->dk, d->dv, d->alpha_mode, d->beta_mode) == REF_OK;
}

int gdr_ref_chunk_fwd(const gdr_ref_desc *d, const void *q, const void *k, const void *k_w, const void *v,
                      const void *alpha, const void *beta_k, const void *beta_v, const float *S0, void *o,
                      float *ST, void *workspace, size_t workspace_bytes, void *stream)
{
    (void)workspace; (void)workspace_bytes; (void)stream;
    if (!ref_desc_ok(d)) return REF_EINVAL;
    const size_t ntok = (size_t)d->B * d->T * d->H, nbh = (size_t)d->B * d->H, sd = (size_t)d->dk * d->dv;
    if (ntok && (!q || !k || !v || !alpha || !beta_k || !o)) return REF_EINVAL;
    if (d->beta_mode == 2 && ntok && !beta_v) return REF_EINVAL;
    int bad = 0;
    const int io = d->io_dtype, gt = d->gate_dtype;
    double *q8 = ref_up(q, ntok * d->dk, io, &bad), *k8 = ref_up(k, ntok * d->dk, io, &bad);
    double *w8 = ref_up(k_w, ntok * d->dk, io, &bad), *v8 = ref_up(v, ntok * d->dv, io, &bad);
    double *a8 = ref_up(alpha, ntok * (d->alpha_mode ? d->dk : 1), gt, &bad);
    double *bk8 = ref_up(beta_k, ntok * (d->beta_mode ? d->dk : 1), gt, &bad);
    double *bv8 = ref_up(d->beta_mode == 2 ? beta_v : NULL, ntok * d->dv, gt, &bad);
    double *s08 = ref_up(S0, nbh * sd, 1, &bad);
    double *o8 = (double *)malloc(sizeof(double) * (ntok * d->dv ? ntok * d->dv : 1));
    double *st8 = (double *)malloc(sizeof(double) * (nbh * sd ? nbh * sd : 1));
    int rc = REF_EINVAL;
    if (!bad && o8 && st8) {
        if (ntok == 0) {  /* no token: S_T = S0 */
            for (size_t i = 0; i < nbh * sd; ++i) st8[i] = s08 ? s08[i] : 0.0;
            rc = REF_OK;
        } else {
            rc = gdr_ref_forward(d->B, d->T, d->H, d->dk, d->dv, d->alpha_mode, d->beta_mode, q8, k8, w8, v8, a8,
                                 bk8, bv8, s08, o8, st8, NULL, 0, 0);
        }
        if (rc == REF_OK) {
            for (size_t i = 0; i < ntok * d->dv; ++i) ref_st(o, i, o8[i], io);
            if (ST)
                for (size_t i = 0; i < nbh * sd; ++i) ST[i] = (float)st8[i];
        }
    }
    free(q8); free(k8); free(w8); free(v8); free(a8); free(bk8); free(bv8); free(s08); free(o8); free(st8);
    return rc;
}

int gdr_ref_decode_step(const gdr_ref_desc *d, const void *q, const void *k, const void *k_w, const void *v,
                        const void *alpha, const void *beta_k, const void *beta_v, float *S, void *o, void *stream)
{
    (void)stream;
    if (!ref_desc_ok(d)) return REF_EINVAL;
    const size_t nbh = (size_t)d->B * d->H, sd = (size_t)d->dk * d->dv;
    if (nbh == 0) return REF_OK;
    if (!q || !k || !v || !alpha || !beta_k || !S || !o) return REF_EINVAL;
    if (d->beta_mode == 2 && !beta_v) return REF_EINVAL;
    int bad = 0;
    const int io = d->io_dtype, gt = d->gate_dtype;
    double *q8 = ref_up(q, nbh * d->dk, io, &bad), *k8 = ref_up(k, nbh * d->dk, io, &bad);
    double *w8 = ref_up(k_w, nbh * d->dk, io, &bad), *v8 = ref_up(v, nbh * d->dv, io, &bad);
    double *a8 = ref_up(alpha, nbh * (d->alpha_mode ? d->dk : 1), gt, &bad);
    double *bk8 = ref_up(beta_k, nbh * (d->beta_mode ? d->dk : 1), gt, &bad);
    double *bv8 = ref_up(d->beta_mode == 2 ? beta_v : NULL, nbh * d->dv, gt, &bad);
    double *s8 = ref_up(S, nbh * sd, 1, &bad);
    double *o8 = (double *)malloc(sizeof(double) * nbh * d->dv);
    int rc = REF_EINVAL;
    if (!bad && o8) {
        rc = gdr_ref_decode_step_f64(d->B, d->H, d->dk, d->dv, d->alpha_mode, d->beta_mode, q8, k8, w8, v8, a8, bk8,
                                     bv8, s8, o8, 0);
        if (rc == REF_OK) {
            for (size_t i = 0; i < nbh * d->dv; ++i) ref_st(o, i, o8[i], io);
            for (size_t i = 0; i < nbh * sd; ++i) S[i] = (float)s8[i];
        }
    }
    free(q8); free(k8); free(w8); free(v8); free(a8); free(bk8); free(bv8); free(s8); free(o8);
    return rc;
}

int gdr_ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
