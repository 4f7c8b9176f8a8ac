/*
 * gdr2_oracle.c -- plain fp64 CPU oracle for the Gated Delta Rule-2 (GDR-2) layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct reference that the
 * HIP kernels are checked against.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the product library never does.  It shares no code,
 * header, table or constant with the HIP path.
 *
 * What it computes (all in double precision, one token at a time, per (batch, head) chain):
 *
 *   Gated Delta Rule-2 update, as printed in the forum summary "Gated DeltaNet-2: Decoupling
 *   Erase and Write Gates in Linear Attention for Better Memory Editing" (zhichai.net, English),
 *   section "Gated Delta Rule-2", update rule:
 *       S_t = (I - k_t (b_t . k_t)^T) D_t S_{t-1} + k_t (w_t . v_t)^T ,   D_t = Diag(alpha_t)
 *   The ainews.random.gg article on NVIDIA's Gated DeltaNet-2, section "Gated Delta Rule-2: two
 *   gates instead of one", states the order used below: the channel-wise decay is applied first,
 *   then the erase reads the decayed state through e_t = b_t . k_t, and the write adds
 *   k_t z_t^T with z_t = w_t . v_t.  Expanding the product gives the form coded here:
 *       Sbar = Diag(alpha_t) S_{t-1};  r = Sbar^T e_t;  S_t = Sbar + k_t (z_t - r)^T.
 *   Read-out: the state "is read with the query" (same article, section "The scalar gate problem
 *   in delta-rule models"); reading: o_t = S_t^T q_t with the post-update state, no query scale.
 *   Decay input: natural log of alpha, one value per key channel (alpha in (0,1]).
 *
 *   Layouts (row-major):  q, k, log_alpha, b : [B][T][H][dk];   v, w, o, dO : [B][T][H][dv];
 *                          S0, ST, dST, dS0 : [B][H][dk][dv].
 *   NULL S0 / dST mean zero; NULL ST / dS0 mean "not wanted".
 *
 * The backward is reverse-mode differentiation of the token recurrence, derived by hand from
 * the four-step forward above (see the comments in gdr2o_backward).  It checkpoints the state
 * every CKPT tokens and recomputes inside each segment.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define CKPT 64

static long idx_tok(long b, long t, long h, long T, long H, long d) {
    return ((b * T + t) * H + h) * d;
}

/* One forward token step on one chain.
 *   S (in/out) [dk][dv]; optional Sbar_out [dk][dv] and r_out [dv] receive the intermediates. */
static void token_step(long dk, long dv, const double* q, const double* k, const double* v,
                       const double* la, const double* b, const double* w, double* S,
                       double* o, double* Sbar_out, double* r_out) {
    double* r = (double*)malloc(sizeof(double) * (size_t)dv);
    /* decay first: Sbar = Diag(alpha) S */
    for (long i = 0; i < dk; ++i) {
        double a = exp(la[i]);
        for (long j = 0; j < dv; ++j) S[i * dv + j] *= a;
    }
    if (Sbar_out) memcpy(Sbar_out, S, sizeof(double) * (size_t)(dk * dv));
    /* gated read of the decayed state: r = Sbar^T (b . k) */
    for (long j = 0; j < dv; ++j) r[j] = 0.0;
    for (long i = 0; i < dk; ++i) {
        double e = b[i] * k[i];
        for (long j = 0; j < dv; ++j) r[j] += S[i * dv + j] * e;
    }
    if (r_out) memcpy(r_out, r, sizeof(double) * (size_t)dv);
    /* erase + gated write along the key direction: S = Sbar + k (w . v - r)^T */
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j) S[i * dv + j] += k[i] * (w[j] * v[j] - r[j]);
    /* read-out with the query on the updated state: o = S^T q */
    if (o) {
        for (long j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * q[i];
            o[j] = acc;
        }
    }
    free(r);
}

void gdr2o_forward(long B, long T, long H, long dk, long dv, const double* q, const double* k,
                   const double* v, const double* la, const double* b, const double* w,
                   const double* S0, double* o, double* ST) {
    long nchain = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long c = 0; c < nchain; ++c) {
        long bb = c / H, h = c % H;
        double* S = (double*)calloc((size_t)(dk * dv), sizeof(double));
        if (S0) memcpy(S, S0 + c * dk * dv, sizeof(double) * (size_t)(dk * dv));
        for (long t = 0; t < T; ++t) {
            long ik = idx_tok(bb, t, h, T, H, dk), iv = idx_tok(bb, t, h, T, H, dv);
            token_step(dk, dv, q + ik, k + ik, v + iv, la + ik, b + ik, w + iv, S, o + iv, NULL,
                       NULL);
        }
        if (ST) memcpy(ST + c * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
        free(S);
    }
}

/* Reverse mode of the token recurrence.
 * Per token, going backwards with G = dL/dS_t (from later tokens plus dST):
 *   o = S_t^T q            ->  dq = S_t do;            Ghat = G + q do^T
 *   S_t = Sbar + k u^T     ->  dSbar = Ghat; dk += Ghat u; rho = Ghat^T k    (u = z - r)
 *   u = z - r              ->  dz = rho;  dr = -rho
 *   r = Sbar^T e           ->  dSbar += e dr^T = -e rho^T;   de = Sbar dr = -Sbar rho
 *   z = w . v              ->  dv = w . rho;   dw = v . rho
 *   e = b . k              ->  db = k . de;    dk += b . de
 *   Sbar = Diag(a) S_{t-1} ->  dS_{t-1} = Diag(a) dSbar;  dlog a_i = sum_j dSbar_ij Sbar_ij
 */
void gdr2o_backward(long B, long T, long H, long dk, long dv, const double* q, const double* k,
                    const double* v, const double* la, const double* b, const double* w,
                    const double* S0, const double* dO, const double* dST, double* dq,
                    double* dkk, double* dvv, double* dla, double* db, double* dw, double* dS0) {
    long nchain = B * H;
    long nseg = (T + CKPT - 1) / CKPT;
    size_t SS = (size_t)(dk * dv);
#pragma omp parallel for schedule(dynamic, 1)
    for (long c = 0; c < nchain; ++c) {
        long bb = c / H, h = c % H;
        double* ck = (double*)calloc((size_t)(nseg > 0 ? nseg : 1) * SS, sizeof(double));
        double* S = (double*)calloc(SS, sizeof(double));
        double* segS = (double*)malloc(sizeof(double) * SS * (CKPT + 1)); /* S_{t-1}, then S_t */
        double* segSbar = (double*)malloc(sizeof(double) * SS * CKPT);
        double* segR = (double*)malloc(sizeof(double) * (size_t)dv * CKPT);
        double* G = (double*)calloc(SS, sizeof(double));
        double* Gh = (double*)malloc(sizeof(double) * SS);
        double* rho = (double*)malloc(sizeof(double) * (size_t)dv);
        double* de = (double*)malloc(sizeof(double) * (size_t)dk);
        if (S0) memcpy(S, S0 + c * SS, sizeof(double) * SS);
        /* forward sweep storing the state at the start of every segment */
        for (long t = 0; t < T; ++t) {
            if (t % CKPT == 0) memcpy(ck + (t / CKPT) * SS, S, sizeof(double) * SS);
            long ik = idx_tok(bb, t, h, T, H, dk), iv = idx_tok(bb, t, h, T, H, dv);
            token_step(dk, dv, q + ik, k + ik, v + iv, la + ik, b + ik, w + iv, S, NULL, NULL,
                       NULL);
        }
        if (dST) memcpy(G, dST + c * SS, sizeof(double) * SS);
        for (long sg = nseg - 1; sg >= 0; --sg) {
            long t0 = sg * CKPT, t1 = t0 + CKPT < T ? t0 + CKPT : T;
            /* recompute the segment: segS[n] = state before token t0+n, segS[n+1] after */
            memcpy(segS, ck + sg * SS, sizeof(double) * SS);
            for (long t = t0; t < t1; ++t) {
                long n = t - t0;
                long ik = idx_tok(bb, t, h, T, H, dk), iv = idx_tok(bb, t, h, T, H, dv);
                memcpy(segS + (n + 1) * SS, segS + n * SS, sizeof(double) * SS);
                token_step(dk, dv, q + ik, k + ik, v + iv, la + ik, b + ik, w + iv,
                           segS + (n + 1) * SS, NULL, segSbar + n * SS, segR + n * dv);
            }
            for (long t = t1 - 1; t >= t0; --t) {
                long n = t - t0;
                long ik = idx_tok(bb, t, h, T, H, dk), iv = idx_tok(bb, t, h, T, H, dv);
                const double *qt = q + ik, *kt = k + ik, *vt = v + iv, *lat = la + ik;
                const double *bt = b + ik, *wt = w + iv, *dot = dO + iv;
                const double* St = segS + (n + 1) * SS;
                const double* Sb = segSbar + n * SS;
                const double* r = segR + n * dv;
                /* read-out */
                for (long i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (long j = 0; j < dv; ++j) acc += St[i * dv + j] * dot[j];
                    dq[ik + i] = acc;
                }
                for (long i = 0; i < dk; ++i)
                    for (long j = 0; j < dv; ++j) Gh[i * dv + j] = G[i * dv + j] + qt[i] * dot[j];
                /* write / erase outer product */
                for (long j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (long i = 0; i < dk; ++i) acc += Gh[i * dv + j] * kt[i];
                    rho[j] = acc;
                }
                for (long i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (long j = 0; j < dv; ++j) acc += Gh[i * dv + j] * (wt[j] * vt[j] - r[j]);
                    dkk[ik + i] = acc;
                }
                for (long j = 0; j < dv; ++j) {
                    dvv[iv + j] = wt[j] * rho[j];
                    dw[iv + j] = vt[j] * rho[j];
                }
                for (long i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (long j = 0; j < dv; ++j) acc += Sb[i * dv + j] * rho[j];
                    de[i] = -acc;
                }
                for (long i = 0; i < dk; ++i) {
                    db[ik + i] = kt[i] * de[i];
                    dkk[ik + i] += bt[i] * de[i];
                }
                /* dSbar = Ghat - e rho^T, then through the decay */
                for (long i = 0; i < dk; ++i) {
                    double e = bt[i] * kt[i];
                    double a = exp(lat[i]);
                    double acc = 0.0;
                    for (long j = 0; j < dv; ++j) {
                        double g = Gh[i * dv + j] - e * rho[j];
                        acc += g * Sb[i * dv + j];
                        G[i * dv + j] = a * g;
                    }
                    dla[ik + i] = acc;
                }
            }
        }
        if (dS0) memcpy(dS0 + c * SS, G, sizeof(double) * SS);
        free(ck); free(S); free(segS); free(segSbar); free(segR); free(G); free(Gh); free(rho);
        free(de);
    }
}

/* One recurrent decode step for N independent sequences x H heads: exactly one token of the
 * update above.  q,k,la,b: [N][H][dk]; v,w,o: [N][H][dv]; S_in (NULL = 0), S_out: [N][H][dk][dv].
 * S_in may equal S_out. */
void gdr2o_decode_step(long N, long H, long dk, long dv, const double* q, const double* k,
                       const double* v, const double* la, const double* b, const double* w,
                       const double* S_in, double* S_out, double* o) {
    long nchain = N * H;
    size_t SS = (size_t)(dk * dv);
#pragma omp parallel for schedule(static)
    for (long c = 0; c < nchain; ++c) {
        double* S = S_out + c * SS;
        if (S_in == NULL)
            memset(S, 0, sizeof(double) * SS);
        else if (S_in != S_out)
            memcpy(S, S_in + c * SS, sizeof(double) * SS);
        token_step(dk, dv, q + c * dk, k + c * dk, v + c * dv, la + c * dk, b + c * dk,
                   w + c * dv, S, o + c * dv, NULL, NULL);
    }
}

/* Reduced rule, Kimi Delta Attention (KDA): the forum summary's section "Gated Delta Rule-2"
 * says GDR-2 with b_t = w_t = beta_t * 1 is KDA, whose update (written in its own form, with one
 * scalar edit strength per token and head) is
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t.
 * With scalar_decay != 0 only la[..][0] is read per token and head: alpha_t is one number,
 * which is Gated DeltaNet.  beta: [B][T][H].  Computed as explicit matrix products (the
 * transition matrix is formed), independently of token_step. */
void gdr2o_kda_forward(long B, long T, long H, long dk, long dv, int scalar_decay,
                       const double* q, const double* k, const double* v, const double* la,
                       const double* beta, const double* S0, double* o, double* ST) {
    long nchain = B * H;
    size_t SS = (size_t)(dk * dv);
#pragma omp parallel for schedule(dynamic, 1)
    for (long c = 0; c < nchain; ++c) {
        long bb = c / H, h = c % H;
        double* S = (double*)calloc(SS, sizeof(double));
        double* Sn = (double*)malloc(sizeof(double) * SS);
        double* M = (double*)malloc(sizeof(double) * (size_t)(dk * dk));
        if (S0) memcpy(S, S0 + c * SS, sizeof(double) * SS);
        for (long t = 0; t < T; ++t) {
            long ik = idx_tok(bb, t, h, T, H, dk), iv = idx_tok(bb, t, h, T, H, dv);
            double bt = beta[(bb * T + t) * H + h];
            /* M = (I - beta k k^T) Diag(alpha) */
            for (long i = 0; i < dk; ++i)
                for (long l = 0; l < dk; ++l) {
                    double al = exp(scalar_decay ? la[ik] : la[ik + l]);
                    M[i * dk + l] = ((i == l ? 1.0 : 0.0) - bt * k[ik + i] * k[ik + l]) * al;
                }
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j) {
                    double acc = bt * k[ik + i] * v[iv + j];
                    for (long l = 0; l < dk; ++l) acc += M[i * dk + l] * S[l * dv + j];
                    Sn[i * dv + j] = acc;
                }
            memcpy(S, Sn, sizeof(double) * SS);
            for (long j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * q[ik + i];
                o[iv + j] = acc;
            }
        }
        if (ST) memcpy(ST + c * SS, S, sizeof(double) * SS);
        free(S); free(Sn); free(M);
    }
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Threads the OpenMP loops above use (1 without OpenMP). */
int gdr2o_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
