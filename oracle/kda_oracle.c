/*
 * kda_oracle.c -- fp64 CPU oracle for the Kimi Delta Attention (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg load it.  It shares no
 * code, header, table or helper with the GPU library (gated_delta_rule_81_amd/),
 * and the GPU library never calls it.
 *
 * What it computes.  One fixed-size state matrix S per (sequence, head), of
 * shape d_k x d_v (key dimension by value dimension: "The fourth layer
 * remembers", section "What each kind of layer keeps").  For every token t,
 * in sequence order:
 *
 *   1. forget, per key channel:  S <- Diag(alpha_t) S,  alpha_t = exp(log_alpha_t)
 *        (one decay rate per key channel instead of one per head: "The fourth
 *        layer remembers", same section; the per-channel decay worked example in
 *        the Teacher guide, chapter 12, section 12.1 "Per-channel decay";
 *        the daily.dev summary of "You Could Have Come Up with Kimi Delta
 *        Attention" describes the gate as a diagonal per-key-channel matrix)
 *   2. read what the memory returns for the key:        e = S^T k_t
 *   3. error against the wanted value, scaled by beta:  u = beta_t (v_t - e)
 *   4. write the correction:                             S <- S + k_t u^T
 *        (steps 2-4 are the delta rule: read, subtract, write the difference,
 *        as in the akshathtiwari.co.in "Kimi Delta Attention" explainer,
 *        delta-rule paragraph, and the weaving.news recap "Attention? More
 *        like notation warfare", Key Points, last bullet)
 *   5. output:                                          o_t = S^T q_t
 *
 * Together: S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T.
 * The read in step 2 sees the already decayed state; the output in step 5
 * sees token t's own write.  No scaling of q and no normalisation of q or k
 * is applied (callers do that).  Everything is fp64; inputs arrive widened
 * exactly from their stored precision.
 *
 * Layouts (row-major, contiguous):
 *   q, k, log_alpha : (B, T, H, d_k)     v, o : (B, T, H, d_v)     beta : (B, T, H)
 *   S0, S_T         : (N, H, d_k, d_v)   N = number of sequences
 *   cu_seqlens      : N+1 offsets into T (requires B == 1); NULL means N = B
 *                     sequences of length T each.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of one (sequence, head).  S is d_k x d_v row-major (row = key
 * channel), updated in place.  work must hold d_v doubles. */
static void kda_oracle_token(double *S, const double *q, const double *k,
                             const double *v, const double *log_alpha,
                             double beta, int dk, int dv, double *o,
                             double *work)
{
    /* 1. forget: row i (key channel i) is scaled by alpha_i */
    for (int i = 0; i < dk; ++i) {
        const double a = exp(log_alpha[i]);
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] *= a;
    }
    /* 2.-3. read e = S^T k, error u = beta (v - e) */
    double *u = work;
    for (int j = 0; j < dv; ++j) {
        double e = 0.0;
        for (int i = 0; i < dk; ++i)
            e += S[(size_t)i * dv + j] * k[i];
        u[j] = beta * (v[j] - e);
    }
    /* 4. write S += k u^T */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] += k[i] * u[j];
    /* 5. output o = S^T q */
    if (o) {
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += S[(size_t)i * dv + j] * q[i];
            o[j] = acc;
        }
    }
}

/* Forward over whole sequences.  Returns 0 on success, -1 on bad arguments. */
int kda_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *log_alpha, const double *beta,
                   const double *S0, const int64_t *cu_seqlens, int num_seqs,
                   int B, int T, int H, int dk, int dv,
                   double *o, double *S_T, int nthreads)
{
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (cu_seqlens) {
        if (B != 1 || num_seqs < 0) return -1;
        if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) return -1;
        for (int s = 0; s < num_seqs; ++s)
            if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
    } else {
        num_seqs = B;
    }
    const long units = (long)num_seqs * H;
    int status = 0;
    if (nthreads <= 0) nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (long unit = 0; unit < units; ++unit) {
        const int s = (int)(unit / H), h = (int)(unit % H);
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *work = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !work) {
            free(S);
            free(work);
#pragma omp atomic write
            status = -2;
            continue;
        }
        const size_t sidx = ((size_t)s * H + h) * dk * dv;
        if (S0) memcpy(S, S0 + sidx, sizeof(double) * (size_t)dk * dv);
        else memset(S, 0, sizeof(double) * (size_t)dk * dv);

        /* token range of this sequence in the flattened (B*T) token index */
        long t0, t1;
        if (cu_seqlens) { t0 = (long)cu_seqlens[s]; t1 = (long)cu_seqlens[s + 1]; }
        else { t0 = (long)s * T; t1 = t0 + T; }

        for (long t = t0; t < t1; ++t) {
            const size_t th = (size_t)t * H + h; /* flattened (token, head) */
            kda_oracle_token(S, q + th * dk, k + th * dk, v + th * dv,
                             log_alpha + th * dk, beta[th], dk, dv,
                             o ? o + th * dv : NULL, work);
        }
        if (S_T) memcpy(S_T + sidx, S, sizeof(double) * (size_t)dk * dv);
        free(S);
        free(work);
    }
    return status;
}

/* One decode step for N independent sequences: the same token update applied
 * once to every (n, h) state of S_cache (N, H, d_k, d_v), in place.
 * q, k, log_alpha : (N, H, d_k); v, o : (N, H, d_v); beta : (N, H). */
int kda_oracle_decode(const double *q, const double *k, const double *v,
                      const double *log_alpha, const double *beta,
                      double *S_cache, int N, int H, int dk, int dv,
                      double *o, int nthreads)
{
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !S_cache) return -1;
    const long units = (long)N * H;
    int status = 0;
    if (nthreads <= 0) nthreads = 1;

#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (long unit = 0; unit < units; ++unit) {
        double *work = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!work) {
#pragma omp atomic write
            status = -2;
            continue;
        }
        kda_oracle_token(S_cache + (size_t)unit * dk * dv, q + (size_t)unit * dk,
                         k + (size_t)unit * dk, v + (size_t)unit * dv,
                         log_alpha + (size_t)unit * dk, beta[unit], dk, dv,
                         o ? o + (size_t)unit * dv : NULL, work);
        free(work);
    }
    return status;
}

/* ---------------------------------------------------------------------------
 * Backward: the gradient of a scalar loss through the forward above.
 *
 * The pages present the chunked form as the one used for efficient training
 * (the daily.dev summary of "You Could Have Come Up with Kimi Delta
 * Attention", Summary section) but print no backward pass, so this is the
 * plain definition: reverse-mode differentiation of the token loop, one token at a
 * time from the last to the first.  Given the loss's gradients dO with
 * respect to every output o_t and dS_T with respect to the final state, it
 * returns the gradients with respect to q, k, v, log_alpha, beta and S0.
 *
 * For token t, with S_prev the state before it and dS the gradient with
 * respect to the state after it (S_t), the forward steps are undone in
 * reverse order:
 *   5. o = S_t^T q         dq = S_t dO_t;          dS += q dO_t^T
 *   4. S_t = S' + k u^T    dk = dS u;              du = dS^T k
 *   3. u = beta (v - e)    dbeta = du . (v - e);   dv = beta du;  de = -beta du
 *   2. e = S'^T k          dk += S' de;            dS' = dS + k de^T
 *   1. S' = Diag(a) S_prev dlog_alpha_i = sum_j dS'_ij S'_ij  (a_i = e^{log_alpha_i});
 *                          dS_prev = Diag(a) dS'
 * and dS0 is dS after the first token.  The states S_prev are recomputed
 * with the forward token step from checkpoints kept every BWD_SEG tokens
 * (the same fp64 operations in the same order, so the values are those of
 * the forward); this only bounds memory.
 *
 * Layouts as for kda_oracle_fwd; dO like o, dS_T and dS0 like S_T.  dS_T may
 * be NULL (zero), S0 may be NULL (zero state).  Outputs dq, dk, dlog_alpha
 * like q; dv like v; dbeta like beta; dS0 (N, H, d_k, d_v).
 * ------------------------------------------------------------------------- */
#define BWD_SEG 64

static void kda_oracle_token_bwd(const double *S_prev, const double *q, const double *k,
                                 const double *v, const double *log_alpha, double beta,
                                 const double *dO, double *dS, int dk, int dv,
                                 double *dq, double *dkt, double *dvt,
                                 double *dlog_alpha, double *dbeta,
                                 double *Sp, double *u, double *e, double *du)
{
    /* recompute the token's forward quantities: S' = Diag(a) S_prev, e, u */
    for (int i = 0; i < dk; ++i) {
        const double a = exp(log_alpha[i]);
        for (int j = 0; j < dv; ++j)
            Sp[(size_t)i * dv + j] = a * S_prev[(size_t)i * dv + j];
    }
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i)
            acc += Sp[(size_t)i * dv + j] * k[i];
        e[j] = acc;
        u[j] = beta * (v[j] - acc);
    }
    /* 5. o = S_t^T q with S_t = S' + k u^T */
    for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j)
            acc += (Sp[(size_t)i * dv + j] + k[i] * u[j]) * dO[j];
        dq[i] = acc;
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            dS[(size_t)i * dv + j] += q[i] * dO[j];
    /* 4. S_t = S' + k u^T */
    for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j)
            acc += dS[(size_t)i * dv + j] * u[j];
        dkt[i] = acc;
    }
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i)
            acc += dS[(size_t)i * dv + j] * k[i];
        du[j] = acc;
    }
    /* 3. u = beta (v - e); from here on du holds de = -beta du */
    double db = 0.0;
    for (int j = 0; j < dv; ++j) {
        db += du[j] * (v[j] - e[j]);
        dvt[j] = beta * du[j];
        du[j] = -beta * du[j];
    }
    *dbeta = db;
    /* 2. e = S'^T k */
    for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dv; ++j)
            acc += Sp[(size_t)i * dv + j] * du[j];
        dkt[i] += acc;
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            dS[(size_t)i * dv + j] += k[i] * du[j];
    /* 1. S' = Diag(a) S_prev; dS becomes the gradient of S_prev */
    for (int i = 0; i < dk; ++i) {
        const double a = exp(log_alpha[i]);
        double acc = 0.0;
        for (int j = 0; j < dv; ++j) {
            acc += dS[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];
            dS[(size_t)i * dv + j] *= a;
        }
        dlog_alpha[i] = acc;
    }
}

int kda_oracle_bwd(const double *q, const double *k, const double *v,
                   const double *log_alpha, const double *beta,
                   const double *S0, const double *dO, const double *dS_T,
                   const int64_t *cu_seqlens, int num_seqs,
                   int B, int T, int H, int dk, int dv,
                   double *dq, double *dk_out, double *dv_out, double *dlog_alpha,
                   double *dbeta, double *dS0, int nthreads)
{
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || !dO) return -1;
    if (cu_seqlens) {
        if (B != 1 || num_seqs < 0) return -1;
        if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) return -1;
        for (int s = 0; s < num_seqs; ++s)
            if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
    } else {
        num_seqs = B;
    }
    const long units = (long)num_seqs * H;
    const size_t SS = (size_t)dk * dv;
    int status = 0;
    if (nthreads <= 0) nthreads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (long unit = 0; unit < units; ++unit) {
        const int s = (int)(unit / H), h = (int)(unit % H);
        long t0, t1;
        if (cu_seqlens) { t0 = (long)cu_seqlens[s]; t1 = (long)cu_seqlens[s + 1]; }
        else { t0 = (long)s * T; t1 = t0 + T; }
        const long len = t1 - t0;
        const long nseg = (len + BWD_SEG - 1) / BWD_SEG;
        /* ck: the state before each segment; seg: the state before each
         * token of one segment; dS: the running state gradient */
        double *ck = (double *)malloc(sizeof(double) * SS * (size_t)(nseg > 0 ? nseg : 1));
        double *seg = (double *)malloc(sizeof(double) * SS * (BWD_SEG + 1));
        double *dS = (double *)malloc(sizeof(double) * SS);
        double *Sp = (double *)malloc(sizeof(double) * SS);
        double *work = (double *)malloc(sizeof(double) * (size_t)dv * 3);
        if (!ck || !seg || !dS || !Sp || !work) {
            free(ck); free(seg); free(dS); free(Sp); free(work);
#pragma omp atomic write
            status = -2;
            continue;
        }
        const size_t sidx = ((size_t)s * H + h) * SS;
        /* forward once, keeping the state at each segment start */
        double *S = seg;
        if (S0) memcpy(S, S0 + sidx, sizeof(double) * SS);
        else memset(S, 0, sizeof(double) * SS);
        for (long t = t0; t < t1; ++t) {
            if ((t - t0) % BWD_SEG == 0) memcpy(ck + (size_t)((t - t0) / BWD_SEG) * SS, S, sizeof(double) * SS);
            const size_t th = (size_t)t * H + h;
            kda_oracle_token(S, q + th * dk, k + th * dk, v + th * dv, log_alpha + th * dk,
                             beta[th], dk, dv, NULL, work);
        }
        if (dS_T) memcpy(dS, dS_T + sidx, sizeof(double) * SS);
        else memset(dS, 0, sizeof(double) * SS);
        /* segments from the last to the first */
        for (long m = nseg - 1; m >= 0; --m) {
            const long a0 = t0 + m * BWD_SEG;
            const long a1 = (a0 + BWD_SEG < t1) ? a0 + BWD_SEG : t1;
            memcpy(seg, ck + (size_t)m * SS, sizeof(double) * SS);
            for (long t = a0; t + 1 < a1; ++t) {
                const size_t th = (size_t)t * H + h;
                double *nxt = seg + (size_t)(t - a0 + 1) * SS;
                memcpy(nxt, nxt - SS, sizeof(double) * SS);
                kda_oracle_token(nxt, q + th * dk, k + th * dk, v + th * dv, log_alpha + th * dk,
                                 beta[th], dk, dv, NULL, work);
            }
            for (long t = a1 - 1; t >= a0; --t) {
                const size_t th = (size_t)t * H + h;
                kda_oracle_token_bwd(seg + (size_t)(t - a0) * SS, q + th * dk, k + th * dk,
                                     v + th * dv, log_alpha + th * dk, beta[th], dO + th * dv,
                                     dS, dk, dv, dq + th * dk, dk_out + th * dk, dv_out + th * dv,
                                     dlog_alpha + th * dk, dbeta + th, Sp, work, work + dv,
                                     work + 2 * (size_t)dv);
            }
        }
        if (dS0) memcpy(dS0 + sidx, dS, sizeof(double) * SS);
        free(ck); free(seg); free(dS); free(Sp); free(work);
    }
    return status;
}

/* Number of threads the OpenMP runtime would use by default (for reports). */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
