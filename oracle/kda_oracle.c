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

/* Number of threads the OpenMP runtime would use by default (for reports). */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
