/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention operator.
 *
 * The operator.  Per (sequence, head) a fixed-size state S of shape d_k x d_v
 * ("key dimension by value dimension": "The fourth layer remembers", section
 * "What each kind of layer keeps") is updated token by token with a delta-rule
 * write and a per-key-channel forget gate:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,      alpha_t = exp(log_alpha_t)  (one value per key channel)
 *
 * (delta rule read-error-write and the Diagonal-Plus-Low-Rank transition:
 * akshathtiwari.co.in "Kimi Delta Attention" explainer; the gate as a diagonal
 * matrix with one entry per key channel: daily.dev summary of "You Could Have
 * Come Up with Kimi Delta Attention" and "The fourth layer remembers").
 * The read inside the update sees the decayed state; o_t sees token t's own
 * write.  No 1/sqrt(d_k) scaling and no normalisation of q or k is applied.
 *
 * Two entry points: a chunkwise forward over whole sequences (the chunkwise
 * form named in the daily.dev summary; training and prefill) and a one-token
 * decode step that rewrites a state cache in place (the recurrent form; the
 * per-token work is constant, "The fourth layer remembers").
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers (HIP global memory) unless stated.
 *   - Tensors are contiguous, row-major, in the layouts listed per argument,
 *     with 16-byte aligned base pointers.
 *   - The caller owns every buffer.  The library allocates nothing, keeps no
 *     state between calls, never synchronises the stream, and is reentrant.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Work is only enqueued; errors of the asynchronous kernels themselves
 *     surface at the caller's next synchronisation.
 *   - Errors are reported by status code only; nothing aborts or throws.
 *     On an error status no work has been enqueued, except KDA_ERR_HIP
 *     (a launch failed).
 *   - dtype applies to q, k, v, log_alpha, beta and o.  States (S0, S_T,
 *     S_cache) are always fp32.
 *   - log_alpha must be finite and <= 0 (alpha in (0, 1]: a forget gate);
 *     beta any finite value.  Inputs outside this domain are not detected.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,   /* NULL required pointer, negative size, misaligned pointer,
                                  cu_seqlens with B != 1, workspace too small */
    KDA_ERR_UNSUPPORTED = 2,   /* a size or dtype combination this build does not implement */
    KDA_ERR_HIP = 3            /* a HIP launch or query failed */
} kda_status;

typedef enum {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char *kda_status_string(kda_status status);

/* Workspace size in bytes that kda_fwd_chunked needs for these sizes
 * (0 when none is needed).  num_seqs is the number of packed sequences when
 * cu_seqlens is used, else B. */
size_t kda_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs);

/*
 * kda_fwd_chunked -- chunkwise forward over whole sequences.
 *
 *   q, k, log_alpha : (B, T, H, dk)      dtype
 *   v               : (B, T, H, dv)      dtype
 *   beta            : (B, T, H)          dtype
 *   S0              : (N, H, dk, dv)     fp32, initial state per sequence; NULL = zeros
 *   cu_seqlens      : (N + 1,)           int32 device array of token offsets,
 *                                        cu_seqlens[0] = 0, nondecreasing,
 *                                        cu_seqlens[N] = T; requires B == 1.
 *                                        NULL = N = B sequences of length T.
 *   num_seqs        : N when cu_seqlens is given (ignored otherwise)
 *   o               : (B, T, H, dv)      dtype, written
 *   S_T             : (N, H, dk, dv)     fp32 final state per sequence; NULL = not written.
 *                                        S_T == S0 (in-place continuation) is allowed;
 *                                        no other aliasing is.
 *   workspace       : device scratch of at least kda_fwd_workspace_bytes(...) bytes
 *                                        (may be NULL when that size is 0)
 *
 * Supported: dk in {64, 128}, dv in {64, 128}; dtype KDA_BF16 for every such
 * size, KDA_F32 for dk = 64.  Zero-length sequences are allowed (S_T = S0).
 * The chunk length is internal (32 tokens for bf16 inputs, 64 for fp32).
 */
kda_status kda_fwd_chunked(const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *beta,
                           const float *S0, const int32_t *cu_seqlens, int num_seqs,
                           int B, int T, int H, int dk, int dv, kda_dtype dtype,
                           void *o, float *S_T,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_decode_step -- one token for each of N independent sequences.
 *
 *   q, k, log_alpha : (N, H, dk)         dtype
 *   v               : (N, H, dv)         dtype
 *   beta            : (N, H)             dtype
 *   S_cache         : (N, H, dk, dv)     fp32, read and rewritten in place
 *   o               : (N, H, dv)         dtype, written
 *
 * Supported: dk, dv in {64, 128}; dtype KDA_BF16 or KDA_F32.
 */
kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *beta,
                           float *S_cache, int N, int H, int dk, int dv,
                           kda_dtype dtype, void *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
