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
 * per-token work is constant, "The fourth layer remembers").  Their *_ex
 * forms add the per-head and absent gates and slot-indexed state pools, and
 * kda_bwd_chunked differentiates the forward (training).
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers (HIP global memory) unless stated.
 *   - Tensors are contiguous, row-major, in the layouts listed per argument,
 *     with 16-byte aligned base pointers.
 *   - The caller owns every buffer.  The library allocates nothing, keeps no
 *     state between calls, never synchronises the stream, and is reentrant.
 *     A call enqueues kernel launches only (no memset or copy), so it can be
 *     captured into a HIP graph and replayed.
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
    KDA_ERR_UNSUPPORTED = 2,   /* a size or dtype combination the library does not implement */
    KDA_ERR_HIP = 3,           /* a HIP launch or query failed */
    KDA_ERR_SCRATCH_LIMIT = 4  /* more packed sequences than kda_fwd_chunked_noalloc's
                                  fixed scratch holds (KDA_NOALLOC_MAX_SEQS) */
} kda_status;

typedef enum {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

/* Layout of the forget gate log_alpha (used by the *_ex entry points).
 *   KDA_GATE_CHANNEL  one value per key channel: the operator above.
 *   KDA_GATE_HEAD     one value per token and head, shared by all key channels
 *                     (log_alpha has beta's shape): the scalar-gated delta rule
 *                     that KDA generalises, Gated DeltaNet ("The fourth layer
 *                     remembers", the paragraph on the forget gate: one decay per
 *                     head per token there, one per key channel in KDA).
 *   KDA_GATE_NONE     no gate, alpha = 1 (log_alpha is not read and may be NULL):
 *                     the plain delta rule, DeltaNet (akshathtiwari.co.in "Kimi
 *                     Delta Attention" explainer, delta-rule paragraph).
 * Each is exactly the channel-gated operator with log_alpha broadcast over the
 * key channels, or zero. */
typedef enum {
    KDA_GATE_CHANNEL = 0,
    KDA_GATE_HEAD = 1,
    KDA_GATE_NONE = 2
} kda_gate;

/* Input preparation folded into the *_ex entry points (bits of `flags`):
 * steps that usually come just before the operator, namely L2-normalised q
 * and k, and a forget gate produced as -softplus of a pre-activation by the
 * gate module in front of the layer ("The fourth layer remembers", the
 * paragraph on the forget-gate module two labs share).
 *   KDA_FLAG_L2NORM_QK      q and k are divided by their Euclidean norm over
 *                           d_k, per token and head, before use (a zero vector
 *                           stays zero).  q and k are not modified in memory.
 *   KDA_FLAG_GATE_SOFTPLUS  the gate tensor holds x, and log_alpha = -softplus(x)
 *                           = -log(1 + e^x), i.e. alpha = 1 / (1 + e^x) in (0, 1):
 *                           any finite x (or -inf, alpha = 1) is valid.  No
 *                           effect with KDA_GATE_NONE.
 * Any other bit is KDA_ERR_INVALID_ARG. */
typedef enum {
    KDA_FLAG_L2NORM_QK = 1,
    KDA_FLAG_GATE_SOFTPLUS = 2
} kda_flags;

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
 * Supported: dk in {64, 128}, dv in {64, 128}; dtype KDA_BF16 or KDA_F32.
 * Zero-length sequences are allowed (S_T = S0).
 * The chunk length is internal (32 tokens for bf16 inputs, 64 for fp32).
 */
kda_status kda_fwd_chunked(const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *beta,
                           const float *S0, const int32_t *cu_seqlens, int num_seqs,
                           int B, int T, int H, int dk, int dv, kda_dtype dtype,
                           void *o, float *S_T,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_fwd_chunked_ex -- kda_fwd_chunked with a gate layout and slot-indexed states.
 *
 * Serving keeps one fixed-size state per live sequence (constant memory per
 * sequence and constant work per decoded token, "The fourth layer remembers")
 * in a pool whose rows are handed out to requests; this entry point continues
 * sequences straight from and into such a pool (chunked prefill, or a few
 * tokens per sequence as multi-token decode).
 *
 *   gate            : layout of log_alpha (kda_gate): (B, T, H, dk) for
 *                     KDA_GATE_CHANNEL, (B, T, H) for KDA_GATE_HEAD, unused for
 *                     KDA_GATE_NONE.
 *   flags           : input preparation, a combination of kda_flags (0: none).
 *   S0, S_T         : as in kda_fwd_chunked when state_idx is NULL.  Otherwise
 *                     pools of shape (pool_size, H, dk, dv) fp32 (each may be
 *                     NULL; S0 == S_T continues the pool in place).
 *   state_idx       : NULL, or (N,) int32 device array: sequence s starts from
 *                     row state_idx[s] of S0 and writes its final state to row
 *                     state_idx[s] of S_T.  An index outside [0, pool_size)
 *                     means no state: the sequence starts from zeros and its
 *                     final state is not written (padding slots).  Valid
 *                     indices must be distinct when S_T is given.
 *   pool_size       : rows of the pools (used only with state_idx).
 * Every other argument, the supported sizes and the errors are those of
 * kda_fwd_chunked, which equals this call with KDA_GATE_CHANNEL, no flags and
 * no state_idx.
 */
kda_status kda_fwd_chunked_ex(const void *q, const void *k, const void *v,
                              const void *log_alpha, const void *beta, kda_gate gate,
                              unsigned flags,
                              const float *S0, float *S_T, const int32_t *state_idx, int pool_size,
                              const int32_t *cu_seqlens, int num_seqs,
                              int B, int T, int H, int dk, int dv, kda_dtype dtype,
                              void *o, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_fwd_chunked_noalloc -- kda_fwd_chunked_ex with no workspace argument.
 *
 * For callers that cannot allocate device memory: code being captured into
 * a graph, tight serving loops, harnesses that forbid allocation.  The call
 * allocates nothing (no hipMalloc, no library allocator); the only scratch
 * the forward needs, the processing order of packed sequences, lives in a
 * fixed array of KDA_NOALLOC_MAX_SEQS int32 entries (256 KiB) that the
 * library holds on each GPU it runs on until the process ends.  Every call
 * on one GPU uses that GPU's array, so calls that overlap on one GPU (on
 * different streams, or from different host threads) race and must not be
 * issued; calls on one stream are ordered and safe.  The array is fully
 * rewritten by each packed call before it is read.
 *
 * Arguments, results, supported sizes and errors are those of
 * kda_fwd_chunked_ex without workspace and workspace_bytes, plus
 * KDA_ERR_SCRATCH_LIMIT when cu_seqlens is given with num_seqs >
 * KDA_NOALLOC_MAX_SEQS (nothing is enqueued then).
 */
#define KDA_NOALLOC_MAX_SEQS 65536
kda_status kda_fwd_chunked_noalloc(const void *q, const void *k, const void *v,
                                   const void *log_alpha, const void *beta, kda_gate gate,
                                   unsigned flags,
                                   const float *S0, float *S_T, const int32_t *state_idx,
                                   int pool_size, const int32_t *cu_seqlens, int num_seqs,
                                   int B, int T, int H, int dk, int dv, kda_dtype dtype,
                                   void *o, void *stream);

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

/*
 * kda_decode_step_ex -- kda_decode_step with a gate layout, a state pool and
 * L consecutive tokens per sequence.
 *
 *   L               : tokens per sequence in this call (L >= 0; 0 does nothing).
 *                     The recurrence runs over them in order (the recurrent
 *                     form, constant work per token: "The fourth layer
 *                     remembers"); each state is read and written once per call.
 *   q, k            : (N, L, H, dk)      dtype
 *   v               : (N, L, H, dv)      dtype
 *   log_alpha       : (N, L, H, dk), (N, L, H) or unused, per `gate` (kda_gate)
 *   flags           : input preparation, a combination of kda_flags (0: none)
 *   beta            : (N, L, H)          dtype
 *   o               : (N, L, H, dv)      dtype, written
 *   S_pool          : fp32 states, read and rewritten in place: (N, H, dk, dv)
 *                     when state_idx is NULL, else (pool_size, H, dk, dv).
 *   state_idx       : NULL, or (N,) int32 device array: sequence n updates row
 *                     state_idx[n] of S_pool.  An index outside [0, pool_size)
 *                     means no state: o is computed from a zero state and
 *                     nothing is written.  Valid indices must be distinct.
 * Every other argument is that of kda_decode_step, which equals this call
 * with KDA_GATE_CHANNEL, no flags, no state_idx and L = 1.
 */
kda_status kda_decode_step_ex(const void *q, const void *k, const void *v,
                              const void *log_alpha, const void *beta, kda_gate gate,
                              unsigned flags,
                              float *S_pool, const int32_t *state_idx, int pool_size,
                              int N, int L, int H, int dk, int dv, kda_dtype dtype, void *o,
                              void *stream);

/* Workspace size in bytes that kda_bwd_chunked needs for these sizes.  It
 * holds, per chunk of 32 tokens and head, the state entering the chunk, the
 * gradient of the state leaving it (fp32, dk x dv each), three 32 x 32 fp32
 * matrices, a flag, three 32 x dv and three 32 x 32 bf16 matrices.  num_seqs
 * is the number of packed sequences when cu_seqlens is used, else B. */
size_t kda_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs);

/*
 * kda_bwd_chunked -- gradients through kda_fwd_chunked_ex (no flags, no slot
 * map): given dL/do and dL/dS_T of a loss L, the gradients of L with respect
 * to q, k, v, log_alpha, beta and S0.  The pages present the chunkwise form
 * as the one used for efficient training (daily.dev summary of "You Could
 * Have Come Up with Kimi Delta Attention", Summary section); this is that
 * form differentiated, recomputing the forward's chunk states.
 *
 *   q, k, v, log_alpha, beta, gate, S0, cu_seqlens, num_seqs, B, T, H, dk,
 *   dv, dtype       : exactly as given to the forward (S0 NULL = zeros).
 *   dO              : (B, T, H, dv)      dtype, dL/do
 *   dS_T            : (N, H, dk, dv)     fp32, dL/dS_T; NULL = zeros
 *   dq, dk_out      : (B, T, H, dk)      dtype, written
 *   dv_out          : (B, T, H, dv)      dtype, written
 *   dlog_alpha      : log_alpha's shape for the gate layout, dtype, written
 *                     (unused for KDA_GATE_NONE; the per-head layout gets the
 *                     sum over key channels)
 *   dbeta           : (B, T, H)          dtype, written
 *   dS0             : (N, H, dk, dv)     fp32, written (also when S0 is NULL);
 *                                        NULL = not written
 *   workspace       : device scratch of at least kda_bwd_workspace_bytes(...)
 *                     bytes, 256-byte aligned; its contents on entry do not matter.
 * No output may alias an input or another output.
 * Supported: dk, dv in {64, 128}; dtype KDA_BF16 or KDA_F32 (all arithmetic
 * fp32).  Zero-length sequences are allowed (dS0 = dS_T).
 */
kda_status kda_bwd_chunked(const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *beta, kda_gate gate,
                           const float *S0, const void *dO, const float *dS_T,
                           const int32_t *cu_seqlens, int num_seqs,
                           int B, int T, int H, int dk, int dv, kda_dtype dtype,
                           void *dq, void *dk_out, void *dv_out, void *dlog_alpha, void *dbeta,
                           float *dS0, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Faults the kernels detect while they run.
 *
 * The chunked forward (and the first kernel of the backward for bf16
 * inputs) hands each chunk from the waves that prepare it to the waves that
 * apply it through flags in on-chip memory.  Every wait on such a flag is
 * bounded.  Should one run out (it does not in correct operation), the
 * workgroup stops instead of hanging: it writes NaN into every output it has
 * not produced yet (the remaining rows of o in its value columns and its
 * columns of S_T; in the backward, the chunk states its later kernels read,
 * so the gradients are not meaningful) and sets KDA_DEVERR_WAIT_TIMEOUT in a
 * sticky per-device error word.  The call itself has already returned KDA_OK
 * by then, since kernels run asynchronously.
 */
typedef enum {
    KDA_DEVERR_WAIT_TIMEOUT = 1
} kda_device_error_bits;

/* Synchronise `stream`, then store the current device's error word (an OR of
 * kda_device_error_bits, 0 when nothing went wrong) in *bits; clear != 0
 * resets it to 0.  Returns KDA_ERR_INVALID_ARG for bits == NULL and
 * KDA_ERR_HIP when the synchronisation or the read fails.  It copies memory
 * and blocks, unlike the compute entry points. */
kda_status kda_device_errors(unsigned *bits, int clear, void *stream);

/* Diagnostics: the number of polls a bounded wait makes before it gives up
 * (default 1048576, about 1e8 GPU cycles).  It applies process-wide to
 * launches made after the call.  Tests of the timeout handling set it to 0,
 * so that every such wait gives up at once.  polls < 0 is
 * KDA_ERR_INVALID_ARG. */
kda_status kda_set_wait_limit(int polls);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
