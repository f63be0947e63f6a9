// kda_api.hip -- C ABI of the KDA operator: argument checks and dispatch.
// Declarations and the contract of every entry point are in include/kda.h.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/kda.h"

namespace kda {
hipError_t decode_step_launch(const void *q, const void *k, const void *v,
                              const void *log_alpha, const void *beta, int gate, int prep, float *S,
                              const int32_t *state_idx, int pool, void *o, int N, int L, int H,
                              int dk, int dv, bool bf16, hipStream_t stream);
hipError_t chunked_fwd_launch(const void *q, const void *k, const void *v, const void *g,
                              const void *beta, int gate, int prep, const float *S0, float *S_T,
                              const int32_t *state_idx, int pool, void *o,
                              const int32_t *cu_seqlens, int num_seqs, int B, int T, int H,
                              int dk, int dv, bool bf16, void *workspace, hipStream_t stream);
size_t bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs);
void ws_set_spin_limit(int polls);
int noalloc_max_seqs();
hipError_t noalloc_scratch(int32_t **out);
hipError_t ws_device_errors(unsigned *bits, bool clear);
hipError_t bwd_launch(const void *q, const void *k, const void *v, const void *g, const void *beta,
                      int gate, const float *S0, const void *dO, const float *dST,
                      const int32_t *cu_seqlens, int num_seqs, int B, int T, int H, int dk, int dv,
                      bool bf16, void *dq, void *dk_out, void *dv_out, void *dg, void *dbeta,
                      float *dS0, void *workspace, hipStream_t stream);
}  // namespace kda

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dim_ok(int d) { return d == 64 || d == 128; }

bool gate_ok(kda_gate g) { return g == KDA_GATE_CHANNEL || g == KDA_GATE_HEAD || g == KDA_GATE_NONE; }

bool flags_ok(unsigned f) { return (f & ~(unsigned)(KDA_FLAG_L2NORM_QK | KDA_FLAG_GATE_SOFTPLUS)) == 0; }

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Element counts must stay addressable with 64-bit offsets and the grid must
// fit a 32-bit block index.
bool sizes_fit(long long a, long long b, long long c, long long d) {
    const long long lim = (long long)1 << 46;
    long long x = a;
    if (b && x > lim / b) return false;
    x *= b;
    if (c && x > lim / c) return false;
    x *= c;
    if (d && x > lim / d) return false;
    return true;
}

}  // namespace

extern "C" {

const char *kda_status_string(kda_status status)
{
    switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    case KDA_ERR_SCRATCH_LIMIT: return "KDA_ERR_SCRATCH_LIMIT";
    }
    return "KDA_ERR_UNKNOWN";
}

size_t kda_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs)
{
    (void)B; (void)T; (void)H; (void)dk; (void)dv;
    // longest-first order of packed sequences
    if (num_seqs <= 1) return 0;
    return ((size_t)num_seqs * sizeof(int32_t) + 255) & ~(size_t)255;
}

kda_status kda_fwd_chunked_ex(const void *q, const void *k, const void *v,
                              const void *log_alpha, const void *beta, kda_gate gate,
                              unsigned flags,
                              const float *S0, float *S_T, const int32_t *state_idx, int pool_size,
                              const int32_t *cu_seqlens, int num_seqs,
                              int B, int T, int H, int dk, int dv, kda_dtype dtype,
                              void *o, void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
    if (!gate_ok(gate) || !flags_ok(flags)) return KDA_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
    if (cu_seqlens && (B != 1 || num_seqs < 0)) return KDA_ERR_INVALID_ARG;
    const int nseq = cu_seqlens ? num_seqs : B;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (!sizes_fit(B, T, H, dk > dv ? dk : dv) || !sizes_fit(nseq, H, dk, dv)) return KDA_ERR_INVALID_ARG;
    if ((long long)nseq * H * 2 >= ((long long)1 << 31)) return KDA_ERR_INVALID_ARG;
    if (state_idx) {
        if (pool_size < 0 || !aligned4(state_idx) || !sizes_fit(pool_size, H, dk, dv))
            return KDA_ERR_INVALID_ARG;
    }
    const long long tokens = (long long)B * T;
    const void *g = gate == KDA_GATE_NONE ? nullptr : log_alpha;
    if (tokens > 0 || nseq > 0) {
        if (tokens > 0 && (!q || !k || !v || !beta || !o)) return KDA_ERR_INVALID_ARG;
        if (tokens > 0 && gate != KDA_GATE_NONE && !log_alpha) return KDA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) ||
            !aligned16(beta) || !aligned16(o) || !aligned16(S0) || !aligned16(S_T))
            return KDA_ERR_INVALID_ARG;
    }
    const size_t need = kda_fwd_workspace_bytes(B, T, H, dk, dv, nseq);
    if (cu_seqlens && need > 0) {
        if (!workspace || workspace_bytes < need || !aligned16(workspace)) return KDA_ERR_INVALID_ARG;
    }
    if (nseq == 0) return KDA_OK;
    hipError_t e = kda::chunked_fwd_launch(q, k, v, g, beta, (int)gate, (int)flags, S0, S_T, state_idx,
                                           pool_size, o, cu_seqlens, nseq, B, T, H, dk, dv,
                                           dtype == KDA_BF16, cu_seqlens ? workspace : nullptr,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_fwd_chunked_noalloc(const void *q, const void *k, const void *v,
                                   const void *log_alpha, const void *beta, kda_gate gate,
                                   unsigned flags,
                                   const float *S0, float *S_T, const int32_t *state_idx,
                                   int pool_size, const int32_t *cu_seqlens, int num_seqs,
                                   int B, int T, int H, int dk, int dv, kda_dtype dtype,
                                   void *o, void *stream)
{
    if (cu_seqlens && num_seqs > kda::noalloc_max_seqs()) return KDA_ERR_SCRATCH_LIMIT;
    void *order = nullptr;
    size_t order_bytes = 0;
    if (cu_seqlens && num_seqs > 1 && B == 1) {
        int32_t *p = nullptr;
        if (kda::noalloc_scratch(&p) != hipSuccess) return KDA_ERR_HIP;
        order = p;
        order_bytes = (size_t)kda::noalloc_max_seqs() * sizeof(int32_t);
    }
    return kda_fwd_chunked_ex(q, k, v, log_alpha, beta, gate, flags, S0, S_T, state_idx, pool_size,
                              cu_seqlens, num_seqs, B, T, H, dk, dv, dtype, o, order, order_bytes,
                              stream);
}

kda_status kda_fwd_chunked(const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *beta,
                           const float *S0, const int32_t *cu_seqlens, int num_seqs,
                           int B, int T, int H, int dk, int dv, kda_dtype dtype,
                           void *o, float *S_T,
                           void *workspace, size_t workspace_bytes, void *stream)
{
    return kda_fwd_chunked_ex(q, k, v, log_alpha, beta, KDA_GATE_CHANNEL, 0u, S0, S_T, nullptr, 0,
                              cu_seqlens, num_seqs, B, T, H, dk, dv, dtype, o, workspace,
                              workspace_bytes, stream);
}

kda_status kda_decode_step_ex(const void *q, const void *k, const void *v,
                              const void *log_alpha, const void *beta, kda_gate gate,
                              unsigned flags,
                              float *S_pool, const int32_t *state_idx, int pool_size,
                              int N, int L, int H, int dk, int dv, kda_dtype dtype, void *o,
                              void *stream)
{
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
    if (!gate_ok(gate) || !flags_ok(flags)) return KDA_ERR_INVALID_ARG;
    if (N < 0 || L < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (!sizes_fit(N, H, dk, dv) || !sizes_fit(N, L, H, dk > dv ? dk : dv)) return KDA_ERR_INVALID_ARG;
    if ((long long)N * H >= ((long long)1 << 31)) return KDA_ERR_INVALID_ARG;
    if (state_idx && (pool_size < 0 || !aligned4(state_idx) || !sizes_fit(pool_size, H, dk, dv)))
        return KDA_ERR_INVALID_ARG;
    if (N == 0 || L == 0) return KDA_OK;
    if (!q || !k || !v || !beta || !S_pool || !o) return KDA_ERR_INVALID_ARG;
    if (gate != KDA_GATE_NONE && !log_alpha) return KDA_ERR_INVALID_ARG;
    if (!aligned16(S_pool)) return KDA_ERR_INVALID_ARG;
    hipError_t e = kda::decode_step_launch(q, k, v, gate == KDA_GATE_NONE ? nullptr : log_alpha,
                                           beta, (int)gate, (int)flags, S_pool, state_idx, pool_size, o, N, L, H,
                                           dk, dv, dtype == KDA_BF16,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *beta,
                           float *S_cache, int N, int H, int dk, int dv,
                           kda_dtype dtype, void *o, void *stream)
{
    return kda_decode_step_ex(q, k, v, log_alpha, beta, KDA_GATE_CHANNEL, 0u, S_cache, nullptr, 0,
                              N, 1, H, dk, dv, dtype, o, stream);
}

size_t kda_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs)
{
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || num_seqs < 0) return 0;
    return kda::bwd_workspace_bytes(B, T, H, dk, dv, num_seqs);
}

kda_status kda_bwd_chunked(const void *q, const void *k, const void *v,
                           const void *log_alpha, const void *beta, kda_gate gate,
                           const float *S0, const void *dO, const float *dS_T,
                           const int32_t *cu_seqlens, int num_seqs,
                           int B, int T, int H, int dk, int dv, kda_dtype dtype,
                           void *dq, void *dk_out, void *dv_out, void *dlog_alpha, void *dbeta,
                           float *dS0, void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
    if (!gate_ok(gate)) return KDA_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARG;
    if (cu_seqlens && (B != 1 || num_seqs < 0)) return KDA_ERR_INVALID_ARG;
    const int nseq = cu_seqlens ? num_seqs : B;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (!sizes_fit(B, T, H, dk > dv ? dk : dv) || !sizes_fit(nseq, H, dk, dv)) return KDA_ERR_INVALID_ARG;
    if ((long long)nseq * H * (dv / 32) >= ((long long)1 << 31)) return KDA_ERR_INVALID_ARG;
    const long long slots = (long long)B * ((T + 31) / 32) + nseq + 1;
    if (slots >= ((long long)1 << 31) || H > 65535) return KDA_ERR_INVALID_ARG;
    const long long tokens = (long long)B * T;
    const void *g = gate == KDA_GATE_NONE ? nullptr : log_alpha;
    void *dg = gate == KDA_GATE_NONE ? nullptr : dlog_alpha;
    if (tokens > 0) {
        if (!q || !k || !v || !beta || !dO || !dq || !dk_out || !dv_out || !dbeta)
            return KDA_ERR_INVALID_ARG;
        if (gate != KDA_GATE_NONE && (!log_alpha || !dlog_alpha)) return KDA_ERR_INVALID_ARG;
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(dO) || !aligned16(S0) || !aligned16(dS_T) || !aligned16(dq) ||
        !aligned16(dk_out) || !aligned16(dv_out) || !aligned16(dg) || !aligned16(dbeta) ||
        !aligned16(dS0))
        return KDA_ERR_INVALID_ARG;
    if (nseq == 0) return KDA_OK;
    const size_t need = kda::bwd_workspace_bytes(B, T, H, dk, dv, nseq);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return KDA_ERR_INVALID_ARG;
    hipError_t e = kda::bwd_launch(q, k, v, g, beta, (int)gate, S0, dO, dS_T, cu_seqlens, nseq, B,
                                   T, H, dk, dv, dtype == KDA_BF16, dq, dk_out, dv_out, dg, dbeta,
                                   dS0, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_device_errors(unsigned *bits, int clear, void *stream)
{
    if (!bits) return KDA_ERR_INVALID_ARG;
    *bits = 0;
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return KDA_ERR_HIP;
    return kda::ws_device_errors(bits, clear != 0) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_set_wait_limit(int polls)
{
    if (polls < 0) return KDA_ERR_INVALID_ARG;
    kda::ws_set_spin_limit(polls);
    return KDA_OK;
}

}  // extern "C"
