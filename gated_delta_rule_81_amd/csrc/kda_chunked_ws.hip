// kda_chunked_ws.hip -- chunkwise KDA forward for bf16 inputs on gfx950,
// producer / consumer waves.
//
// Same chunk algebra as the fp32 kernel (kda_chunked.hip), derived from the
// recurrence S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
// o_t = S_t^T q_t.  Here the chunk is C = 32 tokens and decay factors are
// referenced to the chunk start: with E_r = e^{Gamma_r} (<= 1, Gamma the
// inclusive cumulative log-decay per key channel) and R_r = e^{Gamma_last - Gamma_r}
// (<= 1),
//   K_up = K * E,  Q_up = Q * E,  K_right = K * R,  K_dn = K_right / gamma,
//   A = strict_lower(Diag(beta) K_up K_dn^T),  P = tril_incl(Q_up K_dn^T),
//   T' = (I + A)^{-1} Diag(beta),
//   U = T' (V - K_up S),  O = Q_up S + P U,  S <- Diag(gamma) S + K_right^T U.
// K_dn carries factors up to 1/gamma; a chunk whose decay on some channel
// exceeds 2^100 (or whose keys exceed 2^16 in magnitude) forms A and P
// entry by entry with e^{Gamma_r - Gamma_i} evaluated directly instead.
//
// Work split (one 512-thread workgroup per (sequence, head, value slice)):
//   waves 0-3  consumers: each owns 16-column strips of the fp32 state, kept
//              in MFMA accumulators for the whole sequence, and applies the
//              chunk update from operands a producer left in LDS.
//   waves 4-7  producers: wave p prepares chunks p, p+4, p+8, ... entirely by
//              itself (lane = key channel(s), all 32 rows): cumulative decay
//              products, scaled operands, A and P on MFMA, the 32x32 inverse.
// Producer and consumer waves of a SIMD overlap: VALU-heavy preparation runs
// while the MFMA-heavy state update of an earlier chunk runs.  Handoff is a
// ring of 4 LDS slots, slot p belonging to producer p, with per-slot flags
// (full: chunk id + 1 written by the producer; freed: consumer completions).
// Every wait is bounded; a wait that runs out marks the workgroup dead and
// all waves leave, so a protocol error can never hang the device.  Its
// consumers first write NaN into every output the workgroup has not produced
// yet (o rows, its columns of S_T; the SAVE instantiation's remaining chunk
// states, X and U) and set a bit in the device's error word (g_ws_error,
// read and cleared through kda_device_errors), so a timed-out wait never
// passes for a result.
//
// LDS rows are made of 16-byte chunks stored at position chunk ^ key(row),
// so that the 16 rows one fragment read touches fall in distinct banks
// without row padding (padding would leave no room for four slots).
//
// The SAVE instantiation is the first step of the backward for bf16 inputs:
// the same chain with no o and no final state, keeping instead, per chunk,
// what the gradient kernels read (the entering state, X and U from the
// consumers; T, M0, T^T, P^T, P where flagged and the flag from the
// producers; layouts in WsParams).  The forward's instantiations compile to
// the code they had before it existed.
#include <type_traits>

#include "kda_device.h"

namespace kda {

struct WsParams {
    const void *q, *k, *v, *g, *beta;
    const float *S0;
    float *S_T;
    void *o;
    const int32_t *cu_seqlens;
    const int32_t *order;
    const int32_t *state_idx;   // slot map of S0 / S_T rows (NULL: row = sequence)
    int T, H, DV, units, nslices, pool;
    int spin_limit;             // polls a bounded wait makes before giving up
    // What the backward keeps of the forward (SAVE instantiation), per
    // (chunk slot, head); a sequence's chunks take consecutive slots from
    // floor(cu_seqlens[s] / 32) + s (packed) or s * ceil(T / 32) (dense):
    //   wS  bf16 [d_k][d_v]  the state entering the chunk
    //   wX  bf16 [32][d_v]   X = V - K_up S
    //   wU  bf16 [32][d_v]   U = T Diag(beta) X
    //   wT  fp32 [32][32]    T = (I + A)^{-1}
    //   wM  fp32 [32][32]    M0 = strict_lower(K_up K_dn^T)  (A = Diag(beta) M0)
    //   wP  fp32 [32][32]    P, written only for chunks flagged in wF
    //   wTt, wPt  bf16 [32][32]  T^T and P^T
    //   wF  int32            1 when some channel decays by more than 2^64 over the chunk
    bf16_t *wS, *wX, *wU, *wTt, *wPt;
    float *wT, *wM, *wP;
    int32_t *wF;
};

namespace ws {

constexpr int C = 32;          // chunk length
constexpr int NSLOT = 4;       // LDS ring depth (one slot per producer)
constexpr int NPROD = 4;
constexpr int SPIN_LIMIT = 1 << 20;
constexpr int LA = 36;         // fp32 row stride of the private [32][32] matrices

template <int DK>
struct Lds {
    // one ring slot
    static constexpr int KU = 0;                          // -K_up     [32][DK] bf16
    static constexpr int QU = KU + C * DK * 2;            // Q_up      [32][DK]
    static constexpr int KRT = QU + C * DK * 2;           // K_right^T [DK][32]
    static constexpr int TP = KRT + DK * C * 2;           // T'        [32][32]
    static constexpr int PM = TP + C * C * 2;             // P         [32][32]
    static constexpr int GM = PM + C * C * 2;             // gamma     [DK] fp32
    static constexpr int SLOT = GM + DK * 4;
    // producer-private region: K_dn [32][DK] bf16 while A and P are formed,
    // then A^T and T fp32 [32][LA]; the exact path first uses it to stage
    // 32 channels at a time (log2 Gamma fp32 [32][32], k and q bf16 [32][32])
    static constexpr int P_KD = 0;
    static constexpr int P_AT = 0;
    static constexpr int P_T = C * LA * 4;
    static constexpr int P_USED = (C * DK * 2 > 2 * C * LA * 4) ? C * DK * 2 : 2 * C * LA * 4;
    static constexpr int P_BETA = P_USED > 8192 ? P_USED : 8192;
    static constexpr int P_NORM = P_BETA + C * 4;             // 1/|k_r|, 1/|q_r| fp32 [2][32]
    static constexpr int PRIV = P_NORM + 2 * C * 4;
    static constexpr int PRIV_BASE = NSLOT * SLOT;
    static constexpr int SYNC = PRIV_BASE + NPROD * PRIV;   // full[4], freed[4], dead
    static constexpr int BYTES = SYNC + 64;
    static_assert(SLOT % 16 == 0 && PRIV % 16 == 0, "alignment");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Swizzle key of row r of a [32][DK] array.  Consumer fragment reads touch
// rows 8a + 4h + b (a, b = 0..3, h fixed), producer reads rows 16R + m
// (m = 0..15, R fixed); for both sets the pair (bank half of the row for
// d_k = 64, chunk ^ key) takes 16 distinct values.
template <int DK>
__device__ __forceinline__ int keyK(int r) {
    if constexpr (DK == 128) return ((((r >> 3) & 3) << 2) | (r & 3)) ^ (((r >> 2) & 1) << 3);
    else return ((((r >> 3) & 3) << 1) | ((r >> 1) & 1)) ^ (((r >> 2) & 1) << 2);
}
// [*][32] arrays: 4 rows share the 64 banks; rows 8a + 4h + b get distinct
// (b, chunk ^ a) pairs
__device__ __forceinline__ int key4(int r) { return (r >> 3) & 3; }

// element index of (r, c) in a swizzled [32][DK] array
template <int DK>
__device__ __forceinline__ int idxK(int r, int c) {
    return r * DK + (((c >> 3) ^ keyK<DK>(r)) << 3) + (c & 7);
}
// element index of (r, c) in a swizzled [*][32] array
__device__ __forceinline__ int idx4(int r, int c) {
    return r * C + (((c >> 3) ^ key4(r)) << 3) + (c & 7);
}
// K_right^T [DK][32]: groups of 4 rows (256 bytes, all banks) form one row
// of 16 chunks, chunk (4 (ch & 3) + j) stored at position ^ keyT(ch).  The
// producer writes chunk j = row group of channels 8g + e (fixed e) and the
// consumer reads rows 32 rho + 8a + 4h + b; both sets of 16 lanes then hit
// 16 distinct positions.
__device__ __forceinline__ int keyT(int ch) { return ((ch >> 3) ^ (((ch >> 2) & 1) << 3)) & 15; }
__device__ __forceinline__ int idxT(int ch, int j) {
    return (ch >> 2) * (4 * C) + (((((ch & 3) << 2) | j) ^ keyT(ch)) << 3);
}

// Sticky error bits of this device (kda_device_error_bits in kda.h): set by
// a workgroup whose bounded wait ran out, read and cleared by the host.
__device__ unsigned int g_ws_error;
constexpr unsigned WS_ERR_WAIT_TIMEOUT = 1u;

__device__ __forceinline__ int ld_acquire(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Wait until *p >= target (or, with eq, *p == target).  Returns false when
// the workgroup is dead or the wait ran out (which kills the workgroup).
__device__ __forceinline__ bool wait_flag(const int *p, int target, bool eq, int *dead, int limit) {
    for (int it = 0; it < limit; ++it) {
        const int v = ld_acquire(p);
        if (eq ? (v == target) : (v >= target)) return true;
        if (__hip_atomic_load(dead, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return false;
        __builtin_amdgcn_s_sleep(1);
    }
    __hip_atomic_store(dead, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return false;
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Chunk row held by consumer accumulator tile h (0, 1) at tile row m: the
// 4 registers of a lane of tiles 0 and 1 are then its B-operand k-slots
// 8j..8j+7 of the next MFMA in natural order.
__device__ __forceinline__ int crow(int h, int m) { return 8 * (m >> 2) + 4 * h + (m & 3); }
// Key channel held by state tile (run rho, half h) at tile row m.
__device__ __forceinline__ int srow(int rho, int h, int m) { return 32 * rho + 8 * (m >> 2) + 4 * h + (m & 3); }

typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 (round to nearest even), two values per v_cvt_pk_bf16_f32
__device__ __forceinline__ bf16x8 pack8(const f32x4 lo, const f32x4 hi) {
    const f32x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_convertvector(v, bf16x8);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }

// Raw buffer resource over `base` (uniform): untyped 32-bit format, no
// stride, bounds = 2^31 - 16 bytes.  Accesses at offset OOB_OFF read as zero
// and drop stores, which lets masked rows go without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base) {
    // the address is the same in every lane; saying so keeps the resource in
    // scalar registers (otherwise each access becomes a loop over lanes)
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *u = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, 0, 0x7ffffff0, 0x00020000);
}
constexpr uint32_t OOB_OFF = 0x80000000u;
// The same over `bytes` bytes only: accesses past them read zero and drop
// their stores (the rows of a chunk past its end, with a window of the
// chunk's valid rows).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc_n(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *u = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, 0, bytes, 0x00020000);
}
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Sum over the 16 lanes of a row (lanes 16j .. 16j + 15), in every lane of it:
// pair swaps within quads, then the mirrors of 8 and 16 lanes.
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

// Row r and column i of pair number pidx of the lower triangle (i <= r),
// pairs numbered row by row.
__device__ __forceinline__ void tri_pair(int pidx, int &r, int &i) {
    int rr = (int)((sqrtf(8.0f * pidx + 1.0f) - 1.0f) * 0.5f);
    if ((rr + 1) * (rr + 2) / 2 <= pidx) ++rr;
    if (rr * (rr + 1) / 2 > pidx) --rr;
    r = rr;
    i = pidx - rr * (rr + 1) / 2;
}

}  // namespace ws

// Exact A and P for one 32-token chunk, entry by entry: A_ri = beta_r sum_c
// k_rc k_ic 2^(G_rc - G_ic) (i < r), P_ri = sum_c q_rc k_ic 2^(G_rc - G_ic)
// (i <= r), G the inclusive cumulative decay in log2 units.  The gate of
// (row r, channel c) is bg[r * gstride + c * gch]: gch = 0 for a gate shared
// by the channels of a head.  With PREP_SOFTPLUS the gate is the softplus
// input; with PREP_L2NORM k and q rows are scaled by pNorm (1/|k_r|, 1/|q_r|).  Channels are
// staged 32 at a time in the producer's private LDS region; lane l owns
// pairs l, l+64, ... of the 528 lower pairs.  Writes A^T (fp32, private) and
// P (bf16, slot).  Kept out of line: it runs only for chunks with extreme
// decay, and its registers stay out of the hot path's budget.
template <int DK>
__device__ __forceinline__ void exact_ap_body(int lane, int cl, uint32_t tokk, uint32_t gstride,
                                              uint32_t gch, int prep, const bf16_t *bg,
                                              const bf16_t *bk, const bf16_t *bq,
                                              unsigned char *priv, float *pAt, bf16_t *sP,
                                              const float *pBeta, const float *pNorm, float *gM,
                                              float *gP)
{
    using namespace ws;
    constexpr int CPL = DK / 64;
    constexpr int NPAIR = C * (C + 1) / 2;
    constexpr int PPL = (NPAIR + 63) / 64;
    constexpr int QCH = 32;                 // channels per stage
    constexpr int LPQ = QCH / CPL;          // lanes staging one stage's channels
    float resA[PPL], resP[PPL];
#pragma unroll
    for (int u = 0; u < PPL; ++u) { resA[u] = 0.0f; resP[u] = 0.0f; }
    float *stG = reinterpret_cast<float *>(priv);                     // [32][32] fp32
    bf16_t *stK = reinterpret_cast<bf16_t *>(priv + C * 32 * 4);       // [32][32]
    bf16_t *stQ = reinterpret_cast<bf16_t *>(priv + C * 32 * 4 + C * 32 * 2);
    for (int qd = 0; qd < DK / QCH; ++qd) {
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        if (lane / LPQ == qd) {
            float G[CPL];
#pragma unroll
            for (int e = 0; e < CPL; ++e) G[e] = 0.0f;
            for (int r = 0; r < C; ++r) {
                const uint32_t rr_ = (uint32_t)(r < cl ? r : cl - 1);
                const uint16_t m16 = r < cl ? 0xffffu : 0u;
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                    const int cq = CPL * (lane - qd * LPQ) + e;
                    const int c = QCH * qd + cq;
                    const uint32_t g1 = (uint32_t)(bg[rr_ * gstride + c * gch].x & m16);
                    float kf = bf_lo((uint32_t)(bk[rr_ * tokk + c].x & m16));
                    float qf = bf_lo((uint32_t)(bq[rr_ * tokk + c].x & m16));
                    if (prep & PREP_L2NORM) {
                        kf *= pNorm[r];
                        qf *= pNorm[C + r];
                    }
                    // rows past the end: alpha = 1
                    G[e] += r >= cl ? 0.0f
                          : (prep & PREP_SOFTPLUS) ? log2_alpha_softplus(bf_lo(g1))
                                                   : bf_lo(g1) * kLog2e;
                    stG[r * 32 + cq] = G[e];
                    stK[r * 32 + cq] = to_bf16(kf);
                    stQ[r * 32 + cq] = to_bf16(qf);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
        for (int u = 0; u < PPL; ++u) {
            const int pidx = lane + 64 * u;
            if (pidx < NPAIR) {
                int r, i;
                tri_pair(pidx, r, i);
                float sa = resA[u], sp = resP[u];
                for (int c = 0; c < 32; ++c) {
                    const float f = __builtin_amdgcn_exp2f(stG[r * 32 + c] - stG[i * 32 + c]);
                    const float kic = to_f32(stK[i * 32 + c]) * f;
                    sa += to_f32(stK[r * 32 + c]) * kic;
                    sp += to_f32(stQ[r * 32 + c]) * kic;
                }
                resA[u] = sa;
                resP[u] = sp;
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int u = 0; u < PPL; ++u) {
        const int pidx = lane + 64 * u;
        if (pidx < NPAIR) {
            int r, i;
            tri_pair(pidx, r, i);
            pAt[i * LA + r] = (i < r) ? resA[u] * pBeta[r] : 0.0f;
            sP[idx4(r, i)] = to_bf16(resP[u]);
            // for the backward (when asked): M0 and fp32 P, row-major
            if (gM) gM[r * C + i] = (i < r) ? resA[u] : 0.0f;
            if (gP) gP[r * C + i] = resP[u];
        }
    }
    // strict upper part of P
    for (int idx = lane; idx < C * C; idx += 64) {
        const int r = idx / C, i = idx % C;
        if (i > r) {
            sP[idx4(r, i)] = to_bf16(0.0f);
            if (gM) gM[idx] = 0.0f;
            if (gP) gP[idx] = 0.0f;
        }
    }
}
template <int DK>
__device__ __attribute__((noinline)) void exact_ap(int lane, int cl, uint32_t tokk,
                                                   uint32_t gstride, uint32_t gch, int prep,
                                                   const bf16_t *bg, const bf16_t *bk,
                                                   const bf16_t *bq, unsigned char *priv,
                                                   float *pAt, bf16_t *sP, const float *pBeta,
                                                   const float *pNorm)
{
    exact_ap_body<DK>(lane, cl, tokk, gstride, gch, prep, bg, bk, bq, priv, pAt, sP, pBeta, pNorm,
                      nullptr, nullptr);
}
// the same, also writing M0 and fp32 P for the backward (either may be NULL)
template <int DK>
__device__ __attribute__((noinline)) void exact_ap_save(int lane, int cl, uint32_t tokk,
                                                        uint32_t gstride, uint32_t gch,
                                                        const bf16_t *bg, const bf16_t *bk,
                                                        const bf16_t *bq, unsigned char *priv,
                                                        float *pAt, bf16_t *sP, const float *pBeta,
                                                        float *gM, float *gP)
{
    exact_ap_body<DK>(lane, cl, tokk, gstride, gch, 0, bg, bk, bq, priv, pAt, sP, pBeta, nullptr, gM, gP);
}

template <int DK, int NSTRIP, int GATE, int PREP, bool SAVE>
__global__ __launch_bounds__(512, 1) void chunked_ws_kernel(WsParams p)
{
    using namespace ws;
    using L = Lds<DK>;
    constexpr int NCL = DK / 16;        // key channels per producer lane
    constexpr int NRUN = DK / 32;       // 32-channel MFMA runs over d_k
    constexpr int NKT = DK / 16;        // state tiles over d_k
    constexpr int DVS = 64 * NSTRIP;

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];
    int *s_full = reinterpret_cast<int *>(smem + L::SYNC);
    int *s_freed = s_full + NSLOT;
    int *s_dead = s_full + 2 * NSLOT;

    // ---- work unit: XCD-aware (sequence, head, slice) ------------------------
    // Blocks b and b + 8 run on the same XCD (round-robin dispatch), so the
    // slices of one (sequence, head) are given ids 8 apart and share that
    // XCD's L2 for their common k / q / g reads.
    const int NS = p.nslices;
    const int bid = blockIdx.x;
    const int grp = bid / (8 * NS);
    const int xcd = bid & 7;
    const int slice = (bid >> 3) % NS;
    const int sh = grp * 8 + xcd;
    if (sh >= p.units) return;
    const int H = p.H, DV = p.DV;
    const int seq_rank = sh / H, head = sh - (sh / H) * H;
    const int seq = p.order ? p.order[seq_rank] : seq_rank;
    long t0, len;
    if (p.cu_seqlens) {
        t0 = p.cu_seqlens[seq];
        len = (long)p.cu_seqlens[seq + 1] - t0;
    } else {
        t0 = (long)seq * p.T;
        len = p.T;
    }
    const int nchunks = (int)((len + C - 1) / C);
    const int col0 = slice * DVS;
    const long strow = state_row(p.state_idx, p.pool, seq);
    // first workspace slot of the sequence (SAVE)
    const long sbase = !SAVE ? 0 : p.cu_seqlens ? t0 / C + seq : (long)seq * ((p.T + C - 1) / C);

    const int tid = threadIdx.x;
    // the wave index is uniform across a wave; say so, so that everything
    // derived from it (chunk ids, row bounds) lives in scalar registers
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, jg = lane >> 4, mr = lane & 15;

    const bf16_t *gq = static_cast<const bf16_t *>(p.q);
    const bf16_t *gk = static_cast<const bf16_t *>(p.k);
    const bf16_t *gv = static_cast<const bf16_t *>(p.v);
    const bf16_t *gg = static_cast<const bf16_t *>(p.g);
    const bf16_t *gb = static_cast<const bf16_t *>(p.beta);
    bf16_t *go = static_cast<bf16_t *>(p.o);

    if (tid < 2 * NSLOT + 1) s_full[tid] = 0;
    __syncthreads();

    if (w < 4) {
        // =========================== consumer ==================================
        const uint32_t tokv = (uint32_t)H * DV;
        f32x4 S[NSTRIP][NKT];
#pragma unroll
        for (int s = 0; s < NSTRIP; ++s)
#pragma unroll
            for (int tt = 0; tt < NKT; ++tt) S[s][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (p.S0 && strow >= 0) {
            const float *s0 = p.S0 + ((size_t)strow * H + head) * DK * DV + col0;
#pragma unroll
            for (int s = 0; s < NSTRIP; ++s) {
                const uint32_t co = 16 * (w + 4 * s) + mr;
#pragma unroll
                for (int tt = 0; tt < NKT; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S[s][tt][i] = s0[(uint32_t)srow(tt >> 1, tt & 1, 4 * jg + i) * DV + co];
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
        // v prefetch (raw bf16 bits) of the rows / columns this lane's tiles hold
        uint32_t rawv[NSTRIP][8];
        // byte offset of (chunk row 8 jg, this lane's column) from a chunk's
        // first v element; rows past the end read row 0 instead
        const uint32_t vlane = (uint32_t)(8 * jg) * tokv * 2u + (uint32_t)(16 * w + mr) * 2u;
        // Every load and store of v and o is issued on every chunk (rows past
        // the end go out of the buffer's bounds: zero / dropped), so the
        // number of memory operations in flight is fixed and the wait for
        // the v prefetch never has to include the o stores.
        auto load_v = [&](int n) {
            const long cs = (long)n * C;
            const int cl = (int)((len - cs) < C ? (len - cs) : C);
            // a window of the chunk's cl valid rows: rows past them read zero
            const __amdgpu_buffer_rsrc_t rv =
                buf_rsrc_n(gv + ((size_t)(t0 + cs) * H + head) * DV + col0, (uint32_t)cl * tokv * 2u);
#pragma unroll
            for (int s = 0; s < NSTRIP; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // the aligned 4-byte word holding this column (and its
                        // neighbour): the register is the load's own result
                        const uint32_t off = (vlane + (uint32_t)(4 * h + i) * tokv * 2u + 128u * s) & ~3u;
                        rawv[s][4 * h + i] = __builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, 0);
                    }
        };
        if (nchunks > 0) load_v(0);
        // the first chunk's v has landed before the loop, as it has at the end of
        // every iteration, so the loop head needs no wait on memory
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

        // After a wait ran out (the workgroup is dead): NaN into this wave's
        // columns of every output not yet produced, chunks n_from onwards, and
        // the device's error bit.  Runs only on that failure.
        auto give_up = [&](int n_from) {
            if (lane == 0) atomicOr(&g_ws_error, WS_ERR_WAIT_TIMEOUT);
            const float qnan = __builtin_nanf("");
            for (int m = n_from; m < nchunks; ++m) {
                const long cm = (long)m * C;
                const int cl = (int)((len - cm) < C ? (len - cm) : C);
#pragma unroll
                for (int s = 0; s < NSTRIP; ++s) {
                    const uint32_t co = 16 * (w + 4 * s) + mr;
                    if constexpr (!SAVE) {
                        bf16_t *ob = go + ((size_t)(t0 + cm) * H + head) * DV + col0;
                        for (int r = jg; r < cl; r += 4) ob[(size_t)r * tokv + co] = to_bf16(qnan);
                    } else {
                        const size_t slotm = (size_t)(sbase + m) * H + head;
                        for (int r = jg; r < DK; r += 4)
                            p.wS[slotm * DK * DV + strip_off(r, col0 + co, DK)] = to_bf16(qnan);
                        for (int r = jg; r < C; r += 4) {
                            p.wX[slotm * C * DV + strip_off(r, col0 + co, C)] = to_bf16(qnan);
                            p.wU[slotm * C * DV + strip_off(r, col0 + co, C)] = to_bf16(qnan);
                        }
                    }
                }
            }
            if (p.S_T && strow >= 0) {
                float *st = p.S_T + ((size_t)strow * H + head) * DK * DV + col0;
#pragma unroll
                for (int s = 0; s < NSTRIP; ++s) {
                    const uint32_t co = 16 * (w + 4 * s) + mr;
                    for (int r = jg; r < DK; r += 4) st[(uint32_t)r * DV + co] = qnan;
                }
            }
        };

        int dead_at = -1;
        for (int n = 0; n < nchunks; ++n) {
            const int slot = n % NSLOT;
            const long cs = (long)n * C;
            const int cl = (int)((len - cs) < C ? (len - cs) : C);
            // In a dead workgroup (a bounded wait ran out) every later wait
            // returns at once; the chunks are still walked, on whatever the
            // slots hold, and what was not produced is overwritten with NaN
            // after the loop.  (A loop with one exit keeps the state in place
            // from one chunk to the next.)
            if (!wait_flag(&s_full[slot], n + 1, true, s_dead, p.spin_limit) && dead_at < 0) dead_at = n;
            const unsigned char *sb = smem + slot * L::SLOT;
            const bf16_t *sKU = reinterpret_cast<const bf16_t *>(sb + L::KU);
            const bf16_t *sQU = reinterpret_cast<const bf16_t *>(sb + L::QU);
            const bf16_t *sKRt = reinterpret_cast<const bf16_t *>(sb + L::KRT);
            const bf16_t *sTp = reinterpret_cast<const bf16_t *>(sb + L::TP);
            const bf16_t *sP = reinterpret_cast<const bf16_t *>(sb + L::PM);
            const float *sG = reinterpret_cast<const float *>(sb + L::GM);
            // a window of the chunk's cl valid rows: stores past them are dropped
            const __amdgpu_buffer_rsrc_t ro =
                buf_rsrc_n(go + ((size_t)(t0 + cs) * H + head) * DV + col0, (uint32_t)cl * tokv * 2u);

            // v of this chunk out of the prefetch registers, which then take
            // the next chunk's loads at once (a whole chunk of latency slack).
            // Only the v loads must have landed, not the o stores issued after
            // them: vmcnt counts both, in order, so wait down to the 8 * NSTRIP
            // stores (without this the compiler waits for everything here); the
            // SAVE instantiation issues 8 per fragment of S, X and U instead
            // (the counter field holds at most 63)
            {
                constexpr int nst = SAVE ? (8 * NRUN + 16) * NSTRIP : 8 * NSTRIP;
                constexpr int vm = nst < 63 ? nst : 63;
                __builtin_amdgcn_s_waitcnt(0x0F70 | (vm & 15) | ((vm >> 4) << 14));
            }
            float xv[NSTRIP][8];
            const uint32_t vsh = (mr & 1) ? 0u : 16u;   // odd columns are the high half
#pragma unroll
            for (int s = 0; s < NSTRIP; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        xv[s][4 * h + i] = __uint_as_float((rawv[s][4 * h + i] << vsh) & 0xffff0000u);
            // unconditional (the last chunk reloads itself): a conditional
            // load leaves the registers with two definitions, which the compiler
            // resolves with copies that wait for every outstanding access
            load_v(n + 1 < nchunks ? n + 1 : n);

            // every operand fragment of the chunk, read at once (one LDS
            // round trip instead of one per MFMA stage); with two strips per
            // wave they are read per strip, as holding them for both strips
            // would exceed the register file
            bf16x8 fku[2][NRUN], fqu[2][NRUN], ftp[2], fpm[2], fkr[NKT];
            float4 fgm[NKT];
            auto read_frags = [&]() {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = crow(h, mr);
                    const int kr = keyK<DK>(row);
#pragma unroll
                    for (int rr = 0; rr < NRUN; ++rr) {
                        const int off = row * DK + (((4 * rr + jg) ^ kr) << 3);
                        fku[h][rr] = *reinterpret_cast<const bf16x8 *>(&sKU[off]);
                        if constexpr (!SAVE) fqu[h][rr] = *reinterpret_cast<const bf16x8 *>(&sQU[off]);
                    }
                    ftp[h] = *reinterpret_cast<const bf16x8 *>(&sTp[row * C + ((jg ^ key4(row)) << 3)]);
                    if constexpr (!SAVE) fpm[h] = *reinterpret_cast<const bf16x8 *>(&sP[row * C + ((jg ^ key4(row)) << 3)]);
                }
            };
            auto read_kr = [&]() {
#pragma unroll
                for (int tt = 0; tt < NKT; ++tt) {
                    const int rho = tt >> 1, h = tt & 1;
                    fgm[tt] = *reinterpret_cast<const float4 *>(&sG[srow(rho, h, 4 * jg)]);
                    fkr[tt] = *reinterpret_cast<const bf16x8 *>(&sKRt[idxT(srow(rho, h, mr), jg)]);
                }
            };
            if constexpr (NSTRIP == 1) {
                read_frags();
                read_kr();
            }

#pragma unroll
            for (int s = 0; s < NSTRIP; ++s) {
                if constexpr (NSTRIP > 1) {
                    // a compiler barrier, so the second strip's reads are not
                    // merged with the first's (which would keep both live)
                    asm volatile("" ::: "memory");
                }
                bf16x8 sf[NRUN];
#pragma unroll
                for (int rr = 0; rr < NRUN; ++rr) sf[rr] = pack8(S[s][2 * rr], S[s][2 * rr + 1]);
                // the lane's bf16 values of a [rows][d_v] array in the backward
                // workspace's 16-column strips, element e of a fragment being
                // row r0 + e of column 16 (w + 4 s) + mr: rows r0 .. r0 + 3 and
                // r0 + 4 .. r0 + 7 regrouped within each quad of lanes, so that
                // each of the two stores writes whole 128-byte lines
                auto save_col = [&](bf16_t *base, uint32_t rows, const bf16x8 &f, uint32_t r0) {
                    const __amdgpu_buffer_rsrc_t rs =
                        buf_rsrc(base + ((size_t)(sbase + n) * H + head) * rows * DV +
                                 strip_off(0, col0 + 16 * (w + 4 * s), rows));
                    // the fragment as four words, element e the half e & 1 of word e / 2
                    // (element-wise bit casts of the bf16 vector do not survive here)
                    const uint4 fw = __builtin_bit_cast(uint4, f);
#pragma unroll
                    for (int g = 0; g < 2; ++g)
                        __builtin_amdgcn_raw_buffer_store_b64(
                            quad_rows(g ? fw.z : fw.x, g ? fw.w : fw.y, mr), rs,
                            ((r0 + 4u * g + (uint32_t)quad_row(mr)) * 16u + (uint32_t)(mr & ~3)) * 2u, 0, kStreamStore);
                };
                if constexpr (SAVE) {
                    // S entering the chunk: fragment rr holds rows 32 rr + 8 jg + e
#pragma unroll
                    for (int rr = 0; rr < NRUN; ++rr) save_col(p.wS, DK, sf[rr], 32 * rr + 8 * jg);
                }
                if constexpr (NSTRIP > 1) read_frags();
                // the decay of the old state does not wait for the chain below
                if constexpr (NSTRIP == 1) {
#pragma unroll
                    for (int tt = 0; tt < NKT; ++tt) {
                        S[s][tt][0] *= fgm[tt].x;
                        S[s][tt][1] *= fgm[tt].y;
                        S[s][tt][2] *= fgm[tt].z;
                        S[s][tt][3] *= fgm[tt].w;
                    }
                }
                // X = V - K_up S (the slot holds -K_up), O = Q_up S
                f32x4 X[2], O[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        X[h][i] = xv[s][4 * h + i];
                        O[h][i] = 0.0f;
                    }
#pragma unroll
                for (int rr = 0; rr < NRUN; ++rr)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        X[h] = mfma_bf16(fku[h][rr], sf[rr], X[h]);
                        if constexpr (!SAVE) O[h] = mfma_bf16(fqu[h][rr], sf[rr], O[h]);
                    }
                // U = T' X
                const bf16x8 xf = pack8(X[0], X[1]);
                // chunk rows 8 jg + e (crow): X and U to the workspace
                if constexpr (SAVE) save_col(p.wX, C, xf, 8 * jg);
                f32x4 U[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) U[h] = mfma_bf16(ftp[h], xf, f32x4{0.f, 0.f, 0.f, 0.f});
                const bf16x8 uf = pack8(U[0], U[1]);
                if constexpr (SAVE) save_col(p.wU, C, uf, 8 * jg);
                // S = Diag(gamma) S + K_right^T U;  O += P U
                if constexpr (NSTRIP > 1) {
#pragma unroll
                    for (int tt = 0; tt < NKT; ++tt) {
                        const int rho = tt >> 1, h = tt & 1;
                        const float4 gm = *reinterpret_cast<const float4 *>(&sG[srow(rho, h, 4 * jg)]);
                        S[s][tt][0] *= gm.x;
                        S[s][tt][1] *= gm.y;
                        S[s][tt][2] *= gm.z;
                        S[s][tt][3] *= gm.w;
                        const bf16x8 fa = *reinterpret_cast<const bf16x8 *>(&sKRt[idxT(srow(rho, h, mr), jg)]);
                        S[s][tt] = mfma_bf16(fa, uf, S[s][tt]);
                    }
                } else {
#pragma unroll
                    for (int tt = 0; tt < NKT; ++tt) S[s][tt] = mfma_bf16(fkr[tt], uf, S[s][tt]);
                }
                if constexpr (!SAVE) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) O[h] = mfma_bf16(fpm[h], uf, O[h]);
                    // store O
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t off = vlane + (uint32_t)(4 * h + i) * tokv * 2u + 128u * s;
                            __builtin_amdgcn_raw_buffer_store_b16(to_bf16(O[h][i]).x, ro, off, 0, 0);
                        }
                }
            }
            // all reads of the slot are done once their values were consumed
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            if (lane == 0)
                __hip_atomic_fetch_add(&s_freed[slot], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }

        if (dead_at >= 0) {
            give_up(dead_at);
            return;
        }
        if (p.S_T && strow >= 0) {
            float *st = p.S_T + ((size_t)strow * H + head) * DK * DV + col0;
#pragma unroll
            for (int s = 0; s < NSTRIP; ++s) {
                const uint32_t co = 16 * (w + 4 * s) + mr;
#pragma unroll
                for (int tt = 0; tt < NKT; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        st[(uint32_t)srow(tt >> 1, tt & 1, 4 * jg + i) * DV + co] = S[s][tt][i];
            }
        }
        return;
    }

    // =============================== producer ==================================
    const int pw = w - 4;
    unsigned char *priv = smem + L::PRIV_BASE + pw * L::PRIV;
    bf16_t *pKD = reinterpret_cast<bf16_t *>(priv + L::P_KD);
    float *pAt = reinterpret_cast<float *>(priv + L::P_AT);
    float *pT = reinterpret_cast<float *>(priv + L::P_T);
    float *pBeta = reinterpret_cast<float *>(priv + L::P_BETA);
    float *pNorm = reinterpret_cast<float *>(priv + L::P_NORM);
    const uint32_t tokk = (uint32_t)H * DK;

    // Raw g and k of one chunk, lane (cg, rg) = (lane & 15, lane >> 4)
    // holding channels NCL*cg .. +NCL-1 of rows 8*rg .. 8*rg+7 (one 16- or
    // 8-byte load per row and tensor), and beta of row `lane`.  Rows past the
    // chunk end read row 0 (always in bounds) and are masked where used.
    // A producer requests its next chunk's g and k while it still finishes
    // the current one, which hides their latency.  A per-head gate (gh) is
    // one value per row, laid out like beta; without a gate nothing is read.
    uint32_t gx[8][NCL / 2], gh[8], kx[8][NCL / 2], bx;
    auto load_gk = [&](int n) {
        // the row offsets below are recomputed per chunk from an opaque copy
        // of the lane id instead of being hoisted out of the loop
        int lane_o = tid & 63;
        asm volatile("" : "+v"(lane_o));
        const int lane = lane_o, cg = lane & 15, rg = lane >> 4;
        const int c0 = NCL * cg, r0 = 8 * rg;
        const long cs = (long)n * C;
        const int cl = (int)((len - cs) < C ? (len - cs) : C);
        const size_t tb = (size_t)(t0 + cs) * H + head;
        // windows of the chunk's cl valid rows: rows past them read zero
        // (the decay step below still sets what such rows must hold)
        const uint32_t wbytes = (uint32_t)cl * tokk * 2u;
        const __amdgpu_buffer_rsrc_t rg_ = buf_rsrc_n(gg + (GATE == GATE_CHANNEL ? tb * DK : 0), wbytes);
        const __amdgpu_buffer_rsrc_t rk_ = buf_rsrc_n(gk + tb * DK, wbytes);
        const uint32_t base_off = ((uint32_t)r0 * tokk + (uint32_t)c0) * 2u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t off = base_off + (uint32_t)i * tokk * 2u;
            if constexpr (NCL == 8) {
                if constexpr (GATE == GATE_CHANNEL) {
                    const uint4 g4 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rg_, off, 0, 0));
                    gx[i][0] = g4.x; gx[i][1] = g4.y; gx[i][2] = g4.z; gx[i][3] = g4.w;
                }
                const uint4 k4 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk_, off, 0, 0));
                kx[i][0] = k4.x; kx[i][1] = k4.y; kx[i][2] = k4.z; kx[i][3] = k4.w;
            } else {
                if constexpr (GATE == GATE_CHANNEL) {
                    const uint2 g2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rg_, off, 0, 0));
                    gx[i][0] = g2.x; gx[i][1] = g2.y;
                }
                const uint2 k2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk_, off, 0, 0));
                kx[i][0] = k2.x; kx[i][1] = k2.y;
            }
            if constexpr (GATE == GATE_HEAD)
                gh[i] = (uint32_t)gg[tb + (size_t)(r0 + i < cl ? r0 + i : 0) * H].x;
        }
        const int rb = lane & (C - 1);
        bx = (uint32_t)gb[tb + (size_t)(rb < cl ? rb : cl - 1) * H].x;
    };
    if (pw < nchunks) load_gk(pw);

    for (int n = pw; n < nchunks; n += NPROD) {
        // Lane-derived LDS offsets are recomputed per chunk (a few cheap ops)
        // instead of being hoisted out of the loop and kept live, which would
        // take registers the chunk's working set needs.
        int lane_o = tid & 63;
        asm volatile("" : "+v"(lane_o));
        const int lane = lane_o, jg = lane_o >> 4, mr = lane_o & 15;
        const int slot = pw;                   // n % NSLOT
        const long cs = (long)n * C;
        const int cl = (int)((len - cs) < C ? (len - cs) : C);
        const size_t tb = (size_t)(t0 + cs) * H + head;
        const bf16_t *bg = gg + tb * DK, *bk = gk + tb * DK, *bq = gq + tb * DK;

        // ---- loads ---------------------------------------------------------------
        // g and k of this chunk were requested at the end of the producer's
        // previous chunk; q (first needed after the decay products) now.
        const int cg = lane & 15, rg = lane >> 4;
        const int c0 = NCL * cg, r0 = 8 * rg;
        uint32_t qx[8][NCL / 2];
        {
            const uint32_t base_off = ((uint32_t)r0 * tokk + (uint32_t)c0) * 2u;
            const __amdgpu_buffer_rsrc_t rq_ = buf_rsrc_n(bq, (uint32_t)cl * tokk * 2u);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t off = base_off + (uint32_t)i * tokk * 2u;
                if constexpr (NCL == 8) {
                    const uint4 q4 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq_, off, 0, 0));
                    qx[i][0] = q4.x; qx[i][1] = q4.y; qx[i][2] = q4.z; qx[i][3] = q4.w;
                } else {
                    const uint2 q2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq_, off, 0, 0));
                    qx[i][0] = q2.x; qx[i][1] = q2.y;
                }
            }
        }

        // ---- decay ---------------------------------------------------------------
        if (r0 + 8 > cl) {
            // rows past the chunk end: alpha = 1 (g = 0, or a softplus input
            // of -inf), k = q = 0
            constexpr uint32_t g0 = (PREP & PREP_SOFTPLUS) ? 0xff80ff80u : 0u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t m = (r0 + i) < cl ? 0xffffffffu : 0u;
#pragma unroll
                for (int d = 0; d < NCL / 2; ++d) {
                    if constexpr (GATE == GATE_CHANNEL) gx[i][d] = (gx[i][d] & m) | (g0 & ~m);
                    kx[i][d] &= m;
                    qx[i][d] &= m;
                }
                if constexpr (GATE == GATE_HEAD) gh[i] = (gh[i] & m) | (g0 & 0xffffu & ~m);
            }
        }
        // L2 normalisation of k and q rows: sums of squares over this lane's
        // channels, then over the 16 lanes that hold the row, one row at a
        // time where the forward pass below first needs it.  The factors also
        // go to this wave's LDS area, from which the reverse pass and the
        // exact path read them back row by row, so that none stays live in a
        // register through the decay work.
        auto row_norm = [&](const uint32_t (&x)[NCL / 2]) -> float {
            float ss = 0.0f;
#pragma unroll
            for (int d = 0; d < NCL / 2; ++d) {
                const float a = bf_lo(x[d]), b = bf_hi(x[d]);
                ss += a * a + b * b;
            }
            return inv_norm(row16_sum(ss));
        };
        // norm factor of row r0 + i of k (q: at C + r0 + i); 1 without
        auto nscale = [&](int at) -> float {
            // a volatile read is neither hoisted nor merged with its neighbours
            if constexpr (PREP & PREP_L2NORM) return *static_cast<volatile const float *>(pNorm + at);
            else {
                return 1.0f;
            }
        };
        // alpha of a gate value: e^g, or e^{-softplus(x)}
        auto alpha_of = [](float gv) -> float {
            if constexpr (PREP & PREP_SOFTPLUS) return alpha_softplus(gv);
            else return __builtin_amdgcn_exp2f(gv * kLog2e);
        };
        // Decay factors.  Per key channel: alpha of each (row, channel) and the
        // products over this lane's 8 rows (tot); for a per-head gate the same
        // per row (alh, toth); none without a gate (alpha = 1).
        float al[8][NCL], tot[NCL], alh[8], toth = 1.0f;
        // largest |k| bit pattern per bf16 half (monotonic in |k|)
        uint32_t kbits = 0;
        if constexpr (GATE != GATE_NONE) {
#pragma unroll
            for (int e = 0; e < NCL; ++e) tot[e] = 1.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if constexpr (GATE == GATE_HEAD) {
                    alh[i] = alpha_of(bf_lo(gh[i]));
                    toth *= alh[i];
                }
#pragma unroll
                for (int d = 0; d < NCL / 2; ++d) {
                    if constexpr (GATE == GATE_CHANNEL) {
                        al[i][2 * d] = alpha_of(bf_lo(gx[i][d]));
                        al[i][2 * d + 1] = alpha_of(bf_hi(gx[i][d]));
                        tot[2 * d] *= al[i][2 * d];
                        tot[2 * d + 1] *= al[i][2 * d + 1];
                    }
                    kbits = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
                        __builtin_bit_cast(u16x2, kbits), __builtin_bit_cast(u16x2, kx[i][d] & 0x7fff7fffu)));
                }
            }
        }
        // exclusive prefix / suffix products over the 4 row groups (the 16-lane
        // rows of the wave), so that
        //   E_r = pre * prod_{j <= r, j in group} alpha_j,
        //   R_r = post * prod_{j > r, j in group} alpha_j,
        //   gamma = pre * tot * post.
        // A two-step butterfly on the VALU: v_permlane16_swap gives every row
        // the value of row r ^ 1, v_permlane32_swap the pair product of rows
        // r ^ 2 and r ^ 3 (all lanes take part in both).
        float pre[NCL], post[NCL], gam[NCL], preh = 1.0f, posth = 1.0f, gamh = 1.0f;
        if constexpr (GATE != GATE_NONE) {
            auto scan = [&](float tv, float &pr, float &po) {
                const uint32_t u = __float_as_uint(tv);
                // with both operands u: result[0] holds row r - 1 on odd rows,
                // result[1] row r + 1 on even rows
                const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
                const float p1 = __uint_as_float((rg & 1) ? a[0] : a[1]);
                const uint32_t pu = __float_as_uint(tv * p1);     // v_{2m} v_{2m+1}
                // result[0] holds the lower pair on rows 2, 3; result[1] the upper on rows 0, 1
                const auto b = __builtin_amdgcn_permlane32_swap(pu, pu, false, false);
                const float p2 = __uint_as_float(rg >= 2 ? b[0] : b[1]);
                const float pre1 = (rg & 1) ? p1 : 1.0f, post1 = (rg & 1) ? 1.0f : p1;
                pr = rg >= 2 ? pre1 * p2 : pre1;
                po = rg >= 2 ? post1 : post1 * p2;
            };
            if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
                for (int e = 0; e < NCL; ++e) {
                    scan(tot[e], pre[e], post[e]);
                    gam[e] = pre[e] * tot[e] * post[e];
                }
            } else {
                scan(toth, preh, posth);
                gamh = preh * toth * posth;
            }
        }
        // K_dn stays below 2^116 when gamma >= 2^-100 and |k| <= 2^16 (always,
        // for normalised k); with no gate K_dn = K and the fast path always holds
        bool ok = true;
        if constexpr (GATE != GATE_NONE) {
            if constexpr (!(PREP & PREP_L2NORM))
                ok = (kbits & 0xffffu) <= 0x4780u && (kbits >> 16) <= 0x4780u;   // 0x4780: 2^16
            if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
                for (int e = 0; e < NCL; ++e) ok = ok && (gam[e] >= 7.888609052210118e-31f);
            } else {
                ok = ok && (gamh >= 7.888609052210118e-31f);
            }
        }

        // wait for the slot: the consumers are done with chunk n - NSLOT
        if (n >= NSLOT) {
            if (!wait_flag(&s_freed[slot], 4 * (n / NSLOT), false, s_dead, p.spin_limit)) break;
        }
        if (lane < C) pBeta[lane] = lane < cl ? __uint_as_float(bx << 16) : 0.0f;
        unsigned char *sb = smem + slot * L::SLOT;
        bf16_t *sKU = reinterpret_cast<bf16_t *>(sb + L::KU);
        bf16_t *sQU = reinterpret_cast<bf16_t *>(sb + L::QU);
        bf16_t *sKRt = reinterpret_cast<bf16_t *>(sb + L::KRT);
        bf16_t *sTp = reinterpret_cast<bf16_t *>(sb + L::TP);
        bf16_t *sP = reinterpret_cast<bf16_t *>(sb + L::PM);
        float *sG = reinterpret_cast<float *>(sb + L::GM);
        if (rg == 0) {
#pragma unroll
            for (int e = 0; e < NCL; e += 4) {
                float4 g4;
                if constexpr (GATE == GATE_CHANNEL) g4 = make_float4(gam[e], gam[e + 1], gam[e + 2], gam[e + 3]);
                else g4 = make_float4(gamh, gamh, gamh, gamh);   // 1 without a gate
                *reinterpret_cast<float4 *>(&sG[c0 + e]) = g4;
            }
        }

        // forward: -K_up, Q_up rows
        {
            float E[NCL], Eh = preh;
#pragma unroll
            for (int e = 0; e < NCL; ++e) E[e] = pre[e];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t ku[NCL / 2], qu[NCL / 2];
                if constexpr (GATE == GATE_HEAD) Eh *= alh[i];
                float sk = 1.0f, sq = 1.0f;
                if constexpr (PREP & PREP_L2NORM) {
                    sk = row_norm(kx[i]);
                    sq = row_norm(qx[i]);
                    if (cg == 0) {
                        pNorm[r0 + i] = sk;
                        pNorm[C + r0 + i] = sq;
                    }
                }
#pragma unroll
                for (int d = 0; d < NCL / 2; ++d) {
                    if constexpr (GATE == GATE_CHANNEL) {
                        E[2 * d] *= al[i][2 * d];
                        E[2 * d + 1] *= al[i][2 * d + 1];
                        ku[d] = pack2(-bf_lo(kx[i][d]) * (E[2 * d] * sk), -bf_hi(kx[i][d]) * (E[2 * d + 1] * sk));
                        qu[d] = pack2(bf_lo(qx[i][d]) * (E[2 * d] * sq), bf_hi(qx[i][d]) * (E[2 * d + 1] * sq));
                    } else if constexpr (GATE == GATE_HEAD || (PREP & PREP_L2NORM)) {
                        const float ek = Eh * sk, eq = Eh * sq;   // Eh = 1 without a gate
                        ku[d] = pack2(-bf_lo(kx[i][d]) * ek, -bf_hi(kx[i][d]) * ek);
                        qu[d] = pack2(bf_lo(qx[i][d]) * eq, bf_hi(qx[i][d]) * eq);
                    } else {
                        // E = 1: the inputs themselves, K negated by its sign bits
                        ku[d] = kx[i][d] ^ 0x80008000u;
                        qu[d] = qx[i][d];
                    }
                }
                const int o = idxK<DK>(r0 + i, c0);
                if constexpr (NCL == 8) {
                    *reinterpret_cast<uint4 *>(&sKU[o]) = make_uint4(ku[0], ku[1], ku[2], ku[3]);
                    *reinterpret_cast<uint4 *>(&sQU[o]) = make_uint4(qu[0], qu[1], qu[2], qu[3]);
                } else {
                    *reinterpret_cast<uint2 *>(&sKU[o]) = make_uint2(ku[0], ku[1]);
                    *reinterpret_cast<uint2 *>(&sQU[o]) = make_uint2(qu[0], qu[1]);
                }
            }
        }
        // reverse: K_right (rows of K_right^T, 8 tokens per channel) and K_dn rows
        if constexpr (GATE != GATE_NONE || (PREP & PREP_L2NORM)) {
            float R[NCL], invg[NCL], kr[8][NCL], Rh = posth;
            const float invgh = __builtin_amdgcn_rcpf(gamh);
#pragma unroll
            for (int e = 0; e < NCL; ++e) {
                R[e] = post[e];
                if constexpr (GATE == GATE_CHANNEL) invg[e] = __builtin_amdgcn_rcpf(gam[e]);
            }
#pragma unroll
            for (int i = 7; i >= 0; --i) {
                uint32_t kd[NCL / 2];
                const float sk = nscale(r0 + i);
#pragma unroll
                for (int d = 0; d < NCL / 2; ++d) {
                    if constexpr (GATE == GATE_CHANNEL) {
                        kr[i][2 * d] = bf_lo(kx[i][d]) * (R[2 * d] * sk);
                        kr[i][2 * d + 1] = bf_hi(kx[i][d]) * (R[2 * d + 1] * sk);
                        R[2 * d] *= al[i][2 * d];
                        R[2 * d + 1] *= al[i][2 * d + 1];
                        kd[d] = pack2(kr[i][2 * d] * invg[2 * d], kr[i][2 * d + 1] * invg[2 * d + 1]);
                    } else {
                        // a per-head gate, or none (Rh = gamma = 1)
                        const float rk = Rh * sk;
                        kr[i][2 * d] = bf_lo(kx[i][d]) * rk;
                        kr[i][2 * d + 1] = bf_hi(kx[i][d]) * rk;
                        kd[d] = pack2(kr[i][2 * d] * invgh, kr[i][2 * d + 1] * invgh);
                    }
                }
                if constexpr (GATE == GATE_HEAD) Rh *= alh[i];
                const int o = idxK<DK>(r0 + i, c0);
                if constexpr (NCL == 8)
                    *reinterpret_cast<uint4 *>(&pKD[o]) = make_uint4(kd[0], kd[1], kd[2], kd[3]);
                else
                    *reinterpret_cast<uint2 *>(&pKD[o]) = make_uint2(kd[0], kd[1]);
            }
#pragma unroll
            for (int e = 0; e < NCL; ++e) {
                const int ch = c0 + e;
                *reinterpret_cast<uint4 *>(&sKRt[idxT(ch, rg)]) =
                    make_uint4(pack2(kr[0][e], kr[1][e]), pack2(kr[2][e], kr[3][e]),
                               pack2(kr[4][e], kr[5][e]), pack2(kr[6][e], kr[7][e]));
            }
        } else {
            // R = gamma = 1: K_dn rows are K's rows, and K_right^T takes the
            // bf16 halves of pairs of rows
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int o = idxK<DK>(r0 + i, c0);
                if constexpr (NCL == 8)
                    *reinterpret_cast<uint4 *>(&pKD[o]) = make_uint4(kx[i][0], kx[i][1], kx[i][2], kx[i][3]);
                else
                    *reinterpret_cast<uint2 *>(&pKD[o]) = make_uint2(kx[i][0], kx[i][1]);
            }
#pragma unroll
            for (int e = 0; e < NCL; ++e) {
                const int d = e >> 1;
                // channel e of rows a (low half) and b (high half)
                auto pr = [&](int a, int b) {
                    return (e & 1) ? ((kx[a][d] >> 16) | (kx[b][d] & 0xffff0000u))
                                   : ((kx[a][d] & 0xffffu) | (kx[b][d] << 16));
                };
                *reinterpret_cast<uint4 *>(&sKRt[idxT(c0 + e, rg)]) =
                    make_uint4(pr(0, 1), pr(2, 3), pr(4, 5), pr(6, 7));
            }
        }
        const bool fast = __builtin_amdgcn_ballot_w64(!ok) == 0;
        // SAVE: the backward's own test for its exact path, some channel
        // decaying by more than 2^64 over the chunk
        bool flag64 = false;
        if constexpr (SAVE && GATE != GATE_NONE) {
            bool big = false;
            if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
                for (int e = 0; e < NCL; ++e) big = big || !(gam[e] >= 5.421010862427522e-20f);
            } else {
                big = !(gamh >= 5.421010862427522e-20f);
            }
            flag64 = __builtin_amdgcn_ballot_w64(big) != 0;
        }
        // the workspace of this chunk (SAVE; written by slice 0 only)
        const size_t wcc = ((size_t)(sbase + n) * H + head) * C * C;
        const bool keep = SAVE && slice == 0;
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

        // ---- A and P -----------------------------------------------------------
        // A^T fp32 into the private region (over K_dn, once it has been read),
        // P bf16 into the slot
        if (fast) {
            f32x4 accA[3], accP[3];
            // the operand fragments of both row blocks, each read once
            // (the three tiles share them)
            bf16x8 fk[2][NRUN], fq[2][NRUN], fd[2][NRUN];
#pragma unroll
            for (int R = 0; R < 2; ++R) {
                const int ra = 16 * R + mr;
#pragma unroll
                for (int rr = 0; rr < NRUN; ++rr) {
                    const int ka = ra * DK + (((4 * rr + jg) ^ keyK<DK>(ra)) << 3);
                    fk[R][rr] = *reinterpret_cast<const bf16x8 *>(&sKU[ka]);
                    fq[R][rr] = *reinterpret_cast<const bf16x8 *>(&sQU[ka]);
                    fd[R][rr] = *reinterpret_cast<const bf16x8 *>(&pKD[ka]);
                }
            }
            // tiles (R, I) = (0,0), (1,0), (1,1)
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const int R = (t == 0) ? 0 : 1, I = (t == 2) ? 1 : 0;
                f32x4 a = {0.f, 0.f, 0.f, 0.f}, q = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int rr = 0; rr < NRUN; ++rr) {
                    a = mfma_bf16(fk[R][rr], fd[I][rr], a);
                    // P^T tile: lane ends up with P[16R + mr][16I + 4jg + i]
                    q = mfma_bf16(fd[I][rr], fq[R][rr], q);
                }
                accA[t] = a;
                accP[t] = q;
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            // accA: lane holds A' rows 16R + 4jg + i of column 16I + mr;
            // accP: P row 16R + mr, columns 16I + 4jg + i
            const float4 b4_0 = *reinterpret_cast<const float4 *>(&pBeta[4 * jg]);
            const float4 b4_1 = *reinterpret_cast<const float4 *>(&pBeta[16 + 4 * jg]);
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const int R = (t == 0) ? 0 : 1, I = (t == 2) ? 1 : 0;
                const float4 b4 = R ? b4_1 : b4_0;
                const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
                float a4[4], p4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // the slot's K_up is negated: A = -beta (K_up' K_dn^T)
                    a4[i] = (16 * I + mr < 16 * R + 4 * jg + i) ? -accA[t][i] * bb[i] : 0.0f;
                    p4[i] = (16 * I + 4 * jg + i <= 16 * R + mr) ? accP[t][i] : 0.0f;
                }
                *reinterpret_cast<float4 *>(&pAt[(16 * I + mr) * LA + 16 * R + 4 * jg]) =
                    make_float4(a4[0], a4[1], a4[2], a4[3]);
                *reinterpret_cast<uint2 *>(&sP[idx4(16 * R + mr, 16 * I + 4 * jg)]) =
                    make_uint2(pack2(p4[0], p4[1]), pack2(p4[2], p4[3]));
            }
            // upper block (0,1) of P is zero
            *reinterpret_cast<uint2 *>(&sP[idx4(mr, 16 + 4 * jg)]) = make_uint2(0u, 0u);
            if (keep) {
                // M0 (accA is -M0: the slot's K_up is negated), and P when flagged
                float *gM = p.wM + wcc;
#pragma unroll
                for (int t = 0; t < 3; ++t) {
                    const int R = (t == 0) ? 0 : 1, I = (t == 2) ? 1 : 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * R + 4 * jg + i, col = 16 * I + mr;
                        gM[row * C + col] = col < row ? -accA[t][i] : 0.0f;
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) gM[(4 * jg + i) * C + 16 + mr] = 0.0f;
                if (flag64) {
                    float *gP = p.wP + wcc;
#pragma unroll
                    for (int t = 0; t < 3; ++t) {
                        const int R = (t == 0) ? 0 : 1, I = (t == 2) ? 1 : 0;
                        const int row = 16 * R + mr, c0 = 16 * I + 4 * jg;
                        *reinterpret_cast<float4 *>(&gP[row * C + c0]) =
                            make_float4(c0 <= row ? accP[t][0] : 0.0f, c0 + 1 <= row ? accP[t][1] : 0.0f,
                                        c0 + 2 <= row ? accP[t][2] : 0.0f, c0 + 3 <= row ? accP[t][3] : 0.0f);
                    }
                    *reinterpret_cast<float4 *>(&gP[mr * C + 16 + 4 * jg]) = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
        } else {
            // exact path for chunks whose decay leaves the range of K_dn
            if constexpr (SAVE) {
                // (no input preparation in this instantiation)
                float *gM = keep ? p.wM + wcc : nullptr;
                float *gP = keep && flag64 ? p.wP + wcc : nullptr;
                if constexpr (GATE == GATE_CHANNEL)
                    exact_ap_save<DK>(lane, cl, tokk, tokk, 1u, bg, bk, bq, priv, pAt, sP, pBeta, gM, gP);
                else if constexpr (GATE == GATE_HEAD)
                    exact_ap_save<DK>(lane, cl, tokk, (uint32_t)H, 0u, gg + tb, bk, bq, priv, pAt, sP, pBeta,
                                      gM, gP);
            } else {
                if constexpr (GATE == GATE_CHANNEL)
                    exact_ap<DK>(lane, cl, tokk, tokk, 1u, PREP, bg, bk, bq, priv, pAt, sP, pBeta, pNorm);
                else if constexpr (GATE == GATE_HEAD)
                    exact_ap<DK>(lane, cl, tokk, (uint32_t)H, 0u, PREP, gg + tb, bk, bq, priv, pAt, sP, pBeta,
                                 pNorm);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

        // ---- T = (I + A)^{-1}; T' = T Diag(beta) into the slot ----------------
        {
            // diagonal blocks: lanes with jg & 1 == b solve block b for column
            // mr, right-looking: once t_i is final every later row subtracts
            // A[r][i] t_i, column i of A being row i of A^T (one broadcast read)
            const int blk = jg & 1;
            const float *ab = &pAt[(16 * blk) * LA + 16 * blk];
            // the identity column is rebuilt each chunk (16 selects) rather
            // than kept live across the loop in 16 registers
            int col = mr;
            asm volatile("" : "+v"(col));
            float acc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = (r == col) ? 1.0f : 0.0f;
            // rows i0 .. i0 + 4 of A^T: their needed groups read first, then
            // the five elimination steps
            auto steps = [&](auto i0c) {
                constexpr int i0 = decltype(i0c)::value;
                // keeps the compiler from hoisting every batch's reads to the
                // top, which would need all 36 float4 at once
                asm volatile("" ::: "memory");
                float4 arow[5][4];
#pragma unroll
                for (int ii = 0; ii < 5; ++ii)
#pragma unroll
                    for (int g4 = (i0 + ii + 1) >> 2; g4 < 4; ++g4)
                        arow[ii][g4] = *reinterpret_cast<const float4 *>(ab + (i0 + ii) * LA + 4 * g4);
#pragma unroll
                for (int ii = 0; ii < 5; ++ii) {
                    const int i = i0 + ii;
                    const float ti = acc[i];
#pragma unroll
                    for (int r = i + 1; r < 16; ++r) {
                        const float4 a4 = arow[ii][r >> 2];
                        const float a = (r & 3) == 0 ? a4.x : (r & 3) == 1 ? a4.y : (r & 3) == 2 ? a4.z : a4.w;
                        acc[r] -= a * ti;
                    }
                }
            };
            steps(std::integral_constant<int, 0>{});
            steps(std::integral_constant<int, 5>{});
            steps(std::integral_constant<int, 10>{});
            if (jg < 2) {
#pragma unroll
                for (int r = 0; r < 16; ++r) pT[(16 * blk + r) * LA + 16 * blk + mr] = acc[r];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        {
            // T[1,0] = -T[1,1] (A[1,0] T[0,0]) on fp32 MFMA (k = 4 jg + s per step)
            f32x4 Mx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                Mx = mfma_f32(pAt[(4 * jg + s) * LA + 16 + mr], pT[(4 * jg + s) * LA + mr], Mx);
            const float4 t11 = *reinterpret_cast<const float4 *>(&pT[(16 + mr) * LA + 16 + 4 * jg]);
            f32x4 Tx = {0.f, 0.f, 0.f, 0.f};
            Tx = mfma_f32(t11.x, Mx[0], Tx);
            Tx = mfma_f32(t11.y, Mx[1], Tx);
            Tx = mfma_f32(t11.z, Mx[2], Tx);
            Tx = mfma_f32(t11.w, Mx[3], Tx);
#pragma unroll
            for (int i = 0; i < 4; ++i) pT[(16 + 4 * jg + i) * LA + mr] = -Tx[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        {
            // T' row r = lane / 2, columns 16 (lane & 1) .. +15
            const int r = lane >> 1, cb = (lane & 1) * 16;
            const bool lower = (cb >> 4) <= (r >> 4);
            uint32_t pk[8];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 tv = *reinterpret_cast<const float4 *>(&pT[r * LA + cb + 4 * q4]);
                const float4 bv = *reinterpret_cast<const float4 *>(&pBeta[cb + 4 * q4]);
                pk[2 * q4] = pack2(lower ? tv.x * bv.x : 0.0f, lower ? tv.y * bv.y : 0.0f);
                pk[2 * q4 + 1] = pack2(lower ? tv.z * bv.z : 0.0f, lower ? tv.w * bv.w : 0.0f);
            }
            *reinterpret_cast<uint4 *>(&sTp[r * C + (((cb >> 3) ^ key4(r)) << 3)]) =
                make_uint4(pk[0], pk[1], pk[2], pk[3]);
            *reinterpret_cast<uint4 *>(&sTp[r * C + ((((cb >> 3) + 1) ^ key4(r)) << 3)]) =
                make_uint4(pk[4], pk[5], pk[6], pk[7]);
        }

        // next chunk's g and k (requested once the inverse no longer needs
        // registers; not live across the out-of-line exact path).  SAVE
        // requests them after its stores below, which need registers too.
        if constexpr (!SAVE) {
            if (n + NPROD < nchunks) load_gk(n + NPROD);
        }

        // ---- publish -------------------------------------------------------------
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        if (lane == 0) __hip_atomic_store(&s_full[slot], n + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);

        // ---- for the backward: T, T^T, P^T and the flag ----------------------------
        // (the slot's P stays unchanged until the slot is freed, pT until the
        // next chunk)
        if (keep) {
            const int r = lane >> 1, cb = (lane & 1) * 16;
            const bool lower = (cb >> 4) <= (r >> 4), upper = (cb >> 4) >= (r >> 4);
            float *gT = p.wT + wcc + r * C + cb;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 tv = *reinterpret_cast<const float4 *>(&pT[r * LA + cb + 4 * q4]);
                *reinterpret_cast<float4 *>(gT + 4 * q4) = lower ? tv : make_float4(0.f, 0.f, 0.f, 0.f);
            }
            // row r of T^T and P^T: T[c][r] and P[c][r] for c = cb .. cb + 15
            uint32_t tt[8], pt[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int c = cb + 2 * j;
                tt[j] = upper ? pack2(pT[c * LA + r], pT[(c + 1) * LA + r]) : 0u;
                pt[j] = (uint32_t)sP[idx4(c, r)].x | ((uint32_t)sP[idx4(c + 1, r)].x << 16);
            }
            uint4 *dT = reinterpret_cast<uint4 *>(p.wTt + wcc + r * C + cb);
            uint4 *dP = reinterpret_cast<uint4 *>(p.wPt + wcc + r * C + cb);
            dT[0] = make_uint4(tt[0], tt[1], tt[2], tt[3]);
            dT[1] = make_uint4(tt[4], tt[5], tt[6], tt[7]);
            dP[0] = make_uint4(pt[0], pt[1], pt[2], pt[3]);
            dP[1] = make_uint4(pt[4], pt[5], pt[6], pt[7]);
            if (lane == 0) p.wF[wcc / (C * C)] = flag64 ? 1 : 0;
        }
        if constexpr (SAVE) {
            if (n + NPROD < nchunks) load_gk(n + NPROD);
        }
    }
}

// Polls a bounded wait makes before giving up (process-wide; tests of the
// timeout handling lower it).
static int g_spin_limit = ws::SPIN_LIMIT;

void ws_set_spin_limit(int polls) { g_spin_limit = polls; }

// The device's sticky error bits (current device), cleared when asked.
hipError_t ws_device_errors(unsigned *bits, bool clear)
{
    hipError_t e = hipMemcpyFromSymbol(bits, HIP_SYMBOL(ws::g_ws_error), sizeof(unsigned), 0,
                                       hipMemcpyDeviceToHost);
    if (e != hipSuccess || !clear || *bits == 0) return e;
    const unsigned zero = 0;
    return hipMemcpyToSymbol(HIP_SYMBOL(ws::g_ws_error), &zero, sizeof(unsigned), 0,
                             hipMemcpyHostToDevice);
}

template <int DK, int NSTRIP, int GATE, int PREP, bool SAVE = false>
static hipError_t launch_ws(WsParams p, hipStream_t stream)
{
    p.spin_limit = g_spin_limit;
    const int groups = (p.units + 7) / 8;
    const dim3 grid(groups * 8 * p.nslices);
    hipLaunchKernelGGL((chunked_ws_kernel<DK, NSTRIP, GATE, PREP, SAVE>), grid, dim3(512), 0, stream, p);
    return hipGetLastError();
}

template <int DK, int NSTRIP, int GATE>
static hipError_t launch_ws_prep(const WsParams &p, int prep, hipStream_t stream)
{
    if constexpr (GATE == GATE_NONE) prep &= PREP_L2NORM;   // no gate to transform
    switch (prep) {
    case PREP_L2NORM: return launch_ws<DK, NSTRIP, GATE, PREP_L2NORM>(p, stream);
    case PREP_SOFTPLUS: return launch_ws<DK, NSTRIP, GATE, PREP_SOFTPLUS>(p, stream);
    case PREP_L2NORM | PREP_SOFTPLUS: return launch_ws<DK, NSTRIP, GATE, PREP_L2NORM | PREP_SOFTPLUS>(p, stream);
    default: return launch_ws<DK, NSTRIP, GATE, 0>(p, stream);
    }
}

template <int DK, int NSTRIP>
static hipError_t launch_ws_gate(const WsParams &p, int gate, int prep, hipStream_t stream)
{
    if (gate == GATE_HEAD) return launch_ws_prep<DK, NSTRIP, GATE_HEAD>(p, prep, stream);
    if (gate == GATE_NONE) return launch_ws_prep<DK, NSTRIP, GATE_NONE>(p, prep, stream);
    return launch_ws_prep<DK, NSTRIP, GATE_CHANNEL>(p, prep, stream);
}

hipError_t chunked_ws_launch(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, int gate, int prep, const float *S0, float *S_T,
                             const int32_t *state_idx, int pool, void *o,
                             const int32_t *cu_seqlens, const int32_t *order, int nseq, int T,
                             int H, int dk, int dv, int slice_width, hipStream_t stream)
{
    WsParams p = {};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.S0 = S0; p.S_T = S_T; p.o = o;
    p.cu_seqlens = cu_seqlens;
    p.order = order;
    p.state_idx = state_idx;
    p.pool = pool;
    p.T = T; p.H = H; p.DV = dv;
    p.units = nseq * H;
    p.nslices = dv / slice_width;
    const int nstrip = slice_width / 64;
    if (dk == 128)
        return nstrip == 2 ? launch_ws_gate<128, 2>(p, gate, prep, stream)
                           : launch_ws_gate<128, 1>(p, gate, prep, stream);
    return nstrip == 2 ? launch_ws_gate<64, 2>(p, gate, prep, stream)
                       : launch_ws_gate<64, 1>(p, gate, prep, stream);
}

template <int DK, int NSTRIP>
static hipError_t launch_ws_save(const WsParams &p, int gate, hipStream_t stream)
{
    if (gate == GATE_HEAD) return launch_ws<DK, NSTRIP, GATE_HEAD, 0, true>(p, stream);
    if (gate == GATE_NONE) return launch_ws<DK, NSTRIP, GATE_NONE, 0, true>(p, stream);
    return launch_ws<DK, NSTRIP, GATE_CHANNEL, 0, true>(p, stream);
}

// The forward's chunk chain for the backward (bf16 inputs): no o and no final
// state; per chunk and head the state entering it, X, U, T, M0, the bf16 T^T
// and P^T, P where flagged and the flag, into the backward's workspace
// (layouts as in WsParams).
hipError_t chunked_ws_save_launch(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, int gate, const float *S0,
                                  const int32_t *cu_seqlens, int nseq, int T, int H, int dk, int dv,
                                  int slice_width, bf16_t *wS, bf16_t *wX, bf16_t *wU, bf16_t *wTt,
                                  bf16_t *wPt, float *wT, float *wM, float *wP, int32_t *wF,
                                  hipStream_t stream)
{
    WsParams p = {};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.S0 = S0;
    p.cu_seqlens = cu_seqlens;
    p.T = T; p.H = H; p.DV = dv;
    p.units = nseq * H;
    p.nslices = dv / slice_width;
    p.wS = wS; p.wX = wX; p.wU = wU; p.wTt = wTt; p.wPt = wPt;
    p.wT = wT; p.wM = wM; p.wP = wP; p.wF = wF;
    const int nstrip = slice_width / 64;
    if (dk == 128)
        return nstrip == 2 ? launch_ws_save<128, 2>(p, gate, stream) : launch_ws_save<128, 1>(p, gate, stream);
    return nstrip == 2 ? launch_ws_save<64, 2>(p, gate, stream) : launch_ws_save<64, 1>(p, gate, stream);
}

}  // namespace kda
