// kda_bwd.hip -- backward of the chunked KDA forward (gfx950).
//
// Gradients of a loss L with respect to q, k, v, log_alpha, beta and S0,
// given dL/do and dL/dS_T.  The pages present the chunked form as the one
// used for efficient training (daily.dev summary of "You Could Have Come Up
// with Kimi Delta Attention", Summary section) and give no backward; this is
// the chunked form differentiated.  Per chunk of C = 32 tokens, with Gamma
// the within-chunk running sum of log_alpha per key channel and the decay
// between two rows taken pairwise, F_ric = e^{Gamma_rc - Gamma_ic} <= 1 for
// i <= r:
//   M0 = [sum_c k_rc k_ic F_ric]_{i<r},  P = [sum_c q_rc k_ic F_ric]_{i<=r},
//   T = (I + Diag(beta) M0)^{-1},  K_up = K e^{Gamma},  Q_up = Q e^{Gamma},
//   K_right = K e^{Gamma_c - Gamma},  gamma = e^{Gamma_c},
//   X = V - K_up S,  U = T Diag(beta) X,  O = Q_up S + P U,
//   S_next = Diag(gamma) S + K_right^T U.
// Reverse, with D the gradient of S_next:
//   dU = P^T dO + K_right D,  dX = Diag(beta) T^T dU,  dV = dX,
//   dS = Diag(gamma) D + Q_up^T dO - K_up^T dX                   (the chain),
//   dT' = dU X^T, dP = tril(dO U^T), dbeta from T' and from A = Diag(beta) M0,
//   dA = -T^T (dT' Diag(beta)) T^T, and the pairwise sums of M0 and P taken
//   back to k, q and Gamma; dlog_alpha is the reverse running sum of dGamma
//   plus the chunk-total term (Gamma_c enters gamma and K_right).
//
// Four launches:
//   bwd_prep_kernel    one workgroup per (chunk, head): M0, P (pairwise, no
//                      exponent ever positive) and T by forward substitution;
//   bwd_states_kernel  one per (sequence, head, 32-column slice of d_v): the
//                      forward state chain, storing the state entering each chunk;
//   bwd_dstates_kernel same units, chunks in reverse: the state-gradient chain,
//                      storing D for each chunk, and dS0;
//   bwd_grads_kernel   one per (chunk, head): every input gradient of the chunk.
// All arithmetic is fp32 (fp32 MFMA 16x16x4 for the products, VALU for the
// pairwise decay sums); inputs and outputs are bf16 or fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_device.h"

namespace kda {
namespace bwd {

constexpr int C = 32;        // chunk length
constexpr int NT = 256;      // threads per workgroup
constexpr int W = 32;        // d_v columns per slice
constexpr int CP = C + 1;    // LDS pitch of C x C and C x W matrices
constexpr int WP = W + 1;

struct Params {
    const void *q, *k, *v, *g, *beta, *dO;
    const float *S0, *dST;
    const int32_t *cu;       // packed sequences, or NULL (dense)
    int num_seqs, T, H, DV, gate;
    void *dq, *dk, *dv, *dg, *dbeta;
    float *dS0;
    float *wS, *wD, *wT, *wP, *wM;   // workspace, per (chunk slot, head)
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc += A B for one 16 x 16 tile, K a multiple of 4, operands in LDS:
// A(m, k) = a[m * am + k * ak], B(k, n) = b[k * bk + n * bn] (a, b at the
// tile's origin).  Tile element (4 * (lane >> 4) + i, lane & 15) is acc[i].
__device__ __forceinline__ f32x4 mm(f32x4 acc, const float *a, int am, int ak, const float *b,
                                    int bk, int bn, int K) {
    const int lane = threadIdx.x & 63, r = lane & 15, j = lane >> 4;
    const float *pa = a + r * am + j * ak;
    const float *pb = b + j * bk + r * bn;
#pragma unroll 4
    for (int k0 = 0; k0 < K; k0 += 4) acc = mfma4(pa[k0 * ak], pb[k0 * bk], acc);
    return acc;
}

template <typename Tin>
__device__ __forceinline__ float ld(const void *p, size_t i) {
    return load_elem(static_cast<const Tin *>(p) + i);
}
template <typename Tin>
__device__ __forceinline__ void st(void *p, size_t i, float x) {
    store_elem(static_cast<Tin *>(p) + i, x);
}

// Token range of sequence s and the workspace slot of its first chunk.
// Dense: s * ceil(T / C).  Packed: floor(cu[s] / C) + s, which leaves every
// sequence enough slots for its chunks without overlap.
__device__ __forceinline__ void seq_info(const Params &p, int s, long &t0, int &len, long &base) {
    if (p.cu) {
        t0 = p.cu[s];
        len = p.cu[s + 1] - p.cu[s];
        base = (long)(p.cu[s] / C) + s;
    } else {
        t0 = (long)s * p.T;
        len = p.T;
        base = (long)s * ((p.T + C - 1) / C);
    }
}

// Chunk of a workspace slot: its sequence, first token and length; false for
// a slot no chunk uses.
__device__ __forceinline__ bool slot_chunk(const Params &p, long slot, long &t0, int &cl) {
    int s;
    if (p.cu) {
        int lo = 0, hi = p.num_seqs - 1;     // last s with base(s) <= slot
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((long)(p.cu[mid] / C) + mid <= slot) lo = mid;
            else hi = mid - 1;
        }
        s = lo;
    } else {
        s = (int)(slot / ((p.T + C - 1) / C));
        if (s >= p.num_seqs) return false;
    }
    long ts, base;
    int len;
    seq_info(p, s, ts, len, base);
    const long n = slot - base;
    if (n < 0 || n * C >= len) return false;
    t0 = ts + n * C;
    cl = (int)(len - n * C < C ? len - n * C : C);
    return true;
}

// log2 of alpha for token t, head h, key channel c (0 without a gate)
template <typename Tin, int DK>
__device__ __forceinline__ float log2_alpha(const Params &p, long t, int h, int c) {
    if (p.gate == GATE_CHANNEL) return ld<Tin>(p.g, ((size_t)t * p.H + h) * DK + c) * kLog2e;
    if (p.gate == GATE_HEAD) return ld<Tin>(p.g, (size_t)t * p.H + h) * kLog2e;
    return 0.0f;
}

// Loads the chunk's k (and q) rows and log2-gates into LDS (zeros past the
// chunk end), turns the gates into running sums per channel (in sG) with
// totals gc[c] and gamma = 2^gc; then, per element, K_up = k 2^G,
// Q_up = q 2^G, K_right = k 2^{G_c - G}.  sG may be sKrt (each element is
// read before it is overwritten by the same thread).  Ends with a barrier.
template <typename Tin, int DK, bool WITH_Q>
__device__ void chunk_factors(const Params &p, long t0, int cl, int h, float *sKup, float *sQup,
                              float *sG, float *sKrt, float *gc, float *gam) {
    constexpr int DKP = DK + 1;
    const int tid = threadIdx.x;
    for (int idx = tid; idx < C * DK; idx += NT) {
        const int r = idx / DK, c = idx % DK;
        const bool ok = r < cl;
        const size_t e = ((size_t)(t0 + r) * p.H + h) * DK + c;
        sKup[r * DKP + c] = ok ? ld<Tin>(p.k, e) : 0.0f;
        if constexpr (WITH_Q) sQup[r * DKP + c] = ok ? ld<Tin>(p.q, e) : 0.0f;
        sG[r * DKP + c] = ok ? log2_alpha<Tin, DK>(p, t0 + r, h, c) : 0.0f;
    }
    __syncthreads();
    if (tid < DK) {
        float run = 0.0f;
        for (int r = 0; r < C; ++r) {
            run += sG[r * DKP + tid];
            sG[r * DKP + tid] = run;
        }
        gc[tid] = run;
        gam[tid] = __builtin_amdgcn_exp2f(run);
    }
    __syncthreads();
    for (int idx = tid; idx < C * DK; idx += NT) {
        const int r = idx / DK, c = idx % DK;
        const float G = sG[r * DKP + c], kv = sKup[r * DKP + c];
        const float E = __builtin_amdgcn_exp2f(G);
        sKup[r * DKP + c] = kv * E;
        if constexpr (WITH_Q) sQup[r * DKP + c] *= E;
        sKrt[r * DKP + c] = kv * __builtin_amdgcn_exp2f(gc[c] - G);
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// M0, P and T of one chunk.
template <typename Tin, int DK>
__global__ void __launch_bounds__(NT) bwd_prep_kernel(Params p) {
    constexpr int DKP = DK + 1, NCC = DK / 8;
    __shared__ float sK[C * DKP], sQ[C * DKP], sG[C * DKP];
    __shared__ float sM[C * CP], sP[C * CP], sB[C];
    const long slot = blockIdx.x;
    const int h = blockIdx.y, tid = threadIdx.x;
    long t0;
    int cl;
    if (!slot_chunk(p, slot, t0, cl)) return;
    for (int idx = tid; idx < C * DK; idx += NT) {
        const int r = idx / DK, c = idx % DK;
        const bool ok = r < cl;
        const size_t e = ((size_t)(t0 + r) * p.H + h) * DK + c;
        sK[r * DKP + c] = ok ? ld<Tin>(p.k, e) : 0.0f;
        sQ[r * DKP + c] = ok ? ld<Tin>(p.q, e) : 0.0f;
        sG[r * DKP + c] = ok ? log2_alpha<Tin, DK>(p, t0 + r, h, c) : 0.0f;
    }
    if (tid < C) sB[tid] = tid < cl ? ld<Tin>(p.beta, (size_t)(t0 + tid) * p.H + h) : 0.0f;
    __syncthreads();
    if (tid < DK) {
        float run = 0.0f;
        for (int r = 0; r < C; ++r) {
            run += sG[r * DKP + tid];
            sG[r * DKP + tid] = run;
        }
    }
    __syncthreads();
    // pairwise sums: thread (row r, channel group cg) over channels cg + 8 cc
    {
        const int r = tid >> 3, cg = tid & 7;
        float kr[NCC], qr[NCC], gr[NCC];
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            kr[cc] = sK[r * DKP + cg + 8 * cc];
            qr[cc] = sQ[r * DKP + cg + 8 * cc];
            gr[cc] = sG[r * DKP + cg + 8 * cc];
        }
        for (int i = 0; i < C; ++i) {
            float m = 0.0f, pp = 0.0f;
#pragma unroll
            for (int cc = 0; cc < NCC; ++cc) {
                const int c = cg + 8 * cc;
                const float d = gr[cc] - sG[i * DKP + c];
                const float F = __builtin_amdgcn_exp2f(d < 0.0f ? d : 0.0f);
                const float kf = sK[i * DKP + c] * F;
                m += kr[cc] * kf;
                pp += qr[cc] * kf;
            }
            m += __shfl_xor(m, 1);
            m += __shfl_xor(m, 2);
            m += __shfl_xor(m, 4);
            pp += __shfl_xor(pp, 1);
            pp += __shfl_xor(pp, 2);
            pp += __shfl_xor(pp, 4);
            if (cg == 0) {
                sM[r * CP + i] = i < r ? m : 0.0f;
                sP[r * CP + i] = i <= r ? pp : 0.0f;
            }
        }
    }
    __syncthreads();
    const size_t wi = (size_t)slot * p.H + h;
    float *gT = p.wT + wi * C * C, *gP = p.wP + wi * C * C, *gM = p.wM + wi * C * C;
    for (int idx = tid; idx < C * C; idx += NT) {
        const int r = idx / C, i = idx % C;
        gP[idx] = sP[r * CP + i];
        gM[idx] = sM[r * CP + i];
    }
    // T = (I + A)^{-1}, A = Diag(beta) M0 strictly lower: column i by lane i,
    // rows in order, T_ri = [r == i] - sum_{j < r} A_rj T_ji
    if (tid < C) {
        const int i = tid;
        float t[C];
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float acc = r == i ? 1.0f : 0.0f;
#pragma unroll
            for (int j = 0; j < r; ++j) acc -= sB[r] * sM[r * CP + j] * t[j];
            t[r] = acc;
            gT[r * C + i] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// Forward state chain of one (sequence, head, slice): the state entering
// every chunk goes to the workspace.
template <typename Tin, int DK>
__global__ void __launch_bounds__(NT) bwd_states_kernel(Params p) {
    constexpr int DKP = DK + 1, NTW = DK / 32;   // state tiles per wave
    __shared__ float sS[DK * WP], sKup[C * DKP], sKrt[C * DKP], sV[C * WP], sU[C * WP],
        sT[C * CP], gc[DK], gam[DK], sB[C];
    const int nsl = p.DV / W;
    const int unit = blockIdx.x / nsl, slice = blockIdx.x % nsl;
    const int s = unit / p.H, h = unit % p.H, col0 = slice * W;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lj = lane >> 4;
    long t0s, base;
    int len;
    seq_info(p, s, t0s, len, base);
    const int nch = (len + C - 1) / C;
    // state tiles of this wave: tile index w * NTW + x -> (tm, tn) over (DK/16) x (W/16)
    f32x4 S[NTW];
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
        const int tt = wave * NTW + x, tm = tt >> 1, tn = tt & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * tm + 4 * lj + i, col = col0 + 16 * tn + lr;
            S[x][i] = p.S0 ? p.S0[(((size_t)s * p.H + h) * DK + row) * p.DV + col] : 0.0f;
        }
    }
    for (int n = 0; n < nch; ++n) {
        const long t0 = t0s + (long)n * C;
        const int cl = len - n * C < C ? len - n * C : C;
        const size_t wi = (size_t)(base + n) * p.H + h;
        float *gS = p.wS + wi * DK * p.DV;
#pragma unroll
        for (int x = 0; x < NTW; ++x) {
            const int tt = wave * NTW + x, tm = tt >> 1, tn = tt & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * tm + 4 * lj + i, col = 16 * tn + lr;
                sS[row * WP + col] = S[x][i];
                gS[(size_t)row * p.DV + col0 + col] = S[x][i];
            }
        }
        for (int idx = tid; idx < C * W; idx += NT) {
            const int r = idx / W, c = idx % W;
            sV[r * WP + c] = r < cl ? ld<Tin>(p.v, ((size_t)(t0 + r) * p.H + h) * p.DV + col0 + c) : 0.0f;
        }
        for (int idx = tid; idx < C * C; idx += NT) sT[(idx / C) * CP + idx % C] = p.wT[wi * C * C + idx];
        if (tid < C) sB[tid] = tid < cl ? ld<Tin>(p.beta, (size_t)(t0 + tid) * p.H + h) : 0.0f;
        // sKrt first holds the gate sums
        chunk_factors<Tin, DK, false>(p, t0, cl, h, sKup, nullptr, sKrt, sKrt, gc, gam);
        // X = V - K_up S, kept as beta X
        {
            const int tm = wave >> 1, tn = wave & 1;
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            a = mm(a, sKup + 16 * tm * DKP, DKP, 1, sS + 16 * tn, WP, 1, DK);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * tm + 4 * lj + i, col = 16 * tn + lr;
                sV[row * WP + col] = sB[row] * (sV[row * WP + col] - a[i]);
            }
        }
        __syncthreads();
        // U = T (beta X)
        {
            const int tm = wave >> 1, tn = wave & 1;
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            a = mm(a, sT + 16 * tm * CP, CP, 1, sV + 16 * tn, WP, 1, C);
#pragma unroll
            for (int i = 0; i < 4; ++i) sU[(16 * tm + 4 * lj + i) * WP + 16 * tn + lr] = a[i];
        }
        __syncthreads();
        // S = Diag(gamma) S + K_right^T U
#pragma unroll
        for (int x = 0; x < NTW; ++x) {
            const int tt = wave * NTW + x, tm = tt >> 1, tn = tt & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) S[x][i] *= gam[16 * tm + 4 * lj + i];
            S[x] = mm(S[x], sKrt + 16 * tm, 1, DKP, sU + 16 * tn, WP, 1, C);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// State-gradient chain of one (sequence, head, slice), chunks in reverse: D
// (the gradient of the state leaving each chunk) goes to the workspace, and
// the gradient of the initial state to dS0.
template <typename Tin, int DK>
__global__ void __launch_bounds__(NT) bwd_dstates_kernel(Params p) {
    constexpr int DKP = DK + 1, NTW = DK / 32;
    __shared__ float sD[DK * WP], sKup[C * DKP], sQup[C * DKP], sKrt[C * DKP], sdO[C * WP],
        sdU[C * WP], sdX[C * WP], sT[C * CP], sP[C * CP], gc[DK], gam[DK], sB[C];
    const int nsl = p.DV / W;
    const int unit = blockIdx.x / nsl, slice = blockIdx.x % nsl;
    const int s = unit / p.H, h = unit % p.H, col0 = slice * W;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lj = lane >> 4;
    long t0s, base;
    int len;
    seq_info(p, s, t0s, len, base);
    const int nch = (len + C - 1) / C;
    const size_t so = ((size_t)s * p.H + h) * DK;
    f32x4 D[NTW];
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
        const int tt = wave * NTW + x, tm = tt >> 1, tn = tt & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * tm + 4 * lj + i, col = col0 + 16 * tn + lr;
            D[x][i] = p.dST ? p.dST[(so + row) * p.DV + col] : 0.0f;
        }
    }
    for (int n = nch - 1; n >= 0; --n) {
        const long t0 = t0s + (long)n * C;
        const int cl = len - n * C < C ? len - n * C : C;
        const size_t wi = (size_t)(base + n) * p.H + h;
        float *gD = p.wD + wi * DK * p.DV;
#pragma unroll
        for (int x = 0; x < NTW; ++x) {
            const int tt = wave * NTW + x, tm = tt >> 1, tn = tt & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * tm + 4 * lj + i, col = 16 * tn + lr;
                sD[row * WP + col] = D[x][i];
                gD[(size_t)row * p.DV + col0 + col] = D[x][i];
            }
        }
        for (int idx = tid; idx < C * W; idx += NT) {
            const int r = idx / W, c = idx % W;
            sdO[r * WP + c] = r < cl ? ld<Tin>(p.dO, ((size_t)(t0 + r) * p.H + h) * p.DV + col0 + c) : 0.0f;
        }
        for (int idx = tid; idx < C * C; idx += NT) {
            sT[(idx / C) * CP + idx % C] = p.wT[wi * C * C + idx];
            sP[(idx / C) * CP + idx % C] = p.wP[wi * C * C + idx];
        }
        if (tid < C) sB[tid] = tid < cl ? ld<Tin>(p.beta, (size_t)(t0 + tid) * p.H + h) : 0.0f;
        chunk_factors<Tin, DK, true>(p, t0, cl, h, sKup, sQup, sKrt, sKrt, gc, gam);
        // dU = P^T dO + K_right D
        {
            const int tm = wave >> 1, tn = wave & 1;
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            a = mm(a, sP + 16 * tm, 1, CP, sdO + 16 * tn, WP, 1, C);
            a = mm(a, sKrt + 16 * tm * DKP, DKP, 1, sD + 16 * tn, WP, 1, DK);
#pragma unroll
            for (int i = 0; i < 4; ++i) sdU[(16 * tm + 4 * lj + i) * WP + 16 * tn + lr] = a[i];
        }
        __syncthreads();
        // -dX = -Diag(beta) T^T dU
        {
            const int tm = wave >> 1, tn = wave & 1;
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            a = mm(a, sT + 16 * tm, 1, CP, sdU + 16 * tn, WP, 1, C);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * tm + 4 * lj + i;
                sdX[row * WP + 16 * tn + lr] = -sB[row] * a[i];
            }
        }
        __syncthreads();
        // D = Diag(gamma) D + Q_up^T dO - K_up^T dX
#pragma unroll
        for (int x = 0; x < NTW; ++x) {
            const int tt = wave * NTW + x, tm = tt >> 1, tn = tt & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) D[x][i] *= gam[16 * tm + 4 * lj + i];
            D[x] = mm(D[x], sQup + 16 * tm, 1, DKP, sdO + 16 * tn, WP, 1, C);
            D[x] = mm(D[x], sKup + 16 * tm, 1, DKP, sdX + 16 * tn, WP, 1, C);
        }
        __syncthreads();
    }
    if (p.dS0) {
#pragma unroll
        for (int x = 0; x < NTW; ++x) {
            const int tt = wave * NTW + x, tm = tt >> 1, tn = tt & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * tm + 4 * lj + i, col = col0 + 16 * tn + lr;
                p.dS0[(so + row) * p.DV + col] = D[x][i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Every input gradient of one chunk, from the state entering it (S), the
// gradient of the state leaving it (D), and T, P, M0.
template <int DK>
constexpr int grads_floats() {
    return 4 * C * (DK + 1) + 3 * C * CP + 2 * DK * WP + 6 * C * WP + 3 * DK + 2 * C;
}

template <typename Tin, int DK>
__global__ void __launch_bounds__(NT) bwd_grads_kernel(Params p) {
    constexpr int DKP = DK + 1, NTW = DK / 32, NPART = NT / DK;
    __shared__ float smem[grads_floats<DK>()];
    float *sKup = smem;                  // C x DKP: K_up, later dk
    float *sQup = sKup + C * DKP;        //          Q_up, later dq
    float *sKrt = sQup + C * DKP;        //          K_right, later dGamma
    float *sG = sKrt + C * DKP;          //          running log2 gate sums
    float *sT = sG + C * DKP;            // C x CP
    float *sP = sT + C * CP;
    float *sM = sP + C * CP;             // M0, later dM
    float *sS = sM + C * CP;             // DK x WP (slice of S), later dK_right K_right
    float *sD = sS + DK * WP;            // DK x WP (slice of D)
    float *sX = sD + DK * WP;            // C x WP: V, then X; later dT'
    float *sBX = sX + C * WP;            //         beta X; later dP
    float *sdO = sBX + C * WP;
    float *sU = sdO + C * WP;            //         U; later T^T dT
    float *sdU = sU + C * WP;            //         dU; later dA
    float *sdX = sdU + C * WP;
    float *gc = sdX + C * WP;            // DK
    float *gam = gc + DK;
    float *dgam = gam + DK;
    float *sB = dgam + DK;               // C
    float *dB = sB + C;

    const long slot = blockIdx.x;
    const int h = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lj = lane >> 4;
    long t0;
    int cl;
    if (!slot_chunk(p, slot, t0, cl)) return;
    const size_t wi = (size_t)slot * p.H + h;
    const float *gS = p.wS + wi * DK * p.DV, *gD = p.wD + wi * DK * p.DV;

    for (int idx = tid; idx < C * C; idx += NT) {
        const int r = idx / C, i = idx % C;
        sT[r * CP + i] = p.wT[wi * C * C + idx];
        sP[r * CP + i] = p.wP[wi * C * C + idx];
        sM[r * CP + i] = p.wM[wi * C * C + idx];
    }
    if (tid < C) {
        sB[tid] = tid < cl ? ld<Tin>(p.beta, (size_t)(t0 + tid) * p.H + h) : 0.0f;
        dB[tid] = 0.0f;
    }
    if (tid < DK) dgam[tid] = 0.0f;
    // sKrt holds the gate sums until K_right replaces them; keep a copy in sG
    {
        for (int idx = tid; idx < C * DK; idx += NT) {
            const int r = idx / DK, c = idx % DK;
            const bool ok = r < cl;
            const size_t e = ((size_t)(t0 + r) * p.H + h) * DK + c;
            sKup[r * DKP + c] = ok ? ld<Tin>(p.k, e) : 0.0f;
            sQup[r * DKP + c] = ok ? ld<Tin>(p.q, e) : 0.0f;
            sG[r * DKP + c] = ok ? log2_alpha<Tin, DK>(p, t0 + r, h, c) : 0.0f;
        }
        __syncthreads();
        if (tid < DK) {
            float run = 0.0f;
            for (int r = 0; r < C; ++r) {
                run += sG[r * DKP + tid];
                sG[r * DKP + tid] = run;
            }
            gc[tid] = run;
            gam[tid] = __builtin_amdgcn_exp2f(run);
        }
        __syncthreads();
        for (int idx = tid; idx < C * DK; idx += NT) {
            const int r = idx / DK, c = idx % DK;
            const float G = sG[r * DKP + c], kv = sKup[r * DKP + c];
            const float E = __builtin_amdgcn_exp2f(G);
            sKup[r * DKP + c] = kv * E;
            sQup[r * DKP + c] *= E;
            sKrt[r * DKP + c] = kv * __builtin_amdgcn_exp2f(gc[c] - G);
        }
    }

    // accumulators over the d_v slices: this wave's tiles of dQ_up, dK_up
    // (negated) and dK_right (C x DK, tile w * NTW + x -> (tm, tn) over 2 x
    // DK/16), and of dT' and dP (C x C, tile w -> (w >> 1, w & 1))
    f32x4 aQ[NTW], aK[NTW], aR[NTW], aT = {0.f, 0.f, 0.f, 0.f}, aP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
        aQ[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        aK[x] = aQ[x];
        aR[x] = aQ[x];
    }
    const int tm = wave >> 1, tn = wave & 1;        // this wave's C x W / C x C tile
    for (int col0 = 0; col0 < p.DV; col0 += W) {
        __syncthreads();
        for (int idx = tid; idx < DK * W; idx += NT) {
            const int r = idx / W, c = idx % W;
            sS[r * WP + c] = gS[(size_t)r * p.DV + col0 + c];
            sD[r * WP + c] = gD[(size_t)r * p.DV + col0 + c];
        }
        for (int idx = tid; idx < C * W; idx += NT) {
            const int r = idx / W, c = idx % W;
            const bool ok = r < cl;
            const size_t e = ((size_t)(t0 + r) * p.H + h) * p.DV + col0 + c;
            sX[r * WP + c] = ok ? ld<Tin>(p.v, e) : 0.0f;
            sdO[r * WP + c] = ok ? ld<Tin>(p.dO, e) : 0.0f;
        }
        __syncthreads();
        // X = V - K_up S
        {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            a = mm(a, sKup + 16 * tm * DKP, DKP, 1, sS + 16 * tn, WP, 1, DK);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * tm + 4 * lj + i, o = row * WP + 16 * tn + lr;
                const float x = sX[o] - a[i];
                sX[o] = x;
                sBX[o] = sB[row] * x;
            }
        }
        __syncthreads();
        // U = T (beta X);  dU = P^T dO + K_right D
        {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            a = mm(a, sT + 16 * tm * CP, CP, 1, sBX + 16 * tn, WP, 1, C);
            f32x4 b = {0.f, 0.f, 0.f, 0.f};
            b = mm(b, sP + 16 * tm, 1, CP, sdO + 16 * tn, WP, 1, C);
            b = mm(b, sKrt + 16 * tm * DKP, DKP, 1, sD + 16 * tn, WP, 1, DK);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = (16 * tm + 4 * lj + i) * WP + 16 * tn + lr;
                sU[o] = a[i];
                sdU[o] = b[i];
            }
        }
        __syncthreads();
        // dX = Diag(beta) T^T dU (also dV)
        {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            a = mm(a, sT + 16 * tm, 1, CP, sdU + 16 * tn, WP, 1, C);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * tm + 4 * lj + i, col = 16 * tn + lr;
                const float x = sB[row] * a[i];
                sdX[row * WP + col] = x;
                if (row < cl) st<Tin>(p.dv, ((size_t)(t0 + row) * p.H + h) * p.DV + col0 + col, x);
            }
        }
        // dT' += dU X^T;  dP += dO U^T;  dQ_up += dO S^T;  dK_right += U D^T
        aT = mm(aT, sdU + 16 * tm * WP, WP, 1, sX + 16 * tn * WP, 1, WP, W);
        aP = mm(aP, sdO + 16 * tm * WP, WP, 1, sU + 16 * tn * WP, 1, WP, W);
#pragma unroll
        for (int x = 0; x < NTW; ++x) {
            const int tt = wave * NTW + x, m0 = 16 * (tt / (DK / 16)), n0 = 16 * (tt % (DK / 16));
            aQ[x] = mm(aQ[x], sdO + m0 * WP, WP, 1, sS + n0 * WP, 1, WP, W);
            aR[x] = mm(aR[x], sU + m0 * WP, WP, 1, sD + n0 * WP, 1, WP, W);
        }
        if (tid < DK) {
            float acc = 0.0f;
            for (int j = 0; j < W; ++j) acc += sD[tid * WP + j] * sS[tid * WP + j];
            dgam[tid] += acc;
        }
        __syncthreads();
        // dK_up -= dX S^T
#pragma unroll
        for (int x = 0; x < NTW; ++x) {
            const int tt = wave * NTW + x, m0 = 16 * (tt / (DK / 16)), n0 = 16 * (tt % (DK / 16));
            aK[x] = mm(aK[x], sdX + m0 * WP, WP, 1, sS + n0 * WP, 1, WP, W);
        }
    }
    __syncthreads();

    // direct terms, element by element where the tiles lie:
    //   dq = dQ_up e^G,  dk = dK_up e^G + dK_right e^{G_c - G},
    //   dGamma = dK_up K_up + dQ_up Q_up - dK_right K_right,
    // and dK_right K_right kept for the chunk-total term
    float *sRK = sS;                     // C x DKP
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
        const int tt = wave * NTW + x, m0 = 16 * (tt / (DK / 16)), n0 = 16 * (tt % (DK / 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + 4 * lj + i, col = n0 + lr, o = row * DKP + col;
            const float G = sG[o], E = __builtin_amdgcn_exp2f(G);
            const float R = __builtin_amdgcn_exp2f(gc[col] - G);
            const float dQu = aQ[x][i], dKu = -aK[x][i], dKr = aR[x][i];
            const float ku = sKup[o], qu = sQup[o], kr = sKrt[o];
            sQup[o] = dQu * E;
            sKup[o] = dKu * E + dKr * R;
            sKrt[o] = dKu * ku + dQu * qu - dKr * kr;
            sRK[o] = dKr * kr;
        }
    }
    // dT' and dP (lower, diagonal included) to LDS
    float *sdT = sX, *sdP = sBX, *sY = sU, *sdA = sdU;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * tm + 4 * lj + i, col = 16 * tn + lr;
        sdT[row * WP + col] = aT[i];
        sdP[row * WP + col] = col <= row ? aP[i] : 0.0f;
    }
    __syncthreads();
    // dbeta_i from T' = T Diag(beta); then dT = dT' Diag(beta)
    if (tid < C) {
        float acc = 0.0f;
        for (int r = 0; r < C; ++r) acc += sT[r * CP + tid] * sdT[r * WP + tid];
        dB[tid] = acc;
    }
    __syncthreads();
    for (int idx = tid; idx < C * C; idx += NT) {
        const int r = idx / C, i = idx % C;
        sdT[r * WP + i] *= sB[i];
    }
    __syncthreads();
    // Y = T^T dT;  dA = -(Y T^T), strictly lower
    {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        a = mm(a, sT + 16 * tm, 1, CP, sdT + 16 * tn, WP, 1, C);
#pragma unroll
        for (int i = 0; i < 4; ++i) sY[(16 * tm + 4 * lj + i) * WP + 16 * tn + lr] = a[i];
    }
    __syncthreads();
    {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        a = mm(a, sY + 16 * tm * WP, WP, 1, sT + 16 * tn * CP, 1, CP, C);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * tm + 4 * lj + i, col = 16 * tn + lr;
            sdA[row * WP + col] = col < row ? -a[i] : 0.0f;
        }
    }
    __syncthreads();
    // dbeta_r += sum_i dA_ri M0_ri;  dM = Diag(beta) dA (over M0's place)
    if (tid < C) {
        const int r = tid;
        float acc = 0.0f;
        for (int i = 0; i < C; ++i) {
            const float a = sdA[r * WP + i];
            acc += a * sM[r * CP + i];
            sM[r * CP + i] = sB[r] * a;
        }
        dB[r] += acc;
    }
    __syncthreads();

    // pairwise sums of M0 and P, taken back to k, q and Gamma: thread (channel
    // c, part); part p takes the pairs (r, i <= r) with (r + i) % NPART == p.
    {
        const int c = tid % DK, part = tid / DK;
        float kc[C], qc[C], gcol[C], aq[C], ak[C], ag[C];
#pragma unroll
        for (int r = 0; r < C; ++r) {
            const bool ok = r < cl;
            const size_t e = ((size_t)(t0 + (ok ? r : 0)) * p.H + h) * DK + c;
            kc[r] = ok ? ld<Tin>(p.k, e) : 0.0f;
            qc[r] = ok ? ld<Tin>(p.q, e) : 0.0f;
            gcol[r] = sG[r * DKP + c];
            aq[r] = 0.0f;
            ak[r] = 0.0f;
            ag[r] = 0.0f;
        }
#pragma unroll
        for (int r = 0; r < C; ++r) {
#pragma unroll
            for (int i = 0; i <= r; ++i) {
                if ((r + i) % NPART != part) continue;
                const float F = __builtin_amdgcn_exp2f(gcol[r] - gcol[i]);
                const float a = sdP[r * WP + i] * F;
                const float b = sM[r * CP + i] * F;      // dM, zero on the diagonal
                aq[r] += a * kc[i];
                ak[r] += b * kc[i];
                const float t = a * qc[r] + b * kc[r];
                ak[i] += t;
                const float w = t * kc[i];
                ag[r] += w;
                ag[i] -= w;
            }
        }
        // add the parts into the direct terms, one part at a time
        for (int pp = 0; pp < NPART; ++pp) {
            if (part == pp) {
#pragma unroll
                for (int r = 0; r < C; ++r) {
                    sQup[r * DKP + c] += aq[r];
                    sKup[r * DKP + c] += ak[r];
                    sKrt[r * DKP + c] += ag[r];
                }
            }
            __syncthreads();
        }
    }
    // dlog_alpha: reverse running sum of dGamma plus the chunk-total term
    // sum_r dK_right K_right + dgamma gamma; outputs
    if (tid < DK) {
        const int c = tid;
        float tot = dgam[c] * gam[c];
        for (int r = 0; r < C; ++r) tot += sRK[r * DKP + c];
        float run = tot;
        for (int r = C - 1; r >= 0; --r) {
            run += sKrt[r * DKP + c];
            sKrt[r * DKP + c] = run;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < cl * DK; idx += NT) {
        const int r = idx / DK, c = idx % DK;
        const size_t e = ((size_t)(t0 + r) * p.H + h) * DK + c;
        st<Tin>(p.dq, e, sQup[r * DKP + c]);
        st<Tin>(p.dk, e, sKup[r * DKP + c]);
        if (p.gate == GATE_CHANNEL) st<Tin>(p.dg, e, sKrt[r * DKP + c]);
    }
    if (tid < cl) {
        const size_t e = (size_t)(t0 + tid) * p.H + h;
        st<Tin>(p.dbeta, e, dB[tid]);
        if (p.gate == GATE_HEAD) {
            float acc = 0.0f;
            for (int c = 0; c < DK; ++c) acc += sKrt[tid * DKP + c];
            st<Tin>(p.dg, e, acc);
        }
    }
}

template <typename Tin, int DK>
hipError_t launch(const Params &p, long nslot, int nseq, hipStream_t stream) {
    const dim3 gchunks((unsigned)nslot, (unsigned)p.H);
    const unsigned gunits = (unsigned)((long)nseq * p.H * (p.DV / W));
    if (nslot > 0) hipLaunchKernelGGL((bwd_prep_kernel<Tin, DK>), gchunks, dim3(NT), 0, stream, p);
    hipLaunchKernelGGL((bwd_states_kernel<Tin, DK>), dim3(gunits), dim3(NT), 0, stream, p);
    hipLaunchKernelGGL((bwd_dstates_kernel<Tin, DK>), dim3(gunits), dim3(NT), 0, stream, p);
    if (nslot > 0) hipLaunchKernelGGL((bwd_grads_kernel<Tin, DK>), gchunks, dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace bwd

// Workspace slots per head: enough for dense (B ceil(T/C)) and packed
// (floor(T/C) + N + 1) layouts.
long bwd_slots(int B, int T, int num_seqs) {
    return (long)B * ((T + bwd::C - 1) / bwd::C) + num_seqs + 1;
}

size_t bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs) {
    const size_t per = (size_t)H * bwd_slots(B, T, num_seqs);
    const size_t a = (per * dk * dv * sizeof(float) + 255) & ~(size_t)255;
    const size_t b = (per * bwd::C * bwd::C * sizeof(float) + 255) & ~(size_t)255;
    return 2 * a + 3 * b;
}

hipError_t bwd_launch(const void *q, const void *k, const void *v, const void *g, const void *beta,
                      int gate, const float *S0, const void *dO, const float *dST,
                      const int32_t *cu_seqlens, int num_seqs, int B, int T, int H, int dk, int dv,
                      bool bf16, void *dq, void *dk_out, void *dv_out, void *dg, void *dbeta,
                      float *dS0, void *workspace, hipStream_t stream) {
    bwd::Params p;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.dO = dO;
    p.S0 = S0; p.dST = dST; p.cu = cu_seqlens;
    p.num_seqs = num_seqs; p.T = T; p.H = H; p.DV = dv; p.gate = gate;
    p.dq = dq; p.dk = dk_out; p.dv = dv_out; p.dg = dg; p.dbeta = dbeta; p.dS0 = dS0;
    const size_t per = (size_t)H * bwd_slots(B, T, num_seqs);
    const size_t a = (per * dk * dv * sizeof(float) + 255) & ~(size_t)255;
    const size_t b = (per * bwd::C * bwd::C * sizeof(float) + 255) & ~(size_t)255;
    char *w = static_cast<char *>(workspace);
    p.wS = reinterpret_cast<float *>(w);
    p.wD = reinterpret_cast<float *>(w + a);
    p.wT = reinterpret_cast<float *>(w + 2 * a);
    p.wP = reinterpret_cast<float *>(w + 2 * a + b);
    p.wM = reinterpret_cast<float *>(w + 2 * a + 2 * b);
    const long nslot = cu_seqlens ? (long)(T / bwd::C) + num_seqs + 1
                                  : (long)B * ((T + bwd::C - 1) / bwd::C);
    // with no chunk anywhere only the state-gradient chain runs (dS0 = dS_T)
    const int nseq = num_seqs;
    if (bf16) {
        if (dk == 64) return bwd::launch<bf16_t, 64>(p, nslot, nseq, stream);
        return bwd::launch<bf16_t, 128>(p, nslot, nseq, stream);
    }
    if (dk == 64) return bwd::launch<float, 64>(p, nslot, nseq, stream);
    return bwd::launch<float, 128>(p, nslot, nseq, stream);
}

}  // namespace kda
