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
// fp32 inputs, four launches (all arithmetic fp32: MFMA 16x16x4 for the
// products, VALU for the pairwise decay sums):
//   bwd_prep_kernel    one workgroup per (chunk, head): M0, P (pairwise, no
//                      exponent ever positive) and T by forward substitution;
//   bwd_states_kernel  one per (sequence, head, 32-column slice of d_v): the
//                      forward state chain, storing the state entering each chunk;
//   bwd_dstates_kernel same units, chunks in reverse: the state-gradient chain,
//                      storing D for each chunk, and dS0;
//   bwd_grads_kernel   one per (chunk, head): every input gradient of the chunk.
// bf16 inputs (products on bf16 MFMA 16x16x32 with fp32 accumulation):
//   the forward's fused chunk kernel (kda_chunked_ws.hip) in its saving
//   instantiation: M0, P, T and the forward state chain, storing the state
//   entering each chunk with X and U;
//   bwd_dstates_bf16_kernel  the state-gradient chain (64-column slices; four
//                            waves stage each chunk's operands while four
//                            others carry 16-column strips of D);
//   bwd_grads_bf16_kernel    the chunk gradients where every pairwise decay
//                            factor stays below 2^64 (factorised), and
//   bwd_grads_kernel         the exact instantiation for the other chunks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kda_device.h"

namespace kda {
int chunked_slice_width(int units, int dv);
hipError_t chunked_ws_save_launch(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, int gate, const float *S0,
                                  const int32_t *cu_seqlens, int nseq, int T, int H, int dk, int dv,
                                  int slice_width, bf16_t *wS, bf16_t *wX, bf16_t *wU, bf16_t *wTt,
                                  bf16_t *wPt, float *wT, float *wM, float *wP, int32_t *wF,
                                  hipStream_t stream);

namespace bwd {

constexpr int C = 32;        // chunk length
constexpr int NT = 256;      // threads per workgroup
constexpr int NT2 = 512;     // threads of the bf16 gradient kernel
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
    bf16_t *wX, *wU, *wdU;            // bf16 inputs: X, U, dU of each chunk (C x d_v); dX is dv
    bf16_t *wTt, *wPt;                // bf16 inputs: T^T and P^T (C x C) for the gradient chain
    int32_t *wF;                     // per (chunk slot, head): 1 = exact path
};

// A chunk takes the factorised path (K_dn = K e^{-Gamma} as an MFMA operand)
// when every channel's total log2 decay is at least -64, so that e^{-Gamma}
// stays below 2^64; otherwise every pairwise decay factor is formed directly.
constexpr float kFastMinLog2 = -64.0f;

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

// bf16 MFMA: v_mfma_f32_16x16x32_bf16
__device__ __forceinline__ f32x4 mfma8(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// acc += A B^T for one 16 x 16 tile: A [m][k] and Bt [n][k] bf16 row-major
// with pitches la, lb (multiples of 8), K a multiple of 32.
__device__ __forceinline__ f32x4 mmb(f32x4 acc, const __bf16 *A, int la, const __bf16 *Bt, int lb,
                                     int K) {
    const int lane = threadIdx.x & 63, r = lane & 15, j = lane >> 4;
    const __bf16 *pa = A + r * la + 8 * j;
    const __bf16 *pb = Bt + r * lb + 8 * j;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 32)
        acc = mfma8(*reinterpret_cast<const bf16x8 *>(pa + k0), *reinterpret_cast<const bf16x8 *>(pb + k0),
                    acc);
    return acc;
}

__device__ __forceinline__ __bf16 bf(float x) { return (__bf16)x; }
__device__ __forceinline__ float fb(__bf16 x) { return (float)x; }

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

// NE consecutive elements of one row, fetched with 16-byte (or 8-byte) loads
// and kept as raw bits until used, so that a batch of loads is in flight
// before the first wait.  A masked segment reads offset 0 (always a valid
// address) and yields zeros.
template <typename Tin, int NE> struct Seg;
template <int NE> struct Seg<bf16_t, NE> {
    static_assert(NE == 4 || NE % 8 == 0, "segment length");
    uint32_t w[NE / 2];
    bool ok;
    __device__ __forceinline__ void load(const void *base, size_t off, bool valid) {
        ok = valid;
        const bf16_t *q = static_cast<const bf16_t *>(base) + (valid ? off : 0);
        if constexpr (NE == 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(q);
            w[0] = v.x;
            w[1] = v.y;
        } else {
#pragma unroll
            for (int j = 0; j < NE / 8; ++j) {
                const uint4 v = reinterpret_cast<const uint4 *>(q)[j];
                w[4 * j] = v.x;
                w[4 * j + 1] = v.y;
                w[4 * j + 2] = v.z;
                w[4 * j + 3] = v.w;
            }
        }
    }
    __device__ __forceinline__ float get(int j) const {
        const uint32_t x = w[j >> 1];
        const float f = __uint_as_float((j & 1) ? (x & 0xffff0000u) : (x << 16));
        return ok ? f : 0.0f;
    }
};
template <int NE> struct Seg<float, NE> {
    static_assert(NE % 4 == 0, "segment length");
    float w[NE];
    bool ok;
    __device__ __forceinline__ void load(const void *base, size_t off, bool valid) {
        ok = valid;
        const float *q = static_cast<const float *>(base) + (valid ? off : 0);
#pragma unroll
        for (int j = 0; j < NE / 4; ++j) {
            const float4 v = reinterpret_cast<const float4 *>(q)[j];
            w[4 * j] = v.x;
            w[4 * j + 1] = v.y;
            w[4 * j + 2] = v.z;
            w[4 * j + 3] = v.w;
        }
    }
    __device__ __forceinline__ float get(int j) const { return ok ? w[j] : 0.0f; }
};
// one element, kept as raw bits until used (a conversion at load time would
// make the compiler wait for the load right there)
template <typename Tin> struct One;
template <> struct One<float> {
    float w;
    bool ok;
    __device__ __forceinline__ void load(const void *base, size_t off, bool valid) {
        ok = valid;
        w = static_cast<const float *>(base)[valid ? off : 0];
    }
    __device__ __forceinline__ float get() const { return ok ? w : 0.0f; }
};
template <> struct One<bf16_t> {
    uint32_t w;
    bool ok;
    __device__ __forceinline__ void load(const void *base, size_t off, bool valid) {
        ok = valid;
        w = static_cast<const bf16_t *>(base)[valid ? off : 0].x;
    }
    __device__ __forceinline__ float get() const { return ok ? __uint_as_float(w << 16) : 0.0f; }
};

// NE (4 or 8) consecutive fp32 of an LDS row as 16-byte accesses.  With
// 8, lane groups 4-7 and 8-11 of each 16 take the upper half first, so that
// the first (and the second) access of 8 or 16 neighbouring lanes covers
// distinct banks instead of every other 16-byte column twice.
__device__ __forceinline__ bool row4_swap() {
    const int l = threadIdx.x & 15;
    return (((l >> 2) ^ (l >> 3)) & 1) != 0;
}
// (the halves are chosen element by element and addressed by offset: a
// select between whole vectors becomes a private array in scratch memory)
template <int NE> __device__ __forceinline__ void row4_put(float *dst, const float *v) {
    if constexpr (NE == 4) {
        *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
        const bool sw = row4_swap();
        const int o = sw ? 4 : 0;
        *reinterpret_cast<float4 *>(dst + o) = make_float4(sw ? v[4] : v[0], sw ? v[5] : v[1],
                                                           sw ? v[6] : v[2], sw ? v[7] : v[3]);
        *reinterpret_cast<float4 *>(dst + (4 - o)) = make_float4(sw ? v[0] : v[4], sw ? v[1] : v[5],
                                                                 sw ? v[2] : v[6], sw ? v[3] : v[7]);
    }
}
template <int NE> __device__ __forceinline__ void row4_get(const float *src, float *v) {
    if constexpr (NE == 4) {
        const float4 a = *reinterpret_cast<const float4 *>(src);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    } else {
        const bool sw = row4_swap();
        const int o = sw ? 4 : 0;
        const float4 a = *reinterpret_cast<const float4 *>(src + o);
        const float4 b = *reinterpret_cast<const float4 *>(src + (4 - o));
        v[0] = sw ? b.x : a.x; v[1] = sw ? b.y : a.y; v[2] = sw ? b.z : a.z; v[3] = sw ? b.w : a.w;
        v[4] = sw ? a.x : b.x; v[5] = sw ? a.y : b.y; v[6] = sw ? a.z : b.z; v[7] = sw ? a.w : b.w;
    }
}

// The rows of one chunk that every kernel reads: k (and q) and the gate,
// thread t holding row t / TPROW, channels (t % TPROW) * DK/TPROW onwards
// (TPROW threads per row: 8 with 256 threads, 16 with 512); beta of row t.
template <typename Tin, int DK, bool WITH_Q, int TPROW = 8> struct ChunkIn {
    static constexpr int NE = DK / TPROW, DKP = DK + 1;
    Seg<Tin, NE> k, q, g;
    One<Tin> gh, b;
    // Every load is issued unconditionally (an unused one reads offset 0 of a
    // valid tensor), so that no value merges across branches and forces an
    // early wait.
    __device__ __forceinline__ void load(const Params &p, long t0, int cl, int h) {
        const int tid = threadIdx.x, r = tid / TPROW, c0 = (tid % TPROW) * NE;
        const bool ok = r < cl;
        const size_t e = ((size_t)(t0 + r) * p.H + h) * DK + c0;
        k.load(p.k, e, ok);
        if constexpr (WITH_Q) q.load(p.q, e, ok);
        const bool ch = p.gate == GATE_CHANNEL, hd = p.gate == GATE_HEAD;
        g.load(ch ? p.g : p.k, e, ok && ch);
        gh.load(hd ? p.g : p.beta, (size_t)(t0 + r) * p.H + h, ok && hd);
        b.load(p.beta, (size_t)(t0 + tid) * p.H + h, tid < cl && tid < C);
    }
    // raw k (q), log2 gates and beta into LDS
    __device__ __forceinline__ void store(const Params &p, float *sK, float *sQ, float *sG, float *sB) const {
        const int tid = threadIdx.x, r = tid / TPROW, c0 = (tid % TPROW) * NE;
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            sK[r * DKP + c0 + j] = k.get(j);
            if constexpr (WITH_Q) sQ[r * DKP + c0 + j] = q.get(j);
            float gv = 0.0f;
            if (p.gate == GATE_CHANNEL) gv = g.get(j) * kLog2e;
            else if (p.gate == GATE_HEAD) gv = gh.get() * kLog2e;
            sG[r * DKP + c0 + j] = gv;
        }
        if (tid < C) sB[tid] = b.get();
    }
    // only the log2 gates (row pitch PITCH, a multiple of 4) and beta (k and q
    // stay in the registers), the row segment as 16-byte stores (row4_put)
    template <int PITCH>
    __device__ __forceinline__ void store_gb(const Params &p, float *sG, float *sB) const {
        static_assert(NE == 4 || NE == 8, "row segment of one or two 16-byte stores");
        const int tid = threadIdx.x, r = tid / TPROW, c0 = (tid % TPROW) * NE;
        float gv[NE];
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            gv[j] = 0.0f;
            if (p.gate == GATE_CHANNEL) gv[j] = g.get(j) * kLog2e;
            else if (p.gate == GATE_HEAD) gv[j] = gh.get() * kLog2e;
        }
        row4_put<NE>(sG + r * PITCH + c0, gv);
        if (tid < C) sB[tid] = b.get();
    }
};

// Buffer descriptor over the memory from `base` on (scalar registers; any
// offset from 2^31 on is out of bounds: its stores are dropped).  The bf16
// gradient chain stores its tiles through these, masking rows past the
// sequence end with an out-of-bounds offset instead of a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void *base) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *u = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, 0, 0x7ffffff0, 0x00020000);
}
constexpr uint32_t kDrop = 0x80000000u;   // out-of-bounds offset: the store is dropped
__device__ __forceinline__ void bst16(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, off, 0, 0);
}
// a value the compiler may neither recompute nor share: pinned in a register
template <typename T> __device__ __forceinline__ T pinned(T x) {
    asm volatile("" : "+v"(x));
    return x;
}

// One 16 x 16 tile of a (d_k x d_v) fp32 state from global memory (or zeros),
// as this lane's four accumulator rows.
__device__ __forceinline__ void load_tile(f32x4 &t, const float *src, size_t row0, int ld, int col) {
    const int lane = threadIdx.x & 63, lr = lane & 15, lj = lane >> 4;
    if (!src) {
        t = f32x4{0.f, 0.f, 0.f, 0.f};
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = src[(row0 + 4 * lj + i) * ld + col + lr];
}

// Running sums of the log2 gates down each channel (in place), their totals
// gc and gamma = 2^gc.  Threads below DK take one channel each.  DKP is the
// row pitch of sG.
template <int DK, int DKP = DK + 1>
__device__ __forceinline__ void gate_sums(float *sG, float *gc, float *gam) {
    const int tid = threadIdx.x;
    if (tid < DK) {
        float x[C];
#pragma unroll
        for (int r = 0; r < C; ++r) x[r] = sG[r * DKP + tid];
        float run = 0.0f;
#pragma unroll
        for (int r = 0; r < C; ++r) {
            run += x[r];
            sG[r * DKP + tid] = run;
        }
        if (gc) gc[tid] = run;
        if (gam) gam[tid] = __builtin_amdgcn_exp2f(run);
    }
}

// K_up = k 2^G, Q_up = q 2^G, K_right = k 2^{G_c - G} on this thread's row
// segment (sG may be sKrt: each element is read before it is overwritten).
template <int DK, bool WITH_Q>
__device__ __forceinline__ void scale_rows(float *sKup, float *sQup, const float *sG, float *sKrt,
                                           const float *gc) {
    constexpr int NE = DK / 8, DKP = DK + 1;
    const int tid = threadIdx.x, r = tid >> 3, c0 = (tid & 7) * NE;
#pragma unroll
    for (int j = 0; j < NE; ++j) {
        const int o = r * DKP + c0 + j;
        const float G = sG[o], kv = sKup[o];
        const float E = __builtin_amdgcn_exp2f(G);
        sKup[o] = kv * E;
        if constexpr (WITH_Q) sQup[o] *= E;
        sKrt[o] = kv * __builtin_amdgcn_exp2f(gc[c0 + j] - G);
    }
}

// ---------------------------------------------------------------------------
// M0, P and T of one chunk.
template <typename Tin, int DK>
__global__ void __launch_bounds__(NT) bwd_prep_kernel(Params p) {
    constexpr int DKP = DK + 1, NCC = DK / 8, NE = DK / 8;
    __shared__ __attribute__((aligned(16))) float sKQ[2 * C * DKP];
    __shared__ float sG[C * DKP];
    __shared__ float sM[C * CP], sP[C * CP], sT[C * CP], sY[16 * 17], sB[C], gc[DK];
    float *sK = sKQ, *sQ = sKQ + C * DKP;
    const long slot = blockIdx.x;
    const int h = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    long t0;
    int cl;
    if (!slot_chunk(p, slot, t0, cl)) return;
    {
        ChunkIn<Tin, DK, true> in;
        in.load(p, t0, cl, h);
        in.store(p, sK, sQ, sG, sB);
    }
    __syncthreads();
    gate_sums<DK>(sG, gc, nullptr);
    const size_t wi = (size_t)slot * p.H + h;
    const bool exact = __syncthreads_or(tid < DK && !(gc[tid] >= kFastMinLog2));
    if (tid == 0) p.wF[wi] = exact ? 1 : 0;
    if (!exact) {
        // K_up = k 2^G, Q_up = q 2^G, K_dn = k 2^-G; then M0 = K_up K_dn^T
        // (strictly lower) and P = Q_up K_dn^T (lower) on fp32 MFMA
        const int r = tid >> 3, c0 = (tid & 7) * NE;
        const int tm = wave >> 1, tn = wave & 1, lr = lane & 15, lj = lane >> 4;
        f32x4 m = {0.f, 0.f, 0.f, 0.f}, pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            const int o = r * DKP + c0 + j;
            const float G = sG[o], kv = sK[o];
            sK[o] = kv * __builtin_amdgcn_exp2f(G);
            sQ[o] *= __builtin_amdgcn_exp2f(G);
            sG[o] = kv * __builtin_amdgcn_exp2f(-G);
        }
        __syncthreads();
        m = mm(m, sK + 16 * tm * DKP, DKP, 1, sG + 16 * tn * DKP, 1, DKP, DK);
        pp = mm(pp, sQ + 16 * tm * DKP, DKP, 1, sG + 16 * tn * DKP, 1, DKP, DK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * tm + 4 * lj + i, col = 16 * tn + lr;
            sM[row * CP + col] = col < row ? m[i] : 0.0f;
            sP[row * CP + col] = col <= row ? pp[i] : 0.0f;
        }
    } else {
        // pairwise sums: thread (row r, channel group cg) over channels cg + 8 cc
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
    float *gT = p.wT + wi * C * C, *gP = p.wP + wi * C * C, *gM = p.wM + wi * C * C;
    {
        const int r = (tid * 4) / C, i = (tid * 4) % C;
        *reinterpret_cast<float4 *>(gP + tid * 4) =
            make_float4(sP[r * CP + i], sP[r * CP + i + 1], sP[r * CP + i + 2], sP[r * CP + i + 3]);
        *reinterpret_cast<float4 *>(gM + tid * 4) =
            make_float4(sM[r * CP + i], sM[r * CP + i + 1], sM[r * CP + i + 2], sM[r * CP + i + 3]);
    }
    // T = (I + A)^{-1}, A = Diag(beta) M0 strictly lower, by 16 x 16 blocks:
    // the diagonal blocks by substitution (lane l: block l / 16, column
    // l % 16; T_ri = [r == i] - sum_{j < r} A_rj T_ji), then
    // T_10 = -T_11 A_10 T_00 on MFMA; T_01 = 0.
    if (tid < C) {
        const int b = tid >> 4, i = tid & 15, o = 16 * b;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < r; ++j) acc += sM[(o + r) * CP + o + j] * t[j];
            t[r] = (r == i ? 1.0f : 0.0f) - sB[o + r] * acc;
            sT[(o + r) * CP + o + i] = t[r];
            sT[(o + r) * CP + (16 - o) + i] = 0.0f;        // T_01 (rewritten below for T_10)
        }
    }
    __syncthreads();
    if (wave == 0) {
        const int lr = lane & 15, lj = lane >> 4;
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        y = mm(y, sM + 16 * CP, CP, 1, sT, CP, 1, 16);   // M0_10 T_00
#pragma unroll
        for (int i = 0; i < 4; ++i) sY[(4 * lj + i) * 17 + lr] = sB[16 + 4 * lj + i] * y[i];
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
        t = mm(t, sT + 16 * CP + 16, CP, 1, sY, 17, 1, 16);  // T_11 (A_10 T_00)
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[(16 + 4 * lj + i) * CP + lr] = -t[i];
    }
    __syncthreads();
    {
        const int r = (tid * 4) / C, i = (tid * 4) % C;
        *reinterpret_cast<float4 *>(gT + tid * 4) =
            make_float4(sT[r * CP + i], sT[r * CP + i + 1], sT[r * CP + i + 2], sT[r * CP + i + 3]);
    }
}

// ---------------------------------------------------------------------------
// Forward state chain of one (sequence, head, slice): the state entering
// every chunk goes to the workspace.  The next chunk's inputs are requested
// while the current one is computed.
template <typename Tin, int DK>
__global__ void __launch_bounds__(NT) bwd_states_kernel(Params p) {
    constexpr int DKP = DK + 1, NTW = DK / 32;   // state tiles per wave
    __shared__ float sS[DK * WP], sKup[C * DKP], sKrt[C * DKP], sV[C * WP], sU[C * WP],
        sT[C * CP], gc[DK], gam[DK], sB[C];
    const int nsl = p.DV / W;
    const int unit = blockIdx.x / nsl, slice = blockIdx.x % nsl;
    const int s = unit / p.H, h = unit % p.H, col0 = slice * W;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lj = lane >> 4;
    const int vr = tid >> 3, vc = (tid & 7) * 4;          // this thread's 4 values of a C x W tile
    long t0s, base;
    int len;
    seq_info(p, s, t0s, len, base);
    const int nch = (len + C - 1) / C;
    ChunkIn<Tin, DK, false> in;
    Seg<Tin, 4> vin;
    Seg<float, 4> tin;
    auto issue = [&](int n) {
        const long t0 = t0s + (long)n * C;
        const int cl = len - n * C < C ? len - n * C : C;
        in.load(p, t0, cl, h);
        vin.load(p.v, ((size_t)(t0 + vr) * p.H + h) * p.DV + col0 + vc, vr < cl);
        tin.load(p.wT, ((size_t)(base + n) * p.H + h) * C * C + tid * 4, true);
    };
    if (nch > 0) issue(0);
    // state tiles of this wave: tile index w * NTW + x -> (tm, tn) over (DK/16) x (W/16)
    f32x4 S[NTW];
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
        const int tt = wave * NTW + x, tm = tt >> 1, tn = tt & 1;
        load_tile(S[x], p.S0, ((size_t)s * p.H + h) * DK + 16 * tm, p.DV, col0 + 16 * tn);
    }
    for (int n = 0; n < nch; ++n) {
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
        in.store(p, sKup, nullptr, sKrt, sB);     // sKrt holds the gate sums first
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sV[vr * WP + vc + j] = vin.get(j);
            sT[((tid * 4) / C) * CP + (tid * 4) % C + j] = tin.get(j);
        }
        if (n + 1 < nch) issue(n + 1);
        __syncthreads();
        gate_sums<DK>(sKrt, gc, gam);
        __syncthreads();
        scale_rows<DK, false>(sKup, nullptr, sKrt, sKrt, gc);
        __syncthreads();
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
// the gradient of the initial state to dS0.  The next chunk's inputs are
// requested while the current one is computed.
template <typename Tin, int DK>
__global__ void __launch_bounds__(NT) bwd_dstates_kernel(Params p) {
    constexpr int DKP = DK + 1, NTW = DK / 32;
    __shared__ float sD[DK * WP], sKup[C * DKP], sQup[C * DKP], sKrt[C * DKP], sdO[C * WP],
        sdU[C * WP], sdX[C * WP], sT[C * CP], sP[C * CP], gc[DK], gam[DK], sB[C];
    const int nsl = p.DV / W;
    const int unit = blockIdx.x / nsl, slice = blockIdx.x % nsl;
    const int s = unit / p.H, h = unit % p.H, col0 = slice * W;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lj = lane >> 4;
    const int vr = tid >> 3, vc = (tid & 7) * 4;
    long t0s, base;
    int len;
    seq_info(p, s, t0s, len, base);
    const int nch = (len + C - 1) / C;
    const size_t so = ((size_t)s * p.H + h) * DK;
    ChunkIn<Tin, DK, true> in;
    Seg<Tin, 4> oin;
    Seg<float, 4> tin, pin;
    auto issue = [&](int n) {
        const long t0 = t0s + (long)n * C;
        const int cl = len - n * C < C ? len - n * C : C;
        const size_t wi = (size_t)(base + n) * p.H + h;
        in.load(p, t0, cl, h);
        oin.load(p.dO, ((size_t)(t0 + vr) * p.H + h) * p.DV + col0 + vc, vr < cl);
        tin.load(p.wT, wi * C * C + tid * 4, true);
        pin.load(p.wP, wi * C * C + tid * 4, true);
    };
    if (nch > 0) issue(nch - 1);
    f32x4 D[NTW];
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
        const int tt = wave * NTW + x, tm = tt >> 1, tn = tt & 1;
        load_tile(D[x], p.dST, so + 16 * tm, p.DV, col0 + 16 * tn);
    }
    for (int n = nch - 1; n >= 0; --n) {
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
        in.store(p, sKup, sQup, sKrt, sB);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tr = (tid * 4) / C, tc = (tid * 4) % C + j;
            sdO[vr * WP + vc + j] = oin.get(j);
            sT[tr * CP + tc] = tin.get(j);
            sP[tr * CP + tc] = pin.get(j);
        }
        if (n > 0) issue(n - 1);
        __syncthreads();
        gate_sums<DK>(sKrt, gc, gam);
        __syncthreads();
        scale_rows<DK, true>(sKup, sQup, sKrt, sKrt, gc);
        __syncthreads();
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

template <typename Tin, int DK, bool EXACT>
__global__ void __launch_bounds__(NT) bwd_grads_kernel(Params p, long nslot) {
    constexpr int DKP = DK + 1, NTW = DK / 32, NPART = NT / DK;
    constexpr int NES = DK * W / NT, TPR = W / NES;     // S / D slice: NES values per thread
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

    const int h = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lj = lane >> 4;
    const int vr = tid >> 3, vc = (tid & 7) * 4;          // C x W values of this thread
    const int sr = tid / TPR, sc = (tid % TPR) * NES;     // DK x W values of this thread
    auto chunk = [&](long slot) {
        long t0;
        int cl;
        if (!slot_chunk(p, slot, t0, cl)) return;
        const size_t wi = (size_t)slot * p.H + h;
        // each chunk is done by the instantiation of its path (the flag set by
        // the prep kernel, or for bf16 inputs by the forward's chunk kernel)
        if ((p.wF[wi] != 0) != EXACT) return;
        // states and state gradients are stored in the input precision's kind:
        // fp32 for fp32 inputs, bf16 for bf16 inputs
        const Tin *gS = reinterpret_cast<const Tin *>(p.wS) + wi * DK * p.DV;
        const Tin *gD = reinterpret_cast<const Tin *>(p.wD) + wi * DK * p.DV;

        // every load of the chunk, then the first slice's, before the first wait
        Seg<Tin, NES> sin, din;
        Seg<Tin, 4> vin, oin;
        auto issue_slice = [&](int col0) {
            sin.load(gS, std::is_same<Tin, bf16_t>::value ? strip_off(sr, col0 + sc, DK)
                                                          : (size_t)sr * p.DV + col0 + sc, true);
            din.load(gD, std::is_same<Tin, bf16_t>::value ? strip_off(sr, col0 + sc, DK)
                                                          : (size_t)sr * p.DV + col0 + sc, true);
            const size_t e = ((size_t)(t0 + vr) * p.H + h) * p.DV + col0 + vc;
            vin.load(p.v, e, vr < cl);
            oin.load(p.dO, e, vr < cl);
        };
        {
            ChunkIn<Tin, DK, true> in;
            Seg<float, 4> tin, pin, min;
            in.load(p, t0, cl, h);
            tin.load(p.wT, wi * C * C + tid * 4, true);
            pin.load(p.wP, wi * C * C + tid * 4, true);
            min.load(p.wM, wi * C * C + tid * 4, true);
            issue_slice(0);
            in.store(p, sKup, sQup, sG, sB);
            const int tr = (tid * 4) / C, tc = (tid * 4) % C;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sT[tr * CP + tc + j] = tin.get(j);
                sP[tr * CP + tc + j] = pin.get(j);
                sM[tr * CP + tc + j] = min.get(j);
            }
        }
        if (tid < C) dB[tid] = 0.0f;
        if (tid < DK) dgam[tid] = 0.0f;
        __syncthreads();
        gate_sums<DK>(sG, gc, gam);
        __syncthreads();
        scale_rows<DK, true>(sKup, sQup, sG, sKrt, gc);

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
#pragma unroll
            for (int j = 0; j < NES; ++j) {
                sS[sr * WP + sc + j] = sin.get(j);
                sD[sr * WP + sc + j] = din.get(j);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sX[vr * WP + vc + j] = vin.get(j);
                sdO[vr * WP + vc + j] = oin.get(j);
            }
            if (col0 + W < p.DV) issue_slice(col0 + W);
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
#pragma unroll 8
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
#pragma unroll 8
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
#pragma unroll 8
            for (int i = 0; i < C; ++i) {
                const float a = sdA[r * WP + i];
                acc += a * sM[r * CP + i];
                sM[r * CP + i] = sB[r] * a;
            }
            dB[r] += acc;
        }
        __syncthreads();

        float *sRK = sS;                     // C x DKP: dK_right K_right
        if constexpr (!EXACT) {
            // factorised decay: with K_dn = K e^{-Gamma},
            //   Z1 = dP K_dn,  Z2 = dM K_dn,  Z3 = dM^T K_up + dP^T Q_up,
            //   dq = (dQ_up + Z1) e^G,  dk = (dK_up + Z2) e^G + dK_right e^{G_c - G} + Z3 e^{-G},
            //   dGamma = (dK_up + Z2) K_up + (dQ_up + Z1) Q_up - dK_right K_right - Z3 K_dn
            float *sKdn = sD;                // C x DKP
            {
                constexpr int NE = DK / 8;
                const int r = tid >> 3, c0 = (tid & 7) * NE;
                Seg<Tin, NE> kin;
                kin.load(p.k, ((size_t)(t0 + r) * p.H + h) * DK + c0, r < cl);
#pragma unroll
                for (int j = 0; j < NE; ++j) {
                    const int o = r * DKP + c0 + j;
                    sKdn[o] = kin.get(j) * __builtin_amdgcn_exp2f(-sG[o]);
                }
            }
            __syncthreads();
            f32x4 zrk[NTW];                  // dK_right K_right, stored after the barrier below
#pragma unroll
            for (int x = 0; x < NTW; ++x) {
                const int tt = wave * NTW + x, m0 = 16 * (tt / (DK / 16)), n0 = 16 * (tt % (DK / 16));
                f32x4 z1 = {0.f, 0.f, 0.f, 0.f}, z2 = z1, z3 = z1;
                z1 = mm(z1, sdP + m0 * WP, WP, 1, sKdn + n0, DKP, 1, C);
                z2 = mm(z2, sM + m0 * CP, CP, 1, sKdn + n0, DKP, 1, C);
                z3 = mm(z3, sM + m0, 1, CP, sKup + n0, DKP, 1, C);
                z3 = mm(z3, sdP + m0, 1, WP, sQup + n0, DKP, 1, C);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + 4 * lj + i, col = n0 + lr, o = row * DKP + col;
                    const float G = sG[o], E = __builtin_amdgcn_exp2f(G);
                    const float R = __builtin_amdgcn_exp2f(gc[col] - G);
                    const float Ei = __builtin_amdgcn_exp2f(-G);
                    // aK holds -dK_up
                    const float dQu = aQ[x][i] + z1[i], dKu = z2[i] - aK[x][i], dKr = aR[x][i];
                    const float ku = sKup[o], qu = sQup[o], kr = sKrt[o], kd = sKdn[o];
                    aQ[x][i] = dQu * E;
                    aK[x][i] = dKu * E + dKr * R + z3[i] * Ei;
                    aR[x][i] = dKu * ku + dQu * qu - dKr * kr - z3[i] * kd;
                    zrk[x][i] = dKr * kr;
                }
            }
            __syncthreads();
#pragma unroll
            for (int x = 0; x < NTW; ++x) {
                const int tt = wave * NTW + x, m0 = 16 * (tt / (DK / 16)), n0 = 16 * (tt % (DK / 16));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int o = (m0 + 4 * lj + i) * DKP + n0 + lr;
                    sQup[o] = aQ[x][i];
                    sKup[o] = aK[x][i];
                    sKrt[o] = aR[x][i];
                    sRK[o] = zrk[x][i];
                }
            }
            __syncthreads();
        } else {
        // direct terms, element by element where the tiles lie:
        //   dq = dQ_up e^G,  dk = dK_up e^G + dK_right e^{G_c - G},
        //   dGamma = dK_up K_up + dQ_up Q_up - dK_right K_right,
        // and dK_right K_right kept for the chunk-total term
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
                kc[r] = ld<Tin>(p.k, e);
                qc[r] = ld<Tin>(p.q, e);
                kc[r] = ok ? kc[r] : 0.0f;
                qc[r] = ok ? qc[r] : 0.0f;
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
        }
        // dlog_alpha: reverse running sum of dGamma plus the chunk-total term
        // sum_r dK_right K_right + dgamma gamma; outputs
        if (tid < DK) {
            const int c = tid;
            float x[C];
            float tot = dgam[c] * gam[c];
#pragma unroll
            for (int r = 0; r < C; ++r) {
                tot += sRK[r * DKP + c];
                x[r] = sKrt[r * DKP + c];
            }
            float run = tot;
#pragma unroll
            for (int r = C - 1; r >= 0; --r) {
                run += x[r];
                sKrt[r * DKP + c] = run;
            }
        }
        __syncthreads();
        {
            constexpr int NE = DK / 8;
            const int r = tid >> 3, c0 = (tid & 7) * NE;
            if (r < cl) {
                const size_t e = ((size_t)(t0 + r) * p.H + h) * DK + c0;
#pragma unroll
                for (int j = 0; j < NE; ++j) {
                    st<Tin>(p.dq, e + j, sQup[r * DKP + c0 + j]);
                    st<Tin>(p.dk, e + j, sKup[r * DKP + c0 + j]);
                    if (p.gate == GATE_CHANNEL) st<Tin>(p.dg, e + j, sKrt[r * DKP + c0 + j]);
                }
            }
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
    };
    if constexpr (EXACT) {
        // exact chunks are rare: a reduced grid strides over the slots, NT of
        // them at a time, whose flags the threads read together first
        const long step = gridDim.x;
        for (long first = blockIdx.x; first < nslot; first += step * NT) {
            const long mine = first + tid * step;
            long t0;
            int cl;
            const bool ex = mine < nslot && slot_chunk(p, mine, t0, cl) && p.wF[(size_t)mine * p.H + h] != 0;
            if (!__syncthreads_or(ex)) continue;
            for (int j = 0; j < NT && first + j * step < nslot; ++j) {
                chunk(first + j * step);
                __syncthreads();                      // this chunk is done with LDS
            }
        }
    } else {
        chunk(blockIdx.x);
    }
}


// ---------------------------------------------------------------------------
// bf16 inputs: the state-gradient chain, pipelined over two wave groups.
//
// The chain is separable over d_v columns: column j of
//   dU = P^T dO + K_right D,   dX = Diag(beta) T^T dU,
//   D  <- Diag(gamma) D + Q_up^T dO - K_up^T dX
// reads column j of D, dO and dX and the chunk's matrices only.  So each of
// the four consumer waves of a workgroup (one per sequence, head and
// 64-column slice of d_v) owns a 16-column strip of the slice, keeps its
// strip of D (d_k x 16, fp32) in MFMA accumulators for the whole sequence
// and runs the three products with no synchronisation between waves.  The
// four producer waves meanwhile build the next chunk's operands in the other
// of two LDS slots: running log2 gate sums per key channel, K_right
// (row-major), Q_up^T and -K_up^T, gamma, and T^T, P^T and dO^T as they come
// from memory.  One barrier per chunk hands a slot over.
//
// Accumulator rows are ordered by crow(rho, h, m) = 32 rho + 8 (m >> 2) +
// 4 h + (m & 3): a lane's four values of tiles (rho, 0) and (rho, 1) are then
// exactly its eight k-slots of run rho of a v_mfma_f32_16x16x32_bf16 B
// operand, so D, dU and dX feed the next product straight from registers
// (the A operands are read at the matching permuted rows).
// Arithmetic as before this split: bf16 operands, fp32 accumulation, D kept
// fp32 and rounded to bf16 as an operand and for the workspace.
constexpr int W2 = 64;                 // d_v columns per chain workgroup
constexpr int CTP = C + 8;             // pitch of bf16 [*][C] operand rows
template <int DK> struct ChainSlot {
    static constexpr int KRP = DK + 8;
    static constexpr int KR = 0;                         // bf16 [C][KRP]: K_right
    static constexpr int QT = KR + 2 * C * KRP;          // bf16 [DK][CTP]: Q_up^T
    static constexpr int KT = QT + 2 * DK * CTP;         // bf16 [DK][CTP]: -K_up^T
    static constexpr int TT = KT + 2 * DK * CTP;         // bf16 [C][CTP]: T^T
    static constexpr int PT = TT + 2 * C * CTP;          // bf16 [C][CTP]: P^T
    static constexpr int OT = PT + 2 * C * CTP;          // bf16 [W2][CTP]: dO^T
    static constexpr int GAM = OT + 2 * W2 * CTP;        // fp32 [DK]: gamma
    static constexpr int BETA = GAM + 4 * DK;            // fp32 [C]
    static constexpr int BYTES = BETA + 4 * C;
    static_assert(BYTES % 16 == 0, "slot alignment");
};
__device__ __forceinline__ int crow(int rho, int h, int m) {
    return 32 * rho + 8 * (m >> 2) + 4 * h + (m & 3);
}
__device__ __forceinline__ bf16x8 frag2(f32x4 lo, f32x4 hi) {
    bf16x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = (__bf16)lo[i];
        f[4 + i] = (__bf16)hi[i];
    }
    return f;
}

// (sequence-head unit, d_v slice) of a chain workgroup.  With two slices per
// unit and a multiple of 8 units, the slices of a unit are numbered 8 apart:
// workgroups b and b + 8 run on the same XCD, so the second read of the
// chunk's shared inputs (k, q, gates, T^T, P^T) is served from that XCD's L2.
__device__ __forceinline__ void chain_unit(const Params &p, int b, int &unit, int &slice) {
    const int nsl = p.DV / W2;
    const long units = (long)p.num_seqs * p.H;
    if (nsl == 2 && units % 8 == 0) {
        unit = (b >> 4) * 8 + (b & 7);
        slice = (b >> 3) & 1;
    } else {
        unit = b / nsl;
        slice = b % nsl;
    }
}

// Buffer descriptor over `bytes` bytes from `base` (scalar registers): a load
// past the end reads zeros, which masks rows past a chunk's end for free.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc_n(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *u = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, 0, bytes, 0x00020000);
}

// DPP helpers for the producer's scans: lane i of a row of 16 receives
// x from lane i - s (0 below the row start), or lane n's x.
template <int S> __device__ __forceinline__ float dpp_shr(float x) {
    return __builtin_amdgcn_update_dpp(0.0f, x, 0x110 + S, 0xf, 0xf, false);
}
template <int N> __device__ __forceinline__ float dpp_bcast(float x) {
    return __builtin_amdgcn_update_dpp(0.0f, x, 0x150 + N, 0xf, 0xf, false);
}
// x plus, where `take`, the x of the lane S below.  The shifted copy is
// pinned so that it is formed in every lane: moved under the condition, the
// DPP move would run with the source lanes switched off and read nothing.
template <int S> __device__ __forceinline__ float add_from_below(float x, bool take) {
    const float y = pinned(dpp_shr<S>(x));
    return x + (take ? y : 0.0f);
}

// What one producer thread (pt = 0..255) reads of a chunk: four key
// channels 4 cq .. 4 cq + 3 over RPB consecutive rows RPB rb .. (8-byte
// loads of g, k and q), with rb = lane % NRB running over the NRB row blocks
// within a group of NRB lanes and cq over the groups; four values of T^T and
// of P^T; eight columns of one dO row; beta of row pt.  Buffer loads over
// the chunk's valid rows only: rows past its end read 0.
template <int DK> struct ChainIn {
    static constexpr int RPB = C * DK / 1024;          // 4 (d_k = 128) or 2 (64)
    static constexpr int NRB = C / RPB;                // 8 or 16 row blocks
    uint2 g[RPB], k[RPB], q[RPB];
    uint32_t b;
    uint2 tt, pt;
    uint4 o;
    __device__ __forceinline__ void load(const Params &p, long t0, int cl, int h, size_t wi, int col0, int ptid) {
        const int lane = ptid & 63, rb = lane % NRB, cq = (ptid >> 6) * (64 / NRB) + lane / NRB;
        const uint32_t tokk = (uint32_t)p.H * DK * 2u, tokh = (uint32_t)p.H * 2u;   // bytes between rows
        const size_t rowk = ((size_t)t0 * p.H + h) * DK, rowh = (size_t)t0 * p.H + h;
        const bf16_t *gk = static_cast<const bf16_t *>(p.k), *gq = static_cast<const bf16_t *>(p.q);
        const bf16_t *gg = static_cast<const bf16_t *>(p.g), *gb = static_cast<const bf16_t *>(p.beta);
        const bool ch = p.gate == GATE_CHANNEL, hd = p.gate == GATE_HEAD;
        const __amdgpu_buffer_rsrc_t rk = brsrc_n(gk + rowk, cl * tokk), rq = brsrc_n(gq + rowk, cl * tokk);
        const __amdgpu_buffer_rsrc_t rg =
            brsrc_n(ch ? gg + rowk : hd ? gg + rowh : gk, ch ? cl * tokk : hd ? cl * tokh : 0u);
#pragma unroll
        for (int i = 0; i < RPB; ++i) {
            const uint32_t r = RPB * rb + i, off = r * tokk + 8u * cq;
            k[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, off, 0, 0));
            q[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq, off, 0, 0));
            // a per-head gate: its one value in the low half (spread over the
            // channels when staged; no wait for the load here)
            if (hd) g[i] = make_uint2(__builtin_amdgcn_raw_buffer_load_b16(rg, r * tokh, 0, 0), 0u);
            else g[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rg, off, 0, 0));
        }
        tt = *reinterpret_cast<const uint2 *>(p.wTt + wi * C * C + 4 * ptid);
        pt = *reinterpret_cast<const uint2 *>(p.wPt + wi * C * C + 4 * ptid);
        const uint32_t tokv = (uint32_t)p.H * p.DV * 2u;
        const __amdgpu_buffer_rsrc_t ro =
            brsrc_n(static_cast<const bf16_t *>(p.dO) + ((size_t)t0 * p.H + h) * p.DV + col0, cl * tokv);
        o = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                          ro, (ptid >> 3) * tokv + 16u * (ptid & 7), 0, 0));
        const __amdgpu_buffer_rsrc_t rb_ = brsrc_n(gb + rowh, cl * tokh);
        b = __builtin_amdgcn_raw_buffer_load_b16(rb_, ptid < C ? ptid * tokh : 0x7fffffffu, 0, 0);
    }
    // the chunk's operands into an LDS slot
    __device__ __forceinline__ void stage(const Params &p, unsigned char *slot, int ptid) const {
        using L = ChainSlot<DK>;
        __bf16 *KR = reinterpret_cast<__bf16 *>(slot + L::KR);
        __bf16 *QT = reinterpret_cast<__bf16 *>(slot + L::QT);
        __bf16 *KT = reinterpret_cast<__bf16 *>(slot + L::KT);
        const int lane = ptid & 63, rb = lane % NRB, cq = (ptid >> 6) * (64 / NRB) + lane / NRB;
        const bool gated = p.gate != GATE_NONE;
        auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
        auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
        // running log2-gate sums of this lane's rows (inclusive), per channel
        float G[RPB][4];
#pragma unroll
        for (int i = 0; i < RPB; ++i) {
            const bool hd = p.gate == GATE_HEAD;
            const float x[4] = {lo(g[i].x), hd ? lo(g[i].x) : hi(g[i].x), hd ? lo(g[i].x) : lo(g[i].y),
                                hd ? lo(g[i].x) : hi(g[i].y)};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = gated ? x[j] * kLog2e : 0.0f;
                G[i][j] = i == 0 ? v : G[i - 1][j] + v;
            }
        }
        // exclusive scan of the row-block totals over the NRB lanes of a
        // group, and the chunk total gc (broadcast from the group's last lane)
        float tot[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float x = G[RPB - 1][j];
            x = add_from_below<1>(x, rb >= 1);
            x = add_from_below<2>(x, rb >= 2);
            x = add_from_below<4>(x, rb >= 4);
            if constexpr (NRB == 16) x = add_from_below<8>(x, rb >= 8);
            const float below = pinned(dpp_shr<1>(x));
            const float ex = rb >= 1 ? below : 0.0f;      // sum of the blocks before this one
            if constexpr (NRB == 16) {
                tot[j] = dpp_bcast<15>(x);
            } else {
                const float t7 = dpp_bcast<7>(x), t15 = dpp_bcast<15>(x);
                tot[j] = (lane & 8) ? t15 : t7;
            }
#pragma unroll
            for (int i = 0; i < RPB; ++i) G[i][j] += ex;
        }
        // K_right row-major; Q_up^T and -K_up^T transposed
        bf16x4 qt[4], kt[4];
#pragma unroll
        for (int i = 0; i < RPB; ++i) {
            const float kv[4] = {lo(k[i].x), hi(k[i].x), lo(k[i].y), hi(k[i].y)};
            const float qv[4] = {lo(q[i].x), hi(q[i].x), lo(q[i].y), hi(q[i].y)};
            bf16x4 kr;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float E = __builtin_amdgcn_exp2f(G[i][j]), R = __builtin_amdgcn_exp2f(tot[j] - G[i][j]);
                kr[j] = (__bf16)(kv[j] * R);
                qt[j][i] = (__bf16)(qv[j] * E);
                kt[j][i] = (__bf16)(-kv[j] * E);
            }
            *reinterpret_cast<bf16x4 *>(KR + (RPB * rb + i) * L::KRP + 4 * cq) = kr;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            __bf16 *dq = QT + (4 * cq + j) * CTP + RPB * rb, *dk = KT + (4 * cq + j) * CTP + RPB * rb;
            if constexpr (RPB == 4) {
                *reinterpret_cast<bf16x4 *>(dq) = qt[j];
                *reinterpret_cast<bf16x4 *>(dk) = kt[j];
            } else {
                *reinterpret_cast<bf16x2 *>(dq) = bf16x2{qt[j][0], qt[j][1]};
                *reinterpret_cast<bf16x2 *>(dk) = bf16x2{kt[j][0], kt[j][1]};
            }
        }
        if (rb == NRB - 1) {
            float4 gm;
            gm.x = __builtin_amdgcn_exp2f(tot[0]);
            gm.y = __builtin_amdgcn_exp2f(tot[1]);
            gm.z = __builtin_amdgcn_exp2f(tot[2]);
            gm.w = __builtin_amdgcn_exp2f(tot[3]);
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(slot + L::GAM) + 4 * cq) = gm;
        }
        const int tr = ptid >> 3, tc = 4 * (ptid & 7);
        *reinterpret_cast<uint2 *>(reinterpret_cast<__bf16 *>(slot + L::TT) + tr * CTP + tc) = tt;
        *reinterpret_cast<uint2 *>(reinterpret_cast<__bf16 *>(slot + L::PT) + tr * CTP + tc) = pt;
        // dO^T: this thread's row ro, columns 8 (pt & 7) ..
        __bf16 *OT = reinterpret_cast<__bf16 *>(slot + L::OT);
        const int ro = ptid >> 3, oc = 8 * (ptid & 7);
        const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            OT[(oc + e) * CTP + ro] = __builtin_bit_cast(__bf16, (unsigned short)(ow[e >> 1] >> (16 * (e & 1))));
        if (ptid < C) reinterpret_cast<float *>(slot + L::BETA)[ptid] = __uint_as_float(b << 16);
    }
};

template <int DK>
__global__ void __launch_bounds__(NT2) bwd_dstates_bf16_kernel(Params p) {
    using L = ChainSlot<DK>;
    constexpr int NRUN = DK / 32;
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * L::BYTES];
    int unit, slice;
    chain_unit(p, blockIdx.x, unit, slice);
    const int s = unit / p.H, h = unit % p.H, col0 = slice * W2;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave >= 4;
    const int ln = lane & 15, lj = lane >> 4;
    const int cc = 16 * (wave & 3) + ln;                 // consumer: column within the slice
    long t0s, base;
    int len;
    seq_info(p, s, t0s, len, base);
    const int nch = (len + C - 1) / C;
    const size_t so = ((size_t)s * p.H + h) * DK;
    auto chunk_len = [&](int n) { return len - n * C < C ? len - n * C : C; };
    auto wslot = [&](int n) { return (size_t)(base + n) * p.H + h; };

    // The two wave groups run separate loops with the same number of barriers
    // (one before the first chunk and one per chunk), so that neither keeps
    // the other's loop-invariant values in registers.
    if (producer) {
        // two register sets, so that a chunk's loads are issued two chunks
        // before it is staged (one chunk of work does not cover the memory
        // latency): ia holds chunks nch-1, nch-3, ..., ib the others
        // Loads and stages are unconditional: a chunk index below 0 reads
        // chunk 0 again (or nothing, for an empty sequence) and is staged
        // into the slot no consumer reads, so that every path through the
        // loop leaves the same loads in flight and the waits before a stage
        // cover only the older of the two sets.
        ChainIn<DK> ia, ib;
        const int ptid = tid - 256;
        auto load = [&](ChainIn<DK> &in, int n) {
            n = n > 0 ? n : 0;
            in.load(p, t0s + (long)n * C, chunk_len(n), h, wslot(n), col0, ptid);
        };
        load(ia, nch - 1);
        load(ib, nch - 2);
        ia.stage(p, smem + ((nch - 1) & 1) * L::BYTES, ptid);
        load(ia, nch - 3);
        __syncthreads();
        // while the consumers work on chunk n: stage chunk n - 1, load n - 3
        for (int n = nch - 1; n >= 0; n -= 2) {
            ib.stage(p, smem + ((n - 1) & 1) * L::BYTES, ptid);
            load(ib, n - 3);
            __syncthreads();
            if (n == 0) break;
            ia.stage(p, smem + ((n - 2) & 1) * L::BYTES, ptid);
            load(ia, n - 4);
            __syncthreads();
        }
        return;
    }
    f32x4 D[NRUN][2];
#pragma unroll
    for (int rho = 0; rho < NRUN; ++rho)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                D[rho][hh][i] = p.dST ? p.dST[(so + crow(rho, hh, 4 * lj + i)) * p.DV + col0 + cc] : 0.0f;
            // landed before the loop (otherwise the wait for it would sit
            // inside the loop, draining the memory queue every chunk)
            D[rho][hh] = pinned(D[rho][hh]);
        }
    __syncthreads();
    for (int n = nch - 1; n >= 0; --n) {
        {
            const unsigned char *slot = smem + (n & 1) * L::BYTES;
            const __bf16 *KR = reinterpret_cast<const __bf16 *>(slot + L::KR);
            const __bf16 *QT = reinterpret_cast<const __bf16 *>(slot + L::QT);
            const __bf16 *KT = reinterpret_cast<const __bf16 *>(slot + L::KT);
            const __bf16 *TT = reinterpret_cast<const __bf16 *>(slot + L::TT);
            const __bf16 *PT = reinterpret_cast<const __bf16 *>(slot + L::PT);
            const __bf16 *OT = reinterpret_cast<const __bf16 *>(slot + L::OT);
            const float *gam = reinterpret_cast<const float *>(slot + L::GAM);
            const float *bet = reinterpret_cast<const float *>(slot + L::BETA);
            const size_t wi = wslot(n);
            const int cl = chunk_len(n);
            auto a8 = [&](const __bf16 *m, int pitch, int row, int k0) {
                return *reinterpret_cast<const bf16x8 *>(m + row * pitch + k0 + 8 * lj);
            };
            // D, the gradient of the state leaving chunk n: bf16 B fragments,
            // and to the workspace
            bf16x8 dfr[NRUN];
            {
                const __amdgpu_buffer_rsrc_t r = brsrc(reinterpret_cast<bf16_t *>(p.wD) + wi * DK * p.DV +
                                                       strip_off(0, col0 + 16 * (wave & 3), DK));
#pragma unroll
                for (int rho = 0; rho < NRUN; ++rho) {
                    dfr[rho] = frag2(D[rho][0], D[rho][1]);
                    const uint4 w = __builtin_bit_cast(uint4, dfr[rho]);
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
                        __builtin_amdgcn_raw_buffer_store_b64(
                            quad_rows(hh ? w.z : w.x, hh ? w.w : w.y, ln), r,
                            (uint32_t)((crow(rho, hh, 4 * lj + quad_row(ln)) * 16 + (ln & ~3)) * 2), 0, kStreamStore);
                }
            }
            const bf16x8 ofr = *reinterpret_cast<const bf16x8 *>(OT + cc * CTP + 8 * lj);
            // dU = P^T dO + K_right D (chunk rows in crow order)
            f32x4 u[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int rm = crow(0, hh, ln);
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
                a = mfma8(a8(PT, CTP, rm, 0), ofr, a);
#pragma unroll
                for (int rho = 0; rho < NRUN; ++rho) a = mfma8(a8(KR, L::KRP, rm, 32 * rho), dfr[rho], a);
                u[hh] = a;
            }
            const bf16x8 ufr = frag2(u[0], u[1]);
            // dX = Diag(beta) T^T dU; dX is dv
            f32x4 x[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int rm = crow(0, hh, ln);
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
                a = mfma8(a8(TT, CTP, rm, 0), ufr, a);
                const float4 b4 = *reinterpret_cast<const float4 *>(bet + 8 * lj + 4 * hh);
                x[hh][0] = b4.x * a[0];
                x[hh][1] = b4.y * a[1];
                x[hh][2] = b4.z * a[2];
                x[hh][3] = b4.w * a[3];
            }
            const bf16x8 xfr = frag2(x[0], x[1]);
            {
                const long t0 = t0s + (long)n * C;
                const int cw0 = col0 + 16 * (wave & 3);
                const __amdgpu_buffer_rsrc_t ru = brsrc(p.wdU + wi * C * p.DV + strip_off(0, cw0, C));
                const __amdgpu_buffer_rsrc_t rv =
                    brsrc(static_cast<bf16_t *>(p.dv) + ((size_t)t0 * p.H + h) * p.DV + cw0);
                const uint4 wu = __builtin_bit_cast(uint4, ufr), wx = __builtin_bit_cast(uint4, xfr);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int row = 8 * lj + 4 * hh + quad_row(ln);
                    __builtin_amdgcn_raw_buffer_store_b64(quad_rows(hh ? wu.z : wu.x, hh ? wu.w : wu.y, ln), ru,
                                                          (uint32_t)((row * 16 + (ln & ~3)) * 2), 0, kStreamStore);
                    __builtin_amdgcn_raw_buffer_store_b64(
                        quad_rows(hh ? wx.z : wx.x, hh ? wx.w : wx.y, ln), rv,
                        row < cl ? (uint32_t)((row * p.H * p.DV + (ln & ~3)) * 2) : kDrop, 0, 0);
                }
            }
            // D = Diag(gamma) D + Q_up^T dO - K_up^T dX
#pragma unroll
            for (int rho = 0; rho < NRUN; ++rho)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int rd = crow(rho, hh, ln);
                    const float4 g4 = *reinterpret_cast<const float4 *>(gam + 32 * rho + 8 * lj + 4 * hh);
                    f32x4 d = D[rho][hh];
                    d[0] *= g4.x;
                    d[1] *= g4.y;
                    d[2] *= g4.z;
                    d[3] *= g4.w;
                    d = mfma8(a8(QT, CTP, rd, 0), ofr, d);
                    d = mfma8(a8(KT, CTP, rd, 0), xfr, d);
                    D[rho][hh] = d;
                }
        }
        __syncthreads();
    }
    if (p.dS0) {
#pragma unroll
        for (int rho = 0; rho < NRUN; ++rho)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p.dS0[(so + crow(rho, hh, 4 * lj + i)) * p.DV + col0 + cc] = D[rho][hh][i];
    }
}

// ---------------------------------------------------------------------------
// bf16 inputs, factorised path: the same chunk gradients with the d_v
// products on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  Each
// operand is staged in LDS as bf16 with its contraction index contiguous (a
// matrix used both ways is kept in both orientations); the C x C algebra and
// the decay-weighted sums stay fp32.
// With X, U (state chain) and dU (gradient chain) in the workspace, and dX
// written as dv by the gradient chain, every product left contracts over d_v,
// which is contiguous in every operand: the slices go to LDS row-major as they
// come, with no transposed copies.
constexpr int W3 = 64;                 // d_v columns per slice of the gradient kernel
// LDS of the bf16 gradient kernel, at most 80 KB so that two 512-thread
// workgroups share a CU (one loads while the other runs its C x C algebra).
// The fp32 [C][d_k] arrays have a pitch of d_k + 4: rows stay 16-byte
// aligned (row segments move as 16-byte accesses), and in the MFMA output
// layout (rows 4j + i, columns r: r = lane & 15, j = lane >> 4) the 64 lanes
// of an access fall in distinct banks.
template <int DK> struct GbLayout {
    static constexpr int DKP = DK + 4, WB = W3 + 8;
    static constexpr int G = 0;                                   // fp32 [C][DKP]
    static constexpr int GC = G + 4 * C * DKP;                    // fp32 [DK] x 3
    static constexpr int GAM = GC + 4 * DK;
    static constexpr int DGP = GAM + 4 * DK;
    static constexpr int RKP = DGP + 4 * DK;                      // fp32 [2][DK]
    static constexpr int SB = RKP + 8 * DK;                       // fp32 [C] x 2
    static constexpr int DB = SB + 4 * C;
    static constexpr int DBP = DB + 4 * C;                        // fp32 [2][C]
    static constexpr int AREA = DBP + 8 * C;
    // slice phase (in the area): bf16, row-major
    static constexpr int SR = AREA;                               // [DK][WB]
    static constexpr int DR = SR + 2 * DK * WB;
    static constexpr int XR = DR + 2 * DK * WB;                   // [C][WB]
    static constexpr int UR = XR + 2 * C * WB;
    static constexpr int DUR = UR + 2 * C * WB;
    static constexpr int DXR = DUR + 2 * C * WB;
    static constexpr int DOR = DXR + 2 * C * WB;
    static constexpr int SLICE_END = DOR + 2 * C * WB;
    // after the slices (in the area): M (then beta dA) and dP live to the
    // end; T, dT' and Y only through the C x C algebra, then K_up, Q_up, K_dn
    // take their place (dA itself never leaves the registers)
    static constexpr int MF = AREA;                               // fp32 [C][CP] x 5
    static constexpr int DPF = MF + 4 * C * CP;
    static constexpr int TF = DPF + 4 * C * CP;
    static constexpr int DTF = TF + 4 * C * CP;
    static constexpr int YF = DTF + 4 * C * CP;
    static constexpr int FK = TF;                                 // fp32 [C][DKP] x 3
    static constexpr int FQ = FK + 4 * C * DKP;
    static constexpr int FKD = FQ + 4 * C * DKP;
    static constexpr int TAIL_END = FKD + 4 * C * DKP;
    static constexpr int BYTES = SLICE_END > TAIL_END ? SLICE_END : TAIL_END;
    static_assert(YF + 4 * C * CP <= TAIL_END, "C x C buffers");
    static_assert(BYTES <= 80 * 1024, "two workgroups per CU");
};

template <int DK>
__global__ void __launch_bounds__(NT2, 4) bwd_grads_bf16_kernel(Params p) {
    using L = GbLayout<DK>;
    constexpr int DKP = L::DKP, WB = L::WB;
    constexpr int NTW = DK / 64, NE = DK / 16;      // 8 waves: 2 or 1 C x DK tiles each
    constexpr int NES = DK * W3 / NT2, TPR = W3 / NES;   // S / D slice values per thread
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];
    float *sG = reinterpret_cast<float *>(smem + L::G);
    float *sT = reinterpret_cast<float *>(smem + L::TF);
    float *sM = reinterpret_cast<float *>(smem + L::MF);
    float *gc = reinterpret_cast<float *>(smem + L::GC);
    float *gam = reinterpret_cast<float *>(smem + L::GAM);
    float *dgp = reinterpret_cast<float *>(smem + L::DGP);
    float *rkp = reinterpret_cast<float *>(smem + L::RKP);
    float *sB = reinterpret_cast<float *>(smem + L::SB);
    float *dB = reinterpret_cast<float *>(smem + L::DB);
    __bf16 *Sr = reinterpret_cast<__bf16 *>(smem + L::SR);
    __bf16 *Dr = reinterpret_cast<__bf16 *>(smem + L::DR);
    __bf16 *Xr = reinterpret_cast<__bf16 *>(smem + L::XR);
    __bf16 *Ur = reinterpret_cast<__bf16 *>(smem + L::UR);
    __bf16 *dUr = reinterpret_cast<__bf16 *>(smem + L::DUR);
    __bf16 *dXr = reinterpret_cast<__bf16 *>(smem + L::DXR);
    __bf16 *dOr = reinterpret_cast<__bf16 *>(smem + L::DOR);

    const long slot = blockIdx.x;
    const int h = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lj = lane >> 4;
    const int sr = tid / TPR, sc = (tid % TPR) * NES;     // S / D: row sr, columns sc ..
    const int vr = tid >> 4, vc = (tid & 15) * 4;         // C x W3: row vr, columns vc ..
    const bool vt = tid < 256;                            // C x C values: the first 256 threads
    long t0;
    int cl;
    if (!slot_chunk(p, slot, t0, cl)) return;
    const size_t wi = (size_t)slot * p.H + h;
    if (p.wF[wi] != 0) return;                       // exact chunks: the fp32 kernel
    // states and state gradients are kept as bf16 for bf16 inputs
    const bf16_t *gS = reinterpret_cast<const bf16_t *>(p.wS) + wi * DK * p.DV;
    const bf16_t *gD = reinterpret_cast<const bf16_t *>(p.wD) + wi * DK * p.DV;
    const size_t cx = wi * C * p.DV;

    // one d_v slice of S, D (d_k x W3) and X, U, dU, dX, dO (C x W3)
    struct SliceIn {
        Seg<bf16_t, NES> s, d;
        Seg<bf16_t, 4> x, u, du, dx, o;
    };
    auto issue_slice = [&](SliceIn &in, int col0) {
        in.s.load(gS, strip_off(sr, col0 + sc, DK), true);
        in.d.load(gD, strip_off(sr, col0 + sc, DK), true);
        const size_t w = cx + strip_off(vr, col0 + vc, C);
        in.x.load(p.wX, w, true);
        in.u.load(p.wU, w, true);
        in.du.load(p.wdU, w, true);
        const size_t e = ((size_t)(t0 + vr) * p.H + h) * p.DV + col0 + vc;
        in.dx.load(p.dv, e, vr < cl);
        in.o.load(p.dO, e, vr < cl);
    };
    // both slices (d_v = 2 W3) are in flight from the start; with d_v = W3
    // the second repeats the first and is not used
    SliceIn s0, s1;
    // k and q stay in registers (this thread's row tid / 16, NE columns) until
    // the decay-weighted sums after the C x C algebra
    // as are T and M (first 256 threads, 4 values each), whose LDS the slices use
    ChunkIn<bf16_t, DK, true, 16> in;
    Seg<float, 4> tin, min;
    const int t4 = (tid & 255) * 4;
    in.load(p, t0, cl, h);
    tin.load(p.wT, wi * C * C + t4, vt);
    min.load(p.wM, wi * C * C + t4, vt);
    issue_slice(s0, 0);
    issue_slice(s1, p.DV > W3 ? W3 : 0);
    in.template store_gb<DKP>(p, sG, sB);
    if (tid < C) dB[tid] = 0.0f;
    __syncthreads();
    gate_sums<DK, DKP>(sG, gc, gam);

    f32x4 aQ[NTW], aK[NTW], aR[NTW], aT = {0.f, 0.f, 0.f, 0.f}, aP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
        aQ[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        aK[x] = aQ[x];
        aR[x] = aQ[x];
    }
    float dgacc = 0.0f;                               // S * D over this thread's values
    // waves 0-3: the dT' tiles; waves 4-7: the dP tiles (tile (tm, tn) of C x C)
    const int tm = (wave & 3) >> 1, tn = wave & 1;
    const bool lo = wave < 4;
    auto put = [](__bf16 *dst, const auto &seg, auto count) {
        // raw bf16 bits of a segment, as vector stores
        constexpr int n = decltype(count)::value;
        if constexpr (n == 16) {
            reinterpret_cast<uint4 *>(dst)[0] = make_uint4(seg.w[0], seg.w[1], seg.w[2], seg.w[3]);
            reinterpret_cast<uint4 *>(dst)[1] = make_uint4(seg.w[4], seg.w[5], seg.w[6], seg.w[7]);
        } else if constexpr (n == 8) {
            reinterpret_cast<uint4 *>(dst)[0] = make_uint4(seg.w[0], seg.w[1], seg.w[2], seg.w[3]);
        } else {
            reinterpret_cast<uint2 *>(dst)[0] = make_uint2(seg.w[0], seg.w[1]);
        }
    };
    using n4 = std::integral_constant<int, 4>;
    using nes = std::integral_constant<int, NES>;
    auto slice = [&](const SliceIn &in) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NES; ++j) dgacc += in.s.get(j) * in.d.get(j);
        put(Sr + sr * WB + sc, in.s, nes{});
        put(Dr + sr * WB + sc, in.d, nes{});
        put(Xr + vr * WB + vc, in.x, n4{});
        put(Ur + vr * WB + vc, in.u, n4{});
        put(dUr + vr * WB + vc, in.du, n4{});
        if (in.o.ok) {                                // rows past the sequence end: zeros
            put(dXr + vr * WB + vc, in.dx, n4{});
            put(dOr + vr * WB + vc, in.o, n4{});
        } else {
            *reinterpret_cast<uint2 *>(dXr + vr * WB + vc) = make_uint2(0u, 0u);
            *reinterpret_cast<uint2 *>(dOr + vr * WB + vc) = make_uint2(0u, 0u);
        }
        __syncthreads();
        // dT' += dU X^T (waves 0-3);  dP += dO U^T (waves 4-7);
        // dQ_up += dO S^T;  -dK_up += dX S^T;  dK_right += U D^T
        if (lo) aT = mmb(aT, dUr + 16 * tm * WB, WB, Xr + 16 * tn * WB, WB, W3);
        else aP = mmb(aP, dOr + 16 * tm * WB, WB, Ur + 16 * tn * WB, WB, W3);
#pragma unroll
        for (int x = 0; x < NTW; ++x) {
            const int tt = wave * NTW + x, m0 = 16 * (tt / (DK / 16)), n0 = 16 * (tt % (DK / 16));
            aQ[x] = mmb(aQ[x], dOr + m0 * WB, WB, Sr + n0 * WB, WB, W3);
            aK[x] = mmb(aK[x], dXr + m0 * WB, WB, Sr + n0 * WB, WB, W3);
            aR[x] = mmb(aR[x], Ur + m0 * WB, WB, Dr + n0 * WB, WB, W3);
        }
    };
    slice(s0);
    if (p.DV > W3) slice(s1);
    // dgamma per channel: the S * D sums of the TPR threads of a row
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) dgacc += __shfl_xor(dgacc, off);
    if (tid % TPR == 0) dgp[sr] = dgacc;
    __syncthreads();

    // C x C algebra (fp32)
    float *sdT = reinterpret_cast<float *>(smem + L::DTF), *sdP = reinterpret_cast<float *>(smem + L::DPF);
    float *sY = reinterpret_cast<float *>(smem + L::YF);
    float *dBp = reinterpret_cast<float *>(smem + L::DBP);
    if (vt) {
        const int tr = t4 / C, tc = t4 % C;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sT[tr * CP + tc + j] = tin.get(j);
            sM[tr * CP + tc + j] = min.get(j);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * tm + 4 * lj + i, col = 16 * tn + lr;
        if (lo) sdT[row * CP + col] = aT[i];
        else sdP[row * CP + col] = col <= row ? aP[i] : 0.0f;
    }
    __syncthreads();
    if (lo) {
        // Y = T^T (dT' Diag(beta)) (waves 0-3, one 16 x 16 tile each), the
        // column scale folded into the operand reads: every element this lane
        // reads of dT' lies in its column 16 tn + lr
        const float fb = sB[16 * tn + lr];
        const float *pa = sT + 16 * tm + lr + lj * CP, *pb = sdT + lj * CP + 16 * tn + lr;
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += 4) a = mfma4(pa[k0 * CP], pb[k0 * CP] * fb, a);
#pragma unroll
        for (int i = 0; i < 4; ++i) sY[(16 * tm + 4 * lj + i) * CP + 16 * tn + lr] = a[i];
    } else if (tid < 256 + C) {
        // meanwhile, on waves with no share of the two products: dbeta's first
        // term, the column sums of T o dT'
        const int c = tid - 256;
        float acc = 0.0f;
#pragma unroll 8
        for (int r = 0; r < C; ++r) acc += sT[r * CP + c] * sdT[r * CP + c];
        dB[c] = acc;
    }
    __syncthreads();
    if (lo) {
        // dA = -strict_lower(Y T^T), used where it lands: M <- Diag(beta) dA in
        // place, and dbeta's second term, the row sums of dA o M (M before the
        // update), per tile over its 16 columns (the lanes of a 16-lane group);
        // the two column tiles' sums are added in a fixed order at the output
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        a = mm(a, sY + 16 * tm * CP, CP, 1, sT + 16 * tn * CP, 1, CP, C);
        float part[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * tm + 4 * lj + i, col = 16 * tn + lr;
            const float da = col < row ? -a[i] : 0.0f;
            part[i] = da * sM[row * CP + col];
            sM[row * CP + col] = sB[row] * da;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) part[i] += __shfl_xor(part[i], off);
        if (lr == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) dBp[tn * C + 16 * tm + 4 * lj + i] = part[i];
        }
    }
    // (K_up, Q_up and K_dn take the place of T, dT' and Y, read just above)
    __syncthreads();
    // fp32 K_up, Q_up, K_dn for the decay-weighted sums
    float *fK = reinterpret_cast<float *>(smem + L::FK), *fQ = reinterpret_cast<float *>(smem + L::FQ);
    float *fKd = reinterpret_cast<float *>(smem + L::FKD);
    {
        const int r = tid >> 4, c0 = (tid & 15) * NE, o = r * DKP + c0;
        float G[NE], v[NE];
        row4_get<NE>(sG + o, G);
        // one array at a time, so that few values are live at once
#pragma unroll
        for (int j = 0; j < NE; ++j) v[j] = in.k.get(j) * __builtin_amdgcn_exp2f(-G[j]);
        row4_put<NE>(fKd + o, v);
#pragma unroll
        for (int j = 0; j < NE; ++j) G[j] = __builtin_amdgcn_exp2f(G[j]);
#pragma unroll
        for (int j = 0; j < NE; ++j) v[j] = in.k.get(j) * G[j];
        row4_put<NE>(fK + o, v);
#pragma unroll
        for (int j = 0; j < NE; ++j) v[j] = in.q.get(j) * G[j];
        row4_put<NE>(fQ + o, v);
    }
    __syncthreads();
    // factorised decay sums and the direct terms, combined per element:
    //   Z1 = dP K_dn,  Z2 = dM K_dn,  Z3 = dM^T K_up + dP^T Q_up,
    //   dq = (dQ_up + Z1) e^G,  dk = (dK_up + Z2) e^G + dK_right e^{G_c - G} + Z3 e^{-G},
    //   dGamma = (dK_up + Z2) K_up + (dQ_up + Z1) Q_up - dK_right K_right - Z3 K_dn
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
        const int tt = wave * NTW + x, m0 = 16 * (tt / (DK / 16)), n0 = 16 * (tt % (DK / 16));
        f32x4 z1 = {0.f, 0.f, 0.f, 0.f}, z2 = z1, z3 = z1;
        z1 = mm(z1, sdP + m0 * CP, CP, 1, fKd + n0, DKP, 1, C);
        z2 = mm(z2, sM + m0 * CP, CP, 1, fKd + n0, DKP, 1, C);
        z3 = mm(z3, sM + m0, 1, CP, fK + n0, DKP, 1, C);
        z3 = mm(z3, sdP + m0, 1, CP, fQ + n0, DKP, 1, C);
        float rk = 0.0f;                              // this lane's 4 rows of dK_right K_right
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + 4 * lj + i, col = n0 + lr, o = row * DKP + col;
            const float G = sG[o], E = __builtin_amdgcn_exp2f(G);
            const float R = __builtin_amdgcn_exp2f(gc[col] - G);
            const float Ei = __builtin_amdgcn_exp2f(-G);
            const float dQu = aQ[x][i] + z1[i], dKu = z2[i] - aK[x][i], dKr = aR[x][i];
            const float ku = fK[o], qu = fQ[o], kd = fKd[o];
            const float kr = kd * E * R;
            aQ[x][i] = dQu * E;
            aK[x][i] = dKu * E + dKr * R + z3[i] * Ei;
            aR[x][i] = dKu * ku + dQu * qu - dKr * kr - z3[i] * kd;
            rk += dKr * kr;
        }
        rk += __shfl_xor(rk, 16);
        rk += __shfl_xor(rk, 32);
        if (lj == 0) rkp[(m0 >> 4) * DK + n0 + lr] = rk;
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
        const int tt = wave * NTW + x, m0 = 16 * (tt / (DK / 16)), n0 = 16 * (tt % (DK / 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int o = (m0 + 4 * lj + i) * DKP + n0 + lr;
            fQ[o] = aQ[x][i];
            fK[o] = aK[x][i];
            fKd[o] = aR[x][i];
        }
    }
    __syncthreads();
    // dlog_alpha: reverse running sum of dGamma plus the chunk-total term
    if (tid < DK) {
        const int c = tid;
        float x[C];
        const float tot = rkp[c] + rkp[DK + c] + dgp[c] * gam[c];
#pragma unroll
        for (int r = 0; r < C; ++r) x[r] = fKd[r * DKP + c];
        float run = tot;
#pragma unroll
        for (int r = C - 1; r >= 0; --r) {
            run += x[r];
            fKd[r * DKP + c] = run;
        }
    }
    __syncthreads();
    {
        // each thread's NE consecutive gradients as one vector store
        using vec = typename std::conditional<NE == 8, bf16x8, bf16x4>::type;
        const int r = tid >> 4, c0 = (tid & 15) * NE;
        if (r < cl) {
            const size_t e = ((size_t)(t0 + r) * p.H + h) * DK + c0;
            float v[NE];
            vec a, b, g;
            row4_get<NE>(fQ + r * DKP + c0, v);
#pragma unroll
            for (int j = 0; j < NE; ++j) a[j] = (__bf16)v[j];
            row4_get<NE>(fK + r * DKP + c0, v);
#pragma unroll
            for (int j = 0; j < NE; ++j) b[j] = (__bf16)v[j];
            row4_get<NE>(fKd + r * DKP + c0, v);
#pragma unroll
            for (int j = 0; j < NE; ++j) g[j] = (__bf16)v[j];
            *reinterpret_cast<vec *>(static_cast<bf16_t *>(p.dq) + e) = a;
            *reinterpret_cast<vec *>(static_cast<bf16_t *>(p.dk) + e) = b;
            if (p.gate == GATE_CHANNEL) *reinterpret_cast<vec *>(static_cast<bf16_t *>(p.dg) + e) = g;
        }
    }
    if (tid < cl) {
        const size_t e = (size_t)(t0 + tid) * p.H + h;
        st<bf16_t>(p.dbeta, e, dB[tid] + dBp[tid] + dBp[C + tid]);
        if (p.gate == GATE_HEAD) {
            // each lane starts at its own channel, so that the rows' reads
            // spread over the banks
            float acc = 0.0f;
            for (int i = 0; i < DK; ++i) acc += fKd[tid * DKP + ((i + tid) & (DK - 1))];
            st<bf16_t>(p.dg, e, acc);
        }
    }
}

template <typename Tin, int DK>
hipError_t launch(const Params &p, long nslot, int nseq, hipStream_t stream) {
    const dim3 gchunks((unsigned)nslot, (unsigned)p.H);
    const unsigned gunits = (unsigned)((long)nseq * p.H * (p.DV / W));
    if constexpr (std::is_same<Tin, bf16_t>::value) {
        // the forward's fused chunk kernel, keeping what the gradients need
        // (states, X, U, T, M0, T^T, P^T, flags), then the gradient chain
        const int units = nseq * p.H;
        if (units > 0) {
            const hipError_t e = chunked_ws_save_launch(
                p.q, p.k, p.v, p.g, p.beta, p.gate, p.S0, p.cu, nseq, p.T, p.H, DK, p.DV,
                chunked_slice_width(units, p.DV), reinterpret_cast<bf16_t *>(p.wS), p.wX, p.wU, p.wTt,
                p.wPt, p.wT, p.wM, p.wP, p.wF, stream);
            if (e != hipSuccess) return e;
        }
        const unsigned gu2 = (unsigned)((long)nseq * p.H * (p.DV / W2));
        hipLaunchKernelGGL((bwd_dstates_bf16_kernel<DK>), dim3(gu2), dim3(NT2), 0, stream, p);
    } else {
        if (nslot > 0) hipLaunchKernelGGL((bwd_prep_kernel<Tin, DK>), gchunks, dim3(NT), 0, stream, p);
        hipLaunchKernelGGL((bwd_states_kernel<Tin, DK>), dim3(gunits), dim3(NT), 0, stream, p);
        hipLaunchKernelGGL((bwd_dstates_kernel<Tin, DK>), dim3(gunits), dim3(NT), 0, stream, p);
    }
    if (nslot > 0) {
        if constexpr (std::is_same<Tin, bf16_t>::value)
            hipLaunchKernelGGL((bwd_grads_bf16_kernel<DK>), gchunks, dim3(NT2), 0, stream, p);
        else
            hipLaunchKernelGGL((bwd_grads_kernel<Tin, DK, false>), gchunks, dim3(NT), 0, stream, p, nslot);
        // exact chunks are rare: about 2048 workgroups stride over the slots
        const long gx = std::max(1L, std::min(nslot, 2048L / p.H));
        hipLaunchKernelGGL((bwd_grads_kernel<Tin, DK, true>), dim3((unsigned)gx, (unsigned)p.H), dim3(NT), 0,
                           stream, p, nslot);
    }
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
    const size_t f = (per * sizeof(int32_t) + 255) & ~(size_t)255;
    const size_t x = (per * bwd::C * dv * sizeof(bf16_t) + 255) & ~(size_t)255;
    const size_t y = (per * bwd::C * bwd::C * sizeof(bf16_t) + 255) & ~(size_t)255;
    return 2 * a + 3 * b + f + 3 * x + 2 * y;
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
    p.wF = reinterpret_cast<int32_t *>(w + 2 * a + 3 * b);
    {
        const size_t f = (per * sizeof(int32_t) + 255) & ~(size_t)255;
        const size_t x = (per * bwd::C * dv * sizeof(bf16_t) + 255) & ~(size_t)255;
        char *wx = w + 2 * a + 3 * b + f;
        p.wX = reinterpret_cast<bf16_t *>(wx);
        p.wU = reinterpret_cast<bf16_t *>(wx + x);
        p.wdU = reinterpret_cast<bf16_t *>(wx + 2 * x);
        const size_t y = (per * bwd::C * bwd::C * sizeof(bf16_t) + 255) & ~(size_t)255;
        char *wy = wx + 3 * x;
        p.wTt = reinterpret_cast<bf16_t *>(wy);
        p.wPt = reinterpret_cast<bf16_t *>(wy + y);
    }
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
