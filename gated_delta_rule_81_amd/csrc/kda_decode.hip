// kda_decode.hip -- one-token KDA update over a state cache (gfx950).
//
// The recurrent form of the operator (daily.dev summary of "You Could Have
// Come Up with Kimi Delta Attention": the token-by-token implementation;
// "The fourth layer remembers": constant work per decoded token).  For each
// (sequence n, head h), with S the d_k x d_v fp32 state:
//
//   S' = Diag(alpha) S                 alpha = exp(log_alpha), per key channel
//   e  = S'^T k,   p = S'^T q          (reads of the decayed state)
//   u  = beta (v - e)                  (delta-rule error)
//   S  <- S' + k u^T                   (written back in place)
//   o  = S^T q = p + (k . q) u
//
// The step is bound by HBM: each 64 KB state (d = 128) is read once and
// written once, everything else is ~1.3 KB per (n, h).  A 1024-thread
// workgroup walks (n, h) units with a stride of the grid (a few workgroups
// per CU); thread t holds a 4-column group (16-byte accesses; a wave covers
// two whole 512-byte rows) of d_k / 32 rows, so a unit's state sits in
// registers between its read and its write, and the next unit's state is
// already being read while the current one is reduced and written.  Column
// sums over rows go through LDS.  State traffic uses non-temporal loads and
// stores: every byte is touched once per step, so caching it only costs.
//
// Optional input preparation: k and q divided by their L2 norms (formed with
// k . q by the first wave; e and p use the raw vectors and are rescaled),
// and the gate given as the softplus input x with alpha = 1 / (1 + e^x).
// With L > 1 each sequence takes L consecutive tokens in one call (inputs
// (N, L, H, .)): the state stays in registers across them and is read and
// written once.  The gate is one value per key channel (alpha above), one
// per token and head shared by the channels, or absent (alpha = 1).  With a slot map the state of
// sequence n is row state_idx[n] of a pool; a slot outside the pool starts
// from zeros and is not written.
#include "kda_device.h"

namespace kda {

constexpr int DEC_THREADS = 1024;
// cache-policy operand of the buffer loads: non-temporal (each state byte is
// touched once per step)
constexpr int kNonTemporal = 2;

template <int DK, int DV, typename T, bool MULTI>
__global__ __launch_bounds__(DEC_THREADS) void decode_step_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ log_alpha, const T *__restrict__ beta,
    float *__restrict__ S_cache, T *__restrict__ o, int units, int H, int L_, int gate, int prep,
    const int32_t *__restrict__ state_idx, int pool)
{
    // tokens per sequence: a compile-time 1 for the one-token instantiation
    const int L = MULTI ? L_ : 1;
    constexpr int NT = DEC_THREADS;
    constexpr int CG = DV / 4;     // 16-byte column groups per row
    constexpr int RG = NT / CG;    // row groups
    constexpr int RPT = DK / RG;   // rows per thread
    static_assert(NT % CG == 0 && DK % RG == 0 && RPT >= 1, "decode tiling");
    typedef float f4v __attribute__((ext_vector_type(4)));

    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;

    __shared__ float s_a[DK], s_k[DK], s_q[DK];
    __shared__ __attribute__((aligned(16))) float s_red[2][RG][DV];
    __shared__ __attribute__((aligned(16))) float s_u[DV];
    __shared__ float s_kq, s_ik, s_iq;   // k . q, 1/|k|, 1/|q| (1 without normalisation)

    // state row of a unit (n, h): n's slot, or -1 for no state.  The unit is
    // the same in every lane; saying so keeps the slot-map read a scalar load
    // (a vector load would be counted with the state prefetch, and waiting
    // for it would wait for the prefetch too).
    auto unit_row = [&](int unit) -> long {
        const int n = __builtin_amdgcn_readfirstlane(unit / H);
        const long r = state_row(state_idx, pool, n);
        return r < 0 ? -1L : r * H + (unit - n * H);
    };
    // A unit's state is read through a buffer resource over its 64 KB block;
    // a unit without a state gets a resource of zero bytes, whose loads read
    // zeros.  The loads are then unconditional, so the next unit's prefetch
    // stays in flight (a branch around them would make the compiler wait
    // for them where the two paths join).
    auto load_state = [&](int unit, f4v (&r)[RPT]) {
        const long row = unit_row(unit);
        const float *base = row < 0 ? S_cache : S_cache + (size_t)row * DK * DV;
        const uint64_t a = reinterpret_cast<uint64_t>(base);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), 0, row < 0 ? 0 : DK * DV * 4, 0x00020000);
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            r[i] = __builtin_bit_cast(f4v, __builtin_amdgcn_raw_buffer_load_b128(
                rs, (uint32_t)(((rg + i * RG) * CG + cg) * 16), 0, kNonTemporal));
    };

    // gate, k and q (threads t < DK), v (t < DV) and beta of a unit,
    // requested together with the unit's state one unit ahead and kept as
    // raw bits until used: the wait counter is in order, so a load issued
    // after the prefetch and used in the same step would wait for the
    // prefetch too, and a conversion right after a load would wait for it.
    // One unconditional load each: without a gate the k address stands in,
    // its value unused.
    auto raw = [](const T *ptr) -> uint32_t {
        if constexpr (sizeof(T) == 2) return (uint32_t)reinterpret_cast<const bf16_t *>(ptr)->x;
        else return __float_as_uint(*reinterpret_cast<const float *>(ptr));
    };
    auto val = [](uint32_t r) -> float { return __uint_as_float(sizeof(T) == 2 ? r << 16 : r); };
    // (every thread loads, threads past DK a duplicate of element 0, so that
    // no branch surrounds the loads)
    // token tk (0 .. L-1) of unit u = (n, h) is row (n L + tk) H + h of the
    // (N, L, H, .) inputs
    auto tok_row = [&](int u, int tk) -> size_t {
        const int n = u / H;
        return ((size_t)n * L + tk) * H + (u - n * H);
    };
    struct Small { uint32_t g, k, q, v, b; };
    auto load_small = [&](int u, int tk, Small &r) {
        const size_t row = tok_row(u, tk);
        const size_t idx = row * DK + (t < DK ? t : 0);
        const T *gp = gate == GATE_CHANNEL ? log_alpha + idx
                    : gate == GATE_HEAD    ? log_alpha + row
                                           : k + idx;
        r.g = raw(gp);
        r.k = raw(k + idx);
        r.q = raw(q + idx);
        r.v = raw(v + row * DV + (t < DV ? t : 0));
        r.b = raw(beta + row);
    };

    // Token tk of a unit: its small vectors `cs` were requested one token
    // earlier; the next token's go into `ns`, or after the unit's last token
    // the next unit's state and first token into `nxt` / `sn`.  The state
    // stays in registers across the unit's L tokens and is written back once.
    auto token = [&](int unit, long urow, int tk, f4v (&cur)[RPT], const Small &cs, Small &ns,
                     f4v (&nxt)[RPT], Small &sn) {
        // every wave waits here for this token's loads (an empty asm that
        // reads them), so the compiler knows them, and the state loaded
        // before them, to be complete below; otherwise it sinks the wait into
        // the branches that use them and later waits for the prefetch too
        asm volatile("" ::"v"(cs.g), "v"(cs.k), "v"(cs.q), "v"(cs.v), "v"(cs.b));
        const float a_ = gate == GATE_NONE        ? 1.0f
                       : (prep & PREP_SOFTPLUS) ? 1.0f / (1.0f + expf(val(cs.g)))
                                                : expf(val(cs.g));
        const float k_ = val(cs.k), q_ = val(cs.q), v_ = val(cs.v), b_ = val(cs.b);
        if (t < DK) {
            s_a[t] = a_;
            s_k[t] = k_;
            s_q[t] = q_;
        }
        const bool last = tk + 1 == L;
        const int next = unit + gridDim.x;
        if (!last) {
            load_small(unit, tk + 1, ns);
        } else if (next < units) {
            load_state(next, nxt);
            load_small(next, 0, sn);
        }
        __syncthreads();

        if (t < 64) {   // k . q (and |k|^2, |q|^2 when normalising) by the first wave
            float acc = 0.f, kk2 = 0.f, qq2 = 0.f;
            for (int r = t; r < DK; r += 64) {
                acc += s_k[r] * s_q[r];
                kk2 += s_k[r] * s_k[r];
                qq2 += s_q[r] * s_q[r];
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                acc += __shfl_xor(acc, off);
                kk2 += __shfl_xor(kk2, off);
                qq2 += __shfl_xor(qq2, off);
            }
            if (t == 0) {
                const float ik = (prep & PREP_L2NORM) ? inv_norm(kk2) : 1.0f;
                const float iq = (prep & PREP_L2NORM) ? inv_norm(qq2) : 1.0f;
                s_kq = acc * ik * iq;
                s_ik = ik;
                s_iq = iq;
            }
        }

        f4v e = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg + i * RG;
            cur[i] *= s_a[row];
            e += cur[i] * s_k[row];
            pq += cur[i] * s_q[row];
        }
        *reinterpret_cast<f4v *>(&s_red[0][rg][4 * cg]) = e;
        *reinterpret_cast<f4v *>(&s_red[1][rg][4 * cg]) = pq;
        __syncthreads();

        if (t < DV) {
            float es = 0.f, ps = 0.f;
#pragma unroll 8
            for (int r = 0; r < RG; ++r) {
                es += s_red[0][r][t];
                ps += s_red[1][r][t];
            }
            // with normalisation e and p were formed with the raw k and q
            const float u = b_ * (v_ - es * s_ik);
            s_u[t] = u;
            store_elem(o + tok_row(unit, tk) * DV + t, ps * s_iq + s_kq * u);
        }
        __syncthreads();

        const f4v u4 = *reinterpret_cast<const f4v *>(&s_u[4 * cg]) * s_ik;
#pragma unroll
        for (int i = 0; i < RPT; ++i) cur[i] += s_k[rg + i * RG] * u4;
        if (last) {
            if (urow >= 0) {
                f4v *Sw = reinterpret_cast<f4v *>(S_cache + (size_t)urow * DK * DV);
#pragma unroll
                for (int i = 0; i < RPT; ++i)
                    __builtin_nontemporal_store(cur[i], Sw + (rg + i * RG) * CG + cg);
            }
        }
        __syncthreads();   // the LDS vectors are rewritten for the next token
    };
    // One unit: its state and first token were requested one unit earlier.
    // Tokens alternate between `sc` and a second buffer (unrolled by two), so
    // no prefetched value is ever copied (a copy waits for its load).
    auto step = [&](int unit, f4v (&cur)[RPT], Small &sc, f4v (&nxt)[RPT], Small &sn) {
        const long urow = unit_row(unit);
        if constexpr (!MULTI) {
            token(unit, urow, 0, cur, sc, sc, nxt, sn);
        } else {
            Small tb = {0u, 0u, 0u, 0u, 0u};
            for (int tk = 0; tk < L; tk += 2) {
                token(unit, urow, tk, cur, sc, tb, nxt, sn);
                if (tk + 1 < L) token(unit, urow, tk + 1, cur, tb, sc, nxt, sn);
            }
        }
    };

    // Two register sets take turns (unrolled by two), so a prefetched state
    // is never copied, which would wait for its loads right away.
    f4v sa[RPT], sb[RPT];
    Small ma = {0u, 0u, 0u, 0u, 0u}, mb = {0u, 0u, 0u, 0u, 0u};
    int unit = blockIdx.x;
    if (unit < units) {
        load_state(unit, sa);
        load_small(unit, 0, ma);
    }
    // the first unit's loads have landed before the loop, as the next unit's
    // have (except for the stores issued after them) at the end of every step
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    for (; unit < units; unit += 2 * gridDim.x) {
        step(unit, sa, ma, sb, mb);
        if (unit + (int)gridDim.x >= units) break;
        step(unit + gridDim.x, sb, mb, sa, ma);
    }
}

int cu_count();

template <int DK, int DV, typename T>
static hipError_t launch_decode(const void *q, const void *k, const void *v,
                                const void *log_alpha, const void *beta, float *S,
                                void *o, int units, int H, int L, int gate, int prep,
                                const int32_t *state_idx, int pool, hipStream_t stream)
{
    // four workgroups per CU, each walking units with the grid stride
    const int grid = units < 4 * cu_count() ? units : 4 * cu_count();
    if (L == 1)
        hipLaunchKernelGGL((decode_step_kernel<DK, DV, T, false>), dim3(grid), dim3(DEC_THREADS), 0,
                           stream, (const T *)q, (const T *)k, (const T *)v, (const T *)log_alpha,
                           (const T *)beta, S, (T *)o, units, H, L, gate, prep, state_idx, pool);
    else
        hipLaunchKernelGGL((decode_step_kernel<DK, DV, T, true>), dim3(grid), dim3(DEC_THREADS), 0,
                           stream, (const T *)q, (const T *)k, (const T *)v, (const T *)log_alpha,
                           (const T *)beta, S, (T *)o, units, H, L, gate, prep, state_idx, pool);
    return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_decode_t(const void *q, const void *k, const void *v,
                                    const void *log_alpha, const void *beta, float *S,
                                    void *o, int units, int H, int L, int gate, int prep,
                                    const int32_t *state_idx, int pool, int dk, int dv,
                                    hipStream_t stream)
{
#define KDA_DEC(DK_, DV_) \
    launch_decode<DK_, DV_, T>(q, k, v, log_alpha, beta, S, o, units, H, L, gate, prep, state_idx, pool, \
                               stream)
    if (dk == 128 && dv == 128) return KDA_DEC(128, 128);
    if (dk == 128 && dv == 64) return KDA_DEC(128, 64);
    if (dk == 64 && dv == 128) return KDA_DEC(64, 128);
    return KDA_DEC(64, 64);
#undef KDA_DEC
}

// Host-side launcher used by the C ABI (sizes already validated).
hipError_t decode_step_launch(const void *q, const void *k, const void *v,
                              const void *log_alpha, const void *beta, int gate, int prep, float *S,
                              const int32_t *state_idx, int pool, void *o, int N, int L, int H,
                              int dk, int dv, bool bf16, hipStream_t stream)
{
    const int units = N * H;
    if (units == 0 || L == 0) return hipSuccess;
    if (bf16)
        return dispatch_decode_t<bf16_t>(q, k, v, log_alpha, beta, S, o, units, H, L, gate, prep,
                                         state_idx, pool, dk, dv, stream);
    return dispatch_decode_t<float>(q, k, v, log_alpha, beta, S, o, units, H, L, gate, prep,
                                    state_idx, pool, dk, dv, stream);
}

}  // namespace kda
