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
// written once, everything else is ~1.3 KB per (n, h).  One 256-thread
// workgroup owns one (n, h) state.  Thread t holds a 4-column group (16-byte
// loads/stores, a wave reads two full 512-byte rows per instruction) for
// d_k / 8 rows spread with stride 8, so the whole state sits in registers
// between the read and the write.  Column sums over rows are reduced through
// LDS; all loads of the state are issued before any arithmetic.
#include "kda_device.h"

namespace kda {

template <int DK, int DV, typename T>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ log_alpha, const T *__restrict__ beta,
    float *__restrict__ S_cache, T *__restrict__ o)
{
    constexpr int NT = 256;
    constexpr int CG = DV / 4;     // float4 column groups per row
    constexpr int RG = NT / CG;    // row groups
    constexpr int RPT = DK / RG;   // rows per thread
    static_assert(NT % CG == 0 && DK % RG == 0, "decode tiling");

    const int unit = blockIdx.x;   // flattened (n, h)
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;

    __shared__ float s_a[DK], s_k[DK], s_q[DK];
    __shared__ float s_red[2][RG][DV];
    __shared__ float s_u[DV];
    __shared__ float s_kq;

    float *Su = S_cache + (size_t)unit * DK * DV;
    float4 st[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + i * RG;
        st[i] = *reinterpret_cast<const float4 *>(Su + (size_t)row * DV + 4 * cg);
    }

    if (t < DK) {
        const size_t idx = (size_t)unit * DK + t;
        s_a[t] = expf(load_elem(log_alpha + idx));
        s_k[t] = load_elem(k + idx);
        s_q[t] = load_elem(q + idx);
    }
    __syncthreads();

    if (t < 64) {   // k . q by the first wave
        float acc = 0.f;
        for (int r = t; r < DK; r += 64) acc += s_k[r] * s_q[r];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (t == 0) s_kq = acc;
    }

    float e0 = 0.f, e1 = 0.f, e2 = 0.f, e3 = 0.f;
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + i * RG;
        const float a = s_a[row], kr = s_k[row], qr = s_q[row];
        float4 s = st[i];
        s.x *= a; s.y *= a; s.z *= a; s.w *= a;
        st[i] = s;
        e0 += s.x * kr; e1 += s.y * kr; e2 += s.z * kr; e3 += s.w * kr;
        p0 += s.x * qr; p1 += s.y * qr; p2 += s.z * qr; p3 += s.w * qr;
    }
    *reinterpret_cast<float4 *>(&s_red[0][rg][4 * cg]) = make_float4(e0, e1, e2, e3);
    *reinterpret_cast<float4 *>(&s_red[1][rg][4 * cg]) = make_float4(p0, p1, p2, p3);
    __syncthreads();

    if (t < DV) {
        float e = 0.f, p = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            e += s_red[0][r][t];
            p += s_red[1][r][t];
        }
        const size_t vidx = (size_t)unit * DV + t;
        const float u = load_elem(beta + unit) * (load_elem(v + vidx) - e);
        s_u[t] = u;
        store_elem(o + vidx, p + s_kq * u);
    }
    __syncthreads();

    const float4 u4 = *reinterpret_cast<const float4 *>(&s_u[4 * cg]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + i * RG;
        const float kr = s_k[row];
        float4 s = st[i];
        s.x += kr * u4.x; s.y += kr * u4.y; s.z += kr * u4.z; s.w += kr * u4.w;
        *reinterpret_cast<float4 *>(Su + (size_t)row * DV + 4 * cg) = s;
    }
}

template <int DK, int DV, typename T>
static hipError_t launch_decode(const void *q, const void *k, const void *v,
                                const void *log_alpha, const void *beta, float *S,
                                void *o, int units, hipStream_t stream)
{
    hipLaunchKernelGGL((decode_step_kernel<DK, DV, T>), dim3(units), dim3(256), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, (const T *)log_alpha,
                       (const T *)beta, S, (T *)o);
    return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_decode_t(const void *q, const void *k, const void *v,
                                    const void *log_alpha, const void *beta, float *S,
                                    void *o, int units, int dk, int dv, hipStream_t stream)
{
    if (dk == 128 && dv == 128) return launch_decode<128, 128, T>(q, k, v, log_alpha, beta, S, o, units, stream);
    if (dk == 128 && dv == 64) return launch_decode<128, 64, T>(q, k, v, log_alpha, beta, S, o, units, stream);
    if (dk == 64 && dv == 128) return launch_decode<64, 128, T>(q, k, v, log_alpha, beta, S, o, units, stream);
    return launch_decode<64, 64, T>(q, k, v, log_alpha, beta, S, o, units, stream);
}

// Host-side launcher used by the C ABI (sizes already validated).
hipError_t decode_step_launch(const void *q, const void *k, const void *v,
                              const void *log_alpha, const void *beta, float *S,
                              void *o, int units, int dk, int dv, bool bf16,
                              hipStream_t stream)
{
    if (units == 0) return hipSuccess;
    if (bf16) return dispatch_decode_t<bf16_t>(q, k, v, log_alpha, beta, S, o, units, dk, dv, stream);
    return dispatch_decode_t<float>(q, k, v, log_alpha, beta, S, o, units, dk, dv, stream);
}

}  // namespace kda
