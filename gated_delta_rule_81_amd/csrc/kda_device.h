// kda_device.h -- small device helpers shared by the KDA kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Storage type of a bf16 tensor element (raw bits; conversions below).
struct bf16_t {
    uint16_t x;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t b) { return __uint_as_float((uint32_t)b.x << 16); }

// fp32 -> bf16 with round-to-nearest-even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t to_bf16(float v) {
    __bf16 h = (__bf16)v;
    bf16_t r;
    r.x = __builtin_bit_cast(uint16_t, h);
    return r;
}

__device__ __forceinline__ void store_elem(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(bf16_t *p, float v) { *p = to_bf16(v); }

__device__ __forceinline__ float load_elem(const float *p) { return *p; }
__device__ __forceinline__ float load_elem(const bf16_t *p) { return to_f32(*p); }

constexpr float kLog2e = 1.4426950408889634f;

// Layout of the forget gate log_alpha (values match kda_gate in kda.h):
// one value per key channel, one per (token, head) shared by every key
// channel, or none (alpha = 1).
enum : int { GATE_CHANNEL = 0, GATE_HEAD = 1, GATE_NONE = 2 };

// Input preparation folded into the kernels (bits match kda_flags in kda.h):
// q and k divided by their L2 norm over d_k per token and head; the gate
// tensor holding x with log_alpha = -softplus(x).
enum : int { PREP_L2NORM = 1, PREP_SOFTPLUS = 2 };
// alpha = e^{-softplus(x)} = 1 / (1 + e^x), and its log2 (-softplus(x) log2 e,
// in a form that neither overflows nor loses small values)
__device__ __forceinline__ float alpha_softplus(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * kLog2e));
}
__device__ __forceinline__ float log2_alpha_softplus(float x) {
    const float ax = x < 0.0f ? -x : x;
    return -((x > 0.0f ? x : 0.0f) * kLog2e +
             __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(-ax * kLog2e)));
}
// 1 / |x| for a squared norm, a zero vector staying zero
__device__ __forceinline__ float inv_norm(float sumsq) {
    return sumsq > 0.0f ? __builtin_amdgcn_rsqf(sumsq) : 0.0f;
}

// Row of the state arrays that a sequence (or decode slot) reads and writes:
// the sequence index itself, or state_idx[seq] when a slot map is given;
// -1 (start from zeros, write nothing) for an index outside [0, pool).
__device__ __forceinline__ long state_row(const int32_t *state_idx, int pool, int seq) {
    if (!state_idx) return seq;
    const int r = state_idx[seq];
    return (r >= 0 && r < pool) ? (long)r : -1L;
}

}  // namespace kda
