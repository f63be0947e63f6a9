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

// Layout of the backward's bf16 per-chunk matrices with d_v columns (the
// states S and their gradients D, d_k x d_v; X, U and dU, 32 x d_v) in its
// workspace: 16-column strips, each rows x 16 contiguous.  The kernels that
// write them hold 16-column strips per wave, so every store covers whole
// 128-byte lines.  Element (row, col) of a matrix with `rows` rows:
// Those stores are made non-temporal (the cache-policy operand of the buffer
// store: nt): a later kernel reads the matrices, long after they would have
// left the L2, so allocating them there only pushes out lines still in use.
constexpr int kStreamStore = 2;
__device__ __forceinline__ size_t strip_off(int row, int col, int rows) {
    return (size_t)(col >> 4) * rows * 16 + (size_t)row * 16 + (col & 15);
}

// Four rows of a 16-column strip as bf16 row segments for 8-byte stores.  A
// lane (column n of the strip) holds rows 0..3 of its column as two bf16
// pairs w0 (rows 0, 1) and w1 (rows 2, 3); after two exchanges inside its
// quad of lanes it holds columns (n & ~3) .. + 3 of row quad_row(n), where
// quad_row = 0, 2, 1, 3 for n & 3 = 0, 1, 2, 3.  Every lane of the wave
// must take part (the exchanges read the neighbours' registers).
__device__ __forceinline__ int quad_row(int n) { return ((n & 1) << 1) | ((n >> 1) & 1); }
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 quad_rows(uint32_t w0, uint32_t w1, int n) {
    const bool odd = n & 1, up = n & 2;
    // with lane n ^ 1: the even lane gets rows 0, 1 of columns n, n + 1, the
    // odd lane rows 2, 3 of columns n - 1, n
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? w0 : w1), 0xB1, 0xf, 0xf, false);
    // (selects of plain values first: selects of whole expressions become branches)
    const uint32_t a = odd ? r1 : w0, b = odd ? w1 : r1;    // columns n & ~1 and n | 1
    const uint32_t d0 = __builtin_amdgcn_perm(b, a, 0x05040100u);   // low halves: a.lo, b.lo
    const uint32_t d1 = __builtin_amdgcn_perm(b, a, 0x07060302u);   // high halves: a.hi, b.hi
    // with lane n ^ 2: the other two columns of the kept row
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(up ? d0 : d1), 0x4E, 0xf, 0xf, false);
    u32x2 v;
    v.x = up ? r2 : d0;
    v.y = up ? d1 : r2;
    return v;
}

}  // namespace kda
