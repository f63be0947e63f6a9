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

}  // namespace kda
