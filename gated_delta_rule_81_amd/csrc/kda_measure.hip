// kda_measure.hip -- streaming kernels that measure the practical HBM ceiling
// on this GPU with the access pattern the decode step uses: 16-byte
// non-temporal buffer loads and stores from a persistent grid (four
// 1024-thread workgroups per CU), every load of a batch issued before its
// stores.  Not part of the operator; declared in include/kda_measure.h.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/kda_measure.h"

namespace kda {

int cu_count();

namespace {

constexpr int THREADS = 1024;
constexpr int BATCH = 8;            // 16-byte accesses per thread and block
constexpr int kNonTemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), 0,
                                             bytes, 0x00020000);
}

// dst[i] = src[i] (RMW: src == dst and each value is rewritten after an add
// of zero), over n16 16-byte units.  Each block of THREADS * BATCH units is
// one buffer window; accesses past the window's valid bytes read zero and
// drop their stores, so the ragged last block needs no branch.  As in the
// decode step, the loads of a workgroup's next block are issued before the
// stores of its current one, so a block's worth of reads is always in flight.
template <bool RMW>
__global__ __launch_bounds__(THREADS) void stream_kernel(const uint4 *src, uint4 *dst, size_t n16)
{
    constexpr size_t BLK = (size_t)THREADS * BATCH;
    const size_t nblk = (n16 + BLK - 1) / BLK;
    size_t b = blockIdx.x;
    if (b >= nblk) return;
    auto window = [&](size_t blk) {
        const size_t left = n16 - blk * BLK;
        return (uint32_t)((left < BLK ? left : BLK) * 16);
    };
    auto load = [&](size_t blk, uint4 (&r)[BATCH]) {
        const __amdgpu_buffer_rsrc_t rs = rsrc(src + blk * BLK, window(blk));
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
            r[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rs, (uint32_t)((i * THREADS + threadIdx.x) * 16), 0, kNonTemporal));
    };
    auto store = [&](size_t blk, const uint4 (&r)[BATCH]) {
        const __amdgpu_buffer_rsrc_t rd = rsrc(dst + blk * BLK, window(blk));
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            uint4 v = r[i];
            if constexpr (RMW) {
                v.x = __float_as_uint(__uint_as_float(v.x) + 0.0f);
                v.y = __float_as_uint(__uint_as_float(v.y) + 0.0f);
                v.z = __float_as_uint(__uint_as_float(v.z) + 0.0f);
                v.w = __float_as_uint(__uint_as_float(v.w) + 0.0f);
            }
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, v), rd,
                (uint32_t)((i * THREADS + threadIdx.x) * 16), 0, kNonTemporal);
        }
    };
    uint4 ra[BATCH], rb[BATCH];
    load(b, ra);
    // two register sets alternate, so the prefetched block is never copied
    for (;;) {
        const size_t nb = b + gridDim.x;
        if (nb < nblk) load(nb, rb);
        store(b, ra);
        if (nb >= nblk) return;
        b = nb + gridDim.x;
        if (b < nblk) load(b, ra);
        store(nb, rb);
        if (b >= nblk) return;
    }
}

template <bool RMW>
hipError_t launch(const void *src, void *dst, size_t bytes, hipStream_t stream)
{
    const size_t n16 = bytes / 16;
    const size_t blocks = (n16 + (size_t)THREADS * BATCH - 1) / ((size_t)THREADS * BATCH);
    const size_t grid = blocks < (size_t)(4 * cu_count()) ? blocks : (size_t)(4 * cu_count());
    hipLaunchKernelGGL((stream_kernel<RMW>), dim3((unsigned)grid), dim3(THREADS), 0, stream,
                       static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n16);
    return hipGetLastError();
}

bool ok_args(const void *a, const void *b, size_t bytes) {
    return a && b && (bytes % 16) == 0 && ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15u) == 0;
}

}  // namespace
}  // namespace kda

extern "C" {

kda_status kda_measure_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    if (bytes == 0) return KDA_OK;
    if (!kda::ok_args(src, dst, bytes)) return KDA_ERR_INVALID_ARG;
    return kda::launch<false>(src, dst, bytes, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK
                                                                                              : KDA_ERR_HIP;
}

kda_status kda_measure_rmw(void *buf, size_t bytes, void *stream)
{
    if (bytes == 0) return KDA_OK;
    if (!kda::ok_args(buf, buf, bytes)) return KDA_ERR_INVALID_ARG;
    return kda::launch<true>(buf, buf, bytes, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK
                                                                                             : KDA_ERR_HIP;
}

}  // extern "C"
