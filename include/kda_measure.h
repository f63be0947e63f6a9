/*
 * kda_measure.h -- measurement kernels shipped with the KDA library.
 *
 * Not part of the operator: they give the practical HBM ceiling that the
 * operator's bandwidth-bound kernels are compared with, using the decode
 * step's own access pattern (16-byte non-temporal loads and stores from a
 * persistent grid).  Conventions as in kda.h: device pointers, 16-byte
 * aligned, work enqueued on `stream` (a hipStream_t as void*, NULL = null
 * stream) without synchronising, status codes only.
 */
#ifndef KDA_MEASURE_H_
#define KDA_MEASURE_H_

#include <stddef.h>

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0 .. bytes) = src[0 .. bytes): every byte read once and written once.
 * bytes must be a multiple of 16; the buffers must not overlap.
 * KDA_ERR_INVALID_ARG for NULL or misaligned pointers or a bad size. */
kda_status kda_measure_copy(const void *src, void *dst, size_t bytes, void *stream);

/* buf[0 .. bytes) read and written back in place (fp32 values plus 0), the
 * read-modify-write traffic of the decode step's state cache.  bytes must be
 * a multiple of 16. */
kda_status kda_measure_rmw(void *buf, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_MEASURE_H_ */
