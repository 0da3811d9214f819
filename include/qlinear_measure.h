/* qlinear_measure.h -- a measurement aid of libqlinear.so, outside the
 * method: a streaming kernel with the access pattern of the quantize cast
 * (16-byte non-temporal loads and plain stores, 32 bytes read and
 * optionally 16 bytes written per unit, the same grid shape) and none of
 * its arithmetic.  Its rate is the
 * memory system's ceiling for that pattern, against which the quantize
 * rates are read; the benchmark times it next to them.
 *
 * All pointers are device pointers; the call is asynchronous on `stream`
 * (a hipStream_t, NULL for the default stream).  Status codes as in
 * qlinear.h (QL_OK = 0).
 */
#ifndef QLINEAR_MEASURE_H
#define QLINEAR_MEASURE_H

#include <stdint.h>

#include "qlinear.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads n_units 32-byte units of src.  With dst non-NULL, writes for unit
 * u the 16 bytes dst[16u .. 16u+15] = src[32u .. 32u+15] XOR
 * src[32u+16 .. 32u+31] (bytewise); with dst NULL it writes only one
 * 4-byte word per thread of the grid into sink (sink[0 .. 262143], 1 MiB:
 * the fold of what that thread read, so no load can be dropped).
 *   src, dst, sink: 16-byte aligned; src holds 32*n_units bytes, dst
 *   16*n_units.  Exactly one of dst and sink is non-NULL when n_units > 0.
 * Errors: QL_ERR_VALUE for n_units < 0 or a misaligned pointer, QL_ERR_NULL
 * for a missing buffer, QL_ERR_HIP if the launch fails.  Nothing is
 * enqueued on error.
 */
ql_status ql_stream_probe(const void *src, int64_t n_units, void *dst, void *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_MEASURE_H */
