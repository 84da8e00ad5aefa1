/*
 * moe_probe.h -- measurement reference kernel of libmoe (not part of the MoE
 * layer's path).  Conventions as in moe.h: device pointers, the call only
 * enqueues on `stream`, never allocates or synchronises, and validates its
 * arguments on the host first.
 */
#ifndef MOE_PROBE_H_
#define MOE_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * HBM read-stream ceiling: one pass over `bytes` bytes of `buf`, each wave
 * reading its own contiguous run of kilobytes with one 16-byte non-temporal
 * load per lane per kilobyte (the expert FFN's weight loads), 8 kilobytes in
 * flight per wave, waves_per_cu waves on each compute unit (workgroups of 4
 * waves).  The best rate over launch shapes is the measured ceiling the
 * weight-streaming kernels are compared with [OEA section 4, Eq. 2: the b*T
 * term is a weight fetch].
 *   buf          : device memory, 16-byte aligned; bytes a positive multiple of 16
 *   waves_per_cu : 4, 8, 12, ..., 32
 *   out          : device uint32 [1]; the XOR of every 32-bit word of buf is
 *                  XORed into it (so clear it first to read the checksum)
 * Errors: MOE_EINVAL for null or misaligned pointers or a bad size or shape.
 */
int moe_stream_read(const void *buf, size_t bytes, int waves_per_cu, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PROBE_H_ */
