/*
 * moe_probe.h -- measurement entry points of libmoe (not part of the MoE
 * layer's path): a read-stream reference kernel and a phase-timed copy of the
 * expert FFN call.  Conventions as in moe.h: device pointers, the call only
 * enqueues on `stream`, never allocates or synchronises, and validates its
 * arguments on the host first.
 */
#ifndef MOE_PROBE_H_
#define MOE_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

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

/*
 * The expert FFN with its three launches timed apart: moe_expert_ffn (same
 * arguments, validation, kernels and results) with four caller-created HIP
 * events (hipEvent_t, passed as void*) recorded on `stream` before phase A
 * (gate/up + SwiGLU), after phase A, after phase B (down projection and
 * routing weight) and after the combine.  Elapsed times between them are the
 * phases' durations on the stream the kernels run on; the heaviest phase is
 * the one priced against the HBM roofline [OEA section 4, Eq. 2: each active
 * expert costs one weight fetch].  A null entry of `events` is skipped.
 * Errors: as moe_expert_ffn; MOE_EINVAL for a null `events` array.
 */
int moe_expert_ffn_phase_events(const moe_expert_handle *table, int N, int H, int I, const void *x, int x_dtype,
                                const int32_t *idx, const float *w, const int32_t *offsets, const int32_t *perm,
                                const int32_t *active, const int32_t *T, int B, int k, float *y, void *ws,
                                size_t ws_bytes, void *const *events, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PROBE_H_ */
