/*
 * ssm_calib.h -- a measurement aid beside the scan library, not part of the
 * scan: a plain read-modify-write stream over device memory, the ceiling that
 * a kernel moving the same bytes (one read and one write of each element,
 * nothing else) can reach.  The benchmark runs it over the same slot sets as
 * the decode step, which is almost nothing but that state traffic ("perf(cuda):
 * keep the Mamba2 scan state in registers, stage tokens by chunk #90", How
 * the layout was chosen).  Built into libssmcalib.so, separate from
 * libssmscan.so.
 */
#ifndef SSM_CALIB_H
#define SSM_CALIB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * data[i] = data[i] * a + b for i in [0, 4 * n_float4): one non-temporal
 * 16-byte load and store per element group, `per_lane` (1, 2, 4 or 8) groups
 * per lane, 256 lanes per workgroup, consecutive lanes on consecutive groups.
 * `data` is a 16-byte aligned DEVICE pointer owned by the caller; n_float4
 * must be a positive multiple of 256 * per_lane.  Enqueued on `stream` (a
 * hipStream_t), no allocation, no synchronisation.  Returns 0, -2 (sizes),
 * -4 (alignment), -5 (launch refused).
 */
int ssm_calib_stream_rw(float *data, int64_t n_float4, int32_t per_lane, float a, float b,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_CALIB_H */
