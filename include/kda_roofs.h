/*
 * libkda_roofs — measurement kernels for the roofs the benchmark reports its
 * rates against (HBM streaming bandwidth and the bf16 matrix-core issue rate
 * of one MI355X).  Not part of the KDA path; libkda does not use it.
 *
 * Every call launches on `stream` (a hipStream_t, NULL = the null stream),
 * times its own launches with two HIP events, waits for them, and returns 0
 * on success, 1 on bad arguments (nothing launched), 2 on a HIP error.
 */
#ifndef KDA_ROOFS_H
#define KDA_ROOFS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * kda_roof_stream — mode 0 reads `bytes` of src, 1 writes `bytes` of dst,
 * 2 copies src to dst, 3 updates dst in place (reads each 16-byte vector and
 * writes it back, each word + 1); 16-byte vector accesses.  workgroups > 0:
 * grid-stride over that many workgroups of 256 threads, four vectors in
 * flight per thread; workgroups == 0 (modes 1-3): one vector per thread, the
 * grid covering the buffer.  bytes is a positive multiple of 16; src and dst
 * are 16-byte aligned device buffers of at least `bytes`.  Mode 0 writes one
 * uint32 per thread to `sink` (device, at least workgroups * 256 words).
 * One untimed launch, then `reps` timed back to back: *ms_per_launch is
 * their mean.
 */
int kda_roof_stream(int mode, const void* src, void* dst, int64_t bytes, void* sink, int64_t sink_words,
                    int workgroups, int reps, void* stream, float* ms_per_launch);

/*
 * kda_roof_state_inplace — updates `bytes` of buf in place as 64 KB blocks of
 * 128 x 128 fp32 (each word + 1 after `delay` rounds of dependent arithmetic
 * on it, 0 <= delay <= 4096), one workgroup of 256 threads per block, in the
 * access pattern of kda_decode_step on a d_k = d_v = 128 state: 16-byte loads
 * all in flight, then streaming 16-byte stores.  bytes is a positive
 * multiple of 65536; buf a 16-byte aligned device buffer of at least that.
 * One untimed launch, then `reps` timed back to back: *ms_per_launch is
 * their mean (each launch reads and writes `bytes`).
 */
int kda_roof_state_inplace(void* buf, int64_t bytes, int delay, int reps, void* stream, float* ms_per_launch);

/*
 * kda_roof_mfma — `workgroups` workgroups of four waves, each wave issuing
 * `iters` rounds of eight independent 16x16x32 bf16 matrix-core instructions
 * (fp32 accumulation).  `sink`: device float buffer of workgroups * 256.
 * One untimed launch, then one timed: *ms_per_launch, and the dense flops
 * (2 per multiply-add) it performed in *flops_per_launch.
 */
int kda_roof_mfma(int workgroups, int iters, void* sink, void* stream, float* ms_per_launch,
                  double* flops_per_launch);

#ifdef __cplusplus
}
#endif

#endif /* KDA_ROOFS_H */
