/*
 * moe_probe.h -- ceiling probes of one MI355X (libmoe_probe.so), the measured
 * denominators reported beside the published peaks when the layer's kernels
 * are priced against a roofline. They are not part of the layer.
 *
 * Every pointer is a DEVICE pointer owned by the caller; every call only
 * enqueues one kernel on `stream` (a hipStream_t) and returns 0, -1 for a bad
 * argument (nothing enqueued) or -4 when the launch fails.
 */
#ifndef MOE_PROBE_H_
#define MOE_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Back-to-back matrix-core instructions with no memory traffic: `blocks`
   workgroups of 4 waves, each wave `iters` rounds of 4 independent
   accumulators. kind 0: v_mfma_f32_32x32x16_bf16 on fixed operands; kind 1:
   v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 x E2M1 operands (the scaled-MFMA
   expert path); kinds 2 and 3: the same two instructions on pseudo-random
   operands that change at every instruction, as in a real GEMM; kinds 4 and
   5: v_mfma_f32_16x16x32_bf16 (8 independent accumulators) on fixed and on
   changing operands (iters a multiple of 4 for kinds 2 to 5). out: one float per wave (blocks * 4), written so the work is live; its
   values mean nothing. */
int moe_probe_mfma(int kind, int blocks, int iters, float* out, void* stream);

/* Algorithmic FLOP of one moe_probe_mfma call (host only, no HIP call). */
double moe_probe_mfma_flops(int kind, int blocks, int iters);

/* Streaming read of `bytes` (a multiple of 16; buf 16-byte aligned) by
   `blocks` workgroups of 256 threads, each thread with `unroll & 0xFF` (4, 8
   or 16) 16-byte loads in flight, nontemporal loads when unroll has bit
   0x100. Spans of the buffer go to the blocks grid-stride, or, with bit
   0x200, each block reads one contiguous part (1/blocks of the buffer) from
   start to end. out: blocks * 256 words written. */
int moe_probe_hbm_read(const void* buf, int64_t bytes, int blocks, int unroll, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H_ */
