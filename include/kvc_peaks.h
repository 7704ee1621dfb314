/*
 * libkvc measurement helpers: kernels that measure this machine's own
 * ceilings, so that the roofline fractions of the path's kernels can be given
 * against measured peaks as well as the vendor's. They are not part of the
 * method (no page defines them). Same conventions as kvc.h: plain pointers,
 * asynchronous on the caller's stream, arguments checked on the host before
 * the launch, no state kept, kvc_last_error() for the message.
 */
#ifndef KVC_PEAKS_H_
#define KVC_PEAKS_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HBM read ceiling: one pass of 16-byte nontemporal loads over `bytes` of
 * device memory at `buf` (both multiples of 16), cut into `grid` contiguous
 * spans, one per workgroup of 256 threads (each load instruction covers
 * whole 128-byte lines), eight loads in flight per thread. The XOR of
 * all words read is stored to *sink (device) only if it equals a fixed
 * constant, so no load can be dropped; the caller times the launch.
 * KVC_E_INVAL on NULL pointers, zero or misaligned sizes, grid < 1. */
int kvc_peak_read(const void* buf, size_t bytes, int32_t grid, uint32_t* sink, hipStream_t stream);

/* bf16 MFMA ceiling: `grid` workgroups of 256 threads; every wave runs `iters`
 * rounds of four independent v_mfma_f32_32x32x16_bf16 chains on register
 * operands (no memory traffic in the loop), 4 * 32768 flops a round. Each
 * workgroup stores one sum of its accumulators to sink[blockIdx] (device,
 * `grid` floats). Flops of a launch = grid * 4 * iters * 131072.
 * KVC_E_INVAL on a NULL sink, grid < 1 or iters < 1. */
int kvc_peak_mfma(int32_t grid, int32_t iters, float* sink, hipStream_t stream);

/* Exponential-mix ceiling (the per-logit VALU work of the probe passes):
 * `grid` workgroups of 256 threads; every thread runs `iters` rounds of 8
 * independent chains, each round one v_exp_f32 and three VALU operations
 * (two fused multiply-adds and an add) on registers. Each workgroup stores
 * one sum to sink[blockIdx] (device, `grid` floats). Elements of a launch =
 * grid * 256 * iters * 8. KVC_E_INVAL on a NULL sink, grid < 1 or iters < 1. */
int kvc_peak_exp(int32_t grid, int32_t iters, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_PEAKS_H_ */
