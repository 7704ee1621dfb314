// Measurement helpers: the HBM read ceiling (nontemporal 16-byte loads, one
// contiguous span a workgroup), the bf16 MFMA ceiling (register-only MFMA
// chains) and the exponential-mix ceiling (register-only chains of one
// hardware exponential and three VALU operations) of the device, timed by the
// caller.
#include "kvc_internal.h"
#include "kvc_peaks.h"

namespace {

typedef unsigned int pk_u32x4 __attribute__((ext_vector_type(4)));
constexpr int READ_THREADS = 256;
constexpr int READ_UNROLL = 8;

// each workgroup streams one contiguous span of the buffer (whole 128-byte
// lines per load instruction, nontemporal)
__global__ __launch_bounds__(READ_THREADS) void peak_read_kernel(const pk_u32x4* __restrict__ p, size_t n16,
                                                                 size_t span, uint32_t* sink) {
  const size_t b0 = (size_t)blockIdx.x * span;
  const size_t b1 = b0 + span < n16 ? b0 + span : n16;
  size_t i = b0 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (READ_UNROLL - 1) * READ_THREADS < b1; i += READ_UNROLL * READ_THREADS) {
    pk_u32x4 v[READ_UNROLL];
#pragma unroll
    for (int k = 0; k < READ_UNROLL; ++k) v[k] = __builtin_nontemporal_load(p + i + k * READ_THREADS);
#pragma unroll
    for (int k = 0; k < READ_UNROLL; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < b1; i += READ_THREADS) {
    const pk_u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) *sink = acc;
}

__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  // operands: small distinct values per lane, kept in registers
  kvc_bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)((lane + j) & 7));
    b[j] = (__bf16)(0.001f * (float)((lane * 3 + j) & 7));
  }
  kvc_f32x16 c0, c1, c2, c3;  // distinct starting values keep the four chains apart
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    c0[v] = 0.f;
    c1[v] = 1.f;
    c2[v] = 2.f;
    c3[v] = 3.f;
  }
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  s = wave_sum(s);
  __shared__ float ws[4];
  if (lane == 0) ws[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = ws[0] + ws[1] + ws[2] + ws[3];
}

// Exponential-mix ceiling: every thread runs 8 independent chains, each round
// one base-2 exponential (the hardware v_exp_f32) and three VALU operations,
// x <- fma(e, 0.5, -0.25); e <- exp2(x); s <- s + e; t <- fma(e, h, t), the
// per-logit mix of the probe passes (a shifted exponential, a running sum and
// a weighted sum). Values stay in [2^-0.25, 2^0.25]: no denormals, no overflow.
__global__ __launch_bounds__(256) void peak_exp_kernel(int iters, float* sink) {
  float x[8], s[8], t[8];
  const float h = 0.37f + 1e-3f * (float)(threadIdx.x & 7);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[k] = 0.01f * (float)k;
    s[k] = 0.f;
    t[k] = 0.f;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float e = __builtin_amdgcn_exp2f(x[k]);
      s[k] += e;
      t[k] = fmaf(e, h, t[k]);
      x[k] = fmaf(e, 0.5f, -0.25f);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) r += s[k] + t[k];
  r = wave_sum(r);
  __shared__ float ws[4];
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = ws[0] + ws[1] + ws[2] + ws[3];
}

}  // namespace

extern "C" int kvc_peak_exp(int32_t grid, int32_t iters, float* sink, hipStream_t st) {
  KVC_REQUIRE(sink, KVC_E_INVAL, "kvc_peak_exp: NULL sink");
  KVC_REQUIRE(grid >= 1 && iters >= 1, KVC_E_INVAL, "kvc_peak_exp: grid and iters must be >= 1");
  hipLaunchKernelGGL(peak_exp_kernel, dim3((unsigned)grid), dim3(256), 0, st, iters, sink);
  KVC_LAUNCH_CHECK("peak_exp");
  return KVC_OK;
}

extern "C" int kvc_peak_read(const void* buf, size_t bytes, int32_t grid, uint32_t* sink, hipStream_t st) {
  KVC_REQUIRE(buf && sink, KVC_E_INVAL, "kvc_peak_read: NULL pointer");
  KVC_REQUIRE(bytes > 0 && bytes % 16 == 0 && ((uintptr_t)buf & 15) == 0, KVC_E_INVAL,
              "kvc_peak_read: bytes and buf must be nonzero multiples of 16");
  KVC_REQUIRE(grid >= 1, KVC_E_INVAL, "kvc_peak_read: grid must be >= 1");
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(peak_read_kernel, dim3((unsigned)grid), dim3(READ_THREADS), 0, st, (const pk_u32x4*)buf, n16,
                     (n16 + (size_t)grid - 1) / (size_t)grid, sink);
  KVC_LAUNCH_CHECK("peak_read");
  return KVC_OK;
}

extern "C" int kvc_peak_mfma(int32_t grid, int32_t iters, float* sink, hipStream_t st) {
  KVC_REQUIRE(sink, KVC_E_INVAL, "kvc_peak_mfma: NULL sink");
  KVC_REQUIRE(grid >= 1 && iters >= 1, KVC_E_INVAL, "kvc_peak_mfma: grid and iters must be >= 1");
  hipLaunchKernelGGL(peak_mfma_kernel, dim3((unsigned)grid), dim3(256), 0, st, iters, sink);
  KVC_LAUNCH_CHECK("peak_mfma");
  return KVC_OK;
}
