// MFMA fragments shared by the kernels that run QK^T-style products.
//
// 32x32 output tiles, 16 elements of the reduction dimension per step:
// lane l holds row (l % 32) of A (or column l % 32 of B) and the reduction
// elements [8 (l / 32), 8 (l / 32) + 8) of the current 16-block - the same
// permutation on both operands, so any consistent assignment gives the same
// dot products. bf16 uses one v_mfma_f32_32x32x16_bf16; fp32 inputs use eight
// v_mfma_f32_32x32x2f32 (one per element pair).
// Accumulator register v of lane l holds row acc_row(v, l), column l % 32.
#pragma once

#include "kvc_internal.h"

namespace kvcmf {

template <class T> struct Frag;
template <> struct Frag<uint16_t> { kvc_bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

template <class T>
__device__ __forceinline__ Frag<T> load_frag(const T* p);
template <>
__device__ __forceinline__ Frag<uint16_t> load_frag<uint16_t>(const uint16_t* p) {
  Frag<uint16_t> f;
  uint4 u = *(const uint4*)p;
  f.v = __builtin_bit_cast(kvc_bf16x8, u);
  return f;
}
template <>
__device__ __forceinline__ Frag<float> load_frag<float>(const float* p) {
  Frag<float> f;
  float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}
template <class T>
__device__ __forceinline__ Frag<T> zero_frag() {
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    uint4 z = {0, 0, 0, 0};
    f.v = __builtin_bit_cast(kvc_bf16x8, z);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = 0.f;
  }
  return f;
}
__device__ __forceinline__ void mma(kvc_f32x16& acc, const Frag<uint16_t>& a, const Frag<uint16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(kvc_f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[j], b.v[j], acc, 0, 0, 0);
}
__device__ __forceinline__ int acc_row(int v, int lane) { return (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3); }

// 8 consecutive elements as floats
template <class T> struct Load8;
template <> struct Load8<uint16_t> {
  static __device__ __forceinline__ void f(const uint16_t* p, float* o) {
    uint4 u = *(const uint4*)p;
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Load8<float> {
  static __device__ __forceinline__ void f(const float* p, float* o) {
    float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

}  // namespace kvcmf
