// Internal helpers shared by the libkvc sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <cmath>
#include <stddef.h>
#include <string>
#include <vector>

#include "kvc.h"

namespace kvc {

// ------------------------------------------------------------------ errors
int set_error(int status, const std::string& msg);
#define KVC_REQUIRE(cond, status, msg)                         \
  do {                                                         \
    if (!(cond)) return ::kvc::set_error((status), (msg));     \
  } while (0)
#define KVC_LAUNCH_CHECK(what)                                                        \
  do {                                                                                \
    hipError_t e_ = hipGetLastError();                                                \
    if (e_ != hipSuccess)                                                             \
      return ::kvc::set_error(KVC_E_HIP, std::string(what) + ": " + hipGetErrorString(e_)); \
  } while (0)

// ------------------------------------------------------------------ host shape helpers
struct Regions {
  int64_t pe, c0, c1, ss;  // prompt end, compressible [c0,c1), suffix start
};
inline Regions regions_of(int64_t L, const kvc_params& p) {
  Regions r;
  r.pe = L < p.prompt_exact ? L : p.prompt_exact;
  int64_t ss = L - p.suffix_exact;
  r.ss = ss > r.pe ? ss : r.pe;
  int64_t rs = r.ss - p.recent_exact;
  r.c1 = rs > r.pe ? rs : r.pe;
  r.c0 = r.pe;
  return r;
}
// Head-level hybrid: units of a sequence kept whole, given its allocatable
// budget and its compressible tokens per unit C.
inline int64_t hybrid_units_of(int64_t alloc, int64_t C, int64_t units, const kvc_params& p) {
  if (!(p.hybrid_frac > 0.f) || C <= 0 || alloc <= 0) return 0;
  int64_t k = (int64_t)std::floor((double)p.hybrid_frac * (double)units);
  int64_t byb = alloc / C;
  k = k < byb ? k : byb;
  return k < units ? k : units;
}
// keep[i] = 1 for the top-budget[s] elements of each segment
// [start[s], start[s] + len[s]) of score by (score desc, pos asc) (the element
// index when pos is NULL); other elements of the segments get 0. Host arrays.
size_t ws_topk_segments();
int topk_segments(int S, const int64_t* start, const int64_t* len, const int64_t* budget, const float* score,
                  const int32_t* pos, uint8_t* keep, void* ws, size_t ws_bytes, hipStream_t stream);
int score_strided(const kvc_shape* sh, const kvc_params* p, const void* K, const void* V, const void* Qprobe,
                  float* rel0, float* feats, float* probe_lse, float* probe_ent, float* head_sens, void* ws,
                  size_t ws_bytes, hipStream_t st);
int validate_shape(const kvc_shape* s);
int validate_params(const kvc_shape* s, const kvc_params* p);
int64_t max_len(const kvc_shape* s);

// Bump allocator over the caller's workspace (256-byte aligned pieces).
struct Carver {
  char* base;
  size_t size, off = 0;
  Carver(void* b, size_t n) : base((char*)b), size(n) {}
  template <class T>
  T* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = (T*)(base ? base + off : nullptr);
    off += count * sizeof(T);
    return p;
  }
  bool ok() const { return off <= size; }
};

// Per-stage workspace sizes (each stage file defines its own).
size_t ws_score(const kvc_shape* s, const kvc_params* p);
size_t ws_propagate(const kvc_shape* s, const kvc_params* p);
size_t ws_partition(const kvc_shape* s, const kvc_params* p);
size_t ws_trees(const kvc_shape* s, const kvc_params* p);
size_t ws_auction(const kvc_shape* s, const kvc_params* p);
size_t ws_pack(const kvc_shape* s, const kvc_params* p);

// Segmented selection (select.hip): among elements of each segment, find the
// largest set by 64-bit key (descending) whose summed weight stays <= budget.
struct SelectPlan;

}  // namespace kvc

// ------------------------------------------------------------------ device helpers
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 kvc_bf16x8;
typedef float kvc_f32x16 __attribute__((ext_vector_type(16)));
typedef float kvc_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// The same rounding by gfx950's v_cvt_pk_bf16_f32 (identical bits for every
// fp32 input). Only for values computed in fp32: the compiler may merge a
// preceding double -> float conversion into one double -> bf16 rounding.
__device__ __forceinline__ uint16_t f32_to_bf16_hw(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <class T> struct ElemIO;
template <> struct ElemIO<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct ElemIO<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
  static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// Lane exchanges on the VALU rather than LDS permutes. DPP: quad_perm [1,0,3,2]
// and [2,3,0,1] (neighbours at distance 1 and 2), row_half_mirror (lane i of
// each 8-lane group reads lane 7 - i), row_mirror (lane i of each 16-lane row
// reads lane 15 - i). v_permlane16_swap / v_permlane32_swap with one register
// as both operands leave, per lane, the values of rows {2k, 2k+1} (resp. the
// two 32-lane halves) in the two results. Each step combines a value that is
// uniform over one half of a group with the other half's, and the operations
// used are commutative, so every lane of a group ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
struct OpAdd {
  static __device__ __forceinline__ float f(float x, float y) { return x + y; }
};
struct OpMax {
  static __device__ __forceinline__ float f(float x, float y) { return fmaxf(x, y); }
};
// reduction over aligned groups of W lanes (W = 2, 4, ..., 64), in every lane
// of the group; every lane of a group must be active (for W >= 32, the wave)
template <int W, class Op>
__device__ __forceinline__ float group_reduce(float v) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group width");
  if constexpr (W >= 2) v = Op::f(v, dpp_f32<0xB1>(v));
  if constexpr (W >= 4) v = Op::f(v, dpp_f32<0x4E>(v));
  if constexpr (W >= 8) v = Op::f(v, dpp_f32<0x141>(v));
  if constexpr (W >= 16) v = Op::f(v, dpp_f32<0x140>(v));
  if constexpr (W >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if constexpr (W >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return v;
}
template <int W>
__device__ __forceinline__ float group_sum(float v) { return group_reduce<W, OpAdd>(v); }
template <int W>
__device__ __forceinline__ float group_max(float v) { return group_reduce<W, OpMax>(v); }
// Four sums over the wave at once (the whole wave active). v_permlane32_swap
// on (a, b) leaves the pair sums of a in lanes 0-31 and of b in lanes 32-63,
// likewise for (c, d); v_permlane16_swap on the two results leaves, per
// 16-lane row, a (row 0), c (row 1), b (row 2), d (row 3); DPP finishes each
// row. Returns (sum a, sum b, sum c, sum d), uniform over the wave.
__device__ __forceinline__ float4 wave_sum4(float a, float b, float c, float d) {
  const auto ab = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const auto cd = __builtin_amdgcn_permlane32_swap(__float_as_uint(c), __float_as_uint(d), false, false);
  const float x = __uint_as_float(ab[0]) + __uint_as_float(ab[1]);
  const float y = __uint_as_float(cd[0]) + __uint_as_float(cd[1]);
  const auto xy = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  float v = __uint_as_float(xy[0]) + __uint_as_float(xy[1]);
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  const int iv = __float_as_int(v);
  return make_float4(__int_as_float(__builtin_amdgcn_readlane(iv, 0)), __int_as_float(__builtin_amdgcn_readlane(iv, 32)),
                     __int_as_float(__builtin_amdgcn_readlane(iv, 16)), __int_as_float(__builtin_amdgcn_readlane(iv, 48)));
}
// sum over the lanes i and i ^ 32, in both
__device__ __forceinline__ float group_sum_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// sum over the lanes i, i ^ 16, i ^ 32, i ^ 48 (the four rows), in each of them
__device__ __forceinline__ float cross_row_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}
// minimum of a signed 64-bit value over the wave, in every lane (the same
// exchanges on both 32-bit halves); the whole wave must be active
template <int CTRL>
__device__ __forceinline__ int64_t dpp_i64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)((uint64_t)v >> 32), CTRL, 0xF, 0xF, false);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int64_t wave_min_i64(int64_t v) {
  v = min(v, dpp_i64<0xB1>(v));
  v = min(v, dpp_i64<0x4E>(v));
  v = min(v, dpp_i64<0x141>(v));
  v = min(v, dpp_i64<0x140>(v));
  {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)((uint64_t)v >> 32);
    const auto rl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto rh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const int64_t a = (int64_t)(((uint64_t)rh[0] << 32) | rl[0]), b = (int64_t)(((uint64_t)rh[1] << 32) | rl[1]);
    v = min(a, b);
  }
  {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)((uint64_t)v >> 32);
    const auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const int64_t a = (int64_t)(((uint64_t)rh[0] << 32) | rl[0]), b = (int64_t)(((uint64_t)rh[1] << 32) | rl[1]);
    v = min(a, b);
  }
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// 2^x on the hardware exponential (results below 2^-126 flush to zero; the
// library's denormal-safe exp2f adds a range check and a rescale per call).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Order-preserving map of an fp32 score to uint32 (NaN -> 0, i.e. lowest).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  if (f != f) return 0u;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// 64-bit selection key: larger = earlier; ties on the score go to the lower id.
__device__ __forceinline__ uint64_t make_key(float score, uint32_t id) {
  return ((uint64_t)f32_order_key(score) << 32) | (uint64_t)(0xffffffffu - id);
}
__device__ __forceinline__ uint32_t key_id(uint64_t k) { return 0xffffffffu - (uint32_t)k; }

// Sequence of a global token index (S is small; linear scan).
__device__ __forceinline__ int seq_of(const int64_t* cu, int S, int64_t t) {
  int s = 0;
  while (s + 1 < S && cu[s + 1] <= t) ++s;
  return s;
}

inline unsigned kvc_blocks(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }
