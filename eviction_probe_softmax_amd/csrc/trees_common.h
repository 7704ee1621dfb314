// Definitions shared by the tree kernels: argument block, work-item lookup
// and the hardware square root and reciprocal.
#pragma once

#include "kvc_internal.h"

namespace kvc_tree {

struct TreeKArgs {
  const void* K;
  const void* V;
  const void* Qp;
  const float* lse;        // [S][Ly][H*G][P]
  const float* rel;        // [Ly][H][T]
  const float* sens;       // [S][Ly][H]
  const float* rc;
  const float* rs;
  const int32_t* slot_start;
  const int2* list;        // [S][stride] (start, length) of the slots of this size class
  const int32_t* count;    // [S] their number
  const int64_t* cu;
  int S, Ly, H, G, P, stride, pd, pstride;
  int64_t T;
  float c;                 // 1/sqrt(d)
  float beta, wA, wV;
  float* node_rel;
  float* node_D;
  float* node_mu;
  float* op_util;
  uint8_t* op_cost;
  const uint32_t* topo;    // explicit node records (split_mode 1), else NULL: midpoint trees
};

// the hardware square root and reciprocal (about 1 ulp each) instead of the
// correctly rounded library sequences, which cost a dozen instructions apiece
__device__ __forceinline__ float hw_sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }
__device__ __forceinline__ float hw_div(float x, float y) { return x * __builtin_amdgcn_rcpf(y); }

struct ItemDesc {
  int64_t lh;
  int s, t0, n;
};

// Work item w (unit-major over this size class) -> unit, sequence, slot.
// pre[s] = number of this class's slots in sequences before s (pre[S] = total).
__device__ __forceinline__ ItemDesc item_desc(const TreeKArgs& a, const int* pre, int64_t nsl, int64_t w) {
  ItemDesc d;
  d.lh = w / nsl;
  const int rr = (int)(w - d.lh * nsl);
  int s = 0;
  while (rr >= pre[s + 1]) ++s;
  d.s = s;
  const int2 e = a.list[(int64_t)s * a.stride + (rr - pre[s])];
  d.t0 = e.x;
  d.n = e.y;
  return d;
}

constexpr int MAX_SEQ = 256;  // sequences per call (prefix of the class counts lives in LDS)

// Midpoint trees of slots of at most 64 tokens, bf16 keys and values of head
// dimension 128, on the fixed 64-position layout (trees_v.hip).
int launch_trees_v(const TreeKArgs& a, int64_t bound, int ncu, hipStream_t st);


}  // namespace kvc_tree
