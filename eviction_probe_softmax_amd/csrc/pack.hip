// Physical ragged cache packing.
//
// GraceKV page, '05 Physical cache packing': every (layer, KV head) gets an
// independently sized segment; an unselected root writes nothing, an internal
// frontier node writes its prototype, a singleton writes the original K/V;
// 'Inside one cache entry': the prototype key is the mean of the
// inverse-rotated keys re-rotated at a representative position, the value is
// relevance weighted with a uniform base.
//
// Every taken op adds op_cost stored entries (Add creates the root; a Split
// replaces one node by its children: 1 for a binary split, 2 for a three-way
// one), so the entries of a slot are the costs of the taken ops of its 2n op
// range. Per token t the count c[t] is: 1 for exact tokens, taken[t] in token
// mode, the taken costs of ops 2t and 2t+1 inside slots (the slot starting at
// t0 owns ops [2 t0, 2 t0 + 2n)). One exclusive scan over the
// whole [Ly][H][T] count array - whose order is exactly the (l, h, s, t) order
// of the segments - gives every token's (and every slot's first) output
// offset. Writers: exact/kept tokens copy their bits; one wave per slot walks
// the frontier in pre-order (= position order) and writes leaves and
// prototypes.
#include <algorithm>
#include <cmath>

#include "kvc_internal.h"
#include "mfma_frag.h"

namespace {

constexpr int SCAN_BLOCK = 4096;  // elements per scan block (256 threads x 16)

struct PackArgs {
  const void* K;
  const void* V;
  const float* rel;
  const float* node_rel;
  const float* node_mu;
  const uint8_t* taken;
  const uint8_t* op_cost;   // explicit trees: entries each op adds (NULL: 1 each)
  const uint32_t* topo;     // explicit trees' node records (NULL: midpoint trees)
  const int32_t* slot_start;
  const int32_t* n_slots;
  const float* rc;  // rope cos [pos][d/2]
  const float* rs;
  const int64_t* cu;
  int S, Ly, H, stride, token_mode;
  int64_t T;
  int64_t pe[64], c1[64];   // per sequence: prompt end (= compressible start), compressible end
  int64_t xoff[65];         // prefix over sequences of the exact tokens (prompt + recent + suffix)
  int32_t sbound[65];       // prefix over sequences of a bound on their slot counts (the slot writer's grid)
  float beta;               // uniform share of prototype values
  void* oK;
  void* oV;
  float* olnmu;
  int32_t* opos;
  int64_t capacity;
};

__device__ __forceinline__ int seq_of_tok(const PackArgs& a, int64_t t) { return seq_of(a.cu, a.S, t); }

__global__ void count_kernel(PackArgs a, int32_t* cnt) {
  int64_t E = (int64_t)a.Ly * a.H * a.T;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= E) return;
  int64_t lh = i / a.T, t = i % a.T;
  int s = seq_of_tok(a, t);
  int64_t p = t - a.cu[s];
  int c;
  if (p < a.pe[s] || p >= a.c1[s]) c = 1;
  else if (a.token_mode) c = a.taken[i];
  else {
    int64_t o = lh * 2 * a.T + 2 * t;
    c = a.op_cost ? (a.taken[o] ? a.op_cost[o] : 0) + (a.taken[o + 1] ? a.op_cost[o + 1] : 0)
                  : a.taken[o] + a.taken[o + 1];
  }
  cnt[i] = c;
}

// block-local exclusive scan; block totals to bsum
__global__ __launch_bounds__(256) void scan_local_kernel(const int32_t* cnt, int64_t n, int64_t* out, int64_t* bsum) {
  __shared__ int64_t part[256];
  int64_t b0 = (int64_t)blockIdx.x * SCAN_BLOCK;
  int64_t v[16];
  int64_t run = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    int64_t i = b0 + threadIdx.x * 16 + j;
    v[j] = i < n ? cnt[i] : 0;
    run += v[j];
  }
  part[threadIdx.x] = run;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    int64_t x = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += x;
    __syncthreads();
  }
  int64_t ex = part[threadIdx.x] - run;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    int64_t i = b0 + threadIdx.x * 16 + j;
    if (i < n) out[i] = ex;
    ex += v[j];
  }
  if (threadIdx.x == 255) bsum[blockIdx.x] = part[255];
}

// exclusive scan of the block totals in one block (sequential over chunks)
__global__ __launch_bounds__(256) void scan_blocks_kernel(int64_t* bsum, int64_t nb, int64_t* total) {
  __shared__ int64_t part[256];
  __shared__ int64_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int64_t c0 = 0; c0 < nb; c0 += 256) {
    int64_t i = c0 + threadIdx.x;
    int64_t v = i < nb ? bsum[i] : 0;
    part[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      int64_t x = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
      __syncthreads();
      part[threadIdx.x] += x;
      __syncthreads();
    }
    if (i < nb) bsum[i] = carry + part[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 255) carry += part[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) *total = carry;
}

__global__ void scan_add_kernel(int64_t* out, int64_t n, const int64_t* bsum) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] += bsum[i / SCAN_BLOCK];
}

__global__ void seg_kernel(PackArgs a, const int64_t* off, const int64_t* total, int64_t* seg_off,
                           int32_t* seg_len) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.S * a.Ly * a.H) return;
  int s = i / (a.Ly * a.H), lh = i % (a.Ly * a.H);
  int64_t b = (int64_t)lh * a.T + a.cu[s];
  int64_t e = (int64_t)lh * a.T + a.cu[s + 1];
  int64_t E = (int64_t)a.Ly * a.H * a.T;
  int64_t ob = b < E ? off[b] : *total;
  int64_t oe = e < E ? off[e] : *total;
  seg_off[i] = ob;
  seg_len[i] = (int32_t)(oe - ob);
}

// Exact tokens (prompt, recent window, suffix) of every (unit, sequence): one
// thread per 16-byte piece of a K or V row, over those tokens only.
template <class T, int D>
__global__ __launch_bounds__(256) void write_exact_kernel(PackArgs a, const int64_t* off) {
  constexpr int PPR = D * (int)sizeof(T) / 16;  // 16-byte pieces per row
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t X = a.xoff[a.S];
  const int64_t per_lh = X * 2 * PPR;
  if (g >= (int64_t)a.Ly * a.H * per_lh) return;
  const int64_t lh = g / per_lh, r = g % per_lh;
  const int64_t x = r / (2 * PPR);
  const int pc = (int)(r % (2 * PPR));
  int s = 0;
  while (s + 1 < a.S && a.xoff[s + 1] <= x) ++s;
  const int64_t k = x - a.xoff[s];
  const int64_t p = k < a.pe[s] ? k : a.c1[s] + (k - a.pe[s]);
  const int64_t i = lh * a.T + a.cu[s] + p;
  const int64_t dst = off[i];
  if (dst >= a.capacity) return;
  const bool isv = pc >= PPR;
  const int q = isv ? pc - PPR : pc;
  const uint4* src = (const uint4*)((const T*)(isv ? a.V : a.K) + i * D) + q;
  uint4* o = (uint4*)((T*)(isv ? a.oV : a.oK) + dst * D) + q;
  *o = *src;
  if (pc == 0) {
    a.olnmu[dst] = 0.f;
    a.opos[dst] = (int32_t)p;
  }
}

// Token mode: the kept tokens of the compressible regions, one thread per
// 16-byte piece of a K or V row.
template <class T, int D>
__global__ __launch_bounds__(256) void write_kept_kernel(PackArgs a, const int64_t* off) {
  constexpr int PPR = D * (int)sizeof(T) / 16;
  const int64_t E = (int64_t)a.Ly * a.H * a.T;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t i = g / (2 * PPR);
  const int pc = (int)(g % (2 * PPR));
  if (i >= E || !a.taken[i]) return;
  const int64_t t = i % a.T;
  const int s = seq_of_tok(a, t);
  const int64_t p = t - a.cu[s];
  if (p < a.pe[s] || p >= a.c1[s]) return;
  const int64_t dst = off[i];
  if (dst >= a.capacity) return;
  const bool isv = pc >= PPR;
  const int q = isv ? pc - PPR : pc;
  *((uint4*)((T*)(isv ? a.oV : a.oK) + dst * D) + q) = *((const uint4*)((const T*)(isv ? a.V : a.K) + i * D) + q);
  if (pc == 0) {
    a.olnmu[dst] = 0.f;
    a.opos[dst] = (int32_t)p;
  }
}

// 8 consecutive elements from fp32 values in one 16-byte store (bf16: RNE)
// or two (fp32).
template <class T>
__device__ __forceinline__ void store8(T* p, const float* x) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = (uint32_t)f32_to_bf16_hw(x[2 * q]) | ((uint32_t)f32_to_bf16_hw(x[2 * q + 1]) << 16);
    *(uint4*)p = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *(float4*)p = make_float4(x[0], x[1], x[2], x[3]);
    *(float4*)(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
}

// One workgroup per (unit, slot). Every node decides in parallel whether it
// is on the frontier (its creator op taken, its own Split not taken; the
// root's creator is the Add); a block scan gives the frontier in pre-order,
// which is position order. Then 16-byte pieces of the output rows are spread
// over the threads: leaves are copied, prototype keys (8 rotate-half pairs a
// piece) and values (8 dims a piece) are averaged over the node's tokens by
// SPL threads a piece.
constexpr int WS_THREADS = 256;  // >= 2 * 128 - 1 nodes of the largest slot
constexpr int SPL = 4;           // threads per piece of a prototype

template <class T, int D>
__global__ __launch_bounds__(WS_THREADS) void write_slots_kernel(PackArgs a, const int64_t* off) {
  constexpr int HD = D / 2;
  constexpr int KP = HD / 8;       // key pieces (8 rotate-half pairs each)
  constexpr int VP = D / 8;        // value pieces (8 dims each)
  constexpr int CPN = KP + VP;
  __shared__ int16_t fnode[WS_THREADS], fst[WS_THREADS], fsz[WS_THREADS];
  __shared__ int ioff[WS_THREADS + 1];
  __shared__ int wcnt[WS_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // block -> (unit lh, sequence s, slot k): the grid holds, per unit, a bound
  // on each sequence's slot count (its length over the shortest slot, plus
  // one); blocks past a sequence's slots return at once
  const int64_t b = blockIdx.x, nb = a.sbound[a.S];
  const int64_t lh = b / nb;
  const int r = (int)(b - lh * nb);
  int s = 0;
  while (r >= a.sbound[s + 1]) ++s;
  const int k = r - a.sbound[s];
  if (k >= a.n_slots[s]) return;
  const int32_t* ss = a.slot_start + (int64_t)s * (a.stride + 1);
  const int t0 = ss[k], n = ss[k + 1] - ss[k];
  const int64_t tok0 = a.cu[s] + t0;                 // global token of the slot start
  const int64_t obase = lh * 2 * a.T + 2 * tok0;      // op / node base
  const uint8_t* tk = a.taken + obase;
  if (!tk[0]) return;                                 // Add not taken: no entry
  const int64_t dst0 = off[lh * a.T + tok0];
  // frontier flags: one node per thread (its record, or a pre-order walk of
  // the midpoint tree from the root)
  bool fl = false;
  int st = 0, sz = n;
  if (a.topo) {
    const uint32_t x = tid < 2 * n ? a.topo[obase + tid] : 0xFFFFFFFFu;
    if (x != 0xFFFFFFFFu) {
      st = (int)(x & 255);
      sz = (int)((x >> 8) & 255) + 1;
      const int par = (int)((x >> 16) & 255) - 1;
      fl = tk[par < 0 ? 0 : 1 + par] && !(sz > 1 && tk[1 + tid]);
    }
  } else if (tid < 2 * n - 1) {
    int cur = 0, par = -1;
    while (cur != tid) {
      const int nl = (sz + 1) >> 1;
      par = cur;
      if (tid < cur + 2 * nl) {
        cur += 1;
        sz = nl;
      } else {
        cur += 2 * nl;
        st += nl;
        sz -= nl;
      }
    }
    const int creator = par < 0 ? 0 : 1 + par;
    fl = tk[creator] && !(sz > 1 && tk[1 + tid]);
  }
  const uint64_t bm = __ballot(fl);
  if (lane == 0) wcnt[wave] = __popcll(bm);
  __syncthreads();
  int q = 0, nfr = 0;
#pragma unroll
  for (int w = 0; w < WS_THREADS / 64; ++w) {
    q += w < wave ? wcnt[w] : 0;
    nfr += wcnt[w];
  }
  if (fl) {
    q += __popcll(bm & (lane == 0 ? 0ull : (~0ull >> (64 - lane))));
    fnode[q] = (int16_t)tid;
    fst[q] = (int16_t)st;
    fsz[q] = (int16_t)sz;
  }
  __syncthreads();
  // item ranges: a leaf takes CPN items (one per piece), a prototype SPL * CPN
  // (SPL consecutive threads per piece, each summing every SPL-th token); all
  // ranges are multiples of SPL, so the SPL threads of a piece are
  // neighbouring lanes of one wave
  {
    const int f = tid;
    const int ic = f < nfr ? (fsz[f] == 1 ? CPN : SPL * CPN) : 0;
    int inc = ic;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wcnt[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < WS_THREADS / 64; ++w) {
      base += w < wave ? wcnt[w] : 0;
      tot += wcnt[w];
    }
    if (f < nfr) ioff[f] = base + inc - ic;
    if (tid == 0) ioff[nfr] = tot;
    __syncthreads();
  }
  const int nitems = ioff[nfr];
  const T* Ku = (const T*)a.K + (lh * a.T + a.cu[s]) * D;
  const T* Vu = (const T*)a.V + (lh * a.T + a.cu[s]) * D;
  const float* ru = a.rel + lh * a.T + a.cu[s];
  for (int it = tid; it < nitems; it += WS_THREADS) {
    // entry of this item: the last f with ioff[f] <= it
    int lo = 0, hi = nfr - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ioff[mid] <= it) lo = mid;
      else hi = mid - 1;
    }
    const int f = lo, local = it - ioff[f];
    const int64_t dst = dst0 + f;
    if (dst >= a.capacity) continue;  // every item of the entry skips together
    const int j = fnode[f], a0 = t0 + fst[f], nz = fsz[f];   // sequence positions [a0, a0 + nz)
    T* oK = (T*)a.oK + dst * D;
    T* oV = (T*)a.oV + dst * D;
    if (nz == 1) {  // leaf: bit copy of the token's 16-byte pieces
      const int c = local;
      if (c < KP) {
        *(uint4*)(oK + c * 8) = *(const uint4*)(Ku + (int64_t)a0 * D + c * 8);
        *(uint4*)(oK + HD + c * 8) = *(const uint4*)(Ku + (int64_t)a0 * D + HD + c * 8);
        if constexpr (sizeof(T) == 4) {
          *(uint4*)(oK + c * 8 + 4) = *(const uint4*)(Ku + (int64_t)a0 * D + c * 8 + 4);
          *(uint4*)(oK + HD + c * 8 + 4) = *(const uint4*)(Ku + (int64_t)a0 * D + HD + c * 8 + 4);
        }
      } else {
        const int d0 = (c - KP) * 8;
        *(uint4*)(oV + d0) = *(const uint4*)(Vu + (int64_t)a0 * D + d0);
        if constexpr (sizeof(T) == 4) *(uint4*)(oV + d0 + 4) = *(const uint4*)(Vu + (int64_t)a0 * D + d0 + 4);
      }
      continue;
    }
    const int c = local / SPL, sub = local % SPL;
    if (c < KP) {
      // prototype key: mean of the inverse-rotated keys, re-rotated at the representative position
      const int p0 = c * 8;
      float s0[8], s1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) s0[e] = s1[e] = 0.f;
      for (int i = a0 + sub; i < a0 + nz; i += SPL) {
        float x0[8], x1[8];
        kvcmf::Load8<T>::f(Ku + (int64_t)i * D + p0, x0);
        kvcmf::Load8<T>::f(Ku + (int64_t)i * D + HD + p0, x1);
        const float4 ca = *(const float4*)(a.rc + (int64_t)i * HD + p0), cb = *(const float4*)(a.rc + (int64_t)i * HD + p0 + 4);
        const float4 sa = *(const float4*)(a.rs + (int64_t)i * HD + p0), sb = *(const float4*)(a.rs + (int64_t)i * HD + p0 + 4);
        const float cs[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
        const float sn[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s0[e] += x0[e] * cs[e] + x1[e] * sn[e];   // rotation by -theta
          s1[e] += x1[e] * cs[e] - x0[e] * sn[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // the SPL partial sums, combined in a fixed order
        s0[e] = group_sum<SPL>(s0[e]);
        s1[e] = group_sum<SPL>(s1[e]);
      }
      if (sub != 0) continue;
      const int64_t prep = a0 + (nz - 1) / 2;
      const float4 ca = *(const float4*)(a.rc + prep * HD + p0), cb = *(const float4*)(a.rc + prep * HD + p0 + 4);
      const float4 sa = *(const float4*)(a.rs + prep * HD + p0), sb = *(const float4*)(a.rs + prep * HD + p0 + 4);
      const float cs[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
      const float sn[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
      float k0[8], k1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float m0 = s0[e] / (float)nz, m1 = s1[e] / (float)nz;
        k0[e] = m0 * cs[e] - m1 * sn[e];
        k1[e] = m1 * cs[e] + m0 * sn[e];
      }
      store8<T>(oK + p0, k0);
      store8<T>(oK + HD + p0, k1);
    } else {
      // prototype value: (1 - beta) r_i / rel + beta / n weights (uniform if rel = 0)
      const int d0 = (c - KP) * 8;
      const float rel_n = a.node_rel[obase + j];
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
      for (int i = a0 + sub; i < a0 + nz; i += SPL) {
        const float w = rel_n > 0.f ? (1.f - a.beta) * ru[i] / rel_n + a.beta / (float)nz : 1.f / (float)nz;
        float x[8];
        kvcmf::Load8<T>::f(Vu + (int64_t)i * D + d0, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += w * x[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = group_sum<SPL>(acc[e]);
      if (sub == 0) store8<T>(oV + d0, acc);
    }
  }
  for (int f = tid; f < nfr; f += WS_THREADS) {
    const int64_t dst = dst0 + f;
    if (dst >= a.capacity) continue;
    const int nz = fsz[f];
    a.olnmu[dst] = nz == 1 ? 0.f : logf(a.node_mu[obase + fnode[f]]);
    a.opos[dst] = t0 + fst[f] + (nz - 1) / 2;
  }
}

}  // namespace

namespace kvc {
size_t ws_pack(const kvc_shape* s, const kvc_params* p) {
  int64_t E = (int64_t)s->n_layers * s->n_kv_heads * s->total_tokens;
  int64_t nb = (E + SCAN_BLOCK - 1) / SCAN_BLOCK;
  Carver c(nullptr, 0);
  c.take<int32_t>((size_t)E);
  c.take<int64_t>((size_t)E);
  c.take<int64_t>((size_t)nb + 1);
  c.take<int64_t>(1);
  return c.off + 256;
}
}  // namespace kvc

extern "C" int kvc_pack(const kvc_shape* sh, const kvc_params* p, const void* K, const void* V, const float* rel,
                        const kvc_trees* trees, const uint8_t* op_taken, const int32_t* slot_start,
                        const int32_t* n_slots, const float* rope_cos, const float* rope_sin, kvc_ragged* out,
                        void* ws, size_t ws_bytes, hipStream_t st) {
  int r = kvc::validate_shape(sh);
  if (r) return r;
  if ((r = kvc::validate_params(sh, p))) return r;
  KVC_REQUIRE(sh->n_seq <= 64, KVC_E_SHAPE, "kvc_pack: at most 64 sequences per call");
  KVC_REQUIRE(K && V && op_taken && out, KVC_E_INVAL, "kvc_pack: NULL input");
  KVC_REQUIRE(out->K && out->V && out->lnmu && out->pos && out->seg_off && out->seg_len, KVC_E_INVAL,
              "kvc_pack: NULL output buffer");
  KVC_REQUIRE(out->capacity >= kvc_pack_capacity(sh, p), KVC_E_INVAL, "kvc_pack: capacity below kvc_pack_capacity()");
  KVC_REQUIRE(out->dtype == sh->dtype && out->head_dim == sh->head_dim, KVC_E_DTYPE,
              "kvc_pack: output dtype/head_dim differ from the input");
  if (!p->token_mode)
    KVC_REQUIRE(trees && trees->node_rel && trees->node_mu && rel && slot_start && n_slots && rope_cos && rope_sin,
                KVC_E_INVAL, "kvc_pack: tree mode needs trees, rel, slots and RoPE tables");
  KVC_REQUIRE(ws && ws_bytes >= kvc::ws_pack(sh, p), KVC_E_WORKSPACE, "kvc_pack: workspace too small");
  int64_t E = (int64_t)sh->n_layers * sh->n_kv_heads * sh->total_tokens;
  int64_t nb = (E + SCAN_BLOCK - 1) / SCAN_BLOCK;
  kvc::Carver c(ws, ws_bytes);
  int32_t* cnt = c.take<int32_t>((size_t)E);
  int64_t* off = c.take<int64_t>((size_t)E);
  int64_t* bsum = c.take<int64_t>((size_t)nb + 1);
  int64_t* total = c.take<int64_t>(1);
  PackArgs a{};
  a.K = K;
  a.V = V;
  a.rel = rel;
  a.node_rel = trees ? trees->node_rel : nullptr;
  a.node_mu = trees ? trees->node_mu : nullptr;
  a.taken = op_taken;
  if (!p->token_mode && p->split_mode == 1) {
    KVC_REQUIRE(trees->node_topo && trees->op_cost, KVC_E_INVAL, "kvc_pack: split_mode 1 needs node_topo and op_cost");
    a.topo = trees->node_topo;
    a.op_cost = trees->op_cost;
  }
  a.slot_start = slot_start;
  a.n_slots = n_slots;
  a.rc = rope_cos;
  a.rs = rope_sin;
  a.cu = sh->cu_seqlens_d;
  a.S = sh->n_seq;
  a.Ly = sh->n_layers;
  a.H = sh->n_kv_heads;
  a.stride = p->token_mode ? 1 : kvc_slot_stride(sh, p);
  a.token_mode = p->token_mode;
  a.T = sh->total_tokens;
  a.xoff[0] = 0;
  for (int s = 0; s < sh->n_seq; ++s) {
    const int64_t L = sh->cu_seqlens[s + 1] - sh->cu_seqlens[s];
    kvc::Regions g = kvc::regions_of(L, *p);
    a.pe[s] = g.pe;
    a.c1[s] = g.c1;
    a.xoff[s + 1] = a.xoff[s] + g.pe + (L - g.c1);
  }
  {
    const int64_t smin = std::max<int64_t>(1, p->slot_len > 0 ? p->slot_len : p->slot_min);
    a.sbound[0] = 0;
    for (int s = 0; s < sh->n_seq; ++s) {
      const int64_t L = sh->cu_seqlens[s + 1] - sh->cu_seqlens[s];
      a.sbound[s + 1] = a.sbound[s] + (int32_t)std::min<int64_t>(a.stride, (L + smin - 1) / smin + 1);
    }
  }
  a.beta = p->value_base;
  a.oK = out->K;
  a.oV = out->V;
  a.olnmu = out->lnmu;
  a.opos = out->pos;
  a.capacity = out->capacity;
  if (E == 0) return KVC_OK;
  hipLaunchKernelGGL(count_kernel, dim3(kvc_blocks(E, 256)), dim3(256), 0, st, a, cnt);
  KVC_LAUNCH_CHECK("pack_count");
  hipLaunchKernelGGL(scan_local_kernel, dim3((unsigned)nb), dim3(256), 0, st, cnt, E, off, bsum);
  KVC_LAUNCH_CHECK("pack_scan_local");
  hipLaunchKernelGGL(scan_blocks_kernel, dim3(1), dim3(256), 0, st, bsum, nb, total);
  KVC_LAUNCH_CHECK("pack_scan_blocks");
  hipLaunchKernelGGL(scan_add_kernel, dim3(kvc_blocks(E, 256)), dim3(256), 0, st, off, E, bsum);
  KVC_LAUNCH_CHECK("pack_scan_add");
  int nseg = sh->n_seq * sh->n_layers * sh->n_kv_heads;
  hipLaunchKernelGGL(seg_kernel, dim3(kvc_blocks(nseg, 256)), dim3(256), 0, st, a, off, total, out->seg_off,
                     out->seg_len);
  KVC_LAUNCH_CHECK("pack_seg");
  int d = sh->head_dim;
  const int ppr2 = 2 * d * (sh->dtype == KVC_BF16 ? 2 : 4) / 16;  // 16-byte pieces of a K and a V row
  const int64_t nex = (int64_t)sh->n_layers * sh->n_kv_heads * a.xoff[sh->n_seq] * ppr2;
#define KVC_PACK_T(KERN, GRID)                                                                             \
  if (sh->dtype == KVC_BF16) {                                                                             \
    if (d == 128) hipLaunchKernelGGL((KERN<uint16_t, 128>), GRID, dim3(256), 0, st, a, off);               \
    else hipLaunchKernelGGL((KERN<uint16_t, 64>), GRID, dim3(256), 0, st, a, off);                         \
  } else {                                                                                                 \
    if (d == 128) hipLaunchKernelGGL((KERN<float, 128>), GRID, dim3(256), 0, st, a, off);                  \
    else hipLaunchKernelGGL((KERN<float, 64>), GRID, dim3(256), 0, st, a, off);                            \
  }
  if (nex > 0) {
    KVC_PACK_T(write_exact_kernel, dim3(kvc_blocks(nex, 256)));
    KVC_LAUNCH_CHECK("pack_exact");
  }
  if (p->token_mode) {
    KVC_PACK_T(write_kept_kernel, dim3(kvc_blocks(E * ppr2, 256)));
    KVC_LAUNCH_CHECK("pack_kept");
  } else {
    const dim3 sg((unsigned)((int64_t)sh->n_layers * sh->n_kv_heads * a.sbound[sh->n_seq]));
    if (sh->dtype == KVC_BF16) {
      if (d == 128) hipLaunchKernelGGL((write_slots_kernel<uint16_t, 128>), sg, dim3(WS_THREADS), 0, st, a, off);
      else hipLaunchKernelGGL((write_slots_kernel<uint16_t, 64>), sg, dim3(WS_THREADS), 0, st, a, off);
    } else {
      if (d == 128) hipLaunchKernelGGL((write_slots_kernel<float, 128>), sg, dim3(WS_THREADS), 0, st, a, off);
      else hipLaunchKernelGGL((write_slots_kernel<float, 64>), sg, dim3(WS_THREADS), 0, st, a, off);
    }
    KVC_LAUNCH_CHECK("pack_slots");
  }
#undef KVC_PACK_T
  return KVC_OK;
}
