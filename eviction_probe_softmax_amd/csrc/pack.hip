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
// thread per 16-byte piece of a K or V row, over those tokens only. Grid:
// (pieces of the longest sequence's exact tokens / 256, units, sequences), so
// the sequence and unit of a block are uniform.
template <class T, int D>
__global__ __launch_bounds__(256) void write_exact_kernel(PackArgs a, const int64_t* off) {
  constexpr int PPR = D * (int)sizeof(T) / 16;  // 16-byte pieces per row
  const int s = blockIdx.z;
  const int64_t lh = blockIdx.y;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nx = a.xoff[s + 1] - a.xoff[s];   // exact tokens of sequence s
  if (g >= nx * 2 * PPR) return;
  const int64_t k = g / (2 * PPR);
  const int pc = (int)(g % (2 * PPR));
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

// One wave per (unit, slot); the waves of a workgroup take the same slot of
// consecutive units (units fastest), so the RoPE rows of the slot's
// positions are shared in L2. Each node decides whether it is on the
// frontier (its creator op taken, its own Split not taken; the root's creator
// is the Add), 64 nodes at a time; the frontier nodes in pre-order are the
// slot's output rows in order and cover its tokens in position order. Their
// extents and value-weight terms go to the wave's LDS. Then the wave walks
// the slot's tokens in groups of eight (one round of loads a group), lane p
// holding rotation pair (p, p + d/2) of the key and dims (2p, 2p + 1) of the
// value, and accumulates into the current entry: at an entry's last token a
// leaf writes its token's rows (the loaded values, exact), a prototype the
// mean of its inverse-rotated keys re-rotated at its representative position
// and its weighted value.
constexpr int WS_WAVES = 4;
constexpr int WS_MAXE = 128;   // frontier entries of a slot of at most 128 tokens
constexpr int WS_G = 8;        // tokens a group

template <class T>
__device__ __forceinline__ float ld1(const T* p) {
  if constexpr (sizeof(T) == 2) return bf16_bits_to_f32(*p);
  else return *p;
}
template <class T>
__device__ __forceinline__ float2 ld2(const T* p) {   // two consecutive elements
  if constexpr (sizeof(T) == 2) {
    const uint32_t w = *(const uint32_t*)p;
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
  } else {
    return *(const float2*)p;
  }
}
template <class T>
__device__ __forceinline__ void st1(T* p, float x) {
  if constexpr (sizeof(T) == 2) *p = f32_to_bf16_hw(x);
  else *p = x;
}
template <class T>
__device__ __forceinline__ void st2(T* p, float x, float y) {
  if constexpr (sizeof(T) == 2) *(uint32_t*)p = (uint32_t)f32_to_bf16_hw(x) | ((uint32_t)f32_to_bf16_hw(y) << 16);
  else *(float2*)p = make_float2(x, y);
}

struct WsEntries {
  int16_t sz[WS_MAXE];   // tokens of entry e (its first is the end of the previous one)
  float alpha[WS_MAXE];  // value weight of token i: alpha r_i + gamma
  float gamma[WS_MAXE];
  float lnmu[WS_MAXE];   // log multiplicity (0 for a leaf)
};

template <class T, int D>
__global__ __launch_bounds__(WS_WAVES * 64) void write_slots_kernel(PackArgs a, const int64_t* off) {
  constexpr int HD = D / 2;
  __shared__ WsEntries ent_all[WS_WAVES];
  // the wave index and everything derived from it are wave-uniform: scalar
  // registers and scalar branches
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  WsEntries& ent = ent_all[wv];
  const int64_t nunits = (int64_t)a.Ly * a.H;
  const int64_t w = (int64_t)blockIdx.x * WS_WAVES + wv;
  const int64_t row = w / nunits;              // slot row over the sequences' slot bounds
  const int64_t lh = w - row * nunits;
  if (row >= a.sbound[a.S]) return;
  int s = 0;
  while (row >= a.sbound[s + 1]) ++s;
  const int k = (int)(row - a.sbound[s]);
  if (k >= a.n_slots[s]) return;
  const int32_t* ss = a.slot_start + (int64_t)s * (a.stride + 1);
  const int t0 = ss[k], n = ss[k + 1] - ss[k];
  const int64_t tok0 = a.cu[s] + t0;                 // global token of the slot start
  const int64_t obase = lh * 2 * a.T + 2 * tok0;      // op / node base
  const uint8_t* tk = a.taken + obase;
  if (!tk[0]) return;                                 // Add not taken: no entry
  const int64_t dst0 = off[lh * a.T + tok0];
  // frontier nodes in pre-order -> entries
  const int nn = a.topo ? 2 * n : 2 * n - 1;         // node records of the slot
  int ne = 0;
  for (int base = 0; base < nn; base += 64) {
    const int j = base + lane;
    bool fl = false;
    int sz = n;
    if (j < nn) {
      if (a.topo) {
        const uint32_t x = a.topo[obase + j];
        if (x != 0xFFFFFFFFu) {
          sz = (int)((x >> 8) & 255) + 1;
          const int par = (int)((x >> 16) & 255) - 1;
          fl = tk[par < 0 ? 0 : 1 + par] && !(sz > 1 && tk[1 + j]);
        }
      } else {
        int cur = 0, par = -1;   // pre-order walk of the midpoint tree from the root
        while (cur != j) {
          const int nl = (sz + 1) >> 1;
          par = cur;
          if (j < cur + 2 * nl) {
            cur += 1;
            sz = nl;
          } else {
            cur += 2 * nl;
            sz -= nl;
          }
        }
        fl = tk[par < 0 ? 0 : 1 + par] && !(sz > 1 && tk[1 + j]);
      }
    }
    const uint64_t m = __ballot(fl);
    if (fl) {
      const int e = ne + __popcll(m & ((1ull << lane) - 1ull));
      float al = 0.f, ga = 1.f, lm = 0.f;
      if (sz > 1) {
        const float rel_n = a.node_rel[obase + j];
        al = rel_n > 0.f ? (1.f - a.beta) / rel_n : 0.f;   // weights (1 - beta) r_i / rel + beta / n, or 1 / n
        ga = (rel_n > 0.f ? a.beta : 1.f) / (float)sz;
        lm = logf(a.node_mu[obase + j]);
      }
      ent.sz[e] = (int16_t)sz;
      ent.alpha[e] = al;
      ent.gamma[e] = ga;
      ent.lnmu[e] = lm;
    }
    ne += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();   // the entries are written before any lane reads them
  const T* Ku = (const T*)a.K + (lh * a.T + a.cu[s]) * D;
  const T* Vu = (const T*)a.V + (lh * a.T + a.cu[s]) * D;
  const float* ru = a.rel + lh * a.T + a.cu[s];
  const int p = lane < HD ? lane : HD - 1;   // lanes past the pairs repeat the last one (not stored)
  // the current entry's parameters, read from LDS by every lane, are made
  // scalar so that the flush tests below are uniform branches
  auto uni = [](float x) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x))); };
  int e = 0, ea = t0, esz = __builtin_amdgcn_readfirstlane((int)ent.sz[0]);   // current entry, first position, size
  float al = uni(ent.alpha[0]), ga = uni(ent.gamma[0]);
  float s0 = 0.f, s1 = 0.f, v0 = 0.f, v1 = 0.f, cp = 0.f, sp = 0.f;
  for (int g = t0; g < t0 + n; g += WS_G) {
    float x0[WS_G], x1[WS_G], c[WS_G], sn[WS_G], r[WS_G];
    float2 y[WS_G];
#pragma unroll
    for (int u = 0; u < WS_G; ++u) {   // past the slot: repeats of its last token, unused
      const int i = min(g + u, t0 + n - 1);
      const T* kr = Ku + (int64_t)i * D;
      x0[u] = ld1(kr + p);
      x1[u] = ld1(kr + HD + p);
      c[u] = a.rc[(int64_t)i * HD + p];
      sn[u] = a.rs[(int64_t)i * HD + p];
      y[u] = ld2(Vu + (int64_t)i * D + 2 * p);
      r[u] = ru[i];
    }
#pragma unroll
    for (int u = 0; u < WS_G; ++u) {
      const int i = g + u;
      if (i >= t0 + n) break;
      s0 += x0[u] * c[u] + x1[u] * sn[u];   // rotation by -theta
      s1 += x1[u] * c[u] - x0[u] * sn[u];
      const float wt = fmaf(al, r[u], ga);
      v0 += wt * y[u].x;
      v1 += wt * y[u].y;
      if (i == ea + (esz - 1) / 2) {   // representative position
        cp = c[u];
        sp = sn[u];
      }
      if (i == ea + esz - 1) {   // last token of entry e
        const int64_t d = dst0 + e;
        if (d < a.capacity) {
          T* oK = (T*)a.oK + d * D;
          T* oV = (T*)a.oV + d * D;
          if (lane < HD) {
            if (esz == 1) {   // leaf: the token's rows (values loaded exactly)
              st1(oK + lane, x0[u]);
              st1(oK + HD + lane, x1[u]);
              st2(oV + 2 * lane, y[u].x, y[u].y);
            } else {
              const float m0 = s0 / (float)esz, m1 = s1 / (float)esz;
              st1(oK + lane, m0 * cp - m1 * sp);
              st1(oK + HD + lane, m1 * cp + m0 * sp);
              st2(oV + 2 * lane, v0, v1);
            }
          }
          if (lane == 0) {
            a.olnmu[d] = ent.lnmu[e];   // lane 0 alone: a plain LDS read
            a.opos[d] = ea + (esz - 1) / 2;
          }
        }
        ++e;
        ea = i + 1;
        if (e < ne) {
          esz = __builtin_amdgcn_readfirstlane((int)ent.sz[e]);
          al = uni(ent.alpha[e]);
          ga = uni(ent.gamma[e]);
        }
        s0 = s1 = v0 = v1 = 0.f;
      }
    }
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
  int64_t xmax = 0;   // exact tokens of the longest exact region
  for (int s = 0; s < sh->n_seq; ++s) xmax = std::max<int64_t>(xmax, a.xoff[s + 1] - a.xoff[s]);
  const int64_t nex = xmax * ppr2;
#define KVC_PACK_T(KERN, GRID)                                                                             \
  if (sh->dtype == KVC_BF16) {                                                                             \
    if (d == 128) hipLaunchKernelGGL((KERN<uint16_t, 128>), GRID, dim3(256), 0, st, a, off);               \
    else hipLaunchKernelGGL((KERN<uint16_t, 64>), GRID, dim3(256), 0, st, a, off);                         \
  } else {                                                                                                 \
    if (d == 128) hipLaunchKernelGGL((KERN<float, 128>), GRID, dim3(256), 0, st, a, off);                  \
    else hipLaunchKernelGGL((KERN<float, 64>), GRID, dim3(256), 0, st, a, off);                            \
  }
  if (nex > 0) {
    KVC_PACK_T(write_exact_kernel, dim3(kvc_blocks(nex, 256), (unsigned)(sh->n_layers * sh->n_kv_heads), (unsigned)sh->n_seq));
    KVC_LAUNCH_CHECK("pack_exact");
  }
  if (p->token_mode) {
    KVC_PACK_T(write_kept_kernel, dim3(kvc_blocks(E * ppr2, 256)));
    KVC_LAUNCH_CHECK("pack_kept");
  } else {
    const int64_t nwaves = (int64_t)sh->n_layers * sh->n_kv_heads * a.sbound[sh->n_seq];
    const dim3 sg((unsigned)((nwaves + WS_WAVES - 1) / WS_WAVES));
    if (sh->dtype == KVC_BF16) {
      if (d == 128) hipLaunchKernelGGL((write_slots_kernel<uint16_t, 128>), sg, dim3(WS_WAVES * 64), 0, st, a, off);
      else hipLaunchKernelGGL((write_slots_kernel<uint16_t, 64>), sg, dim3(WS_WAVES * 64), 0, st, a, off);
    } else {
      if (d == 128) hipLaunchKernelGGL((write_slots_kernel<float, 128>), sg, dim3(WS_WAVES * 64), 0, st, a, off);
      else hipLaunchKernelGGL((write_slots_kernel<float, 64>), sg, dim3(WS_WAVES * 64), 0, st, a, off);
    }
    KVC_LAUNCH_CHECK("pack_slots");
  }
#undef KVC_PACK_T
  return KVC_OK;
}
