// Budget spending: token-level top-B, singleton floor, Add/Split auction.
//
// DistillCache paper, Algorithm 1 (keep the top-B tokens by score);
// GraceKV page, 'Exact-information safeguard' (singleton floor: high-value
// leaves first, each paying its untaken tree path, under a hard cap) and
// '04 Top-down budget flow' (one global queue of exposed Add/Split ops; the
// highest affordable utility wins next).
//
// Everything is integer selection on 64-bit keys (score bits above, inverted
// id below, so larger = earlier and ties go to the lower id):
//
// * select(): per sequence, the largest key T whose cumulative weight from the
//   top first exceeds the budget; keys above T are the answer. MSB-first radix
//   over 8 digits; each digit is a grid-wide histogram (integer atomics, so
//   the result is exact and repeatable) plus a one-block choose step.
// * Auction: the best-first greedy pops ops in non-increasing order of
//   beta(op) = min over the op's untaken root path of (u, -id); ties in beta
//   are exactly the ops that share the op b* achieving that minimum, and they
//   are popped together in best-first order below b*. So the taken set is
//   {beta > T} plus the first k best-first pops of the tied group, which one
//   block per sequence finishes inside b*'s slot.
// * Floor: top-F leaves by fp32(s * r); every candidate's marginal path cost
//   assuming all earlier candidates were accepted (first coverer of each op by
//   atomicMax of keys); a weighted select finds the first candidate that does
//   not fit; the few candidates after it are resolved by at most
//   (remaining budget) rounds of "earliest candidate whose current path cost
//   fits".
#include <algorithm>
#include <cmath>

#include "kvc_internal.h"

namespace {

constexpr int MAXS = 64;
constexpr int CH = 2048;  // elements per workgroup in the histogram pass

struct Ranges {
  int S, U;                 // segments (sequences) and units per segment
  int64_t unit_stride;      // element index stride between units
  int64_t start[MAXS];      // first element of segment s within a unit
  int64_t len[MAXS];        // elements of segment s per unit
  int64_t nchunk[MAXS];     // ceil(len / CH)
};

__device__ __forceinline__ bool range_work(const Ranges& r, int64_t b, int& s, int64_t& base, int64_t& n) {
  int64_t acc = 0;
  for (int q = 0; q < r.S; ++q) {
    int64_t nb = r.nchunk[q] * r.U;
    if (b < acc + nb) {
      int64_t x = b - acc;
      int64_t u = x / r.nchunk[q], c = x % r.nchunk[q];
      s = q;
      int64_t off = c * CH;
      base = u * r.unit_stride + r.start[q] + off;
      n = r.len[q] - off < CH ? r.len[q] - off : CH;
      return true;
    }
    acc += nb;
  }
  return false;
}

struct SelState {
  uint64_t prefix;
  int64_t above;    // weight of keys strictly above the prefix range
  int64_t budget;
  int all;          // total weight <= budget: everything is selected
  int pad;
};

// ------------------------------------------------------------------ sources
// Per-sequence host values carried through kernel arguments.
struct PerSeq {
  int64_t v[MAXS];
};

struct TokSrc {       // token mode: rel of every compressible token
  const float* rel;
  const uint8_t* full;  // [S][Ly][H] units kept whole (head-level hybrid), or NULL
  int64_t T;
  int LH;
  __device__ bool get(int64_t i, int s, uint64_t& k, int64_t& w) const {
    if (full && full[(int64_t)s * LH + i / T]) return false;
    k = make_key(rel[i], (uint32_t)i);
    w = 1;
    return true;
  }
};
struct LeafSrc {      // floor candidates: fp32(s_lh * r_i)
  const float* rel;
  const float* sens;  // [S][Ly][H]
  const uint8_t* full;  // units kept whole: not candidates
  int64_t T;
  int LH;
  __device__ bool get(int64_t i, int s, uint64_t& k, int64_t& w) const {
    int lh = (int)(i / T);
    if (full && full[(int64_t)s * LH + lh]) return false;
    float v = __fmul_rn(sens[(int64_t)s * LH + lh], rel[i]);
    k = make_key(v, (uint32_t)i);
    w = 1;
    return true;
  }
};
struct CandSrc {      // floor candidates with their marginal path costs
  const uint64_t* key;
  const int32_t* cost;
  __device__ bool get(int64_t i, int s, uint64_t& k, int64_t& w) const {
    k = key[i];
    w = cost[i];
    return true;
  }
};
struct OpSrc {        // auction: untaken real ops keyed by beta, weighted by the entries they add
  const uint64_t* beta;
  const uint8_t* cost;
  const uint8_t* taken;
  __device__ bool get(int64_t i, int s, uint64_t& k, int64_t& w) const {
    if (cost[i] == 0 || taken[i]) return false;
    k = beta[i];
    w = cost[i];
    return true;
  }
};

template <class Src>
__global__ __launch_bounds__(256) void hist_kernel(Ranges r, Src src, const SelState* st, int pass,
                                                   unsigned long long* hist) {
  __shared__ unsigned long long h[256];
  int s;
  int64_t base, n;
  if (!range_work(r, blockIdx.x, s, base, n)) return;
  SelState S_ = st[s];
  if (S_.all) return;
  h[threadIdx.x] = 0;
  __syncthreads();
  int shift = 56 - 8 * pass;
  uint64_t hmask = pass == 0 ? 0ull : (~0ull << (64 - 8 * pass));
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    uint64_t k;
    int64_t w;
    if (!src.get(base + i, s, k, w)) continue;
    if ((k & hmask) == S_.prefix && w) atomicAdd(&h[(k >> shift) & 255], (unsigned long long)w);
  }
  __syncthreads();
  if (h[threadIdx.x]) atomicAdd(&hist[s * 256 + threadIdx.x], h[threadIdx.x]);
}

// one block per segment: pick the digit where the cumulative weight first
// exceeds the budget, then clear the histogram for the next pass
__global__ __launch_bounds__(256) void choose_kernel(SelState* st, int pass, unsigned long long* hist) {
  __shared__ unsigned long long h[256];
  int s = blockIdx.x;
  h[threadIdx.x] = hist[s * 256 + threadIdx.x];
  hist[s * 256 + threadIdx.x] = 0;
  __syncthreads();
  if (threadIdx.x == 0 && !st[s].all) {
    SelState S_ = st[s];
    int64_t acc = S_.above;
    int shift = 56 - 8 * pass;
    int dsel = -1;
    for (int d = 255; d >= 0; --d) {
      if (acc + (int64_t)h[d] > S_.budget) {
        dsel = d;
        break;
      }
      acc += (int64_t)h[d];
    }
    if (dsel < 0) {
      // only possible on the first pass: the whole segment fits
      st[s].all = 1;
      st[s].above = acc;
    } else {
      st[s].above = acc;
      st[s].prefix = S_.prefix | ((uint64_t)dsel << shift);
    }
  }
}

__global__ void init_state_kernel(SelState* st, int S, const int64_t* budget_dev, Ranges r_host_budget,
                                  int use_dev, const int64_t* subtract) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  SelState x;
  x.prefix = 0;
  x.above = 0;
  int64_t b = use_dev ? budget_dev[s] : r_host_budget.len[s];
  if (subtract) b -= subtract[s];
  x.budget = b < 0 ? 0 : b;
  x.all = 0;
  x.pad = 0;
  st[s] = x;
}

__global__ void zero_u64_kernel(unsigned long long* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}
__global__ void zero_u8_kernel(uint8_t* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ void zero16_kernel(uint4* p, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0u, 0u, 0u, 0u);
}
// nbytes zero bytes at p: 16-byte stores over the aligned part, bytes elsewhere
void zero_bytes(void* p, int64_t nbytes, hipStream_t stream) {
  if (nbytes <= 0) return;
  int64_t head = 0;
  if ((uintptr_t)p & 15) head = std::min<int64_t>(nbytes, 16 - (int64_t)((uintptr_t)p & 15));
  if (head) hipLaunchKernelGGL(zero_u8_kernel, dim3(1), dim3(256), 0, stream, (uint8_t*)p, head);
  const int64_t n16 = (nbytes - head) / 16, tail = nbytes - head - 16 * n16;
  if (n16) hipLaunchKernelGGL(zero16_kernel, dim3(kvc_blocks(n16, 256)), dim3(256), 0, stream, (uint4*)((uint8_t*)p + head), n16);
  if (tail)
    hipLaunchKernelGGL(zero_u8_kernel, dim3(1), dim3(256), 0, stream, (uint8_t*)p + head + 16 * n16, tail);
}

int64_t ranges_blocks(const Ranges& r) {
  int64_t n = 0;
  for (int s = 0; s < r.S; ++s) n += r.nchunk[s] * r.U;
  return n;
}

template <class Src>
int run_passes(const Ranges& r, const Src& src, SelState* st, unsigned long long* hist, hipStream_t stream, int p0,
               int p1) {
  int64_t nb = ranges_blocks(r);
  for (int pass = p0; pass < p1; ++pass) {
    if (nb > 0) {
      hipLaunchKernelGGL(hist_kernel<Src>, dim3((unsigned)nb), dim3(256), 0, stream, r, src, st, pass, hist);
      KVC_LAUNCH_CHECK("select_hist");
    }
    hipLaunchKernelGGL(choose_kernel, dim3(r.S), dim3(256), 0, stream, st, pass, hist);
    KVC_LAUNCH_CHECK("select_choose");
  }
  return KVC_OK;
}
template <class Src>
int run_select(const Ranges& r, const Src& src, SelState* st, unsigned long long* hist, hipStream_t stream) {
  return run_passes(r, src, st, hist, stream, 0, 8);
}

// The elements still in the running after the first two passes (key matching
// the 16-bit prefix, weight > 0), appended per sequence as (key, weight)
// pairs: a block stages its chunk's matches in LDS (one LDS atomic a wave),
// reserves their place with one global atomic, then copies them out. A
// sequence's count may pass cap (then its list is incomplete and the caller
// selects over the full source).
template <class Src>
__global__ __launch_bounds__(256) void compact_kernel(Ranges r, Src src, const SelState* st, uint64_t* ckey,
                                                     int32_t* cw, unsigned int* ccnt, int64_t cap) {
  __shared__ uint64_t sk[CH];
  __shared__ int32_t sw[CH];
  __shared__ unsigned int nloc, gbase;
  int s;
  int64_t base, n;
  if (!range_work(r, blockIdx.x, s, base, n)) return;
  const SelState S_ = st[s];
  if (S_.all) return;
  if (threadIdx.x == 0) nloc = 0;
  __syncthreads();
  const uint64_t hmask = ~0ull << 48;
  const int lane = threadIdx.x & 63;
  for (int64_t i0 = 0; i0 < n; i0 += 256) {   // a uniform trip count: every lane takes part in the ballot
    const int64_t i = i0 + threadIdx.x;
    uint64_t k = 0;
    int64_t w = 0;
    bool m = false;
    if (i < n && src.get(base + i, s, k, w)) m = w > 0 && (k & hmask) == S_.prefix;
    const uint64_t b = __ballot(m);
    if (!b) continue;
    const int lead = __builtin_ctzll(b);
    unsigned int pos = 0;
    if (lane == lead) pos = atomicAdd(&nloc, (unsigned int)__popcll(b));
    pos = __shfl(pos, lead, 64);
    if (m) {
      const unsigned int q = pos + (unsigned int)__popcll(b & ((1ull << lane) - 1ull));
      sk[q] = k;
      sw[q] = (int32_t)w;
    }
  }
  __syncthreads();
  const unsigned int cnt = nloc;
  if (cnt == 0) return;
  if (threadIdx.x == 0) gbase = atomicAdd(&ccnt[s], cnt);
  __syncthreads();
  for (unsigned int q = threadIdx.x; q < cnt; q += 256) {
    const int64_t idx = (int64_t)gbase + q;
    if (idx < cap) {
      ckey[(int64_t)s * cap + idx] = sk[q];
      cw[(int64_t)s * cap + idx] = sw[q];
    }
  }
}

// A select over every element of r for two passes, then over the elements
// still in the running, compacted into per-sequence lists (lkey, lw: cap a
// sequence; lcnt their counts); all eight passes over every element if a
// list overflows. Reads the counts back: waits on stream once.
template <class Src>
int select_compact(const Ranges& r, const Src& src, SelState* st, unsigned long long* hist, hipStream_t stream,
                   uint64_t* lkey, int32_t* lw, unsigned int* lcnt, int64_t cap) {
  int rc;
  if ((rc = run_passes(r, src, st, hist, stream, 0, 2))) return rc;
  zero_bytes(lcnt, (int64_t)MAXS * sizeof(unsigned int), stream);
  const int64_t nb = ranges_blocks(r);
  if (nb > 0) {
    hipLaunchKernelGGL(compact_kernel<Src>, dim3((unsigned)nb), dim3(256), 0, stream, r, src, st, lkey, lw, lcnt, cap);
    KVC_LAUNCH_CHECK("select_compact");
  }
  std::vector<unsigned int> hc(r.S);
  KVC_REQUIRE(hipMemcpyAsync(hc.data(), lcnt, sizeof(unsigned int) * r.S, hipMemcpyDeviceToHost, stream) == hipSuccess &&
                  hipStreamSynchronize(stream) == hipSuccess,
              KVC_E_HIP, "kvc_auction: reading the candidate counts failed");
  bool over = false;
  Ranges cr{};
  cr.S = r.S;
  cr.U = 1;
  cr.unit_stride = 0;
  for (int s = 0; s < r.S; ++s) {
    over |= (int64_t)hc[s] > cap;
    cr.start[s] = (int64_t)s * cap;
    cr.len[s] = hc[s];
    cr.nchunk[s] = (cr.len[s] + CH - 1) / CH;
  }
  if (over) return run_passes(r, src, st, hist, stream, 2, 8);
  CandSrc lsrc{lkey, lw};
  return run_passes(cr, lsrc, st, hist, stream, 2, 8);
}

// ------------------------------------------------------------------ token mode
__global__ __launch_bounds__(256) void mark_tokens_kernel(Ranges r, TokSrc src, const SelState* st, uint8_t* taken,
                                                          int64_t* spent) {
  int s;
  int64_t base, n;
  if (!range_work(r, blockIdx.x, s, base, n)) return;
  SelState S_ = st[s];
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    uint64_t k;
    int64_t w;
    if (!src.get(base + i, s, k, w)) {  // a unit kept whole
      taken[base + i] = 1;
      continue;
    }
    if (S_.all || k > S_.prefix) taken[base + i] = 1;
  }
}
__global__ void token_spent_kernel(const SelState* st, const Ranges r, PerSeq whole, int64_t* spent,
                                   int64_t* spent_floor) {
  int s = threadIdx.x;
  if (s >= r.S) return;
  spent[s] = st[s].above + whole.v[s];
  if (spent_floor) spent_floor[s] = 0;
}

// ------------------------------------------------------------------ head-level hybrid
// One block per sequence: a unit is kept whole when fewer than K units rank
// above it by (head sensitivity desc, unit index asc); NaN ranks last.
__global__ __launch_bounds__(256) void hybrid_units_kernel(const float* sens, int LH, PerSeq K, uint8_t* full) {
  __shared__ float sv[4096];
  const int s = blockIdx.x;
  for (int u = threadIdx.x; u < LH; u += 256) {
    float v = sens[(int64_t)s * LH + u];
    sv[u] = v != v ? -INFINITY : v;
  }
  __syncthreads();
  for (int u = threadIdx.x; u < LH; u += 256) {
    const float x = sv[u];
    int64_t rank = 0;
    for (int v = 0; v < LH; ++v) {
      const float y = sv[v];
      rank += (y > x) || (y == x && v < u);
    }
    full[(int64_t)s * LH + u] = rank < K.v[s] ? 1 : 0;
  }
}
// every real op of a unit kept whole is taken before the floor and the auction
__global__ __launch_bounds__(256) void hybrid_take_kernel(Ranges r, const uint8_t* cost, const uint8_t* full, int LH,
                                                          uint8_t* taken) {
  int s;
  int64_t base, n;
  if (!range_work(r, blockIdx.x, s, base, n)) return;
  if (!full[(int64_t)s * LH + base / r.unit_stride]) return;
  for (int64_t i = threadIdx.x; i < n; i += 256)
    if (cost[base + i]) taken[base + i] = 1;
}
__global__ void add_whole_kernel(int S, PerSeq whole, int64_t* spent) {
  int s = threadIdx.x;
  if (s < S) spent[s] += whole.v[s];
}

// ------------------------------------------------------------------ slot / tree helpers
struct TreeArgs {
  const int64_t* cu;
  const int32_t* slot_start;  // [S][stride+1]
  const int32_t* n_slots;
  const uint32_t* topo;       // node records [Ly][H][2T] (split_mode 1), or NULL: midpoint trees
  int stride;
  int S, Ly, H;
  int64_t T;
};
constexpr uint32_t TOPO_NONE = 0xFFFFFFFFu;
constexpr int MAX_PATH = 16;  // internal nodes on a root-to-leaf path: 7 for midpoint trees of 128
                              // tokens, 14 for the explicit trees (children <= n - ceil(n/4) tokens)
__device__ __forceinline__ int topo_len(uint32_t x) { return (int)((x >> 8) & 255) + 1; }
__device__ __forceinline__ int topo_parent(uint32_t x) { return (int)((x >> 16) & 255) - 1; }

// slot of sequence position t (binary search over the slot starts)
__device__ __forceinline__ int slot_of(const TreeArgs& a, int s, int t, int& t0, int& n) {
  const int32_t* ss = a.slot_start + (int64_t)s * (a.stride + 1);
  int lo = 0, hi = a.n_slots[s] - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (ss[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  t0 = ss[lo];
  n = ss[lo + 1] - ss[lo];
  return lo;
}

// Root-to-leaf path of token t in a slot [t0, t0+n): writes internal node
// pre-order indices, returns their count. rec: the slot's node records, or
// NULL for the midpoint tree.
__device__ __forceinline__ int leaf_path(const uint32_t* rec, int t0, int n, int t, int* nodes) {
  int c = 0;
  if (rec) {
    const int tr = t - t0;
    int j = 0;
    uint32_t x = rec[0];
    while (topo_len(x) > 1 && c < MAX_PATH) {
      nodes[c++] = j;
      int ch = j + 1;
      uint32_t y = rec[ch];
      while ((int)(y & 255) + topo_len(y) <= tr && (y >> 24) != 0) {   // the child holding t
        ch = (int)(y >> 24);
        y = rec[ch];
      }
      j = ch;
      x = y;
    }
    return c;
  }
  int j = 0, st = t0, sz = n;
  while (sz > 1) {
    nodes[c++] = j;
    int nl = (sz + 1) >> 1;
    if (t < st + nl) {
      j += 1;
      sz = nl;
    } else {
      j += 2 * nl;
      st += nl;
      sz -= nl;
    }
  }
  return c;
}

// ------------------------------------------------------------------ floor
struct FloorArgs {
  TreeArgs ta;
  const float* rel;
  const float* sens;
  const uint8_t* op_cost;
  uint8_t* taken;
  uint64_t* cover;     // [Ly][H][2T] first coverer key per op
  uint64_t* ckey;      // [S][Fmax]
  int32_t* cid;        // [S][Fmax] leaf flat index
  int32_t* ccost;      // [S][Fmax]
  int32_t* ccount;     // [S]
  int2* cslot;         // [S][Fmax] the candidate's slot (start, length), set by floor_cover
  int64_t Fmax;
};

__global__ __launch_bounds__(256) void floor_collect_kernel(Ranges r, LeafSrc src, const SelState* st, FloorArgs f) {
  int s;
  int64_t base, n;
  if (!range_work(r, blockIdx.x, s, base, n)) return;
  SelState S_ = st[s];
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    uint64_t k;
    int64_t w;
    if (!src.get(base + i, s, k, w)) continue;
    if (S_.all || k > S_.prefix) {
      int slot = atomicAdd(&f.ccount[s], 1);
      if (slot < f.Fmax) {
        f.ckey[(int64_t)s * f.Fmax + slot] = k;
        f.cid[(int64_t)s * f.Fmax + slot] = (int32_t)(base + i);
      }
    }
  }
}

// root path of a candidate leaf whose slot [t0, t0 + n) is known
__device__ __forceinline__ void cand_path_at(const FloorArgs& f, int s, int64_t leaf, int t0, int n, int64_t* ops,
                                             int& nops) {
  const TreeArgs& a = f.ta;
  int64_t lh = leaf / a.T;
  int t = (int)(leaf % a.T - a.cu[s]);
  int nodes[MAX_PATH];
  int64_t base = lh * 2 * a.T + 2 * (a.cu[s] + t0);
  int c = leaf_path(a.topo ? a.topo + base : nullptr, t0, n, t, nodes);
  ops[0] = base;
  for (int q = 0; q < c; ++q) ops[1 + q] = base + 1 + nodes[q];
  nops = 1 + c;
}
__device__ __forceinline__ void cand_path(const FloorArgs& f, int s, int64_t leaf, int64_t* ops, int& nops) {
  int t0, n;
  slot_of(f.ta, s, (int)(leaf % f.ta.T - f.ta.cu[s]), t0, n);
  cand_path_at(f, s, leaf, t0, n, ops, nops);
}

// one thread per candidate slot of every sequence
__global__ void floor_cover_kernel(FloorArgs f, int S) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int s = (int)(i / f.Fmax);
  int64_t k = i % f.Fmax;
  if (s >= S || k >= min((int64_t)f.ccount[s], f.Fmax)) return;
  int64_t ops[MAX_PATH + 1];
  int nops;
  const int64_t leaf = f.cid[i];
  int t0, n;
  slot_of(f.ta, s, (int)(leaf % f.ta.T - f.ta.cu[s]), t0, n);
  f.cslot[i] = make_int2(t0, n);   // kept for the tail's rounds
  cand_path_at(f, s, leaf, t0, n, ops, nops);
  uint64_t key = f.ckey[i];
  for (int q = 0; q < nops; ++q) atomicMax((unsigned long long*)&f.cover[ops[q]], (unsigned long long)key);
}
__global__ void floor_cost_kernel(FloorArgs f, int S) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int s = (int)(i / f.Fmax);
  int64_t k = i % f.Fmax;
  if (s >= S || k >= min((int64_t)f.ccount[s], f.Fmax)) return;
  int64_t ops[MAX_PATH + 1];
  int nops;
  cand_path(f, s, f.cid[i], ops, nops);
  uint64_t key = f.ckey[i];
  int c = 0;
  for (int q = 0; q < nops; ++q)
    if (f.cover[ops[q]] == key) c += f.op_cost[ops[q]];
  f.ccost[i] = c;
}
// accept the prefix (keys above the first candidate that does not fit)
__global__ void floor_accept_kernel(FloorArgs f, int S, const SelState* st) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int s = (int)(i / f.Fmax);
  int64_t k = i % f.Fmax;
  if (s >= S || k >= min((int64_t)f.ccount[s], f.Fmax)) return;
  SelState S_ = st[s];
  if (!(S_.all || f.ckey[i] > S_.prefix)) return;
  int64_t ops[MAX_PATH + 1];
  int nops;
  cand_path(f, s, f.cid[i], ops, nops);
  for (int q = 0; q < nops; ++q) f.taken[ops[q]] = 1;
}
// Candidates after the first one that did not fit, in order; one block per
// sequence (FT_THREADS threads: every round scans all candidates). Each round
// accepts the earliest remaining candidate whose current
// path cost is between 1 and the remaining floor budget (candidates before it
// cost more than what is left, or nothing); at most `remaining` rounds.
constexpr int FT_THREADS = 1024;
__global__ __launch_bounds__(FT_THREADS) void floor_tail_kernel(FloorArgs f, const SelState* st, Ranges fb,
                                                         int64_t* spent_floor) {
  __shared__ unsigned long long best;
  __shared__ unsigned long long pre;
  __shared__ int64_t rem_s;
  int s = blockIdx.x;
  SelState S_ = st[s];
  int64_t F = fb.len[s];
  int64_t cnt = min((int64_t)f.ccount[s], f.Fmax);
  if (threadIdx.x == 0) pre = 0;
  __syncthreads();
  unsigned long long loc = 0;
  for (int64_t k = threadIdx.x; k < cnt; k += FT_THREADS) {
    int64_t i = (int64_t)s * f.Fmax + k;
    if (S_.all || f.ckey[i] > S_.prefix) loc += (unsigned long long)f.ccost[i];
  }
  if (loc) atomicAdd(&pre, loc);
  __syncthreads();
  if (threadIdx.x == 0) rem_s = F - (int64_t)pre;
  __syncthreads();
  uint64_t pos = S_.prefix;  // the first candidate that did not fit; only later ones remain
  for (int round = 0; round < 64 && !S_.all; ++round) {
    int64_t rem = rem_s;
    if (rem <= 0) break;
    if (threadIdx.x == 0) best = 0;
    __syncthreads();
    for (int64_t k = threadIdx.x; k < cnt; k += FT_THREADS) {
      int64_t i = (int64_t)s * f.Fmax + k;
      uint64_t key = f.ckey[i];
      if (key >= pos) continue;
      int64_t ops[MAX_PATH + 1];
      int nops;
      const int2 sl = f.cslot[i];
      cand_path_at(f, s, f.cid[i], sl.x, sl.y, ops, nops);
      int c = 0;
      for (int q = 0; q < nops; ++q)
        if (!f.taken[ops[q]]) c += f.op_cost[ops[q]];
      if (c >= 1 && c <= rem) atomicMax(&best, (unsigned long long)key);
    }
    __syncthreads();
    uint64_t win = best;
    __syncthreads();
    if (win == 0) break;
    for (int64_t k = threadIdx.x; k < cnt; k += FT_THREADS) {
      int64_t i = (int64_t)s * f.Fmax + k;
      if (f.ckey[i] != win) continue;
      int64_t ops[MAX_PATH + 1];
      int nops;
      const int2 sl = f.cslot[i];
      cand_path_at(f, s, f.cid[i], sl.x, sl.y, ops, nops);
      int c = 0;
      for (int q = 0; q < nops; ++q)
        if (!f.taken[ops[q]]) c += f.op_cost[ops[q]];
      for (int q = 0; q < nops; ++q) f.taken[ops[q]] = 1;
      rem_s = rem - c;
    }
    pos = win;
    __syncthreads();
  }
  __syncthreads();
  if (threadIdx.x == 0) spent_floor[s] = F - rem_s;
}

// ------------------------------------------------------------------ auction
struct AucArgs {
  TreeArgs ta;
  const float* util;
  const uint8_t* cost;
  uint8_t* taken;
  uint64_t* beta;
  int64_t c0[MAXS], c1[MAXS];  // compressible region per sequence
};

__device__ __forceinline__ uint64_t op_key(const AucArgs& a, int64_t op) {
  float u = a.util[op];
  return make_key(u, (uint32_t)op);
}

// beta of every op = min key over the untaken part of its root path
__global__ void beta_kernel(AucArgs a, Ranges r) {
  int s;
  int64_t base, n;
  if (!range_work(r, blockIdx.x, s, base, n)) return;
  const TreeArgs& ta = a.ta;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    int64_t op = base + i;
    uint64_t b = 0;
    if (a.cost[op] != 0 && !a.taken[op]) {
      int64_t lh = op / (2 * ta.T);
      int64_t x = op % (2 * ta.T);
      int t = (int)(x / 2 - ta.cu[s]);
      int t0, nn;
      slot_of(ta, s, t, t0, nn);
      int64_t sbase = lh * 2 * ta.T + 2 * (ta.cu[s] + t0);
      int jop = (int)(op - sbase);  // 0 = Add, 1+j = Split(node j)
      b = ~0ull;
      // Add
      if (!a.taken[sbase]) b = op_key(a, sbase);
      if (jop > 0 && ta.topo) {     // explicit trees: up the parent chain
        const uint32_t* rec = ta.topo + sbase;
        for (int j = jop - 1; j >= 0; j = topo_parent(rec[j])) {
          const int64_t o = sbase + 1 + j;
          if (!a.taken[o]) {
            uint64_t k = op_key(a, o);
            if (k < b) b = k;
          }
        }
      } else if (jop > 0) {
        int target = jop - 1;
        int j = 0, sz = nn;
        while (true) {
          int64_t o = sbase + 1 + j;
          if (!a.taken[o]) {
            uint64_t k = op_key(a, o);
            if (k < b) b = k;
          }
          if (j == target) break;
          int nl = (sz + 1) >> 1;
          if (target < j + 2 * nl) {
            j += 1;
            sz = nl;
          } else {
            j += 2 * nl;
            sz -= nl;
          }
        }
      }
    }
    a.beta[op] = b;
  }
}

// The same for midpoint trees, one wave per (unit, slot): every node's path
// minimum B(j) = min(B(parent), key of Split j if untaken), B above the root
// the Add's key if untaken, computed depth by depth in LDS from one load of the
// slot's taken flags and utilities. The waves of a workgroup take the same
// slot of consecutive units. beta of an untaken op that adds entries: its
// node's B (the Add: its own key); of any other op: 0.
constexpr int BS_WAVES = 4;
struct SlotRows {
  int32_t sbound[MAXS + 1];   // prefix over sequences of a bound on their slot counts
};
__global__ __launch_bounds__(BS_WAVES * 64) void beta_slot_kernel(AucArgs a, SlotRows sr) {
  __shared__ uint64_t Bs[BS_WAVES][256];
  const TreeArgs& ta = a.ta;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nunits = (int64_t)ta.Ly * ta.H;
  const int64_t w = (int64_t)blockIdx.x * BS_WAVES + wv;
  const int64_t row = w / nunits;
  const int64_t lh = w - row * nunits;
  if (row >= sr.sbound[ta.S]) return;
  int s = 0;
  while (row >= sr.sbound[s + 1]) ++s;
  const int k = (int)(row - sr.sbound[s]);
  if (k >= ta.n_slots[s]) return;
  const int32_t* ss = ta.slot_start + (int64_t)s * (ta.stride + 1);
  const int n = ss[k + 1] - ss[k];
  const int64_t sbase = lh * 2 * ta.T + 2 * (ta.cu[s] + ss[k]);
  const bool add_taken = a.taken[sbase] != 0;
  const uint64_t kadd = add_taken ? ~0ull : op_key(a, sbase);
  const int nn = 2 * n - 1;   // nodes of the midpoint tree
  int par[4], dep[4];
  uint64_t key[4];
  int maxd = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = lane + 64 * q;
    par[q] = -1;
    dep[q] = -1;
    key[q] = ~0ull;
    if (j < nn) {
      int cur = 0, sz = n, d = 0;
      while (cur != j) {   // pre-order walk from the root
        const int nl = (sz + 1) >> 1;
        par[q] = cur;
        ++d;
        if (j < cur + 2 * nl) {
          cur += 1;
          sz = nl;
        } else {
          cur += 2 * nl;
          sz -= nl;
        }
      }
      dep[q] = d;
      maxd = d > maxd ? d : maxd;
      const int64_t o = sbase + 1 + j;
      if (!a.taken[o]) key[q] = op_key(a, o);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const int x = __shfl_xor(maxd, o, 64);
    maxd = x > maxd ? x : maxd;
  }
  uint64_t* B = Bs[wv];
  for (int d = 0; d <= maxd; ++d) {   // parents before children: a wave's LDS accesses stay in order
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (dep[q] == d) {
        const uint64_t pb = par[q] < 0 ? kadd : B[par[q]];
        B[lane + 64 * q] = pb < key[q] ? pb : key[q];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (lane == 0) a.beta[sbase] = (a.cost[sbase] != 0 && !add_taken) ? kadd : 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = lane + 64 * q;
    if (j < nn) {
      const int64_t o = sbase + 1 + j;
      a.beta[o] = (a.cost[o] != 0 && !a.taken[o]) ? B[j] : 0;
    }
  }
}

__global__ void auction_mark_kernel(AucArgs a, Ranges r, const SelState* st) {
  int s;
  int64_t base, n;
  if (!range_work(r, blockIdx.x, s, base, n)) return;
  SelState S_ = st[s];
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    int64_t op = base + i;
    if (a.cost[op] == 0 || a.taken[op]) continue;
    if (S_.all || a.beta[op] > S_.prefix) a.taken[op] = 2;  // 2 = taken by the auction in this call
  }
}

// Finish the tied group below b* with a best-first walk; one block per
// sequence (thread 0 works: the slot holds at most 2*128 ops). An op that
// costs more than what is left is discarded with its subtree (only a
// three-way split, cost 2, can meet 1 entry left). kleft[s] receives what is
// left after the walk (0 or 1).
__global__ __launch_bounds__(64) void auction_fixup_kernel(AucArgs a, const SelState* st, const int64_t* spent_floor,
                                                           int64_t* spent, int64_t* kleft) {
  __shared__ int sz_[256], ns_[256];
  __shared__ uint8_t exposed[257];
  int s = blockIdx.x;
  if (threadIdx.x != 0) return;
  kleft[s] = 0;
  SelState S_ = st[s];
  if (S_.all) {
    spent[s] = spent_floor[s] + S_.above;
    return;
  }
  int64_t k = S_.budget - S_.above;
  spent[s] = spent_floor[s] + S_.budget;
  if (k <= 0) return;
  const uint64_t T = S_.prefix;
  const int64_t bop = (int64_t)key_id(T);
  const TreeArgs& ta = a.ta;
  int64_t lh = bop / (2 * ta.T);
  int64_t x = bop % (2 * ta.T);
  int t = (int)(x / 2 - ta.cu[s]);
  int t0, nn;
  slot_of(ta, s, t, t0, nn);
  const int64_t sbase = lh * 2 * ta.T + 2 * (ta.cu[s] + t0);
  // node table of the slot: sizes and next siblings (children of j: j + 1,
  // then the sibling chain)
  int m = 0;
  if (ta.topo) {
    const uint32_t* rec = ta.topo + sbase;
    for (; m < 2 * nn && rec[m] != TOPO_NONE; ++m) {
      sz_[m] = topo_len(rec[m]);
      ns_[m] = (int)(rec[m] >> 24);
    }
  } else {   // midpoint tree: pop a frame, number it, push right then left
    struct Fr { int sz, sib_of; };
    Fr fr[20];
    int ftop = 0;
    fr[ftop++] = {nn, -1};
    while (ftop > 0) {
      Fr q = fr[--ftop];
      int j = m++;
      sz_[j] = q.sz;
      ns_[j] = 0;
      if (q.sib_of >= 0) ns_[q.sib_of] = j;   // a right child is its left sibling's next
      if (q.sz > 1) {
        int nl = (q.sz + 1) >> 1;
        fr[ftop++] = {q.sz - nl, j + 1};
        fr[ftop++] = {nl, -1};
      }
    }
  }
  // exposed[0] = Add, exposed[1+j] = Split(node j)
  for (int q = 0; q <= m; ++q) exposed[q] = 0;
  exposed[bop - sbase] = 1;
  while (k > 0) {
    int best = -1;
    uint64_t bk = 0;
    for (int q = 0; q <= m; ++q) {
      if (!exposed[q]) continue;
      uint64_t kk = op_key(a, sbase + q);
      if (best < 0 || kk > bk) {
        best = q;
        bk = kk;
      }
    }
    if (best < 0) break;
    exposed[best] = 0;
    const int c = a.cost[sbase + best];
    if (c > k) continue;
    a.taken[sbase + best] = 2;
    k -= c;
    // the ops of the nodes it creates: the root's split for Add, the
    // children's splits for a split
    int first = best == 0 ? 0 : best;                 // node index of the first created node
    for (int ch = first; ; ) {
      if (sz_[ch] > 1) {
        int64_t o = sbase + 1 + ch;
        if (a.cost[o] != 0 && a.taken[o] == 0 && a.beta[o] == T) exposed[1 + ch] = 1;
      }
      if (best == 0) break;
      ch = ns_[ch];
      if (ch == 0) break;
    }
  }
  spent[s] = spent_floor[s] + S_.budget - k;
  kleft[s] = k;
}

// After the walk, budget may be left that the tied group could not use (a
// three-way split met 1 entry left): the greedy goes on with the best-keyed
// op that is exposed (its creator taken) and fits. One pass finds it per
// sequence (keys are unique), a second takes it; with at most 1 entry left
// and costs of 1 or 2, one such op ends the auction.
__global__ void auction_extend_kernel(AucArgs a, Ranges r, const int64_t* kleft, unsigned long long* best) {
  int s;
  int64_t base, n;
  if (!range_work(r, blockIdx.x, s, base, n)) return;
  const int64_t k = kleft[s];
  if (k <= 0) return;
  const TreeArgs& ta = a.ta;
  unsigned long long loc = 0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t op = base + i;
    const int c = a.cost[op];
    if (c == 0 || c > k || a.taken[op]) continue;
    const int64_t lh = op / (2 * ta.T);
    const int tt = (int)(op % (2 * ta.T) / 2 - ta.cu[s]);
    int t0, nn;
    slot_of(ta, s, tt, t0, nn);
    const int64_t sbase = lh * 2 * ta.T + 2 * (ta.cu[s] + t0);
    const int jop = (int)(op - sbase);
    int64_t creator = -1;                 // Add has none
    if (jop == 1) creator = sbase;
    else if (jop > 1) creator = sbase + 1 + topo_parent(ta.topo[sbase + jop - 1]);
    if (creator >= 0 && !a.taken[creator]) continue;
    const unsigned long long kk = op_key(a, op);
    if (kk > loc) loc = kk;
  }
  if (loc) atomicMax(&best[s], loc);
}

__global__ void auction_extend_take_kernel(AucArgs a, int S, const unsigned long long* best, int64_t* kleft,
                                           int64_t* spent) {
  const int s = threadIdx.x;
  if (s >= S || kleft[s] <= 0 || best[s] == 0) return;
  const int64_t op = (int64_t)key_id(best[s]);
  const int c = a.cost[op];
  a.taken[op] = 2;
  kleft[s] -= c;
  spent[s] += c;
}

// ------------------------------------------------------------------ per-segment top-B
struct SegSrc {       // step-wise eviction: policy score per cached token, ties to the earlier position
  const float* score;
  const int32_t* pos;  // or NULL: the element index orders ties
  __device__ bool get(int64_t i, int s, uint64_t& k, int64_t& w) const {
    k = make_key(score[i], pos ? (uint32_t)pos[i] : (uint32_t)i);
    w = 1;
    return true;
  }
};
__global__ __launch_bounds__(256) void mark_keep_kernel(Ranges r, SegSrc src, const SelState* st, uint8_t* keep) {
  int s;
  int64_t base, n;
  if (!range_work(r, blockIdx.x, s, base, n)) return;
  SelState S_ = st[s];
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    uint64_t k;
    int64_t w;
    src.get(base + i, s, k, w);
    keep[base + i] = (S_.all || k > S_.prefix) ? 1 : 0;
  }
}

__global__ void taken_normalize_kernel(uint8_t* taken, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n && taken[i]) taken[i] = 1;
}

// ------------------------------------------------------------------ host helpers
void fill_ranges(Ranges& r, const kvc_shape* sh, const kvc_params* p, int per_token, bool ops) {
  r.S = sh->n_seq;
  r.U = sh->n_layers * sh->n_kv_heads;
  int mul = ops ? 2 : 1;
  r.unit_stride = mul * sh->total_tokens;
  for (int s = 0; s < sh->n_seq; ++s) {
    int64_t L = sh->cu_seqlens[s + 1] - sh->cu_seqlens[s];
    kvc::Regions g = kvc::regions_of(L, *p);
    r.start[s] = mul * (sh->cu_seqlens[s] + g.c0);
    r.len[s] = mul * (g.c1 - g.c0);
    r.nchunk[s] = (r.len[s] + CH - 1) / CH;
  }
  (void)per_token;
}

}  // namespace

namespace kvc {
// capacity of a sequence's candidate list in the auction's select: 2^20, or
// fewer where no sequence has that many ops
int64_t auction_cand_cap(const kvc_shape* s, const kvc_params* p) {
  Ranges ops{};
  fill_ranges(ops, s, p, 0, true);
  int64_t mx = 1;
  for (int q = 0; q < s->n_seq; ++q) mx = std::max<int64_t>(mx, ops.len[q] * ops.U);
  return std::min<int64_t>(mx, (int64_t)1 << 20);
}
size_t ws_auction(const kvc_shape* s, const kvc_params* p) {
  int64_t E = (int64_t)s->n_layers * s->n_kv_heads * s->total_tokens;
  std::vector<int64_t> B(s->n_seq), A(s->n_seq), F(s->n_seq);
  kvc_budgets(s, p, B.data(), A.data(), F.data());
  int64_t Fmax = 1;
  for (int i = 0; i < s->n_seq; ++i) Fmax = F[i] > Fmax ? F[i] : Fmax;
  Carver c(nullptr, 0);
  c.take<SelState>(MAXS);
  c.take<unsigned long long>((size_t)MAXS * 256);
  c.take<int64_t>(MAXS * 2);
  c.take<uint8_t>((size_t)s->n_seq * s->n_layers * s->n_kv_heads);  // units kept whole
  if (!p->token_mode) {
    c.take<uint64_t>((size_t)E * 2);       // cover / beta
    c.take<uint64_t>((size_t)s->n_seq * Fmax);
    c.take<int32_t>((size_t)s->n_seq * Fmax);
    c.take<int32_t>((size_t)s->n_seq * Fmax);
    c.take<int32_t>(MAXS);
    c.take<int64_t>(MAXS);               // budget left after the tied group's walk
    c.take<unsigned long long>(MAXS);    // best op that still fits
    const int64_t cap = auction_cand_cap(s, p);
    c.take<uint64_t>((size_t)s->n_seq * cap);  // the auction's candidates after two passes: keys
    c.take<int32_t>((size_t)s->n_seq * cap);   // and weights
    c.take<unsigned int>(MAXS);                // their counts
    c.take<int2>((size_t)s->n_seq * Fmax);     // floor candidates' slots
  }
  return c.off + 256;
}
}  // namespace kvc

extern "C" int kvc_auction(const kvc_shape* sh, const kvc_params* p, const kvc_trees* trees, const float* rel,
                           const float* head_sens, const int32_t* slot_start, const int32_t* n_slots,
                           uint8_t* op_taken, int64_t* spent, int64_t* spent_floor, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  int r = kvc::validate_shape(sh);
  if (r) return r;
  if ((r = kvc::validate_params(sh, p))) return r;
  KVC_REQUIRE(sh->n_seq <= MAXS, KVC_E_SHAPE, "kvc_auction: at most 64 sequences per call");
  KVC_REQUIRE(op_taken && spent, KVC_E_INVAL, "kvc_auction: NULL output");
  KVC_REQUIRE(ws && ws_bytes >= kvc::ws_auction(sh, p), KVC_E_WORKSPACE, "kvc_auction: workspace too small");
  std::vector<int64_t> B(sh->n_seq), A(sh->n_seq), F(sh->n_seq);
  if ((r = kvc_budgets(sh, p, B.data(), A.data(), F.data()))) return r;
  int64_t E = (int64_t)sh->n_layers * sh->n_kv_heads * sh->total_tokens;
  const int LH = sh->n_layers * sh->n_kv_heads;
  kvc::Carver c(ws, ws_bytes);
  SelState* st = c.take<SelState>(MAXS);
  unsigned long long* hist = c.take<unsigned long long>((size_t)MAXS * 256);
  int64_t* dev_i64 = c.take<int64_t>(MAXS * 2);
  uint8_t* full_mask = c.take<uint8_t>((size_t)sh->n_seq * LH);
  int64_t* sfloor = spent_floor ? spent_floor : dev_i64;
  Ranges budget_r{};  // carries host budgets through kernel arguments
  budget_r.S = sh->n_seq;
  hipLaunchKernelGGL(zero_u64_kernel, dim3(kvc_blocks(MAXS * 256, 256)), dim3(256), 0, stream, hist,
                     (int64_t)MAXS * 256);
  KVC_LAUNCH_CHECK("zero_hist");
  // head-level hybrid: units kept whole and the entries they take
  PerSeq whole{}, nfull{};
  bool hybrid = false;
  for (int s = 0; s < sh->n_seq; ++s) {
    kvc::Regions g = kvc::regions_of(sh->cu_seqlens[s + 1] - sh->cu_seqlens[s], *p);
    nfull.v[s] = kvc::hybrid_units_of(A[s], g.c1 - g.c0, LH, *p);
    whole.v[s] = nfull.v[s] * (g.c1 - g.c0);
    hybrid |= nfull.v[s] > 0;
  }
  const uint8_t* full = nullptr;
  if (hybrid) {
    KVC_REQUIRE(head_sens, KVC_E_INVAL, "kvc_auction: the head-level hybrid needs head_sens");
    hipLaunchKernelGGL(hybrid_units_kernel, dim3(sh->n_seq), dim3(256), 0, stream, head_sens, LH, nfull, full_mask);
    KVC_LAUNCH_CHECK("hybrid_units");
    full = full_mask;
  }

  if (p->token_mode) {
    KVC_REQUIRE(rel, KVC_E_INVAL, "kvc_auction: token mode needs rel");
    zero_bytes(op_taken, E, stream);
    KVC_LAUNCH_CHECK("zero_taken");
    Ranges rg{};
    fill_ranges(rg, sh, p, 1, false);
    for (int s = 0; s < sh->n_seq; ++s) budget_r.len[s] = A[s] - whole.v[s];
    hipLaunchKernelGGL(init_state_kernel, dim3(1), dim3(MAXS), 0, stream, st, sh->n_seq, (const int64_t*)nullptr,
                       budget_r, 0, (const int64_t*)nullptr);
    KVC_LAUNCH_CHECK("init_state");
    TokSrc src{rel, full, sh->total_tokens, LH};
    if ((r = run_select(rg, src, st, hist, stream))) return r;
    int64_t nb = ranges_blocks(rg);
    if (nb > 0) {
      hipLaunchKernelGGL(mark_tokens_kernel, dim3((unsigned)nb), dim3(256), 0, stream, rg, src, st, op_taken, spent);
      KVC_LAUNCH_CHECK("mark_tokens");
    }
    hipLaunchKernelGGL(token_spent_kernel, dim3(1), dim3(MAXS), 0, stream, st, rg, whole, spent, spent_floor);
    KVC_LAUNCH_CHECK("token_spent");
    return KVC_OK;
  }

  KVC_REQUIRE(trees && trees->op_util && trees->op_cost && rel && head_sens && slot_start && n_slots, KVC_E_INVAL,
              "kvc_auction: tree mode needs trees, rel, head_sens and slots");
  int64_t Fmax = 1;
  for (int s = 0; s < sh->n_seq; ++s) Fmax = F[s] > Fmax ? F[s] : Fmax;
  uint64_t* cover = c.take<uint64_t>((size_t)E * 2);  // reused as beta by the auction
  uint64_t* ckey = c.take<uint64_t>((size_t)sh->n_seq * Fmax);
  int32_t* cid = c.take<int32_t>((size_t)sh->n_seq * Fmax);
  int32_t* ccost = c.take<int32_t>((size_t)sh->n_seq * Fmax);
  int32_t* ccount = c.take<int32_t>(MAXS);
  int64_t* kleft = c.take<int64_t>(MAXS);
  unsigned long long* xbest = c.take<unsigned long long>(MAXS);
  const int64_t lcap = kvc::auction_cand_cap(sh, p);   // candidate lists of the leaf and op selects
  uint64_t* lkey = c.take<uint64_t>((size_t)sh->n_seq * lcap);
  int32_t* lw = c.take<int32_t>((size_t)sh->n_seq * lcap);
  unsigned int* lcnt = c.take<unsigned int>(MAXS);
  int2* cslot = c.take<int2>((size_t)sh->n_seq * Fmax);
  int64_t E2 = 2 * E;
  zero_bytes(op_taken, E2, stream);
  KVC_LAUNCH_CHECK("zero_taken");
  zero_bytes(cover, E2 * 8, stream);
  KVC_LAUNCH_CHECK("zero_cover");
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(MAXS), 0, stream, (unsigned long long*)ccount, (int64_t)MAXS / 2);
  KVC_LAUNCH_CHECK("zero_count");

  KVC_REQUIRE(p->split_mode == 0 || trees->node_topo, KVC_E_INVAL, "kvc_auction: split_mode 1 needs node_topo");
  TreeArgs ta{};
  ta.cu = sh->cu_seqlens_d;
  ta.slot_start = slot_start;
  ta.n_slots = n_slots;
  ta.topo = p->split_mode == 1 ? trees->node_topo : nullptr;
  ta.stride = kvc_slot_stride(sh, p);
  ta.S = sh->n_seq;
  ta.Ly = sh->n_layers;
  ta.H = sh->n_kv_heads;
  ta.T = sh->total_tokens;
  Ranges ops{};
  fill_ranges(ops, sh, p, 0, true);
  int64_t nbo = ranges_blocks(ops);
  if (full && nbo > 0) {
    hipLaunchKernelGGL(hybrid_take_kernel, dim3((unsigned)nbo), dim3(256), 0, stream, ops, trees->op_cost, full, LH,
                       op_taken);
    KVC_LAUNCH_CHECK("hybrid_take");
  }

  // ---- floor: top-F leaves
  Ranges leaves{};
  fill_ranges(leaves, sh, p, 1, false);
  for (int s = 0; s < sh->n_seq; ++s) budget_r.len[s] = F[s];
  hipLaunchKernelGGL(init_state_kernel, dim3(1), dim3(MAXS), 0, stream, st, sh->n_seq, (const int64_t*)nullptr,
                     budget_r, 0, (const int64_t*)nullptr);
  KVC_LAUNCH_CHECK("init_state");
  LeafSrc lsrc{rel, head_sens, full, sh->total_tokens, LH};
  if ((r = select_compact(leaves, lsrc, st, hist, stream, lkey, lw, lcnt, lcap))) return r;
  FloorArgs fa{};
  fa.ta = ta;
  fa.rel = rel;
  fa.sens = head_sens;
  fa.op_cost = trees->op_cost;
  fa.taken = op_taken;
  fa.cover = cover;
  fa.ckey = ckey;
  fa.cid = cid;
  fa.ccost = ccost;
  fa.ccount = ccount;
  fa.cslot = cslot;
  fa.Fmax = Fmax;
  int64_t nb = ranges_blocks(leaves);
  bool any_floor = false;
  for (int s = 0; s < sh->n_seq; ++s) any_floor |= F[s] > 0;
  if (nb > 0 && any_floor) {
    // a sequence with F = 0 selects nothing: its budget is 0, so no key fits
    hipLaunchKernelGGL(floor_collect_kernel, dim3((unsigned)nb), dim3(256), 0, stream, leaves, lsrc, st, fa);
    KVC_LAUNCH_CHECK("floor_collect");
  }
  int64_t ncand = (int64_t)sh->n_seq * Fmax;
  hipLaunchKernelGGL(floor_cover_kernel, dim3(kvc_blocks(ncand, 256)), dim3(256), 0, stream, fa, sh->n_seq);
  KVC_LAUNCH_CHECK("floor_cover");
  hipLaunchKernelGGL(floor_cost_kernel, dim3(kvc_blocks(ncand, 256)), dim3(256), 0, stream, fa, sh->n_seq);
  KVC_LAUNCH_CHECK("floor_cost");
  // weighted select over the candidates: first candidate that does not fit
  Ranges cr{};
  cr.S = sh->n_seq;
  cr.U = 1;
  cr.unit_stride = 0;
  int64_t nleaf_unit = 0;
  for (int s = 0; s < sh->n_seq; ++s) {
    nleaf_unit = leaves.len[s] * leaves.U;
    cr.start[s] = (int64_t)s * Fmax;
    cr.len[s] = F[s] < nleaf_unit ? F[s] : nleaf_unit;
    cr.nchunk[s] = (cr.len[s] + CH - 1) / CH;
  }
  hipLaunchKernelGGL(init_state_kernel, dim3(1), dim3(MAXS), 0, stream, st, sh->n_seq, (const int64_t*)nullptr,
                     budget_r, 0, (const int64_t*)nullptr);
  KVC_LAUNCH_CHECK("init_state");
  CandSrc csrc{ckey, ccost};
  if ((r = run_select(cr, csrc, st, hist, stream))) return r;
  hipLaunchKernelGGL(floor_accept_kernel, dim3(kvc_blocks(ncand, 256)), dim3(256), 0, stream, fa, sh->n_seq, st);
  KVC_LAUNCH_CHECK("floor_accept");
  hipLaunchKernelGGL(floor_tail_kernel, dim3(sh->n_seq), dim3(FT_THREADS), 0, stream, fa, st, budget_r, sfloor);
  KVC_LAUNCH_CHECK("floor_tail");

  // ---- auction over every untaken op
  AucArgs aa{};
  aa.ta = ta;
  aa.util = trees->op_util;
  aa.cost = trees->op_cost;
  aa.taken = op_taken;
  aa.beta = cover;
  if (nbo > 0 && !ta.topo) {   // midpoint trees: one wave a (unit, slot)
    SlotRows sr{};
    const int64_t smin = std::max<int64_t>(1, p->slot_len > 0 ? p->slot_len : p->slot_min);
    for (int s = 0; s < sh->n_seq; ++s) {
      const int64_t L = sh->cu_seqlens[s + 1] - sh->cu_seqlens[s];
      sr.sbound[s + 1] = sr.sbound[s] + (int32_t)std::min<int64_t>(ta.stride, (L + smin - 1) / smin + 1);
    }
    const int64_t nw = (int64_t)LH * sr.sbound[sh->n_seq];
    if (nw > 0) {
      hipLaunchKernelGGL(beta_slot_kernel, dim3((unsigned)((nw + BS_WAVES - 1) / BS_WAVES)), dim3(BS_WAVES * 64), 0,
                         stream, aa, sr);
      KVC_LAUNCH_CHECK("beta_slot");
    }
  } else if (nbo > 0) {
    hipLaunchKernelGGL(beta_kernel, dim3((unsigned)nbo), dim3(256), 0, stream, aa, ops);
    KVC_LAUNCH_CHECK("beta");
  }
  for (int s = 0; s < sh->n_seq; ++s) budget_r.len[s] = A[s] - whole.v[s];
  hipLaunchKernelGGL(init_state_kernel, dim3(1), dim3(MAXS), 0, stream, st, sh->n_seq, (const int64_t*)nullptr,
                     budget_r, 0, (const int64_t*)sfloor);
  KVC_LAUNCH_CHECK("init_state");
  OpSrc osrc{cover, trees->op_cost, op_taken};
  // two passes over every op; then the ops still in the running go to the
  // candidate lists and the last six passes read those
  if ((r = select_compact(ops, osrc, st, hist, stream, lkey, lw, lcnt, lcap))) return r;
  if (nbo > 0) {
    hipLaunchKernelGGL(auction_mark_kernel, dim3((unsigned)nbo), dim3(256), 0, stream, aa, ops, st);
    KVC_LAUNCH_CHECK("auction_mark");
  }
  hipLaunchKernelGGL(auction_fixup_kernel, dim3(sh->n_seq), dim3(64), 0, stream, aa, st, (const int64_t*)sfloor,
                     spent, kleft);
  KVC_LAUNCH_CHECK("auction_fixup");
  if (ta.topo && nbo > 0) {   // only three-way splits (cost 2) can leave budget after the walk
    hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(MAXS), 0, stream, xbest, (int64_t)MAXS);
    KVC_LAUNCH_CHECK("zero_extend");
    hipLaunchKernelGGL(auction_extend_kernel, dim3((unsigned)nbo), dim3(256), 0, stream, aa, ops,
                       (const int64_t*)kleft, xbest);
    KVC_LAUNCH_CHECK("auction_extend");
    hipLaunchKernelGGL(auction_extend_take_kernel, dim3(1), dim3(MAXS), 0, stream, aa, sh->n_seq,
                       (const unsigned long long*)xbest, kleft, spent);
    KVC_LAUNCH_CHECK("auction_extend_take");
  }
  if (hybrid) {
    hipLaunchKernelGGL(add_whole_kernel, dim3(1), dim3(MAXS), 0, stream, sh->n_seq, whole, spent);
    KVC_LAUNCH_CHECK("add_whole");
  }
  hipLaunchKernelGGL(taken_normalize_kernel, dim3(kvc_blocks(E2, 256)), dim3(256), 0, stream, op_taken, E2);
  KVC_LAUNCH_CHECK("taken_normalize");
  return KVC_OK;
}

extern "C" int kvc_hybrid_units(const kvc_shape* sh, const kvc_params* p, const float* head_sens,
                                uint8_t* unit_full, hipStream_t stream) {
  int r = kvc::validate_shape(sh);
  if (r) return r;
  if ((r = kvc::validate_params(sh, p))) return r;
  KVC_REQUIRE(sh->n_seq <= MAXS, KVC_E_SHAPE, "kvc_hybrid_units: at most 64 sequences per call");
  const int LH = sh->n_layers * sh->n_kv_heads;
  KVC_REQUIRE(LH <= 4096, KVC_E_SHAPE, "kvc_hybrid_units: n_layers * n_kv_heads must be <= 4096");
  KVC_REQUIRE(head_sens && unit_full, KVC_E_INVAL, "kvc_hybrid_units: NULL pointer");
  std::vector<int64_t> B(sh->n_seq), A(sh->n_seq);
  if ((r = kvc_budgets(sh, p, B.data(), A.data(), nullptr))) return r;
  PerSeq nfull{};
  for (int s = 0; s < sh->n_seq; ++s) {
    kvc::Regions g = kvc::regions_of(sh->cu_seqlens[s + 1] - sh->cu_seqlens[s], *p);
    nfull.v[s] = kvc::hybrid_units_of(A[s], g.c1 - g.c0, LH, *p);
  }
  hipLaunchKernelGGL(hybrid_units_kernel, dim3(sh->n_seq), dim3(256), 0, stream, head_sens, LH, nfull, unit_full);
  KVC_LAUNCH_CHECK("hybrid_units");
  return KVC_OK;
}

namespace kvc {
size_t ws_topk_segments() {
  Carver c(nullptr, 0);
  c.take<SelState>(MAXS);
  c.take<unsigned long long>((size_t)MAXS * 256);
  return c.off + 256;
}

int topk_segments(int S, const int64_t* start, const int64_t* len, const int64_t* budget, const float* score,
                  const int32_t* pos, uint8_t* keep, void* ws, size_t ws_bytes, hipStream_t stream) {
  KVC_REQUIRE(S >= 1 && S <= MAXS, KVC_E_SHAPE, "top-B: 1 to 64 segments");
  KVC_REQUIRE(ws && ws_bytes >= ws_topk_segments(), KVC_E_WORKSPACE, "top-B: workspace too small");
  Carver c(ws, ws_bytes);
  SelState* st = c.take<SelState>(MAXS);
  unsigned long long* hist = c.take<unsigned long long>((size_t)MAXS * 256);
  hipLaunchKernelGGL(zero_u64_kernel, dim3(kvc_blocks(MAXS * 256, 256)), dim3(256), 0, stream, hist,
                     (int64_t)MAXS * 256);
  KVC_LAUNCH_CHECK("zero_hist");
  Ranges r{};
  r.S = S;
  r.U = 1;
  r.unit_stride = 0;
  Ranges budget_r{};
  budget_r.S = S;
  for (int s = 0; s < S; ++s) {
    r.start[s] = start[s];
    r.len[s] = len[s];
    r.nchunk[s] = (len[s] + CH - 1) / CH;
    budget_r.len[s] = budget[s];
  }
  hipLaunchKernelGGL(init_state_kernel, dim3(1), dim3(MAXS), 0, stream, st, S, (const int64_t*)nullptr, budget_r, 0,
                     (const int64_t*)nullptr);
  KVC_LAUNCH_CHECK("init_state");
  SegSrc src{score, pos};
  int rc = run_select(r, src, st, hist, stream);
  if (rc) return rc;
  int64_t nb = ranges_blocks(r);
  if (nb > 0) {
    hipLaunchKernelGGL(mark_keep_kernel, dim3((unsigned)nb), dim3(256), 0, stream, r, src, st, keep);
    KVC_LAUNCH_CHECK("mark_keep");
  }
  return KVC_OK;
}
}  // namespace kvc
