// Step-wise eviction: after every decode step the cache is scored by a small
// policy network over per-token features and pruned to the top-B tokens.
//
// DistillCache paper, Sec. 3.1.1 (state: for each cached token, its mean
// attention mass, value norm, variance of the mass across heads, the
// attention-weighted entropy of the recent queries and its position),
// Sec. 3.1.2 (deterministic top-B at inference) and Algorithm 1 (append the
// new pair, score, prune to B = max(floor(r * |C_t|), B_min); the pruned
// cache serves the next step).
//
// The student cache keeps one slot region per sequence, [Ly][H][cap][d]; a
// token occupies the same slot in every (l, h), so one eviction moves one
// row per unit. Slots are not kept in position order: an evicted slot below
// the new length is refilled by a kept token from past it, so a step that
// evicts one token moves one row per unit instead of shifting the cache.
//
// Per step and sequence:
// 1. the probe pass (rowstats / colsum of the scoring path) with the w
//    window queries as probes writes per-(l, h) features of every slot;
// 2. policy_kernel folds them over all (l, h) into the five features and
//    runs the MLP, 16 tokens per workgroup, weights in LDS;
// 3. the segmented radix select keeps the top-B by (score, position);
// 4. evict_pairs_kernel pairs holes below the new length with kept slots
//    past it; move_rows_kernel copies those rows (K, V, position).
#include <cmath>
#include <vector>

#include "kvc_internal.h"

namespace {

constexpr int HID = 128;
constexpr float LN_EPS = 1e-5f;
constexpr int MAXS = 64;

struct PerSeq {
  int64_t v[MAXS];
};

// ------------------------------------------------------------------ features + policy
struct PolArgs {
  const float* feats;   // per-(l, h) features [5][U][stride] (already offset to the sequence's first row)
  int64_t stride;       // rows per (l, h) unit in feats
  int U, G, P;
  int n;                // tokens of the sequence
  const int32_t* pos;   // token positions [n] (NULL: the row index)
  float inv_seen;       // 1 / max(n_seen - 1, 1)
  kvc_policy pol;
  float* x_out;         // [5][x_stride] or NULL
  int64_t x_stride;
  float* score;         // [n]
};

// A workgroup scores TOK tokens; its NSL slices of TOK threads split the
// fold over units and the hidden units of both layers (JS each), meeting in
// LDS for the LayerNorm statistics and the output sum.
constexpr int PT = 256;
constexpr int TOK = 16;
constexpr int NSL = PT / TOK;    // 16 slices
constexpr int JS = HID / NSL;    // 8 hidden units per slice
constexpr int W1N = HID * 5, W2N = HID * HID;
constexpr int HPAD = HID + 1;    // h1 and w2 rows padded against bank conflicts
constexpr int W2S = HPAD * HID;

__device__ __forceinline__ float slice_sum(float* red, int q, int tok, float v) {
  // sum of v over the NSL slices of one token (all threads return it)
  red[q * TOK + tok] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < NSL; ++k) t += red[k * TOK + tok];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(PT) void policy_kernel(PolArgs a) {
  extern __shared__ float pl[];
  float* w1 = pl;                 // [128][5]
  float* b1 = w1 + W1N;
  float* g1 = b1 + HID;
  float* be1 = g1 + HID;
  float* w2 = be1 + HID;          // [128][HPAD]
  float* b2 = w2 + W2S;
  float* g2 = b2 + HID;
  float* be2 = g2 + HID;
  float* w3 = be2 + HID;
  float* h1 = w3 + HID;           // [TOK][HPAD]
  float* red = h1 + TOK * HPAD;   // [NSL][TOK]
  for (int i = threadIdx.x; i < W1N; i += PT) w1[i] = a.pol.w1[i];
  for (int i = threadIdx.x; i < W2N; i += PT) w2[(i / HID) * HPAD + i % HID] = a.pol.w2[i];
  for (int i = threadIdx.x; i < HID; i += PT) {
    b1[i] = a.pol.b1[i];
    g1[i] = a.pol.g1[i];
    be1[i] = a.pol.be1[i];
    b2[i] = a.pol.b2[i];
    g2[i] = a.pol.g2[i];
    be2[i] = a.pol.be2[i];
    w3[i] = a.pol.w3[i];
  }
  __syncthreads();
  const int tok = threadIdx.x % TOK, q = threadIdx.x / TOK;
  const int i = blockIdx.x * TOK + tok;
  const bool live = i < a.n;
  const int ic = live ? i : a.n - 1;
  // fold the per-(l, h) features over every unit: slice q takes units q, q+NSL, ...
  const int64_t plane = (int64_t)a.U * a.stride;
  const float* f0 = a.feats + ic;
  float p0 = 0.f, p1 = 0.f, p3 = 0.f;
  for (int u = q; u < a.U; u += NSL) {
    const int64_t o = (int64_t)u * a.stride;
    const float m = f0[o];
    p0 += m;
    p1 += f0[plane + o];
    p3 += f0[3 * plane + o] * m;
  }
  const float s0 = slice_sum(red, q, tok, p0);
  const float s1 = slice_sum(red, q, tok, p1);
  const float s3 = slice_sum(red, q, tok, p3);
  // variance over all U*G query heads of the per-head mass: the mean of the
  // per-unit variances plus the variance of the per-unit means
  const float M = s0 / (float)(a.U * a.G);
  float pv = 0.f;
  for (int u = q; u < a.U; u += NSL) {
    const int64_t o = (int64_t)u * a.stride;
    const float dm = f0[o] / (float)a.G - M;
    pv += f0[2 * plane + o] + dm * dm;
  }
  const float sv = slice_sum(red, q, tok, pv);
  float x[5];
  x[0] = s0 / (float)(a.U * a.G * a.P);
  x[1] = s1 / (float)a.U;
  x[2] = sv / (float)a.U / ((float)a.P * (float)a.P);
  x[3] = s0 > 0.f ? s3 / s0 : 0.f;
  x[4] = (float)(a.pos ? a.pos[ic] : ic) * a.inv_seen;
  if (a.x_out && live && q < 5) a.x_out[q * a.x_stride + i] = x[q];
  // layer 1 (slice q: hidden units q*JS ..), LayerNorm over all 128, ReLU
  float z[JS];
  float pm = 0.f;
#pragma unroll
  for (int jj = 0; jj < JS; ++jj) {
    const int k = q * JS + jj;
    float v = b1[k];
#pragma unroll
    for (int c = 0; c < 5; ++c) v += w1[k * 5 + c] * x[c];
    z[jj] = v;
    pm += v;
  }
  float mu = slice_sum(red, q, tok, pm) * (1.f / HID);
  float pq = 0.f;
#pragma unroll
  for (int jj = 0; jj < JS; ++jj) pq += (z[jj] - mu) * (z[jj] - mu);
  float rs = 1.f / sqrtf(slice_sum(red, q, tok, pq) * (1.f / HID) + LN_EPS);
#pragma unroll
  for (int jj = 0; jj < JS; ++jj) {
    const int k = q * JS + jj;
    h1[tok * HPAD + k] = fmaxf((z[jj] - mu) * rs * g1[k] + be1[k], 0.f);
  }
  __syncthreads();
  // layer 2 (slice q: outputs q*JS ..), LayerNorm, ReLU, output layer
  pm = 0.f;
#pragma unroll
  for (int jj = 0; jj < JS; ++jj) {
    const int j = q * JS + jj;
    const float* wr = w2 + j * HPAD;
    const float* hr = h1 + tok * HPAD;
    float v = b2[j];
#pragma unroll 16
    for (int k = 0; k < HID; ++k) v += wr[k] * hr[k];
    z[jj] = v;
    pm += v;
  }
  mu = slice_sum(red, q, tok, pm) * (1.f / HID);
  pq = 0.f;
#pragma unroll
  for (int jj = 0; jj < JS; ++jj) pq += (z[jj] - mu) * (z[jj] - mu);
  rs = 1.f / sqrtf(slice_sum(red, q, tok, pq) * (1.f / HID) + LN_EPS);
  float po = 0.f;
#pragma unroll
  for (int jj = 0; jj < JS; ++jj) {
    const int j = q * JS + jj;
    po += w3[j] * fmaxf((z[jj] - mu) * rs * g2[j] + be2[j], 0.f);
  }
  const float out = slice_sum(red, q, tok, po) + a.pol.b3[0];
  if (live && q == 0) a.score[i] = out;
}

size_t policy_smem() { return (size_t)(W1N + W2S + 7 * HID + TOK * HPAD + NSL * TOK) * sizeof(float); }

int run_policy(PolArgs a, hipStream_t st) {
  if (a.n <= 0) return KVC_OK;
  const int sm = (int)policy_smem();
  (void)hipFuncSetAttribute((const void*)policy_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, sm);
  hipLaunchKernelGGL(policy_kernel, dim3((unsigned)((a.n + TOK - 1) / TOK)), dim3(PT), sm, st, a);
  KVC_LAUNCH_CHECK("policy");
  return KVC_OK;
}

// ------------------------------------------------------------------ cache moves
struct Pair {
  int32_t dst, src;  // slot indices (student) or source token index (init)
};

// Init: the kept tokens of sequence s, in position order, go to slots
// off_s + rank. One block per sequence.
__global__ __launch_bounds__(1024) void init_pairs_kernel(const uint8_t* keep, const int64_t* cu, PerSeq off,
                                                          PerSeq base, Pair* pairs, int32_t* pos) {
  __shared__ int wsum[16];
  __shared__ int carry;
  const int s = blockIdx.x;
  const int64_t a0 = cu[s], L = cu[s + 1] - cu[s];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int64_t c0 = 0; c0 < L; c0 += 1024) {
    const int64_t i = c0 + threadIdx.x;
    const int k = (i < L && keep[a0 + i]) ? 1 : 0;
    const uint64_t bal = __ballot(k);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int wbase = 0;
    for (int q = 0; q < wave; ++q) wbase += wsum[q];
    const int rank = carry + wbase + pre;
    if (k) {
      pairs[base.v[s] + rank] = Pair{(int32_t)(off.v[s] + rank), (int32_t)(a0 + i)};
      pos[off.v[s] + rank] = (int32_t)i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int tot = 0;
      for (int q = 0; q < 16; ++q) tot += wsum[q];
      carry += tot;
    }
    __syncthreads();
  }
}

// Step: holes (evicted slots below the new length) take the kept slots past
// it, both in slot order. One block per sequence; npair[s] receives the count.
__global__ __launch_bounds__(1024) void evict_pairs_kernel(const uint8_t* keep, PerSeq off, PerSeq len_old,
                                                           PerSeq len_new, int64_t pmax, Pair* pairs,
                                                           int32_t* npair) {
  __shared__ int hs[16], ms[16];
  __shared__ int hc, mc;
  const int s = blockIdx.x;
  const int64_t o = off.v[s], n = len_old.v[s], n2 = len_new.v[s];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) hc = mc = 0;
  __syncthreads();
  Pair* pr = pairs + (int64_t)s * pmax;
  for (int64_t c0 = 0; c0 < n; c0 += 1024) {
    const int64_t j = c0 + threadIdx.x;
    const bool in = j < n;
    const bool kp = in && keep[o + j];
    const int hole = (in && j < n2 && !kp) ? 1 : 0;
    const int mover = (in && j >= n2 && kp) ? 1 : 0;
    const uint64_t bh = __ballot(hole), bm = __ballot(mover);
    const uint64_t below = (1ull << lane) - 1ull;
    if (lane == 0) {
      hs[wave] = __popcll(bh);
      ms[wave] = __popcll(bm);
    }
    __syncthreads();
    int hb = 0, mb = 0;
    for (int q = 0; q < wave; ++q) {
      hb += hs[q];
      mb += ms[q];
    }
    if (hole) {
      const int r = hc + hb + __popcll(bh & below);
      if (r < pmax) pr[r].dst = (int32_t)(o + j);
    }
    if (mover) {
      const int r = mc + mb + __popcll(bm & below);
      if (r < pmax) pr[r].src = (int32_t)(o + j);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int q = 0; q < 16; ++q) {
        hc += hs[q];
        mc += ms[q];
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) npair[s] = hc < mc ? hc : mc;
}

// Copy rows for every (l, h): one thread per 16-byte piece. Pairs of
// sequence s sit at pairs[s * pmax + r], r < npair[s] (npair NULL: the
// first `count` pairs, src indexes the source layout).
struct MoveArgs {
  const char* src_k;
  const char* src_v;
  char* dst_k;
  char* dst_v;
  int64_t src_stride, dst_stride;  // rows per (l, h) unit
  int row_bytes;
  int U;
  const Pair* pairs;
  const int32_t* npair;
  int64_t pmax;
  int S;
  int64_t count;
  int32_t* pos;  // student positions (moved with the rows when npair != NULL)
};
__global__ __launch_bounds__(256) void move_rows_kernel(MoveArgs a) {
  const int pieces = a.row_bytes / 16;
  const int64_t per_pair = (int64_t)a.U * pieces;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pr = g / per_pair;
  const int64_t rem = g % per_pair;
  const int u = (int)(rem / pieces), pc = (int)(rem % pieces);
  Pair p;
  if (a.npair) {
    const int s = (int)(pr / a.pmax);
    const int64_t r = pr % a.pmax;
    if (s >= a.S || r >= a.npair[s]) return;
    p = a.pairs[pr];
    if (u == 0 && pc == 0) a.pos[p.dst] = a.pos[p.src];
  } else {
    if (pr >= a.count) return;
    p = a.pairs[pr];
  }
  const int64_t so = ((int64_t)u * a.src_stride + p.src) * a.row_bytes + pc * 16;
  const int64_t d0 = ((int64_t)u * a.dst_stride + p.dst) * a.row_bytes + pc * 16;
  *(uint4*)(a.dst_k + d0) = *(const uint4*)(a.src_k + so);
  *(uint4*)(a.dst_v + d0) = *(const uint4*)(a.src_v + so);
}

int launch_moves(const MoveArgs& a, int64_t n_pairs_total, hipStream_t st) {
  const int64_t nthr = n_pairs_total * a.U * (a.row_bytes / 16);
  if (nthr <= 0) return KVC_OK;
  hipLaunchKernelGGL(move_rows_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, st, a);
  KVC_LAUNCH_CHECK("move_rows");
  return KVC_OK;
}

// Append decode token t of every sequence to slot off_s + len_s of every
// (l, h); one thread per 16-byte piece.
__global__ __launch_bounds__(256) void append_kernel(const char* kt, const char* vt, char* K, char* V, int32_t* pos,
                                                     int S, int U, int64_t cap, int row_bytes, int t, int t_cap,
                                                     PerSeq slot, PerSeq p_new) {
  const int pieces = row_bytes / 16;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_seq = (int64_t)U * pieces;
  if (g >= (int64_t)S * per_seq) return;
  const int s = (int)(g / per_seq);
  const int u = (int)((g % per_seq) / pieces), pc = (int)(g % pieces);
  const int64_t src = (((int64_t)u * S + s) * t_cap + t) * row_bytes + pc * 16;
  const int64_t dst = ((int64_t)u * cap + slot.v[s]) * row_bytes + pc * 16;
  *(uint4*)(K + dst) = *(const uint4*)(kt + src);
  *(uint4*)(V + dst) = *(const uint4*)(vt + src);
  if (u == 0 && pc == 0) pos[slot.v[s]] = (int32_t)p_new.v[s];
}

// Window rows: init copies the last w prefill queries, a push overwrites
// ring slot t mod w with the decode query. One thread per 16-byte piece.
__global__ __launch_bounds__(256) void window_init_kernel(const char* qctx, char* qwin, const int64_t* cu, int S,
                                                          int HGL, int64_t T, int w, int row_bytes) {
  const int pieces = row_bytes / 16;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_seq = (int64_t)HGL * w * pieces;
  if (g >= (int64_t)S * per_seq) return;
  const int s = (int)(g / per_seq);
  const int64_t r = g % per_seq;
  const int hq = (int)(r / ((int64_t)w * pieces));  // (l, query head)
  const int j = (int)((r / pieces) % w), pc = (int)(r % pieces);
  const int64_t tok = cu[s + 1] - w + j;
  const int64_t src = ((int64_t)hq * T + tok) * row_bytes + pc * 16;
  const int64_t dst = ((((int64_t)s * HGL + hq) * w) + j) * row_bytes + pc * 16;
  *(uint4*)(qwin + dst) = *(const uint4*)(qctx + src);
}
__global__ __launch_bounds__(256) void window_push_kernel(const char* q, char* qwin, int S, int HGL, int w, int slot,
                                                          int row_bytes) {
  const int pieces = row_bytes / 16;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= (int64_t)S * HGL * pieces) return;
  const int64_t row = g / pieces;  // s * HGL + (l, query head)
  const int pc = (int)(g % pieces);
  *(uint4*)(qwin + ((row * w) + slot) * row_bytes + pc * 16) = *(const uint4*)(q + row * row_bytes + pc * 16);
}

__global__ void view_kernel(int64_t* seg_off, int32_t* seg_len, int S, int U, int64_t cap, PerSeq off, PerSeq len) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= S * U) return;
  const int s = g / U, u = g % U;
  seg_off[g] = (int64_t)u * cap + off.v[s];
  seg_len[g] = (int32_t)len.v[s];
}

__global__ void set_cu_kernel(int64_t* cu, int64_t n) {
  cu[0] = 0;
  cu[1] = n;
}

int64_t step_budget(int64_t n_seen, const kvc_params* p) {
  int64_t b = (int64_t)std::floor((double)p->budget_ratio * (double)n_seen);
  return b < p->budget_min ? p->budget_min : b;
}

int check_step(const kvc_shape* sh, const kvc_params* p) {
  int r = kvc::validate_shape(sh);
  if (r) return r;
  KVC_REQUIRE(p, KVC_E_INVAL, "params is NULL");
  KVC_REQUIRE(sh->n_seq <= MAXS, KVC_E_SHAPE, "step-wise eviction: at most 64 sequences");
  KVC_REQUIRE(p->window >= 8 && p->window % 8 == 0 && (int64_t)p->window * sh->group <= 256, KVC_E_INVAL,
              "window must be a multiple of 8 with window * group <= 256");
  KVC_REQUIRE(p->budget_ratio >= 0.f && p->budget_ratio <= 1.f && p->budget_min >= 1, KVC_E_INVAL,
              "step-wise eviction needs budget_ratio in [0, 1] and budget_min >= 1");
  for (int s = 0; s < sh->n_seq; ++s)
    KVC_REQUIRE(sh->cu_seqlens[s + 1] - sh->cu_seqlens[s] >= p->window, KVC_E_SHAPE,
                "step-wise eviction: every sequence needs at least `window` tokens");
  return KVC_OK;
}

kvc_params window_params(const kvc_params* p) {
  kvc_params q = *p;
  q.n_probe = p->window;  // the window queries play the probes
  return q;
}

struct StepWs {
  float* feats;     // [5][U][stride]
  float* rel0;      // [U][stride]
  float* lse;       // [S][U*G][w]
  float* ent;
  float* hsens;     // [S*U]
  float* score;     // [stride]
  uint8_t* keep;    // [stride]
  Pair* pairs;      // [stride]
  int32_t* npair;   // [MAXS]
  int64_t* cu1;     // [2]
  void* sws;        // probe-pass workspace
  size_t sws_bytes;
  void* tws;        // top-B workspace
  size_t tws_bytes;
};

size_t carve(const kvc_shape* sh, const kvc_params* p, int64_t cap_total, void* ws, size_t ws_bytes, StepWs* out) {
  const int64_t U = (int64_t)sh->n_layers * sh->n_kv_heads;
  const int64_t stride = cap_total > sh->total_tokens ? cap_total : sh->total_tokens;
  kvc_params q = window_params(p);
  // probe-pass workspace: the larger of the whole-batch call and one sequence
  // over the student. A shorter sequence may pick a narrower key tile and
  // need more splits; a sequence four times the capacity bounds them all
  // (its split count is at least that of the narrowest tile over cap_total).
  size_t sws = kvc::ws_score(sh, &q);
  int64_t cu1[2] = {0, 4 * cap_total};
  kvc_shape one = *sh;
  one.n_seq = 1;
  one.total_tokens = cu1[1];
  one.cu_seqlens = cu1;
  size_t s1 = kvc::ws_score(&one, &q);
  sws = s1 > sws ? s1 : sws;
  kvc::Carver c(ws, ws_bytes);
  StepWs w{};
  w.feats = c.take<float>((size_t)5 * U * stride);
  w.rel0 = c.take<float>((size_t)U * stride);
  w.lse = c.take<float>((size_t)sh->n_seq * U * sh->group * p->window);
  w.ent = c.take<float>((size_t)sh->n_seq * U * sh->group * p->window);
  w.hsens = c.take<float>((size_t)sh->n_seq * U);
  w.score = c.take<float>((size_t)stride);
  w.keep = c.take<uint8_t>((size_t)stride);
  w.pairs = c.take<Pair>((size_t)stride);
  w.npair = c.take<int32_t>(MAXS);
  w.cu1 = c.take<int64_t>(2);
  w.sws_bytes = sws;
  w.sws = c.take<char>(sws);
  w.tws_bytes = kvc::ws_topk_segments();
  w.tws = c.take<char>(w.tws_bytes);
  if (out) *out = w;
  return c.off + 256;
}

void refresh_view(const kvc_shape* sh, const kvc_student* st, hipStream_t stream) {
  const int U = sh->n_layers * sh->n_kv_heads;
  PerSeq off{}, len{};
  for (int s = 0; s < sh->n_seq; ++s) {
    off.v[s] = st->seq_off[s];
    len.v[s] = st->seq_len[s];
  }
  hipLaunchKernelGGL(view_kernel, dim3((unsigned)((sh->n_seq * U + 255) / 256)), dim3(256), 0, stream, st->seg_off,
                     st->seg_len, sh->n_seq, U, st->cap_total, off, len);
}

}  // namespace

extern "C" int kvc_step_capacity(const kvc_shape* sh, const kvc_params* p, int32_t t_steps, int32_t* seq_cap) {
  int r = check_step(sh, p);
  if (r) return r;
  KVC_REQUIRE(t_steps >= 0 && seq_cap, KVC_E_INVAL, "kvc_step_capacity: bad arguments");
  for (int s = 0; s < sh->n_seq; ++s) {
    const int64_t L = sh->cu_seqlens[s + 1] - sh->cu_seqlens[s];
    int64_t c = step_budget(L + t_steps, p) + 1;
    if (c > L + t_steps) c = L + t_steps;
    seq_cap[s] = (int32_t)c;
  }
  return KVC_OK;
}

extern "C" size_t kvc_step_workspace(const kvc_shape* sh, const kvc_params* p, int64_t cap_total) {
  if (check_step(sh, p) || cap_total < 1) return 0;
  return carve(sh, p, cap_total, nullptr, 0, nullptr);
}

extern "C" int kvc_step_init(const kvc_shape* sh, const kvc_params* p, const void* K, const void* V,
                             const void* Qctx, const kvc_policy* pol, kvc_student* st, float* feats_out,
                             float* scores_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int r = check_step(sh, p);
  if (r) return r;
  KVC_REQUIRE(K && V && Qctx && pol && st && st->K && st->V && st->pos && st->Qwin && st->seg_off && st->seg_len &&
                  st->seq_off && st->seq_cap && st->seq_len,
              KVC_E_INVAL, "kvc_step_init: NULL argument");
  KVC_REQUIRE(ws && ws_bytes >= kvc_step_workspace(sh, p, st->cap_total), KVC_E_WORKSPACE,
              "kvc_step_init: workspace too small");
  const int S = sh->n_seq, U = sh->n_layers * sh->n_kv_heads, G = sh->group, w = p->window;
  const int elt = sh->dtype == KVC_BF16 ? 2 : 4, row_bytes = sh->head_dim * elt;
  std::vector<int64_t> start(S), len(S), bud(S);
  PerSeq off{}, base{};
  int64_t kept = 0;
  for (int s = 0; s < S; ++s) {
    const int64_t L = sh->cu_seqlens[s + 1] - sh->cu_seqlens[s];
    start[s] = sh->cu_seqlens[s];
    len[s] = L;
    bud[s] = step_budget(L, p);
    const int64_t k = bud[s] < L ? bud[s] : L;
    KVC_REQUIRE(st->seq_off[s] >= 0 && k <= st->seq_cap[s] && st->seq_off[s] + st->seq_cap[s] <= st->cap_total,
                KVC_E_SHAPE, "kvc_step_init: a sequence's slot region is too small or out of range");
    off.v[s] = st->seq_off[s];
    base.v[s] = kept;
    kept += k;
  }
  StepWs W;
  carve(sh, p, st->cap_total, ws, ws_bytes, &W);
  // window: the last w prefill queries of every sequence
  const int HGL = sh->n_layers * sh->n_kv_heads * G;
  int64_t nthr = (int64_t)S * HGL * w * (row_bytes / 16);
  hipLaunchKernelGGL(window_init_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, stream,
                     (const char*)Qctx, (char*)st->Qwin, sh->cu_seqlens_d, S, HGL, sh->total_tokens, w, row_bytes);
  KVC_LAUNCH_CHECK("window_init");
  // probe pass with the window over the prefill cache (row stride T)
  kvc_params q = window_params(p);
  r = kvc::score_strided(sh, &q, K, V, st->Qwin, W.rel0, W.feats, W.lse, W.ent, W.hsens, W.sws, W.sws_bytes, stream);
  if (r) return r;
  for (int s = 0; s < S; ++s) {
    PolArgs a{};
    a.feats = W.feats + start[s];
    a.stride = sh->total_tokens;
    a.U = U;
    a.G = G;
    a.P = w;
    a.n = (int)len[s];
    a.pos = nullptr;
    a.inv_seen = 1.f / (float)(len[s] > 1 ? len[s] - 1 : 1);
    a.pol = *pol;
    a.x_out = feats_out ? feats_out + start[s] : nullptr;
    a.x_stride = sh->total_tokens;
    a.score = (scores_out ? scores_out : W.score) + start[s];
    if ((r = run_policy(a, stream))) return r;
  }
  const float* score = scores_out ? scores_out : W.score;
  if ((r = kvc::topk_segments(S, start.data(), len.data(), bud.data(), score, nullptr, W.keep, W.tws, W.tws_bytes,
                              stream)))
    return r;
  hipLaunchKernelGGL(init_pairs_kernel, dim3(S), dim3(1024), 0, stream, W.keep, sh->cu_seqlens_d, off, base, W.pairs,
                     st->pos);
  KVC_LAUNCH_CHECK("init_pairs");
  MoveArgs m{};
  m.src_k = (const char*)K;
  m.src_v = (const char*)V;
  m.dst_k = (char*)st->K;
  m.dst_v = (char*)st->V;
  m.src_stride = sh->total_tokens;
  m.dst_stride = st->cap_total;
  m.row_bytes = row_bytes;
  m.U = U;
  m.pairs = W.pairs;
  m.npair = nullptr;
  m.count = kept;
  if ((r = launch_moves(m, kept, stream))) return r;
  for (int s = 0; s < S; ++s) st->seq_len[s] = (int32_t)(bud[s] < len[s] ? bud[s] : len[s]);
  refresh_view(sh, st, stream);
  KVC_LAUNCH_CHECK("view");
  return KVC_OK;
}

extern "C" int kvc_step_append(const kvc_shape* sh, const kvc_params* p, kvc_student* st, const void* K_tail,
                               const void* V_tail, const void* Q_t, int32_t t, int32_t t_cap, hipStream_t stream) {
  int r = check_step(sh, p);
  if (r) return r;
  KVC_REQUIRE(st && K_tail && V_tail && Q_t && t >= 0 && t < t_cap, KVC_E_INVAL, "kvc_step_append: bad arguments");
  const int S = sh->n_seq, U = sh->n_layers * sh->n_kv_heads;
  const int row_bytes = sh->head_dim * (sh->dtype == KVC_BF16 ? 2 : 4);
  PerSeq slot{}, pnew{};
  for (int s = 0; s < S; ++s) {
    KVC_REQUIRE(st->seq_len[s] < st->seq_cap[s], KVC_E_SHAPE, "kvc_step_append: a sequence has no free slot");
    slot.v[s] = st->seq_off[s] + st->seq_len[s];
    pnew.v[s] = sh->cu_seqlens[s + 1] - sh->cu_seqlens[s] + t;
  }
  int64_t nthr = (int64_t)S * U * (row_bytes / 16);
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, stream,
                     (const char*)K_tail, (const char*)V_tail, (char*)st->K, (char*)st->V, st->pos, S, U,
                     st->cap_total, row_bytes, t, t_cap, slot, pnew);
  KVC_LAUNCH_CHECK("append");
  const int HGL = U * sh->group;
  nthr = (int64_t)S * HGL * (row_bytes / 16);
  hipLaunchKernelGGL(window_push_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, stream,
                     (const char*)Q_t, (char*)st->Qwin, S, HGL, p->window, t % p->window, row_bytes);
  KVC_LAUNCH_CHECK("window_push");
  for (int s = 0; s < S; ++s) st->seq_len[s] += 1;
  refresh_view(sh, st, stream);
  KVC_LAUNCH_CHECK("view");
  return KVC_OK;
}

extern "C" int kvc_step_prune(const kvc_shape* sh, const kvc_params* p, kvc_student* st, int32_t t,
                              const kvc_policy* pol, float* feats_out, float* scores_out, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  int r = check_step(sh, p);
  if (r) return r;
  KVC_REQUIRE(st && pol && t >= 0, KVC_E_INVAL, "kvc_step_prune: bad arguments");
  KVC_REQUIRE(ws && ws_bytes >= kvc_step_workspace(sh, p, st->cap_total), KVC_E_WORKSPACE,
              "kvc_step_prune: workspace too small");
  const int S = sh->n_seq, U = sh->n_layers * sh->n_kv_heads, G = sh->group, w = p->window;
  const int row_bytes = sh->head_dim * (sh->dtype == KVC_BF16 ? 2 : 4);
  StepWs W;
  carve(sh, p, st->cap_total, ws, ws_bytes, &W);
  kvc_params q = window_params(p);
  float* score = scores_out ? scores_out : W.score;
  std::vector<int64_t> start(S), len(S), bud(S);
  PerSeq off{}, lold{}, lnew{};
  int64_t pmax = 1;
  for (int s = 0; s < S; ++s) {
    const int64_t L = sh->cu_seqlens[s + 1] - sh->cu_seqlens[s];
    const int64_t n = st->seq_len[s];
    start[s] = st->seq_off[s];
    len[s] = n;
    bud[s] = step_budget(L + t + 1, p);
    off.v[s] = st->seq_off[s];
    lold.v[s] = n;
    lnew.v[s] = bud[s] < n ? bud[s] : n;
    pmax = n - lnew.v[s] > pmax ? n - lnew.v[s] : pmax;
    // probe pass over this sequence's slots: one sequence, row stride cap_total
    int64_t cuh[2] = {0, n};
    kvc_shape one = *sh;
    one.n_seq = 1;
    one.total_tokens = st->cap_total;
    one.cu_seqlens = cuh;
    one.cu_seqlens_d = W.cu1;
    hipLaunchKernelGGL(set_cu_kernel, dim3(1), dim3(1), 0, stream, W.cu1, n);
    KVC_LAUNCH_CHECK("set_cu");
    const size_t qrow = (size_t)U * G * w * row_bytes;
    r = kvc::score_strided(&one, &q, (const char*)st->K + (size_t)start[s] * row_bytes,
                           (const char*)st->V + (size_t)start[s] * row_bytes, (const char*)st->Qwin + s * qrow,
                           W.rel0 + start[s], W.feats + start[s], W.lse, W.ent, W.hsens, W.sws, W.sws_bytes, stream);
    if (r) return r;
    PolArgs a{};
    a.feats = W.feats + start[s];
    a.stride = st->cap_total;
    a.U = U;
    a.G = G;
    a.P = w;
    a.n = (int)n;
    a.pos = st->pos + start[s];
    const int64_t seen = L + t + 1;
    a.inv_seen = 1.f / (float)(seen > 1 ? seen - 1 : 1);
    a.pol = *pol;
    a.x_out = feats_out ? feats_out + start[s] : nullptr;
    a.x_stride = st->cap_total;
    a.score = score + start[s];
    if ((r = run_policy(a, stream))) return r;
  }
  KVC_REQUIRE(pmax * S <= st->cap_total, KVC_E_SHAPE, "kvc_step_prune: eviction list exceeds the workspace");
  if ((r = kvc::topk_segments(S, start.data(), len.data(), bud.data(), score, st->pos, W.keep, W.tws, W.tws_bytes,
                              stream)))
    return r;
  hipLaunchKernelGGL(evict_pairs_kernel, dim3(S), dim3(1024), 0, stream, W.keep, off, lold, lnew, pmax, W.pairs,
                     W.npair);
  KVC_LAUNCH_CHECK("evict_pairs");
  MoveArgs m{};
  m.src_k = (const char*)st->K;
  m.src_v = (const char*)st->V;
  m.dst_k = (char*)st->K;
  m.dst_v = (char*)st->V;
  m.src_stride = m.dst_stride = st->cap_total;
  m.row_bytes = row_bytes;
  m.U = U;
  m.pairs = W.pairs;
  m.npair = W.npair;
  m.pmax = pmax;
  m.S = S;
  m.pos = st->pos;
  if ((r = launch_moves(m, (int64_t)S * pmax, stream))) return r;
  for (int s = 0; s < S; ++s) st->seq_len[s] = (int32_t)lnew.v[s];
  refresh_view(sh, st, stream);
  KVC_LAUNCH_CHECK("view");
  return KVC_OK;
}
