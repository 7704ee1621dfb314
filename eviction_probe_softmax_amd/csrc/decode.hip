// One decode step of attention over a ragged (compressed or full) cache.
//
// GraceKV page, '05 Physical cache packing': decoding reads the physical
// ragged cache and newly generated tokens are appended with multiplicity one;
// 'Inside one cache entry': a prototype counts for mu tokens (logit + ln mu).
// DistillCache paper, Sec. 3.1.3: the full and the pruned cache both append
// each new (k, v).
//
// Split-K: each workgroup takes up to CHUNK entries of one (s, l, h) segment
// (or of its appended tail), computes the G query heads' logits, a local
// softmax and the weighted value sum, and writes (max, sum, o[d]) per head.
// The combine kernel merges the chunks of every (s, l, h, g), normalizes and
// sums the layers in order into x. The step is HBM-bound: every packed K and
// V byte is read once, 16 bytes per lane, rows of one entry across
// D/8 consecutive lanes.
#include <cmath>

#include "kvc_internal.h"

namespace {

constexpr int CHUNK = 256;
constexpr int THREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;

struct DecArgs {
  const void* K;
  const void* V;
  const float* lnmu;
  const int64_t* seg_off;
  const int32_t* seg_len;
  const void* Kt;
  const void* Vt;
  const void* Q;
  int S, Ly, H, G, t_valid, t_cap, nchunk;
  float scale2;  // log2(e)/sqrt(d)
};

template <class T> struct Vec8;
template <> struct Vec8<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* f) {
    uint4 u = *(const uint4*)p;
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* f) {
    float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

// partial layout: [unit][chunk][G][D + 2] = o[D], max2, sum
template <class T, int D>
__global__ __launch_bounds__(THREADS) void decode_partial_kernel(DecArgs a, float* part) {
  constexpr int LPE = D / 8;       // lanes per entry
  constexpr int EPI = 64 / LPE;    // entries per wave iteration
  constexpr int GMAX = 8;
  __shared__ float z_s[GMAX][CHUNK];
  __shared__ float m_s[GMAX], l_s[GMAX];
  __shared__ float o_s[4][GMAX][D];
  const int unit = blockIdx.x / a.nchunk, chunk = blockIdx.x % a.nchunk;
  const int s = unit / (a.Ly * a.H), lh = unit % (a.Ly * a.H);
  const int l = lh / a.H, h = lh % a.H;
  const int seg_idx = (s * a.Ly + l) * a.H + h;
  const int64_t slen = a.seg_len[seg_idx];
  // the grid covers max_seg entries per segment; never index past it
  const int nseg = min((int)((slen + CHUNK - 1) / CHUNK), a.nchunk - (a.t_cap + CHUNK - 1) / CHUNK);
  const T* Kb;
  const T* Vb;
  const float* lm = nullptr;
  int64_t e0, n;
  if (chunk < nseg) {
    int64_t off = a.seg_off[seg_idx];
    e0 = (int64_t)chunk * CHUNK;
    n = slen - e0 < CHUNK ? slen - e0 : CHUNK;
    Kb = (const T*)a.K + (off + e0) * D;
    Vb = (const T*)a.V + (off + e0) * D;
    if (a.lnmu) lm = a.lnmu + off + e0;
  } else {
    int tc = chunk - nseg;
    e0 = (int64_t)tc * CHUNK;
    if (e0 >= a.t_valid) return;
    n = a.t_valid - e0 < CHUNK ? a.t_valid - e0 : CHUNK;
    int64_t tb = (((int64_t)l * a.H + h) * a.S + s) * a.t_cap + e0;
    Kb = (const T*)a.Kt + tb * D;
    Vb = (const T*)a.Vt + tb * D;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPE, slot = lane / LPE;
  const int G = a.G;
  // query slice of every head of the group for this lane's 8 dims
  float q[GMAX][8];
  const T* Qb = (const T*)a.Q + (((int64_t)s * a.Ly + l) * a.H * G + (int64_t)h * G) * D + sub * 8;
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
    if (g < G) Vec8<T>::load(Qb + (int64_t)g * D, q[g]);
  // phase 1: logits
  for (int e = wave * EPI + slot; e < CHUNK; e += 4 * EPI) {
    float k[8];
    bool ok = e < n;
    if (ok) Vec8<T>::load(Kb + (int64_t)e * D + sub * 8, k);
    else {
#pragma unroll
      for (int j = 0; j < 8; ++j) k[j] = 0.f;
    }
    float bias = (ok && lm) ? lm[e] * LOG2E : 0.f;
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) break;
      float dsum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) dsum += q[g][j] * k[j];
#pragma unroll
      for (int o = LPE / 2; o > 0; o >>= 1) dsum += __shfl_xor(dsum, o, 64);
      if (sub == 0 && e < CHUNK) z_s[g][e] = ok ? dsum * a.scale2 + bias : -INFINITY;
    }
  }
  __syncthreads();
  // phase 2: per-head max and exponentials (one wave per head, strided)
  for (int g = wave; g < G; g += 4) {
    float mx = -INFINITY;
    for (int e = lane; e < CHUNK; e += 64) mx = fmaxf(mx, z_s[g][e]);
    mx = wave_max(mx);
    float sm = 0.f;
    for (int e = lane; e < CHUNK; e += 64) {
      float p = mx == -INFINITY ? 0.f : exp2f(z_s[g][e] - mx);
      z_s[g][e] = p;
      sm += p;
    }
    sm = wave_sum(sm);
    if (lane == 0) {
      m_s[g] = mx;
      l_s[g] = sm;
    }
  }
  __syncthreads();
  // phase 3: o_g = sum_e p_g(e) v_e over this lane's 8 dims
  float acc[GMAX][8];
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[g][j] = 0.f;
  for (int e = wave * EPI + slot; e < n; e += 4 * EPI) {
    float v[8];
    Vec8<T>::load(Vb + (int64_t)e * D + sub * 8, v);
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) break;
      float p = z_s[g][e];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[g][j] += p * v[j];
    }
  }
  // reduce over the wave's entry slots (lanes sharing `sub`)
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g >= G) break;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = acc[g][j];
#pragma unroll
      for (int o = LPE; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
      if (slot == 0) o_s[wave][g][sub * 8 + j] = x;
    }
  }
  __syncthreads();
  float* pb = part + ((int64_t)unit * a.nchunk + chunk) * G * (D + 2);
  for (int i = threadIdx.x; i < G * D; i += THREADS) {
    int g = i / D, dd = i % D;
    pb[g * (D + 2) + dd] = o_s[0][g][dd] + o_s[1][g][dd] + o_s[2][g][dd] + o_s[3][g][dd];
  }
  if (threadIdx.x < G) {
    pb[threadIdx.x * (D + 2) + D] = m_s[threadIdx.x];
    pb[threadIdx.x * (D + 2) + D + 1] = l_s[threadIdx.x];
  }
}

// one workgroup per (s, h, g); D threads; layers summed in order
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecArgs a, const float* part, float* x_out,
                                                           int64_t x_stride, float* o_out) {
  const int G = a.G;
  const int s = blockIdx.x / (a.H * G);
  const int hg = blockIdx.x % (a.H * G);
  const int h = hg / G, g = hg % G;
  const int dd = threadIdx.x;
  float x = 0.f;
  for (int l = 0; l < a.Ly; ++l) {
    const int seg_idx = (s * a.Ly + l) * a.H + h;
    const int unit = (s * a.Ly + l) * a.H + h;  // same numbering as the partial kernel
    const int64_t slen = a.seg_len[seg_idx];
    const int nseg = min((int)((slen + CHUNK - 1) / CHUNK), a.nchunk - (a.t_cap + CHUNK - 1) / CHUNK);
    const int ntail = (a.t_valid + CHUNK - 1) / CHUNK;
    float m = -INFINITY, sum = 0.f, o = 0.f;
    for (int c = 0; c < nseg + ntail; ++c) {
      const float* pb = part + (((int64_t)unit * a.nchunk + c) * G + g) * (D + 2);
      float mc = pb[D], lc = pb[D + 1];
      if (mc == -INFINITY) continue;
      float mn = fmaxf(m, mc);
      float f1 = exp2f(m - mn), f2 = exp2f(mc - mn);
      sum = sum * f1 + lc * f2;
      o = o * f1 + pb[dd] * f2;
      m = mn;
    }
    float ov = sum > 0.f ? o / sum : 0.f;
    if (o_out) o_out[(((int64_t)s * a.Ly + l) * a.H * G + hg) * D + dd] = ov;
    x += ov;
  }
  x_out[(int64_t)s * x_stride + (int64_t)hg * D + dd] = x;
}

int nchunk_of(const kvc_ragged* c, int t_cap) {
  return (c->max_seg + CHUNK - 1) / CHUNK + (t_cap + CHUNK - 1) / CHUNK;
}

}  // namespace

extern "C" size_t kvc_decode_workspace(const kvc_ragged* c, int32_t group, int32_t t_cap) {
  if (!c || group < 1 || t_cap < 0 || c->max_seg < 0) return 0;
  int64_t units = (int64_t)c->n_seq * c->n_layers * c->n_kv_heads;
  return (size_t)units * nchunk_of(c, t_cap) * group * (c->head_dim + 2) * sizeof(float) + 256;
}

extern "C" int kvc_decode_attn(const kvc_ragged* c, const void* K_tail, const void* V_tail, int32_t t_valid,
                               int32_t t_cap, const void* Q, int32_t group, float* x_out, int64_t x_stride,
                               float* o_out, void* ws, size_t ws_bytes, hipStream_t st) {
  KVC_REQUIRE(c != nullptr, KVC_E_INVAL, "cache is NULL");
  KVC_REQUIRE(c->seg_off && c->seg_len && Q && x_out, KVC_E_INVAL, "kvc_decode_attn: NULL pointer");
  KVC_REQUIRE(c->capacity >= 0 && (c->capacity == 0 || (c->K && c->V)), KVC_E_INVAL,
              "kvc_decode_attn: NULL cache K/V with a nonzero capacity");
  KVC_REQUIRE(c->head_dim == 64 || c->head_dim == 128, KVC_E_SHAPE, "head_dim must be 64 or 128");
  KVC_REQUIRE(c->dtype == KVC_BF16 || c->dtype == KVC_F32, KVC_E_DTYPE, "cache dtype must be bf16 or f32");
  KVC_REQUIRE(group >= 1 && group <= 8, KVC_E_SHAPE, "group must be in [1, 8]");
  KVC_REQUIRE(c->n_seq >= 1 && c->n_layers >= 1 && c->n_kv_heads >= 1, KVC_E_SHAPE, "empty cache shape");
  KVC_REQUIRE(t_valid >= 0 && t_valid <= t_cap, KVC_E_INVAL, "need 0 <= t_valid <= t_cap");
  KVC_REQUIRE(t_valid == 0 || (K_tail && V_tail), KVC_E_INVAL, "tail pointers are NULL");
  KVC_REQUIRE(x_stride >= (int64_t)c->n_kv_heads * group * c->head_dim, KVC_E_INVAL, "x_stride too small");
  KVC_REQUIRE(c->max_seg >= 0, KVC_E_INVAL, "max_seg must be >= 0");
  KVC_REQUIRE(ws && ws_bytes >= kvc_decode_workspace(c, group, t_cap), KVC_E_WORKSPACE,
              "kvc_decode_attn: workspace too small");
  DecArgs a{};
  a.K = c->K;
  a.V = c->V;
  a.lnmu = c->lnmu;
  a.seg_off = c->seg_off;
  a.seg_len = c->seg_len;
  a.Kt = K_tail;
  a.Vt = V_tail;
  a.Q = Q;
  a.S = c->n_seq;
  a.Ly = c->n_layers;
  a.H = c->n_kv_heads;
  a.G = group;
  a.t_valid = t_valid;
  a.t_cap = t_cap;
  a.nchunk = nchunk_of(c, t_cap);
  a.scale2 = 1.4426950408889634f / sqrtf((float)c->head_dim);
  int64_t units = (int64_t)a.S * a.Ly * a.H;
  float* part = (float*)ws;
  dim3 grid((unsigned)(units * a.nchunk));
  int d = c->head_dim;
  if (c->dtype == KVC_BF16) {
    if (d == 128) hipLaunchKernelGGL((decode_partial_kernel<uint16_t, 128>), grid, dim3(THREADS), 0, st, a, part);
    else hipLaunchKernelGGL((decode_partial_kernel<uint16_t, 64>), grid, dim3(THREADS), 0, st, a, part);
  } else {
    if (d == 128) hipLaunchKernelGGL((decode_partial_kernel<float, 128>), grid, dim3(THREADS), 0, st, a, part);
    else hipLaunchKernelGGL((decode_partial_kernel<float, 64>), grid, dim3(THREADS), 0, st, a, part);
  }
  KVC_LAUNCH_CHECK("decode_partial");
  dim3 cg((unsigned)(a.S * a.H * group));
  if (d == 128) hipLaunchKernelGGL((decode_combine_kernel<128>), cg, dim3(128), 0, st, a, part, x_out, x_stride, o_out);
  else hipLaunchKernelGGL((decode_combine_kernel<64>), cg, dim3(64), 0, st, a, part, x_out, x_stride, o_out);
  KVC_LAUNCH_CHECK("decode_combine");
  return KVC_OK;
}
