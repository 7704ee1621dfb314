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
  typedef uint4 Raw;   // 8 bf16 in 4 registers
  static __device__ __forceinline__ Raw raw(const uint16_t* p) { return *(const uint4*)p; }
  static __device__ __forceinline__ void cvt(const Raw& u, float* f) {
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void load(const uint16_t* p, float* f) { cvt(raw(p), f); }
};
template <> struct Vec8<float> {
  struct Raw { float4 a, b; };
  static __device__ __forceinline__ Raw raw(const float* p) { return Raw{*(const float4*)p, *(const float4*)(p + 4)}; }
  static __device__ __forceinline__ void cvt(const Raw& r, float* f) {
    f[0] = r.a.x; f[1] = r.a.y; f[2] = r.a.z; f[3] = r.a.w;
    f[4] = r.b.x; f[5] = r.b.y; f[6] = r.b.z; f[7] = r.b.w;
  }
  static __device__ __forceinline__ void load(const float* p, float* f) { cvt(raw(p), f); }
};

// partial layout: [unit][chunk][G][D + 2] = o[D], max2, sum
template <class T, int D, int G>
__global__ __launch_bounds__(THREADS) void decode_partial_kernel(DecArgs a, float* part) {
  constexpr int LPE = D / 8;       // lanes per entry
  constexpr int EPI = 64 / LPE;    // entries per wave iteration
  constexpr int STEP = 4 * EPI;    // entries per workgroup iteration
  constexpr int ITER = CHUNK / STEP;
  __shared__ float z_s[G][CHUNK];
  __shared__ float m_s[G], l_s[G];
  __shared__ float o_s[4][G][D];
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
  // query slice of every head of the group for this lane's 8 dims
  float q[G][8];
  const T* Qb = (const T*)a.Q + (((int64_t)s * a.Ly + l) * a.H * G + (int64_t)h * G) * D + sub * 8;
#pragma unroll
  for (int g = 0; g < G; ++g) Vec8<T>::load(Qb + (int64_t)g * D, q[g]);
  // phase 1: logits; every lane issues all of its K loads before using them
  typename Vec8<T>::Raw kraw[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    int e = it * STEP + wave * EPI + slot;
    if (e < n) kraw[it] = Vec8<T>::raw(Kb + (int64_t)e * D + sub * 8);
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    int e = it * STEP + wave * EPI + slot;
    bool ok = e < n;
    float bias = (ok && lm) ? lm[e] * LOG2E : 0.f;
    float kf[8];
    Vec8<T>::cvt(kraw[it], kf);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float dsum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) dsum += q[g][j] * (ok ? kf[j] : 0.f);
#pragma unroll
      for (int o = LPE / 2; o > 0; o >>= 1) dsum += __shfl_xor(dsum, o, 64);
      if (sub == 0) z_s[g][e] = ok ? dsum * a.scale2 + bias : -INFINITY;
    }
  }
  // V loads go out before the softmax barrier
  typename Vec8<T>::Raw vraw[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    int e = it * STEP + wave * EPI + slot;
    if (e < n) vraw[it] = Vec8<T>::raw(Vb + (int64_t)e * D + sub * 8);
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
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[g][j] = 0.f;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    int e = it * STEP + wave * EPI + slot;
    if (e < n) {
      float vf[8];
      Vec8<T>::cvt(vraw[it], vf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float p = z_s[g][e];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[g][j] += p * vf[j];
      }
    }
  }
  // reduce over the wave's entry slots (lanes sharing `sub`)
#pragma unroll
  for (int g = 0; g < G; ++g) {
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

// Merge the chunks of every (s, l, h): one workgroup of G*D threads per unit;
// o[s][l][h*G+g][d] normalized.
template <int D>
__global__ __launch_bounds__(1024) void decode_merge_kernel(DecArgs a, const float* part, float* o) {
  const int G = a.G;
  const int unit = blockIdx.x;                         // (s*Ly + l)*H + h
  const int g = threadIdx.x / D, dd = threadIdx.x % D;
  if (g >= G) return;
  const int64_t slen = a.seg_len[unit];
  const int nseg = min((int)((slen + CHUNK - 1) / CHUNK), a.nchunk - (a.t_cap + CHUNK - 1) / CHUNK);
  const int ntail = (a.t_valid + CHUNK - 1) / CHUNK;
  float m = -INFINITY, sum = 0.f, acc = 0.f;
  const int nc = nseg + ntail;
  constexpr int BATCH = 8;
  for (int c0 = 0; c0 < nc; c0 += BATCH) {
    float mc[BATCH], lc[BATCH], oc[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      mc[q] = -INFINITY;
      lc[q] = oc[q] = 0.f;
      if (c0 + q < nc) {
        const float* pb = part + (((int64_t)unit * a.nchunk + c0 + q) * G + g) * (D + 2);
        mc[q] = pb[D];
        lc[q] = pb[D + 1];
        oc[q] = pb[dd];
      }
    }
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      if (mc[q] == -INFINITY) continue;
      float mn = fmaxf(m, mc[q]);
      float f1 = exp2f(m - mn), f2 = exp2f(mc[q] - mn);
      sum = sum * f1 + lc[q] * f2;
      acc = acc * f1 + oc[q] * f2;
      m = mn;
    }
  }
  o[((int64_t)unit * G + g) * D + dd] = sum > 0.f ? acc / sum : 0.f;
}

// x[s][j] = sum over layers (in order) of o[s][l][j], j < H*G*D
__global__ void decode_layersum_kernel(DecArgs a, int D, const float* o, float* x_out, int64_t x_stride) {
  const int64_t HGD = (int64_t)a.H * a.G * D;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.S * HGD) return;
  int s = (int)(i / HGD);
  int64_t j = i % HGD;
  float x = 0.f;
  for (int l = 0; l < a.Ly; ++l) x += o[((int64_t)s * a.Ly + l) * HGD + j];
  x_out[(int64_t)s * x_stride + j] = x;
}

int nchunk_of(const kvc_ragged* c, int t_cap) {
  return (c->max_seg + CHUNK - 1) / CHUNK + (t_cap + CHUNK - 1) / CHUNK;
}

}  // namespace

extern "C" size_t kvc_decode_workspace(const kvc_ragged* c, int32_t group, int32_t t_cap) {
  if (!c || group < 1 || t_cap < 0 || c->max_seg < 0) return 0;
  int64_t units = (int64_t)c->n_seq * c->n_layers * c->n_kv_heads;
  kvc::Carver cv(nullptr, 0);
  cv.take<float>((size_t)units * nchunk_of(c, t_cap) * group * (c->head_dim + 2));
  cv.take<float>((size_t)units * group * c->head_dim);
  return cv.off + 256;
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
  kvc::Carver cv(ws, ws_bytes);
  float* part = cv.take<float>((size_t)units * a.nchunk * group * (c->head_dim + 2));
  float* obuf = o_out ? o_out : cv.take<float>((size_t)units * group * c->head_dim);
  dim3 grid((unsigned)(units * a.nchunk));
  int d = c->head_dim;
#define KVC_DEC(TT, DD, GG) hipLaunchKernelGGL((decode_partial_kernel<TT, DD, GG>), grid, dim3(THREADS), 0, st, a, part)
#define KVC_DEC_G(TT, DD)                      \
  switch (group) {                             \
    case 1: KVC_DEC(TT, DD, 1); break;         \
    case 2: KVC_DEC(TT, DD, 2); break;         \
    case 4: KVC_DEC(TT, DD, 4); break;         \
    default: KVC_DEC(TT, DD, 8); break;        \
  }
  KVC_REQUIRE(group == 1 || group == 2 || group == 4 || group == 8, KVC_E_UNSUPPORTED,
              "kvc_decode_attn: group must be 1, 2, 4 or 8");
  if (c->dtype == KVC_BF16) {
    if (d == 128) { KVC_DEC_G(uint16_t, 128); } else { KVC_DEC_G(uint16_t, 64); }
  } else {
    if (d == 128) { KVC_DEC_G(float, 128); } else { KVC_DEC_G(float, 64); }
  }
#undef KVC_DEC_G
#undef KVC_DEC
  KVC_LAUNCH_CHECK("decode_partial");
  if (d == 128)
    hipLaunchKernelGGL((decode_merge_kernel<128>), dim3((unsigned)units), dim3(group * 128), 0, st, a, part, obuf);
  else
    hipLaunchKernelGGL((decode_merge_kernel<64>), dim3((unsigned)units), dim3(group * 64), 0, st, a, part, obuf);
  KVC_LAUNCH_CHECK("decode_merge");
  int64_t nx = (int64_t)a.S * a.H * group * d;
  hipLaunchKernelGGL(decode_layersum_kernel, dim3(kvc_blocks(nx, 256)), dim3(256), 0, st, a, d, obuf, x_out, x_stride);
  KVC_LAUNCH_CHECK("decode_layersum");
  return KVC_OK;
}
