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
#include "mfma_frag.h"

namespace {

constexpr int CHUNK = 256;   // entries per workgroup, fp32 caches (VALU kernel)
constexpr int MCHUNK = 512;  // entries per workgroup, bf16 caches (MFMA kernel)
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
  int chunk;     // entries per partial (CHUNK or MCHUNK)
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

// bf16 caches: the logits of a 32-entry group come from one MFMA chain
// (A = the G query heads padded to 32 rows, B = the entries' keys), each wave
// runs an online softmax over rounds of 64 entries, and the values are
// accumulated on the VALU with the probabilities broadcast through LDS.
// Partial layout as the VALU kernel: [unit][chunk][G][D + 2].
template <int D, int G>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(G == 8 ? 2 : 3))) void decode_mfma_kernel(DecArgs a, float* part) {
  using namespace kvcmf;
  constexpr int KS = D / 16;          // MFMA steps per group (16 dims each)
  constexpr int LPE = D / 8;          // lanes per entry in the value pass
  constexpr int EPI = 64 / LPE;       // entries per value iteration
  constexpr int VIT = 32 / EPI;       // value iterations per 32-entry round
  constexpr int WE = MCHUNK / 4;      // entries per wave
  constexpr int GP = G < 4 ? G : 4;   // heads held per logit lane
  constexpr int PS = G <= 4 ? 4 : 8;  // row stride of the probability table
  __shared__ __align__(16) uint16_t qs[G][D];
  __shared__ __align__(16) float pw[4][32][PS];
  __shared__ float mw[4][G], lw[4][G];
  __shared__ __align__(16) float ow[4][G][D];
  const int unit = blockIdx.x / a.nchunk, chunk = blockIdx.x % a.nchunk;
  const int s = unit / (a.Ly * a.H), lh = unit % (a.Ly * a.H);
  const int l = lh / a.H, h = lh % a.H;
  const int seg_idx = (s * a.Ly + l) * a.H + h;
  const int64_t slen = a.seg_len[seg_idx];
  const int nseg = min((int)((slen + MCHUNK - 1) / MCHUNK), a.nchunk - (a.t_cap + MCHUNK - 1) / MCHUNK);
  const uint16_t* Kb;
  const uint16_t* Vb;
  const float* lm = nullptr;
  int64_t n;
  if (chunk < nseg) {
    const int64_t off = a.seg_off[seg_idx], e0 = (int64_t)chunk * MCHUNK;
    n = slen - e0 < MCHUNK ? slen - e0 : MCHUNK;
    Kb = (const uint16_t*)a.K + (off + e0) * D;
    Vb = (const uint16_t*)a.V + (off + e0) * D;
    if (a.lnmu) lm = a.lnmu + off + e0;
  } else {
    const int64_t e0 = (int64_t)(chunk - nseg) * MCHUNK;
    if (e0 >= a.t_valid) return;
    n = a.t_valid - e0 < MCHUNK ? a.t_valid - e0 : MCHUNK;
    const int64_t tb = (((int64_t)l * a.H + h) * a.S + s) * a.t_cap + e0;
    Kb = (const uint16_t*)a.Kt + tb * D;
    Vb = (const uint16_t*)a.Vt + tb * D;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int es = lane / LPE, sub = lane % LPE;
  {
    const uint16_t* Qb = (const uint16_t*)a.Q + (((int64_t)s * a.Ly + l) * a.H * G + (int64_t)h * G) * D;
    for (int i = threadIdx.x; i < G * D / 8; i += THREADS) *(uint4*)&qs[0][i * 8] = *(const uint4*)(Qb + i * 8);
  }
  float m[GP], lsum[GP], acc[G][8];
#pragma unroll
  for (int j = 0; j < GP; ++j) {
    m[j] = -INFINITY;
    lsum[j] = 0.f;
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[g][j] = 0.f;
  __syncthreads();
  const int wbase = wave * WE;
  // Rounds of 32 entries; many waves per SIMD hide the load latency. Loads
  // past the chunk read its last entry (always valid) and are masked
  // afterwards, so no load sits behind a branch.
  const float* lmp = lm ? lm : (const float*)Kb;
#pragma unroll 1
  for (int rb = wbase; rb < wbase + WE && rb < n; rb += 32) {  // a wave past the entries only joins the combine
    const int ek = rb + col, ekc = min(ek, (int)n - 1);
    const float bv = lmp[ekc];  // unconditional, selected away without ln mu
    uint4 kr[KS], vr[VIT];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kr[ks] = *(const uint4*)(Kb + (int64_t)ekc * D + half * (D / 2) + ks * 8);
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int e = min(rb + it * EPI + es, (int)n - 1);
      vr[it] = *(const uint4*)(Vb + (int64_t)e * D + sub * 8);
    }
    const float bias = lm ? bv * LOG2E : 0.f;
    // logits on MFMA: A = query heads (rows, zero past G), B = keys (columns);
    // lane (half, col) receives heads 4*half + j of entry col; lane half
    // `half` holds the dims [half*D/2, half*D/2 + D/2) in 8-wide steps
    kvc_f32x16 sacc = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Frag<uint16_t> qf, kf;
      qf = col < G ? load_frag<uint16_t>(&qs[col < G ? col : 0][half * (D / 2) + ks * 8]) : zero_frag<uint16_t>();
      kf.v = __builtin_bit_cast(kvc_bf16x8, kr[ks]);
      mma(sacc, qf, kf);
    }
    // online softmax: new running max per head over the 32 lanes of a half
#pragma unroll
    for (int j = 0; j < GP; ++j) {
      const bool ok = ek < n && 4 * half + j < G;
      const float z = ok ? sacc[j] * a.scale2 + bias : -INFINITY;
      float mx = z;
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float mn = fmaxf(m[j], mx);
      const float ea = fast_exp2(m[j] - mn), ep = fast_exp2(z - mn);
      const float alpha = mn == -INFINITY ? 1.f : ea;
      m[j] = mn;
      const float p = mn == -INFINITY ? 0.f : ep;
      lsum[j] = lsum[j] * alpha + p;
      if (4 * half + j < G) pw[wave][col][4 * half + j] = p;
      // every lane rescales its value sums of the heads this (half, j) holds
#pragma unroll
      for (int hh = 0; hh < (G + 3) / 4; ++hh) {
        if (4 * hh + j >= G) continue;
        const float f = __shfl(alpha, hh * 32, 64);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[4 * hh + j][q] *= f;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int el = it * EPI + es;
      float vf[8];
      const uint32_t w4[4] = {vr[it].x, vr[it].y, vr[it].z, vr[it].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        vf[2 * q] = __uint_as_float(w4[q] << 16);
        vf[2 * q + 1] = __uint_as_float(w4[q] & 0xffff0000u);
      }
      float pg[G];
      if constexpr (G >= 4) {
#pragma unroll
        for (int g4 = 0; g4 < G; g4 += 4) {
          const float4 t = *(const float4*)&pw[wave][el][g4];
          pg[g4] = t.x; pg[g4 + 1] = t.y; pg[g4 + 2] = t.z; pg[g4 + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) pg[g] = pw[wave][el][g];
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[g][q] = fmaf(pg[g], vf[q], acc[g][q]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the next round rewrites pw
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // wave totals: probability sums over the 32 lanes of a half, value sums over
  // the lanes that share `sub`
#pragma unroll
  for (int j = 0; j < GP; ++j) {
    float t = lsum[j];
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) t += __shfl_xor(t, o, 64);
    lsum[j] = t;
  }
  if (col == 0) {
#pragma unroll
    for (int j = 0; j < GP; ++j)
      if (4 * half + j < G) {
        mw[wave][4 * half + j] = m[j];
        lw[wave][4 * half + j] = lsum[j];
      }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = acc[g][j];
#pragma unroll
      for (int o = LPE; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
      if (es == 0) ow[wave][g][sub * 8 + j] = x;
    }
  __syncthreads();
  float* pb = part + ((int64_t)unit * a.nchunk + chunk) * G * (D + 2);
  for (int i = threadIdx.x; i < G * D; i += THREADS) {
    const int g = i / D, dd = i % D;
    float mx = mw[0][g];
#pragma unroll
    for (int w = 1; w < 4; ++w) mx = fmaxf(mx, mw[w][g]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (mw[w][g] != -INFINITY) o += ow[w][g][dd] * exp2f(mw[w][g] - mx);
    pb[g * (D + 2) + dd] = o;
  }
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float mx = mw[0][g];
#pragma unroll
    for (int w = 1; w < 4; ++w) mx = fmaxf(mx, mw[w][g]);
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (mw[w][g] != -INFINITY) t += lw[w][g] * exp2f(mw[w][g] - mx);
    pb[g * (D + 2) + D] = mx;
    pb[g * (D + 2) + D + 1] = t;
  }
}

// Merge the chunks of every (s, l, h, g): one workgroup of D threads per
// (unit, head). The chunk statistics go to LDS first, the chunk weights
// exp2(m_c - max) and 1 / sum follow from two block reductions, then every
// thread sums its dimension over the chunks with all loads independent.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecArgs a, const float* part, float* o) {
  extern __shared__ float ms[];            // [2][nchunk]: chunk max, then weight; chunk sum
  __shared__ float red[D / 64];
  const int G = a.G;
  const int unit = blockIdx.x / G, g = blockIdx.x % G;  // unit = (s*Ly + l)*H + h
  const int tid = threadIdx.x;
  float* mc = ms;
  float* lc = ms + a.nchunk;
  const int64_t slen = a.seg_len[unit];
  const int ck = a.chunk;
  const int nseg = min((int)((slen + ck - 1) / ck), a.nchunk - (a.t_cap + ck - 1) / ck);
  const int nc = nseg + (a.t_valid + ck - 1) / ck;
  const int64_t cs = (int64_t)G * (D + 2);  // chunk stride
  const float* pb = part + ((int64_t)unit * a.nchunk * G + g) * (D + 2);
  float mx = -INFINITY;
  for (int c = tid; c < nc; c += D) {
    const float m = pb[c * cs + D];
    mc[c] = m;
    lc[c] = pb[c * cs + D + 1];
    mx = fmaxf(mx, m);
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < D / 64; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  float sm = 0.f;
  for (int c = tid; c < nc; c += D) {
    const float w = mc[c] == -INFINITY ? 0.f : exp2f(mc[c] - mx);
    mc[c] = w;
    sm += lc[c] * w;
  }
  sm = wave_sum(sm);
  if ((tid & 63) == 0) red[tid >> 6] = sm;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < D / 64; ++w) tot += red[w];
  float acc = 0.f;
#pragma unroll 8
  for (int c = 0; c < nc; ++c) acc += pb[c * cs + tid] * mc[c];
  o[((int64_t)unit * G + g) * D + tid] = tot > 0.f ? acc / tot : 0.f;
}

// x[s][j] = sum over layers (in order) of o[s][l][j], j < H*G*D
__global__ void decode_layersum_kernel(DecArgs a, int D, const float* o, float* x_out, int64_t x_stride) {
  const int64_t HGD = (int64_t)a.H * a.G * D;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.S * HGD) return;
  int s = (int)(i / HGD);
  int64_t j = i % HGD;
  const float* os = o + (int64_t)s * a.Ly * HGD + j;
  float x = 0.f;
#pragma unroll 8
  for (int l = 0; l < a.Ly; ++l) x += os[(int64_t)l * HGD];
  x_out[(int64_t)s * x_stride + j] = x;
}

int nchunk_of(const kvc_ragged* c, int t_cap, int chunk) {
  return (c->max_seg + chunk - 1) / chunk + (t_cap + chunk - 1) / chunk;
}

}  // namespace

extern "C" size_t kvc_decode_workspace(const kvc_ragged* c, int32_t group, int32_t t_cap) {
  if (!c || group < 1 || t_cap < 0 || c->max_seg < 0) return 0;
  int64_t units = (int64_t)c->n_seq * c->n_layers * c->n_kv_heads;
  kvc::Carver cv(nullptr, 0);
  cv.take<float>((size_t)units * nchunk_of(c, t_cap, CHUNK) * group * (c->head_dim + 2));  // bound for both kernels
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
  a.chunk = c->dtype == KVC_BF16 ? MCHUNK : CHUNK;
  a.nchunk = nchunk_of(c, t_cap, a.chunk);
  a.scale2 = 1.4426950408889634f / sqrtf((float)c->head_dim);
  int64_t units = (int64_t)a.S * a.Ly * a.H;
  kvc::Carver cv(ws, ws_bytes);
  float* part = cv.take<float>((size_t)units * a.nchunk * group * (c->head_dim + 2));
  float* obuf = o_out ? o_out : cv.take<float>((size_t)units * group * c->head_dim);
  dim3 grid((unsigned)(units * a.nchunk));
  int d = c->head_dim;
#define KVC_DEC(TT, DD, GG) hipLaunchKernelGGL((decode_partial_kernel<TT, DD, GG>), grid, dim3(THREADS), 0, st, a, part)
#define KVC_DECM(DD, GG) hipLaunchKernelGGL((decode_mfma_kernel<DD, GG>), grid, dim3(THREADS), 0, st, a, part)
#define KVC_DEC_G(MAC, ...)                    \
  switch (group) {                             \
    case 1: MAC(__VA_ARGS__, 1); break;        \
    case 2: MAC(__VA_ARGS__, 2); break;        \
    case 4: MAC(__VA_ARGS__, 4); break;        \
    default: MAC(__VA_ARGS__, 8); break;       \
  }
  KVC_REQUIRE(group == 1 || group == 2 || group == 4 || group == 8, KVC_E_UNSUPPORTED,
              "kvc_decode_attn: group must be 1, 2, 4 or 8");
  if (c->dtype == KVC_BF16) {
    if (d == 128) { KVC_DEC_G(KVC_DECM, 128); } else { KVC_DEC_G(KVC_DECM, 64); }
  } else {
    if (d == 128) { KVC_DEC_G(KVC_DEC, float, 128); } else { KVC_DEC_G(KVC_DEC, float, 64); }
  }
#undef KVC_DEC_G
#undef KVC_DECM
#undef KVC_DEC
  KVC_LAUNCH_CHECK("decode_partial");
  const size_t msm = (size_t)2 * a.nchunk * sizeof(float);
  if (d == 128)
    hipLaunchKernelGGL((decode_merge_kernel<128>), dim3((unsigned)(units * group)), dim3(128), msm, st, a, part, obuf);
  else
    hipLaunchKernelGGL((decode_merge_kernel<64>), dim3((unsigned)(units * group)), dim3(64), msm, st, a, part, obuf);
  KVC_LAUNCH_CHECK("decode_merge");
  int64_t nx = (int64_t)a.S * a.H * group * d;
  hipLaunchKernelGGL(decode_layersum_kernel, dim3(kvc_blocks(nx, 256)), dim3(256), 0, st, a, d, obuf, x_out, x_stride);
  KVC_LAUNCH_CHECK("decode_layersum");
  return KVC_OK;
}
