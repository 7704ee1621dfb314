// Probe attention (scores + features) and token-to-token propagation.
//
// Both are "a set of query rows attends over one unit's keys, then every key
// collects a weighted column sum of the softmax". GraceKV page, '03 Bottom-up
// value flow' (direct probe relevance, then two hops of propagation);
// DistillCache paper, Sec. 3.1.1 (per-token features).
//
// Two passes per unit (the softmax needs each row's log-partition before any
// column can be summed):
//   rowstats: split-K over the keys; per row an online (max, sum 2^x, sum 2^x x)
//             in base-2 logits; partials merged by rowcombine.
//   colsum:   recompute the logits, p = 2^(x - lse2_row), column sums.
// The QK^T tiles run on MFMA (bf16: v_mfma_f32_32x32x16_bf16, fp32 inputs:
// v_mfma_f32_32x32x2f32). The query rows of the unit sit in LDS in fragment
// order; every wave streams its own 32-key blocks from HBM straight into
// registers. In rowstats the MFMA computes K Q^T so a lane owns one query row
// (its statistics never leave the lane); in colsum it computes Q K^T so a
// lane owns one key (its column sums never leave the lane pair).
#include <algorithm>
#include <cmath>

#include "kvc_internal.h"

namespace {

constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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
// acc += A(32 x 16) * B(16 x 32); lane l holds A[l%32][8(l/32)..+8) and
// B[8(l/32)..+8)[l%32] (the same k permutation on both sides).
__device__ __forceinline__ void mma(kvc_f32x16& acc, const Frag<uint16_t>& a, const Frag<uint16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(kvc_f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[j], b.v[j], acc, 0, 0, 0);
}
// row (within a 32-block) of accumulator register v for lane l
__device__ __forceinline__ int acc_row(int v, int lane) { return (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3); }

struct AttnArgs {
  const void* K;          // [Ly][H][T][d]
  const void* V;          // score: [Ly][H][T][d]
  const void* Q;          // score: Qprobe [S][Ly][H*G][P][d]; prop: Qctx [Ly][H*G][T][d]
  const int64_t* cu;      // device cu_seqlens
  const int32_t* seeds;   // prop: [S][Ly][H][M]
  const float* prev;      // prop: delta_{t-1} [Ly][H][T]
  int S, Ly, H, G, P, M;
  int64_t T;
  int R, Rpad;            // query rows per unit and rows rounded up to 32
  int KW;                 // keys per workgroup (multiple of 32*WAVES)
  float scale2;           // log2(e) / sqrt(d)
  float hop_w;            // prop: w / G
  int accumulate;         // prop: add this call's increments to delta (row blocks of the dense rollout)
  const float* kval;      // "A r" pass: a scalar value per key (delta_{t-1}) averaged by each row's softmax
  float* part_v;          // "A r" pass: per split and row, the value sum at the split's max
};

// Largest seed position of a unit (-1 if none): keys past it see no row.
__device__ __forceinline__ int max_seed(const AttnArgs& a, int unit) {
  int m = -1;
  for (int k = 0; k < a.M; ++k) m = max(m, a.seeds[(int64_t)unit * a.M + k]);
  return m;
}

struct Work {
  int s, l, h, split, ns;
  int64_t L, k0, k1, tok0;  // tok0 = cu[s]
  int unit;                 // (s*Ly + l)*H + h
};

// Workgroup -> (sequence, layer, head, split). Sequences are few (<= tens),
// so each workgroup walks cu once.
__device__ __forceinline__ Work decode_work(const AttnArgs& a, int64_t b) {
  Work w;
  int64_t base = 0;
  for (int s = 0; s < a.S; ++s) {
    int64_t L = a.cu[s + 1] - a.cu[s];
    int64_t ns = (L + a.KW - 1) / a.KW;
    int64_t n = ns * a.Ly * a.H;
    if (b < base + n) {
      int64_t r = b - base;
      int lh = (int)(r / ns);
      w.s = s;
      w.l = lh / a.H;
      w.h = lh % a.H;
      w.split = (int)(r % ns);
      w.ns = (int)ns;
      w.L = L;
      w.k0 = (int64_t)w.split * a.KW;
      w.k1 = w.k0 + a.KW < L ? w.k0 + a.KW : L;
      w.tok0 = a.cu[s];
      w.unit = (s * a.Ly + w.l) * a.H + w.h;
      return w;
    }
    base += n;
  }
  w.s = -1;
  return w;
}

// Stage the unit's query rows in LDS in fragment order:
// frag (rb, ks, lane) = row rb*32 + lane%32, elements [16 ks + 8 (lane/32), +8).
template <class T, int D>
__device__ void stage_rows(const AttnArgs& a, const Work& w, int mode, Frag<T>* qf, int* lim_s) {
  constexpr int KS = D / 16;
  const T* Q = (const T*)a.Q;
  int nchunk = a.Rpad * (D / 8);
  for (int c = threadIdx.x; c < nchunk; c += THREADS) {
    int row = c / (D / 8);
    int col8 = c % (D / 8);
    const T* src = nullptr;
    if (row < a.R) {
      if (mode == 0) {
        int g = row / a.P, p = row % a.P;
        src = Q + ((((int64_t)w.s * a.Ly + w.l) * a.H * a.G + (int64_t)w.h * a.G + g) * a.P + p) * D;
      } else {
        int k = row / a.G, g = row % a.G;
        int j = a.seeds[(int64_t)w.unit * a.M + k];
        if (j >= 0)
          src = Q + (((int64_t)w.l * a.H * a.G + (int64_t)w.h * a.G + g) * a.T + w.tok0 + j) * D;
      }
    }
    int rb = row >> 5, ks = col8 >> 1, lane = (row & 31) + 32 * (col8 & 1);
    qf[(rb * KS + ks) * 64 + lane] = src ? load_frag<T>(src + col8 * 8) : zero_frag<T>();
  }
  if (lim_s) {
    for (int r = threadIdx.x; r < a.Rpad; r += THREADS) {
      int lim = -1;
      if (r < a.R) {
        if (mode == 0) lim = 0x7fffffff;
        else lim = a.seeds[(int64_t)w.unit * a.M + r / a.G];
      }
      lim_s[r] = lim;
    }
  }
}

// ------------------------------------------------------------------ pass 1
template <class T, int D, bool VAL = false>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 4 : 2))) void rowstats_kernel(
    AttnArgs a, int mode, float* part) {
  constexpr int KS = D / 16;
  extern __shared__ __align__(16) char smem[];
  Frag<T>* qf = (Frag<T>*)smem;
  int* lim_s = (int*)(smem + (size_t)a.Rpad * D * sizeof(T));
  float* red = (float*)smem;  // [WAVES][Rpad][3] (+ [WAVES][Rpad]), over the staged rows once the keys are done
  Work w = decode_work(a, blockIdx.x);
  if (w.s < 0) return;
  if (mode == 1 && w.k0 > max_seed(a, w.unit)) {
    // no row reaches this split's keys: an empty partial
    for (int r = threadIdx.x; r < a.Rpad; r += THREADS) {
      float* o = part + ((size_t)blockIdx.x * a.Rpad + r) * 3;
      o[0] = -INFINITY;
      o[1] = 0.f;
      o[2] = 0.f;
      if constexpr (VAL) a.part_v[(size_t)blockIdx.x * a.Rpad + r] = 0.f;
    }
    return;
  }
  stage_rows<T, D>(a, w, mode, qf, lim_s);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nrb = a.Rpad >> 5;
  float m[8], sm[8], tt[8], vv[8];
  int minlim[8], maxl[8];  // the smallest and the largest last key over each row block
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) {
    m[rb] = -INFINITY;
    sm[rb] = 0.f;
    tt[rb] = 0.f;
    vv[rb] = 0.f;
    int mnl = rb < nrb ? lim_s[rb * 32 + (lane & 31)] : -1, mxl = mnl;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) {
      mnl = min(mnl, __shfl_xor(mnl, o, 64));
      mxl = max(mxl, __shfl_xor(mxl, o, 64));
    }
    minlim[rb] = __builtin_amdgcn_readfirstlane(mnl);
    maxl[rb] = __builtin_amdgcn_readfirstlane(mxl);
  }
  int maxlim = -1;
  for (int r = 0; r < a.Rpad; ++r) maxlim = max(maxlim, lim_s[r]);
  const T* K = (const T*)a.K + (((int64_t)w.l * a.H + w.h) * a.T + w.tok0) * D;
  for (int64_t kb = w.k0 + wave * 32; kb < w.k1; kb += WAVES * 32) {
    if (kb > maxlim) break;
    int64_t key = kb + (lane & 31);
    Frag<T> kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = key < w.k1 ? load_frag<T>(K + key * D + ks * 16 + 8 * (lane >> 5)) : zero_frag<T>();
    // "A r" pass: the values of the 16 keys a lane's registers hold (clamped
    // into the sequence; masked keys get zero weight)
    float dv[VAL ? 16 : 1];
    if constexpr (VAL) {
      const float* kv = a.kval + ((int64_t)w.l * a.H + w.h) * a.T + w.tok0;
#pragma unroll
      for (int v = 0; v < 16; ++v) dv[v] = kv[min(kb + acc_row(v, lane), w.k1 - 1)];
    }
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
      if (rb >= nrb) break;
      if (kb > maxl[rb]) continue;   // no row of the block sees these keys (seed rows ascend by position)
      kvc_f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) mma(acc, kf[ks], qf[(rb * KS + ks) * 64 + lane]);
      // lane owns query row rb*32 + lane%32; register v holds key kb + acc_row(v)
      if (!VAL && kb + 31 < w.k1 && kb + 31 <= minlim[rb]) {
        // every key of the block is visible to every row of the block: no
        // masks; the maximum of the raw products scales to the logits' (the
        // scale is positive), and 2^x x is summed as 2^x times the raw product
        float mx = acc[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, acc[v]);
        const float mn = fmaxf(m[rb], mx * a.scale2);
        const float f = fast_exp2(m[rb] - mn);
        float s2 = 0.f, t2 = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float e = fast_exp2(fmaf(acc[v], a.scale2, -mn));
          s2 += e;
          t2 = fmaf(e, acc[v], t2);
        }
        sm[rb] = fmaf(sm[rb], f, s2);
        tt[rb] = fmaf(tt[rb], f, t2 * a.scale2);
        m[rb] = mn;
        continue;
      }
      float x[16];
      float mx = -INFINITY;
      const int lim = lim_s[rb * 32 + (lane & 31)];  // this lane's row's last key
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        int64_t kk = kb + acc_row(v, lane);
        bool ok = kk < w.k1 && kk <= lim;
        x[v] = ok ? acc[v] * a.scale2 : -INFINITY;
        mx = fmaxf(mx, x[v]);
      }
      if (mx == -INFINITY) continue;
      float mn = fmaxf(m[rb], mx);
      float f = fast_exp2(m[rb] - mn);
      float s2 = 0.f, t2 = 0.f, v2 = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float e = fast_exp2(x[v] - mn);
        s2 += e;
        t2 += x[v] == -INFINITY ? 0.f : e * x[v];
        if constexpr (VAL) v2 += e * dv[v];
      }
      sm[rb] = sm[rb] * f + s2;
      tt[rb] = tt[rb] * f + t2;
      if constexpr (VAL) vv[rb] = vv[rb] * f + v2;
      m[rb] = mn;
    }
  }
  __syncthreads();  // every wave is done with the staged rows: the merge area overwrites them
  // merge the lane pair (l, l+32) that shares a row, then the waves
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) {
    if (rb >= nrb) break;
    float m2 = __shfl_xor(m[rb], 32, 64), s2 = __shfl_xor(sm[rb], 32, 64), t2 = __shfl_xor(tt[rb], 32, 64);
    float v2 = VAL ? __shfl_xor(vv[rb], 32, 64) : 0.f;
    float mn = fmaxf(m[rb], m2);
    if (mn != -INFINITY) {
      float f1 = exp2f(m[rb] - mn), f2 = exp2f(m2 - mn);
      sm[rb] = sm[rb] * f1 + s2 * f2;
      tt[rb] = tt[rb] * f1 + t2 * f2;
      if constexpr (VAL) vv[rb] = vv[rb] * f1 + v2 * f2;
    }
    m[rb] = mn;
    if (lane < 32) {
      float* r = red + ((size_t)wave * a.Rpad + rb * 32 + lane) * 3;
      r[0] = m[rb];
      r[1] = sm[rb];
      r[2] = tt[rb];
      if constexpr (VAL) red[(size_t)WAVES * a.Rpad * 3 + (size_t)wave * a.Rpad + rb * 32 + lane] = vv[rb];
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < a.Rpad; r += THREADS) {
    float mm = -INFINITY, ss = 0.f, ts = 0.f, vs = 0.f;
    for (int wv = 0; wv < WAVES; ++wv) {
      const float* q = red + ((size_t)wv * a.Rpad + r) * 3;
      float mn = fmaxf(mm, q[0]);
      if (mn == -INFINITY) continue;
      float f1 = exp2f(mm - mn), f2 = exp2f(q[0] - mn);
      ss = ss * f1 + q[1] * f2;
      ts = ts * f1 + q[2] * f2;
      if constexpr (VAL) vs = vs * f1 + red[(size_t)WAVES * a.Rpad * 3 + (size_t)wv * a.Rpad + r] * f2;
      mm = mn;
    }
    float* o = part + ((size_t)blockIdx.x * a.Rpad + r) * 3;
    o[0] = mm;
    o[1] = ss;
    o[2] = ts;
    if constexpr (VAL) a.part_v[(size_t)blockIdx.x * a.Rpad + r] = vs;
  }
}

// "A r" pass: merge the split partials of every (unit, row) into the row's
// softmax average of the key values, then hand w/G of the G rows of each
// position to that position (every position lies in exactly one row block).
__global__ void rowval_kernel(AttnArgs a, const float* part, int64_t block, float* cur, float* rel) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_units = (int64_t)a.S * a.Ly * a.H;
  if (i >= n_units * a.M) return;
  const int64_t unit = i / a.M;
  const int k = (int)(i % a.M);
  const int s = (int)(unit / ((int64_t)a.Ly * a.H));
  const int lh = (int)(unit % ((int64_t)a.Ly * a.H));
  const int64_t L = a.cu[s + 1] - a.cu[s];
  const int64_t pos = block * a.M + k;
  if (pos >= L) return;
  int64_t base = 0, ns = 0;
  for (int q = 0; q <= s; ++q) {
    const int64_t Lq = a.cu[q + 1] - a.cu[q];
    ns = (Lq + a.KW - 1) / a.KW;
    if (q < s) base += ns * a.Ly * a.H;
  }
  base += (int64_t)lh * ns;
  float tot = 0.f;
  for (int g = 0; g < a.G; ++g) {
    const int r = k * a.G + g;
    float mm = -INFINITY, ss = 0.f, vs = 0.f;
    for (int64_t sp = 0; sp < ns; ++sp) {
      const float* q = part + ((base + sp) * a.Rpad + r) * 3;
      const float mn = fmaxf(mm, q[0]);
      if (mn == -INFINITY) continue;
      const float f1 = exp2f(mm - mn), f2 = exp2f(q[0] - mn);
      ss = ss * f1 + q[1] * f2;
      vs = vs * f1 + a.part_v[(base + sp) * a.Rpad + r] * f2;
      mm = mn;
    }
    tot += ss > 0.f ? vs / ss : 0.f;
  }
  const int64_t tix = (int64_t)lh * a.T + a.cu[s] + pos;
  const float d = a.hop_w * tot;
  cur[tix] = d;
  rel[tix] += d;
}

// Merge the split partials of each (unit, row): lse2 (base 2) and H.
__global__ void rowcombine_kernel(AttnArgs a, const float* part, float2* rowstat, float* lse_out,
                                  float* ent_out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t n_units = (int64_t)a.S * a.Ly * a.H;
  if (i >= n_units * a.Rpad) return;
  int64_t unit = i / a.Rpad;
  int r = (int)(i % a.Rpad);
  int s = (int)(unit / ((int64_t)a.Ly * a.H));
  int lh = (int)(unit % ((int64_t)a.Ly * a.H));
  // first split of this unit
  int64_t base = 0;
  int64_t ns = 0;
  for (int q = 0; q <= s; ++q) {
    int64_t L = a.cu[q + 1] - a.cu[q];
    ns = (L + a.KW - 1) / a.KW;
    if (q < s) base += ns * a.Ly * a.H;
  }
  base += (int64_t)lh * ns;
  float mm = -INFINITY, ss = 0.f, ts = 0.f;
  for (int64_t k = 0; k < ns; ++k) {
    const float* q = part + ((base + k) * a.Rpad + r) * 3;
    float mn = fmaxf(mm, q[0]);
    if (mn == -INFINITY) continue;
    float f1 = exp2f(mm - mn), f2 = exp2f(q[0] - mn);
    ss = ss * f1 + q[1] * f2;
    ts = ts * f1 + q[2] * f2;
    mm = mn;
  }
  float lse2 = mm == -INFINITY ? -INFINITY : mm + log2f(ss);
  float H = mm == -INFINITY ? 0.f : LN2 * (lse2 - ts / ss);
  rowstat[i] = make_float2(lse2, H);
  if (lse_out && r < a.R) {
    lse_out[unit * a.R + r] = lse2 * LN2;
    ent_out[unit * a.R + r] = H;
  }
}

// ------------------------------------------------------------------ pass 2
template <class T, int D, int MODE>
__global__ __launch_bounds__(THREADS) void colsum_kernel(AttnArgs a, const float2* rowstat,
                                                          float* out0, float* feats, float* head_part,
                                                          const float* rel_in, float* rel_out) {
  constexpr int mode = MODE;
  constexpr int KS = D / 16;
  extern __shared__ __align__(16) char smem[];
  Frag<T>* qf = (Frag<T>*)smem;
  int* lim_s = (int*)(smem + (size_t)a.Rpad * D * sizeof(T));
  float* lse_s = (float*)(lim_s + a.Rpad);
  float* ent_s = lse_s + a.Rpad;
  float* w_s = ent_s + a.Rpad;
  float* hred = w_s + a.Rpad;  // [WAVES][2]
  Work w = decode_work(a, blockIdx.x);
  if (w.s < 0) return;
  // accumulating calls add nothing to keys past every row
  if (MODE == 1 && a.accumulate && w.k0 > max_seed(a, w.unit)) return;
  stage_rows<T, D>(a, w, mode, qf, lim_s);
  for (int r = threadIdx.x; r < a.Rpad; r += THREADS) {
    float2 st = rowstat[(int64_t)w.unit * a.Rpad + r];
    lse_s[r] = st.x;
    ent_s[r] = st.y;
    float wt = 1.f;
    if (mode == 1) {
      wt = 0.f;
      if (r < a.R) {
        int j = a.seeds[(int64_t)w.unit * a.M + r / a.G];
        if (j >= 0) wt = a.hop_w * a.prev[((int64_t)w.l * a.H + w.h) * a.T + w.tok0 + j];
      }
    }
    w_s[r] = wt;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nrb = a.Rpad >> 5;
  int maxlim = -1;
  for (int r = 0; r < a.Rpad; ++r) maxlim = max(maxlim, lim_s[r]);
  const int64_t ubase = ((int64_t)w.l * a.H + w.h) * a.T + w.tok0;
  const T* K = (const T*)a.K + ubase * D;
  float hs_num = 0.f, hs_den = 0.f;
  // the smallest and the largest last key over each row block (every row of
  // a probe pass sees every key)
  int minlim[8], maxl[8];
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) {
    int mnl = rb < nrb ? lim_s[rb * 32 + (lane & 31)] : -1, mxl = mnl;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) {
      mnl = min(mnl, __shfl_xor(mnl, o, 64));
      mxl = max(mxl, __shfl_xor(mxl, o, 64));
    }
    minlim[rb] = __builtin_amdgcn_readfirstlane(mnl);
    maxl[rb] = __builtin_amdgcn_readfirstlane(mxl);
  }
  // a lane owns one key; past the end it reads the last key (masked by kvalid)
  for (int64_t kb = w.k0 + wave * 32; kb < w.k1; kb += WAVES * 32) {
    int64_t key = kb + (lane & 31);
    bool kvalid = key < w.k1;
    const int64_t keyc = kvalid ? key : w.k1 - 1;
    Frag<T> kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = load_frag<T>(K + keyc * D + ks * 16 + 8 * (lane >> 5));
    float vn = 0.f;
    if constexpr (MODE == 0) {
      // value norm: lanes l and l+32 each sum half of the row
      const T* Vr = (const T*)a.V + (ubase + keyc) * D + (lane >> 5) * (D / 2);
      float vs = 0.f;
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        const Frag<T> vrow = load_frag<T>(Vr + j * 8);
        if constexpr (sizeof(T) == 2) {
          // squares of bf16 pairs summed in fp32 (v_dot2c_f32_bf16)
          const uint4 u = __builtin_bit_cast(uint4, vrow.v);
          const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2_t x = __builtin_bit_cast(bf16x2_t, w4[e]);
            vs = __builtin_amdgcn_fdot2_f32_bf16(x, x, vs, false);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) vs += vrow.v[e] * vrow.v[e];
        }
      }
      if (!kvalid) vs = 0.f;
      vs += __shfl_xor(vs, 32, 64);
      vn = sqrtf(vs);
    }
    float colsum = 0.f, hsum = 0.f;
    float mg[8], csr[8];  // per query head; per row block (fast path, assigned to heads below)
#pragma unroll
    for (int g = 0; g < 8; ++g) mg[g] = csr[g] = 0.f;
    if (kb <= maxlim) {
#pragma unroll
      for (int rb = 0; rb < 8; ++rb) {
        if (rb >= nrb) break;
        if (MODE == 1 && kb > maxl[rb]) continue;   // no row of the block sees these keys: they add 0
        kvc_f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma(acc, qf[(rb * KS + ks) * 64 + lane], kf[ks]);
        // lane owns key `key`; register v holds query row rb*32 + acc_row(v),
        // and registers 4q..4q+3 hold four consecutive rows
        if (kb + 31 < w.k1 && (MODE == 0 || kb + 31 <= minlim[rb]) && (MODE == 1 || a.P % 32 == 0)) {
          // every key of the block is in range for every row of the block: no
          // masks (a probe block lies inside one query head)
          float cs = 0.f, hs = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row0 = rb * 32 + acc_row(q * 4, lane);
            const float4 ls4 = *(const float4*)(lse_s + row0);
            const float4 o4 = *(const float4*)((MODE == 0 ? ent_s : w_s) + row0);
            const float lsv[4] = {ls4.x, ls4.y, ls4.z, ls4.w}, ov[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
            for (int vv = 0; vv < 4; ++vv) {
              const float p = fast_exp2(fmaf(acc[q * 4 + vv], a.scale2, -lsv[vv]));
              if constexpr (MODE == 0) {
                cs += p;
                hs = fmaf(p, ov[vv], hs);
              } else {
                cs = fmaf(ov[vv], p, cs);
              }
            }
          }
          colsum += cs;
          if constexpr (MODE == 0) {
            hsum += hs;
            csr[rb] += cs;
          }
          continue;
        }
        float rbs = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float part_g = 0.f;
          const int row0 = rb * 32 + acc_row(q * 4, lane);
          const float4 ls4 = *(const float4*)(lse_s + row0);
          const float lsv[4] = {ls4.x, ls4.y, ls4.z, ls4.w};
          float env[4] = {0.f, 0.f, 0.f, 0.f}, wv[4] = {1.f, 1.f, 1.f, 1.f};
          int lmv[4] = {0x7fffffff, 0x7fffffff, 0x7fffffff, 0x7fffffff};
          if constexpr (MODE == 0) {
            const float4 e4 = *(const float4*)(ent_s + row0);
            env[0] = e4.x; env[1] = e4.y; env[2] = e4.z; env[3] = e4.w;
          } else {
            const float4 w4 = *(const float4*)(w_s + row0);
            wv[0] = w4.x; wv[1] = w4.y; wv[2] = w4.z; wv[3] = w4.w;
            const int4 l4 = *(const int4*)(lim_s + row0);
            lmv[0] = l4.x; lmv[1] = l4.y; lmv[2] = l4.z; lmv[3] = l4.w;
          }
#pragma unroll
          for (int vv = 0; vv < 4; ++vv) {
            int v = q * 4 + vv;
            bool ok = kvalid && (MODE == 0 || key <= lmv[vv]);
            const float e = fast_exp2(acc[v] * a.scale2 - lsv[vv]);
            float p = ok ? e : 0.f;
            if constexpr (MODE == 0) {
              colsum += p;
              hsum += p * env[vv];
            } else {
              colsum += wv[vv] * p;
            }
            part_g += p;
          }
          if (mode == 0) {
            // an 8-row group lies inside one query head (P is a multiple of 8);
            // with P a multiple of 32 the whole 32-row block does
            if (a.P % 32 == 0) {
              rbs += part_g;
            } else {
              int g = (rb * 32 + q * 8) / a.P;
#pragma unroll
              for (int gg = 0; gg < 8; ++gg)
                if (gg == g) mg[gg] += part_g;
            }
          }
        }
        if (mode == 0 && a.P % 32 == 0) {
          const int g = rb * 32 / a.P;
#pragma unroll
          for (int gg = 0; gg < 8; ++gg)
            if (gg == g) mg[gg] += rbs;
        }
      }
    }
    if (mode == 0 && a.P % 32 == 0) {
      // row block rb belongs to query head rb * 32 / P
      const int bph = a.P >> 5;
      if (bph == 1) {
#pragma unroll
        for (int g = 0; g < 8; ++g) mg[g] += csr[g];
      } else if (bph == 2) {
#pragma unroll
        for (int g = 0; g < 4; ++g) mg[g] += csr[2 * g] + csr[2 * g + 1];
      } else if (bph == 4) {
        mg[0] += (csr[0] + csr[1]) + (csr[2] + csr[3]);
        mg[1] += (csr[4] + csr[5]) + (csr[6] + csr[7]);
      } else {
        mg[0] += ((csr[0] + csr[1]) + (csr[2] + csr[3])) + ((csr[4] + csr[5]) + (csr[6] + csr[7]));
      }
    }
    colsum += __shfl_xor(colsum, 32, 64);
    if (mode == 0) {
      hsum += __shfl_xor(hsum, 32, 64);
#pragma unroll
      for (int g = 0; g < 8; ++g) mg[g] += __shfl_xor(mg[g], 32, 64);
      if (lane < 32 && kvalid) {
        float mean = colsum / (float)a.G;
        float var = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g)
          if (g < a.G) var += (mg[g] - mean) * (mg[g] - mean);
        var /= (float)a.G;
        int64_t tix = ubase + key;
        int64_t plane = (int64_t)a.Ly * a.H * a.T;
        out0[tix] = colsum;
        if (feats) {
          feats[tix] = colsum;
          feats[plane + tix] = vn;
          feats[2 * plane + tix] = var;
          feats[3 * plane + tix] = colsum > 0.f ? hsum / colsum : 0.f;
          feats[4 * plane + tix] = (float)key / (float)(w.L > 1 ? w.L - 1 : 1);
        }
        hs_num += colsum * vn;
        hs_den += colsum;
      }
    } else if (lane < 32 && kvalid) {
      int64_t tix = ubase + key;
      out0[tix] = a.accumulate ? out0[tix] + colsum : colsum;  // delta_t
      rel_out[tix] = rel_in[tix] + colsum;                      // running relevance
    }
  }
  if (mode == 0) {
    hs_num = wave_sum(hs_num);
    hs_den = wave_sum(hs_den);
    if (lane == 0) {
      hred[wave * 2] = hs_num;
      hred[wave * 2 + 1] = hs_den;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float n = 0.f, d = 0.f;
      for (int wv = 0; wv < WAVES; ++wv) {
        n += hred[wv * 2];
        d += hred[wv * 2 + 1];
      }
      head_part[blockIdx.x * 2] = n;
      head_part[blockIdx.x * 2 + 1] = d;
    }
  }
}

__global__ void headsens_kernel(AttnArgs a, const float* head_part, float* head_sens) {
  int64_t unit = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t n_units = (int64_t)a.S * a.Ly * a.H;
  if (unit >= n_units) return;
  int s = (int)(unit / ((int64_t)a.Ly * a.H));
  int lh = (int)(unit % ((int64_t)a.Ly * a.H));
  int64_t base = 0, ns = 0;
  for (int q = 0; q <= s; ++q) {
    int64_t L = a.cu[q + 1] - a.cu[q];
    ns = (L + a.KW - 1) / a.KW;
    if (q < s) base += ns * a.Ly * a.H;
  }
  base += (int64_t)lh * ns;
  double n = 0.0, d = 0.0;
  for (int64_t k = 0; k < ns; ++k) {
    n += head_part[(base + k) * 2];
    d += head_part[(base + k) * 2 + 1];
  }
  head_sens[unit] = d > 0.0 ? (float)(n / d) : 0.f;
}

// ------------------------------------------------------------------ seeds
// Top-M tokens of delta per unit by (value desc, index asc), written in
// ascending position order, -1 padded. One workgroup per unit: an 8-pass MSB
// radix select on the 64-bit keys, then an ordered compaction.
// Top-M seeds of one unit: an 8-pass MSB radix select over 64-bit keys
// (score, then the lower index first) held in registers, each pass a shared
// histogram and a parallel suffix scan of its 256 bins, then an ordered
// compaction (per-thread contiguous index ranges, a block scan of the counts).
constexpr int SEED_THREADS = 1024;
constexpr int SEED_PER = 16;  // keys a thread keeps in registers; longer sequences loop over global memory
__device__ __forceinline__ int block_excl_scan_seed(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SEED_THREADS / 64; ++w) {
    base += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();  // wsum is reused by the next scan
  *total = tot;
  return base + inc - v;
}

__global__ __launch_bounds__(SEED_THREADS) void seeds_kernel(AttnArgs a, const float* delta, int32_t* seeds) {
  __shared__ uint32_t hist[256];
  __shared__ int wsum[SEED_THREADS / 64];
  __shared__ uint64_t s_prefix;
  __shared__ int64_t s_need;
  __shared__ int s_done;
  const int unit = blockIdx.x;
  const int s = unit / (a.Ly * a.H);
  const int lh = unit % (a.Ly * a.H);
  const int64_t tok0 = a.cu[s];
  const int64_t L = a.cu[s + 1] - tok0;
  const float* dl = delta + (int64_t)lh * a.T + tok0;
  int32_t* out = seeds + (int64_t)unit * a.M;
  const int tid = threadIdx.x;
  // thread t owns the contiguous index range [t*per, t*per + per)
  const int64_t per = (L + SEED_THREADS - 1) / SEED_THREADS;
  const int64_t b0 = min((int64_t)tid * per, L), b1 = min(b0 + per, L);
  const bool inreg = per <= SEED_PER;
  uint64_t kr[SEED_PER];
#pragma unroll
  for (int q = 0; q < SEED_PER; ++q) {
    const int64_t i = b0 + q;
    kr[q] = (inreg && i < b1) ? make_key(dl[i], (uint32_t)i) : 0ull;
  }
  uint64_t thr = 0;  // select keys >= thr
  if (L > a.M) {
    if (tid == 0) {
      s_prefix = 0;
      s_need = a.M;
      s_done = 0;
    }
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      const uint64_t prefix = s_prefix;
      const uint64_t hmask = pass == 0 ? 0ull : (~0ull << (64 - 8 * pass));
      if (inreg) {
#pragma unroll
        for (int q = 0; q < SEED_PER; ++q)
          if (b0 + q < b1 && (kr[q] & hmask) == prefix) atomicAdd(&hist[(kr[q] >> shift) & 255], 1u);
      } else {
        for (int64_t i = b0; i < b1; ++i) {
          const uint64_t k = make_key(dl[i], (uint32_t)i);
          if ((k & hmask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1u);
        }
      }
      __syncthreads();
      // bins in descending digit order: thread t < 256 holds bin 255 - t; the
      // selected bin is the one where the running count first reaches `need`
      const int hv = tid < 256 ? (int)hist[255 - tid] : 0;
      int tot;
      const int above = block_excl_scan_seed(hv, wsum, &tot);
      const int64_t need = s_need;
      __syncthreads();  // every thread has read s_need and s_prefix
      if (tid < 256 && above < need && above + hv >= need) {
        s_need = need - above;
        s_prefix = prefix | ((uint64_t)(255 - tid) << shift);
        // the whole bin is taken: its prefix (lower bits zero) already
        // separates the M largest keys from the rest
        s_done = above + hv == need;
      }
      __syncthreads();
      if (s_done) break;
    }
    thr = s_prefix;  // the M-th largest key, or the prefix of the last bin taken whole
  }
  // ordered compaction
  int c = 0;
  if (inreg) {
#pragma unroll
    for (int q = 0; q < SEED_PER; ++q)
      if (b0 + q < b1 && (L <= a.M || kr[q] >= thr)) ++c;
  } else {
    for (int64_t i = b0; i < b1; ++i)
      if (L <= a.M || make_key(dl[i], (uint32_t)i) >= thr) ++c;
  }
  int tot;
  int o = block_excl_scan_seed(c, wsum, &tot);
  if (inreg) {
#pragma unroll
    for (int q = 0; q < SEED_PER; ++q)
      if (b0 + q < b1 && (L <= a.M || kr[q] >= thr)) out[o++] = (int32_t)(b0 + q);
  } else {
    for (int64_t i = b0; i < b1; ++i)
      if (L <= a.M || make_key(dl[i], (uint32_t)i) >= thr) out[o++] = (int32_t)i;
  }
  const int total = L < a.M ? (int)L : a.M;
  for (int k = total + tid; k < a.M; k += SEED_THREADS) out[k] = -1;
}

__global__ void copy_f32_kernel(const float* src, float* dst, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// ------------------------------------------------------------------ host
// Key split of the probe and seed passes: the widest of 1024 / 512 / 256 keys
// that still gives 2048 workgroups (each stages its query rows once, so wider
// splits stage less; 1024 against 512 saves 0.33 ms of the 3.3 ms of probe and
// seed passes on the full-depth workload).
int pick_kw(const kvc_shape* sh) {
  int64_t units = (int64_t)sh->n_layers * sh->n_kv_heads;
  for (int kw : {4096, 2048, 1024, 512, 256}) {
    int64_t n = 0;
    for (int s = 0; s < sh->n_seq; ++s) n += units * ((sh->cu_seqlens[s + 1] - sh->cu_seqlens[s] + kw - 1) / kw);
    if (n >= 2048) return kw;
  }
  return 128;
}

int64_t n_splits(const kvc_shape* sh, int kw) {
  int64_t units = (int64_t)sh->n_layers * sh->n_kv_heads, n = 0;
  for (int s = 0; s < sh->n_seq; ++s) n += units * ((sh->cu_seqlens[s + 1] - sh->cu_seqlens[s] + kw - 1) / kw);
  return n;
}

AttnArgs base_args(const kvc_shape* sh, const kvc_params* p, int kw) {
  AttnArgs a{};
  a.cu = sh->cu_seqlens_d;
  a.S = sh->n_seq;
  a.Ly = sh->n_layers;
  a.H = sh->n_kv_heads;
  a.G = sh->group;
  a.P = p->n_probe;
  a.M = p->n_seeds;
  a.T = sh->total_tokens;
  a.KW = kw;
  a.scale2 = LOG2E / sqrtf((float)sh->head_dim);
  return a;
}

size_t smem_rows(const AttnArgs& a, int d, int elt) { return (size_t)a.Rpad * d * elt; }

template <class T, int D>
int launch_pass1(const AttnArgs& a, int mode, int64_t nsplit, float* part, hipStream_t st) {
  // the staged rows and their limits, then (over them) the per-wave merge area
  size_t sm = std::max(smem_rows(a, D, sizeof(T)) + a.Rpad * sizeof(int), (size_t)WAVES * a.Rpad * 3 * sizeof(float));
  (void)hipFuncSetAttribute((const void*)rowstats_kernel<T, D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  hipLaunchKernelGGL((rowstats_kernel<T, D>), dim3((unsigned)nsplit), dim3(THREADS), sm, st, a, mode, part);
  KVC_LAUNCH_CHECK("rowstats");
  return KVC_OK;
}
template <class T, int D>
int launch_pass2(const AttnArgs& a, int mode, int64_t nsplit, const float2* rowstat, float* out0,
                 float* feats, float* head_part, const float* rel_in, float* rel_out, hipStream_t st) {
  size_t sm = smem_rows(a, D, sizeof(T)) + a.Rpad * sizeof(int) + 3 * a.Rpad * sizeof(float) +
              WAVES * 2 * sizeof(float);
  if (mode == 0) {
    (void)hipFuncSetAttribute((const void*)colsum_kernel<T, D, 0>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    hipLaunchKernelGGL((colsum_kernel<T, D, 0>), dim3((unsigned)nsplit), dim3(THREADS), sm, st, a, rowstat, out0,
                       feats, head_part, rel_in, rel_out);
  } else {
    (void)hipFuncSetAttribute((const void*)colsum_kernel<T, D, 1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    hipLaunchKernelGGL((colsum_kernel<T, D, 1>), dim3((unsigned)nsplit), dim3(THREADS), sm, st, a, rowstat, out0,
                       feats, head_part, rel_in, rel_out);
  }
  KVC_LAUNCH_CHECK("colsum");
  return KVC_OK;
}

template <class T, int D>
int run_passes(const AttnArgs& a, int mode, int64_t nsplit, float* part, float2* rowstat, float* lse_out,
               float* ent_out, float* out0, float* feats, float* head_part, const float* rel_in,
               float* rel_out, hipStream_t st) {
  int r = launch_pass1<T, D>(a, mode, nsplit, part, st);
  if (r) return r;
  int64_t nr = (int64_t)a.S * a.Ly * a.H * a.Rpad;
  hipLaunchKernelGGL(rowcombine_kernel, dim3(kvc_blocks(nr, 256)), dim3(256), 0, st, a, part, rowstat, lse_out,
                     ent_out);
  KVC_LAUNCH_CHECK("rowcombine");
  return launch_pass2<T, D>(a, mode, nsplit, rowstat, out0, feats, head_part, rel_in, rel_out, st);
}

template <class... Args>
int dispatch(int dtype, int d, const AttnArgs& a, int mode, int64_t nsplit, Args... rest) {
  if (dtype == KVC_BF16) {
    if (d == 128) return run_passes<uint16_t, 128>(a, mode, nsplit, rest...);
    return run_passes<uint16_t, 64>(a, mode, nsplit, rest...);
  }
  if (d == 128) return run_passes<float, 128>(a, mode, nsplit, rest...);
  return run_passes<float, 64>(a, mode, nsplit, rest...);
}

// Dense rollout: row block b of every unit lists positions b*M .. b*M+M-1
// (-1 past the sequence) as its "seeds".
__global__ void dense_seeds_kernel(AttnArgs a, int64_t block, int32_t* seeds) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_units = (int64_t)a.S * a.Ly * a.H;
  if (i >= n_units * a.M) return;
  const int s = (int)(i / ((int64_t)a.Ly * a.H * a.M));
  const int64_t pos = block * a.M + i % a.M;
  seeds[i] = pos < a.cu[s + 1] - a.cu[s] ? (int32_t)pos : -1;
}
__global__ void zero_f32_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

namespace kvc {

size_t ws_score(const kvc_shape* s, const kvc_params* p) {
  int kw = pick_kw(s);
  int64_t ns = n_splits(s, kw);
  int rpad = ((s->group * p->n_probe) + 31) / 32 * 32;
  int64_t units = (int64_t)s->n_seq * s->n_layers * s->n_kv_heads;
  Carver c(nullptr, 0);
  c.take<float>((size_t)ns * rpad * 3);
  c.take<float2>((size_t)units * rpad);
  c.take<float>((size_t)ns * 2);
  return c.off + 256;
}

size_t ws_propagate(const kvc_shape* s, const kvc_params* p) {
  int kw = pick_kw(s);
  int64_t ns = n_splits(s, kw);
  int rpad = ((s->group * p->n_seeds) + 31) / 32 * 32;
  int64_t units = (int64_t)s->n_seq * s->n_layers * s->n_kv_heads;
  int64_t E = (int64_t)s->n_layers * s->n_kv_heads * s->total_tokens;
  Carver c(nullptr, 0);
  c.take<float>((size_t)ns * rpad * 3);
  c.take<float2>((size_t)units * rpad);
  c.take<float>((size_t)E * 2);
  c.take<int32_t>((size_t)units * p->n_seeds);
  return c.off + 256;
}

}  // namespace kvc

namespace kvc {
// The probe pass with sh->total_tokens as the row stride of K, V and the
// per-token outputs, which may exceed cu_seqlens[S] (the step-wise student
// keeps spare slots past each sequence's tokens).
int score_strided(const kvc_shape* sh, const kvc_params* p, const void* K, const void* V, const void* Qprobe,
                  float* rel0, float* feats, float* probe_lse, float* probe_ent, float* head_sens, void* ws,
                  size_t ws_bytes, hipStream_t st) {
  int r;
  KVC_REQUIRE(ws_bytes >= kvc::ws_score(sh, p) && ws, KVC_E_WORKSPACE, "kvc_score: workspace too small");
  int kw = pick_kw(sh);
  int64_t ns = n_splits(sh, kw);
  if (ns == 0) return KVC_OK;
  AttnArgs a = base_args(sh, p, kw);
  a.K = K;
  a.V = V;
  a.Q = Qprobe;
  a.R = sh->group * p->n_probe;
  a.Rpad = (a.R + 31) / 32 * 32;
  int64_t units = (int64_t)sh->n_seq * sh->n_layers * sh->n_kv_heads;
  kvc::Carver c(ws, ws_bytes);
  float* part = c.take<float>((size_t)ns * a.Rpad * 3);
  float2* rowstat = c.take<float2>((size_t)units * a.Rpad);
  float* head_part = c.take<float>((size_t)ns * 2);
  r = dispatch(sh->dtype, sh->head_dim, a, 0, ns, part, rowstat, probe_lse, probe_ent, rel0, feats, head_part,
               (const float*)nullptr, (float*)nullptr, st);
  if (r) return r;
  hipLaunchKernelGGL(headsens_kernel, dim3(kvc_blocks(units, 256)), dim3(256), 0, st, a, head_part, head_sens);
  KVC_LAUNCH_CHECK("headsens");
  return KVC_OK;
}
}  // namespace kvc

extern "C" int kvc_score(const kvc_shape* sh, const kvc_params* p, const void* K, const void* V,
                         const void* Qprobe, float* rel0, float* feats, float* probe_lse, float* probe_ent,
                         float* head_sens, void* ws, size_t ws_bytes, hipStream_t st) {
  int r = kvc::validate_shape(sh);
  if (r) return r;
  if ((r = kvc::validate_params(sh, p))) return r;
  KVC_REQUIRE(K && V && Qprobe && rel0 && probe_lse && probe_ent && head_sens, KVC_E_INVAL,
              "kvc_score: NULL input or output");
  return kvc::score_strided(sh, p, K, V, Qprobe, rel0, feats, probe_lse, probe_ent, head_sens, ws, ws_bytes, st);
}

extern "C" int kvc_propagate(const kvc_shape* sh, const kvc_params* p, const void* K, const void* Qctx,
                             const float* rel0, float* rel, int32_t* seeds, void* ws, size_t ws_bytes,
                             hipStream_t st) {
  int r = kvc::validate_shape(sh);
  if (r) return r;
  if ((r = kvc::validate_params(sh, p))) return r;
  KVC_REQUIRE(K && Qctx && rel0 && rel, KVC_E_INVAL, "kvc_propagate: NULL input or output");
  KVC_REQUIRE(ws_bytes >= kvc::ws_propagate(sh, p) && ws, KVC_E_WORKSPACE, "kvc_propagate: workspace too small");
  int kw = pick_kw(sh);
  int64_t ns = n_splits(sh, kw);
  int64_t E = (int64_t)sh->n_layers * sh->n_kv_heads * sh->total_tokens;
  int64_t units = (int64_t)sh->n_seq * sh->n_layers * sh->n_kv_heads;
  if (E == 0) return KVC_OK;
  AttnArgs a = base_args(sh, p, kw);
  a.K = K;
  a.Q = Qctx;
  a.R = sh->group * p->n_seeds;
  a.Rpad = (a.R + 31) / 32 * 32;
  a.hop_w = p->hop_weight / (float)sh->group;
  kvc::Carver c(ws, ws_bytes);
  float* part = c.take<float>((size_t)ns * a.Rpad * 3);
  float2* rowstat = c.take<float2>((size_t)units * a.Rpad);
  float* dbuf = c.take<float>((size_t)E * 2);
  int32_t* seed_tmp = c.take<int32_t>((size_t)units * p->n_seeds);
  // rel = rel0; delta_0 = rel0
  hipLaunchKernelGGL(copy_f32_kernel, dim3(kvc_blocks(E, 256)), dim3(256), 0, st, rel0, rel, E);
  KVC_LAUNCH_CHECK("copy");
  const float* prev = rel0;
  for (int hop = 0; hop < p->n_hops; ++hop) {
    int32_t* sd = seeds ? seeds + (int64_t)hop * units * p->n_seeds : seed_tmp;
    hipLaunchKernelGGL(seeds_kernel, dim3((unsigned)units), dim3(SEED_THREADS), 0, st, a, prev, sd);
    KVC_LAUNCH_CHECK("seeds");
    float* cur = dbuf + (int64_t)(hop & 1) * E;
    a.seeds = sd;
    a.prev = prev;
    // tokens no workgroup visits keep delta 0 (every token is visited, but
    // clear anyway so a reader never sees stale values)
    r = dispatch(sh->dtype, sh->head_dim, a, 1, ns, part, rowstat, (float*)nullptr, (float*)nullptr, cur,
                 (float*)nullptr, (float*)nullptr, (const float*)rel, rel, st);
    if (r) return r;
    prev = cur;
  }
  return KVC_OK;
}

namespace {
template <class T, int D>
int launch_rowval(const AttnArgs& a, int64_t nsplit, float* part, hipStream_t st) {
  const size_t sm = std::max(smem_rows(a, D, sizeof(T)) + a.Rpad * sizeof(int), (size_t)WAVES * a.Rpad * 4 * sizeof(float));
  (void)hipFuncSetAttribute((const void*)rowstats_kernel<T, D, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)sm);
  hipLaunchKernelGGL((rowstats_kernel<T, D, true>), dim3((unsigned)nsplit), dim3(THREADS), sm, st, a, 1, part);
  KVC_LAUNCH_CHECK("rowstats_val");
  return KVC_OK;
}
int dispatch_rowval(int dtype, int d, const AttnArgs& a, int64_t nsplit, float* part, hipStream_t st) {
  if (dtype == KVC_BF16) return d == 128 ? launch_rowval<uint16_t, 128>(a, nsplit, part, st)
                                         : launch_rowval<uint16_t, 64>(a, nsplit, part, st);
  return d == 128 ? launch_rowval<float, 128>(a, nsplit, part, st) : launch_rowval<float, 64>(a, nsplit, part, st);
}
int dense_rows(const kvc_shape* sh) { return (256 / sh->group) < 64 ? 256 / sh->group : 64; }
// Key split of the dense passes, a multiple of 512 keys: every row
// block stages its 256 query rows once per split, and a block's rows see a
// whole causal prefix, so wide splits stage far less (fewer splits than the
// workspace, sized with pick_kw, holds). Measured on the full-depth workload
// (16,384 tokens): the dense rollout 769 ms at 1x, 425 ms at 16x (523 ms at
// 32x, where one split a unit leaves its column-sum pass too few workgroups);
// the "A r" direction, a row pass only, 739 ms at 1x, 221 ms at 32x.
int dense_kw(int mult) { return 512 * mult; }  // >= pick_kw for mult >= 2
}  // namespace

extern "C" size_t kvc_propagate_dense_workspace(const kvc_shape* sh, const kvc_params* p) {
  if (kvc::validate_shape(sh) || !p) return 0;
  kvc_params q = *p;
  q.n_seeds = dense_rows(sh);
  return kvc::ws_propagate(sh, &q);
}

extern "C" int kvc_propagate_dense(const kvc_shape* sh, const kvc_params* p, const void* K, const void* Qctx,
                                   const float* rel0, float* rel, void* ws, size_t ws_bytes, hipStream_t st) {
  int r = kvc::validate_shape(sh);
  if (r) return r;
  KVC_REQUIRE(p, KVC_E_INVAL, "params is NULL");
  KVC_REQUIRE(p->n_hops >= 0 && p->n_hops <= 8, KVC_E_INVAL, "n_hops must be in [0, 8]");
  KVC_REQUIRE(K && Qctx && rel0 && rel, KVC_E_INVAL, "kvc_propagate_dense: NULL input or output");
  KVC_REQUIRE(ws && ws_bytes >= kvc_propagate_dense_workspace(sh, p), KVC_E_WORKSPACE,
              "kvc_propagate_dense: workspace too small");
  kvc_params q = *p;
  q.n_seeds = dense_rows(sh);
  const int kw = dense_kw(16);
  const int64_t ns = n_splits(sh, kw);
  const int64_t E = (int64_t)sh->n_layers * sh->n_kv_heads * sh->total_tokens;
  const int64_t units = (int64_t)sh->n_seq * sh->n_layers * sh->n_kv_heads;
  if (E == 0) return KVC_OK;
  AttnArgs a = base_args(sh, &q, kw);
  a.K = K;
  a.Q = Qctx;
  a.R = sh->group * q.n_seeds;
  a.Rpad = (a.R + 31) / 32 * 32;
  a.hop_w = p->hop_weight / (float)sh->group;
  a.accumulate = 1;
  kvc::Carver c(ws, ws_bytes);
  float* part = c.take<float>((size_t)ns * a.Rpad * 3);
  float2* rowstat = c.take<float2>((size_t)units * a.Rpad);
  float* dbuf = c.take<float>((size_t)E * 2);
  int32_t* seeds = c.take<int32_t>((size_t)units * q.n_seeds);
  hipLaunchKernelGGL(copy_f32_kernel, dim3(kvc_blocks(E, 256)), dim3(256), 0, st, rel0, rel, E);
  KVC_LAUNCH_CHECK("copy");
  const int64_t nblk = (kvc::max_len(sh) + q.n_seeds - 1) / q.n_seeds;
  const float* prev = rel0;
  for (int hop = 0; hop < p->n_hops; ++hop) {
    float* cur = dbuf + (int64_t)(hop & 1) * E;
    hipLaunchKernelGGL(zero_f32_kernel, dim3(kvc_blocks(E, 256)), dim3(256), 0, st, cur, E);
    KVC_LAUNCH_CHECK("zero");
    a.prev = prev;
    a.seeds = seeds;
    for (int64_t b = 0; b < nblk; ++b) {
      hipLaunchKernelGGL(dense_seeds_kernel, dim3(kvc_blocks(units * q.n_seeds, 256)), dim3(256), 0, st, a, b,
                         seeds);
      KVC_LAUNCH_CHECK("dense_seeds");
      r = dispatch(sh->dtype, sh->head_dim, a, 1, ns, part, rowstat, (float*)nullptr, (float*)nullptr, cur,
                   (float*)nullptr, (float*)nullptr, (const float*)rel, rel, st);
      if (r) return r;
    }
    prev = cur;
  }
  return KVC_OK;
}

extern "C" size_t kvc_propagate_ar_workspace(const kvc_shape* sh, const kvc_params* p) {
  if (kvc::validate_shape(sh) || !p) return 0;
  kvc_params q = *p;
  q.n_seeds = dense_rows(sh);
  const int64_t ns = n_splits(sh, pick_kw(sh));
  const int rpad = (sh->group * q.n_seeds + 31) / 32 * 32;
  return kvc::ws_propagate(sh, &q) + (size_t)ns * rpad * sizeof(float) + 256;
}

extern "C" int kvc_propagate_ar(const kvc_shape* sh, const kvc_params* p, const void* K, const void* Qctx,
                                const float* rel0, float* rel, void* ws, size_t ws_bytes, hipStream_t st) {
  int r = kvc::validate_shape(sh);
  if (r) return r;
  KVC_REQUIRE(p, KVC_E_INVAL, "params is NULL");
  KVC_REQUIRE(p->n_hops >= 0 && p->n_hops <= 8, KVC_E_INVAL, "n_hops must be in [0, 8]");
  KVC_REQUIRE(K && Qctx && rel0 && rel, KVC_E_INVAL, "kvc_propagate_ar: NULL input or output");
  KVC_REQUIRE(ws && ws_bytes >= kvc_propagate_ar_workspace(sh, p), KVC_E_WORKSPACE,
              "kvc_propagate_ar: workspace too small");
  kvc_params q = *p;
  q.n_seeds = dense_rows(sh);
  const int kw = dense_kw(32);
  const int64_t ns = n_splits(sh, kw);
  const int64_t E = (int64_t)sh->n_layers * sh->n_kv_heads * sh->total_tokens;
  const int64_t units = (int64_t)sh->n_seq * sh->n_layers * sh->n_kv_heads;
  if (E == 0) return KVC_OK;
  AttnArgs a = base_args(sh, &q, kw);
  a.K = K;
  a.Q = Qctx;
  a.R = sh->group * q.n_seeds;
  a.Rpad = (a.R + 31) / 32 * 32;
  a.hop_w = p->hop_weight / (float)sh->group;
  kvc::Carver c(ws, ws_bytes);
  float* part = c.take<float>((size_t)ns * a.Rpad * 3);
  c.take<float2>((size_t)units * a.Rpad);  // same carving as the propagation workspace
  float* dbuf = c.take<float>((size_t)E * 2);
  int32_t* seeds = c.take<int32_t>((size_t)units * q.n_seeds);
  a.part_v = c.take<float>((size_t)ns * a.Rpad);
  hipLaunchKernelGGL(copy_f32_kernel, dim3(kvc_blocks(E, 256)), dim3(256), 0, st, rel0, rel, E);
  KVC_LAUNCH_CHECK("copy");
  const int64_t nblk = (kvc::max_len(sh) + q.n_seeds - 1) / q.n_seeds;
  const float* prev = rel0;
  a.seeds = seeds;
  for (int hop = 0; hop < p->n_hops; ++hop) {
    float* cur = dbuf + (int64_t)(hop & 1) * E;
    a.kval = prev;
    for (int64_t b = 0; b < nblk; ++b) {
      hipLaunchKernelGGL(dense_seeds_kernel, dim3(kvc_blocks(units * q.n_seeds, 256)), dim3(256), 0, st, a, b,
                         seeds);
      KVC_LAUNCH_CHECK("dense_seeds");
      if ((r = dispatch_rowval(sh->dtype, sh->head_dim, a, ns, part, st))) return r;
      hipLaunchKernelGGL(rowval_kernel, dim3(kvc_blocks(units * q.n_seeds, 256)), dim3(256), 0, st, a, part, b, cur,
                         rel);
      KVC_LAUNCH_CHECK("rowval");
    }
    prev = cur;
  }
  return KVC_OK;
}
