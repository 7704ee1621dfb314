// Per-step KL(full || compressed) through the vocab projection.
//
// DistillCache paper, Sec. 3.1.4 (Reward): the fidelity signal is
// D_KL(P_t || P^_t) between the next-token distributions of the full-cache
// and the pruned-cache model, from logits with numerical stabilization.
//
// 1. rmsnorm_cast: x^ = x / sqrt(mean x^2 + 1e-6) in fp64, cast to W's
//    dtype; the full and compressed rows of pair p become rows 2p and 2p+1.
// 2. gemm_kl: y = x^ W^T on MFMA (W is [vocab][d_model], so both operands
//    are contiguous along d_model). A workgroup owns 128 vocab columns and
//    up to 128 rows; its epilogue reduces each pair over its columns to
//    (max_f, sum_f, max_c, sum_c, sum e^(y-max_f) (y - y^)) - the logits
//    never reach memory.
// 3. kl_combine: merge the column-tile partials of every pair.
#include <cmath>

#include "kvc_internal.h"

namespace {

constexpr int THREADS = 256;
constexpr int NT = 128;    // vocab columns per workgroup (4 waves x 32)
constexpr int MT = 128;    // rows per workgroup (4 row blocks of 32)
constexpr int KC = 128;    // d_model chunk staged in LDS
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// The normalisation runs in fp64 and is rounded fp64 -> fp32 -> W's dtype:
// the cast is a rounding decision, and taking it from a correctly rounded
// fp64 value keeps it independent of the summation order.
template <class T>
__global__ __launch_bounds__(256) void rmsnorm_cast_kernel(const float* xf, const float* xc, int64_t n_pairs,
                                                           int dm, int64_t m_pad, T* out) {
  int64_t row = blockIdx.x;
  T* o = out + row * dm;
  if (row >= 2 * n_pairs) {  // padding rows
    for (int i = threadIdx.x; i < dm; i += blockDim.x) ElemIO<T>::st(o, i, 0.f);
    return;
  }
  const float* x = ((row & 1) ? xc : xf) + (row >> 1) * dm;
  __shared__ double red[8];
  double ss = 0.0;
  for (int i = threadIdx.x; i < dm; i += blockDim.x) ss += (double)x[i] * (double)x[i];
  ss = wave_sum_d(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  double tot = 0.0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += red[w];
  const double r = 1.0 / sqrt(tot / (double)dm + 1e-6);
  for (int i = threadIdx.x; i < dm; i += blockDim.x) ElemIO<T>::st(o, i, (float)((double)x[i] * r));
}

template <class T> struct Frag;
template <> struct Frag<uint16_t> { kvc_bf16x8 v; };
template <> struct Frag<float> { float v[8]; };
__device__ __forceinline__ Frag<uint16_t> ldfrag(const uint16_t* p) {
  Frag<uint16_t> f;
  f.v = __builtin_bit_cast(kvc_bf16x8, *(const uint4*)p);
  return f;
}
__device__ __forceinline__ Frag<float> ldfrag(const float* p) {
  Frag<float> f;
  float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}
__device__ __forceinline__ void mma(kvc_f32x16& acc, const Frag<uint16_t>& a, const Frag<uint16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(kvc_f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

struct Stat5 {
  float mf, sf, mc, sc, t;
};
// Contraction stays off here: the full and the compressed statistics must go
// through identical roundings so that identical rows give KL = 0 exactly.
__device__ __forceinline__ Stat5 merge5(Stat5 a, Stat5 b) {
#pragma clang fp contract(off)
  Stat5 r;
  r.mf = fmaxf(a.mf, b.mf);
  float fa = a.mf == -INFINITY ? 0.f : exp2f(a.mf - r.mf), fb = b.mf == -INFINITY ? 0.f : exp2f(b.mf - r.mf);
  r.sf = a.sf * fa + b.sf * fb;
  r.t = a.t * fa + b.t * fb;
  r.mc = fmaxf(a.mc, b.mc);
  float ga = a.mc == -INFINITY ? 0.f : exp2f(a.mc - r.mc), gb = b.mc == -INFINITY ? 0.f : exp2f(b.mc - r.mc);
  r.sc = a.sc * ga + b.sc * gb;
  return r;
}

// grid: (vocab / NT, m_pad / MT). part: [n_pairs][n_col_tiles][5]
template <class T>
__global__ __launch_bounds__(THREADS) void gemm_kl_kernel(const T* xh, const T* W, int64_t n_pairs, int dm,
                                                          int vocab, int64_t m_pad, float* part) {
  __shared__ __align__(16) Frag<T> af[MT / 32][KC / 16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)blockIdx.y * MT;
  const int nrb = (int)((m_pad - r0) < MT ? (m_pad - r0) / 32 : MT / 32);
  const int col = blockIdx.x * NT + wave * 32 + (lane & 31);
  const bool cvalid = col < vocab;
  const T* wrow = W + (int64_t)(cvalid ? col : 0) * dm;
  kvc_f32x16 acc[MT / 32];
#pragma unroll
  for (int rb = 0; rb < MT / 32; ++rb) acc[rb] = kvc_f32x16{};
  for (int k0 = 0; k0 < dm; k0 += KC) {
    __syncthreads();
    // stage x^ rows [r0, r0 + 32 nrb) x [k0, k0 + KC) in fragment order
    for (int c = threadIdx.x; c < nrb * 32 * (KC / 8); c += THREADS) {
      int row = c / (KC / 8), c8 = c % (KC / 8);
      int rb = row >> 5, ks = c8 >> 1, ln = (row & 31) + 32 * (c8 & 1);
      af[rb][ks][ln] = ldfrag(xh + (r0 + row) * dm + k0 + c8 * 8);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KC / 16; ++ks) {
      Frag<T> b = ldfrag(wrow + k0 + ks * 16 + 8 * (lane >> 5));
#pragma unroll
      for (int rb = 0; rb < MT / 32; ++rb)
        if (rb < nrb) mma(acc[rb], af[rb][ks][lane], b);
    }
  }
  // epilogue: lane owns column `col`; registers v, v+1 (v%4 in {0,2}) hold
  // rows 2p and 2p+1 of one pair
  const int ntile = (vocab + NT - 1) / NT;
#pragma unroll
  for (int rb = 0; rb < MT / 32; ++rb) {
    if (rb >= nrb) break;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      int row = rb * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
      int64_t pair = (r0 + row) >> 1;
      // base-2 logits for the partition sums; the logit difference is taken
      // from the accumulators themselves so identical rows give exactly 0
      float y = acc[rb][v] * LOG2E, yh = acc[rb][v + 1] * LOG2E;
      float dy = acc[rb][v] - acc[rb][v + 1];
      Stat5 st;
      if (cvalid) {
        st.mf = y; st.sf = 1.f; st.mc = yh; st.sc = 1.f; st.t = dy;
      } else {
        st.mf = -INFINITY; st.sf = 0.f; st.mc = -INFINITY; st.sc = 0.f; st.t = 0.f;
      }
      // reduce over the 32 lanes (columns) that share this row pair
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        Stat5 other;
        other.mf = __shfl_xor(st.mf, o, 64);
        other.sf = __shfl_xor(st.sf, o, 64);
        other.mc = __shfl_xor(st.mc, o, 64);
        other.sc = __shfl_xor(st.sc, o, 64);
        other.t = __shfl_xor(st.t, o, 64);
        st = merge5(st, other);
      }
      if ((lane & 31) == 0 && pair < n_pairs) {
        // column sub-tile of this wave: tiles of 32 columns
        float* p = part + ((pair * ntile + blockIdx.x) * 4 + wave) * 5;
        p[0] = st.mf; p[1] = st.sf; p[2] = st.mc; p[3] = st.sc; p[4] = st.t;
      }
    }
  }
}

__global__ void kl_combine_kernel(const float* part, int64_t n_pairs, int nsub, float* kl) {
#pragma clang fp contract(off)
  int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= n_pairs) return;
  Stat5 st{-INFINITY, 0.f, -INFINITY, 0.f, 0.f};
  const float* q = part + p * nsub * 5;
  for (int i = 0; i < nsub; ++i) {
    Stat5 o{q[i * 5], q[i * 5 + 1], q[i * 5 + 2], q[i * 5 + 3], q[i * 5 + 4]};
    st = merge5(st, o);
  }
  // natural-log partition functions from base-2 maxima
  float lse_f = (st.mf + log2f(st.sf)) * LN2, lse_c = (st.mc + log2f(st.sc)) * LN2;
  float v = st.t / st.sf - lse_f + lse_c;
  kl[p] = v;
}

}  // namespace

extern "C" size_t kvc_kl_workspace(int64_t n_pairs, int32_t d_model, int32_t vocab, int32_t w_dtype) {
  if (n_pairs <= 0 || d_model <= 0 || vocab <= 0) return 0;
  int64_t m_pad = (2 * n_pairs + 31) / 32 * 32;
  size_t elt = w_dtype == KVC_BF16 ? 2 : 4;
  int64_t ntile = (vocab + NT - 1) / NT;
  kvc::Carver c(nullptr, 0);
  c.take<char>((size_t)m_pad * d_model * elt);
  c.take<float>((size_t)n_pairs * ntile * 4 * 5);
  return c.off + 256;
}

extern "C" int kvc_kl(int64_t n_pairs, int32_t d_model, int32_t vocab, const float* x_full, const float* x_comp,
                      const void* W, int32_t w_dtype, float* kl_out, void* ws, size_t ws_bytes, hipStream_t st) {
  KVC_REQUIRE(n_pairs >= 0 && vocab >= 1, KVC_E_INVAL, "kvc_kl: bad sizes");
  KVC_REQUIRE(d_model >= KC && d_model % KC == 0, KVC_E_SHAPE, "kvc_kl: d_model must be a multiple of 128");
  KVC_REQUIRE(w_dtype == KVC_BF16 || w_dtype == KVC_F32, KVC_E_DTYPE, "kvc_kl: W must be bf16 or f32");
  if (n_pairs == 0) return KVC_OK;
  KVC_REQUIRE(x_full && x_comp && W && kl_out, KVC_E_INVAL, "kvc_kl: NULL pointer");
  KVC_REQUIRE(ws && ws_bytes >= kvc_kl_workspace(n_pairs, d_model, vocab, w_dtype), KVC_E_WORKSPACE,
              "kvc_kl: workspace too small");
  int64_t m_pad = (2 * n_pairs + 31) / 32 * 32;
  int64_t ntile = (vocab + NT - 1) / NT;
  kvc::Carver c(ws, ws_bytes);
  size_t elt = w_dtype == KVC_BF16 ? 2 : 4;
  char* xh = c.take<char>((size_t)m_pad * d_model * elt);
  float* part = c.take<float>((size_t)n_pairs * ntile * 4 * 5);
  dim3 g2((unsigned)ntile, (unsigned)((m_pad + MT - 1) / MT));
  if (w_dtype == KVC_BF16) {
    hipLaunchKernelGGL(rmsnorm_cast_kernel<uint16_t>, dim3((unsigned)m_pad), dim3(256), 0, st, x_full, x_comp,
                       n_pairs, d_model, m_pad, (uint16_t*)xh);
    KVC_LAUNCH_CHECK("rmsnorm_cast");
    hipLaunchKernelGGL(gemm_kl_kernel<uint16_t>, g2, dim3(THREADS), 0, st, (const uint16_t*)xh, (const uint16_t*)W,
                       n_pairs, d_model, vocab, m_pad, part);
  } else {
    hipLaunchKernelGGL(rmsnorm_cast_kernel<float>, dim3((unsigned)m_pad), dim3(256), 0, st, x_full, x_comp, n_pairs,
                       d_model, m_pad, (float*)xh);
    KVC_LAUNCH_CHECK("rmsnorm_cast");
    hipLaunchKernelGGL(gemm_kl_kernel<float>, g2, dim3(THREADS), 0, st, (const float*)xh, (const float*)W, n_pairs,
                       d_model, vocab, m_pad, part);
  }
  KVC_LAUNCH_CHECK("gemm_kl");
  hipLaunchKernelGGL(kl_combine_kernel, dim3(kvc_blocks(n_pairs, 256)), dim3(256), 0, st, part, n_pairs,
                     (int)(ntile * 4), kl_out);
  KVC_LAUNCH_CHECK("kl_combine");
  return KVC_OK;
}
