// Slot partition of each sequence's compressible region.
//
// GraceKV page, '01 Curvature-guided partition' and technical details: the
// normalized hidden states form a trajectory; cut where it turns; a dynamic
// program also weighs within-slot dispersion and reasonable slot lengths
// (16-128 tokens, target 64).
//
// Costs are quantized to integers (round(x * 2^20)) so the DP itself is exact
// integer arithmetic: given the same quantized costs it reproduces the same
// cuts on any machine.
//   turning: one workgroup per token, three dot products per window.
//   costs:   one wave per slot END token; the wave walks back over at most
//            slot_max tokens keeping the window sum in registers (lane = 64
//            hidden dims), so every (end, length) dispersion is
//            sum ||h^||^2 - ||sum h^||^2 / n without a prefix-sum cancellation.
//   dp:      one 1024-thread workgroup per sequence. A slot is at least
//            slot_min tokens long, so the values of slot_min consecutive ends
//            depend only on earlier ends: wave w evaluates end e0 + w, all
//            candidates of a lane pair packed into one int64 key
//            (value * 256 + (255 - (n - slot_min))) whose minimum breaks ties
//            toward the longer last slot (the earlier cut).
#include <cmath>

#include "kvc_internal.h"
#include "mfma_frag.h"

namespace {

constexpr double QSCALE = 1048576.0;  // 2^20
constexpr int64_t INF_Q = (int64_t)1 << 52;

constexpr int MAXD = 4;  // sampled depths of the trajectory

struct PartArgs {
  const void* hidden;       // [nd][T][Dh]
  int Dh;
  int nd;                   // sampled depths
  int64_t dstride;          // elements between depths (T * Dh)
  const float* surp;        // [T] surprisal, or NULL
  float lam_surp;
  float* smax;              // [S] largest surprisal of each sequence
  const int64_t* cu;
  int S;
  int64_t T;
  int nmin, nmax, target, stride;
  float lam_len, lam_curv;
  int64_t c0[64], c1[64];   // compressible region per sequence (sequence positions)
  int64_t* cost_q;          // [T][nmax - nmin + 1]
  int64_t* cut_q;           // [T]
  float* inv;               // [nd][T] 1/||h_t||
  float* nrm2;              // [nd][T] ||h^_t||^2
  int32_t* slot_start;      // [S][stride + 1]
  int32_t* n_slots;         // [S]
};

template <class T>
__global__ __launch_bounds__(256) void norm_kernel(PartArgs a) {
  const int64_t t = blockIdx.x, dep = blockIdx.y;
  const T* h = (const T*)a.hidden + dep * a.dstride + t * a.Dh;
  float ss = 0.f;
  for (int i = threadIdx.x; i < a.Dh; i += 256) {
    float x = ElemIO<T>::ld(h, i);
    ss += x * x;
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float tot = red[0] + red[1] + red[2] + red[3];
    float iv = tot > 0.f ? 1.f / sqrtf(tot) : 0.f;
    a.inv[dep * a.T + t] = iv;
    a.nrm2[dep * a.T + t] = tot * iv * iv;
  }
}

__device__ __forceinline__ int64_t qround(double x) { return (int64_t)floor(x * QSCALE + 0.5); }

// Largest surprisal of each sequence (one block per sequence).
__global__ __launch_bounds__(256) void surp_max_kernel(PartArgs a) {
  const int s = blockIdx.x;
  float m = -INFINITY;
  for (int64_t t = a.cu[s] + threadIdx.x; t < a.cu[s + 1]; t += 256) m = fmaxf(m, a.surp[t]);
  __shared__ float red[4];
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) a.smax[s] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// kappa_b = mean over valid (depth, window) pairs of
// (1 - cos(h^_b - h^_{b-w}, h^_{b+w} - h^_b)) / 2; the cut bonus adds the
// surprisal over its sequence maximum
template <class T>
__global__ __launch_bounds__(256) void turning_kernel(PartArgs a) {
  int64_t t = blockIdx.x;
  int s = seq_of(a.cu, a.S, t);
  int64_t L = a.cu[s + 1] - a.cu[s];
  int64_t b = t - a.cu[s];
  __shared__ float red[4][3];
  const int ws[2] = {2, 8};
  float acc = 0.f;
  int nval = 0;
  for (int dep = 0; dep < a.nd; ++dep)
  for (int wi = 0; wi < 2; ++wi) {
    const T* H = (const T*)a.hidden + dep * a.dstride;
    const float* inv = a.inv + dep * a.T;
    int w = ws[wi];
    if (b - w < 0 || b + w > L - 1) continue;
    float ib = inv[t], ip = inv[t - w], iq = inv[t + w];
    float uv = 0.f, uu = 0.f, vv = 0.f;
    for (int i = threadIdx.x; i < a.Dh; i += 256) {
      float xb = ElemIO<T>::ld(H, t * a.Dh + i) * ib;
      float u = xb - ElemIO<T>::ld(H, (t - w) * a.Dh + i) * ip;
      float v = ElemIO<T>::ld(H, (t + w) * a.Dh + i) * iq - xb;
      uv += u * v;
      uu += u * u;
      vv += v * v;
    }
    uv = wave_sum(uv);
    uu = wave_sum(uu);
    vv = wave_sum(vv);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
      red[threadIdx.x >> 6][0] = uv;
      red[threadIdx.x >> 6][1] = uu;
      red[threadIdx.x >> 6][2] = vv;
    }
    __syncthreads();
    float UV = red[0][0] + red[1][0] + red[2][0] + red[3][0];
    float UU = red[0][1] + red[1][1] + red[2][1] + red[3][1];
    float VV = red[0][2] + red[1][2] + red[2][2] + red[3][2];
    if (UU > 0.f && VV > 0.f) {
      acc += (1.f - UV / (sqrtf(UU) * sqrtf(VV))) * 0.5f;
      ++nval;
    }
  }
  if (threadIdx.x == 0) {
    float kap = nval ? acc / (float)nval : 0.f;
    double bonus = (double)a.lam_curv * (double)kap;
    if (a.surp && a.smax[s] > 0.f) bonus += (double)a.lam_surp * (double)a.surp[t] / (double)a.smax[s];
    a.cut_q[t] = qround(bonus);
  }
}

// Banded Gram matrix of the normalized trajectory on MFMA:
// G[i][k] = <h^_i, h^_{i+k}> for 0 <= k < BW, tokens of one sequence only.
// Tiles of 32 x 32 token pairs; the bf16 hidden states enter the MFMA as they
// are (products exact, fp32 sums) and the two inverse norms scale the result.
constexpr int BW = 128;   // band width = longest slot
constexpr int GRAM_WAVES = 5;  // one 32x32 tile of the band each (5 tiles cover 128 diagonals + the block)
constexpr int GRAM_UNROLL = 8; // 16-wide k steps whose loads are in flight together
template <class T>
__global__ __launch_bounds__(GRAM_WAVES * 64) void gram_kernel(PartArgs a, float* G) {
  using namespace kvcmf;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // block = 32-row i-block; wave w takes the j-block ib + w
  const int64_t ib = blockIdx.x, dep = blockIdx.y;
  const int64_t i0 = ib * 32;
  if (i0 >= a.T) return;
  const T* H = (const T*)a.hidden + dep * a.dstride;
  const float* inv = a.inv + dep * a.T;
  G += dep * a.T * BW;
  const int jt = wave;
  const int64_t j0 = i0 + (int64_t)jt * 32;
  if (j0 >= a.T) return;
  kvc_f32x16 acc = {};
  // rows past the end re-read the last row (in bounds); their products are never stored
  const int64_t ri = min(i0 + (lane & 31), a.T - 1), rj = min(j0 + (lane & 31), a.T - 1);
  const T* Hi = H + ri * a.Dh + 8 * (lane >> 5);
  const T* Hj = H + rj * a.Dh + 8 * (lane >> 5);
  int c = 0;
  for (; c + 16 * GRAM_UNROLL <= a.Dh; c += 16 * GRAM_UNROLL) {
    Frag<T> fa[GRAM_UNROLL], fb[GRAM_UNROLL];
#pragma unroll
    for (int u = 0; u < GRAM_UNROLL; ++u) {
      fa[u] = load_frag<T>(Hi + c + 16 * u);
      fb[u] = load_frag<T>(Hj + c + 16 * u);
    }
#pragma unroll
    for (int u = 0; u < GRAM_UNROLL; ++u) mma(acc, fa[u], fb[u]);
  }
  for (; c < a.Dh; c += 16) mma(acc, load_frag<T>(Hi + c), load_frag<T>(Hj + c));
  // register v: row i = i0 + acc_row(v), column j = j0 + lane % 32
  const int64_t jj = j0 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t i = i0 + acc_row(v, lane);
    const int64_t kk = jj - i;
    if (i < a.T && jj < a.T && kk >= 0 && kk < BW) G[i * BW + kk] = acc[v] * inv[i] * inv[jj];
  }
}

// Inclusive prefix sums along every band row, in place.
__global__ void band_prefix_kernel(PartArgs a, float* G) {
  int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // row of every depth
  if (g >= a.T * a.nd) return;
  float* r = G + g * BW;
  float run = 0.f;
  for (int k = 0; k < BW; ++k) {
    run += r[k];
    r[k] = run;
  }
}

// One thread per slot END token e (inclusive last token): growing the window
// [a, e] one token to the left adds 2 sum_{j=a+1..e} G[a][j-a] + G[a][0],
// read from the band-row prefix sums.
__global__ __launch_bounds__(256) void window_cost_kernel(PartArgs a, const float* G) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.T) return;
  int s = seq_of(a.cu, a.S, t);
  int64_t p = t - a.cu[s];
  if (p < a.c0[s] || p >= a.c1[s]) return;
  const int ncol = a.nmax - a.nmin + 1;
  int64_t* row = a.cost_q + t * ncol;
  float W[MAXD], sq[MAXD];
#pragma unroll
  for (int dd = 0; dd < MAXD; ++dd) W[dd] = sq[dd] = 0.f;
  for (int n = 1; n <= a.nmax; ++n) {
    int64_t i = p - n + 1;                    // token joining the window
    if (i < a.c0[s]) break;
    int64_t g = a.cu[s] + i;
    double disp = 0.0;
#pragma unroll
    for (int dd = 0; dd < MAXD; ++dd) {
      if (dd >= a.nd) break;
      const float* gr = G + (dd * a.T + g) * BW;
      float g0 = gr[0];
      W[dd] += 2.f * (gr[n - 1] - g0) + g0;
      sq[dd] += a.nrm2[dd * a.T + g];
      disp += (double)sq[dd] - (double)W[dd] / (double)n;
    }
    if (n >= a.nmin) {
      double x = ((double)n - a.target) / (double)a.target;
      row[n - a.nmin] = qround(disp / (double)a.nd + (double)a.lam_len * x * x);
    }
  }
}

// exact integer DP; one 1024-thread block per sequence
constexpr int DP_PF = 4;  // DP steps whose cost loads are in flight
__global__ __launch_bounds__(1024) void dp_kernel(PartArgs a) {
  constexpr int RING = 512;
  __shared__ int64_t fr[RING];
  __shared__ uint8_t arg[32768 + 8];
  const int s = blockIdx.x;
  const int64_t c0 = a.c0[s], c1 = a.c1[s];
  const int64_t Lc = c1 - c0;
  int32_t* out = a.slot_start + (int64_t)s * (a.stride + 1);
  if (Lc <= 0) {
    if (threadIdx.x == 0) {
      a.n_slots[s] = 0;
      out[0] = (int32_t)c0;
    }
    return;
  }
  if (Lc < a.nmin) {
    if (threadIdx.x == 0) {
      a.n_slots[s] = 1;
      out[0] = (int32_t)c0;
      out[1] = (int32_t)c1;
    }
    return;
  }
  const int ncol = a.nmax - a.nmin + 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t gbase = a.cu[s] + c0;    // global token of region position 0
  if (threadIdx.x == 0) fr[0] = 0;
  __syncthreads();
  const int step = a.nmin < 16 ? a.nmin : 16;  // ends that depend only on earlier ends
  // The cost and cut terms do not depend on the recurrence, so their loads run
  // DP_PF steps ahead in a ring of register sets: every load is unconditional
  // (indices clamped into the arrays) and selected away where it does not
  // apply, so the waits before each step stay partial.
  int64_t cqb[DP_PF][2], kqb[DP_PF][2];
  auto issue = [&](int j, int64_t e0s) {
    const int64_t e = min(e0s + wave, Lc);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = min(lane + 64 * q, ncol - 1);
      const int64_t pv = max(e - (a.nmin + c), (int64_t)0);
      cqb[j][q] = a.cost_q[(gbase + e - 1) * ncol + c];
      kqb[j][q] = a.cut_q[gbase + pv];
    }
  };
#pragma unroll
  for (int j = 0; j < DP_PF; ++j) issue(j, 1 + (int64_t)j * step);
  for (int64_t eb = 1; eb <= Lc; eb += (int64_t)DP_PF * step) {
#pragma unroll
    for (int j = 0; j < DP_PF; ++j) {
      const int64_t e0 = eb + (int64_t)j * step;
      if (e0 > Lc) break;
      int64_t e = e0 + wave;               // region-relative end (exclusive)
      int64_t best = INT64_MAX;
      const bool mine = wave < step && e <= Lc;
      if (mine) {
        int64_t fv[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int c = lane + 64 * q;
          const int64_t pv = e - (a.nmin + c);
          fv[q] = (c < ncol && pv >= 0) ? fr[pv % RING] : INF_Q;
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int c = lane + 64 * q;
          if (fv[q] >= INF_Q) continue;
          const int64_t pv = e - (a.nmin + c);
          const int64_t kq = pv > 0 ? kqb[j][q] : 0;
          const int64_t v = fv[q] + cqb[j][q] - kq;
          const int64_t key = v * 256 + (255 - c);
          best = key < best ? key : best;
        }
        best = wave_min_i64(best);
      }
      issue(j, e0 + (int64_t)DP_PF * step);  // this register set now serves a later step
      // no barrier before the writes: this step reads ends e0 - nmax .. e0 - 1
      // and writes e0 .. e0 + step - 1 (step <= nmin, and the ring holds more
      // than nmax + step ends), so no write meets a read of the same step
      if (mine && lane == 0) {
        if (best == INT64_MAX) {
          fr[e % RING] = INF_Q;
          arg[e] = 255;
        } else {
          const int64_t v = best >= 0 ? best / 256 : -((-best + 255) / 256);
          const int c = 255 - (int)(best - v * 256);
          fr[e % RING] = v;
          arg[e] = (uint8_t)c;
        }
      }
      __syncthreads();  // the next step reads these ends
    }
  }
  if (threadIdx.x == 0) {
    // backtrack twice: count, then write the starts in position order
    int m = 0;
    for (int64_t e = Lc; e > 0; e -= a.nmin + arg[e]) ++m;
    a.n_slots[s] = m;
    out[m] = (int32_t)c1;
    int k = m;
    for (int64_t e = Lc; e > 0;) {
      e -= a.nmin + arg[e];
      out[--k] = (int32_t)(c0 + e);
    }
  }
}

__global__ void fixed_slots_kernel(PartArgs a, int slot_len) {
  int s = blockIdx.x;
  int64_t c0 = a.c0[s], c1 = a.c1[s];
  int64_t n = c1 > c0 ? (c1 - c0 + slot_len - 1) / slot_len : 0;
  int32_t* out = a.slot_start + (int64_t)s * (a.stride + 1);
  for (int64_t k = threadIdx.x; k <= n; k += blockDim.x) {
    int64_t v = c0 + k * slot_len;
    out[k] = (int32_t)(v < c1 ? v : c1);
  }
  if (threadIdx.x == 0) a.n_slots[s] = (int32_t)n;
}

}  // namespace

namespace kvc {
size_t ws_partition(const kvc_shape* s, const kvc_params* p) {
  int ncol = p->slot_max - p->slot_min + 1;
  const int nd = p->n_depth > 1 ? p->n_depth : 1;
  Carver c(nullptr, 0);
  c.take<float>((size_t)s->total_tokens * nd);
  c.take<float>((size_t)s->total_tokens * nd);
  c.take<int64_t>((size_t)s->total_tokens * (ncol > 0 ? ncol : 1));
  c.take<int64_t>((size_t)s->total_tokens);
  c.take<float>((size_t)s->total_tokens * BW * nd);
  c.take<float>(64);
  return c.off + 256;
}
}  // namespace kvc

extern "C" int kvc_partition(const kvc_shape* sh, const kvc_params* p, const void* hidden, int32_t hidden_dim,
                             int32_t mode, int64_t* dp_cost_q, int64_t* dp_cut_q, int32_t* slot_start,
                             int32_t* n_slots, void* ws, size_t ws_bytes, hipStream_t st) {
  return kvc_partition_ex(sh, p, hidden, hidden_dim, nullptr, mode, dp_cost_q, dp_cut_q, slot_start, n_slots, ws,
                          ws_bytes, st);
}

extern "C" int kvc_partition_ex(const kvc_shape* sh, const kvc_params* p, const void* hidden, int32_t hidden_dim,
                                const float* surprisal, int32_t mode, int64_t* dp_cost_q, int64_t* dp_cut_q,
                                int32_t* slot_start, int32_t* n_slots, void* ws, size_t ws_bytes, hipStream_t st) {
  int r = kvc::validate_shape(sh);
  if (r) return r;
  if ((r = kvc::validate_params(sh, p))) return r;
  KVC_REQUIRE(!p->token_mode, KVC_E_INVAL, "kvc_partition: token mode has no slots");
  KVC_REQUIRE(sh->n_seq <= 64, KVC_E_SHAPE, "kvc_partition: at most 64 sequences per call");
  KVC_REQUIRE(slot_start && n_slots, KVC_E_INVAL, "kvc_partition: NULL output");
  KVC_REQUIRE(mode == 0 || mode == 1, KVC_E_INVAL, "kvc_partition: mode must be 0 or 1");
  PartArgs a{};
  a.cu = sh->cu_seqlens_d;
  a.S = sh->n_seq;
  a.T = sh->total_tokens;
  a.nmin = p->slot_min;
  a.nmax = p->slot_max;
  a.target = p->slot_target;
  a.stride = kvc_slot_stride(sh, p);
  a.lam_len = p->lambda_len;
  a.lam_curv = p->lambda_curv;
  a.slot_start = slot_start;
  a.n_slots = n_slots;
  for (int s = 0; s < sh->n_seq; ++s) {
    kvc::Regions g = kvc::regions_of(sh->cu_seqlens[s + 1] - sh->cu_seqlens[s], *p);
    a.c0[s] = g.c0;
    a.c1[s] = g.c1;
  }
  if (p->slot_len > 0) {
    hipLaunchKernelGGL(fixed_slots_kernel, dim3(sh->n_seq), dim3(256), 0, st, a, p->slot_len);
    KVC_LAUNCH_CHECK("fixed_slots");
    return KVC_OK;
  }
  KVC_REQUIRE(kvc::max_len(sh) <= 32768, KVC_E_SHAPE, "kvc_partition: DP slots need sequences <= 32768 tokens");
  KVC_REQUIRE(ws && ws_bytes >= kvc::ws_partition(sh, p), KVC_E_WORKSPACE, "kvc_partition: workspace too small");
  int ncol = p->slot_max - p->slot_min + 1;
  KVC_REQUIRE(p->n_depth >= 0 && p->n_depth <= MAXD, KVC_E_INVAL, "kvc_partition: n_depth must be in [1, 4]");
  a.nd = p->n_depth > 1 ? p->n_depth : 1;
  a.dstride = sh->total_tokens * (int64_t)hidden_dim;
  a.surp = surprisal;
  a.lam_surp = p->lambda_surp;
  kvc::Carver c(ws, ws_bytes);
  a.inv = c.take<float>((size_t)sh->total_tokens * a.nd);
  a.nrm2 = c.take<float>((size_t)sh->total_tokens * a.nd);
  int64_t* cq = c.take<int64_t>((size_t)sh->total_tokens * ncol);
  int64_t* kq = c.take<int64_t>((size_t)sh->total_tokens);
  float* gband = c.take<float>((size_t)sh->total_tokens * BW * a.nd);
  a.smax = c.take<float>(64);
  if (mode == 1) {
    KVC_REQUIRE(dp_cost_q && dp_cut_q, KVC_E_INVAL, "kvc_partition: mode 1 needs dp_cost_q and dp_cut_q");
    a.cost_q = dp_cost_q;
    a.cut_q = dp_cut_q;
  } else {
    KVC_REQUIRE(hidden && hidden_dim >= 1 && hidden_dim <= 4096, KVC_E_INVAL,
                "kvc_partition: hidden states with 1 <= hidden_dim <= 4096 are required");
    a.hidden = hidden;
    a.Dh = hidden_dim;
    a.cost_q = dp_cost_q ? dp_cost_q : cq;
    a.cut_q = dp_cut_q ? dp_cut_q : kq;
    KVC_REQUIRE(p->slot_max <= BW, KVC_E_UNSUPPORTED, "kvc_partition: slot_max above 128");
    KVC_REQUIRE(hidden_dim % 16 == 0, KVC_E_SHAPE, "kvc_partition: hidden_dim must be a multiple of 16");
    dim3 gt((unsigned)sh->total_tokens), gn((unsigned)sh->total_tokens, (unsigned)a.nd);
    dim3 gg(kvc_blocks(sh->total_tokens, 32), (unsigned)a.nd), gw(kvc_blocks(sh->total_tokens, 256));
    if (sh->total_tokens > 0) {
      if (surprisal) {
        hipLaunchKernelGGL(surp_max_kernel, dim3(sh->n_seq), dim3(256), 0, st, a);
        KVC_LAUNCH_CHECK("surp_max");
      }
      if (sh->dtype == KVC_BF16) {
        hipLaunchKernelGGL(norm_kernel<uint16_t>, gn, dim3(256), 0, st, a);
        hipLaunchKernelGGL(turning_kernel<uint16_t>, gt, dim3(256), 0, st, a);
        hipLaunchKernelGGL(gram_kernel<uint16_t>, gg, dim3(GRAM_WAVES * 64), 0, st, a, gband);
      } else {
        hipLaunchKernelGGL(norm_kernel<float>, gn, dim3(256), 0, st, a);
        hipLaunchKernelGGL(turning_kernel<float>, gt, dim3(256), 0, st, a);
        hipLaunchKernelGGL(gram_kernel<float>, gg, dim3(GRAM_WAVES * 64), 0, st, a, gband);
      }
      hipLaunchKernelGGL(band_prefix_kernel, dim3(kvc_blocks(sh->total_tokens * a.nd, 256)), dim3(256), 0, st, a,
                         gband);
      hipLaunchKernelGGL(window_cost_kernel, gw, dim3(256), 0, st, a, (const float*)gband);
      KVC_LAUNCH_CHECK("partition_costs");
    }
  }
  hipLaunchKernelGGL(dp_kernel, dim3(sh->n_seq), dim3(1024), 0, st, a);
  KVC_LAUNCH_CHECK("partition_dp");
  return KVC_OK;
}
