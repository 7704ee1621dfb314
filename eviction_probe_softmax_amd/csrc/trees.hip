// Prototype trees per (sequence, layer, KV head, slot).
//
// GraceKV page: '02 Progressively refinable representation' (one tree per
// (layer, KV head, slot); a frontier is how the slot is stored); 'Inside one
// cache entry' (key: inverse-rotate, average, re-rotate at a representative
// position; value: relevance weighted with a 10% uniform base; multiplicity
// from key coherence); '03 Bottom-up value flow' (a parent's value is the sum
// of its children's); technical details (probe-based distortion,
// attention-partition : value-aggregate error = 0.25 : 0.75); '04 Top-down
// budget flow' (utility per entry = relevance x fidelity gain x head
// sensitivity / new entries).
//
// One workgroup per slot. The slot's keys, values, the distortion probe rows
// and their softmax weights a[i][rho] = exp(<q_rho,k_i>/sqrt d - lse_rho) sit
// in LDS; node relevance is summed bottom-up by one thread (so a parent is
// exactly the fp32 sum of its children); the internal nodes are independent
// and spread over the waves. Per node a wave forms the prototype key (lane =
// rotate-half pair) and value, then lane rho accumulates
// u_rho = sum_node a[i][rho] v_i in registers so that ||u_rho - Z_rho v^|| and
// ||u_rho|| never leave the lane.
#include <cmath>

#include "kvc_internal.h"

namespace {

constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int PDMAX = 64;

struct TreeKArgs {
  const void* K;
  const void* V;
  const void* Qp;
  const float* lse;        // [S][Ly][H*G][P]
  const float* rel;        // [Ly][H][T]
  const float* sens;       // [S][Ly][H]
  const float* rc;
  const float* rs;
  const int32_t* slot_start;
  const int32_t* n_slots;
  const int64_t* cu;
  int S, Ly, H, G, P, stride, nmax, pd, pstride;
  int64_t T;
  float c;                 // 1/sqrt(d)
  float beta, wA, wV;
  float* node_rel;
  float* node_D;
  float* node_mu;
  float* op_util;
  uint8_t* op_cost;
};

template <class T, int D>
__global__ __launch_bounds__(THREADS) void tree_kernel(TreeKArgs a) {
  constexpr int HD = D / 2;
  extern __shared__ __align__(16) char smem[];
  const int nmax = a.nmax;
  T* Kl = (T*)smem;                                   // [nmax][D]
  T* Vl = Kl + (size_t)nmax * D;                      // [nmax][D]
  float* A = (float*)(Vl + (size_t)nmax * D);         // [nmax][PDMAX]
  T* Ql = (T*)(A + (size_t)nmax * PDMAX);             // [D][PDMAX]
  float* lse_s = (float*)(Ql + (size_t)D * PDMAX);    // [PDMAX]
  float* knorm = lse_s + PDMAX;                       // [nmax]
  float* rtok = knorm + nmax;                         // [nmax]
  float* nrel = rtok + nmax;                          // [2 nmax]
  float* nD = nrel + 2 * nmax;                        // [2 nmax]
  float* nmu = nD + 2 * nmax;                         // [2 nmax]
  int* nst = (int*)(nmu + 2 * nmax);                  // [2 nmax]
  int* nsz = nst + 2 * nmax;
  int* nlc = nsz + 2 * nmax;
  int* nrc = nlc + 2 * nmax;
  float* scratch = (float*)(nrc + 2 * nmax);          // [WAVES][2][D]
  __shared__ int n_nodes;

  int64_t b = blockIdx.x;
  const int k = (int)(b % a.stride);
  int64_t rest = b / a.stride;
  const int s = (int)(rest % a.S);
  const int64_t lh = rest / a.S;
  if (k >= a.n_slots[s]) return;
  const int l = (int)(lh / a.H), h = (int)(lh % a.H);
  const int32_t* ss = a.slot_start + (int64_t)s * (a.stride + 1);
  const int t0 = ss[k], n = ss[k + 1] - ss[k];
  const int64_t tok0 = a.cu[s] + t0;
  const int64_t obase = lh * 2 * a.T + 2 * tok0;
  const T* Kg = (const T*)a.K + (lh * a.T + tok0) * D;
  const T* Vg = (const T*)a.V + (lh * a.T + tok0) * D;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = (s * a.Ly + l) * a.H + h;
  const float sens = a.sens[unit];

  // ---- stage K, V, distortion probe rows (transposed), lse, relevance
  for (int i = tid; i < n * D; i += THREADS) {
    Kl[i] = Kg[i];
    Vl[i] = Vg[i];
  }
  const T* Qu = (const T*)a.Qp + ((((int64_t)s * a.Ly + l) * a.H * a.G + (int64_t)h * a.G) * a.P) * D;
  for (int i = tid; i < a.pd * D; i += THREADS) {
    int rho = i / D, dd = i % D;
    Ql[dd * PDMAX + rho] = Qu[(int64_t)rho * a.pstride * D + dd];
  }
  for (int rho = tid; rho < a.pd; rho += THREADS) lse_s[rho] = a.lse[(int64_t)unit * a.G * a.P + (int64_t)rho * a.pstride];
  for (int i = tid; i < n; i += THREADS) rtok[i] = a.rel[lh * a.T + tok0 + i];
  if (tid == 0) {
    // pre-order node table: pop, number, push right then left
    int fs[24], fz[24], fp[24], fd[24], top = 0, m = 0;
    fs[top] = 0; fz[top] = n; fp[top] = -1; fd[top] = 0; ++top;
    while (top > 0) {
      --top;
      int st = fs[top], sz = fz[top], par = fp[top], side = fd[top];
      int j = m++;
      nst[j] = st;
      nsz[j] = sz;
      nlc[j] = -1;
      nrc[j] = -1;
      if (par >= 0) {
        if (side == 0) nlc[par] = j;
        else nrc[par] = j;
      }
      if (sz > 1) {
        int nl = (sz + 1) >> 1;
        fs[top] = st + nl; fz[top] = sz - nl; fp[top] = j; fd[top] = 1; ++top;
        fs[top] = st; fz[top] = nl; fp[top] = j; fd[top] = 0; ++top;
      }
    }
    n_nodes = m;
  }
  __syncthreads();
  // key norms (rotation keeps the norm) and softmax weights of the probe rows
  for (int i = tid; i < n; i += THREADS) {
    float q = 0.f;
    for (int dd = 0; dd < D; ++dd) {
      float x = ElemIO<T>::ld(Kl, (int64_t)i * D + dd);
      q += x * x;
    }
    knorm[i] = sqrtf(q);
  }
  for (int i = tid; i < n * PDMAX; i += THREADS) {
    int t = i / PDMAX, rho = i % PDMAX;
    float v = 0.f;
    if (rho < a.pd) {
      float dot = 0.f;
      for (int dd = 0; dd < D; ++dd) dot += ElemIO<T>::ld(Ql, dd * PDMAX + rho) * ElemIO<T>::ld(Kl, (int64_t)t * D + dd);
      v = expf(dot * a.c - lse_s[rho]);
    }
    A[i] = v;
  }
  if (tid == 0) {
    // bottom-up value flow: reverse pre-order visits children before parents
    for (int j = n_nodes - 1; j >= 0; --j) nrel[j] = nlc[j] < 0 ? rtok[nst[j]] : nrel[nlc[j]] + nrel[nrc[j]];
  }
  __syncthreads();
  const int m = n_nodes;
  float* kh = scratch + (size_t)wave * 2 * D;
  float* vh = kh + D;
  for (int j = wave; j < m; j += WAVES) {
    const int st = nst[j], sz = nsz[j];
    if (sz == 1) {
      if (lane == 0) {
        nD[j] = 0.f;
        nmu[j] = 1.f;
      }
      continue;
    }
    const float reln = nrel[j];
    // prototype key and coherence: lane = rotate-half pair
    float s0 = 0.f, s1 = 0.f, kn = 0.f;
    for (int i = st; i < st + sz; ++i) kn += knorm[i];
    if (lane < HD) {
      for (int i = st; i < st + sz; ++i) {
        float x0 = ElemIO<T>::ld(Kl, (int64_t)i * D + lane), x1 = ElemIO<T>::ld(Kl, (int64_t)i * D + lane + HD);
        int64_t pos = t0 + i;
        float c = a.rc[pos * HD + lane], sn = a.rs[pos * HD + lane];
        s0 += x0 * c + x1 * sn;
        s1 += x1 * c - x0 * sn;
      }
    }
    float nrm2 = wave_sum(lane < HD ? s0 * s0 + s1 * s1 : 0.f);
    float coh = kn > 0.f ? sqrtf(nrm2) / kn : 1.f;
    float mu = fmaxf(1.f, (float)sz * coh);
    if (lane < HD) {
      float m0 = s0 / (float)sz, m1 = s1 / (float)sz;
      int64_t prep = t0 + st + (sz - 1) / 2;
      float c = a.rc[prep * HD + lane], sn = a.rs[prep * HD + lane];
      kh[lane] = m0 * c - m1 * sn;
      kh[lane + HD] = m1 * c + m0 * sn;
    }
    for (int dd = lane; dd < D; dd += 64) {
      float acc = 0.f;
      for (int i = st; i < st + sz; ++i) {
        float w = reln > 0.f ? (1.f - a.beta) * rtok[i] / reln + a.beta / (float)sz : 1.f / (float)sz;
        acc += w * ElemIO<T>::ld(Vl, (int64_t)i * D + dd);
      }
      vh[dd] = acc;
    }
    __builtin_amdgcn_wave_barrier();  // kh/vh written by this wave's lanes, read below
    // lane rho: Z, Z_hat and the value aggregate u_rho
    float eAn = 0.f, eAd = 0.f, eVn = 0.f, eVd = 0.f;
    if (lane < a.pd) {
      const int rho = lane;
      float dot = 0.f;
      for (int dd = 0; dd < D; ++dd) dot += ElemIO<T>::ld(Ql, dd * PDMAX + rho) * kh[dd];
      float zh = mu * expf(dot * a.c - lse_s[rho]);
      float z = 0.f;
      for (int i = st; i < st + sz; ++i) z += A[i * PDMAX + rho];
      float u[D];
#pragma unroll
      for (int dd = 0; dd < D; ++dd) u[dd] = 0.f;
      for (int i = st; i < st + sz; ++i) {
        float ai = A[i * PDMAX + rho];
#pragma unroll
        for (int dd = 0; dd < D; ++dd) u[dd] += ai * ElemIO<T>::ld(Vl, (int64_t)i * D + dd);
      }
      float n1 = 0.f, n2 = 0.f;
#pragma unroll
      for (int dd = 0; dd < D; ++dd) {
        float df = u[dd] - z * vh[dd];
        n1 += df * df;
        n2 += u[dd] * u[dd];
      }
      eAn = fabsf(zh - z);
      eAd = z;
      eVn = sqrtf(n1);
      eVd = sqrtf(n2);
    }
    eAn = wave_sum(eAn);
    eAd = wave_sum(eAd);
    eVn = wave_sum(eVn);
    eVd = wave_sum(eVd);
    if (lane == 0) {
      float eA = eAd > 0.f ? eAn / eAd : 0.f;
      float eV = eVd > 0.f ? eVn / eVd : 0.f;
      nD[j] = fminf(1.f, a.wA * eA + a.wV * eV);
      nmu[j] = mu;
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // ---- outputs: node arrays and op utilities
  for (int j = tid; j < m; j += THREADS) {
    a.node_rel[obase + j] = nrel[j];
    a.node_D[obase + j] = nD[j];
    a.node_mu[obase + j] = nmu[j];
  }
  for (int q = tid; q < 2 * n; q += THREADS) {
    float u = 0.f;
    uint8_t cst = 0;
    if (q == 0) {
      u = sens * (nrel[0] * (1.f - nD[0]));
      cst = 1;
    } else if (q - 1 < m && nlc[q - 1] >= 0) {
      int j = q - 1, lc = nlc[j], rc = nrc[j];
      float gain = nrel[j] * nD[j] - (nrel[lc] * nD[lc] + nrel[rc] * nD[rc]);
      u = sens * gain;
      cst = 1;
    }
    a.op_util[obase + q] = u;
    a.op_cost[obase + q] = cst;
  }
}

size_t tree_smem(int nmax, int d, int elt) {
  size_t b = (size_t)nmax * d * elt * 2;
  b += (size_t)nmax * PDMAX * 4;
  b += (size_t)d * PDMAX * elt;
  b += PDMAX * 4 + (size_t)nmax * 4 * 2;
  b += (size_t)2 * nmax * 4 * 3 + (size_t)2 * nmax * 4 * 4;
  b += (size_t)WAVES * 2 * d * 4;
  return b + 64;
}

int slot_nmax(const kvc_params* p) { return p->slot_len > 0 ? p->slot_len : p->slot_max; }

}  // namespace

namespace kvc {
size_t ws_trees(const kvc_shape*, const kvc_params*) { return 0; }
}  // namespace kvc

extern "C" int kvc_build_trees(const kvc_shape* sh, const kvc_params* p, const void* K, const void* V,
                               const void* Qprobe, const float* probe_lse, const float* rel, const float* head_sens,
                               const float* rope_cos, const float* rope_sin, const int32_t* slot_start,
                               const int32_t* n_slots, kvc_trees* out, void* ws, size_t ws_bytes,
                               hipStream_t st) {
  int r = kvc::validate_shape(sh);
  if (r) return r;
  if ((r = kvc::validate_params(sh, p))) return r;
  KVC_REQUIRE(!p->token_mode, KVC_E_INVAL, "kvc_build_trees: token mode has no trees");
  KVC_REQUIRE(K && V && Qprobe && probe_lse && rel && head_sens && rope_cos && rope_sin && slot_start && n_slots &&
                  out && out->node_rel && out->node_D && out->node_mu && out->op_util && out->op_cost,
              KVC_E_INVAL, "kvc_build_trees: NULL pointer");
  TreeKArgs a{};
  a.K = K;
  a.V = V;
  a.Qp = Qprobe;
  a.lse = probe_lse;
  a.rel = rel;
  a.sens = head_sens;
  a.rc = rope_cos;
  a.rs = rope_sin;
  a.slot_start = slot_start;
  a.n_slots = n_slots;
  a.cu = sh->cu_seqlens_d;
  a.S = sh->n_seq;
  a.Ly = sh->n_layers;
  a.H = sh->n_kv_heads;
  a.G = sh->group;
  a.P = p->n_probe;
  a.stride = kvc_slot_stride(sh, p);
  a.nmax = slot_nmax(p);
  int R = sh->group * p->n_probe;
  a.pd = p->n_dprobe < R ? p->n_dprobe : R;
  a.pstride = R / a.pd;
  a.T = sh->total_tokens;
  a.c = 1.0f / sqrtf((float)sh->head_dim);
  a.beta = p->value_base;
  a.wA = p->w_attn;
  a.wV = p->w_value;
  a.node_rel = out->node_rel;
  a.node_D = out->node_D;
  a.node_mu = out->node_mu;
  a.op_util = out->op_util;
  a.op_cost = out->op_cost;
  int d = sh->head_dim;
  int elt = sh->dtype == KVC_BF16 ? 2 : 4;
  size_t sm = tree_smem(a.nmax, d, elt);
  KVC_REQUIRE(sm <= 160 * 1024, KVC_E_UNSUPPORTED, "kvc_build_trees: slot too large for LDS at this dtype/head_dim");
  int64_t nb = (int64_t)sh->n_layers * sh->n_kv_heads * sh->n_seq * a.stride;
  if (nb == 0) return KVC_OK;
#define KVC_TREE_LAUNCH(TT, DD)                                                                             \
  do {                                                                                                      \
    (void)hipFuncSetAttribute((const void*)tree_kernel<TT, DD>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                              (int)sm);                                                                     \
    hipLaunchKernelGGL((tree_kernel<TT, DD>), dim3((unsigned)nb), dim3(THREADS), sm, st, a);                 \
  } while (0)
  if (sh->dtype == KVC_BF16) {
    if (d == 128) KVC_TREE_LAUNCH(uint16_t, 128);
    else KVC_TREE_LAUNCH(uint16_t, 64);
  } else {
    if (d == 128) KVC_TREE_LAUNCH(float, 128);
    else KVC_TREE_LAUNCH(float, 64);
  }
#undef KVC_TREE_LAUNCH
  KVC_LAUNCH_CHECK("tree_build");
  (void)ws;
  (void)ws_bytes;
  return KVC_OK;
}
