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
#include "mfma_frag.h"

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

// hi/lo bf16 split of 8 fp32 softmax weights (for the fp32-accurate MFMA)
__device__ __forceinline__ void split8(const float* x, kvc_bf16x8& hi, kvc_bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t u = __float_as_uint(x[j]) & 0xffff0000u;
    float r = x[j] - __uint_as_float(u);
    hi[j] = __builtin_bit_cast(__bf16, (uint16_t)(u >> 16));
    lo[j] = __builtin_bit_cast(__bf16, f32_to_bf16_bits(r));
  }
}

template <class T, int D>
__global__ __launch_bounds__(THREADS) void tree_kernel(TreeKArgs a) {
  using namespace kvcmf;
  constexpr int HD = D / 2;
  constexpr int KS = D / 16;
  constexpr int NPV = 136;   // token stride of the transposed values (68 dwords: b128 reads conflict-free)
  constexpr int NPA = 132;   // token stride of the transposed softmax weights
  extern __shared__ __align__(16) char smem[];
  const int nmax = a.nmax;
  float* Kt = (float*)smem;                                        // [nmax][D] unrotated keys (fp32)
  T* Vt = (T*)(Kt + (size_t)nmax * D);                             // [D][NPV] values, transposed
  float* At = (float*)(Vt + (size_t)D * NPV);                      // [PDMAX][NPA] softmax weights
  float* lse_s = At + (size_t)PDMAX * NPA;                         // [PDMAX]
  float* knorm = lse_s + PDMAX;                                    // [nmax]
  float* rtok = knorm + nmax;                                      // [nmax]
  float* nrel = rtok + nmax;                                       // [2 nmax]
  float* nD = nrel + 2 * nmax;                                     // [2 nmax]
  float* nmu = nD + 2 * nmax;                                      // [2 nmax]
  int16_t* nst = (int16_t*)(nmu + 2 * nmax);                       // [2 nmax]
  int16_t* nsz = nst + 2 * nmax;                                   // [2 nmax]
  float* scratch = (float*)(nsz + 2 * nmax);                       // [WAVES][2][D]

  int64_t b = blockIdx.x;
  const int k = (int)(b % a.stride);
  int64_t rest = b / a.stride;
  const int s = (int)(rest % a.S);
  const int64_t lh = rest / a.S;
  if (k >= a.n_slots[s]) return;
  const int l = (int)(lh / a.H), h = (int)(lh % a.H);
  const int32_t* ss = a.slot_start + (int64_t)s * (a.stride + 1);
  const int t0 = ss[k], n = ss[k + 1] - ss[k];
  const int n16 = (n + 15) & ~15;
  const int m = 2 * n - 1;
  const int64_t tok0 = a.cu[s] + t0;
  const int64_t obase = lh * 2 * a.T + 2 * tok0;
  const T* Kg = (const T*)a.K + (lh * a.T + tok0) * D;
  const T* Vg = (const T*)a.V + (lh * a.T + tok0) * D;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = (s * a.Ly + l) * a.H + h;
  const float sens = a.sens[unit];
  const T* Qu = (const T*)a.Qp + ((((int64_t)s * a.Ly + l) * a.H * a.G + (int64_t)h * a.G) * a.P) * D;

  // ---- stage transposed values (bf16; zero past the slot up to a 16 multiple),
  // lse, r, node table; unrotated keys and key norms straight from HBM
  for (int i = tid; i < n16 * (D / 8); i += THREADS) {
    int r = i / (D / 8), c = (i % (D / 8)) * 8;
    float x[8];
    if (r < n) Load8<T>::f(Vg + (int64_t)r * D + c, x);
    else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ElemIO<T>::st(Vt, (int64_t)(c + j) * NPV + r, x[j]);
  }
  for (int rho = tid; rho < a.pd; rho += THREADS) lse_s[rho] = a.lse[(int64_t)unit * a.G * a.P + (int64_t)rho * a.pstride];
  for (int i = tid; i < n; i += THREADS) rtok[i] = a.rel[lh * a.T + tok0 + i];
  for (int j = tid; j < m; j += THREADS) {
    int cur = 0, st = 0, sz = n;
    while (cur != j) {
      int nl = (sz + 1) >> 1;
      if (j < cur + 2 * nl) {
        cur += 1;
        sz = nl;
      } else {
        cur += 2 * nl;
        st += nl;
        sz -= nl;
      }
    }
    nst[j] = (int16_t)st;
    nsz[j] = (int16_t)sz;
  }
  for (int it = tid; it < n * HD; it += THREADS) {
    int i = it / HD, p = it % HD;
    float x0 = ElemIO<T>::ld(Kg, (int64_t)i * D + p), x1 = ElemIO<T>::ld(Kg, (int64_t)i * D + p + HD);
    int64_t pos = t0 + i;
    float c = a.rc[pos * HD + p], sn = a.rs[pos * HD + p];
    Kt[(size_t)i * D + p] = x0 * c + x1 * sn;       // rotation by -theta
    Kt[(size_t)i * D + p + HD] = x1 * c - x0 * sn;
  }
  for (int i = tid; i < n; i += THREADS) {
    float q = 0.f;
    for (int c = 0; c < D; c += 8) {
      float x[8];
      Load8<T>::f(Kg + (int64_t)i * D + c, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) q += x[j] * x[j];
    }
    knorm[i] = sqrtf(q);
  }
  // softmax weights of the distortion rows on MFMA (K Q^T), stored transposed;
  // zero for tokens past the slot up to the 16 multiple
  {
    const int ntb = (n16 + 31) / 32, nrb = (a.pd + 31) / 32;
    for (int tile = wave; tile < ntb * nrb; tile += WAVES) {
      int tb = tile / nrb, rb = tile % nrb;
      int tok = tb * 32 + (lane & 31), rho = rb * 32 + (lane & 31);
      kvc_f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        int c = ks * 16 + 8 * (lane >> 5);
        Frag<T> ka = tok < n ? load_frag<T>(Kg + (int64_t)tok * D + c) : zero_frag<T>();
        Frag<T> qb = rho < a.pd ? load_frag<T>(Qu + (int64_t)rho * a.pstride * D + c) : zero_frag<T>();
        mma(acc, ka, qb);
      }
      float ls = rho < a.pd ? a.lse[(int64_t)unit * a.G * a.P + (int64_t)rho * a.pstride] : 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        int ti = tb * 32 + acc_row(v, lane);
        if (ti < n16 && rho < PDMAX)
          At[rho * NPA + ti] = (ti < n && rho < a.pd) ? expf(acc[v] * a.c - ls) : 0.f;
      }
    }
  }
  __syncthreads();
  // ---- bottom-up value flow by height (a parent is the exact fp32 sum of its
  // children; children of pre-order node j are j+1 and j + 2 ceil(sz/2))
  for (int j = tid; j < m; j += THREADS)
    if (nsz[j] == 1) nrel[j] = rtok[nst[j]];
  __syncthreads();
  for (int ht = 1; (1 << (ht - 1)) < n; ++ht) {
    for (int j = tid; j < m; j += THREADS) {
      int sz = nsz[j];
      if (sz > 1 && 32 - __clz(sz - 1) == ht) nrel[j] = nrel[j + 1] + nrel[j + 2 * ((sz + 1) >> 1)];
    }
    __syncthreads();
  }
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
    if (lane < HD) {
#pragma unroll 8
      for (int i = st; i < st + sz; ++i) {
        s0 += Kt[(size_t)i * D + lane];
        s1 += Kt[(size_t)i * D + lane + HD];
        kn += knorm[i];
      }
    }
    float nrm2 = wave_sum(lane < HD ? s0 * s0 + s1 * s1 : 0.f);
    kn = __shfl(kn, 0, 64);
    float coh = kn > 0.f ? sqrtf(nrm2) / kn : 1.f;
    float mu = fmaxf(1.f, (float)sz * coh);
    if (lane < HD) {
      float m0 = s0 / (float)sz, m1 = s1 / (float)sz;
      int64_t prep = t0 + st + (sz - 1) / 2;
      float c = a.rc[prep * HD + lane], sn = a.rs[prep * HD + lane];
      kh[lane] = m0 * c - m1 * sn;
      kh[lane + HD] = m1 * c + m0 * sn;
    }
    // prototype value: (1 - beta) r_i / rel + beta / n, lane = dimension
    for (int dd = lane; dd < D; dd += 64) {
      float acc = 0.f;
#pragma unroll 8
      for (int i = st; i < st + sz; ++i) {
        float w = reln > 0.f ? (1.f - a.beta) * rtok[i] / reln + a.beta / (float)sz : 1.f / (float)sz;
        acc += w * ElemIO<T>::ld(Vt, (int64_t)dd * NPV + i);
      }
      vh[dd] = acc;
    }
    __builtin_amdgcn_wave_barrier();  // kh/vh written by this wave's lanes, read below
    // lane rho: Z and Z_hat
    float z = 0.f, zh = 0.f;
    if (lane < a.pd) {
      for (int i = st; i < st + sz; ++i) z += At[lane * NPA + i];
      const T* qr = Qu + (int64_t)lane * a.pstride * D;
      float dot = 0.f;
#pragma unroll 4
      for (int c = 0; c < D; c += 8) {
        float x[8];
        Load8<T>::f(qr + c, x);
        float4 k0 = *(const float4*)(kh + c), k1 = *(const float4*)(kh + c + 4);
        dot += x[0] * k0.x + x[1] * k0.y + x[2] * k0.z + x[3] * k0.w + x[4] * k1.x + x[5] * k1.y +
               x[6] * k1.z + x[7] * k1.w;
      }
      zh = mu * expf(dot * a.c - lse_s[lane]);
    }
    // u^T = V_node^T A_node^T on MFMA: rows = value dims, columns = probe rows;
    // lane keeps column rho = pb*32 + lane%32 and 16 of the 32 rows of a tile
    float eVn = 0.f, eVd = 0.f;
    const int kb0 = st >> 4, kb1 = (st + sz + 15) >> 4;
#pragma unroll 1
    for (int pb = 0; pb < (a.pd + 31) / 32; ++pb) {
      const int rho = pb * 32 + (lane & 31);
      const float zr = __shfl(z, rho, 64);
      float n1 = 0.f, n2 = 0.f;
#pragma unroll 1
      for (int db = 0; db < D / 32; ++db) {
        kvc_f32x16 acc = {};
        for (int kb = kb0; kb < kb1; ++kb) {
          const int t8 = kb * 16 + 8 * (lane >> 5);
          Frag<T> va = load_frag<T>(Vt + (size_t)(db * 32 + (lane & 31)) * NPV + t8);
          float w8[8];
          float4 w0 = *(const float4*)(At + rho * NPA + t8), w1 = *(const float4*)(At + rho * NPA + t8 + 4);
          w8[0] = w0.x; w8[1] = w0.y; w8[2] = w0.z; w8[3] = w0.w;
          w8[4] = w1.x; w8[5] = w1.y; w8[6] = w1.z; w8[7] = w1.w;
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (t8 + q < st || t8 + q >= st + sz) w8[q] = 0.f;   // tokens outside the node
          if constexpr (sizeof(T) == 2) {
            Frag<uint16_t> hi, lo;
            split8(w8, hi.v, lo.v);
            mma(acc, va, hi);
            mma(acc, va, lo);
          } else {
            Frag<float> wf;
#pragma unroll
            for (int q = 0; q < 8; ++q) wf.v[q] = w8[q];
            mma(acc, va, wf);
          }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float u = acc[v];
          float df = u - zr * vh[db * 32 + acc_row(v, lane)];
          n1 += df * df;
          n2 += u * u;
        }
      }
      n1 += __shfl_xor(n1, 32, 64);
      n2 += __shfl_xor(n2, 32, 64);
      if (lane < 32 && rho < a.pd) {
        eVn += sqrtf(n1);
        eVd += sqrtf(n2);
      }
    }
    float eAn = lane < a.pd ? fabsf(zh - z) : 0.f, eAd = lane < a.pd ? z : 0.f;
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
    } else if (q - 1 < m && nsz[q - 1] > 1) {
      int j = q - 1, lc = j + 1, rc = j + 2 * ((nsz[j] + 1) >> 1);
      float gain = nrel[j] * nD[j] - (nrel[lc] * nD[lc] + nrel[rc] * nD[rc]);
      u = sens * gain;
      cst = 1;
    }
    a.op_util[obase + q] = u;
    a.op_cost[obase + q] = cst;
  }
}

size_t tree_smem(int nmax, int d, int elt) {
  size_t b = (size_t)nmax * d * 4;                  // unrotated keys
  b += (size_t)d * 136 * elt;                       // transposed values
  b += (size_t)PDMAX * 132 * 4;                     // transposed softmax weights
  b += PDMAX * 4 + (size_t)nmax * 4 * 2;            // lse, norms, r
  b += (size_t)2 * nmax * 4 * 3 + (size_t)2 * nmax * 2 * 2;  // node values, starts, sizes
  b += (size_t)WAVES * 2 * d * 4;                   // per-wave prototype scratch
  return b;
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
  a.nmax = (slot_nmax(p) + 7) & ~7;  // LDS layout keeps every array 16-byte aligned
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
