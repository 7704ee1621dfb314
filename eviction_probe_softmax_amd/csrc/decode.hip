// One decode step of attention over a ragged (compressed or full) cache.
//
// GraceKV page, '05 Physical cache packing': decoding reads the physical
// ragged cache and newly generated tokens are appended with multiplicity one;
// 'Inside one cache entry': a prototype counts for mu tokens (logit + ln mu).
// DistillCache paper, Sec. 3.1.3: the full and the pruned cache both append
// each new (k, v).
//
// Split-K over pieces. A plan, made once per cache by a one-workgroup kernel,
// cuts every (s, l, h) segment into near-equal pieces of at most `chunk`
// entries and writes one 32-byte record per piece, so a decode step launches
// the pieces there are and no more (a 25% cache launches a quarter of the
// full cache's workgroups, each with a full share of work) and a workgroup
// needs one load before its first K load. The appended tail tokens of every
// unit form pieces of their own after the segment pieces, computed from the
// step's tail length. Each piece computes its G query heads' logits, a local
// softmax and the weighted value sum, and writes (o[G][D], (max, sum)[G]).
// The merge kernel combines the pieces of every unit into o; a third launch
// sums o over the layers, in layer order, into x (the launch boundary is
// what makes every unit's o visible to it). The step is HBM-bound: every
// packed K and V byte is read once, 16 bytes per lane.
#include <cmath>
#include <mutex>
#include <string>

#include "kvc_internal.h"
#include "mfma_frag.h"

namespace {

constexpr int CHUNK = 256;   // entries per piece, at most: fp32 caches (VALU kernel)
constexpr int MCHUNK = 768;  // entries per piece, at most: bf16 caches (MFMA kernel)
constexpr int THREADS = 256;
constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_PER = 8;  // units per plan thread per round, at most
// waves of a merge workgroup (LDS holds one G*D row per wave): wide
// workgroups when there are few units (one wave-batch of pieces each), narrow
// ones when there are many, so that more of them are resident at once
template <int G> constexpr int mrg_waves() { return G <= 4 ? 16 : 8; }
constexpr int MRG_NARROW = 4;
constexpr int64_t MRG_NARROW_UNITS = 1024;  // units from which the narrow merge is used
constexpr int MRG_NPW = 4;    // pieces per wave per merge batch of loads
constexpr float LOG2E = 1.4426950408889634f;

// What a segment piece's workgroup needs, in one 32-byte load.
struct __align__(16) PieceRec {
  int64_t off;  // first row of the piece in the packed cache
  int32_t u;    // unit (s*Ly + l)*H + h
  int32_t n;    // entries in the piece (>= 1)
  int32_t pad0, pad1, pad2, pad3;
};

struct DecArgs {
  const void* K;
  const void* V;
  const float* lnmu;
  const int64_t* seg_off;
  const int32_t* seg_len;
  const void* Kt;
  const void* Vt;
  const void* Q;
  int S, Ly, H, G, D, t_valid, t_cap;
  int chunk;     // entries per piece, at most (CHUNK or MCHUNK)
  int maxs;      // segment pieces the plan can hold; tail pieces start here
  int ntp;       // tail pieces per unit in this step
  float scale2;  // log2(e)/sqrt(d)
  // the plan
  int32_t* n_pieces;  // [1] segment pieces in use (<= maxs)
  PieceRec* piece;    // [maxs]
  int2* upieces;      // [units] (first segment piece, segment pieces) of each unit
  // results
  float* part_o;      // [maxs + units*ntp][G][D] value sums of each piece, scaled by 2^-max
  float2* part_ml;    // [maxs + units*ntp][G] (max of the base-2 logits, sum of 2^(z - max))
  float* o;           // [units][G][D]
  float* x;
  int64_t x_stride;
};

// The plan: pieces per unit (ceil(len / chunk), the length split evenly, the
// first len % np pieces one entry longer), an exclusive scan over the units
// (rounds of PLAN_THREADS * per units), one record per piece, each unit's
// piece range and the number of pieces.
__global__ __launch_bounds__(PLAN_THREADS) void decode_plan_kernel(DecArgs a) {
  __shared__ int wsum[PLAN_THREADS / 64];
  const int units = a.S * a.Ly * a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = min(PLAN_PER, (units + PLAN_THREADS - 1) / PLAN_THREADS);
  int carry = 0;
  for (int base = 0; base < units; base += PLAN_THREADS * per) {
    const int u0 = base + tid * per;
    int sl[PLAN_PER], np[PLAN_PER];
    int64_t off[PLAN_PER];
    int local = 0;
#pragma unroll
    for (int k = 0; k < PLAN_PER; ++k) {
      const int u = u0 + k;
      const bool ok = k < per && u < units;
      sl[k] = ok ? a.seg_len[u] : 0;
      off[k] = ok ? a.seg_off[u] : 0;
      np[k] = (sl[k] + a.chunk - 1) / a.chunk;
      local += np[k];
    }
    int inc = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int run = carry + inc - local, total = 0;
#pragma unroll
    for (int w = 0; w < PLAN_THREADS / 64; ++w) {
      if (w < wave) run += wsum[w];
      total += wsum[w];
    }
#pragma unroll
    for (int k = 0; k < PLAN_PER; ++k) {
      const int u = u0 + k;
      if (k < per && u < units) {
        a.upieces[u] = make_int2(run, np[k]);
        if (np[k] > 0) {
          const int q = sl[k] / np[k], r = sl[k] % np[k];
          int64_t e = off[k];
          for (int j = 0; j < np[k] && run + j < a.maxs; ++j) {
            PieceRec rec;
            rec.off = e;
            rec.u = u;
            rec.n = q + (j < r);
            rec.pad0 = rec.pad1 = rec.pad2 = rec.pad3 = 0;
            a.piece[run + j] = rec;
            e += rec.n;
          }
        }
        run += np[k];
      }
    }
    carry += total;
    __syncthreads();  // wsum is rewritten by the next round
  }
  if (tid == 0) *a.n_pieces = carry < a.maxs ? carry : a.maxs;
}

// 16 bytes of a value row, read once per step: a nontemporal load. A wave's
// value loads cover whole rows (16 lanes per 256-byte row), and streaming them
// past the caches leaves the key lines in L2 for the eight loads that each
// assemble (a key row is split across lanes in MFMA fragment order, so one
// key line is touched by eight load instructions). Measured on the full-depth
// workload: 116 -> 100 us per call over the 25% cache, 390 -> 360-380 us over
// the full cache; nontemporal key loads instead are 1.5x slower.
typedef unsigned int dec_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint16_t* p) {
  const dec_u32x4 v = __builtin_nontemporal_load((const dec_u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// A piece: its rows and ln mu (nullptr for the tail) and its unit.
template <class T>
struct Piece {
  const T* Kb;
  const T* Vb;
  const float* lm;
  int n;  // entries (>= 1)
  int u;
};

// Workgroups [0, maxs) take the plan's segment pieces (those past the plan's
// count return); workgroups from maxs on take tail piece (b - maxs) % ntp of
// unit (b - maxs) / ntp, the step's t_valid tail tokens split evenly.
template <class T, int D>
__device__ __forceinline__ bool load_piece(const DecArgs& a, Piece<T>& pc) {
  const int b = blockIdx.x;
  if (b < a.maxs) {
    const int np = *a.n_pieces;
    const PieceRec r = a.piece[b];
    if (b >= np) return false;
    pc.Kb = (const T*)a.K + r.off * D;
    pc.Vb = (const T*)a.V + r.off * D;
    pc.lm = a.lnmu ? a.lnmu + r.off : nullptr;
    pc.n = r.n;
    pc.u = r.u;
    return true;
  }
  const int qa = b - a.maxs;
  const int u = qa / a.ntp, j = qa % a.ntp;
  const int s = u / (a.Ly * a.H), lh = u % (a.Ly * a.H);
  const int l = lh / a.H, h = lh % a.H;
  const int q = a.t_valid / a.ntp, r = a.t_valid % a.ntp;
  const int64_t e = (((int64_t)l * a.H + h) * a.S + s) * a.t_cap + (int64_t)j * q + min(j, r);
  pc.Kb = (const T*)a.Kt + e * D;
  pc.Vb = (const T*)a.Vt + e * D;
  pc.lm = nullptr;
  pc.n = q + (j < r);
  pc.u = u;
  return true;
}

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

// fp32 caches: a piece of up to CHUNK entries on the VALU (logits by lane
// groups of D/8 lanes, one pass of max and exponentials per head in LDS).
template <class T, int D, int G>
__global__ __launch_bounds__(THREADS) void decode_partial_kernel(DecArgs a) {
  constexpr int LPE = D / 8;       // lanes per entry
  constexpr int EPI = 64 / LPE;    // entries per wave iteration
  constexpr int STEP = 4 * EPI;    // entries per workgroup iteration
  constexpr int ITER = CHUNK / STEP;
  __shared__ float z_s[G][CHUNK];
  __shared__ float m_s[G], l_s[G];
  __shared__ float o_s[4][G][D];
  Piece<T> pc;
  if (!load_piece<T, D>(a, pc)) return;
  const T* Kb = pc.Kb;
  const T* Vb = pc.Vb;
  const float* lm = pc.lm;
  const int n = pc.n;
  const int s = pc.u / (a.Ly * a.H), lh = pc.u % (a.Ly * a.H);
  const int l = lh / a.H, h = lh % a.H;
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
  const int64_t p = blockIdx.x;
  float* po = a.part_o + p * G * D;
  for (int i = threadIdx.x; i < G * D; i += THREADS) {
    const int g = i / D, dd = i % D;
    po[i] = o_s[0][g][dd] + o_s[1][g][dd] + o_s[2][g][dd] + o_s[3][g][dd];
  }
  if (threadIdx.x < G) a.part_ml[p * G + threadIdx.x] = make_float2(m_s[threadIdx.x], l_s[threadIdx.x]);
}

// bf16 caches: the logits of a 32-entry group come from one MFMA chain
// (A = the G query heads padded to 32 rows, B = the entries' keys), each wave
// runs an online softmax over rounds of 64 entries, and the values are
// accumulated on the VALU with the probabilities broadcast through LDS.
template <int D, int G>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(G == 8 ? 2 : 3))) void decode_mfma_kernel(DecArgs a) {
  using namespace kvcmf;
  constexpr int KS = D / 16;          // MFMA steps per group (16 dims each)
  constexpr int LPE = D / 8;          // lanes per entry in the value pass
  constexpr int EPI = 64 / LPE;       // entries per value iteration
  constexpr int VIT = 32 / EPI;       // value iterations per 32-entry round
  constexpr int GP = G < 4 ? G : 4;   // heads held per logit lane
  constexpr int PS = G <= 4 ? 4 : 8;  // row stride of the probability table
  __shared__ __align__(16) uint16_t qs[G][D];
  __shared__ __align__(16) float pw[4][32][PS];
  __shared__ float mw[4][G], lw[4][G];
  __shared__ __align__(16) float ow[4][G][D];
  Piece<uint16_t> pc;
  if (!load_piece<uint16_t, D>(a, pc)) return;
  const uint16_t* Kb = pc.Kb;
  const uint16_t* Vb = pc.Vb;
  const float* lm = pc.lm;
  const int n = pc.n;
  const int s = pc.u / (a.Ly * a.H), lh = pc.u % (a.Ly * a.H);
  const int l = lh / a.H, h = lh % a.H;
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
  // each wave takes a run of whole 32-entry rounds
  const int WE = (((n + 3) >> 2) + 31) & ~31;
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
      vr[it] = ld_stream(Vb + (int64_t)e * D + sub * 8);
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
      const float mx = group_max<32>(z);
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
        const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), hh * 32));
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
    lsum[j] = group_sum<32>(lsum[j]);
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
      if constexpr (LPE == 16) {
        x = cross_row_sum(x);
      } else {
#pragma unroll
        for (int o = LPE; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
      }
      if (es == 0) ow[wave][g][sub * 8 + j] = x;
    }
  __syncthreads();
  const int64_t p = blockIdx.x;
  float* po = a.part_o + p * G * D;
  for (int i = threadIdx.x; i < G * D; i += THREADS) {
    const int g = i / D, dd = i % D;
    float mx = mw[0][g];
#pragma unroll
    for (int w = 1; w < 4; ++w) mx = fmaxf(mx, mw[w][g]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (mw[w][g] != -INFINITY) o += ow[w][g][dd] * exp2f(mw[w][g] - mx);
    po[i] = o;
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
    a.part_ml[p * G + g] = make_float2(mx, t);
  }
}

// One workgroup of mrg_waves<G>() waves per unit: the unit's pieces (its segment
// pieces, then its tail pieces) are dealt to the waves, each wave loads its
// MRG_NPW pieces of a batch together and merges them online (lane = OPL
// consecutive outputs of one head), the waves are combined through LDS and o
// is normalized and stored. The layer sum reads it in the next launch.
template <int D, int G, int MRG_WAVES>
__global__ __launch_bounds__(MRG_WAVES * 64) void decode_merge_kernel(DecArgs a) {
  constexpr int GD = G * D;
  constexpr int OPL = GD / 64;  // merged outputs per lane, all of one head
  constexpr int NT = MRG_WAVES * 64;
  __shared__ float accs[MRG_WAVES][GD];
  __shared__ float msw[MRG_WAVES][G], lsw[MRG_WAVES][G];
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int2 up = a.upieces[u];
  const int p0 = up.x, nps = max(0, min(up.y, a.maxs - up.x));
  const int npt = nps + a.ntp;
  const int64_t t0 = (int64_t)a.maxs + (int64_t)u * a.ntp - nps;  // piece id of list index j >= nps
  const int g = lane * OPL / D;
  float M = -INFINITY, L = 0.f, acc[OPL];
#pragma unroll
  for (int q = 0; q < OPL; ++q) acc[q] = 0.f;
  for (int j0 = 0; j0 < npt; j0 += MRG_WAVES * MRG_NPW) {
    float2 ml[MRG_NPW];
    float v[MRG_NPW][OPL];
#pragma unroll
    for (int k = 0; k < MRG_NPW; ++k) {
      const int j = min(j0 + wave + MRG_WAVES * k, npt - 1);
      const int64_t p = j < nps ? (int64_t)p0 + j : t0 + j;
      ml[k] = a.part_ml[p * G + g];
      const float* po = a.part_o + p * GD + lane * OPL;
      if constexpr (OPL >= 4) {
#pragma unroll
        for (int q = 0; q < OPL; q += 4) {
          const float4 t = *(const float4*)(po + q);
          v[k][q] = t.x; v[k][q + 1] = t.y; v[k][q + 2] = t.z; v[k][q + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < OPL; ++q) v[k][q] = po[q];
      }
    }
#pragma unroll
    for (int k = 0; k < MRG_NPW; ++k) {
      if (j0 + wave + MRG_WAVES * k >= npt || ml[k].x == -INFINITY) continue;
      const float nm = fmaxf(M, ml[k].x);
      const float f0 = M == -INFINITY ? 0.f : exp2f(M - nm), f1 = exp2f(ml[k].x - nm);
      L = L * f0 + ml[k].y * f1;
#pragma unroll
      for (int q = 0; q < OPL; ++q) acc[q] = acc[q] * f0 + v[k][q] * f1;
      M = nm;
    }
  }
#pragma unroll
  for (int q = 0; q < OPL; ++q) accs[wave][lane * OPL + q] = acc[q];
  if ((lane * OPL) % D == 0) {
    msw[wave][g] = M;
    lsw[wave][g] = L;
  }
  __syncthreads();
  for (int i = tid; i < GD; i += NT) {
    const int gg = i / D;
    float mx = msw[0][gg];
#pragma unroll
    for (int w = 1; w < MRG_WAVES; ++w) mx = fmaxf(mx, msw[w][gg]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < MRG_WAVES; ++w)
      if (msw[w][gg] != -INFINITY) {
        const float f = exp2f(msw[w][gg] - mx);
        num += accs[w][i] * f;
        den += lsw[w][gg] * f;
      }
    a.o[(int64_t)u * GD + i] = den > 0.f ? num / den : 0.f;
  }
}

// x[s][h*G*D + i] = sum over l, in layer order, of o[s][l][h][i]: one thread
// an output, LS_THREADS outputs a workgroup, the layers' loads unrolled so
// they are all in flight together.
constexpr int LS_THREADS = 128;
__global__ __launch_bounds__(LS_THREADS) void decode_layersum_kernel(DecArgs a, int gd) {
  const int64_t i = (int64_t)blockIdx.x * LS_THREADS + threadIdx.x;
  const int64_t per_s = (int64_t)a.H * gd;
  if (i >= (int64_t)a.S * per_s) return;
  const int s = (int)(i / per_s);
  const int64_t r = i % per_s;
  const float* os = a.o + (int64_t)s * a.Ly * per_s + r;
  float xs = 0.f;
#pragma unroll 32
  for (int l = 0; l < a.Ly; ++l) xs += os[l * per_s];
  a.x[(int64_t)s * a.x_stride + r] = xs;
}

int64_t units_of(const kvc_ragged* c) { return (int64_t)c->n_seq * c->n_layers * c->n_kv_heads; }
int chunk_of(const kvc_ragged* c) { return c->dtype == KVC_BF16 ? MCHUNK : CHUNK; }
// Segment pieces, at most: ceil(len / chunk) < len / chunk + 1 per unit, and
// the segments hold at most `capacity` entries.
int64_t max_seg_pieces(const kvc_ragged* c) { return c->capacity / chunk_of(c) + units_of(c); }
int tail_pieces(const kvc_ragged* c, int32_t t) { return (t + chunk_of(c) - 1) / chunk_of(c); }

struct DecWs {
  int32_t* n_pieces;
  PieceRec* piece;
  int2* upieces;
  float* part_o;
  float2* part_ml;
  float* obuf;
};

// The plan comes first, so that a workspace sized for a larger t_cap keeps
// the plan where a smaller one puts it.
DecWs carve_dec(kvc::Carver& cv, const kvc_ragged* c, int32_t group, int32_t t_cap) {
  const int64_t units = units_of(c), maxs = max_seg_pieces(c);
  const int64_t np = maxs + units * tail_pieces(c, t_cap);
  const int64_t gd = (int64_t)group * c->head_dim;
  DecWs w;
  w.n_pieces = cv.take<int32_t>(1);
  w.piece = cv.take<PieceRec>((size_t)(maxs > 0 ? maxs : 1));
  w.upieces = cv.take<int2>((size_t)units);
  w.part_o = cv.take<float>((size_t)(np * gd));
  w.part_ml = cv.take<float2>((size_t)(np * group));
  w.obuf = cv.take<float>((size_t)(units * gd));
  return w;
}

int check_cache(const kvc_ragged* c, int32_t group, int32_t t_cap, void* ws, size_t ws_bytes) {
  KVC_REQUIRE(c != nullptr, KVC_E_INVAL, "cache is NULL");
  KVC_REQUIRE(c->seg_off && c->seg_len, KVC_E_INVAL, "kvc_decode: NULL segment arrays");
  KVC_REQUIRE(c->capacity >= 0 && (c->capacity == 0 || (c->K && c->V)), KVC_E_INVAL,
              "kvc_decode: NULL cache K/V with a nonzero capacity");
  KVC_REQUIRE(c->head_dim == 64 || c->head_dim == 128, KVC_E_SHAPE, "head_dim must be 64 or 128");
  KVC_REQUIRE(c->dtype == KVC_BF16 || c->dtype == KVC_F32, KVC_E_DTYPE, "cache dtype must be bf16 or f32");
  KVC_REQUIRE(group >= 1 && group <= 8, KVC_E_SHAPE, "group must be in [1, 8]");
  KVC_REQUIRE(group == 1 || group == 2 || group == 4 || group == 8, KVC_E_UNSUPPORTED,
              "kvc_decode: group must be 1, 2, 4 or 8");
  KVC_REQUIRE(c->n_seq >= 1 && c->n_layers >= 1 && c->n_kv_heads >= 1, KVC_E_SHAPE, "empty cache shape");
  KVC_REQUIRE(c->max_seg >= 0, KVC_E_INVAL, "max_seg must be >= 0");
  KVC_REQUIRE(t_cap >= 0, KVC_E_INVAL, "t_cap must be >= 0");
  KVC_REQUIRE(units_of(c) <= INT32_MAX / 2 && max_seg_pieces(c) + units_of(c) * tail_pieces(c, t_cap) <= INT32_MAX,
              KVC_E_SHAPE, "kvc_decode: cache too large");
  KVC_REQUIRE(ws && ws_bytes >= kvc_decode_workspace(c, group, t_cap), KVC_E_WORKSPACE,
              "kvc_decode: workspace too small");
  return KVC_OK;
}

DecArgs make_args(const kvc_ragged* c, int32_t group, int32_t t_valid, int32_t t_cap, const DecWs& w) {
  DecArgs a{};
  a.K = c->K;
  a.V = c->V;
  a.lnmu = c->lnmu;
  a.seg_off = c->seg_off;
  a.seg_len = c->seg_len;
  a.S = c->n_seq;
  a.Ly = c->n_layers;
  a.H = c->n_kv_heads;
  a.G = group;
  a.D = c->head_dim;
  a.t_valid = t_valid;
  a.t_cap = t_cap;
  a.chunk = chunk_of(c);
  a.maxs = (int)max_seg_pieces(c);
  a.ntp = tail_pieces(c, t_valid);
  a.scale2 = 1.4426950408889634f / sqrtf((float)c->head_dim);
  a.n_pieces = w.n_pieces;
  a.piece = w.piece;
  a.upieces = w.upieces;
  a.part_o = w.part_o;
  a.part_ml = w.part_ml;
  return a;
}

}  // namespace

extern "C" size_t kvc_decode_workspace(const kvc_ragged* c, int32_t group, int32_t t_cap) {
  if (!c || group < 1 || t_cap < 0 || c->capacity < 0 || c->head_dim < 1 || c->n_seq < 1 || c->n_layers < 1 ||
      c->n_kv_heads < 1)
    return 0;
  kvc::Carver cv(nullptr, 0);
  carve_dec(cv, c, group, t_cap);
  return cv.off + 256;
}

extern "C" int kvc_decode_plan(const kvc_ragged* c, int32_t group, int32_t t_cap, void* ws, size_t ws_bytes,
                               hipStream_t st) {
  const int rc = check_cache(c, group, t_cap, ws, ws_bytes);
  if (rc != KVC_OK) return rc;
  kvc::Carver cv(ws, ws_bytes);
  const DecWs w = carve_dec(cv, c, group, t_cap);
  const DecArgs a = make_args(c, group, 0, t_cap, w);
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, st, a);
  KVC_LAUNCH_CHECK("decode_plan");
  return KVC_OK;
}

namespace {
int check_step(const kvc_ragged* c, const void* K_tail, const void* V_tail, int32_t t_valid, int32_t t_cap,
               const void* Q, int32_t group, float* x_out, int64_t x_stride, void* ws, size_t ws_bytes) {
  const int rc = check_cache(c, group, t_cap, ws, ws_bytes);
  if (rc != KVC_OK) return rc;
  KVC_REQUIRE(Q && x_out, KVC_E_INVAL, "kvc_decode_attn: NULL pointer");
  KVC_REQUIRE(t_valid >= 0 && t_valid <= t_cap, KVC_E_INVAL, "need 0 <= t_valid <= t_cap");
  KVC_REQUIRE(t_valid == 0 || (K_tail && V_tail), KVC_E_INVAL, "tail pointers are NULL");
  KVC_REQUIRE(x_stride >= (int64_t)c->n_kv_heads * group * c->head_dim, KVC_E_INVAL, "x_stride too small");
  return KVC_OK;
}
}  // namespace

extern "C" int kvc_decode_attn_planned(const kvc_ragged* c, const void* K_tail, const void* V_tail,
                                       int32_t t_valid, int32_t t_cap, const void* Q, int32_t group, float* x_out,
                                       int64_t x_stride, float* o_out, void* ws, size_t ws_bytes, hipStream_t st) {
  const int rc = check_step(c, K_tail, V_tail, t_valid, t_cap, Q, group, x_out, x_stride, ws, ws_bytes);
  if (rc != KVC_OK) return rc;
  kvc::Carver cv(ws, ws_bytes);
  const DecWs w = carve_dec(cv, c, group, t_cap);
  DecArgs a = make_args(c, group, t_valid, t_cap, w);
  a.Kt = K_tail;
  a.Vt = V_tail;
  a.Q = Q;
  a.o = o_out ? o_out : w.obuf;
  a.x = x_out;
  a.x_stride = x_stride;
  const dim3 grid((unsigned)(a.maxs + units_of(c) * a.ntp));  // maxs >= units >= 1
  const int d = c->head_dim;
#define KVC_DEC(TT, DD, GG) hipLaunchKernelGGL((decode_partial_kernel<TT, DD, GG>), grid, dim3(THREADS), 0, st, a)
#define KVC_DECM(DD, GG) hipLaunchKernelGGL((decode_mfma_kernel<DD, GG>), grid, dim3(THREADS), 0, st, a)
#define KVC_MRG(DD, GG)                                                                                       \
  if (units_of(c) >= MRG_NARROW_UNITS)                                                                       \
    hipLaunchKernelGGL((decode_merge_kernel<DD, GG, MRG_NARROW>), mgrid, dim3(MRG_NARROW * 64), 0, st, a);   \
  else                                                                                                        \
    hipLaunchKernelGGL((decode_merge_kernel<DD, GG, mrg_waves<GG>()>), mgrid, dim3(mrg_waves<GG>() * 64), 0, st, a)
#define KVC_DEC_G(MAC, ...)                    \
  switch (group) {                             \
    case 1: MAC(__VA_ARGS__, 1); break;        \
    case 2: MAC(__VA_ARGS__, 2); break;        \
    case 4: MAC(__VA_ARGS__, 4); break;        \
    default: MAC(__VA_ARGS__, 8); break;       \
  }
  if (c->dtype == KVC_BF16) {
    if (d == 128) { KVC_DEC_G(KVC_DECM, 128); } else { KVC_DEC_G(KVC_DECM, 64); }
  } else {
    if (d == 128) { KVC_DEC_G(KVC_DEC, float, 128); } else { KVC_DEC_G(KVC_DEC, float, 64); }
  }
  KVC_LAUNCH_CHECK("decode_pieces");
  const dim3 mgrid((unsigned)units_of(c));
  if (d == 128) { KVC_DEC_G(KVC_MRG, 128); } else { KVC_DEC_G(KVC_MRG, 64); }
  KVC_LAUNCH_CHECK("decode_merge");
  const int gd = group * d;
  const int64_t nx = (int64_t)c->n_seq * c->n_kv_heads * gd;
  hipLaunchKernelGGL(decode_layersum_kernel, dim3(kvc_blocks(nx, LS_THREADS)), dim3(LS_THREADS), 0, st, a, gd);
  KVC_LAUNCH_CHECK("decode_layersum");
#undef KVC_DEC_G
#undef KVC_MRG
#undef KVC_DECM
#undef KVC_DEC
  return KVC_OK;
}

extern "C" int kvc_decode_attn(const kvc_ragged* c, const void* K_tail, const void* V_tail, int32_t t_valid,
                               int32_t t_cap, const void* Q, int32_t group, float* x_out, int64_t x_stride,
                               float* o_out, void* ws, size_t ws_bytes, hipStream_t st) {
  // every argument is checked before the first launch
  int rc = check_step(c, K_tail, V_tail, t_valid, t_cap, Q, group, x_out, x_stride, ws, ws_bytes);
  if (rc != KVC_OK) return rc;
  rc = kvc_decode_plan(c, group, t_cap, ws, ws_bytes, st);
  if (rc != KVC_OK) return rc;
  return kvc_decode_attn_planned(c, K_tail, V_tail, t_valid, t_cap, Q, group, x_out, x_stride, o_out, ws, ws_bytes,
                                 st);
}

// ------------------------------------------------------------------ no-allocation entry point
// For callers that cannot allocate device memory: the workspace of one decode
// step lives in a file-scope device array, one copy per GPU in the library's
// code object, held until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// the device address comes from hipGetSymbolAddress, taken once per device on
// the first call with that device current, and is used for every launch.
namespace {
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)64 << 20;
constexpr int MAX_DEVICES = 64;
static __device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  KVC_REQUIRE(e == hipSuccess, KVC_E_HIP, std::string("kvc_decode_attn_static: hipGetDevice: ") + hipGetErrorString(e));
  KVC_REQUIRE(dev >= 0 && dev < MAX_DEVICES, KVC_E_UNSUPPORTED, "kvc_decode_attn_static: device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    KVC_REQUIRE(e == hipSuccess && p != nullptr, KVC_E_HIP,
                std::string("kvc_decode_attn_static: hipGetSymbolAddress: ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVC_OK;
}
}  // namespace

extern "C" size_t kvc_decode_static_limit(void) { return STATIC_SCRATCH_BYTES; }

extern "C" int kvc_decode_attn_static(const kvc_ragged* c, const void* K_tail, const void* V_tail, int32_t t_valid,
                                      int32_t t_cap, const void* Q, int32_t group, float* x_out, int64_t x_stride,
                                      float* o_out, hipStream_t st) {
  KVC_REQUIRE(c != nullptr, KVC_E_INVAL, "cache is NULL");
  const size_t need = kvc_decode_workspace(c, group, t_cap);
  KVC_REQUIRE(need > 0, KVC_E_INVAL, "kvc_decode_attn_static: bad cache description, group or t_cap");
  if (need > STATIC_SCRATCH_BYTES)
    return kvc::set_error(KVC_E_WORKSPACE, "kvc_decode_attn_static: this cache and t_cap need " + std::to_string(need) +
                                          " bytes of scratch, above the " + std::to_string(STATIC_SCRATCH_BYTES) +
                                          " the library holds per GPU; call kvc_decode_attn with a workspace");
  void* ws = nullptr;
  const int rc = scratch_of_current_device(&ws);
  if (rc != KVC_OK) return rc;
  return kvc_decode_attn(c, K_tail, V_tail, t_valid, t_cap, Q, group, x_out, x_stride, o_out, ws,
                         STATIC_SCRATCH_BYTES, st);
}
