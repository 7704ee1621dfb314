// Prototype trees of midpoint-split slots of at most 64 tokens (bf16 keys and
// values, head dimension 128), per (sequence, layer, KV head, slot).
//
// GraceKV page: '02 Progressively refinable representation' (one tree per
// (layer, KV head, slot)); 'Inside one cache entry' (key: inverse-rotate,
// average, re-rotate at a representative position; value: relevance weighted
// with a 10% uniform base; multiplicity from key coherence); '03 Bottom-up
// value flow' (a parent's value is the sum of its children's); 'Technical
// details and default settings' (probe-based distortion, attention-partition
// : value-aggregate error = 0.25 : 0.75); '04 Top-down budget flow' (utility
// per entry = relevance x fidelity gain x head sensitivity / new entries).
//
// Fixed layout. The midpoint tree of n <= 64 tokens (left child: the first
// ceil(size/2) tokens) is laid on the complete binary tree over 64
// positions: the root covers positions [0, 64), a node on [p, p + 2h) gives
// [p, p + h) to its left child and [p + h, p + 2h) to its right child, and a
// leaf token sits at the first position of the block it reaches. A node of
// depth l holds at most ceil(n / 2^l) <= 64 / 2^l tokens, so it fits its
// block; positions without a token hold zeros. Blocks are numbered as a heap
// (root 1, children 2b and 2b + 1; 64 + v is position v). Every node is then
// an aligned block: its sums are fixed trees of additions and its quadratic
// forms are block-diagonal matrix products.
//
// Value-aggregate error of a node (probe row rho, weights a_i, value weights
// w_i = alpha r_i + gamma summing to 1, Z = sum a_i, values centred on the
// slot mean m, G' their Gram matrix, s_i = <v_i - m, m>): with c = a - Z w,
//   ||u - Z v^||^2 = c^T G' c = sum_i c_i (T_i - Z g_i),  T = G'_node a,
//   g = G'_node w,
//   ||u||^2 = a^T G' a + 2 Z a.s + Z^2 |m|^2 = sum_i a_i T_i + ...
// T for every node of one depth is one block-diagonal product G'_depth a on
// MFMA (both operands as hi/lo bf16 pieces); g is the same for every row.
//
// Per slot, eight waves:
//  S0 token of each position, node of each block, relevance by blocks;
//  S1 waves 0-3: softmax weights a[v][rho] = exp(<q_rho, k_v>/sqrt d -
//     lse_rho) on MFMA, value column sums; waves 4-7 (lane = rotation pair,
//     16 positions each): inverse-rotated keys, key norms, key sums of the
//     blocks of up to 16 positions, their multiplicities and prototype keys;
//  S2 waves 0-2: the centred value Gram matrix on MFMA, a 32 x 32 tile each
//     (partial row sums, a barrier, then each stores its tile); waves 4-6: the
//     blocks of 32 and 64 positions;
//  S3 waves 0-3: prototype logits on MFMA; waves 4-7: w and g per depth;
//  S4 waves 0-5 (probe-row half x two depths): T on MFMA, then per node and
//     row the two value forms and the attention-partition terms, summed over
//     the rows by a reduce-scatter across lanes;
//  S5 D per node, node arrays in pre-order, op utilities.
#include "kvc_internal.h"
#include "mfma_frag.h"
#include "trees_common.h"

namespace {

using namespace kvc_tree;
using namespace kvcmf;

constexpr int NV = 64;        // positions of the fixed layout
constexpr int DH = 128;       // head dimension
constexpr int HD = DH / 2;    // rotation pairs
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int GS = 72;        // row stride (bf16 elements) of the Gram pieces
constexpr int KR = 136;       // row stride (bf16 elements) of the prototype-key pieces
constexpr float L2E = 1.4426950408889634f;

// LDS layout (bytes). Regions sharing an offset are live in disjoint stages.
struct VL {
  static constexpr size_t at = 0;                           // float [NV][64] softmax weights a[v][rho]
  static constexpr size_t gh = at + NV * 64 * 4;            // bf16 [NV][GS] G' hi piece
  static constexpr size_t gl = gh + NV * GS * 2;            // bf16 [NV][GS] G' lo piece
  static constexpr size_t kh = gl + NV * GS * 2;            // bf16 [64][KR] prototype keys, hi (S1-S3)
  static constexpr size_t kl = kh + 64 * KR * 2;            // bf16 [64][KR] prototype keys, lo (S1-S3)
  static constexpr size_t zh = kh;                          // float [64][64] Zhat[b][rho] (S3-S4)
  static constexpr size_t gw = kl + 64 * KR * 2;            // float2 [6][NV] (g, w) per depth (S3-S4)
  static constexpr size_t ks16 = gw + 6 * NV * 8;           // float2 [4][HD] key sums of the 16-blocks (S1-S2)
  static constexpr size_t red = ks16;                       // float [2][64][4] row sums per block (S4-S5)
  static constexpr size_t wl = ks16 + 4 * HD * 8;           // float [6][NV] value weights per depth (S3); row means of G (S2)
  static constexpr size_t lse = wl + 6 * NV * 4;            // float [64]
  static constexpr size_t rv = lse + 64 * 4;                // float [NV] relevance at each position
  static constexpr size_t sdv = rv + NV * 4;                // float [NV] <v - m, m>
  static constexpr size_t knv = sdv + NV * 4;               // float [NV] key norms
  static constexpr size_t bn2 = knv + NV * 4;               // float [64] squared norm of the block key sums
  static constexpr size_t bmu = bn2 + 64 * 4;               // float [64] block multiplicity
  static constexpr size_t relb = bmu + 64 * 4;              // float [128] block relevance
  static constexpr size_t bD = relb + 128 * 4;              // float [128] block distortion
  static constexpr size_t bsz = bD + 128 * 4;               // short [128] tokens in the block
  static constexpr size_t bst = bsz + 128 * 2;              // short [128] first token of the block (slot-relative)
  static constexpr size_t jb = bst + 128 * 2;               // short [128] block of pre-order node j
  static constexpr size_t tok = jb + 128 * 2;               // int [NV] token at each position (-1: none)
  static constexpr size_t misc = tok + NV * 4;              // float [4]: |m|^2
  static constexpr size_t total = misc + 16;
};
static_assert(4 * HD * 8 >= 2 * 64 * 4 * 4, "row sums fit over the key sums");
static_assert(64 * 64 * 4 <= 2 * 64 * KR * 2, "Zhat fits over the prototype keys");

// x = hi + lo in bf16 pieces, each the round-to-nearest-even of the
// remainder so far: |x - hi - lo| <= 2^-18 |x|
__device__ __forceinline__ void split8v(const float* x, kvc_bf16x8& hi, kvc_bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint16_t b = f32_to_bf16_hw(x[j]);
    hi[j] = __builtin_bit_cast(__bf16, b);
    lo[j] = __builtin_bit_cast(__bf16, f32_to_bf16_hw(x[j] - bf16_bits_to_f32(b)));
  }
}

// partner's value for the DPP exchanges inside a 16-lane row: E = 8 (lane i
// and 15 - i), 4 (i and 7 - i in each 8-lane group), 2 (i ^ 2), 1 (i ^ 1)
template <int E>
__device__ __forceinline__ float xpart(float v) {
  if constexpr (E == 8) return dpp_f32<0x140>(v);
  else if constexpr (E == 4) return dpp_f32<0x141>(v);
  else if constexpr (E == 2) return dpp_f32<0x4E>(v);
  else return dpp_f32<0xB1>(v);
}

// Reduce-scatter of N values per lane over the lanes differing in the bits
// E, E/2, ..., 1 (E = 32: the whole wave; E = 16: each 32-lane half). Each
// exchange pairs lanes that differ in that bit (16 and 32 by permlane swaps;
// below, DPP mirrors, whose pairs also differ in that bit); while more than
// one value is left, the lane with the bit clear keeps the lower half of the
// values and the other the upper half, both summed over the pair; then the
// single value is summed. Afterwards x[0 .. max(N >> steps, 1)) of a lane
// hold the totals of the indices base + j; base collects the upper halves kept.
template <int N, int E>
__device__ __forceinline__ void reduce_scatter(float* x, int lane, int& base) {
  if constexpr (E > 0) {
    if constexpr (N > 1) {
      constexpr int H = N / 2;
      if constexpr (E >= 16) {
#pragma unroll
        for (int k = 0; k < H; ++k) {
          const auto r = E == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x[k]), __float_as_uint(x[k + H]), false, false)
                                 : __builtin_amdgcn_permlane16_swap(__float_as_uint(x[k]), __float_as_uint(x[k + H]), false, false);
          x[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
      } else {
        const bool up = (lane & E) != 0;
#pragma unroll
        for (int k = 0; k < H; ++k) {
          const float keep = up ? x[k + H] : x[k], send = up ? x[k] : x[k + H];
          x[k] = keep + xpart<E>(send);
        }
      }
      if (lane & E) base += H;
      reduce_scatter<H, E / 2>(x, lane, base);
    } else {
      if constexpr (E >= 16) {
        const auto r = E == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x[0]), __float_as_uint(x[0]), false, false)
                               : __builtin_amdgcn_permlane16_swap(__float_as_uint(x[0]), __float_as_uint(x[0]), false, false);
        x[0] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      } else {
        x[0] += xpart<E>(x[0]);
      }
      reduce_scatter<1, E / 2>(x, lane, base);
    }
  }
}

struct SlotRefs {
  const float* At;
  const uint16_t* Gh;
  const uint16_t* Gl;
  const float* Zh;
  const float2* gw;
  const float* sdv;
  float* red;
  float mm;
  int rt, lane;
};

// One tile of 32 positions or, for the root, both: the value-error forms and
// the attention-partition terms of every node of depth LEV in it, summed over
// this wave's 32 probe rows, written to red[rt][block][0..3] = (sum
// sqrt(c^T G' c), sum ||u||, sum |Zhat - Z|, sum Z). Lane l holds the rows
// (positions) 8 g + 4 (l >> 5) + e of a tile, e < 4, and probe row l % 32.
template <int LEV>
__device__ __forceinline__ void depth_forms(const SlotRefs& R) {
  constexpr int S = NV >> LEV;                  // block size
  constexpr int NT = S == 64 ? 1 : 2;           // passes (the root spans both tiles)
  constexpr int NTL = S == 64 ? 2 : 1;          // tiles in a pass
  constexpr int NBL = S >= 32 ? 1 : (S == 16 ? 2 : (S >= 4 ? 4 : 8));  // blocks per lane and pass
  const int lane = R.lane, hb = lane >> 5, l32 = lane & 31;
  const int rho = R.rt * 32 + l32;
  auto bk = [](int g, int e) { return S >= 32 ? 0 : (S == 16 ? (g >> 1) : (S >= 4 ? g : (2 * g + (e >> 1)))); };
#pragma unroll 1
  for (int pass = 0; pass < NT; ++pass) {
    float Z[NBL], AS[NBL], num[NBL], den[NBL];
#pragma unroll
    for (int k = 0; k < NBL; ++k) Z[k] = AS[k] = num[k] = den[k] = 0.f;
    float av[16];
    // the block sums Z and a.s
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
      const int vt = S == 64 ? tt : pass;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int v0 = vt * 32 + 8 * g + 4 * hb;
        const float4 s4 = *(const float4*)(R.sdv + v0);
        const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = R.At[(v0 + e) * 64 + rho];
          av[4 * g + e] = x;
          Z[bk(g, e)] += x;
          AS[bk(g, e)] = fmaf(x, sv[e], AS[bk(g, e)]);
        }
      }
    }
    if constexpr (S >= 8) {
#pragma unroll
      for (int k = 0; k < NBL; ++k) {
        Z[k] = group_sum_x32(Z[k]);
        AS[k] = group_sum_x32(AS[k]);
      }
    }
    // T = G'_depth a on MFMA, then the forms
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
      const int vt = S == 64 ? tt : pass;
      const int v = vt * 32 + l32;           // A-operand row of this lane
      kvc_f32x16 acc = {};
      constexpr int KN = S == 64 ? 4 : 2;
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
        const int kap = S == 64 ? kk : 2 * vt + kk;   // 16-position step of the reduction
        const int c0 = kap * 16 + 8 * hb;
        uint4 gh = *(const uint4*)(R.Gh + v * GS + c0), gl = *(const uint4*)(R.Gl + v * GS + c0);
        float xa[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xa[e] = R.At[(c0 + e) * 64 + rho];
        if constexpr (S == 16) {
          if ((v >> 4) != kap) gh = gl = make_uint4(0, 0, 0, 0);
        } else if constexpr (S <= 8) {
          const bool same8 = (v >> 3) == 2 * kap + hb;
          if constexpr (S == 8) {
            if (!same8) gh = gl = make_uint4(0, 0, 0, 0);
          } else if constexpr (S == 4) {
            const int hsel = (v >> 2) & 1;
            const bool k0 = same8 && hsel == 0, k1 = same8 && hsel == 1;
            gh = make_uint4(k0 ? gh.x : 0u, k0 ? gh.y : 0u, k1 ? gh.z : 0u, k1 ? gh.w : 0u);
            gl = make_uint4(k0 ? gl.x : 0u, k0 ? gl.y : 0u, k1 ? gl.z : 0u, k1 ? gl.w : 0u);
          } else {
            const int q = (v >> 1) & 3;
            gh = make_uint4(same8 && q == 0 ? gh.x : 0u, same8 && q == 1 ? gh.y : 0u, same8 && q == 2 ? gh.z : 0u,
                            same8 && q == 3 ? gh.w : 0u);
            gl = make_uint4(same8 && q == 0 ? gl.x : 0u, same8 && q == 1 ? gl.y : 0u, same8 && q == 2 ? gl.z : 0u,
                            same8 && q == 3 ? gl.w : 0u);
          }
        }
        Frag<uint16_t> fh, fl, ah, al;
        fh.v = __builtin_bit_cast(kvc_bf16x8, gh);
        fl.v = __builtin_bit_cast(kvc_bf16x8, gl);
        split8v(xa, ah.v, al.v);
        mma(acc, fh, ah);
        mma(acc, fh, al);
        mma(acc, fl, ah);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int v0 = vt * 32 + 8 * g + 4 * hb;
        const float4 p0 = *(const float4*)(R.gw + LEV * NV + v0), p1 = *(const float4*)(R.gw + LEV * NV + v0 + 2);
        const float gg[4] = {p0.x, p0.z, p1.x, p1.z}, ww[4] = {p0.y, p0.w, p1.y, p1.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e, k = bk(g, e);
          const float x = NTL == 1 ? av[r] : R.At[(v0 + e) * 64 + rho], t = acc[r];
          const float c = fmaf(-Z[k], ww[e], x);
          const float tc = fmaf(-Z[k], gg[e], t);
          num[k] = fmaf(c, tc, num[k]);
          den[k] = fmaf(x, t, den[k]);
        }
      }
    }
    if constexpr (S >= 8) {
#pragma unroll
      for (int k = 0; k < NBL; ++k) {
        num[k] = group_sum_x32(num[k]);
        den[k] = group_sum_x32(den[k]);
      }
    }
    // heap index of block k of this lane and pass
    const int vt = pass;
    auto heap = [&](int k) {
      if constexpr (S == 64) return 1;
      else if constexpr (S == 32) return 2 + vt;
      else if constexpr (S == 16) return 4 + 2 * vt + k;
      else if constexpr (S == 8) return 8 + 4 * vt + k;
      else if constexpr (S == 4) return 16 + 8 * vt + 2 * k + hb;
      else return 32 + 16 * vt + 4 * (k >> 1) + 2 * hb + (k & 1);
    };
    // per block and row: the four terms, then their sums over the rows
    constexpr int NVAL = 4 * NBL;
    float xs[NVAL];
#pragma unroll
    for (int k = 0; k < NBL; ++k) {
      const float dn = fmaf(Z[k] * Z[k], R.mm, fmaf(2.f * Z[k], AS[k], den[k]));
      xs[4 * k + 0] = hw_sqrt(fmaxf(num[k], 0.f));
      xs[4 * k + 1] = hw_sqrt(fmaxf(dn, 0.f));
      xs[4 * k + 2] = fabsf(R.Zh[heap(k) * 64 + rho] - Z[k]);
      xs[4 * k + 3] = Z[k];
    }
    int base = 0;
    reduce_scatter<NVAL, 16>(xs, lane, base);
    constexpr int CNT = NVAL >= 32 ? NVAL / 32 : 1;
    if (S <= 4 || hb == 0) {
#pragma unroll
      for (int j = 0; j < CNT; ++j) {
        const int idx = base + j;
        R.red[(R.rt * 64 + heap(idx >> 2)) * 4 + (idx & 3)] = xs[j];
      }
    }
  }
}

// g = G'_block w for every position at depth LEV (lane = position), from the
// hi/lo pieces of G' and the value weights of that depth
template <int LEV>
__device__ __forceinline__ void depth_g(const uint16_t* Gh, const uint16_t* Gl, const float* wl, float2* gw, int v) {
  constexpr int S = NV >> LEV;
  const int v0 = v & ~(S - 1);
  const float* wd = wl + LEV * NV;
  float g = 0.f;
  if constexpr (S >= 8) {
#pragma unroll
    for (int i = 0; i < S; i += 8) {
      const uint4 h = *(const uint4*)(Gh + v * GS + v0 + i), l = *(const uint4*)(Gl + v * GS + v0 + i);
      const float4 w0 = *(const float4*)(wd + v0 + i), w1 = *(const float4*)(wd + v0 + i + 4);
      const uint32_t hh[4] = {h.x, h.y, h.z, h.w}, ll[4] = {l.x, l.y, l.z, l.w};
      const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ga = __uint_as_float(hh[e] << 16) + __uint_as_float(ll[e] << 16);
        const float gb = __uint_as_float(hh[e] & 0xffff0000u) + __uint_as_float(ll[e] & 0xffff0000u);
        g = fmaf(ga, ww[2 * e], g);
        g = fmaf(gb, ww[2 * e + 1], g);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < S; ++i) g = fmaf(bf16_bits_to_f32(Gh[v * GS + v0 + i]) + bf16_bits_to_f32(Gl[v * GS + v0 + i]), wd[v0 + i], g);
  }
  gw[LEV * NV + v] = make_float2(g, wd[v]);
}

__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(4))) void tree_v_kernel(TreeKArgs a) {
  extern __shared__ __align__(16) char smem[];
  float* At = (float*)(smem + VL::at);
  uint16_t* Gh = (uint16_t*)(smem + VL::gh);
  uint16_t* Gl = (uint16_t*)(smem + VL::gl);
  uint16_t* Kh = (uint16_t*)(smem + VL::kh);
  uint16_t* Kl = (uint16_t*)(smem + VL::kl);
  float* Zh = (float*)(smem + VL::zh);
  float2* gw = (float2*)(smem + VL::gw);
  float2* ks16 = (float2*)(smem + VL::ks16);
  float* red = (float*)(smem + VL::red);
  float* wl = (float*)(smem + VL::wl);
  float* lse_s = (float*)(smem + VL::lse);
  float* rv = (float*)(smem + VL::rv);
  float* sdv = (float*)(smem + VL::sdv);
  float* knv = (float*)(smem + VL::knv);
  float* bn2 = (float*)(smem + VL::bn2);
  float* bmu = (float*)(smem + VL::bmu);
  float* relb = (float*)(smem + VL::relb);
  float* bD = (float*)(smem + VL::bD);
  short* bsz = (short*)(smem + VL::bsz);
  short* bst = (short*)(smem + VL::bst);
  short* jb = (short*)(smem + VL::jb);
  int* tok = (int*)(smem + VL::tok);
  float* misc = (float*)(smem + VL::misc);

  __shared__ int pre[MAX_SEQ + 1];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pd = a.pd;
  if (tid == 0) {
    int acc = 0;
    pre[0] = 0;
    for (int s = 0; s < a.S; ++s) pre[s + 1] = (acc += a.count[s]);
  }
  __syncthreads();
  const int64_t nsl = pre[a.S];
  const int64_t nitems = (int64_t)a.Ly * a.H * nsl;
  // a contiguous range of items per workgroup: neighbouring slots of one unit
  // share their probe rows and sit next to each other in HBM
  const int64_t wb = (int64_t)blockIdx.x * nitems / gridDim.x, we = (int64_t)(blockIdx.x + 1) * nitems / gridDim.x;
  ItemDesc nxt{};
  if (wb < we) nxt = item_desc(a, pre, nsl, wb);
  // the next slot's token relevance (wave 0, lane = position) and probe-row
  // lse (wave 2), loaded while this slot's forms run
  float rel_pf = 0.f, lse_pf = 0.f;

  for (int64_t w = wb; w < we; ++w) {
    const ItemDesc cur = nxt;
    if (w + 1 < we) nxt = item_desc(a, pre, nsl, w + 1);  // in flight during this slot
    // the lane index as a value of this iteration: addresses derived from it
    // are formed where they are used instead of being held across the loop
    int lane;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lane) : "v"(tid & 63));
    const int hb = lane >> 5, l32 = lane & 31;
    const int64_t lh = cur.lh;
    const int s = cur.s, t0 = cur.t0, n = cur.n;
    const int l = (int)(lh / a.H), h = (int)(lh % a.H);
    const int64_t tok0 = a.cu[s] + t0;
    const int64_t obase = lh * 2 * a.T + 2 * tok0;
    const uint16_t* Kg = (const uint16_t*)a.K + (lh * a.T + tok0) * DH;
    const uint16_t* Vg = (const uint16_t*)a.V + (lh * a.T + tok0) * DH;
    const int unit = (s * a.Ly + l) * a.H + h;
    const uint16_t* Qu = (const uint16_t*)a.Qp + ((((int64_t)s * a.Ly + l) * a.H * a.G + (int64_t)h * a.G) * a.P) * DH;
    const float* lse_g = a.lse + (int64_t)unit * a.G * a.P;

    // ---- S0: tokens of the positions, nodes of the blocks, block relevance
    if (wave == 0) {
      int st = 0, sz = n;  // descend by the bits of position v = lane
#pragma unroll
      for (int lev = 0; lev < 6; ++lev) {
        const int bit = (lane >> (5 - lev)) & 1;
        if (sz >= 2) {
          const int nl = (sz + 1) >> 1;
          if (bit) {
            st += nl;
            sz -= nl;
          } else {
            sz = nl;
          }
        } else if (bit) {
          sz = 0;
        }
      }
      const int t = sz == 1 ? st : -1;
      tok[lane] = t;
      const float r = w > wb ? rel_pf : (t >= 0 ? a.rel[lh * a.T + tok0 + t] : 0.f);
      rv[lane] = r;
      relb[64 + lane] = r;
      // a parent is the fp32 sum of its two children (the same in both lanes of a pair)
      float x = r + dpp_f32<0xB1>(r);
      if ((lane & 1) == 0) relb[32 + (lane >> 1)] = x;
      x += dpp_f32<0x4E>(x);
      if ((lane & 3) == 0) relb[16 + (lane >> 2)] = x;
      x += dpp_f32<0x141>(x);
      if ((lane & 7) == 0) relb[8 + (lane >> 3)] = x;
      x += dpp_f32<0x140>(x);
      if ((lane & 15) == 0) relb[4 + (lane >> 4)] = x;
      {
        const auto rr = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(rr[0]) + __uint_as_float(rr[1]);
      }
      if ((lane & 31) == 0) relb[2 + (lane >> 5)] = x;
      x = group_sum_x32(x);
      if (lane == 0) relb[1] = x;
    } else if (wave == 1) {
      // blocks lane and 64 + lane: descend from the root along the bits of b;
      // a block is a node if it holds a token and is the root or its parent
      // block was split (deeper blocks under a leaf only carry that leaf)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int b = half * 64 + lane;
        if (b == 0) {
          bsz[0] = 0;
          bst[0] = 0;
          continue;
        }
        const int dep = 31 - __clz(b);
        int st = 0, sz = n, j = 0, psz = n;
        for (int k = dep - 1; k >= 0; --k) {
          const int bit = (b >> k) & 1;
          psz = sz;
          if (sz >= 2) {
            const int nl = (sz + 1) >> 1;
            if (bit) {
              st += nl;
              j += 2 * nl;
              sz -= nl;
            } else {
              j += 1;
              sz = nl;
            }
          } else if (bit) {
            sz = 0;
          }
        }
        bsz[b] = (short)sz;
        bst[b] = (short)st;
        if (sz >= 1 && (dep == 0 || psz >= 2)) jb[j] = (short)b;
      }
    } else if (wave == 2) {
      lse_s[lane] = w > wb ? lse_pf : (lane < pd ? lse_g[(int64_t)lane * a.pstride] : 0.f);
    }
    __syncthreads();

    // ---- S1
    if (wave < 4) {
      const int vt = wave >> 1, rt = wave & 1;
      const int rho = rt * 32 + l32;
      Frag<uint16_t> qf[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        qf[k] = rho < pd ? load_frag<uint16_t>(Qu + (int64_t)rho * a.pstride * DH + k * 16 + 8 * hb)
                         : zero_frag<uint16_t>();
      const int t = tok[vt * 32 + l32];
      Frag<uint16_t> kf[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        kf[k] = t >= 0 ? load_frag<uint16_t>(Kg + (int64_t)t * DH + k * 16 + 8 * hb) : zero_frag<uint16_t>();
      kvc_f32x16 acc = {};
#pragma unroll
      for (int k = 0; k < 8; ++k) mma(acc, kf[k], qf[k]);
      const float ls = lse_s[rho];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int v0 = vt * 32 + 8 * g + 4 * hb;
        const int4 t4 = *(const int4*)(tok + v0);
        const int tt[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          At[(v0 + e) * 64 + rho] = (rho < pd && tt[e] >= 0) ? fast_exp2((acc[4 * g + e] * a.c - ls) * L2E) : 0.f;
      }
    } else {
      // keys: lane = rotation pair (p, p + 64), positions [16 kw, 16 kw + 16)
      const int kw = wave - 4, p = lane, v0 = 16 * kw;
      float y0[16], y1[16], q[16];
      {
        float cc[16], ss[16];
        int tk[16];
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          const int4 t4 = *(const int4*)(tok + v0 + j);
          tk[j] = t4.x;
          tk[j + 1] = t4.y;
          tk[j + 2] = t4.z;
          tk[j + 3] = t4.w;
        }
        float x0[16], x1[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (tk[j] >= 0) {
            x0[j] = bf16_bits_to_f32(Kg[(int64_t)tk[j] * DH + p]);
            x1[j] = bf16_bits_to_f32(Kg[(int64_t)tk[j] * DH + HD + p]);
            const int64_t pr = (int64_t)(t0 + tk[j]) * HD + p;
            cc[j] = a.rc[pr];
            ss[j] = a.rs[pr];
          } else {
            x0[j] = x1[j] = cc[j] = ss[j] = 0.f;
          }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          y0[j] = x0[j] * cc[j] + x1[j] * ss[j];   // rotation by -theta
          y1[j] = x1[j] * cc[j] - x0[j] * ss[j];
          q[j] = x0[j] * x0[j] + x1[j] * x1[j];
        }
      }
      // key norms: the 16 positions' sums over the lanes, one per lane group
      {
        int base = 0;
        reduce_scatter<16, 32>(q, lane, base);
        if ((lane & 3) == 0) knv[v0 + base] = hw_sqrt(q[0]);
      }
      // key sums of the blocks of 2, 4, 8 and 16 positions (in heap order
      // within this range: 8 pairs, 4 quads, 2 octets, 1)
      float b0[15], b1[15];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        b0[k] = y0[2 * k] + y0[2 * k + 1];
        b1[k] = y1[2 * k] + y1[2 * k + 1];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        b0[8 + k] = b0[2 * k] + b0[2 * k + 1];
        b1[8 + k] = b1[2 * k] + b1[2 * k + 1];
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        b0[12 + k] = b0[8 + 2 * k] + b0[8 + 2 * k + 1];
        b1[12 + k] = b1[8 + 2 * k] + b1[8 + 2 * k + 1];
      }
      b0[14] = b0[12] + b0[13];
      b1[14] = b1[12] + b1[13];
      ks16[kw * HD + p] = make_float2(b0[14], b1[14]);
      // heap block of range-local block k
      auto blk = [&](int k) {
        return k < 8 ? 32 + 8 * kw + k : (k < 12 ? 16 + 4 * kw + (k - 8) : (k < 14 ? 8 + 2 * kw + (k - 12) : 4 + kw));
      };
      {
        float nq[16];
#pragma unroll
        for (int k = 0; k < 15; ++k) nq[k] = b0[k] * b0[k] + b1[k] * b1[k];
        nq[15] = 0.f;
        int base = 0;
        reduce_scatter<16, 32>(nq, lane, base);
        if ((lane & 3) == 0 && base < 15) bn2[blk(base)] = nq[0];
      }
      __builtin_amdgcn_wave_barrier();  // this wave's key norms and block norms are in LDS (wave order)
      float kb[15];
#pragma unroll
      for (int j = 0; j < 16; j += 4) {
        const float4 x = *(const float4*)(knv + v0 + j);
        kb[j >> 1] = x.x + x.y;
        kb[(j >> 1) + 1] = x.z + x.w;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) kb[8 + k] = kb[2 * k] + kb[2 * k + 1];
      kb[12] = kb[8] + kb[9];
      kb[13] = kb[10] + kb[11];
      kb[14] = kb[12] + kb[13];
      // multiplicity and prototype key of every node among these blocks (the
      // rotation at the representative positions loaded a batch at a time;
      // those rows were just read for the keys, so these are cache hits)
#pragma unroll
      for (int k0 = 0; k0 < 15; k0 += 8) {
        constexpr int NBAT = 8;
        float pc[NBAT], ps[NBAT];
#pragma unroll
        for (int u = 0; u < NBAT; ++u) {
          if (k0 + u >= 15) break;
          const int b = blk(k0 + u);
          const int sz = bsz[b];
          const int prep = bst[b] + (sz > 0 ? (sz - 1) / 2 : 0);
          const int64_t pr = (int64_t)(t0 + prep) * HD + p;
          pc[u] = a.rc[pr];
          ps[u] = a.rs[pr];
        }
#pragma unroll
        for (int u = 0; u < NBAT; ++u) {
          const int k = k0 + u;
          if (k >= 15) break;
          const int b = blk(k);
          const int szi = bsz[b];
          if (szi < 2) continue;
          const float sz = (float)szi;
          const float coh = kb[k] > 0.f ? hw_div(hw_sqrt(bn2[b]), kb[k]) : 1.f;
          if (lane == 0) bmu[b] = fmaxf(1.f, sz * coh);
          const float rsz = __builtin_amdgcn_rcpf(sz);
          const float m0 = b0[k] * rsz, m1 = b1[k] * rsz;
          const float k0v = m0 * pc[u] - m1 * ps[u], k1v = m1 * pc[u] + m0 * ps[u];
          const uint16_t h0 = f32_to_bf16_hw(k0v), h1 = f32_to_bf16_hw(k1v);
          Kh[b * KR + p] = h0;
          Kh[b * KR + HD + p] = h1;
          Kl[b * KR + p] = f32_to_bf16_hw(k0v - bf16_bits_to_f32(h0));
          Kl[b * KR + HD + p] = f32_to_bf16_hw(k1v - bf16_bits_to_f32(h1));
        }
      }
    }
    __syncthreads();

    // ---- S2
    // Waves 0-2: one tile each of the Gram matrix of the slot's values (the
    // bf16 values are exact MFMA inputs, so G = V V^T is exact up to the fp32
    // accumulation): tiles (0, 0), (0, 1) and (1, 1) of 32 x 32 positions, and
    // their partial row sums (tile (0, 1) also gives the row sums of (1, 0) as
    // its column sums): part0 = wl[0, 64) from the diagonal tiles, part1 =
    // wl[64, 128) from the off-diagonal one. After the barrier each wave
    // centres and stores its tile: G'_vi = G_vi - r_v - r_i + R with the row
    // means r_v = (part0_v + part1_v) / n = <v_v, m> and R = |m|^2 (m the
    // slot's value mean; positions without a token are 0).
    kvc_f32x16 gt = {};
    const int gti = wave == 2 ? 1 : 0, gtj = wave == 0 ? 0 : 1;
    if (wave < 3) {
      const int ra = tok[gti * 32 + l32], rb = tok[gtj * 32 + l32];
#pragma unroll 2
      for (int k = 0; k < 8; ++k) {
        const int c = k * 16 + 8 * hb;
        const Frag<uint16_t> fa = ra >= 0 ? load_frag<uint16_t>(Vg + (int64_t)ra * DH + c) : zero_frag<uint16_t>();
        if (wave == 1) {
          const Frag<uint16_t> fb = rb >= 0 ? load_frag<uint16_t>(Vg + (int64_t)rb * DH + c) : zero_frag<uint16_t>();
          mma(gt, fa, fb);
        } else {
          mma(gt, fa, fa);
        }
      }
      float* part = wl + (wave == 1 ? 64 : 0) + 32 * gti;
      {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = gt[r];
        int base = 0;
        reduce_scatter<16, 16>(x, lane, base);
        if ((lane & 1) == 0) part[8 * (base >> 2) + 4 * hb + (base & 3)] = x[0];
      }
      if (wave == 1) {
        float cs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) cs += gt[r];
        cs = group_sum_x32(cs);
        if (hb == 0) wl[64 + 32 + l32] = cs;
      }
    } else if (wave >= 4 && wave < 7) {
      // blocks 1 (the root, 64 positions), 2 and 3 (32 positions each) from
      // the 16-position key sums; waves 3 and 7 have no work in this stage
      const int b = wave - 3, p = lane;
      const int g0 = b == 3 ? 2 : 0, g1 = b == 2 ? 2 : 4;
      float k0s = 0.f, k1s = 0.f;
      for (int g = g0; g < g1; ++g) {
        const float2 x = ks16[g * HD + p];
        k0s += x.x;
        k1s += x.y;
      }
      const float n2 = group_sum<64>(k0s * k0s + k1s * k1s);
      const int vlo = 16 * g0, vhi = 16 * g1;
      const float knb = group_sum<64>(lane >= vlo && lane < vhi ? knv[lane] : 0.f);
      const int sz = bsz[b];
      if (sz >= 2) {
        const int prep = bst[b] + (sz - 1) / 2;
        const int64_t pr = (int64_t)(t0 + prep) * HD + p;
        const float pcs = a.rc[pr], psn = a.rs[pr];
        const float coh = knb > 0.f ? hw_div(hw_sqrt(n2), knb) : 1.f;
        if (lane == 0) bmu[b] = fmaxf(1.f, (float)sz * coh);
        const float rsz = __builtin_amdgcn_rcpf((float)sz);
        const float m0 = k0s * rsz, m1 = k1s * rsz;
        const float k0 = m0 * pcs - m1 * psn, k1 = m1 * pcs + m0 * psn;
        const uint16_t h0 = f32_to_bf16_hw(k0), h1 = f32_to_bf16_hw(k1);
        Kh[b * KR + p] = h0;
        Kh[b * KR + HD + p] = h1;
        Kl[b * KR + p] = f32_to_bf16_hw(k0 - bf16_bits_to_f32(h0));
        Kl[b * KR + HD + p] = f32_to_bf16_hw(k1 - bf16_bits_to_f32(h1));
      }
    }
    __syncthreads();
    if (wave < 3) {
      const float rn = 1.f / (float)n;
      const float rl = (wl[lane] + wl[64 + lane]) * rn;
      const float R = group_sum<64>(rl) * rn;
      if (wave == 0) {
        sdv[lane] = rl - R;
        if (lane == 0) misc[0] = R;
      }
      const int col = gtj * 32 + l32;
      const float rc = (wl[col] + wl[64 + col]) * rn;
      const bool cok = tok[col] >= 0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = gti * 32 + 8 * g + 4 * hb;
        const float4 p0 = *(const float4*)(wl + r0), p1 = *(const float4*)(wl + 64 + r0);
        const int4 tt = *(const int4*)(tok + r0);
        const float rrv[4] = {(p0.x + p1.x) * rn, (p0.y + p1.y) * rn, (p0.z + p1.z) * rn, (p0.w + p1.w) * rn};
        const int ttv[4] = {tt.x, tt.y, tt.z, tt.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = r0 + e;
          const float gv = (cok && ttv[e] >= 0) ? ((gt[4 * g + e] - rrv[e]) - rc) + R : 0.f;
          const uint16_t hi = f32_to_bf16_hw(gv), lo = f32_to_bf16_hw(gv - bf16_bits_to_f32(hi));
          Gh[row * GS + col] = hi;
          Gl[row * GS + col] = lo;
          if (gti != gtj) {
            Gh[col * GS + row] = hi;
            Gl[col * GS + row] = lo;
          }
        }
      }
    }
    __syncthreads();

    // ---- S3: prototype logits (waves 0-3); value weights and g per depth (waves 4-7)
    kvc_f32x16 lacc = {};
    if (wave < 4) {
      const int row = (wave >> 1) * 32 + l32;
      const int rho = (wave & 1) * 32 + l32;
#pragma unroll
      for (int k0 = 0; k0 < 8; k0 += 4) {
        Frag<uint16_t> qf[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          qf[u] = rho < pd ? load_frag<uint16_t>(Qu + (int64_t)rho * a.pstride * DH + (k0 + u) * 16 + 8 * hb)
                           : zero_frag<uint16_t>();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = (k0 + u) * 16 + 8 * hb;
          mma(lacc, load_frag<uint16_t>(Kh + row * KR + c), qf[u]);
          mma(lacc, load_frag<uint16_t>(Kl + row * KR + c), qf[u]);
        }
      }
    } else {
      const int v = lane;
      auto weight = [&](int lev) {
        const int b = (1 << lev) + (v >> (6 - lev));
        const int sz = bsz[b];
        const float rl = relb[b];
        const float al = rl > 0.f ? hw_div(1.f - a.beta, rl) : 0.f;
        const float ga = hw_div(rl > 0.f ? a.beta : 1.f, (float)(sz > 0 ? sz : 1));
        wl[lev * NV + v] = (sz >= 2 && tok[v] >= 0) ? fmaf(al, rv[v], ga) : 0.f;
      };
      if (wave == 4) {
        weight(0);
        __builtin_amdgcn_wave_barrier();
        depth_g<0>(Gh, Gl, wl, gw, v);
      } else if (wave == 5) {
        weight(1);
        weight(5);
        __builtin_amdgcn_wave_barrier();
        depth_g<1>(Gh, Gl, wl, gw, v);
        depth_g<5>(Gh, Gl, wl, gw, v);
      } else if (wave == 6) {
        weight(2);
        weight(4);
        __builtin_amdgcn_wave_barrier();
        depth_g<2>(Gh, Gl, wl, gw, v);
        depth_g<4>(Gh, Gl, wl, gw, v);
      } else {
        weight(3);
        __builtin_amdgcn_wave_barrier();
        depth_g<3>(Gh, Gl, wl, gw, v);
      }
    }
    __syncthreads();  // every read of the prototype keys is done before Zhat overwrites them
    if (wave < 4) {
      const int rho = (wave & 1) * 32 + l32;
      const float ls = lse_s[rho];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int b = (wave >> 1) * 32 + acc_row(r, lane);
        Zh[b * 64 + rho] = (rho < pd && bsz[b] >= 2) ? bmu[b] * fast_exp2((lacc[r] * a.c - ls) * L2E) : 0.f;
      }
    }
    __syncthreads();

    // ---- S4: value-error forms per depth (waves 0-5)
    if (w + 1 < we && (wave == 0 || wave == 2)) {
      const int64_t tok0n = a.cu[nxt.s] + nxt.t0;
      if (wave == 0) {
        int st = 0, sz = nxt.n;
#pragma unroll
        for (int lev = 0; lev < 6; ++lev) {
          const int bit = (lane >> (5 - lev)) & 1;
          if (sz >= 2) {
            const int nl = (sz + 1) >> 1;
            if (bit) {
              st += nl;
              sz -= nl;
            } else {
              sz = nl;
            }
          } else if (bit) {
            sz = 0;
          }
        }
        rel_pf = sz == 1 ? a.rel[nxt.lh * a.T + tok0n + st] : 0.f;
      } else {
        const int ln = (int)(nxt.lh / a.H), hn = (int)(nxt.lh % a.H);
        const int unitn = (nxt.s * a.Ly + ln) * a.H + hn;
        lse_pf = lane < pd ? a.lse[(int64_t)unitn * a.G * a.P + (int64_t)lane * a.pstride] : 0.f;
      }
    }
    if (wave < 6) {
      const int rt = wave & 1, lg = wave >> 1;
      const int rho = rt * 32 + l32;
      SlotRefs R{At, Gh, Gl, Zh, gw, sdv, red, misc[0], rt, lane};
      if (lg == 0) {
        depth_forms<0>(R);
        depth_forms<5>(R);
      } else if (lg == 1) {
        depth_forms<1>(R);
        depth_forms<4>(R);
      } else {
        depth_forms<2>(R);
        depth_forms<3>(R);
      }
    }
    __syncthreads();

    // ---- S5: D per node, outputs
    const int ti = wave * 64 + lane;
    if (ti < 128) {
      const int b = ti;
      float D = 0.f;
      if (b >= 1 && b < 64 && bsz[b] >= 2) {
        const float* r0 = red + b * 4;
        const float* r1 = red + (64 + b) * 4;
        const float sn = r0[0] + r1[0], sd = r0[1] + r1[1], an = r0[2] + r1[2], ad = r0[3] + r1[3];
        const float eV = sd > 0.f ? hw_div(sn, sd) : 0.f;
        const float eA = ad > 0.f ? hw_div(an, ad) : 0.f;
        D = fminf(1.f, a.wA * eA + a.wV * eV);
      }
      bD[b] = D;
    }
    __syncthreads();
    const int m = 2 * n - 1;
    for (int j = ti; j < m; j += THREADS) {
      const int b = jb[j];
      const bool inner = b < 64 && bsz[b] >= 2;
      a.node_rel[obase + j] = relb[b];
      a.node_D[obase + j] = bD[b];
      a.node_mu[obase + j] = inner ? bmu[b] : 1.f;
    }
    const float sens = a.sens[unit];
    for (int q = ti; q < 2 * n; q += THREADS) {
      float u = 0.f;
      uint8_t cst = 0;
      if (q == 0) {
        u = sens * (relb[1] * (1.f - bD[1]));
        cst = 1;
      } else if (q - 1 < m) {
        const int b = jb[q - 1];
        if (b < 64 && bsz[b] >= 2) {
          const int lc = 2 * b, rc = 2 * b + 1;
          u = sens * (relb[b] * bD[b] - (relb[lc] * bD[lc] + relb[rc] * bD[rc]));
          cst = 1;
        }
      }
      a.op_util[obase + q] = u;
      a.op_cost[obase + q] = cst;
    }
    __syncthreads();
  }
}

}  // namespace

namespace kvc_tree {

int launch_trees_v(const TreeKArgs& a, int64_t bound, int ncu, hipStream_t st) {
  static_assert(VL::total <= 80 * 1024 - 1040, "two workgroups a CU");
  auto kfn = tree_v_kernel;
  (void)hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)VL::total);
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kfn, THREADS, VL::total) != hipSuccess || per < 1) per = 1;
  int64_t grid = (int64_t)ncu * per;
  if (grid > bound) grid = bound;
  if (grid < 1) return KVC_OK;
  hipLaunchKernelGGL(kfn, dim3((unsigned)grid), dim3(THREADS), VL::total, st, a);
  KVC_LAUNCH_CHECK("tree_build_v");
  return KVC_OK;
}

}  // namespace kvc_tree
