// Per-step KL(full || compressed) through the vocab projection.
//
// DistillCache paper, Sec. 3.1.4 (Reward): the fidelity signal is
// D_KL(P_t || P^_t) between the next-token distributions of the full-cache
// and the pruned-cache model, from logits with numerical stabilization.
//
// 1. rmsnorm_cast: x^ = x / sqrt(mean x^2 + 1e-6) in fp64, cast to W's
//    dtype; the full and compressed rows of pair p become rows 2p and 2p+1.
// 2. gemm_kl: y = x^ W^T on MFMA (W is [vocab][d_model], so both operands
//    are contiguous along d_model). A workgroup owns 64 vocab columns and
//    up to 128 rows; its epilogue reduces each pair over its columns to
//    (max_f, sum_f, max_c, sum_c, sum e^(y-max_f) (y - y^)) - the logits
//    never reach memory.
// 3. kl_combine: merge the column-tile partials of every pair (one
//    workgroup per pair).
#include <cmath>

#include "kvc_internal.h"

namespace {

constexpr int THREADS = 256;
constexpr int NT = 128;    // vocab columns per workgroup (4 column waves x 32)
constexpr int MT = 128;    // rows per workgroup (4 blocks of 32 per wave)
constexpr int NCW = NT / 32;           // column waves
constexpr int RBW = MT / 32 / (4 / NCW);  // 32-row blocks per wave
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

// The same for bf16 output with d_model a multiple of 4 up to 8192: each
// thread keeps its float4 pieces of the row in registers (one read of x) and
// stores four bf16 at a time. Same arithmetic: the fp64 sum of squares (in
// another order: the sum is exact to far below the roundings that follow),
// then x * r in fp64 rounded to fp32 and to bf16.
constexpr int RMS_V4 = 8;   // float4 pieces a thread holds: d_model <= 4 * 256 * 8
__global__ __launch_bounds__(256) void rmsnorm_cast_bf16_kernel(const float* xf, const float* xc, int64_t n_pairs,
                                                                int dm, uint16_t* out) {
  const int64_t row = blockIdx.x;
  const int n4 = dm >> 2, tid = threadIdx.x;
  uint2* o = (uint2*)(out + row * dm);
  if (row >= 2 * n_pairs) {  // padding rows
    for (int i = tid; i < n4; i += 256) o[i] = make_uint2(0u, 0u);
    return;
  }
  const float4* x = (const float4*)(((row & 1) ? xc : xf) + (row >> 1) * dm);
  __shared__ double red[4];
  float4 v[RMS_V4];
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < RMS_V4; ++k) {
    const int i = tid + 256 * k;
    v[k] = i < n4 ? x[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    ss += (double)v[k].x * (double)v[k].x + (double)v[k].y * (double)v[k].y + (double)v[k].z * (double)v[k].z +
          (double)v[k].w * (double)v[k].w;
  }
  ss = wave_sum_d(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const double r = 1.0 / sqrt((red[0] + red[1] + red[2] + red[3]) / (double)dm + 1e-6);
#pragma unroll
  for (int k = 0; k < RMS_V4; ++k) {
    const int i = tid + 256 * k;
    if (i < n4) {
      const uint32_t b0 = f32_to_bf16_bits((float)((double)v[k].x * r));
      const uint32_t b1 = f32_to_bf16_bits((float)((double)v[k].y * r));
      const uint32_t b2 = f32_to_bf16_bits((float)((double)v[k].z * r));
      const uint32_t b3 = f32_to_bf16_bits((float)((double)v[k].w * r));
      o[i] = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    }
  }
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
__device__ __forceinline__ Frag<uint16_t> keep(Frag<uint16_t> f, bool k) {
  f.v = k ? f.v : kvc_bf16x8{};
  return f;
}
__device__ __forceinline__ Frag<float> keep(Frag<float> f, bool k) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = k ? f.v[j] : 0.f;
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

// Both operands go through LDS in fragment order, two stages deep: while the
// waves run the MFMAs of one k chunk, every thread already has the loads of
// the next two chunks' 16-byte pieces in flight (row-contiguous, fully
// coalesced loads of W and x^). One barrier per chunk suffices with two
// stages. Each workgroup starts at a different k chunk so that the W rows
// the grid reads at one moment do not all share an address phase. With few
// rows the kernel streams W once and is bound by HBM.
typedef unsigned int kl_u32x4 __attribute__((ext_vector_type(4)));

template <class T> struct KlTile {
  static constexpr int KC = sizeof(T) == 2 ? 128 : 64;  // k per chunk: 256 bytes of a row
  static constexpr int NKS = KC / 16;                   // 16-k MFMA steps per chunk
  static constexpr int NPC = sizeof(T) * 8 / 16;        // 16-byte pieces per fragment
  static constexpr int ELP = 16 / sizeof(T);            // elements per piece
  static constexpr int PPR = KC / ELP;                  // pieces per tile row (16)
  static constexpr int RPP = THREADS / PPR;             // tile rows per pass of the workgroup (16)
  static constexpr int XP = MT / RPP;                   // passes over the x^ tile
  static constexpr int WP = NT / RPP;                   // passes over the W tile
  static constexpr int RG = 16 / PPR;                   // rows per group of 16 storing threads
  static constexpr int SWZ = 16 / NPC - 1;              // fragment-lane swizzle mask
  static constexpr int XS = (MT / 32) * NKS * 64 * NPC; // pieces of the x^ tile
  static constexpr int WS = (NT / 32) * NKS * 64 * NPC; // pieces of the W tile
};

// LDS slot (in 16-byte pieces) of piece p of tile row `row`. Fragments are
// stored lane-contiguous; the lane index is XOR-swizzled by the fragment's
// k position so that each group of 16 storing threads (RG rows x PPR
// pieces) hits 16 different bank groups, while a wave reading one fragment
// still touches each bank group once.
template <class T>
__device__ __forceinline__ int frag_slot(int row, int p) {
  using L = KlTile<T>;
  const int k = p * L::ELP, ks = k >> 4, half = (k >> 3) & 1, sub = (k & 7) / L::ELP;
  const int ln = ((row & 31) + 32 * half) ^ (((2 * ks + half) * L::RG) & L::SWZ);
  return (((row >> 5) * L::NKS + ks) * 64 + ln) * L::NPC + sub;
}
template <class T>
__device__ __forceinline__ int frag_read(int blk, int ks, int lane) {
  using L = KlTile<T>;
  return (blk * L::NKS + ks) * 64 + (lane ^ (((2 * ks + (lane >> 5)) * L::RG) & L::SWZ));
}

// grid: (vocab / NT, m_pad / MT). part: [n_pairs][vocab / 32 column tiles][5]
template <class T>
__global__ __launch_bounds__(THREADS) void gemm_kl_kernel(const T* xh, const T* W, int64_t n_pairs, int dm,
                                                          int vocab, int64_t m_pad, float* part) {
  using L = KlTile<T>;
  extern __shared__ __align__(16) kl_u32x4 kl_lds[];  // [2][XS + WS]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cw = wave % NCW, rw = wave / NCW;
  const int64_t r0 = (int64_t)blockIdx.y * MT;
  const int nrb = (int)((m_pad - r0) < MT ? (m_pad - r0) / 32 : MT / 32);
  const int col = blockIdx.x * NT + cw * 32 + (lane & 31);
  const bool cvalid = col < vocab;
  const int nch = dm / L::KC;
  const int c0 = (int)(blockIdx.x % (unsigned)nch);
  // pieces of this thread: rows trow + RPP*i of both tiles, piece index tp
  const int trow = threadIdx.x / L::PPR, tp = threadIdx.x % L::PPR;
  const T* xb = xh + tp * L::ELP;
  const int64_t wc0 = (int64_t)blockIdx.x * NT + trow;
  const T* wb = W + tp * L::ELP;
  kl_u32x4 xr[2][L::XP], wr[2][L::WP];
  kvc_f32x16 acc[RBW];
#pragma unroll
  for (int j = 0; j < RBW; ++j) acc[j] = kvc_f32x16{};
  // Two register sets hold the next two chunks, so two chunks' loads are in
  // flight while a third is multiplied out of LDS.
  // Every fetch is issued, also past the last chunk (then it re-reads the
  // chunk of two steps before, which is still in L2): a branch around the
  // loads would make the wait before each LDS store count conservatively
  // and drain both register sets.
  auto fetch = [&](int r, int it) {
    int ch = c0 + (it < nch ? it : it - 2);
    ch = ch >= nch ? ch - nch : ch;
    ch = ch < 0 ? 0 : ch;
    const int k0 = ch * L::KC;
    // rows past the last valid one re-read row m_pad - 1: every load is
    // unconditional and in bounds, and those rows' products are never used
#pragma unroll
    for (int i = 0; i < L::XP; ++i) {
      const int64_t xrow = min(r0 + trow + L::RPP * i, m_pad - 1);
      xr[r][i] = *(const kl_u32x4*)(xb + xrow * dm + k0);
    }
#pragma unroll
    for (int i = 0; i < L::WP; ++i) {
      const int64_t wc = min(wc0 + L::RPP * i, (int64_t)vocab - 1);
      wr[r][i] = *(const kl_u32x4*)(wb + wc * dm + k0);
    }
  };
  auto step = [&](int r, int it) {
    const bool live = it < nch;  // false only for the padding step of an odd chunk count
    kl_u32x4* stg = kl_lds + r * (L::XS + L::WS);
#pragma unroll
    for (int i = 0; i < L::XP; ++i) stg[frag_slot<T>(trow + L::RPP * i, tp)] = xr[r][i];
#pragma unroll
    for (int i = 0; i < L::WP; ++i) stg[L::XS + frag_slot<T>(trow + L::RPP * i, tp)] = wr[r][i];
    __syncthreads();
    fetch(r, it + 2);
    const Frag<T>* xf = (const Frag<T>*)stg;
    const Frag<T>* wf = (const Frag<T>*)(stg + L::XS);
    // the fragments of step ks + 1 are read from LDS before the products of
    // step ks are issued (no branches around the MFMAs)
    Frag<T> b[2], a[2][RBW];
    b[0] = wf[frag_read<T>(cw, 0, lane)];
#pragma unroll
    for (int j = 0; j < RBW; ++j) a[0][j] = xf[frag_read<T>(rw * RBW + j, 0, lane)];
#pragma unroll
    for (int ks = 0; ks < L::NKS; ++ks) {
      const int c = ks & 1, n = c ^ 1;
      if (ks + 1 < L::NKS) {
        b[n] = wf[frag_read<T>(cw, ks + 1, lane)];
#pragma unroll
        for (int j = 0; j < RBW; ++j) a[n][j] = xf[frag_read<T>(rw * RBW + j, ks + 1, lane)];
      }
      const Frag<T> bk = keep(b[c], live);
#pragma unroll
      for (int j = 0; j < RBW; ++j) mma(acc[j], a[c][j], bk);
    }
  };
  fetch(0, 0);
  fetch(1, nch > 1 ? 1 : 0);
  // an odd chunk count gets one padding step whose W fragments are zero, so
  // the loop body has no branch
  for (int it = 0; it < nch; it += 2) {
    step(0, it);
    step(1, it + 1);
  }
  // epilogue: lane owns column `col`; registers v, v+1 (v%4 in {0,2}) hold
  // rows 2p and 2p+1 of one pair. Each pair's statistics over the wave's 32
  // columns: the maxima first, then one exponential per lane and sums.
  // Contraction stays off so that identical rows give identical statistics.
  const int ntile = (vocab + NT - 1) / NT;
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    const int rb = rw * RBW + j;
    if (rb >= nrb) break;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
#pragma clang fp contract(off)
      const int row = rb * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
      const int64_t pair = (r0 + row) >> 1;
      // base-2 logits for the partition sums; the logit difference is taken
      // from the accumulators themselves so identical rows give exactly 0
      const float y = cvalid ? acc[j][v] * LOG2E : -INFINITY;
      const float yh = cvalid ? acc[j][v + 1] * LOG2E : -INFINITY;
      const float dy = cvalid ? acc[j][v] - acc[j][v + 1] : 0.f;
      float mf = y, mc = yh;
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        mf = fmaxf(mf, __shfl_xor(mf, o, 64));
        mc = fmaxf(mc, __shfl_xor(mc, o, 64));
      }
      // all 32 columns past the vocab: an empty statistic
      const float ef = mf == -INFINITY ? 0.f : fast_exp2(y - mf);
      const float ec = mc == -INFINITY ? 0.f : fast_exp2(yh - mc);
      float sf = ef, sc = ec, t = ef * dy;
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        sf += __shfl_xor(sf, o, 64);
        sc += __shfl_xor(sc, o, 64);
        t += __shfl_xor(t, o, 64);
      }
      if ((lane & 31) == 0 && pair < n_pairs) {
        // column sub-tile of this wave: tiles of 32 columns
        float* p = part + ((pair * ntile + blockIdx.x) * NCW + cw) * 5;
        p[0] = mf; p[1] = sf; p[2] = mc; p[3] = sc; p[4] = t;
      }
    }
  }
}

// ------------------------------------------------------------------ many rows
// From a thousand rows on the projection is MFMA work (2 * rows * vocab *
// d_model flops against one read of W), and the small kernel above is bound
// by LDS traffic: every 32x32x16 product needs 1.25 KB of fragment reads.
// Here a workgroup of 4 waves (one per SIMD) owns a 256 x 256 output tile and
// each wave a 128 x 128 block as 8 x 8 accumulators of 16 x 16 (256
// registers a lane, held in the accumulation registers). With one wave a
// SIMD, chains of 16x16x32 products keep the matrix cores busier than
// 32x32x16 ones (94% against 76% of the bf16 peak in a register-only chain
// on MI355X). A stage is 64 k: two 16x16x32 steps of 16 fragment reads and
// 64 products a wave. Operand tiles go global -> LDS with the direct 16-byte
// LDS loads (no register staging), two stages (128 KB). A load of 64 lanes
// covers 8 tile rows x 128 bytes: whole cache lines, since the fetch rate of
// a CU is set by how many line requests it keeps in flight (half-line
// requests of 32-k stages held it near 12 bytes a clock). Lane L brings row
// L / 8, piece (L % 8) ^ f(row) of that row's 128-byte chunk, and writes it
// to the next 16 bytes of LDS, so LDS holds every row with its eight pieces
// permuted by f(row) = (row ^ (row >> 3)) & 7: a fragment read of 16
// consecutive rows at one k piece touches distinct banks. Stage it + 2 is
// fetched as soon as every wave has finished reading stage it (the barrier
// between its two steps), so the loads have a whole stage of products to
// land. The loads and the next step's fragment reads are spread over the
// products, one every four products: issued in a block, they held up the
// product issue (2.06 -> 1.89 ms a call at 8,192 rows x 4,096 x 32,768).
// Consecutive workgroups take consecutive row tiles of one column tile, so
// the W chunks in flight are shared by the workgroups running together.
constexpr int BT = 256;            // rows and vocab columns of a workgroup tile
constexpr int BK = 64;             // k of one LDS stage (two 16x16x32 products): 128 bytes a row
constexpr int BIG_MIN_ROWS = 1024; // the tiled kernel from this many (padded) rows on

__device__ __forceinline__ int kl_swz(int row) { return (row ^ (row >> 3)) & 7; }

constexpr int BIG_THREADS = 256;   // 4 waves: 1 per SIMD, each 128 rows x 128 columns
constexpr int BIG_LOADS = BT / 8 / (BIG_THREADS / 64);    // 8-row loads per operand, wave and stage (8)

typedef float kl_f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(BIG_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kl_big_kernel(const uint16_t* xh, const uint16_t* W, int64_t n_pairs, int dm, int vocab, int ntr, int ntc,
                        float* part) {
  __shared__ __align__(16) uint16_t lds[2][2][BT * BK];   // [stage][x^, W][row][k], pieces permuted
  // every argument in registers before the main loop: a scalar load still in
  // flight there would make each wait for fragment reads a wait for all of
  // them (scalar and LDS reads share one counter)
  asm volatile("" ::"s"(n_pairs), "s"(vocab), "s"(part), "s"(xh), "s"(W));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int ntiles = ntr * ntc;
  // The workgroup walks tiles blockIdx.x, + gridDim.x, ...: tile t is row
  // tile t % ntr of column tile t / ntr (row tiles fastest).
  // This lane's source in each of the wave's loads per operand and stage:
  // load j covers tile rows 8 (8 wave + j) .. + 7. The loads address each
  // operand's 256-row tile through a buffer resource (its byte size the
  // range: a load past it reads zeros), with a byte offset per lane and load
  // that is the same for both operands, every chunk and every tile, and the
  // chunk's offset in a scalar.
  const int lrow = lane >> 3;
  const int row0 = BIG_LOADS * 8 * wave + lrow;
  const int tile_bytes = BT * dm * 2;
  auto xres_of = [&](int t) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(xh + (int64_t)(t % ntr) * BT * dm), 0, tile_bytes, 0x00020000);
  };
  auto wres_of = [&](int t) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)(t / ntr) * BT * dm), 0, tile_bytes, 0x00020000);
  };
  unsigned voff[BIG_LOADS];
#pragma unroll
  for (int j = 0; j < BIG_LOADS; ++j)
    voff[j] = (unsigned)(((row0 + 8 * j) * dm + ((lane & 7) ^ kl_swz(row0 + 8 * j)) * 8) * 2);
  const int nch = dm / BK;   // even: d_model is a multiple of 128
  kl_f32x4 acc[8][8];
  // Wait states between register writes and the written-out products that
  // read them (and between those products and the reads of the results):
  // each row of accumulators passes through a no-op that takes it as an
  // operand, so the writes come before it and the reads after it.
  auto settle = [&](int a) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(acc[a][0]), "+a"(acc[a][1]), "+a"(acc[a][2]), "+a"(acc[a][3]), "+a"(acc[a][4]),
                   "+a"(acc[a][5]), "+a"(acc[a][6]), "+a"(acc[a][7]));
  };
  auto clear = [&]() {
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[a][b] = kl_f32x4{};
#pragma unroll
    for (int a = 0; a < 8; ++a) settle(a);
  };
  // load j of chunk ch (tile rows 8 (8 wave + j) .. + 7) into stage st
  auto load_x = [&](__amdgpu_buffer_rsrc_t res, int ch, int st, int j) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        res, (__attribute__((address_space(3))) void*)(lds[st][0] + (BIG_LOADS * wave + j) * 8 * BK), 16, voff[j],
        ch * BK * 2, 0, 0);
  };
  auto load_w = [&](__amdgpu_buffer_rsrc_t res, int ch, int st, int j) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        res, (__attribute__((address_space(3))) void*)(lds[st][1] + (BIG_LOADS * wave + j) * 8 * BK), 16, voff[j],
        ch * BK * 2, 0, 0);
  };
  // fragments of step ks of a stage: lane L holds row 16 u + (L & 15) of the
  // wave's x^ rows (fa[u]) and of its W rows (fb[u]), k piece 4 ks + L / 16
  // (8 consecutive k)
  const int ra = wr * 128 + (lane & 15), rb = wc * 128 + (lane & 15), kp = lane >> 4;
  auto frags = [&](int st, int ks, kvc_bf16x8* fa, kvc_bf16x8* fb) {
    const uint16_t* sx = lds[st][0];
    const uint16_t* sw = lds[st][1];
    const int q = 4 * ks + kp;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int xr = ra + 16 * u, wr2 = rb + 16 * u;
      fa[u] = __builtin_bit_cast(kvc_bf16x8, *(const uint4*)(sx + xr * BK + ((q ^ kl_swz(xr)) * 8)));
      fb[u] = __builtin_bit_cast(kvc_bf16x8, *(const uint4*)(sw + wr2 * BK + ((q ^ kl_swz(wr2)) * 8)));
    }
  };
  // Products of one step, column block by column block: fb[v] is dead after
  // its 8 products, so the next step's fb[v] (and fa'[v]) are read right
  // after them, one LDS read per four products. The next x^ fragments need a
  // second register set (fa is live to the last column), the W fragments do
  // not. The product is written out so that it accumulates in place in its
  // accumulation registers: with the reads interleaved, the compiler's own
  // register assignment moved accumulators between register files around
  // nearly every product. Volatile, so the products and the LDS reads issue
  // in this order; the inputs' waits for LDS reads are the compiler's, and
  // no product reads an accumulator written fewer than 64 products before.
  auto mfma = [](kl_f32x4& c, const kvc_bf16x8& a, const kvc_bf16x8& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  };
  // With lx/lw given the step also issues this wave's loads of chunk lch
  // into stage lst, one operand piece every four products.
  auto step = [&](const kvc_bf16x8* fa, kvc_bf16x8* fb, int nst, int nks, kvc_bf16x8* na, bool load,
                  __amdgpu_buffer_rsrc_t lx, __amdgpu_buffer_rsrc_t lw, int lch, int lst) {
    const uint16_t* sx = lds[nst][0];
    const uint16_t* sw = lds[nst][1];
    const int q = 4 * nks + kp;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
#pragma unroll
      for (int a = 0; a < 4; ++a) mfma(acc[a][v], fa[a], fb[v]);
      const int xr = ra + 16 * v;
      na[v] = __builtin_bit_cast(kvc_bf16x8, *(const uint4*)(sx + xr * BK + ((q ^ kl_swz(xr)) * 8)));
      if (load) load_x(lx, lch, lst, v);
#pragma unroll
      for (int a = 4; a < 8; ++a) mfma(acc[a][v], fa[a], fb[v]);
      if (load) load_w(lw, lch, lst, v);
      const int wr2 = rb + 16 * v;
      fb[v] = __builtin_bit_cast(kvc_bf16x8, *(const uint4*)(sw + wr2 * BK + ((q ^ kl_swz(wr2)) * 8)));
    }
  };
  // While direct LDS loads are in flight the compiler can only wait for all
  // LDS reads at once, so each fragment set is consumed (ready()) right after
  // the products that hide its reads.
  auto ready = [](const kvc_bf16x8* f) {
    asm volatile("" ::"v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]), "v"(f[4]), "v"(f[5]), "v"(f[6]), "v"(f[7]));
  };
  // epilogue of tile t: lane owns columns c0 + wc*128 + 16 v + (lane & 15),
  // v = 0..7; element i of accumulator [u][v] is row wr*128 + 16 u +
  // 4 (lane >> 4) + i, so elements 0, 1 and 2, 3 are rows 2p and 2p+1 of a
  // pair. Each pair's statistics over the wave's 128 columns: the lane's 8,
  // then the 16 lanes of its row group.
  const int nsub = vocab / 128;
  auto epilogue = [&](int t) {
    const int64_t r0 = (int64_t)(t % ntr) * BT;
    const int tc = t / ntr;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
#pragma clang fp contract(off)
        const int row = wr * 128 + 16 * u + 4 * (lane >> 4) + i;
        const int64_t pair = (r0 + row) >> 1;
        float y[8], yh[8];
        float mf = -INFINITY, mc = -INFINITY;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          y[v] = acc[u][v][i] * LOG2E;
          yh[v] = acc[u][v][i + 1] * LOG2E;
          mf = fmaxf(mf, y[v]);
          mc = fmaxf(mc, yh[v]);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          mf = fmaxf(mf, __shfl_xor(mf, o, 64));
          mc = fmaxf(mc, __shfl_xor(mc, o, 64));
        }
        float sf = 0.f, sc = 0.f, tt = 0.f;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float ef = fast_exp2(y[v] - mf), ec = fast_exp2(yh[v] - mc);
          sf += ef;
          sc += ec;
          tt += ef * (acc[u][v][i] - acc[u][v][i + 1]);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          sf += __shfl_xor(sf, o, 64);
          sc += __shfl_xor(sc, o, 64);
          tt += __shfl_xor(tt, o, 64);
        }
        if ((lane & 15) == 0 && pair < n_pairs) {
          float* pp = part + (pair * nsub + (int64_t)tc * 2 + wc) * 5;
          pp[0] = mf; pp[1] = sf; pp[2] = mc; pp[3] = sc; pp[4] = tt;
        }
      }
    }
  };
  // Iteration it of a tile multiplies stage it & 1 (chunk it) in two steps.
  // The first step reads the second step's fragments of the same stage;
  // then this wave's loads of the next chunk (the only ones in flight) are
  // waited for, and the barrier makes every wave's loads of it visible and
  // guarantees that every read of chunk it is complete, so the chunk two
  // ahead may refill its stage. A plain s_barrier, since __syncthreads would
  // also wait for the loads just issued. The second step reads the first
  // step's fragments of the next chunk and loads the chunk two ahead: in the
  // last two iterations of a tile these are chunks 0 and 1 of the
  // workgroup's next tile, so its first products wait for no load; after the
  // last tile the loads repeat the last chunk (no branch around them) and
  // nothing reads that copy, nor the fragments read past the last chunk.
  int t = blockIdx.x;
  __amdgpu_buffer_rsrc_t xres = xres_of(t), wres = wres_of(t);
#pragma unroll
  for (int j = 0; j < BIG_LOADS; ++j) {
    load_x(xres, 0, 0, j);
    load_w(wres, 0, 0, j);
  }
#pragma unroll
  for (int j = 0; j < BIG_LOADS; ++j) {
    load_x(xres, 1, 1, j);
    load_w(wres, 1, 1, j);
  }
  asm volatile("s_waitcnt vmcnt(16)" ::: "memory");   // chunk 0 landed
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  clear();
  kvc_bf16x8 fa0[8], fa1[8], fb[8];
  frags(0, 0, fa0, fb);
  ready(fa0);
  ready(fb);
  for (; t < ntiles; t += gridDim.x) {
    const int tn = t + gridDim.x;
    const bool more = tn < ntiles;
    const __amdgpu_buffer_rsrc_t nxres = more ? xres_of(tn) : xres, nwres = more ? wres_of(tn) : wres;
    for (int it = 0; it < nch; ++it) {
      const int st = it & 1;
      step(fa0, fb, st, 1, fa1, false, xres, wres, 0, 0);
      ready(fa1);
      ready(fb);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the next chunk landed
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const bool cross = it + 2 >= nch;
      const int lch = !cross ? it + 2 : (more ? it + 2 - nch : nch - 1);
      step(fa1, fb, st ^ 1, 0, fa0, true, cross ? nxres : xres, cross ? nwres : wres, lch, st);
      ready(fa0);
      ready(fb);
    }
#pragma unroll
    for (int a = 0; a < 8; ++a) settle(a);
    epilogue(t);
    clear();
    xres = nxres;
    wres = nwres;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the repeated loads of the last chunk
}

// One workgroup per pair: threads merge strided subsets of the column-tile
// partials, then the wave and the workgroup merge theirs.
__global__ __launch_bounds__(256) void kl_combine_kernel(const float* part, int64_t n_pairs, int nsub, float* kl) {
#pragma clang fp contract(off)
  __shared__ Stat5 red[4];
  const int64_t p = blockIdx.x;
  const float* q = part + p * nsub * 5;
  Stat5 st{-INFINITY, 0.f, -INFINITY, 0.f, 0.f};
  for (int i = threadIdx.x; i < nsub; i += blockDim.x) {
    Stat5 o{q[i * 5], q[i * 5 + 1], q[i * 5 + 2], q[i * 5 + 3], q[i * 5 + 4]};
    st = merge5(st, o);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    Stat5 other;
    other.mf = __shfl_xor(st.mf, o, 64);
    other.sf = __shfl_xor(st.sf, o, 64);
    other.mc = __shfl_xor(st.mc, o, 64);
    other.sc = __shfl_xor(st.sc, o, 64);
    other.t = __shfl_xor(st.t, o, 64);
    st = merge5(st, other);
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = st;
  __syncthreads();
  if (threadIdx.x != 0) return;
  st = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) st = merge5(st, red[w]);
  // natural-log partition functions from base-2 maxima
  float lse_f = (st.mf + log2f(st.sf)) * LN2, lse_c = (st.mc + log2f(st.sc)) * LN2;
  kl[p] = st.t / st.sf - lse_f + lse_c;
}

// rows padded for the kernel that will run: 256 for the tiled one, else 32
bool kl_big(int64_t n_pairs, int32_t d_model, int32_t vocab, int32_t w_dtype) {
  return w_dtype == KVC_BF16 && 2 * n_pairs >= BIG_MIN_ROWS && vocab % BT == 0 && d_model % 64 == 0;
}
int64_t kl_rows_padded(int64_t n_pairs, int32_t d_model, int32_t vocab, int32_t w_dtype) {
  const int64_t q = kl_big(n_pairs, d_model, vocab, w_dtype) ? BT : 32;
  return (2 * n_pairs + q - 1) / q * q;
}

}  // namespace

extern "C" size_t kvc_kl_workspace(int64_t n_pairs, int32_t d_model, int32_t vocab, int32_t w_dtype) {
  if (n_pairs <= 0 || d_model <= 0 || vocab <= 0) return 0;
  int64_t m_pad = kl_rows_padded(n_pairs, d_model, vocab, w_dtype);
  size_t elt = w_dtype == KVC_BF16 ? 2 : 4;
  int64_t ntile = (vocab + NT - 1) / NT;
  kvc::Carver c(nullptr, 0);
  c.take<char>((size_t)m_pad * d_model * elt);
  c.take<float>((size_t)n_pairs * ntile * NCW * 5);
  return c.off + 256;
}

extern "C" int kvc_kl(int64_t n_pairs, int32_t d_model, int32_t vocab, const float* x_full, const float* x_comp,
                      const void* W, int32_t w_dtype, float* kl_out, void* ws, size_t ws_bytes, hipStream_t st) {
  KVC_REQUIRE(n_pairs >= 0 && vocab >= 1, KVC_E_INVAL, "kvc_kl: bad sizes");
  KVC_REQUIRE(d_model >= 128 && d_model % 128 == 0, KVC_E_SHAPE, "kvc_kl: d_model must be a multiple of 128");
  KVC_REQUIRE(w_dtype == KVC_BF16 || w_dtype == KVC_F32, KVC_E_DTYPE, "kvc_kl: W must be bf16 or f32");
  if (n_pairs == 0) return KVC_OK;
  KVC_REQUIRE(x_full && x_comp && W && kl_out, KVC_E_INVAL, "kvc_kl: NULL pointer");
  KVC_REQUIRE(ws && ws_bytes >= kvc_kl_workspace(n_pairs, d_model, vocab, w_dtype), KVC_E_WORKSPACE,
              "kvc_kl: workspace too small");
  const bool big = kl_big(n_pairs, d_model, vocab, w_dtype);
  int64_t m_pad = kl_rows_padded(n_pairs, d_model, vocab, w_dtype);
  int64_t ntile = (vocab + NT - 1) / NT;
  kvc::Carver c(ws, ws_bytes);
  size_t elt = w_dtype == KVC_BF16 ? 2 : 4;
  char* xh = c.take<char>((size_t)m_pad * d_model * elt);
  float* part = c.take<float>((size_t)n_pairs * ntile * NCW * 5);
  dim3 g2((unsigned)ntile, (unsigned)((m_pad + MT - 1) / MT));
  if (w_dtype == KVC_BF16) {
    if (d_model <= 4 * 256 * RMS_V4)
      hipLaunchKernelGGL(rmsnorm_cast_bf16_kernel, dim3((unsigned)m_pad), dim3(256), 0, st, x_full, x_comp, n_pairs,
                         d_model, (uint16_t*)xh);
    else
      hipLaunchKernelGGL(rmsnorm_cast_kernel<uint16_t>, dim3((unsigned)m_pad), dim3(256), 0, st, x_full, x_comp,
                         n_pairs, d_model, m_pad, (uint16_t*)xh);
    KVC_LAUNCH_CHECK("rmsnorm_cast");
    if (big) {
      const int ntr = (int)(m_pad / BT), ntc = vocab / BT;
      // one workgroup a CU (128 KB of LDS, one wave a SIMD), each walking
      // its tiles
      int dev = 0, ncu = 0;
      (void)hipGetDevice(&dev);
      if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) ncu = 256;
      const int grid = ntr * ntc < ncu ? ntr * ntc : ncu;
      hipLaunchKernelGGL(gemm_kl_big_kernel, dim3((unsigned)grid), dim3(BIG_THREADS), 0, st,
                         (const uint16_t*)xh, (const uint16_t*)W, n_pairs, d_model, vocab, ntr, ntc, part);
      KVC_LAUNCH_CHECK("gemm_kl_big");
      hipLaunchKernelGGL(kl_combine_kernel, dim3((unsigned)n_pairs), dim3(256), 0, st, part, n_pairs, vocab / 128,
                         kl_out);
      KVC_LAUNCH_CHECK("kl_combine");
      return KVC_OK;
    }
    const int sm = 2 * (KlTile<uint16_t>::XS + KlTile<uint16_t>::WS) * 16;
    (void)hipFuncSetAttribute((const void*)gemm_kl_kernel<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize, sm);
    hipLaunchKernelGGL(gemm_kl_kernel<uint16_t>, g2, dim3(THREADS), sm, st, (const uint16_t*)xh,
                       (const uint16_t*)W, n_pairs, d_model, vocab, m_pad, part);
  } else {
    hipLaunchKernelGGL(rmsnorm_cast_kernel<float>, dim3((unsigned)m_pad), dim3(256), 0, st, x_full, x_comp, n_pairs,
                       d_model, m_pad, (float*)xh);
    KVC_LAUNCH_CHECK("rmsnorm_cast");
    const int sm = 2 * (KlTile<float>::XS + KlTile<float>::WS) * 16;
    (void)hipFuncSetAttribute((const void*)gemm_kl_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize, sm);
    hipLaunchKernelGGL(gemm_kl_kernel<float>, g2, dim3(THREADS), sm, st, (const float*)xh, (const float*)W, n_pairs,
                       d_model, vocab, m_pad, part);
  }
  KVC_LAUNCH_CHECK("gemm_kl");
  hipLaunchKernelGGL(kl_combine_kernel, dim3((unsigned)n_pairs), dim3(256), 0, st, part, n_pairs,
                     (int)(ntile * NCW), kl_out);
  KVC_LAUNCH_CHECK("kl_combine");
  return KVC_OK;
}
