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
// A persistent grid walks the slots of every (layer, KV head) unit; one
// workgroup builds one tree at a time, entirely in LDS:
//  A. node table (pre-order), relevance summed bottom-up by height (a parent
//     is exactly the fp32 sum of its children), inverse-rotated keys, and the
//     distortion rows' softmax weights a[i][rho] = exp(<q_rho,k_i>/sqrt d -
//     lse_rho) from K Q^T on MFMA;
//  B. per internal node (one wave each, lane = rotate-half pair) the summed
//     key, coherence and multiplicity and the re-rotated prototype key; the
//     prototype logits <q_rho, k^> of 32 nodes at a time on MFMA (hi/lo bf16
//     split of the fp32 keys); the attention-partition error from them;
//  C. the value-aggregate error. With c_i = a_i - Z w_i (w = the prototype's
//     value weights, sum c = 0), u - Z v^ = sum_i c_i v_i, so
//     ||u - Z v^||^2 = c^T G c and ||u||^2 = a^T G a + 2 Z a.s + Z^2 |m|^2 with
//     G the Gram matrix of the slot's values centred on their mean m (on MFMA,
//     hi/lo split) and s_i = <v_i - m, m>. Lane rho evaluates its two forms
//     over the node's block of G; the root and its children are spread over
//     every wave by 8-row blocks, deeper nodes take one wave each.
#include <cmath>

#include "kvc_internal.h"
#include "mfma_frag.h"
#include "trees_common.h"

namespace {

using namespace kvc_tree;

constexpr int PDMAX = 64;   // distortion rows (one per lane)
constexpr int PA = 64;      // token stride of the softmax weights a[i][rho]
constexpr int NB = 32;      // internal nodes per prototype-logit batch
constexpr int LGS = PDMAX + 4;
constexpr int SMALL = 64;   // slots up to this length use the small-slot variant


// LDS layout (byte offsets, 16-byte aligned) for slots of at most NMAX tokens.
template <int NMAX, int D, int WAVES>
struct TreeLayout {
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr int N32 = (NMAX + 31) & ~31;
  static constexpr int NG = N32 + 4;  // row stride of the Gram matrix
  static constexpr size_t KT = (size_t)NMAX * D * 4, GM = (size_t)N32 * NG * 4;
  // prototype keys of a batch: [NB][D + 8] as two bf16 pieces (hi, lo) for bf16 inputs, one fp32 row otherwise
  static constexpr size_t KHB = (size_t)NB * (D + 8) * 4, PARTB = (size_t)WAVES * 3 * 2 * PDMAX * 4;
  // Small slots stage the centred values in fp32 ([N32][D + 4]) over the keys
  // and put the Gram matrix over the prototype keys; large slots keep the Gram
  // matrix over the keys and centre on the fly.
  static constexpr bool STAGED = NMAX <= SMALL;
  static constexpr int VS = D + 8;    // row stride of the staged centred values (elements)
  static constexpr size_t VSB = STAGED ? (size_t)N32 * VS * 4 : 0;
  static constexpr size_t R1B = STAGED ? (KT > VSB ? KT : VSB) : (KT > GM ? KT : GM);
  static constexpr size_t KHR = STAGED ? (KHB > GM ? KHB : GM) : (KHB > PARTB ? KHB : PARTB);
  static_assert(!STAGED || PARTB <= R1B, "partials fit over the staged values");
  static constexpr size_t r1 = 0;
  static constexpr size_t at = al(r1 + R1B);
  static constexpr size_t kh = al(at + (size_t)NMAX * PA * 4);
  // the logits of a batch overwrite its prototype keys once the MFMA has read them
  static constexpr size_t lg = kh;
  static_assert((size_t)NB * LGS * 4 <= KHB, "logits fit over the prototype keys");
  static constexpr size_t vm = al(kh + KHR);
  static constexpr size_t sdot = al(vm + (size_t)D * 4);
  static constexpr size_t knorm = al(sdot + (size_t)NMAX * 4);
  static constexpr size_t rtok = al(knorm + (size_t)NMAX * 4);
  static constexpr size_t lse = al(rtok + (size_t)NMAX * 4);
  static constexpr size_t zc = al(lse + PDMAX * 4);
  static constexpr size_t nrel = al(zc + 3 * 2 * PDMAX * 4);
  static constexpr size_t nmu = al(nrel + (size_t)2 * NMAX * 4);
  static constexpr size_t nD = al(nmu + (size_t)2 * NMAX * 4);
  static constexpr size_t nst = al(nD + (size_t)2 * NMAX * 4);
  static constexpr size_t nsz = al(nst + (size_t)2 * NMAX * 2);
  static constexpr size_t ndep = al(nsz + (size_t)2 * NMAX * 2);
  static constexpr size_t ilist = al(ndep + (size_t)2 * NMAX * 2);
  static constexpr size_t npar = al(ilist + (size_t)NMAX * 2);
  static constexpr size_t nsib = al(npar + (size_t)2 * NMAX * 2);
  static constexpr size_t misc = al(nsib + (size_t)2 * NMAX * 2);
  static constexpr size_t total = al(misc + 32);
  // value-error scratch of midpoint trees (small slots), over the staged values
  // once the Gram matrix is formed: cross-block partials, the (a^T G a, Z, a.s)
  // of the children and grandchildren of the root, the big nodes' G w vectors
  // and w^T G w, and the root's a^T G w partials
  static constexpr int MP_ITEMS = 20;
  // with room in r1 the Gram matrix of midpoint trees goes there too, so the
  // prototype logits (over kh) survive until the value error is formed and
  // both errors of a node are finished together
  static constexpr size_t MP_BYTES = 3 * 6 * PDMAX * 4 + 3 * NMAX * 4 + 16 + 4 * PDMAX * 4 + MP_ITEMS * PDMAX * 4 + 5 * 16;
  static constexpr bool LGKEEP = STAGED && al(GM) + MP_BYTES <= R1B;
  static constexpr size_t mp_part = LGKEEP ? al(GM) : 0;
  static constexpr size_t mp_q = al(mp_part + (size_t)MP_ITEMS * PDMAX * 4);
  static constexpr size_t mp_gv = al(mp_q + (size_t)3 * 6 * PDMAX * 4);
  static constexpr size_t mp_w = al(mp_gv + (size_t)3 * NMAX * 4);
  static constexpr size_t mp_rq = al(mp_w + 16);
  static constexpr size_t mp_end = al(mp_rq + (size_t)4 * PDMAX * 4);
  static_assert(!STAGED || mp_end <= R1B, "midpoint value-error scratch fits over the staged values");
  // phase-A scratch for the per-group value column sums lives in the weight array
  static_assert((size_t)(WAVES * 64 / (D / 8)) * D * 4 <= (size_t)NMAX * PA * 4, "value-sum scratch");
};


// x = hi + lo in bf16 pieces, each the round-to-nearest-even of the
// remainder so far: |x - hi - lo| <= 2^-18 |x|
__device__ __forceinline__ void split8(float* x, kvc_bf16x8& hi, kvc_bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint16_t b = f32_to_bf16_hw(x[j]);
    x[j] -= bf16_bits_to_f32(b);
    hi[j] = __builtin_bit_cast(__bf16, b);
    uint16_t c = f32_to_bf16_hw(x[j]);
    x[j] -= bf16_bits_to_f32(c);
    lo[j] = __builtin_bit_cast(__bf16, c);
  }
}

// 8 raw elements (loaded now, converted later, so that many loads are in flight)
template <class T> struct Raw8;
template <> struct Raw8<uint16_t> {
  uint4 u;
  __device__ __forceinline__ void load(const uint16_t* p) { u = *(const uint4*)p; }
  __device__ __forceinline__ void zero() { u = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void get(float* o) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) { a = *(const float4*)p; b = *(const float4*)(p + 4); }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void get(float* o) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

// One 8-row block [i0, i0+8) of a node's two quadratic forms for lane rho,
// using the symmetry of G: for every row i of the block, the columns j < i of
// the node count twice and j = i once, so that summing over all blocks gives
// num += c^T G c and den += a^T G a.
__device__ __forceinline__ void qform_block(const float* Gm, int NG, const float* At, const float* rtok, int lane,
                                            int i0, int st, int sz, float Z, float al, float ga, float& num,
                                            float& den) {
  float ci[8], ai[8], tc[8], ta[8];
  const int e = st + sz;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = i0 + k;
    float av = 0.f, cv = 0.f;
    if (i >= st && i < e) {
      av = At[i * PA + lane];
      cv = av - Z * fmaf(al, rtok[i], ga);
    }
    ai[k] = av;
    ci[k] = cv;
    tc[k] = 0.f;
    ta[k] = 0.f;
  }
  // columns before the block: every row of the block lies below them
  const int jm = min(i0, e);
#pragma unroll 2
  for (int j = st; j < jm; ++j) {
    const float4 g0 = *(const float4*)(Gm + j * NG + i0), g1 = *(const float4*)(Gm + j * NG + i0 + 4);
    const float aj = At[j * PA + lane];
    const float cj = aj - Z * fmaf(al, rtok[j], ga);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      tc[k] = fmaf(g[k], cj, tc[k]);
      ta[k] = fmaf(g[k], aj, ta[k]);
    }
  }
  // the block's own columns: weight 1 below the diagonal, 1/2 on it
  for (int j = max(i0, st); j < min(i0 + 8, e); ++j) {
    const float4 g0 = *(const float4*)(Gm + j * NG + i0), g1 = *(const float4*)(Gm + j * NG + i0 + 4);
    const float aj = At[j * PA + lane];
    const float cj = aj - Z * fmaf(al, rtok[j], ga);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const int jj = j - i0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float w = k > jj ? g[k] : (k == jj ? 0.5f * g[k] : 0.f);
      tc[k] = fmaf(w, cj, tc[k]);
      ta[k] = fmaf(w, aj, ta[k]);
    }
  }
  float sn = 0.f, sd = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sn = fmaf(ci[k], tc[k], sn);
    sd = fmaf(ai[k], ta[k], sd);
  }
  num = fmaf(2.f, sn, num);
  den = fmaf(2.f, sd, den);
}

// Value-aggregate forms of one node of at most S tokens, lane = distortion row:
// Z = sum a_i, as = sum a_i s_i and, with c_i = a_i - Z w_i (w_i = al r_i + ga),
// num = c^T G c and qa = a^T G a over the node's block of the centred value
// Gram, each pair of tokens once by symmetry. sz is uniform over the wave.
template <int S>
__device__ __forceinline__ void small_forms(const float* Gm, int NG, const float* At, const float* rtok,
                                            const float* sdot, int lane, int st, int sz, int nrows, float al,
                                            float ga, float& Z, float& as, float& num, float& qa) {
  // a window of S tokens [ws, ws + S) inside the first nrows rows (where the
  // Gram matrix is written) holds the node; tokens of the window outside the
  // node are masked to zero, and every load is an immediate offset from one
  // base, so the whole block of loads can be in flight at once
  const int ws = min(st, nrows - S);
  const float* Ab = At + ws * PA + lane;
  const float* Gb = Gm + ws * NG + ws;
  float av[S], cv[S];
  bool in[S];
  Z = 0.f;
  as = 0.f;
#pragma unroll
  for (int k = 0; k < S; ++k) {
    in[k] = ws + k >= st && ws + k < st + sz;
    const float x = Ab[k * PA], sd = sdot[ws + k];
    av[k] = in[k] ? x : 0.f;
    Z += av[k];
    as = fmaf(av[k], in[k] ? sd : 0.f, as);
  }
#pragma unroll
  for (int k = 0; k < S; ++k) {
    const float c = av[k] - Z * fmaf(al, rtok[ws + k], ga);
    cv[k] = in[k] ? c : 0.f;
  }
  num = 0.f;
  qa = 0.f;
#pragma unroll
  for (int k = 0; k < S; ++k) {
    const float gd = 0.5f * Gb[k * NG + k];
    float tc = gd * cv[k], ta = gd * av[k];
#pragma unroll
    for (int l = k + 1; l < S; ++l) {
      const float g = Gb[k * NG + l];
      tc = fmaf(g, cv[l], tc);
      ta = fmaf(g, av[l], ta);
    }
    num = fmaf(cv[k], tc, num);
    qa = fmaf(av[k], ta, qa);
  }
  num *= 2.f;
  qa *= 2.f;
}

// Pairs of one cross block: rows [r_lo, r_hi) inside the aligned 4-row group
// g, columns [c_lo, c_hi): sum_r a_r sum_j G_rj a_j for lane = distortion row
// (G is symmetric, so the group's four entries of row j are one 16-byte read).
__device__ __forceinline__ float cross_block(const float* Gm, int NG, const float* At, int lane, int g, int r_lo,
                                             int r_hi, int c_lo, int c_hi) {
  float ar[4], t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * g + e;
    ar[e] = (r >= r_lo && r < r_hi) ? At[r * PA + lane] : 0.f;
  }
#pragma unroll 4
  for (int j = c_lo; j < c_hi; ++j) {
    const float aj = At[j * PA + lane];
    const float4 g4 = *(const float4*)(Gm + j * NG + 4 * g);
    t[0] = fmaf(g4.x, aj, t[0]);
    t[1] = fmaf(g4.y, aj, t[1]);
    t[2] = fmaf(g4.z, aj, t[2]);
    t[3] = fmaf(g4.w, aj, t[3]);
  }
  return fmaf(ar[0], t[0], fmaf(ar[1], t[1], fmaf(ar[2], t[2], ar[3] * t[3])));
}


template <class T, int D, int NMAX, int WAVES, int OCC>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(OCC))) void tree_kernel(TreeKArgs a) {
  using namespace kvcmf;
  using Lo = TreeLayout<NMAX, D, WAVES>;
  constexpr int THREADS = WAVES * 64;
  constexpr int HD = D / 2;
  constexpr int KS = D / 16;
  constexpr int KHS = D + 8;                // row stride of the prototype-key pieces (elements)
  constexpr int NG = Lo::NG;
  constexpr int CH = HD / 8;              // 8-wide chunks per key half
  constexpr int VC = D / 8;               // 8-wide chunks per value row
  constexpr int VG = THREADS / VC;        // token groups for the value statistics
  constexpr int VR = (NMAX + VG - 1) / VG;
  constexpr int NPW = NB / WAVES;         // nodes per wave in a logit batch
  extern __shared__ __align__(16) char smem[];
  constexpr bool STAGED = Lo::STAGED;
  float* Kt = (float*)(smem + Lo::r1);     // [NMAX][D] inverse-rotated keys (phases A, B)
  float* Vc = (float*)(smem + Lo::r1);     // [N32][VS] centred values (phase C, small slots)
  float* Gm = (float*)(smem + (STAGED ? Lo::kh : Lo::r1));  // [N32][NG] centred value Gram (phase C)
  float* At = (float*)(smem + Lo::at);     // [NMAX][PA] softmax weights of the distortion rows
  float* vsum = (float*)(smem + Lo::at);   // [VG][D] value column sums (phase A, before At)
  float* KH = (float*)(smem + Lo::kh);     // [NB][KHS] fp32 prototype keys of one batch (fp32 inputs)
  uint16_t* KHh = (uint16_t*)(smem + Lo::kh);          // [NB][KHS] hi bf16 pieces (bf16 inputs)
  uint16_t* KHl = KHh + (size_t)NB * KHS;               // [NB][KHS] lo bf16 pieces
                                           // then [NB][LGS] their logits
  float* part = (float*)(smem + (STAGED ? Lo::r1 : Lo::kh));  // [WAVES][3][2][PDMAX] quadratic-form partials (C)
  float* LG = (float*)(smem + Lo::lg);     // [NB][LGS] prototype logits of one batch (over KH)
  float* vm = (float*)(smem + Lo::vm);     // [D] value mean of the slot
  float* sdot = (float*)(smem + Lo::sdot); // [NMAX] <v_i - m, m>
  float* knorm = (float*)(smem + Lo::knorm);
  float* rtok = (float*)(smem + Lo::rtok);
  float* lse_s = (float*)(smem + Lo::lse);
  float* zc = (float*)(smem + Lo::zc);     // [3][2][PDMAX] Z and a.s of the root and its children
  float* nrel = (float*)(smem + Lo::nrel);
  float* nmu = (float*)(smem + Lo::nmu);
  float* nD = (float*)(smem + Lo::nD);
  int16_t* nst = (int16_t*)(smem + Lo::nst);
  int16_t* nsz = (int16_t*)(smem + Lo::nsz);
  int16_t* ndep = (int16_t*)(smem + Lo::ndep);
  int16_t* ilist = (int16_t*)(smem + Lo::ilist);
  int16_t* npar = (int16_t*)(smem + Lo::npar);   // explicit trees: parent index (-1 root)
  int16_t* nsib = (int16_t*)(smem + Lo::nsib);   // explicit trees: next sibling (0 none)
  float* misc = (float*)(smem + Lo::misc);
  int* imisc = (int*)(misc + 4);           // explicit trees: node count, deepest level, root's last child

  __shared__ int pre[MAX_SEQ + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  for (int64_t w = wb; w < we; ++w) {
    const ItemDesc cur = nxt;
    if (w + 1 < we) nxt = item_desc(a, pre, nsl, w + 1);  // in flight during this slot
    const int64_t lh = cur.lh;
    const int s = cur.s, t0 = cur.t0, n = cur.n;
    const int l = (int)(lh / a.H), h = (int)(lh % a.H);
    int m = 2 * n - 1, nint = n - 1;       // midpoint trees; explicit trees set these below
    const int n32 = (n + 31) & ~31;
    const int64_t tok0 = a.cu[s] + t0;
    const int64_t obase = lh * 2 * a.T + 2 * tok0;
    const T* Kg = (const T*)a.K + (lh * a.T + tok0) * D;
    const T* Vg = (const T*)a.V + (lh * a.T + tok0) * D;
    const int unit = (s * a.Ly + l) * a.H + h;
    const T* Qu = (const T*)a.Qp + ((((int64_t)s * a.Ly + l) * a.H * a.G + (int64_t)h * a.G) * a.P) * D;
    const float* lse_g = a.lse + (int64_t)unit * a.G * a.P;

    // ---- A: node table, token data, value statistics, softmax weights
    // (in any pre-order tree whose leaves are the tokens in order, the nodes
    // before j are its ancestors and the subtrees left of it, whose leaves are
    // the tokens left of st: so j - st internal nodes precede j)
    if (a.topo) {
      const uint32_t* rec = a.topo + obase;
      for (int j = tid; j < 2 * n; j += THREADS) {
        const uint32_t x = rec[j];
        if (x == 0xFFFFFFFFu) continue;
        const int st = (int)(x & 255), sz = (int)((x >> 8) & 255) + 1, par = (int)((x >> 16) & 255) - 1;
        nst[j] = (int16_t)st;
        nsz[j] = (int16_t)sz;
        npar[j] = (int16_t)par;
        nsib[j] = (int16_t)(x >> 24);
        if (j + 1 == 2 * n || rec[j + 1] == 0xFFFFFFFFu) imisc[0] = j + 1;
        if (par == 0 && (x >> 24) == 0) imisc[2] = j;
        if (sz > 1) ilist[j - st] = (int16_t)j;
        else {
          nD[j] = 0.f;
          nmu[j] = 1.f;
        }
      }
      if (tid == 0) imisc[1] = 0;
      __syncthreads();
      m = imisc[0];
      nint = m - n;
      for (int j = tid; j < m; j += THREADS) {
        int dep = 0;
        for (int p = npar[j]; p >= 0; p = npar[p]) ++dep;
        ndep[j] = (int16_t)dep;
        if (nsz[j] > 1) atomicMax(&imisc[1], dep);
      }
    } else {
      for (int j = tid; j < m; j += THREADS) {
        int cu = 0, st = 0, sz = n, dep = 0;
        while (cu != j) {
          int nl = (sz + 1) >> 1;
          if (j < cu + 2 * nl) {
            cu += 1;
            sz = nl;
          } else {
            cu += 2 * nl;
            st += nl;
            sz -= nl;
          }
          ++dep;
        }
        nst[j] = (int16_t)st;
        nsz[j] = (int16_t)sz;
        ndep[j] = (int16_t)dep;
        if (sz > 1) ilist[j - st] = (int16_t)j;
        else {
          nD[j] = 0.f;
          nmu[j] = 1.f;
        }
      }
    }
    for (int rho = tid; rho < PDMAX; rho += THREADS) lse_s[rho] = rho < pd ? lse_g[(int64_t)rho * a.pstride] : 0.f;
    for (int i = tid; i < n; i += THREADS) rtok[i] = a.rel[lh * a.T + tok0 + i];
    // the value rows for the statistics below, loaded first so that they arrive
    // while the keys are rotated: thread (group g, chunk vc) keeps tokens g, g+VG, ...
    const int vc = (tid % VC) * 8, vg = tid / VC;
    Raw8<T> vr[VR];
#pragma unroll
    for (int r = 0; r < VR; ++r) {
      const int i = vg + r * VG;
      if (i < n) vr[r].load(Vg + (int64_t)i * D + vc);
      else vr[r].zero();
    }
    // inverse-rotated keys and key norms: one 8-pair chunk per item, all loads issued together
#pragma unroll
    for (int r = 0; r < (NMAX * CH + THREADS - 1) / THREADS; ++r) {
      const int it = tid + r * THREADS;
      const int i = it / CH, c = (it % CH) * 8;
      const bool ok = i < n;
      Raw8<T> k0, k1;
      float4 c0, c1, s0, s1;
      if (ok) {
        k0.load(Kg + (int64_t)i * D + c);
        k1.load(Kg + (int64_t)i * D + c + HD);
        const int64_t pr = (int64_t)(t0 + i) * HD + c;
        c0 = *(const float4*)(a.rc + pr);
        c1 = *(const float4*)(a.rc + pr + 4);
        s0 = *(const float4*)(a.rs + pr);
        s1 = *(const float4*)(a.rs + pr + 4);
      } else {
        k0.zero();
        k1.zero();
        c0 = c1 = s0 = s1 = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      float x0[8], x1[8];
      k0.get(x0);
      k1.get(x1);
      const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      float q = 0.f, y0[8], y1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        q += x0[e] * x0[e] + x1[e] * x1[e];
        y0[e] = x0[e] * cs[e] + x1[e] * sn[e];   // rotation by -theta
        y1[e] = x1[e] * cs[e] - x0[e] * sn[e];
      }
      q = group_sum<CH>(q);
      if (ok) {
        if constexpr (STAGED) {
          // the two halves of each rotation pair side by side: (d, d + HD) at 2d, 2d + 1
          float* d0 = Kt + (size_t)i * D + 2 * c;
#pragma unroll
          for (int e = 0; e < 8; e += 2) *(float4*)(d0 + 2 * e) = make_float4(y0[e], y1[e], y0[e + 1], y1[e + 1]);
        } else {
          float* d0 = Kt + (size_t)i * D + c;
          *(float4*)d0 = make_float4(y0[0], y0[1], y0[2], y0[3]);
          *(float4*)(d0 + 4) = make_float4(y0[4], y0[5], y0[6], y0[7]);
          *(float4*)(d0 + HD) = make_float4(y1[0], y1[1], y1[2], y1[3]);
          *(float4*)(d0 + HD + 4) = make_float4(y1[4], y1[5], y1[6], y1[7]);
        }
        if (c == 0) knorm[i] = hw_sqrt(q);
      }
    }
    // value statistics (the value rows were loaded before the keys)
    {
      float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < VR; ++r) {
        float x[8];
        vr[r].get(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] += x[e];
      }
      float* dst = vsum + (size_t)vg * D + vc;
      *(float4*)dst = make_float4(cs[0], cs[1], cs[2], cs[3]);
      *(float4*)(dst + 4) = make_float4(cs[4], cs[5], cs[6], cs[7]);
    }
    __syncthreads();
    for (int dd = tid; dd < D; dd += THREADS) {
      float acc = 0.f;
#pragma unroll
      for (int g = 0; g < VG; ++g) acc += vsum[g * D + dd];
      vm[dd] = hw_div(acc, (float)n);
    }
    __syncthreads();
    {
      float vmc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vmc[e] = vm[vc + e];
#pragma unroll
      for (int r = 0; r < VR; ++r) {
        const int i = vg + r * VG;
        float x[8], q = 0.f;
        vr[r].get(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) q = fmaf(x[e] - vmc[e], vmc[e], q);
        q = group_sum<VC>(q);
        if (i < n && (tid % VC) == 0) sdot[i] = q;
      }
      if (wave == 0) {
        float q = 0.f;
        for (int dd = lane; dd < D; dd += 64) q += vm[dd] * vm[dd];
        q = group_sum<64>(q);
        if (lane == 0) misc[0] = q;
      }
    }
    // softmax weights of the distortion rows on MFMA (K Q^T); the value-sum
    // scratch in the same array was consumed before the barrier above
    {
      const int ntb = n32 / 32, nrb = (pd + 31) / 32;
      for (int tile = wave; tile < ntb * nrb; tile += WAVES) {
        int tb = tile / nrb, rb = tile % nrb;
        int tok = tb * 32 + (lane & 31), rho = rb * 32 + (lane & 31);
        kvc_f32x16 acc = {};
#pragma unroll
        for (int k0 = 0; k0 < KS; k0 += KS / 2) {  // half the steps' loads in flight at a time
          Frag<T> ka[KS / 2], qb[KS / 2];
#pragma unroll
          for (int u = 0; u < KS / 2; ++u) {
            int c = (k0 + u) * 16 + 8 * (lane >> 5);
            ka[u] = tok < n ? load_frag<T>(Kg + (int64_t)tok * D + c) : zero_frag<T>();
            qb[u] = rho < pd ? load_frag<T>(Qu + (int64_t)rho * a.pstride * D + c) : zero_frag<T>();
          }
#pragma unroll
          for (int u = 0; u < KS / 2; ++u) mma(acc, ka[u], qb[u]);
        }
        float ls = lse_s[rho];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          int ti = tb * 32 + acc_row(v, lane);
          if (ti < n && rho < pd) At[ti * PA + rho] = fast_exp2((acc[v] * a.c - ls) * 1.4426950408889634f);
        }
      }
      if (pd < PDMAX)
        for (int it = tid; it < n * (PDMAX - pd); it += THREADS) At[(it / (PDMAX - pd)) * PA + pd + it % (PDMAX - pd)] = 0.f;
    }
    // bottom-up value flow: a parent is the fp32 sum of its children, left to
    // right. One wave (idle in the weights' MFMA for slots of up to 64 tokens)
    // runs every level; its LDS accesses stay in order, so the levels need no
    // workgroup barrier; the barriers of phase B publish nrel before C reads it.
    if (wave == WAVES - 1) {
      for (int j = lane; j < m; j += 64)
        if (nsz[j] == 1) nrel[j] = rtok[nst[j]];
      if (a.topo) {  // by depth, deepest internal level first (first child j+1, then the sibling chain)
        for (int dd = imisc[1]; dd >= 0; --dd) {
          __builtin_amdgcn_wave_barrier();
          for (int j = lane; j < m; j += 64)
            if (nsz[j] > 1 && ndep[j] == dd) {
              float sum = nrel[j + 1];
              for (int c = nsib[j + 1]; c != 0; c = nsib[c]) sum += nrel[c];
              nrel[j] = sum;
            }
        }
      } else {  // by height (children of pre-order node j: j+1 and j + 2 ceil(sz/2))
        for (int ht = 1; (1 << (ht - 1)) < n; ++ht) {
          __builtin_amdgcn_wave_barrier();
          for (int j = lane; j < m; j += 64) {
            int sz = nsz[j];
            if (sz > 1 && 32 - __clz(sz - 1) == ht) nrel[j] = nrel[j + 1] + nrel[j + 2 * ((sz + 1) >> 1)];
          }
        }
      }
    }

    // ---- B: prototype keys, multiplicity, attention-partition error
    const int nrb = (pd + 31) / 32;
    if constexpr (STAGED) {
      // Every internal node at once (at most 63): each wave forms the summed
      // keys, multiplicities and prototype keys of its nodes in registers; once
      // every sum has read the inverse-rotated keys, the prototype keys replace
      // them (bf16 hi/lo pieces, or fp32) and each of up to four waves runs one
      // 32x32 tile of the prototype logits on MFMA.
      constexpr int NPW2 = (NMAX + WAVES - 1) / WAVES;
      const int nbk = (nint + 31) / 32;
      const int ntile = nrb * nbk;
      const int trb = wave % max(nrb, 1), tnb = wave / max(nrb, 1);
      const int rho_t = trb * 32 + (lane & 31);
      // Summed keys: a wave instruction reads NR rows of the interleaved keys,
      // 16 bytes a lane (lane = (row of the instruction, 4-float column)); the
      // rows of the other lane groups are added by lane swaps, after which a
      // lane of the first two groups keeps one rotation pair (d, d + HD)
      constexpr int R4 = D / 4, NR = 64 / R4;
      static_assert(NR == 2 || NR == 4, "rows per instruction");
      const int rsub = lane / R4, kq = lane % R4;
      const int dsel = 2 * kq + (rsub & 1);
      const bool own = rsub < 2;
      const float4* Kt4 = (const float4*)Kt;
      float pc[NPW2], ps[NPW2];
#pragma unroll
      for (int u = 0; u < NPW2; ++u) {
        const int qq = wave + u * WAVES;
        pc[u] = ps[u] = 0.f;
        if (qq < nint && own) {
          const int j = ilist[qq];
          const int64_t prep = t0 + nst[j] + (nsz[j] - 1) / 2;
          pc[u] = a.rc[prep * HD + dsel];
          ps[u] = a.rs[prep * HD + dsel];
        }
      }
      float kp0[NPW2], kp1[NPW2];
#pragma unroll
      for (int u = 0; u < NPW2; ++u) {
        const int qq = wave + u * WAVES;
        kp0[u] = kp1[u] = 0.f;
        if (qq >= nint) continue;
        const int j = ilist[qq];
        const int st = nst[j], sz = nsz[j];
        float4 ac = make_float4(0.f, 0.f, 0.f, 0.f);
        float kn = 0.f;
#pragma unroll 4
        for (int i = st + rsub; i < st + sz; i += NR) {
          const float4 x = Kt4[(size_t)i * R4 + kq];
          ac.x += x.x;
          ac.y += x.y;
          ac.z += x.z;
          ac.w += x.w;
          kn += knorm[i];
        }
        if constexpr (NR == 2) {
          ac.x = group_sum_x32(ac.x);
          ac.y = group_sum_x32(ac.y);
          ac.z = group_sum_x32(ac.z);
          ac.w = group_sum_x32(ac.w);
          kn = group_sum_x32(kn);
        } else {
          ac.x = cross_row_sum(ac.x);
          ac.y = cross_row_sum(ac.y);
          ac.z = cross_row_sum(ac.z);
          ac.w = cross_row_sum(ac.w);
          kn = cross_row_sum(kn);
        }
        const float nrm2 = group_sum<R4>(ac.x * ac.x + ac.y * ac.y + ac.z * ac.z + ac.w * ac.w);
        const float coh = kn > 0.f ? hw_div(hw_sqrt(nrm2), kn) : 1.f;
        const float mu = fmaxf(1.f, (float)sz * coh);
        if (lane == 0) nmu[j] = mu;
        const float rsz = __builtin_amdgcn_rcpf((float)sz);
        const float m0 = ((rsub & 1) ? ac.z : ac.x) * rsz, m1 = ((rsub & 1) ? ac.w : ac.y) * rsz;
        kp0[u] = m0 * pc[u] - m1 * ps[u];
        kp1[u] = m1 * pc[u] + m0 * ps[u];
      }
      __syncthreads();  // every sum has read the inverse-rotated keys
      uint16_t* PKh = (uint16_t*)(smem + Lo::r1);  // [64][KHS] hi pieces (bf16 inputs)
      uint16_t* PKl = PKh + (size_t)64 * KHS;       // [64][KHS] lo pieces
      float* PK = (float*)(smem + Lo::r1);         // [64][KHS] fp32 keys (fp32 inputs)
      static_assert((size_t)64 * KHS * 4 <= Lo::R1B, "prototype keys of every node fit over the keys");
#pragma unroll
      for (int u = 0; u < NPW2; ++u) {
        const int qq = wave + u * WAVES;
        if (qq >= nint || !own) continue;
        if constexpr (sizeof(T) == 2) {
          // k^ = hi + lo with |k^ - hi - lo| <= 2^-18 |k^|; the queries are exact in bf16
          const uint16_t h0 = f32_to_bf16_hw(kp0[u]), h1 = f32_to_bf16_hw(kp1[u]);
          PKh[qq * KHS + dsel] = h0;
          PKh[qq * KHS + dsel + HD] = h1;
          PKl[qq * KHS + dsel] = f32_to_bf16_hw(kp0[u] - bf16_bits_to_f32(h0));
          PKl[qq * KHS + dsel + HD] = f32_to_bf16_hw(kp1[u] - bf16_bits_to_f32(h1));
        } else {
          PK[qq * KHS + dsel] = kp0[u];
          PK[qq * KHS + dsel + HD] = kp1[u];
        }
      }
      __syncthreads();
      float* LGa = (float*)(smem + Lo::kh);  // [64][LGS] prototype logits of every node
      static_assert((size_t)64 * LGS * 4 <= Lo::KHR, "logits of every node fit");
      if (wave < ntile) {
        kvc_f32x16 acc = {};
        const int row = tnb * 32 + (lane & 31);
#pragma unroll
        for (int u = 0; u < KS; ++u) {
          const int c = u * 16 + 8 * (lane >> 5);
          const Frag<T> qf = rho_t < pd ? load_frag<T>(Qu + (int64_t)rho_t * a.pstride * D + c) : zero_frag<T>();
          if constexpr (sizeof(T) == 2) {
            mma(acc, load_frag<uint16_t>(PKh + row * KHS + c), qf);
            mma(acc, load_frag<uint16_t>(PKl + row * KHS + c), qf);
          } else {
            mma(acc, load_frag<T>(PK + row * KHS + c), qf);
          }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) LGa[(tnb * 32 + acc_row(v, lane)) * LGS + rho_t] = acc[v];
      }
      __syncthreads();
      // the attention-partition error: here for explicit trees (and when the
      // logits cannot be kept), else with the value error in C
#pragma unroll
      for (int u = 0; u < NPW2; ++u) {
        if (Lo::LGKEEP && !a.topo) break;
        const int qq = wave + u * WAVES;
        if (qq >= nint) continue;
        const int j = ilist[qq];
        const int st = nst[j], sz = nsz[j];
        float z = 0.f, zh = 0.f;
        if (lane < pd) {
#pragma unroll 8
          for (int i = st; i < st + sz; ++i) z += At[i * PA + lane];
          zh = nmu[j] * fast_exp2((LGa[qq * LGS + lane] * a.c - lse_s[lane]) * 1.4426950408889634f);
        }
        const float eAn = group_sum<64>(fabsf(zh - z)), eAd = group_sum<64>(z);
        if (lane == 0) nD[j] = eAd > 0.f ? hw_div(eAn, eAd) : 0.f;
      }
      // the value staging of C overwrites the keys only after its own barrier
    } else
    for (int q0 = 0; q0 < nint; q0 += NB) {
      const int nb = min(NB, nint - q0);
      float pc[NPW], ps[NPW];
#pragma unroll
      for (int u = 0; u < NPW; ++u) {  // rotation of every node this wave will form, loaded up front
        const int qq = wave + u * WAVES;
        pc[u] = ps[u] = 0.f;
        if (qq < nb && lane < HD) {
          const int j = ilist[q0 + qq];
          const int64_t prep = t0 + nst[j] + (nsz[j] - 1) / 2;
          pc[u] = a.rc[prep * HD + lane];
          ps[u] = a.rs[prep * HD + lane];
        }
      }
#pragma unroll
      for (int u = 0; u < NPW; ++u) {
        const int qq = wave + u * WAVES;
        if (qq >= nb) {
          for (int c = lane; c < D; c += 64) {
            if constexpr (sizeof(T) == 2) KHh[qq * KHS + c] = KHl[qq * KHS + c] = 0;
            else KH[qq * KHS + c] = 0.f;
          }
          continue;
        }
        const int j = ilist[q0 + qq];
        const int st = nst[j], sz = nsz[j];
        float s0 = 0.f, s1 = 0.f, kn = 0.f;
        if (lane < HD) {
#pragma unroll 4
          for (int i = st; i < st + sz; ++i) {
            s0 += Kt[(size_t)i * D + lane];
            s1 += Kt[(size_t)i * D + lane + HD];
            kn += knorm[i];
          }
        }
        float nrm2 = group_sum<64>(lane < HD ? s0 * s0 + s1 * s1 : 0.f);
        kn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kn), 0));
        float coh = kn > 0.f ? hw_div(hw_sqrt(nrm2), kn) : 1.f;
        float mu = fmaxf(1.f, (float)sz * coh);
        if (lane == 0) nmu[j] = mu;
        if (lane < HD) {
          const float rsz = __builtin_amdgcn_rcpf((float)sz);
          float m0 = s0 * rsz, m1 = s1 * rsz;
          const float k0 = m0 * pc[u] - m1 * ps[u], k1 = m1 * pc[u] + m0 * ps[u];
          if constexpr (sizeof(T) == 2) {
            // k^ = hi + lo with |k^ - hi - lo| <= 2^-18 |k^|; the queries are exact in bf16
            const uint16_t h0 = f32_to_bf16_hw(k0), h1 = f32_to_bf16_hw(k1);
            KHh[qq * KHS + lane] = h0;
            KHh[qq * KHS + lane + HD] = h1;
            KHl[qq * KHS + lane] = f32_to_bf16_hw(k0 - bf16_bits_to_f32(h0));
            KHl[qq * KHS + lane + HD] = f32_to_bf16_hw(k1 - bf16_bits_to_f32(h1));
          } else {
            KH[qq * KHS + lane] = k0;
            KH[qq * KHS + lane + HD] = k1;
          }
        }
      }
      __syncthreads();
      kvc_f32x16 acc = {};
      if (wave < nrb) {
        const int rho = wave * 32 + (lane & 31);
#pragma unroll
        for (int k0 = 0; k0 < KS; k0 += KS / 2) {
          Frag<T> qf[KS / 2];
#pragma unroll
          for (int u = 0; u < KS / 2; ++u) {
            int c = (k0 + u) * 16 + 8 * (lane >> 5);
            qf[u] = rho < pd ? load_frag<T>(Qu + (int64_t)rho * a.pstride * D + c) : zero_frag<T>();
          }
#pragma unroll
          for (int u = 0; u < KS / 2; ++u) {
            int c = (k0 + u) * 16 + 8 * (lane >> 5);
            if constexpr (sizeof(T) == 2) {
              Frag<uint16_t> hi = load_frag<uint16_t>(KHh + (lane & 31) * KHS + c);
              Frag<uint16_t> lo = load_frag<uint16_t>(KHl + (lane & 31) * KHS + c);
              mma(acc, hi, qf[u]);
              mma(acc, lo, qf[u]);
            } else {
              Frag<T> x = load_frag<T>(KH + (lane & 31) * KHS + c);
              mma(acc, x, qf[u]);
            }
          }
        }
      }
      __syncthreads();  // every read of the prototype keys is done before the logits overwrite them
      if (wave < nrb) {
        const int rho = wave * 32 + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) LG[acc_row(v, lane) * LGS + rho] = acc[v];
      }
      __syncthreads();
      for (int qq = wave; qq < nb; qq += WAVES) {
        const int j = ilist[q0 + qq];
        const int st = nst[j], sz = nsz[j];
        float z = 0.f, zh = 0.f;
        if (lane < pd) {
          #pragma unroll 8
          for (int i = st; i < st + sz; ++i) z += At[i * PA + lane];
          zh = nmu[j] * fast_exp2((LG[qq * LGS + lane] * a.c - lse_s[lane]) * 1.4426950408889634f);
        }
        float eAn = group_sum<64>(fabsf(zh - z)), eAd = group_sum<64>(z);
        if (lane == 0) nD[j] = eAd > 0.f ? hw_div(eAn, eAd) : 0.f;
      }
      __syncthreads();  // the next batch's keys overwrite these logits
    }

    // ---- C: value-aggregate error
    if (nint > 0) {
      const int nt = n32 / 32;
      if constexpr (STAGED) {
        // centred values (zero rows past the slot), re-read in the value-statistics
        // chunk order (an L2 hit; holding them in registers across the error pass
        // costs spills): as two bf16 pieces for bf16 inputs
        // (|v' - hi - lo| <= 2^-18 |v'|), in fp32 otherwise
        static_assert(Lo::N32 == VR * VG, "staging covers the value-statistics chunks");
        uint16_t* Vh = (uint16_t*)Vc;
        uint16_t* Vl = Vh + (size_t)Lo::N32 * Lo::VS;
#pragma unroll
        for (int r = 0; r < VR; ++r) {
          const int i = vg + r * VG;
          float x[8];
          Raw8<T> rl;
          rl.load(Vg + (int64_t)min(i, n - 1) * D + vc);
          rl.get(x);
#pragma unroll
          for (int q = 0; q < 8; ++q) x[q] = i < n ? x[q] - vm[vc + q] : 0.f;
          if constexpr (sizeof(T) == 2) {
            uint16_t hb[8], lb[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              hb[q] = f32_to_bf16_hw(x[q]);
              lb[q] = f32_to_bf16_hw(x[q] - bf16_bits_to_f32(hb[q]));
            }
            *(uint4*)(Vh + i * Lo::VS + vc) = make_uint4(hb[0] | (uint32_t)hb[1] << 16, hb[2] | (uint32_t)hb[3] << 16,
                                                          hb[4] | (uint32_t)hb[5] << 16, hb[6] | (uint32_t)hb[7] << 16);
            *(uint4*)(Vl + i * Lo::VS + vc) = make_uint4(lb[0] | (uint32_t)lb[1] << 16, lb[2] | (uint32_t)lb[3] << 16,
                                                          lb[4] | (uint32_t)lb[5] << 16, lb[6] | (uint32_t)lb[7] << 16);
          } else {
            float* d0 = Vc + i * Lo::VS + vc;
            *(float4*)d0 = make_float4(x[0], x[1], x[2], x[3]);
            *(float4*)(d0 + 4) = make_float4(x[4], x[5], x[6], x[7]);
          }
        }
        __syncthreads();
        // at most three tiles (slots of at most 64 tokens): one per wave, written
        // once every wave has read the staged values (midpoint trees keep the
        // Gram matrix over them)
        static_assert(Lo::N32 <= 64 && WAVES >= 3, "one Gram tile per wave");
        const int ti = wave >= nt ? 1 : 0, tj = wave >= nt ? 1 : wave;
        kvc_f32x16 acc = {};
        if (wave < nt * (nt + 1) / 2) {
          const int oa = (ti * 32 + (lane & 31)) * Lo::VS + 8 * (lane >> 5);
          const int ob = (tj * 32 + (lane & 31)) * Lo::VS + 8 * (lane >> 5);
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              const Frag<uint16_t> ha = load_frag<uint16_t>(Vh + oa + ks * 16), la = load_frag<uint16_t>(Vl + oa + ks * 16);
              const Frag<uint16_t> hb = load_frag<uint16_t>(Vh + ob + ks * 16), lb = load_frag<uint16_t>(Vl + ob + ks * 16);
              mma(acc, ha, hb);
              mma(acc, ha, lb);
              mma(acc, la, hb);
              mma(acc, la, lb);
            }
          } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) mma(acc, load_frag<float>(Vc + oa + ks * 16), load_frag<float>(Vc + ob + ks * 16));
          }
        }
        if (Lo::LGKEEP && !a.topo) __syncthreads();
        if (wave < nt * (nt + 1) / 2) {
          float* Gd = (Lo::LGKEEP && !a.topo) ? (float*)(smem + Lo::r1) : Gm;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = ti * 32 + acc_row(v, lane), cc = tj * 32 + (lane & 31);
            Gd[r * NG + cc] = acc[v];
            if (ti != tj) Gd[cc * NG + r] = acc[v];
          }
        }
      } else
      for (int tile = wave; tile < nt * (nt + 1) / 2; tile += WAVES) {
        int ti = 0, rem = tile;
        while (rem >= nt - ti) {
          rem -= nt - ti;
          ++ti;
        }
        const int tj = ti + rem;
        const int ra = ti * 32 + (lane & 31), rb = tj * 32 + (lane & 31);
        kvc_f32x16 acc = {};
#pragma unroll
        for (int k0 = 0; k0 < KS; k0 += KS / 2) {  // half the steps' loads in flight at a time
        Raw8<T> xa[KS / 2], xb[KS / 2];
#pragma unroll
        for (int u = 0; u < KS / 2; ++u) {
          const int c = (k0 + u) * 16 + 8 * (lane >> 5);
          if (ra < n) xa[u].load(Vg + (int64_t)ra * D + c);
          else xa[u].zero();
          if (rb < n) xb[u].load(Vg + (int64_t)rb * D + c);
          else xb[u].zero();
        }
#pragma unroll
        for (int u = 0; u < KS / 2; ++u) {
          const int c = (k0 + u) * 16 + 8 * (lane >> 5);
          float ya[8], yb[8];
          xa[u].get(ya);
          xb[u].get(yb);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            ya[q] = ra < n ? ya[q] - vm[c + q] : 0.f;
            yb[q] = rb < n ? yb[q] - vm[c + q] : 0.f;
          }
          if constexpr (sizeof(T) == 2) {
            Frag<uint16_t> ha, la, hb, lb;
            split8(ya, ha.v, la.v);
            split8(yb, hb.v, lb.v);
            mma(acc, ha, hb);
            mma(acc, ha, lb);
            mma(acc, la, hb);
            mma(acc, la, lb);
          } else {
            Frag<float> fa, fb;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              fa.v[q] = ya[q];
              fb.v[q] = yb[q];
            }
            mma(acc, fa, fb);
          }
        }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = ti * 32 + acc_row(v, lane), cc = tj * 32 + (lane & 31);
          Gm[r * NG + cc] = acc[v];
          if (ti != tj) Gm[cc * NG + r] = acc[v];
        }
      }
      if (STAGED && !a.topo) {
        // Midpoint trees of at most 64 tokens. Nodes of at most 16 tokens take
        // one wave each and evaluate c^T G c and a^T G a directly. The larger
        // ones (the root and its children) are assembled from their children:
        // a^T G a = sum over children + 2 x (pairs across children), the cross
        // pairs spread over every wave in aligned 4-row groups; with w the
        // node's value weights, c^T G c = a^T G a - 2 Z a^T G w + Z^2 w^T G w.
        __syncthreads();  // the Gram matrix is complete; the staged values are free
        const float* G2 = Lo::LGKEEP ? (const float*)(smem + Lo::r1) : Gm;
        const float* LGa = (const float*)(smem + Lo::kh);  // [64][LGS] prototype logits (when kept)
        constexpr int SMALLN = 16;
        float* mpart = (float*)(smem + Lo::r1 + Lo::mp_part);  // [MP_ITEMS][PDMAX]
        float* mq = (float*)(smem + Lo::r1 + Lo::mp_q);         // [3: a^T G a, Z, a.s][6 slots][PDMAX]
        float* mgv = (float*)(smem + Lo::r1 + Lo::mp_gv);       // [3: root, L, R][NMAX]
        float* mww = (float*)(smem + Lo::r1 + Lo::mp_w);        // [3] w^T G w
        float* mrq = (float*)(smem + Lo::r1 + Lo::mp_rq);       // [4][PDMAX]
        const float mm = misc[0];
        const int nl = (n + 1) >> 1, nr = n - nl;
        const int nll = (nl + 1) >> 1, nrl = (nr + 1) >> 1;
        const int jR = 2 * nl;
        const bool bigT = n > SMALLN, bigL = nl > SMALLN, bigR = nr > SMALLN;
        // cross items: root (rows [0, nl) x columns [nl, n)), L (rows [0, nll) x
        // [nll, nl)), R (rows [nl, nl + nrl) x [nl + nrl, n)), in 4-row groups
        const int K0 = bigT ? (nl + 3) >> 2 : 0;
        const int K1 = bigL ? (nll + 3) >> 2 : 0;
        const int g2 = nl >> 2;
        const int K2 = bigR ? ((nl + nrl + 3) >> 2) - g2 : 0;
        // slot of a node whose (a^T G a, Z, a.s) a big parent reads
        auto slot_of = [&](int j) {
          if (bigT && j == 1) return 0;
          if (bigT && j == jR) return 1;
          if (bigL && j == 2) return 2;
          if (bigL && j == 1 + 2 * nll) return 3;
          if (bigR && j == jR + 1) return 4;
          if (bigR && j == jR + 2 * nrl) return 5;
          return -1;
        };
        auto weights = [&](int j, int sz, float& al, float& ga) {
          const float rl = nrel[j];
          al = rl > 0.f ? hw_div(1.f - a.beta, rl) : 0.f;
          ga = hw_div(rl > 0.f ? a.beta : 1.f, (float)sz);
        };
        // D = min(1, wA eA + wV eV); with the logits kept, eA is formed here from
        // the node's Z (the four sums over the distortion rows in one reduction)
        auto finish = [&](int j, float Z, float num, float den) {
          const float sn = lane < pd ? hw_sqrt(fmaxf(num, 0.f)) : 0.f, sd = lane < pd ? hw_sqrt(fmaxf(den, 0.f)) : 0.f;
          float eA;
          float4 r;
          if constexpr (Lo::LGKEEP) {
            float an = 0.f, ad = 0.f;
            if (lane < pd) {
              const float zh = nmu[j] * fast_exp2((LGa[(j - nst[j]) * LGS + lane] * a.c - lse_s[lane]) * 1.4426950408889634f);
              an = fabsf(zh - Z);
              ad = Z;
            }
            r = wave_sum4(sn, sd, an, ad);
            eA = r.w > 0.f ? hw_div(r.z, r.w) : 0.f;
          } else {
            r = wave_sum4(sn, sd, 0.f, 0.f);
            eA = nD[j];
          }
          if (lane == 0) {
            const float eV = r.y > 0.f ? hw_div(r.x, r.y) : 0.f;
            nD[j] = fminf(1.f, a.wA * eA + a.wV * eV);
          }
        };
        // cross items, dealt to the waves in order
        for (int k = wave; k < K0 + K1 + K2; k += WAVES) {
          float x;
          if (k < K0) x = cross_block(G2, NG, At, lane, k, 0, nl, nl, n);
          else if (k < K0 + K1) x = cross_block(G2, NG, At, lane, k - K0, 0, nll, nll, nl);
          else x = cross_block(G2, NG, At, lane, g2 + (k - K0 - K1), nl, nl + nrl, nl + nrl, n);
          mpart[k * PDMAX + lane] = x;
        }
        // G w of the big nodes (lane = token), and w^T G w
        if (wave == WAVES - 2 && bigT) {
          float al, ga;
          weights(0, n, al, ga);
          float gv = 0.f;
          if (lane < n) {
#pragma unroll 4
            for (int j = 0; j < n; ++j) gv = fmaf(G2[j * NG + lane], fmaf(al, rtok[j], ga), gv);
            mgv[lane] = gv;
          }
          const float ww = group_sum<64>(lane < n ? fmaf(al, rtok[lane], ga) * gv : 0.f);
          if (lane == 0) mww[0] = ww;
        }
        if (wave == WAVES - 1 && (bigL || bigR)) {
          const bool inL = lane < nl;
          float alL, gaL, alR, gaR;
          weights(1, nl, alL, gaL);
          weights(jR, nr, alR, gaR);
          const float al = inL ? alL : alR, ga = inL ? gaL : gaR;
          const int vst = inL ? 0 : nl, vn = inL ? nl : nr;
          float gv = 0.f;
          if (lane < n) {
            for (int j = 0; j < vn; ++j) gv = fmaf(G2[(vst + j) * NG + lane], fmaf(al, rtok[vst + j], ga), gv);
            mgv[(inL ? 1 : 2) * NMAX + lane] = gv;
          }
          const float wg = lane < n ? fmaf(al, rtok[lane], ga) * gv : 0.f;
          const float wwL = group_sum<64>(inL ? wg : 0.f), wwR = group_sum<64>(inL ? 0.f : wg);
          if (lane == 0) {
            mww[1] = wwL;
            mww[2] = wwR;
          }
        }
        // nodes of at most 16 tokens, one wave each
        for (int q = wave; q < nint; q += WAVES) {
          const int j = ilist[q];
          const int st = nst[j], sz = nsz[j];
          if (sz > SMALLN) continue;
          float al, ga;
          weights(j, sz, al, ga);
          float Z, as, num, qa;
          if (sz <= 2) small_forms<2>(G2, NG, At, rtok, sdot, lane, st, sz, n32, al, ga, Z, as, num, qa);
          else if (sz <= 4) small_forms<4>(G2, NG, At, rtok, sdot, lane, st, sz, n32, al, ga, Z, as, num, qa);
          else if (sz <= 8) small_forms<8>(G2, NG, At, rtok, sdot, lane, st, sz, n32, al, ga, Z, as, num, qa);
          else small_forms<16>(G2, NG, At, rtok, sdot, lane, st, sz, n32, al, ga, Z, as, num, qa);
          const int sl = slot_of(j);
          if (sl >= 0) {
            mq[(0 * 6 + sl) * PDMAX + lane] = qa;
            mq[(1 * 6 + sl) * PDMAX + lane] = Z;
            mq[(2 * 6 + sl) * PDMAX + lane] = as;
          }
          finish(j, Z, num, fmaf(2.f * Z, as, fmaf(Z * Z, mm, qa)));
        }
        __syncthreads();
        // big children of the root, from their children; the root's a^T G w in quarters
        auto big_node = [&](int j, int vst, int sz, int k0, int k1, int c0, int gvs, float qaw) {
          float x = 0.f;
          for (int k = k0; k < k1; ++k) x += mpart[k * PDMAX + lane];
          const float qa = mq[(0 * 6 + c0) * PDMAX + lane] + mq[(0 * 6 + c0 + 1) * PDMAX + lane] + 2.f * x;
          const float Z = mq[(1 * 6 + c0) * PDMAX + lane] + mq[(1 * 6 + c0 + 1) * PDMAX + lane];
          const float as = mq[(2 * 6 + c0) * PDMAX + lane] + mq[(2 * 6 + c0 + 1) * PDMAX + lane];
          if (gvs > 0) {  // a^T G w over the node's tokens (gvs 1, 2: L, R)
            qaw = 0.f;
#pragma unroll 4
            for (int i = vst; i < vst + sz; ++i) qaw = fmaf(At[i * PA + lane], mgv[gvs * NMAX + i], qaw);
          }
          const float num = fmaf(Z * Z, mww[gvs], fmaf(-2.f * Z, qaw, qa));
          finish(j, Z, num, fmaf(2.f * Z, as, fmaf(Z * Z, mm, qa)));
          return make_float3(qa, Z, as);
        };
        if (wave == 0 && bigL) {
          const float3 r = big_node(1, 0, nl, K0, K0 + K1, 2, 1, 0.f);
          mq[(0 * 6 + 0) * PDMAX + lane] = r.x;
          mq[(1 * 6 + 0) * PDMAX + lane] = r.y;
          mq[(2 * 6 + 0) * PDMAX + lane] = r.z;
        }
        if (wave == 1 && bigR) {
          const float3 r = big_node(jR, nl, nr, K0 + K1, K0 + K1 + K2, 4, 2, 0.f);
          mq[(0 * 6 + 1) * PDMAX + lane] = r.x;
          mq[(1 * 6 + 1) * PDMAX + lane] = r.y;
          mq[(2 * 6 + 1) * PDMAX + lane] = r.z;
        }
        if (wave >= 2 && wave < 6 && bigT) {
          const int i0 = (wave - 2) * 16, i1 = min(i0 + 16, n);
          float p = 0.f;
          for (int i = i0; i < i1; ++i) p = fmaf(At[i * PA + lane], mgv[i], p);
          mrq[(wave - 2) * PDMAX + lane] = p;
        }
        __syncthreads();
        if (wave == 0 && bigT) {
          const float qaw = mrq[lane] + mrq[PDMAX + lane] + mrq[2 * PDMAX + lane] + mrq[3 * PDMAX + lane];
          big_node(0, 0, n, 0, K0, 0, 0, qaw);  // the root's a^T G w is summed from the quarters
        }
        __syncthreads();
      } else {
      // the root (c = 0) and its first and last children (c = 1, 2) are shared by
      // every wave; a three-way root's middle child is a single token
      const int rlast = a.topo ? imisc[2] : 2 * ((n + 1) >> 1);
      auto coop_j = [&](int c) { return c == 0 ? 0 : (c == 1 ? 1 : rlast); };
      auto coop_ok = [&](int c) { return nsz[coop_j(c)] >= 2; };
      if (wave < 3 && coop_ok(wave)) {
        const int j = coop_j(wave);
        const int st = nst[j], sz = nsz[j];
        float z = 0.f, as = 0.f;
        #pragma unroll 8
        for (int i = st; i < st + sz; ++i) {
          float av = At[i * PA + lane];
          z += av;
          as = fmaf(av, sdot[i], as);
        }
        zc[(wave * 2) * PDMAX + lane] = z;
        zc[(wave * 2 + 1) * PDMAX + lane] = as;
      }
      __syncthreads();
      {
        float pn[3] = {0.f, 0.f, 0.f}, pq[3] = {0.f, 0.f, 0.f};
        int item = 0;
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          if (!coop_ok(c)) continue;
          const int j = coop_j(c);
          const int st = nst[j], sz = nsz[j];
          const float Z = zc[(c * 2) * PDMAX + lane];
          const float rl = nrel[j];
          const float al = rl > 0.f ? hw_div(1.f - a.beta, rl) : 0.f;
          const float ga = hw_div(rl > 0.f ? a.beta : 1.f, (float)sz);
          const int b0 = st >> 3, b1 = (st + sz + 7) >> 3;
          for (int b = b0; b < b1; ++b, ++item)
            if (item % WAVES == wave) qform_block(Gm, NG, At, rtok, lane, b * 8, st, sz, Z, al, ga, pn[c], pq[c]);
        }
#pragma unroll
        for (int c = 0; c < 3; ++c) {
          part[((wave * 3 + c) * 2) * PDMAX + lane] = pn[c];
          part[((wave * 3 + c) * 2 + 1) * PDMAX + lane] = pq[c];
        }
      }
      __syncthreads();
      const float mm = misc[0];
      for (int q = wave; q < nint; q += WAVES) {
        const int j = ilist[q];
        const int st = nst[j], sz = nsz[j];
        float num = 0.f, den = 0.f, Z, as;
        if (ndep[j] <= 1) {
          const int c = j == 0 ? 0 : (j == 1 ? 1 : 2);
#pragma unroll
          for (int w2 = 0; w2 < WAVES; ++w2) {
            num += part[((w2 * 3 + c) * 2) * PDMAX + lane];
            den += part[((w2 * 3 + c) * 2 + 1) * PDMAX + lane];
          }
          Z = zc[(c * 2) * PDMAX + lane];
          as = zc[(c * 2 + 1) * PDMAX + lane];
        } else {
          Z = 0.f;
          as = 0.f;
          #pragma unroll 8
          for (int i = st; i < st + sz; ++i) {
            float av = At[i * PA + lane];
            Z += av;
            as = fmaf(av, sdot[i], as);
          }
          const float rl = nrel[j];
          const float al = rl > 0.f ? hw_div(1.f - a.beta, rl) : 0.f;
          const float ga = hw_div(rl > 0.f ? a.beta : 1.f, (float)sz);
          for (int b = st >> 3; b < (st + sz + 7) >> 3; ++b)
            qform_block(Gm, NG, At, rtok, lane, b * 8, st, sz, Z, al, ga, num, den);
        }
        den = den + 2.f * Z * as + Z * Z * mm;
        float eVn = group_sum<64>(lane < pd ? hw_sqrt(fmaxf(num, 0.f)) : 0.f);
        float eVd = group_sum<64>(lane < pd ? hw_sqrt(fmaxf(den, 0.f)) : 0.f);
        if (lane == 0) {
          float eA = nD[j];
          float eV = eVd > 0.f ? hw_div(eVn, eVd) : 0.f;
          nD[j] = fminf(1.f, a.wA * eA + a.wV * eV);
        }
      }
      __syncthreads();
      }
    }
    // ---- outputs: node arrays and op utilities
    const float sens = a.sens[unit];
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
        const int j = q - 1;
        if (a.topo) {  // children: j+1, then the sibling chain; cost = children - 1
          int c = j + 1, k = 1;
          float sub = nrel[c] * nD[c];
          for (c = nsib[c]; c != 0; c = nsib[c], ++k) sub += nrel[c] * nD[c];
          u = sens * (nrel[j] * nD[j] - sub) / (float)(k - 1);
          cst = (uint8_t)(k - 1);
        } else {
          const int lc = j + 1, rc = j + 2 * ((nsz[j] + 1) >> 1);
          u = sens * (nrel[j] * nD[j] - (nrel[lc] * nD[lc] + nrel[rc] * nD[rc]));
          cst = 1;
        }
      }
      a.op_util[obase + q] = u;
      a.op_cost[obase + q] = cst;
    }
    __syncthreads();
  }
}

// Split each sequence's slots into two size classes (ids in slot order).
__global__ __launch_bounds__(1024) void tree_bucket_kernel(const int32_t* slot_start, const int32_t* n_slots,
                                                           int stride, int split, int2* lists,
                                                           int32_t* counts, int S) {
  __shared__ int wtot[2][16];
  __shared__ int base[2];
  const int s = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = n_slots[s];
  const int32_t* ss = slot_start + (int64_t)s * (stride + 1);
  if (tid < 2) base[tid] = 0;
  __syncthreads();
  for (int k0 = 0; k0 < ns; k0 += 1024) {
    const int k = k0 + tid;
    const bool valid = k < ns;
    const int len = valid ? ss[k + 1] - ss[k] : 0;
    const bool big = len > split;
    uint64_t m[2] = {__ballot(valid && !big), __ballot(valid && big)};
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (lane == 0) {
      wtot[0][wave] = __popcll(m[0]);
      wtot[1][wave] = __popcll(m[1]);
    }
    __syncthreads();
    if (valid) {
      const int b = big ? 1 : 0;
      int off = base[b];
      for (int w2 = 0; w2 < wave; ++w2) off += wtot[b][w2];
      off += __popcll(m[b] & below);
      lists[((int64_t)b * S + s) * stride + off] = make_int2(ss[k], len);
    }
    __syncthreads();
    if (tid < 2) {
      int t = 0;
      for (int w2 = 0; w2 < 16; ++w2) t += wtot[tid][w2];
      base[tid] += t;
    }
    if (tid < 32) wtot[tid >> 4][tid & 15] = 0;
    __syncthreads();
  }
  if (tid < 2) counts[tid * S + s] = base[tid];
}

// ------------------------------------------------------------------ explicit tree shapes
// GraceKV page, 'Technical details and default settings': high-curvature
// split candidates beside the midpoint, a salient token isolated in a
// three-way child set. One thread builds one slot's tree depth-first (node j
// numbered when popped, so in pre-order) with its stack in LDS, and writes
// the node records; a record's next-sibling field is known once that sibling
// is numbered, so a node with a later sibling hands its record to the
// sibling's stack entry, which writes it. Children are at most n - ceil(n/4)
// tokens (or n - 1 - max(floor(n/4), 1) for a three-way split's sides), so a
// 128-token slot is at most 14 internal levels deep and at most 2 later
// siblings wait per level: 32 stack entries suffice.
constexpr int TOPO_THREADS = 64;
constexpr int TOPO_STACK = 32;

struct TopoArgs {
  const float* rel;        // [Ly][H][T]
  const int64_t* cut;      // [T] partition cut scores or NULL
  const int32_t* slot_start;
  const int32_t* n_slots;
  const int64_t* cu;
  uint32_t* topo;          // [Ly][H][2T]
  int S, stride, mode;
  int64_t T, items;        // items = Ly*H*S*stride
};

// children of the node [st, st+n) (sequence positions; n >= 2): returns 2 or 3
__device__ int topo_children(const float* r, const int64_t* cut, int mode, int st, int n, int* ca, int* cn) {
  int b = (n + 1) >> 1;
  if (mode == 1) {
    if (n >= 3) {
      int i = 0;
      float rmax = r[st];
      double S = 0.0;
      for (int k = 0; k < n; ++k) {   // left to right: the order the decision is defined in
        const float v = r[st + k];
        S += (double)v;
        if (v > rmax) {
          rmax = v;
          i = k;
        }
      }
      const int q = max(n >> 2, 1);
      if (S > 0.0 && 2.0 * (double)rmax > S && i >= q && i <= n - 1 - q) {
        ca[0] = st, cn[0] = i;
        ca[1] = st + i, cn[1] = 1;
        ca[2] = st + i + 1, cn[2] = n - i - 1;
        return 3;
      }
    }
    if (cut) {
      const int m4 = (n + 3) >> 2;
      const int lo = max(1, m4), hi = min(n - 1, n - m4);
      int best = b;
      int64_t bv = cut[st + b];
      for (int c = lo; c <= hi; ++c) {
        const int64_t v = cut[st + c];
        const int dc = abs(c - b), db = abs(best - b);
        if (v > bv || (v == bv && (dc < db || (dc == db && c < best)))) {
          best = c;
          bv = v;
        }
      }
      b = best;
    }
  }
  ca[0] = st, cn[0] = b;
  ca[1] = st + b, cn[1] = n - b;
  return 2;
}

__global__ __launch_bounds__(TOPO_THREADS) void tree_topo_kernel(TopoArgs a) {
  __shared__ uint2 stk[TOPO_STACK][TOPO_THREADS];   // x: entry, y: the previous sibling's record + index
  const int tid = threadIdx.x;
  const int64_t i = (int64_t)blockIdx.x * TOPO_THREADS + tid;
  if (i >= a.items) return;
  const int k = (int)(i % a.stride);
  const int64_t rest = i / a.stride;
  const int s = (int)(rest % a.S);
  const int64_t lh = rest / a.S;
  if (k >= a.n_slots[s]) return;
  const int32_t* ss = a.slot_start + (int64_t)s * (a.stride + 1);
  const int t0 = ss[k], n = ss[k + 1] - ss[k];
  if (n <= 0) return;
  const float* r = a.rel + lh * a.T + a.cu[s];               // sequence positions
  const int64_t* cut = a.cut ? a.cut + a.cu[s] : nullptr;
  uint32_t* rec = a.topo + lh * 2 * a.T + 2 * (a.cu[s] + t0);
  // entry x: bits 0-7 start - t0, 8-15 length - 1, 16-23 parent + 1, 24 has a
  // later sibling, 25 y holds the previous sibling's record
  int top = 0, m = 0;
  stk[top++][tid] = make_uint2((uint32_t)(n - 1) << 8, 0u);
  while (top > 0) {
    const uint2 e = stk[--top][tid];
    const int j = m++;
    if (e.x & (1u << 25)) rec[e.y >> 24] = (e.y & 0xFFFFFFu) | ((uint32_t)j << 24);
    const uint32_t low = e.x & 0xFFFFFFu;
    if (e.x & (1u << 24)) {
      uint2 nx = stk[top - 1][tid];
      nx.x |= 1u << 25;
      nx.y = low | ((uint32_t)j << 24);
      stk[top - 1][tid] = nx;
    } else {
      rec[j] = low;
    }
    const int st = (int)(e.x & 255), len = (int)((e.x >> 8) & 255) + 1;
    if (len > 1) {
      int ca[3], cn[3];
      const int nc = topo_children(r, cut, a.mode, t0 + st, len, ca, cn);
      for (int c = nc - 1; c >= 0 && top < TOPO_STACK; --c)
        stk[top++][tid] = make_uint2((uint32_t)(ca[c] - t0) | ((uint32_t)(cn[c] - 1) << 8) |
                                         ((uint32_t)(j + 1) << 16) | (c < nc - 1 ? 1u << 24 : 0u),
                                     0u);
    }
  }
  for (int j = m; j < 2 * n; ++j) rec[j] = 0xFFFFFFFFu;
}

int slot_nmax(const kvc_params* p) { return p->slot_len > 0 ? p->slot_len : p->slot_max; }

template <class T, int D, int NMAX, int WAVES, int OCC>
int launch_trees(const TreeKArgs& a, int64_t bound, int ncu, hipStream_t st) {
  using Lo = TreeLayout<NMAX, D, WAVES>;
  static_assert(Lo::total <= 160 * 1024, "tree LDS");
  auto kfn = tree_kernel<T, D, NMAX, WAVES, OCC>;
  (void)hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lo::total);
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kfn, WAVES * 64, Lo::total) != hipSuccess || per < 1) per = 1;
  int64_t grid = (int64_t)ncu * per;
  if (grid > bound) grid = bound;
  if (grid < 1) return KVC_OK;
  hipLaunchKernelGGL(kfn, dim3((unsigned)grid), dim3(WAVES * 64), Lo::total, st, a);
  KVC_LAUNCH_CHECK("tree_build");
  return KVC_OK;
}

template <class T, int D>
int launch_both(TreeKArgs a, int2* lists, int32_t* counts, int64_t bound, int nmax, int ncu, hipStream_t st) {
  a.list = lists;
  a.count = counts;
  // small slots: two 8-wave workgroups per CU (4 waves per SIMD); large: one.
  // Midpoint trees of bf16 slots with head dimension 128 take the kernel on
  // the fixed 64-position layout.
  int r;
  if constexpr (sizeof(T) == 2 && D == 128)
    r = a.topo == nullptr ? launch_trees_v(a, bound, ncu, st) : launch_trees<T, D, SMALL, 8, 4>(a, bound, ncu, st);
  else
    r = launch_trees<T, D, SMALL, 8, 4>(a, bound, ncu, st);
  if (r || nmax <= SMALL) return r;
  a.list = lists + (int64_t)a.S * a.stride;
  a.count = counts + a.S;
  return launch_trees<T, D, 128, 8, 2>(a, bound, ncu, st);
}

}  // namespace

namespace kvc {
// size-class lists [2][S][stride] of (start, length) and their counts [2][S] int32
size_t ws_trees(const kvc_shape* sh, const kvc_params* p) {
  if (p->token_mode) return 0;
  int64_t stride = kvc_slot_stride(sh, p);
  if (stride < 0) return 0;
  Carver c(nullptr, 0);
  c.take<int2>((size_t)2 * sh->n_seq * stride);
  c.take<int32_t>((size_t)2 * sh->n_seq);
  return c.off;
}
}  // namespace kvc

extern "C" int kvc_build_trees(const kvc_shape* sh, const kvc_params* p, const void* K, const void* V,
                               const void* Qprobe, const float* probe_lse, const float* rel, const float* head_sens,
                               const float* rope_cos, const float* rope_sin, const int32_t* slot_start,
                               const int32_t* n_slots, kvc_trees* out, void* ws, size_t ws_bytes,
                               hipStream_t st) {
  return kvc_build_trees_ex(sh, p, K, V, Qprobe, probe_lse, rel, head_sens, rope_cos, rope_sin, slot_start, n_slots,
                            nullptr, out, ws, ws_bytes, st);
}

extern "C" int kvc_build_trees_ex(const kvc_shape* sh, const kvc_params* p, const void* K, const void* V,
                                  const void* Qprobe, const float* probe_lse, const float* rel,
                                  const float* head_sens, const float* rope_cos, const float* rope_sin,
                                  const int32_t* slot_start, const int32_t* n_slots, const int64_t* dp_cut_q,
                                  kvc_trees* out, void* ws, size_t ws_bytes, hipStream_t st) {
  int r = kvc::validate_shape(sh);
  if (r) return r;
  if ((r = kvc::validate_params(sh, p))) return r;
  KVC_REQUIRE(!p->token_mode, KVC_E_INVAL, "kvc_build_trees: token mode has no trees");
  KVC_REQUIRE(K && V && Qprobe && probe_lse && rel && head_sens && rope_cos && rope_sin && slot_start && n_slots &&
                  out && out->node_rel && out->node_D && out->node_mu && out->op_util && out->op_cost,
              KVC_E_INVAL, "kvc_build_trees: NULL pointer");
  KVC_REQUIRE(p->split_mode == 0 || out->node_topo, KVC_E_INVAL,
              "kvc_build_trees: split_mode 1 needs out->node_topo");
  const int d = sh->head_dim;
  KVC_REQUIRE(d == 64 || d == 128, KVC_E_UNSUPPORTED, "kvc_build_trees: head_dim must be 64 or 128");
  const size_t need = kvc::ws_trees(sh, p);
  KVC_REQUIRE(ws && ws_bytes >= need, KVC_E_WORKSPACE, "kvc_build_trees: workspace too small");
  KVC_REQUIRE(sh->n_seq <= MAX_SEQ, KVC_E_UNSUPPORTED, "kvc_build_trees: at most 256 sequences per call");
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
  a.cu = sh->cu_seqlens_d;
  a.S = sh->n_seq;
  a.Ly = sh->n_layers;
  a.H = sh->n_kv_heads;
  a.G = sh->group;
  a.P = p->n_probe;
  a.stride = kvc_slot_stride(sh, p);
  int R = sh->group * p->n_probe;
  a.pd = p->n_dprobe < R ? p->n_dprobe : R;
  a.pstride = R / a.pd;
  a.T = sh->total_tokens;
  a.c = 1.0f / sqrtf((float)d);
  a.beta = p->value_base;
  a.wA = p->w_attn;
  a.wV = p->w_value;
  a.node_rel = out->node_rel;
  a.node_D = out->node_D;
  a.node_mu = out->node_mu;
  a.op_util = out->op_util;
  a.op_cost = out->op_cost;
  a.topo = p->split_mode == 1 ? out->node_topo : nullptr;
  const int64_t bound = (int64_t)sh->n_layers * sh->n_kv_heads * sh->n_seq * a.stride;  // slot count bound
  if (bound == 0) return KVC_OK;
  if (out->node_topo) {
    TopoArgs ta{};
    ta.rel = rel;
    ta.cut = p->split_mode == 1 ? dp_cut_q : nullptr;
    ta.slot_start = slot_start;
    ta.n_slots = n_slots;
    ta.cu = sh->cu_seqlens_d;
    ta.topo = out->node_topo;
    ta.S = sh->n_seq;
    ta.stride = a.stride;
    ta.mode = p->split_mode;
    ta.T = sh->total_tokens;
    ta.items = bound;
    hipLaunchKernelGGL(tree_topo_kernel, dim3((unsigned)((bound + TOPO_THREADS - 1) / TOPO_THREADS)),
                       dim3(TOPO_THREADS), 0, st, ta);
    KVC_LAUNCH_CHECK("tree_topo");
  }
  kvc::Carver cv(ws, ws_bytes);
  int2* lists = cv.take<int2>((size_t)2 * a.S * a.stride);
  int32_t* counts = cv.take<int32_t>((size_t)2 * a.S);
  hipLaunchKernelGGL(tree_bucket_kernel, dim3((unsigned)a.S), dim3(1024), 0, st, slot_start, n_slots, a.stride,
                     SMALL, lists, counts, a.S);
  KVC_LAUNCH_CHECK("tree_bucket");
  int dev = 0, ncu = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) ncu = 256;
  const int nmax = slot_nmax(p);
  if (sh->dtype == KVC_BF16)
    return d == 128 ? launch_both<uint16_t, 128>(a, lists, counts, bound, nmax, ncu, st)
                    : launch_both<uint16_t, 64>(a, lists, counts, bound, nmax, ncu, st);
  return d == 128 ? launch_both<float, 128>(a, lists, counts, bound, nmax, ncu, st)
                  : launch_both<float, 64>(a, lists, counts, bound, nmax, ncu, st);
}
