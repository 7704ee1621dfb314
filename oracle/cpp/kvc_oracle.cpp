// kvc_oracle -- plain CPU oracle of the KV-cache compression path (C++17,
// OpenMP over units, fp64). TEST INFRASTRUCTURE ONLY: see kvc_oracle.h.
//
// Each function restates one stage of the path in the order and notation of
// the pages, with the readings the Python oracle states where the pages are
// silent (probe rows see every cached key; relevance is the probe mass summed
// over probes and query heads; propagation follows the seeds' causal prefill
// attention rows; binary midpoint trees, or with split_mode 1 curvature-
// candidate cuts and salient three-way splits; mu = max(1, n rho); distortion over
// strided probe rows at 0.25 : 0.75; gains as the decrease of the frontier
// loss; capped best-first auction; ln mu as a decode logit bias). Sums use
// `omp simd` reductions, so only their rounding order differs from a
// left-to-right sum.
#include "kvc_oracle.h"

#include <omp.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>
#include <queue>
#include <vector>

namespace {

using std::vector;

// ------------------------------------------------------------------ scalars
double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}
double elem(const void* p, int dtype, int64_t i) {
  if (dtype == 1) return bf16_to_double(((const uint16_t*)p)[i]);
  return (double)((const float*)p)[i];
}
// fp64 -> fp32 (nearest even) -> bf16 (nearest even): the two roundings a
// value takes when an fp64 result is stored in a bf16 tensor through fp32
uint16_t double_to_bf16(double x) {
  float f = (float)x;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
void store(void* p, int dtype, int64_t i, double x) {
  if (dtype == 1)
    ((uint16_t*)p)[i] = double_to_bf16(x);
  else
    ((float*)p)[i] = (float)x;
}
// fp32 ranking key: NaN ranks below everything
double rank_key(float v) { return v != v ? -std::numeric_limits<double>::infinity() : (double)v; }

double dot(const double* a, const double* b, int n) {
  double s = 0.0;
#pragma omp simd reduction(+ : s)
  for (int k = 0; k < n; ++k) s += a[k] * b[k];
  return s;
}

// rows [first, first + n) of a [.][d] array in `dtype`, as fp64
void rows(const void* p, int dtype, int64_t first, int64_t n, int d, vector<double>& out) {
  out.resize((size_t)(n * d));
  for (int64_t i = 0; i < n * d; ++i) out[(size_t)i] = elem(p, dtype, first * d + i);
}

// Progress lines on stderr for long stages (one every 30 s at most).
struct Progress {
  const char* what;
  int64_t total;
  std::atomic<int64_t> done{0};
  std::chrono::steady_clock::time_point t0 = std::chrono::steady_clock::now(), last = t0;
  Progress(const char* w, int64_t n) : what(w), total(n) {}
  void tick() {
    const int64_t k = ++done;
    if (omp_get_thread_num() != 0) return;
    auto now = std::chrono::steady_clock::now();
    if (std::chrono::duration<double>(now - last).count() > 30.0) {
      last = now;
      std::fprintf(stderr, "[oracle] %s: %lld/%lld units, %.0f s\n", what, (long long)k, (long long)total,
                   std::chrono::duration<double>(now - t0).count());
      std::fflush(stderr);
    }
  }
};

// ------------------------------------------------------------------ regions, budgets
struct Reg {
  int64_t pe, c0, c1, ss;
};
// GraceKV page, 'Core idea' / 'Exact-information safeguard': the prompt and
// the suffix stay exact outside the budget, a recent window before the suffix
// stays exact inside it; short sequences give up the prompt last, then the
// suffix, then the recent window.
Reg regions_of(int64_t L, const ko_params* p) {
  Reg r;
  r.pe = std::min<int64_t>(p->prompt_exact, L);
  r.ss = std::max<int64_t>(r.pe, L - p->suffix_exact);
  r.c1 = std::max<int64_t>(r.pe, r.ss - p->recent_exact);
  r.c0 = r.pe;
  return r;
}

// DistillCache, Algorithm 1: B = max(floor(r |C|), B_min), |C| = L Ly H (one
// budget per sequence over all its entries); the recent window is charged
// first; the floor may spend floor(phi * allocatable).
void budgets_of(const ko_shape* sh, const ko_params* p, int s, int64_t* B, int64_t* alloc, int64_t* F) {
  const int64_t L = sh->cu[s + 1] - sh->cu[s];
  const int64_t U = (int64_t)sh->Ly * sh->H;
  int64_t b = (int64_t)std::floor((double)p->budget_ratio * (double)(L * U));
  if (b < p->budget_min) b = p->budget_min;
  const Reg r = regions_of(L, p);
  const int64_t a = b - (r.ss - r.c1) * U;
  *B = b;
  *alloc = a;
  *F = a > 0 ? (int64_t)std::floor((double)p->floor_frac * (double)a) : 0;
}

// ------------------------------------------------------------------ RoPE (rotate-half pairs)
// theta_j(pos) = pos * base^(-2j/d); pair (j, j + d/2) rotated by +-theta.
// The table holds cos and sin of theta_j(pos) for pos < n_pos.
struct Rope {
  int d = 0;
  vector<double> cs, sn;  // [n_pos][d/2]
  void make(int64_t n_pos, int dd, double base) {
    d = dd;
    const int h = d / 2;
    vector<double> inv(h);
    for (int j = 0; j < h; ++j) inv[j] = std::pow(base, -2.0 * (double)j / (double)d);
    cs.resize((size_t)(n_pos * h));
    sn.resize((size_t)(n_pos * h));
    for (int64_t p = 0; p < n_pos; ++p)
      for (int j = 0; j < h; ++j) {
        const double th = (double)p * inv[j];
        cs[(size_t)(p * h + j)] = std::cos(th);
        sn[(size_t)(p * h + j)] = std::sin(th);
      }
  }
  // sign +1 rotates, -1 rotates back
  void apply(const double* x, int64_t pos, double sign, double* out) const {
    const int h = d / 2;
    const double* c = &cs[(size_t)(pos * h)];
    const double* s = &sn[(size_t)(pos * h)];
    for (int j = 0; j < h; ++j) {
      out[j] = x[j] * c[j] - x[j + h] * (sign * s[j]);
      out[j + h] = x[j + h] * c[j] + x[j] * (sign * s[j]);
    }
  }
};

// ------------------------------------------------------------------ trees
struct Node {
  int64_t st, n;
  int ch[3], nch;  // children in position order (nch 0: leaf)
  int parent;      // -1: root
};
constexpr uint32_t TOPO_NONE = 0xFFFFFFFFu;

// left-to-right float64 sum of fp32 values
double seq_sum(const float* x, int64_t n) {
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += (double)x[i];
  return s;
}

// Child intervals of the node [st, st+n), n >= 2 (r and cut indexed by
// sequence position; cut nullable). split_mode 0: midpoint, left ceil(n/2).
// split_mode 1 (GraceKV page, 'Technical details and default settings':
// high-curvature candidates beside the midpoint, a salient token isolated in
// a three-way child set): the first position i of the node's largest fp32
// relevance splits the node three ways when n >= 3, the node's relevance S (a
// left-to-right float64 sum) is positive, 2 r_i > S and i is at least
// max(floor(n/4), 1) tokens from either end; otherwise one cut among those
// that leave both children at least ceil(n/4) tokens, the largest cut score
// winning (ties: the midpoint, then the nearest cut, then the lower one), or
// the midpoint without cut scores.
int split_children(int64_t st, int64_t n, const float* r, const int64_t* cut, int mode, int64_t* ca, int64_t* cn) {
  int64_t b = (n + 1) / 2;
  if (mode == 1) {
    if (n >= 3) {
      int64_t i = 0;
      for (int64_t k = 1; k < n; ++k)
        if (r[st + k] > r[st + i]) i = k;
      const double S = seq_sum(r + st, n);
      const int64_t q = std::max<int64_t>(n / 4, 1);
      if (S > 0 && 2.0 * (double)r[st + i] > S && i >= q && i <= n - 1 - q) {
        ca[0] = st, cn[0] = i;
        ca[1] = st + i, cn[1] = 1;
        ca[2] = st + i + 1, cn[2] = n - i - 1;
        return 3;
      }
    }
    if (cut) {
      const int64_t m4 = (n + 3) / 4;
      const int64_t lo = std::max<int64_t>(1, m4), hi = std::min<int64_t>(n - 1, n - m4);
      int64_t best = b, bv = cut[st + b];
      for (int64_t c = lo; c <= hi; ++c) {
        const int64_t v = cut[st + c];
        const int64_t dc = c > b ? c - b : b - c, db = best > b ? best - b : b - best;
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

// pre-order nodes of the slot [a, a+n)
void build_tree(int64_t a, int64_t n, const float* r, const int64_t* cut, int mode, vector<Node>& out) {
  out.clear();
  struct Rec {
    static int go(int64_t st, int64_t m, int parent, const float* r, const int64_t* cut, int mode, vector<Node>& o) {
      const int j = (int)o.size();
      o.push_back(Node{st, m, {-1, -1, -1}, 0, parent});
      if (m > 1) {
        int64_t ca[3], cn[3];
        const int k = split_children(st, m, r, cut, mode, ca, cn);
        for (int x = 0; x < k; ++x) {
          const int c = go(ca[x], cn[x], j, r, cut, mode, o);
          o[j].ch[x] = c;
        }
        o[j].nch = k;
      }
      return j;
    }
  };
  Rec::go(a, n, -1, r, cut, mode, out);
}

// the midpoint tree
void tree_nodes(int64_t a, int64_t n, vector<Node>& out) { build_tree(a, n, nullptr, nullptr, 0, out); }

// node records: bits 0-7 first token - slot start, 8-15 length - 1, 16-23
// parent + 1, 24-31 next sibling (0: none); TOPO_NONE past the last node
void encode_topo(const vector<Node>& nodes, int64_t a, int64_t n, uint32_t* rec) {
  for (int64_t j = 0; j < 2 * n; ++j) rec[j] = TOPO_NONE;
  vector<int> nxt(nodes.size(), 0);
  for (const Node& nd : nodes)
    for (int x = 0; x + 1 < nd.nch; ++x) nxt[nd.ch[x]] = nd.ch[x + 1];
  for (size_t j = 0; j < nodes.size(); ++j)
    rec[j] = (uint32_t)(nodes[j].st - a) | ((uint32_t)(nodes[j].n - 1) << 8) | ((uint32_t)(nodes[j].parent + 1) << 16) |
             ((uint32_t)nxt[j] << 24);
}
void decode_topo(const uint32_t* rec, int64_t a, int64_t n, vector<Node>& out) {
  out.clear();
  for (int64_t j = 0; j < 2 * n && rec[j] != TOPO_NONE; ++j)
    out.push_back(Node{a + (rec[j] & 255), (int64_t)((rec[j] >> 8) & 255) + 1, {-1, -1, -1}, 0,
                       (int)((rec[j] >> 16) & 255) - 1});
  for (size_t j = 0; j < out.size(); ++j)
    if (out[j].parent >= 0) {
      Node& p = out[out[j].parent];
      p.ch[p.nch++] = (int)j;
    }
}
// the nodes of a slot: from the records when given, else the midpoint tree
void slot_nodes(const uint32_t* topo, int64_t unit, int64_t T, int64_t a0, int64_t st, int64_t n, vector<Node>& out) {
  if (!topo) {
    tree_nodes(st, n, out);
    return;
  }
  decode_topo(topo + unit * 2 * T + 2 * (a0 + st), st, n, out);
}

vector<int> dprobe_rows(int G, int P, int n_dprobe) {
  const int R = G * P;
  const int Pd = std::min(n_dprobe, R);
  const int stride = R / Pd;
  vector<int> r;
  for (int k = 0; k < Pd; ++k) r.push_back(k * stride);
  return r;
}

struct SlotList {
  vector<std::pair<int64_t, int64_t>> v;  // (start, n) in sequence positions
};
SlotList slots_of(const int32_t* slot_start, const int32_t* n_slots, int stride, int s) {
  SlotList out;
  const int32_t* ss = slot_start + (int64_t)s * (stride + 1);
  for (int k = 0; k < n_slots[s]; ++k) out.v.push_back({ss[k], (int64_t)ss[k + 1] - ss[k]});
  return out;
}

}  // namespace

extern "C" int ko_threads(void) { return omp_get_max_threads(); }

extern "C" void ko_regions(int64_t L, const ko_params* p, int64_t* out) {
  const Reg r = regions_of(L, p);
  out[0] = r.pe;
  out[1] = r.c0;
  out[2] = r.c1;
  out[3] = r.ss;
}

extern "C" void ko_budgets(const ko_shape* sh, const ko_params* p, int64_t* B, int64_t* alloc, int64_t* F) {
  for (int s = 0; s < sh->S; ++s) budgets_of(sh, p, s, B + s, alloc + s, F + s);
}

// ------------------------------------------------------------------ O1 probe scores
// GraceKV page, '03 Bottom-up value flow' (direct relevance from question and
// tail probes); DistillCache paper, Sec. 3.1.1 (features). For each probe row
// rho of a unit: s = c <q, k_i>, lse, a = exp(s - lse), H = lse - sum a s.
// r0_i = sum_rho a; features (r0, ||v||, variance over g of sum_p a,
// sum a H / r0, i / (L-1)); sensitivity sum r0 ||v|| / sum r0.
extern "C" void ko_probe_scores(const ko_shape* sh, const void* K, const void* V, const void* Qp, float* r0_out,
                                float* feats, float* lse_out, float* ent_out, float* sens_out) {
  const int S = sh->S, Ly = sh->Ly, H = sh->H, G = sh->G, d = sh->d, P = sh->P, dt = sh->dtype;
  const int64_t T = sh->T;
  const int R = G * P;
  const double c = 1.0 / std::sqrt((double)d);
  const int64_t units = (int64_t)S * Ly * H;
  Progress prog("probe scores", units);
#pragma omp parallel
  {
    vector<double> Ku, Vu, Q, Sm;
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
      const int s = (int)(u / (Ly * H)), l = (int)(u / H % Ly), h = (int)(u % H);
      const int64_t a = sh->cu[s], L = sh->cu[s + 1] - sh->cu[s];
      if (L == 0) {
        prog.tick();
        continue;
      }
      const int64_t ubase = ((int64_t)l * H + h) * T;
      rows(K, dt, ubase + a, L, d, Ku);
      rows(V, dt, ubase + a, L, d, Vu);
      rows(Qp, dt, (((int64_t)s * Ly + l) * H * G + (int64_t)h * G) * P, R, d, Q);
      Sm.resize((size_t)(R * L));
      for (int64_t i0 = 0; i0 < L; i0 += 64)  // 64 keys at a time stay in cache for every row
        for (int rr = 0; rr < R; ++rr)
          for (int64_t i = i0; i < std::min<int64_t>(L, i0 + 64); ++i)
            Sm[(size_t)(rr * L + i)] = c * dot(&Q[(size_t)rr * d], &Ku[(size_t)i * d], d);
      vector<double> lse(R), ent(R), r0(L, 0.0), wsum(L, 0.0), mg((size_t)(G * L), 0.0);
      for (int rr = 0; rr < R; ++rr) {
        double* srow = &Sm[(size_t)(rr * L)];
        double m = -std::numeric_limits<double>::infinity();
        for (int64_t i = 0; i < L; ++i) m = std::max(m, srow[i]);
        double z = 0.0;
        for (int64_t i = 0; i < L; ++i) z += std::exp(srow[i] - m);
        lse[rr] = m + std::log(z);
        double as = 0.0;
        for (int64_t i = 0; i < L; ++i) {
          const double ai = std::exp(srow[i] - lse[rr]);
          as += ai * srow[i];
          srow[i] = ai;  // the row now holds a
        }
        ent[rr] = lse[rr] - as;
      }
      for (int rr = 0; rr < R; ++rr) {
        const double* arow = &Sm[(size_t)(rr * L)];
        const int g = rr / P;
        for (int64_t i = 0; i < L; ++i) {
          r0[i] += arow[i];
          wsum[i] += arow[i] * ent[rr];
          mg[(size_t)(g * L + i)] += arow[i];
        }
      }
      double num = 0.0, den = 0.0;
      for (int64_t i = 0; i < L; ++i) {
        const double vn = std::sqrt(dot(&Vu[(size_t)i * d], &Vu[(size_t)i * d], d));
        double mean = 0.0;
        for (int g = 0; g < G; ++g) mean += mg[(size_t)(g * L + i)];
        mean /= G;
        double var = 0.0;
        for (int g = 0; g < G; ++g) {
          const double e = mg[(size_t)(g * L + i)] - mean;
          var += e * e;
        }
        var /= G;
        const double Hi = r0[i] > 0 ? wsum[i] / r0[i] : 0.0;
        const double pos = (double)i / (double)std::max<int64_t>(L - 1, 1);
        const int64_t o = ubase + a + i;
        r0_out[o] = (float)r0[i];
        if (feats) {
          const int64_t E = (int64_t)Ly * H * T;
          feats[0 * E + o] = (float)r0[i];
          feats[1 * E + o] = (float)vn;
          feats[2 * E + o] = (float)var;
          feats[3 * E + o] = (float)Hi;
          feats[4 * E + o] = (float)pos;
        }
        num += r0[i] * vn;
        den += r0[i];
      }
      for (int rr = 0; rr < R; ++rr) {
        const int64_t o = (((int64_t)s * Ly + l) * H * G + (int64_t)h * G) * P + rr;
        lse_out[o] = (float)lse[rr];
        ent_out[o] = (float)ent[rr];
      }
      sens_out[u] = (float)(den > 0 ? num / den : 0.0);
      prog.tick();
    }
  }
}

// ------------------------------------------------------------------ O2 propagation
// GraceKV page, '03 Bottom-up value flow' and technical details (two graph
// hops, weight 0.3). delta_0 = r0; hop t: seeds = top-M of delta_{t-1}
// (ties to the lower index, all when L <= M); each seed j passes
// w delta_{t-1}(j) over its causal prefill softmax row, averaged over the G
// query heads; rel = r0 + delta_1 + delta_2.
extern "C" void ko_propagate(const ko_shape* sh, const ko_params* p, const void* K, const void* Qctx,
                             const float* r0, float* rel, int32_t* seeds) {
  const int S = sh->S, Ly = sh->Ly, H = sh->H, G = sh->G, d = sh->d, dt = sh->dtype;
  const int64_t T = sh->T;
  const int M = p->n_seeds, hops = p->n_hops;
  const double w = (double)p->hop_weight;
  const double c = 1.0 / std::sqrt((double)d);
  const int64_t units = (int64_t)S * Ly * H;
  if (seeds)
    for (int64_t i = 0; i < (int64_t)hops * units * M; ++i) seeds[i] = -1;
  Progress prog("propagation", units);
#pragma omp parallel
  {
    vector<double> Ku, q(d), lg;
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
      const int s = (int)(u / (Ly * H)), l = (int)(u / H % Ly), h = (int)(u % H);
      const int64_t a = sh->cu[s], L = sh->cu[s + 1] - sh->cu[s];
      const int64_t ubase = ((int64_t)l * H + h) * T;
      if (L == 0) {
        prog.tick();
        continue;
      }
      rows(K, dt, ubase + a, L, d, Ku);
      vector<double> prev(L), total(L);
      for (int64_t i = 0; i < L; ++i) prev[i] = total[i] = (double)r0[ubase + a + i];
      for (int t = 0; t < hops; ++t) {
        vector<int64_t> order(L);
        for (int64_t i = 0; i < L; ++i) order[i] = i;
        std::stable_sort(order.begin(), order.end(), [&](int64_t x, int64_t y) { return prev[x] > prev[y]; });
        vector<int64_t> sd(order.begin(), order.begin() + std::min<int64_t>(M, L));
        std::sort(sd.begin(), sd.end());
        if (seeds)
          for (size_t k = 0; k < sd.size(); ++k) seeds[((int64_t)t * units + u) * M + (int64_t)k] = (int32_t)sd[k];
        vector<double> delta(L, 0.0), bm;
        for (int64_t j : sd) {
          bm.assign((size_t)(j + 1), 0.0);
          lg.resize((size_t)(j + 1));
          for (int g = 0; g < G; ++g) {
            const int64_t qrow = (((int64_t)l * H * G + (int64_t)h * G + g) * T) + a + j;
            for (int k = 0; k < d; ++k) q[k] = elem(Qctx, dt, qrow * d + k);
            double m = -std::numeric_limits<double>::infinity();
            for (int64_t i = 0; i <= j; ++i) {
              lg[i] = c * dot(q.data(), &Ku[(size_t)i * d], d);
              m = std::max(m, lg[i]);
            }
            double z = 0.0;
            for (int64_t i = 0; i <= j; ++i) z += std::exp(lg[i] - m);
            const double lse = m + std::log(z);
            for (int64_t i = 0; i <= j; ++i) bm[i] += std::exp(lg[i] - lse);
          }
          for (int64_t i = 0; i <= j; ++i) delta[i] += w * prev[j] * (bm[i] / G);
        }
        for (int64_t i = 0; i < L; ++i) total[i] += delta[i];
        prev.swap(delta);
      }
      for (int64_t i = 0; i < L; ++i) rel[ubase + a + i] = (float)total[i];
      prog.tick();
    }
  }
}

// ------------------------------------------------------------------ O3 slots
namespace {
int64_t quant(double x) {  // round half away from zero, x * 2^20
  const double q = 1048576.0;
  return x >= 0 ? (int64_t)std::floor(x * q + 0.5) : -(int64_t)std::floor(-x * q + 0.5);
}
}  // namespace

// GraceKV page, '01 Curvature-guided partition' and technical details (turns
// of the normalized trajectory across sampled depths and windows; dispersion
// and length in a DP; surprisal a smaller auxiliary signal). kappa_b = mean
// over valid (depth, window in {2, 8}) of (1 - cos(h_b - h_{b-w},
// h_{b+w} - h_b)) / 2; a slot costs its mean dispersion over depths plus
// lambda_len ((n - target) / target)^2; a cut earns lambda_curv kappa plus
// lambda_surp s_b / max s. Both quantized to integers before the DP.
extern "C" void ko_slot_costs(const ko_shape* sh, const ko_params* p, const void* hidden, int32_t dim,
                              int32_t n_depth, const float* surprisal, int64_t* cost_q, int64_t* cut_q) {
  const int64_t T = sh->T;
  const int nmin = p->slot_min, nmax = p->slot_max, NW = nmax - nmin + 1;
  const int D = std::max(1, (int)n_depth);
  const double lam_c = (double)p->lambda_curv, lam_s = (double)p->lambda_surp, lam_len = (double)p->lambda_len;
  const double tl = (double)p->slot_target;
  std::memset(cost_q, 0, sizeof(int64_t) * (size_t)(T * NW));
  std::memset(cut_q, 0, sizeof(int64_t) * (size_t)T);
  for (int s = 0; s < sh->S; ++s) {
    const int64_t a0 = sh->cu[s], L = sh->cu[s + 1] - a0;
    if (L == 0) continue;
    // normalized trajectories of every depth
    vector<double> hn((size_t)(D * L * dim));
#pragma omp parallel for schedule(static)
    for (int64_t x = 0; x < (int64_t)D * L; ++x) {
      const int dd = (int)(x / L);
      const int64_t i = x % L;
      double* o = &hn[(size_t)(x * dim)];
      const int64_t src = ((int64_t)dd * T + a0 + i) * dim;
      for (int k = 0; k < dim; ++k) o[k] = elem(hidden, sh->dtype, src + k);
      const double nr = std::sqrt(dot(o, o, dim));
      for (int k = 0; k < dim; ++k) o[k] = nr > 0 ? o[k] / nr : 0.0;
    }
    const Reg rg = regions_of(L, p);
    double smax = 0.0;
    if (surprisal) {
      smax = -std::numeric_limits<double>::infinity();
      for (int64_t i = 0; i < L; ++i) smax = std::max(smax, (double)surprisal[a0 + i]);
    }
    const int W[2] = {2, 8};
#pragma omp parallel for schedule(static)
    for (int64_t b = rg.c0; b < rg.c1; ++b) {
      double sum = 0.0;
      int cnt = 0;
      vector<double> u(dim), v(dim);
      for (int dd = 0; dd < D; ++dd)
        for (int wi = 0; wi < 2; ++wi) {
          const int w = W[wi];
          if (b - w < 0 || b + w > L - 1) continue;
          const double* P0 = &hn[(size_t)((dd * L + b - w) * dim)];
          const double* P1 = &hn[(size_t)((dd * L + b) * dim)];
          const double* P2 = &hn[(size_t)((dd * L + b + w) * dim)];
          for (int k = 0; k < dim; ++k) {
            u[k] = P1[k] - P0[k];
            v[k] = P2[k] - P1[k];
          }
          const double nu = std::sqrt(dot(u.data(), u.data(), dim)), nv = std::sqrt(dot(v.data(), v.data(), dim));
          if (nu == 0 || nv == 0) continue;
          sum += (1.0 - dot(u.data(), v.data(), dim) / (nu * nv)) / 2.0;
          ++cnt;
        }
      double bonus = lam_c * (cnt ? sum / cnt : 0.0);
      if (surprisal && smax > 0) bonus += lam_s * (double)surprisal[a0 + b] / smax;
      cut_q[a0 + b] = quant(bonus);
    }
    // every (end, length) window of the compressible region, its dispersion
    // evaluated from its definition
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t e = rg.c0 + 1; e <= rg.c1; ++e) {
      vector<double> mean(dim);
      for (int n = nmin; n <= nmax; ++n) {
        const int64_t st = e - n;
        if (st < rg.c0) break;
        double disp = 0.0;
        for (int dd = 0; dd < D; ++dd) {
          std::fill(mean.begin(), mean.end(), 0.0);
          for (int64_t i = st; i < e; ++i) {
            const double* x = &hn[(size_t)((dd * L + i) * dim)];
            for (int k = 0; k < dim; ++k) mean[k] += x[k];
          }
          for (int k = 0; k < dim; ++k) mean[k] /= n;
          double sd = 0.0;
          for (int64_t i = st; i < e; ++i) {
            const double* x = &hn[(size_t)((dd * L + i) * dim)];
            double acc = 0.0;
#pragma omp simd reduction(+ : acc)
            for (int k = 0; k < dim; ++k) acc += (x[k] - mean[k]) * (x[k] - mean[k]);
            sd += acc;
          }
          disp += sd;
        }
        const double cost = disp / D + lam_len * ((n - tl) / tl) * ((n - tl) / tl);
        cost_q[(a0 + e - 1) * NW + (n - nmin)] = quant(cost);
      }
    }
  }
}

// Minimum of sum(slot costs) - sum(cut bonuses of internal cuts) over
// segmentations of the compressible region into slot_min..slot_max tokens
// (exact integer DP, ties to the earlier previous cut); a region shorter than
// slot_min is one slot. Fixed-length slots when slot_len > 0.
extern "C" void ko_slots(const ko_shape* sh, const ko_params* p, const int64_t* cost_q, const int64_t* cut_q,
                         int32_t stride, int32_t* slot_start, int32_t* n_slots) {
  const int nmin = p->slot_min, nmax = p->slot_max, NW = nmax - nmin + 1;
  for (int s = 0; s < sh->S; ++s) {
    const int64_t a0 = sh->cu[s], L = sh->cu[s + 1] - a0;
    const Reg rg = regions_of(L, p);
    int32_t* ss = slot_start + (int64_t)s * (stride + 1);
    vector<std::pair<int64_t, int64_t>> out;
    const int64_t Lc = rg.c1 - rg.c0;
    if (p->token_mode || Lc <= 0) {
    } else if (p->slot_len > 0) {
      for (int64_t x = rg.c0; x < rg.c1; x += p->slot_len) out.push_back({x, std::min<int64_t>(p->slot_len, rg.c1 - x)});
    } else if (Lc < nmin) {
      out.push_back({rg.c0, Lc});
    } else {
      const int64_t NONE = std::numeric_limits<int64_t>::max();
      vector<int64_t> f((size_t)(Lc + 1), NONE);
      vector<int> arg((size_t)(Lc + 1), 0);
      f[0] = 0;
      for (int64_t e = 1; e <= Lc; ++e) {
        int64_t best = NONE;
        int bn = 0;
        for (int64_t n = std::min<int64_t>(nmax, e); n >= nmin; --n) {  // larger n = earlier cut first
          const int64_t pcut = e - n;
          if (f[pcut] == NONE) continue;
          int64_t v = f[pcut] + cost_q[(a0 + rg.c0 + e - 1) * NW + (n - nmin)];
          if (pcut > 0) v -= cut_q[a0 + rg.c0 + pcut];
          if (best == NONE || v < best) {
            best = v;
            bn = (int)n;
          }
        }
        f[e] = best;
        arg[e] = bn;
      }
      vector<std::pair<int64_t, int64_t>> rev;
      for (int64_t e = Lc; e > 0; e -= arg[e]) rev.push_back({rg.c0 + e - arg[e], arg[e]});
      out.assign(rev.rbegin(), rev.rend());
    }
    n_slots[s] = (int32_t)out.size();
    for (int k = 0; k <= stride; ++k) ss[k] = 0;
    for (size_t k = 0; k < out.size(); ++k) ss[k] = (int32_t)out[k].first;
    if (!out.empty()) ss[out.size()] = (int32_t)(out.back().first + out.back().second);
  }
}

// ------------------------------------------------------------------ O4 trees
// GraceKV page, '02 Progressively refinable representation', 'Inside one
// cache entry', '03 Bottom-up value flow', '04 Top-down budget flow' and the
// technical details (prototype fidelity 0.25 : 0.75). Per node [a, a+n):
// rel = sum of children (leaves r_i); k~ = RoPE^-1(k_i, i); k^ = RoPE(mean k~,
// a + (n-1)/2); v^ = sum ((1-beta) r_i / rel + beta / n) v_i (uniform when
// rel = 0); mu = max(1, n ||sum k~|| / sum ||k~||); over the distortion rows
// rho: Z = sum a, Z^ = mu exp(c <q, k^> - lse), u = sum a v;
// e_A = sum |Z^ - Z| / sum Z, e_V = sum ||u - Z v^|| / sum ||u||,
// D = min(1, w_A e_A + w_V e_V), leaves D = 0. Ops: Add gains
// rel_root (1 - D_root), Split(j) gains rel_j D_j - sum_c rel_c D_c and costs
// (children - 1), utility fp32(sens * gain / cost). The tree of a slot comes
// from split_children (the partition's cut scores cut_q, nullable), or from
// given node records topo_in (nullable).
extern "C" void ko_build_trees(const ko_shape* sh, const ko_params* p, const void* K, const void* V,
                               const void* Qp, const float* lse_in, const float* rel_in, const float* sens_in,
                               const int32_t* slot_start, const int32_t* n_slots, int32_t stride,
                               const int64_t* cut_q, const uint32_t* topo_in, float* node_rel, float* node_D,
                               float* node_mu, float* op_util, uint8_t* op_cost, uint32_t* node_topo) {
  const int S = sh->S, Ly = sh->Ly, H = sh->H, G = sh->G, d = sh->d, P = sh->P, dt = sh->dtype;
  const int64_t T = sh->T;
  const double c = 1.0 / std::sqrt((double)d), base = p->rope_base;
  const double beta = (double)p->value_base, wA = (double)p->w_attn, wV = (double)p->w_value;
  const vector<int> drows = dprobe_rows(G, P, p->n_dprobe);
  const int Pd = (int)drows.size();
  const int64_t units = (int64_t)S * Ly * H;
  int64_t max_len = 0;
  for (int s = 0; s < S; ++s) max_len = std::max<int64_t>(max_len, sh->cu[s + 1] - sh->cu[s]);
  Rope rope;
  rope.make(max_len, d, base);
  Progress prog("trees", units);
#pragma omp parallel
  {
    vector<double> Ku, Vu, ktil, knorm, Q((size_t)Pd * d), ls(Pd), Ad, r;
    vector<Node> nodes;
    vector<double> rel, D, mu, skt(d), khat(d), kbar(d), vhat(d), u(d), Z(Pd), Zh(Pd), U;
#pragma omp for schedule(dynamic, 1)
    for (int64_t uu = 0; uu < units; ++uu) {
      const int s = (int)(uu / (Ly * H)), l = (int)(uu / H % Ly), h = (int)(uu % H);
      const int64_t a0 = sh->cu[s], L = sh->cu[s + 1] - a0;
      const SlotList sl = slots_of(slot_start, n_slots, stride, s);
      if (L == 0 || sl.v.empty()) {
        prog.tick();
        continue;
      }
      const int64_t ubase = ((int64_t)l * H + h) * T;
      rows(K, dt, ubase + a0, L, d, Ku);
      rows(V, dt, ubase + a0, L, d, Vu);
      ktil.resize((size_t)(L * d));
      knorm.resize((size_t)L);
      for (int64_t i = 0; i < L; ++i) {
        rope.apply(&Ku[(size_t)i * d], i, -1.0, &ktil[(size_t)i * d]);
        knorm[i] = std::sqrt(dot(&ktil[(size_t)i * d], &ktil[(size_t)i * d], d));
      }
      const int64_t qb = (((int64_t)s * Ly + l) * H * G + (int64_t)h * G) * P;
      for (int k = 0; k < Pd; ++k) {
        for (int x = 0; x < d; ++x) Q[(size_t)k * d + x] = elem(Qp, dt, (qb + drows[k]) * d + x);
        ls[k] = (double)lse_in[qb + drows[k]];
      }
      Ad.resize((size_t)(Pd * L));
      for (int k = 0; k < Pd; ++k)
        for (int64_t i = 0; i < L; ++i)
          Ad[(size_t)(k * L + i)] = std::exp(c * dot(&Q[(size_t)k * d], &Ku[(size_t)i * d], d) - ls[k]);
      r.resize((size_t)L);
      for (int64_t i = 0; i < L; ++i) r[i] = (double)rel_in[ubase + a0 + i];
      const double sens = (double)sens_in[uu];
      const float* r32 = rel_in + ubase + a0;
      const int64_t* cq = cut_q ? cut_q + a0 : nullptr;
      for (const auto& slot : sl.v) {
        if (topo_in)
          slot_nodes(topo_in, (int64_t)l * H + h, T, a0, slot.first, slot.second, nodes);
        else
          build_tree(slot.first, slot.second, r32, cq, p->split_mode, nodes);
        const int m = (int)nodes.size();
        rel.assign(m, 0.0);
        D.assign(m, 0.0);
        mu.assign(m, 1.0);
        for (int j = m - 1; j >= 0; --j) {
          if (nodes[j].nch == 0) {
            rel[j] = r[nodes[j].st];
            continue;
          }
          double sum = 0.0;
          for (int x = 0; x < nodes[j].nch; ++x) sum += rel[nodes[j].ch[x]];
          rel[j] = sum;
        }
        for (int j = 0; j < m; ++j) {
          const int64_t st = nodes[j].st, n = nodes[j].n;
          std::fill(skt.begin(), skt.end(), 0.0);
          double sn = 0.0;
          for (int64_t i = st; i < st + n; ++i) {
            for (int x = 0; x < d; ++x) skt[x] += ktil[(size_t)i * d + x];
            sn += knorm[i];
          }
          const double rho = sn > 0 ? std::sqrt(dot(skt.data(), skt.data(), d)) / sn : 1.0;
          mu[j] = std::max(1.0, (double)n * rho);
          for (int x = 0; x < d; ++x) kbar[x] = skt[x] / (double)n;
          rope.apply(kbar.data(), st + (n - 1) / 2, 1.0, khat.data());
          std::fill(vhat.begin(), vhat.end(), 0.0);
          for (int64_t i = st; i < st + n; ++i) {
            const double wi = rel[j] > 0 ? (1.0 - beta) * r[i] / rel[j] + beta / (double)n : 1.0 / (double)n;
            for (int x = 0; x < d; ++x) vhat[x] += wi * Vu[(size_t)i * d + x];
          }
          if (nodes[j].nch == 0) continue;
          double numA = 0.0, denA = 0.0, numV = 0.0, denV = 0.0;
          for (int k = 0; k < Pd; ++k) {
            const double* arow = &Ad[(size_t)(k * L)];
            double z = 0.0;
            std::fill(u.begin(), u.end(), 0.0);
            for (int64_t i = st; i < st + n; ++i) {
              z += arow[i];
              for (int x = 0; x < d; ++x) u[x] += arow[i] * Vu[(size_t)i * d + x];
            }
            const double zh = mu[j] * std::exp(c * dot(&Q[(size_t)k * d], khat.data(), d) - ls[k]);
            numA += std::fabs(zh - z);
            denA += z;
            double e2 = 0.0, u2 = 0.0;
            for (int x = 0; x < d; ++x) {
              const double e = u[x] - z * vhat[x];
              e2 += e * e;
              u2 += u[x] * u[x];
            }
            numV += std::sqrt(e2);
            denV += std::sqrt(u2);
          }
          const double eA = denA > 0 ? numA / denA : 0.0, eV = denV > 0 ? numV / denV : 0.0;
          D[j] = std::min(1.0, wA * eA + wV * eV);
        }
        const int64_t ob = ubase * 2 + 2 * (a0 + slot.first);
        for (int j = 0; j < m; ++j) {
          node_rel[ob + j] = (float)rel[j];
          node_D[ob + j] = (float)D[j];
          node_mu[ob + j] = (float)mu[j];
        }
        op_util[ob] = (float)(sens * (rel[0] * (1.0 - D[0])));
        op_cost[ob] = 1;
        for (int j = 0; j < m; ++j) {
          if (nodes[j].nch == 0) continue;
          double sub = 0.0;
          for (int x = 0; x < nodes[j].nch; ++x) sub += rel[nodes[j].ch[x]] * D[nodes[j].ch[x]];
          const double gain = rel[j] * D[j] - sub;
          op_util[ob + 1 + j] = (float)(sens * gain / (double)(nodes[j].nch - 1));
          op_cost[ob + 1 + j] = (uint8_t)(nodes[j].nch - 1);
        }
        if (node_topo) encode_topo(nodes, slot.first, slot.second, node_topo + ob);
      }
      prog.tick();
    }
  }
}

// ------------------------------------------------------------------ O5 floor, O6 auction
namespace {
// internal nodes on the path from the root to the leaf of position i
void leaf_path(const vector<Node>& nodes, int64_t i, vector<int>& path) {
  path.clear();
  int j = 0;
  while (nodes[j].nch > 0) {
    path.push_back(j);
    int next = nodes[j].ch[0];
    for (int x = 0; x < nodes[j].nch; ++x) {
      const Node& c = nodes[nodes[j].ch[x]];
      if (i >= c.st && i < c.st + c.n) next = nodes[j].ch[x];
    }
    j = next;
  }
}
}  // namespace

// GraceKV page, 'Exact-information safeguard' and technical details: the
// compressible leaves ranked by fp32(s_lh r_i) (desc; flat id asc), the first
// F scanned in order, each paying the not-yet-taken ops of its root-to-leaf
// path and accepted while the floor spend stays <= F.
extern "C" void ko_floor(const ko_shape* sh, const ko_params* p, const float* rel, const float* sens,
                         const uint8_t* op_cost, const uint32_t* node_topo, const int32_t* slot_start,
                         const int32_t* n_slots, int32_t stride, uint8_t* taken, int64_t* spent) {
  const int Ly = sh->Ly, H = sh->H;
  const int64_t T = sh->T;
  std::memset(taken, 0, (size_t)((int64_t)Ly * H * 2 * T));
#pragma omp parallel for schedule(dynamic, 1)
  for (int s = 0; s < sh->S; ++s) {
    int64_t B, A, F;
    budgets_of(sh, p, s, &B, &A, &F);
    spent[s] = 0;
    const SlotList sl = slots_of(slot_start, n_slots, stride, s);
    if (F <= 0 || sl.v.empty()) continue;
    const int64_t a0 = sh->cu[s];
    struct Cand {
      double key;
      int64_t fid;
    };
    vector<Cand> cands;
    for (int l = 0; l < Ly; ++l)
      for (int h = 0; h < H; ++h) {
        const double sv = (double)sens[((int64_t)s * Ly + l) * H + h];
        for (const auto& slot : sl.v)
          for (int64_t i = slot.first; i < slot.first + slot.second; ++i) {
            const float v = (float)(sv * (double)rel[((int64_t)l * H + h) * T + a0 + i]);
            cands.push_back({rank_key(v), ((int64_t)l * H + h) * T + a0 + i});
          }
      }
    std::sort(cands.begin(), cands.end(),
              [](const Cand& x, const Cand& y) { return x.key != y.key ? x.key > y.key : x.fid < y.fid; });
    vector<Node> nodes;
    vector<int> path;
    vector<int64_t> ops;
    const int64_t nscan = std::min<int64_t>(F, (int64_t)cands.size());
    for (int64_t k = 0; k < nscan; ++k) {
      const int64_t fid = cands[k].fid;
      const int64_t unit = fid / T, i = fid % T - a0;
      // the slot holding position i
      const auto it = std::upper_bound(sl.v.begin(), sl.v.end(), i,
                                       [](int64_t x, const std::pair<int64_t, int64_t>& y) { return x < y.first; });
      const auto& slot = *(it - 1);
      slot_nodes(node_topo, unit, T, a0, slot.first, slot.second, nodes);
      leaf_path(nodes, i, path);
      const int64_t base = unit * 2 * T + 2 * (a0 + slot.first);
      ops.assign(1, base);
      for (int j : path) ops.push_back(base + 1 + j);
      int64_t cst = 0;
      for (int64_t o : ops)
        if (!taken[o]) cst += op_cost[o];
      if (spent[s] + cst <= F) {
        for (int64_t o : ops) taken[o] = 1;
        spent[s] += cst;
      }
    }
  }
}

// GraceKV page, '04 Top-down budget flow': every exposed Add and Split in one
// queue per sequence, the highest utility (lower op id on ties) popped next,
// taken if it fits the remaining budget (discarded otherwise), exposing the
// ops of the nodes it creates; until the budget is spent or the queue is
// empty. NaN utilities rank below everything.
extern "C" void ko_auction(const ko_shape* sh, const ko_params* p, const float* op_util, const uint8_t* op_cost,
                           const uint32_t* node_topo, const int32_t* slot_start, const int32_t* n_slots,
                           int32_t stride, uint8_t* taken, int64_t* spent) {
  const int Ly = sh->Ly, H = sh->H;
  const int64_t T = sh->T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int s = 0; s < sh->S; ++s) {
    const SlotList sl = slots_of(slot_start, n_slots, stride, s);
    if (sl.v.empty()) continue;
    int64_t B, A, F;
    budgets_of(sh, p, s, &B, &A, &F);
    const int64_t a0 = sh->cu[s];
    int64_t rem = A - spent[s];
    struct Item {
      double key;
      int64_t op;
      int64_t base;  // the slot's first op
      int slot;      // index into the sequence's slot list
      int node;      // -1: the slot's Add, else the node the Split splits
    };
    auto worse = [](const Item& x, const Item& y) { return x.key != y.key ? x.key < y.key : x.op > y.op; };
    std::priority_queue<Item, vector<Item>, decltype(worse)> heap(worse);
    // per (l, h, slot) node lists: the trees differ between units
    const int64_t nsl = (int64_t)sl.v.size();
    vector<vector<Node>> trees((size_t)(Ly * H * nsl));
    for (int l = 0; l < Ly; ++l)
      for (int h = 0; h < H; ++h)
        for (int64_t k = 0; k < nsl; ++k)
          slot_nodes(node_topo, (int64_t)l * H + h, T, a0, sl.v[k].first, sl.v[k].second,
                     trees[(size_t)(((int64_t)l * H + h) * nsl + k)]);
    auto push = [&](int64_t base, int slot, int node) {
      const int64_t o = node < 0 ? base : base + 1 + node;
      heap.push(Item{rank_key(op_util[o]), o, base, slot, node});
    };
    // the ops an op exposes: Add exposes the root's Split, a Split the
    // Splits of its internal children
    auto children = [&](int slot, int node, vector<int>& out) {
      const vector<Node>& nd = trees[slot];
      out.clear();
      if (node < 0) {
        if (nd[0].nch > 0) out.push_back(0);
      } else {
        for (int x = 0; x < nd[node].nch; ++x)
          if (nd[nd[node].ch[x]].nch > 0) out.push_back(nd[node].ch[x]);
      }
    };
    vector<int> stack, ch;
    for (int l = 0; l < Ly; ++l)
      for (int h = 0; h < H; ++h)
        for (int64_t k = 0; k < nsl; ++k) {
          const int64_t base = ((int64_t)l * H + h) * 2 * T + 2 * (a0 + sl.v[k].first);
          const int tid = (int)(((int64_t)l * H + h) * nsl + k);
          // exposed ops given the floor's choices
          stack.assign(1, -1);
          while (!stack.empty()) {
            const int node = stack.back();
            stack.pop_back();
            const int64_t o = node < 0 ? base : base + 1 + node;
            if (taken[o]) {
              children(tid, node, ch);
              stack.insert(stack.end(), ch.begin(), ch.end());
            } else {
              push(base, tid, node);
            }
          }
        }
    while (!heap.empty() && rem > 0) {
      const Item it = heap.top();
      heap.pop();
      const int64_t cst = op_cost[it.op];
      if (cst > rem) continue;
      taken[it.op] = 1;
      rem -= cst;
      spent[s] += cst;
      children(it.slot, it.node, ch);
      for (int c2 : ch) push(it.base, it.slot, c2);
    }
  }
}

// DistillCache paper, Sec. 3.1.2 and Algorithm 1 (token mode): the first
// B_alloc compressible tokens of a sequence by (rel desc, flat id asc).
extern "C" void ko_token_topk(const ko_shape* sh, const ko_params* p, const float* rel, uint8_t* taken,
                              int64_t* spent) {
  const int Ly = sh->Ly, H = sh->H;
  const int64_t T = sh->T;
  std::memset(taken, 0, (size_t)((int64_t)Ly * H * T));
#pragma omp parallel for schedule(dynamic, 1)
  for (int s = 0; s < sh->S; ++s) {
    const int64_t a0 = sh->cu[s], L = sh->cu[s + 1] - a0;
    const Reg rg = regions_of(L, p);
    int64_t B, A, F;
    budgets_of(sh, p, s, &B, &A, &F);
    struct Cand {
      double key;
      int64_t fid;
    };
    vector<Cand> c;
    for (int l = 0; l < Ly; ++l)
      for (int h = 0; h < H; ++h)
        for (int64_t i = rg.c0; i < rg.c1; ++i) {
          const int64_t fid = ((int64_t)l * H + h) * T + a0 + i;
          c.push_back({rank_key(rel[fid]), fid});
        }
    std::sort(c.begin(), c.end(), [](const Cand& x, const Cand& y) { return x.key != y.key ? x.key > y.key : x.fid < y.fid; });
    const int64_t k = std::max<int64_t>(0, std::min<int64_t>(A, (int64_t)c.size()));
    for (int64_t x = 0; x < k; ++x) taken[c[x].fid] = 1;
    spent[s] = k;
  }
}

// ------------------------------------------------------------------ O7 pack
namespace {
// frontier of a slot (pre-order, so in position order): nodes whose creating
// op is taken and whose own split is not
void frontier(const vector<Node>& nodes, const uint8_t* taken, int64_t base, vector<int>& out) {
  out.clear();
  if (!taken[base]) return;
  vector<int> stack(1, 0);
  while (!stack.empty()) {
    const int j = stack.back();
    stack.pop_back();
    if (nodes[j].nch > 0 && taken[base + 1 + j]) {
      for (int x = nodes[j].nch - 1; x >= 0; --x) stack.push_back(nodes[j].ch[x]);
    } else {
      out.push_back(j);
    }
  }
}

// entries of one (s, l, h) segment: (kind, a, m, node) with kind 0 = token a,
// 1 = prototype of node covering [a, a+m)
struct Ent {
  int kind;
  int64_t a, m;
  int node;
  int64_t slot_first;
};
void segment_entries(const ko_shape* sh, const ko_params* p, const uint8_t* taken, const uint32_t* node_topo,
                     const SlotList& sl, int s, int l, int h, vector<Ent>& out) {
  const int H = sh->H;
  const int64_t T = sh->T, a0 = sh->cu[s], L = sh->cu[s + 1] - a0;
  const Reg rg = regions_of(L, p);
  out.clear();
  for (int64_t i = 0; i < rg.pe; ++i) out.push_back({0, i, 1, -1, 0});
  if (p->token_mode) {
    for (int64_t i = rg.c0; i < rg.c1; ++i)
      if (taken[((int64_t)l * H + h) * T + a0 + i]) out.push_back({0, i, 1, -1, 0});
  } else {
    vector<Node> nodes;
    vector<int> fr;
    for (const auto& slot : sl.v) {
      slot_nodes(node_topo, (int64_t)l * H + h, T, a0, slot.first, slot.second, nodes);
      const int64_t base = ((int64_t)l * H + h) * 2 * T + 2 * (a0 + slot.first);
      frontier(nodes, taken, base, fr);
      for (int j : fr) {
        if (nodes[j].n == 1)
          out.push_back({0, nodes[j].st, 1, -1, 0});
        else
          out.push_back({1, nodes[j].st, nodes[j].n, j, slot.first});
      }
    }
  }
  for (int64_t i = rg.c1; i < L; ++i) out.push_back({0, i, 1, -1, 0});
}
}  // namespace

extern "C" int64_t ko_pack_count(const ko_shape* sh, const ko_params* p, const uint8_t* taken,
                                 const uint32_t* node_topo, const int32_t* slot_start, const int32_t* n_slots,
                                 int32_t stride) {
  int64_t tot = 0;
#pragma omp parallel for reduction(+ : tot) schedule(dynamic, 1)
  for (int64_t x = 0; x < (int64_t)sh->Ly * sh->H * sh->S; ++x) {
    const int l = (int)(x / (sh->H * sh->S)), h = (int)(x / sh->S % sh->H), s = (int)(x % sh->S);
    vector<Ent> ents;
    segment_entries(sh, p, taken, node_topo, slots_of(slot_start, n_slots, stride, s), s, l, h, ents);
    tot += (int64_t)ents.size();
  }
  return tot;
}

// GraceKV page, '05 Physical cache packing': segments in (l, h, s) order;
// within a segment in position order: prompt, each slot's frontier (a leaf's
// original bits with ln mu 0 and its position; an internal node's prototype
// rounded to the cache dtype, ln mu and p_rep), recent window, suffix.
extern "C" void ko_pack(const ko_shape* sh, const ko_params* p, const void* K, const void* V, const float* rel,
                        const float* node_rel, const float* node_mu, const uint32_t* node_topo, const uint8_t* taken,
                        const int32_t* slot_start, const int32_t* n_slots, int32_t stride, void* Kp, void* Vp,
                        float* lnmu, int32_t* pos, int64_t* seg_off, int32_t* seg_len) {
  const int Ly = sh->Ly, H = sh->H, S = sh->S, d = sh->d, dt = sh->dtype;
  const int64_t T = sh->T;
  const double base = p->rope_base, beta = (double)p->value_base;
  const int64_t nseg = (int64_t)Ly * H * S;
  int64_t max_len = 0;
  for (int s = 0; s < S; ++s) max_len = std::max<int64_t>(max_len, sh->cu[s + 1] - sh->cu[s]);
  Rope rope;
  rope.make(max_len, d, base);
  vector<int64_t> cnt((size_t)nseg);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t x = 0; x < nseg; ++x) {
    const int l = (int)(x / (H * S)), h = (int)(x / S % H), s = (int)(x % S);
    vector<Ent> ents;
    segment_entries(sh, p, taken, node_topo, slots_of(slot_start, n_slots, stride, s), s, l, h, ents);
    cnt[x] = (int64_t)ents.size();
  }
  vector<int64_t> off((size_t)nseg);
  int64_t run = 0;
  for (int64_t x = 0; x < nseg; ++x) {
    off[x] = run;
    run += cnt[x];
    const int l = (int)(x / (H * S)), h = (int)(x / S % H), s = (int)(x % S);
    seg_off[((int64_t)s * Ly + l) * H + h] = off[x];
    seg_len[((int64_t)s * Ly + l) * H + h] = (int32_t)cnt[x];
  }
#pragma omp parallel
  {
    vector<Ent> ents;
    vector<double> kt(d), kbar(d), kh(d), vh(d), tmp(d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t x = 0; x < nseg; ++x) {
      const int l = (int)(x / (H * S)), h = (int)(x / S % H), s = (int)(x % S);
      const int64_t a0 = sh->cu[s];
      const int64_t ub = ((int64_t)l * H + h) * T + a0;
      segment_entries(sh, p, taken, node_topo, slots_of(slot_start, n_slots, stride, s), s, l, h, ents);
      int64_t e = off[x];
      for (const Ent& en : ents) {
        if (en.kind == 0) {
          for (int k = 0; k < d; ++k) {
            if (dt == 1) {
              ((uint16_t*)Kp)[e * d + k] = ((const uint16_t*)K)[(ub + en.a) * d + k];
              ((uint16_t*)Vp)[e * d + k] = ((const uint16_t*)V)[(ub + en.a) * d + k];
            } else {
              ((float*)Kp)[e * d + k] = ((const float*)K)[(ub + en.a) * d + k];
              ((float*)Vp)[e * d + k] = ((const float*)V)[(ub + en.a) * d + k];
            }
          }
          lnmu[e] = 0.f;
          pos[e] = (int32_t)en.a;
        } else {
          const int64_t nb = ((int64_t)l * H + h) * 2 * T + 2 * (a0 + en.slot_first) + en.node;
          const double rl = (double)node_rel[nb], mu = (double)node_mu[nb];
          std::fill(kbar.begin(), kbar.end(), 0.0);
          std::fill(vh.begin(), vh.end(), 0.0);
          for (int64_t i = en.a; i < en.a + en.m; ++i) {
            for (int k = 0; k < d; ++k) tmp[k] = elem(K, dt, (ub + i) * d + k);
            rope.apply(tmp.data(), i, -1.0, kt.data());
            for (int k = 0; k < d; ++k) kbar[k] += kt[k];
            const double wi = rl > 0 ? (1.0 - beta) * (double)rel[ub + i] / rl + beta / (double)en.m
                                     : 1.0 / (double)en.m;
            for (int k = 0; k < d; ++k) vh[k] += wi * elem(V, dt, (ub + i) * d + k);
          }
          for (int k = 0; k < d; ++k) kbar[k] /= (double)en.m;
          const int64_t prep = en.a + (en.m - 1) / 2;
          rope.apply(kbar.data(), prep, 1.0, kh.data());
          for (int k = 0; k < d; ++k) {
            store(Kp, dt, e * d + k, kh[k]);
            store(Vp, dt, e * d + k, vh[k]);
          }
          lnmu[e] = (float)std::log(mu);
          pos[e] = (int32_t)prep;
        }
        ++e;
      }
    }
  }
}

// ------------------------------------------------------------------ O8 decode
// GraceKV page, '05 Physical cache packing' and 'Inside one cache entry';
// DistillCache paper, Sec. 3.1.3: per (s, l, h, g), z_e = c <q, k_e> + ln mu_e
// over the segment and the appended tokens 0..t (mu 1), o = softmax(z) V;
// x[s] = sum over layers (in order) of the concatenated heads, stored fp32.
extern "C" void ko_decode_step(int32_t S, int32_t Ly, int32_t H, int32_t G, int32_t d, int32_t dtype,
                               const void* Kc, const void* Vc, const float* lnmu, const int64_t* seg_off,
                               const int32_t* seg_len, const void* Kd, const void* Vd, int32_t T_dec, int32_t t,
                               const void* Qd_t, float* x) {
  const double c = 1.0 / std::sqrt((double)d);
  const int64_t units = (int64_t)S * Ly * H;
  vector<double> o((size_t)(units * G * d), 0.0);
#pragma omp parallel
  {
    vector<double> q(d), kr(d), z;
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
      const int s = (int)(u / (Ly * H)), l = (int)(u / H % Ly), h = (int)(u % H);
      const int64_t off = seg_off[u], n = seg_len[u], ne = n + t + 1;
      z.resize((size_t)ne);
      for (int g = 0; g < G; ++g) {
        const int64_t qrow = (((int64_t)s * Ly + l) * H * G + (int64_t)h * G + g) * d;
        for (int k = 0; k < d; ++k) q[k] = elem(Qd_t, dtype, qrow + k);
        double m = -std::numeric_limits<double>::infinity();
        for (int64_t e = 0; e < ne; ++e) {
          const int64_t r = e < n ? off + e : (((int64_t)l * H + h) * S + s) * T_dec + (e - n);
          const void* src = e < n ? Kc : Kd;
          for (int k = 0; k < d; ++k) kr[k] = elem(src, dtype, r * d + k);
          z[e] = c * dot(q.data(), kr.data(), d) + (e < n && lnmu ? (double)lnmu[off + e] : 0.0);
          m = std::max(m, z[e]);
        }
        double sum = 0.0;
        for (int64_t e = 0; e < ne; ++e) sum += std::exp(z[e] - m);
        const double lse = m + std::log(sum);
        double* ou = &o[(size_t)((u * G + g) * d)];
        for (int64_t e = 0; e < ne; ++e) {
          const double pr = std::exp(z[e] - lse);
          const int64_t r = e < n ? off + e : (((int64_t)l * H + h) * S + s) * T_dec + (e - n);
          const void* src = e < n ? Vc : Vd;
          for (int k = 0; k < d; ++k) ou[k] += pr * elem(src, dtype, r * d + k);
        }
      }
    }
  }
  const int64_t HGd = (int64_t)H * G * d;
  for (int s = 0; s < S; ++s)
    for (int64_t k = 0; k < HGd; ++k) {
      double acc = 0.0;
      for (int l = 0; l < Ly; ++l) acc += o[(size_t)((((int64_t)s * Ly + l) * H) * G * d + k)];
      x[(int64_t)s * HGd + k] = (float)acc;
    }
}

// ------------------------------------------------------------------ O9 KL
// DistillCache paper, Sec. 3.1.4: KL(P || P^) of the next-token
// distributions. x^ = x / sqrt(mean x^2 + 1e-6) rounded to W's dtype (through
// fp32), y = x^ W^T, KL = sum P (y - y^) - lse(y) + lse(y^).
extern "C" void ko_kl_rows(int64_t n, int32_t dm, int32_t vocab, const float* x_full, const float* x_comp,
                           const void* W, int32_t w_dtype, float* kl) {
  vector<double> Wd((size_t)vocab * dm);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)vocab * dm; ++i) Wd[(size_t)i] = elem(W, w_dtype, i);
  for (int64_t r = 0; r < n; ++r) {
    vector<double> xh[2];
    for (int side = 0; side < 2; ++side) {
      const float* x = (side ? x_comp : x_full) + r * dm;
      double ss = 0.0;
      for (int k = 0; k < dm; ++k) ss += (double)x[k] * (double)x[k];
      const double rs = 1.0 / std::sqrt(ss / dm + 1e-6);
      xh[side].resize((size_t)dm);
      for (int k = 0; k < dm; ++k) {
        const double v = (double)x[k] * rs;
        xh[side][k] = w_dtype == 1 ? bf16_to_double(double_to_bf16(v)) : (double)(float)v;
      }
    }
    vector<double> y((size_t)vocab), yh((size_t)vocab);
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < vocab; ++v) {
      y[v] = dot(xh[0].data(), &Wd[(size_t)(v * dm)], dm);
      yh[v] = dot(xh[1].data(), &Wd[(size_t)(v * dm)], dm);
    }
    double my = -std::numeric_limits<double>::infinity(), myh = my;
    for (int64_t v = 0; v < vocab; ++v) {
      my = std::max(my, y[v]);
      myh = std::max(myh, yh[v]);
    }
    double sy = 0.0, syh = 0.0;
    for (int64_t v = 0; v < vocab; ++v) {
      sy += std::exp(y[v] - my);
      syh += std::exp(yh[v] - myh);
    }
    const double ly = my + std::log(sy), lyh = myh + std::log(syh);
    double acc = 0.0;
    for (int64_t v = 0; v < vocab; ++v) acc += std::exp(y[v] - ly) * (y[v] - yh[v]);
    kl[r] = (float)(acc - ly + lyh);
  }
}
