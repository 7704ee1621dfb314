// Host-side ABI pieces: status strings, defaults, validation, budgets,
// capacities, workspace dispatch, RoPE tables and the full-cache view.
#include <cmath>
#include <cstring>
#include <string>

#include "kvc_internal.h"

namespace kvc {

static thread_local std::string g_last_error;

int set_error(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int validate_shape(const kvc_shape* s) {
  KVC_REQUIRE(s != nullptr, KVC_E_INVAL, "shape is NULL");
  KVC_REQUIRE(s->n_seq >= 1 && s->n_layers >= 1 && s->n_kv_heads >= 1, KVC_E_SHAPE,
              "n_seq, n_layers and n_kv_heads must be >= 1");
  KVC_REQUIRE(s->group >= 1 && s->group <= 8, KVC_E_SHAPE, "group must be in [1, 8]");
  KVC_REQUIRE(s->head_dim == 64 || s->head_dim == 128, KVC_E_SHAPE, "head_dim must be 64 or 128");
  KVC_REQUIRE(s->dtype == KVC_BF16 || s->dtype == KVC_F32, KVC_E_DTYPE, "dtype must be KVC_BF16 or KVC_F32");
  KVC_REQUIRE(s->cu_seqlens != nullptr && s->cu_seqlens_d != nullptr, KVC_E_INVAL,
              "cu_seqlens (host) and cu_seqlens_d (device) are required");
  KVC_REQUIRE(s->cu_seqlens[0] == 0, KVC_E_SHAPE, "cu_seqlens[0] must be 0");
  for (int i = 0; i < s->n_seq; ++i)
    KVC_REQUIRE(s->cu_seqlens[i + 1] >= s->cu_seqlens[i], KVC_E_SHAPE, "cu_seqlens must be nondecreasing");
  KVC_REQUIRE(s->cu_seqlens[s->n_seq] == s->total_tokens, KVC_E_SHAPE, "cu_seqlens[S] must equal total_tokens");
  // op ids are 32-bit: (l*H+h)*2T + 2t + j must fit
  KVC_REQUIRE((int64_t)s->n_layers * s->n_kv_heads * 2 * s->total_tokens < (int64_t)0xffffffffLL,
              KVC_E_SHAPE, "Ly*H*2T must be below 2^32");
  return KVC_OK;
}

int validate_params(const kvc_shape* s, const kvc_params* p) {
  KVC_REQUIRE(p != nullptr, KVC_E_INVAL, "params is NULL");
  KVC_REQUIRE(p->budget_ratio >= 0.f && std::isfinite(p->budget_ratio), KVC_E_INVAL, "budget_ratio must be >= 0");
  KVC_REQUIRE(p->budget_min >= 0, KVC_E_INVAL, "budget_min must be >= 0");
  KVC_REQUIRE(p->prompt_exact >= 0 && p->recent_exact >= 0 && p->suffix_exact >= 0, KVC_E_INVAL,
              "exact region sizes must be >= 0");
  KVC_REQUIRE(p->n_probe >= 8 && p->n_probe % 8 == 0, KVC_E_INVAL, "n_probe must be a positive multiple of 8");
  KVC_REQUIRE((int64_t)s->group * p->n_probe <= 256, KVC_E_SHAPE, "group * n_probe must be <= 256");
  KVC_REQUIRE(p->n_hops >= 0 && p->n_hops <= 8, KVC_E_INVAL, "n_hops must be in [0, 8]");
  KVC_REQUIRE(p->n_seeds >= 1 && p->n_seeds <= 64 && (int64_t)p->n_seeds * s->group <= 256, KVC_E_INVAL,
              "n_seeds must be in [1, 64] with n_seeds * group <= 256");
  KVC_REQUIRE(p->n_dprobe >= 1 && p->n_dprobe <= 64, KVC_E_INVAL, "n_dprobe must be in [1, 64]");
  KVC_REQUIRE(p->floor_frac >= 0.f && p->floor_frac <= 1.f, KVC_E_INVAL, "floor_frac must be in [0, 1]");
  KVC_REQUIRE(p->hybrid_frac >= 0.f && p->hybrid_frac <= 1.f, KVC_E_INVAL, "hybrid_frac must be in [0, 1]");
  KVC_REQUIRE(p->hybrid_frac == 0.f || (int64_t)s->n_layers * s->n_kv_heads <= 4096, KVC_E_SHAPE,
              "the head-level hybrid needs n_layers * n_kv_heads <= 4096");
  if (!p->token_mode) {
    KVC_REQUIRE(p->slot_len >= 0 && p->slot_len <= 128, KVC_E_INVAL, "slot_len must be in [0, 128]");
    KVC_REQUIRE(p->slot_min >= 1 && p->slot_min <= p->slot_max && p->slot_max <= 128, KVC_E_INVAL,
                "need 1 <= slot_min <= slot_max <= 128");
    KVC_REQUIRE(p->slot_len > 0 || p->slot_max >= 2 * p->slot_min - 1, KVC_E_INVAL,
                "slot_max must be >= 2*slot_min-1 so every long region can be cut");
    KVC_REQUIRE(p->slot_target >= 1, KVC_E_INVAL, "slot_target must be >= 1");
  }
  KVC_REQUIRE(p->split_mode == 0 || p->split_mode == 1, KVC_E_INVAL, "split_mode must be 0 or 1");
  return KVC_OK;
}

int64_t max_len(const kvc_shape* s) {
  int64_t m = 0;
  for (int i = 0; i < s->n_seq; ++i) {
    int64_t L = s->cu_seqlens[i + 1] - s->cu_seqlens[i];
    if (L > m) m = L;
  }
  return m;
}

}  // namespace kvc

using namespace kvc;

extern "C" const char* kvc_strerror(int st) {
  switch (st) {
    case KVC_OK: return "ok";
    case KVC_E_INVAL: return "invalid argument";
    case KVC_E_SHAPE: return "inconsistent or unsupported shape";
    case KVC_E_DTYPE: return "unsupported dtype";
    case KVC_E_WORKSPACE: return "workspace too small";
    case KVC_E_BUDGET: return "exact regions exceed the budget";
    case KVC_E_HIP: return "HIP launch failed";
    case KVC_E_UNSUPPORTED: return "unsupported";
    default: return "unknown status";
  }
}

extern "C" const char* kvc_last_error(void) { return kvc::g_last_error.c_str(); }

extern "C" void kvc_params_default(kvc_params* p) {
  if (!p) return;
  std::memset(p, 0, sizeof(*p));
  p->budget_ratio = 0.25f;
  p->budget_min = 32;
  p->n_probe = 64;
  p->n_hops = 2;
  p->n_seeds = 32;
  p->hop_weight = 0.3f;
  p->n_dprobe = 64;
  p->w_attn = 0.25f;
  p->w_value = 0.75f;
  p->value_base = 0.1f;
  p->floor_frac = 0.02f;
  p->token_mode = 0;
  p->slot_len = 64;
  p->slot_min = 16;
  p->slot_max = 128;
  p->slot_target = 64;
  p->lambda_len = 1.0f;
  p->lambda_curv = 4.0f;
  p->rope_base = 1e6f;
  p->window = 64;
  p->n_depth = 1;
  p->lambda_surp = 1.0f;
  p->split_mode = 0;
}

extern "C" int kvc_budgets(const kvc_shape* shape, const kvc_params* prm, int64_t* B,
                           int64_t* alloc, int64_t* floor_cap) {
  int st = validate_shape(shape);
  if (st) return st;
  KVC_REQUIRE(prm != nullptr, KVC_E_INVAL, "params is NULL");
  int bad = 0;
  for (int s = 0; s < shape->n_seq; ++s) {
    int64_t L = shape->cu_seqlens[s + 1] - shape->cu_seqlens[s];
    int64_t units = (int64_t)shape->n_layers * shape->n_kv_heads;
    int64_t b = (int64_t)std::floor((double)prm->budget_ratio * (double)(L * units));
    if (b < prm->budget_min) b = prm->budget_min;
    Regions r = regions_of(L, *prm);
    int64_t a = b - (r.ss - r.c1) * units;
    // the floor shares what the units kept whole leave
    int64_t rest = a - hybrid_units_of(a, r.c1 - r.c0, units, *prm) * (r.c1 - r.c0);
    int64_t f = rest > 0 ? (int64_t)std::floor((double)prm->floor_frac * (double)rest) : 0;
    if (B) B[s] = b;
    if (alloc) alloc[s] = a;
    if (floor_cap) floor_cap[s] = f;
    if (a < 0) bad = 1;
  }
  if (bad) return set_error(KVC_E_BUDGET, "a sequence's recent window costs more than its budget");
  return KVC_OK;
}

extern "C" int64_t kvc_pack_capacity(const kvc_shape* shape, const kvc_params* prm) {
  if (validate_shape(shape) || !prm) return -1;
  int64_t units = (int64_t)shape->n_layers * shape->n_kv_heads;
  int64_t tot = 0;
  for (int s = 0; s < shape->n_seq; ++s) {
    int64_t L = shape->cu_seqlens[s + 1] - shape->cu_seqlens[s];
    int64_t b = (int64_t)std::floor((double)prm->budget_ratio * (double)(L * units));
    if (b < prm->budget_min) b = prm->budget_min;
    Regions r = regions_of(L, *prm);
    int64_t comp = (r.c1 - r.c0) * units;
    int64_t a = b - (r.ss - r.c1) * units;
    if (a < 0) a = 0;
    if (a > comp) a = comp;
    tot += a + (r.pe + (L - r.c1)) * units;
  }
  return tot;
}

extern "C" int32_t kvc_slot_stride(const kvc_shape* shape, const kvc_params* prm) {
  if (validate_shape(shape) || !prm) return -1;
  int64_t m = max_len(shape);
  int64_t smin = prm->slot_len > 0 ? prm->slot_len : prm->slot_min;
  if (smin < 1) smin = 1;
  return (int32_t)((m + smin - 1) / smin + 1);
}

extern "C" size_t kvc_workspace_size(const kvc_shape* shape, const kvc_params* prm, int32_t stage) {
  if (validate_shape(shape) || !prm) return 0;
  switch (stage) {
    case KVC_STAGE_SCORE: return ws_score(shape, prm);
    case KVC_STAGE_PROPAGATE: return ws_propagate(shape, prm);
    case KVC_STAGE_PARTITION: return ws_partition(shape, prm);
    case KVC_STAGE_TREES: return ws_trees(shape, prm);
    case KVC_STAGE_AUCTION: return ws_auction(shape, prm);
    case KVC_STAGE_PACK: return ws_pack(shape, prm);
    default: return 0;
  }
}

// ------------------------------------------------------------------ RoPE tables
__global__ void rope_table_kernel(double base, int d, int n_pos, float* cs, float* sn) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int h = d / 2;
  if (i >= (int64_t)n_pos * h) return;
  int64_t p = i / h;
  int j = (int)(i % h);
  double inv = pow(base, -2.0 * (double)j / (double)d);
  double a = (double)p * inv;
  cs[i] = (float)cos(a);
  sn[i] = (float)sin(a);
}

extern "C" int kvc_rope_table(float base, int32_t head_dim, int32_t n_pos, float* cos_out,
                              float* sin_out, hipStream_t stream) {
  KVC_REQUIRE(cos_out && sin_out, KVC_E_INVAL, "rope table outputs are NULL");
  KVC_REQUIRE(head_dim > 0 && head_dim % 2 == 0 && n_pos >= 0 && base > 1.f, KVC_E_INVAL,
              "bad rope table arguments");
  int64_t n = (int64_t)n_pos * (head_dim / 2);
  if (n == 0) return KVC_OK;
  hipLaunchKernelGGL(rope_table_kernel, dim3(kvc_blocks(n, 256)), dim3(256), 0, stream,
                     (double)base, head_dim, n_pos, cos_out, sin_out);
  KVC_LAUNCH_CHECK("rope_table");
  return KVC_OK;
}

// ------------------------------------------------------------------ full-cache view
__global__ void full_view_kernel(const int64_t* cu, int S, int Ly, int H, int64_t T, int64_t* off,
                                 int32_t* len) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= S * Ly * H) return;
  int s = i / (Ly * H);
  int lh = i % (Ly * H);
  off[i] = (int64_t)lh * T + cu[s];
  len[i] = (int32_t)(cu[s + 1] - cu[s]);
}

extern "C" int kvc_full_view(const kvc_shape* shape, int64_t* seg_off, int32_t* seg_len,
                             hipStream_t stream) {
  int st = validate_shape(shape);
  if (st) return st;
  KVC_REQUIRE(seg_off && seg_len, KVC_E_INVAL, "seg_off/seg_len are NULL");
  int n = shape->n_seq * shape->n_layers * shape->n_kv_heads;
  hipLaunchKernelGGL(full_view_kernel, dim3(kvc_blocks(n, 256)), dim3(256), 0, stream,
                     shape->cu_seqlens_d, shape->n_seq, shape->n_layers, shape->n_kv_heads,
                     shape->total_tokens, seg_off, seg_len);
  KVC_LAUNCH_CHECK("full_view");
  return KVC_OK;
}
