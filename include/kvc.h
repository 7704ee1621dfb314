/*
 * libkvc -- probe-scored KV-cache compression and decode on MI355X (gfx950).
 *
 * C ABI. Every entry point takes plain host/device pointers and sizes and is
 * asynchronous on the caller's HIP stream: arguments are validated on the host
 * before anything is launched, the library never synchronizes the device, and
 * it keeps no device memory or state between calls (one exception:
 * kvc_decode_attn_static's per-GPU scratch array). The caller owns every
 * buffer, including a scratch workspace whose size the matching
 * kvc_*_workspace query returns. On an error return nothing was launched,
 * except KVC_E_HIP (a launch failed: outputs are undefined). kvc_last_error()
 * gives a thread-local message for the last failing call.
 *
 * The operations follow three pages: the DistillCache paper (KL-guided
 * eviction), the KVLearn README (keep/evict decision library) and the GraceKV
 * project page (global Add/Split auction over prototype trees). Each entry
 * point cites the passage that defines what it computes.
 *
 * Shapes: S sequences of lengths L_s (tokens of all sequences concatenated,
 * T = sum L_s, offsets cu_seqlens[S+1]), Ly layers, H KV heads, G query heads
 * per KV head, d head dim (64 or 128), P probe queries per query head.
 * Common layouts (row-major, innermost last):
 *   K, V       [Ly][H][T][d]            cached keys (post-RoPE) and values
 *   Qprobe     [S][Ly][H*G][P][d]       probe queries (post-RoPE)
 *   Qctx       [Ly][H*G][T][d]          prefill queries of the cached tokens
 *   rel-like   [Ly][H][T]  fp32         one value per cached entry
 *   tree arrays [Ly][H][2T]             the slot starting at global token t0
 *                                       of unit (l,h) owns indices
 *                                       (l*H+h)*2T + 2*t0 + [0, 2n); node j of
 *                                       its tree (pre-order, j < 2n-1) at +j;
 *                                       op 0 = Add(slot), op 1+j = Split(node j)
 * Keys, queries and values are KVC_BF16 (or KVC_F32 end to end for small
 * float32 workloads); all accumulation is fp32.
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kvc_status {
  KVC_OK = 0,
  KVC_E_INVAL = -1,        /* NULL pointer or out-of-range parameter */
  KVC_E_SHAPE = -2,        /* inconsistent or unsupported sizes */
  KVC_E_DTYPE = -3,        /* unsupported dtype */
  KVC_E_WORKSPACE = -4,    /* workspace smaller than the query returned */
  KVC_E_BUDGET = -5,       /* exact regions alone exceed a sequence's budget */
  KVC_E_HIP = -6,          /* a HIP launch failed */
  KVC_E_UNSUPPORTED = -7
};

enum kvc_dtype { KVC_F32 = 0, KVC_BF16 = 1 };

typedef struct kvc_shape {
  int32_t n_seq;                /* S */
  int32_t n_layers;             /* Ly */
  int32_t n_kv_heads;           /* H */
  int32_t group;                /* G (1..8) */
  int32_t head_dim;             /* d: 64 or 128 */
  int32_t dtype;                /* kvc_dtype of K/V/queries */
  int64_t total_tokens;         /* T */
  const int64_t* cu_seqlens;    /* HOST [S+1], cu[0] = 0, nondecreasing */
  const int64_t* cu_seqlens_d;  /* DEVICE copy of the same [S+1] */
} kvc_shape;

typedef struct kvc_params {
  float budget_ratio;      /* r: entries kept per sequence = max(floor(r*L*Ly*H), budget_min) */
  int32_t budget_min;      /* B_min = 32 (DistillCache, Algorithm 1) */
  int32_t prompt_exact;    /* leading tokens kept exactly, outside the budget */
  int32_t recent_exact;    /* tokens before the suffix kept exactly, charged to the budget */
  int32_t suffix_exact;    /* trailing tokens kept exactly, outside the budget */
  int32_t n_probe;         /* P probe queries per query head (G*P <= 256) */
  int32_t n_hops;          /* propagation hops (GraceKV: 2) */
  int32_t n_seeds;         /* seeds per hop per (l,h) (<= 64) */
  float hop_weight;        /* w = 0.3 (GraceKV technical details) */
  int32_t n_dprobe;        /* probe rows used by the distortion (<= 64) */
  float w_attn, w_value;   /* 0.25 : 0.75 (GraceKV technical details) */
  float value_base;        /* uniform share of prototype values, 0.1 */
  float floor_frac;        /* singleton-floor cap as a fraction of the allocatable budget */
  int32_t token_mode;      /* 1: token-level top-B only (no slots, trees or floor) */
  int32_t slot_len;        /* fixed slot length; 0: slots from kvc_partition's DP */
  int32_t slot_min, slot_max, slot_target;  /* 16, 128, 64 (GraceKV technical details) */
  float lambda_len;        /* DP slot-length penalty weight */
  float lambda_curv;       /* DP turning-score reward weight */
  float rope_base;         /* RoPE theta base */
  float hybrid_frac;       /* head-level hybrid: share of (l, h) units kept whole (0 = off) */
  int32_t window;          /* step-wise eviction: recent queries behind the features (w = 64) */
  int32_t n_depth;         /* sampled depths of the hidden-state trajectory (1..4) */
  float lambda_surp;       /* DP weight of surprisal / its sequence maximum at a cut */
  int32_t split_mode;      /* trees: 0 midpoint binary splits; 1 curvature-candidate cuts and
                              salient three-way splits (see kvc_build_trees_ex) */
} kvc_params;

typedef struct kvc_trees {
  float* node_rel;         /* [Ly][H][2T] node relevance (sum of its tokens' r) */
  float* node_D;           /* [Ly][H][2T] node distortion in [0, 1] */
  float* node_mu;          /* [Ly][H][2T] node multiplicity >= 1 */
  float* op_util;          /* [Ly][H][2T] utility per new entry of each op */
  uint8_t* op_cost;        /* [Ly][H][2T] entries an op adds (0 = no such op) */
  uint32_t* node_topo;     /* [Ly][H][2T] node records (nullable when split_mode = 0, where the
                              trees are the implicit midpoint trees; required when split_mode = 1):
                              node j of the slot at global token t0 of unit (l,h) at
                              (l*H+h)*2T + 2*t0 + j holds bits 0-7 its first token - t0, 8-15 its
                              length - 1, 16-23 its parent's index + 1 (0: the root), 24-31 its
                              next sibling's index (0: none); 0xFFFFFFFF past the slot's last node.
                              Nodes are in pre-order, children in position order. */
} kvc_trees;

typedef struct kvc_ragged {
  void* K;                 /* [capacity][d] packed keys (cache dtype) */
  void* V;                 /* [capacity][d] packed values */
  float* lnmu;             /* [capacity] ln(multiplicity), or NULL = all 0 */
  int32_t* pos;            /* [capacity] sequence position of each entry (may be NULL for decode) */
  int64_t* seg_off;        /* [S][Ly][H] first entry of each (s, l, h) segment */
  int32_t* seg_len;        /* [S][Ly][H] entries in each segment */
  int32_t n_seq, n_layers, n_kv_heads, head_dim, dtype;
  int32_t max_seg;         /* host upper bound on any seg_len (>= 0; informational) */
  int64_t capacity;        /* entries the K/V/lnmu/pos buffers hold */
} kvc_ragged;

/* ------------------------------------------------------------------ misc */
const char* kvc_strerror(int status);
const char* kvc_last_error(void);
/* Defaults of every parameter (values the pages state where they state one). */
void kvc_params_default(kvc_params* p);
/* Per-sequence budget (host arithmetic): B_s, the allocatable part (B_s minus
 * the recent window's Ly*H*n entries) and the floor cap floor(frac*rest),
 * rest = alloc minus the entries of the units the head-level hybrid keeps
 * whole (rest = alloc when hybrid_frac = 0).
 * Returns KVC_E_BUDGET if any allocatable budget is negative. Any output
 * pointer may be NULL. */
int kvc_budgets(const kvc_shape* shape, const kvc_params* prm, int64_t* B, int64_t* alloc,
                int64_t* floor_cap);
/* Upper bound on entries kvc_pack writes (size of the ragged buffers). */
int64_t kvc_pack_capacity(const kvc_shape* shape, const kvc_params* prm);
/* Slots per sequence the slot_start rows hold: slot_start is [S][stride+1]. */
int32_t kvc_slot_stride(const kvc_shape* shape, const kvc_params* prm);

enum kvc_stage {
  KVC_STAGE_SCORE = 0, KVC_STAGE_PROPAGATE, KVC_STAGE_PARTITION, KVC_STAGE_TREES,
  KVC_STAGE_AUCTION, KVC_STAGE_PACK
};
/* Workspace bytes for a compression stage (0 is a valid answer). */
size_t kvc_workspace_size(const kvc_shape* shape, const kvc_params* prm, int32_t stage);

/* RoPE tables cos/sin [n_pos][d/2] in fp32, computed in fp64 on the device:
 * theta_j(pos) = pos * base^(-2j/d), rotate-half pairing (j, j + d/2). */
int kvc_rope_table(float base, int32_t head_dim, int32_t n_pos, float* cos_out, float* sin_out,
                   hipStream_t stream);

/* ------------------------------------------------------------------ A1/A2
 * kvc_score: probe attention and per-token features.
 * GraceKV page, '03 Bottom-up value flow' (direct relevance from question and
 * sequence-tail probes); DistillCache paper, Sec. 3.1.1 (features: attention
 * mass, value norm, variance across heads, attention-weighted entropy,
 * normalized position).
 * For every (s, l, h) and probe row rho = g*P + p (rows of the KV group):
 *   a_rho,i = softmax_i(<q_rho, k_i>/sqrt(d)) over all L_s keys,
 *   lse_rho, H_rho = -sum_i a log a.
 * Outputs (device): rel0 [Ly][H][T] = sum_rho a_rho,i;
 *   feats [5][Ly][H][T] = (rel0, ||v_i||, var_g(sum_p a_(g,p),i),
 *   sum_rho a H_rho / rel0, i/(L_s-1));
 *   probe_lse, probe_ent [S][Ly][H*G][P]; head_sens [S][Ly][H] =
 *   sum_i rel0_i ||v_i|| / sum_i rel0_i. feats may be NULL. */
int kvc_score(const kvc_shape* shape, const kvc_params* prm, const void* K, const void* V,
              const void* Qprobe, float* rel0, float* feats, float* probe_lse, float* probe_ent,
              float* head_sens, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ A3
 * kvc_propagate: token-to-token propagation of relevance.
 * GraceKV page, '03 Bottom-up value flow' and technical details (two graph
 * hops with weight 0.3 recover indirect evidence). Per (s, l, h), starting
 * from delta_0 = rel0, hop t takes the n_seeds tokens with the largest
 * delta_{t-1} (ties to the lower index) and
 *   delta_t(i) = w * sum_seeds delta_{t-1}(j) * mean_g softmax_{i<=j}(<q_jg,k_i>/sqrt d)
 * with the prefill queries Qctx; rel = rel0 + delta_1 + ... (device, fp32).
 * seeds (nullable) [n_hops][S][Ly][H][n_seeds] int32: seed token positions,
 * ascending, -1 padded. */
int kvc_propagate(const kvc_shape* shape, const kvc_params* prm, const void* K, const void* Qctx,
                  const float* rel0, float* rel, int32_t* seeds, void* ws, size_t ws_bytes,
                  hipStream_t stream);

/* Dense rollout: the same hops with every token a seed (the full L x L
 * causal prefill attention graph, GQA-averaged), so relevance reaches every
 * token any earlier-relevant token attends, with no seed cut-off:
 *   delta_t = w * A_hat^T delta_{t-1},  rel = rel0 + delta_1 + ...
 * (GraceKV page, '03 Bottom-up value flow'; the hop count and weight of
 * prm). The rows run in blocks of min(64, 256/G) positions per (s, l, h),
 * each block one pass over the keys up to its last position; the cost is
 * that of a causal prefill attention per hop. n_seeds is ignored. */
size_t kvc_propagate_dense_workspace(const kvc_shape* shape, const kvc_params* prm);
int kvc_propagate_dense(const kvc_shape* shape, const kvc_params* prm, const void* K, const void* Qctx,
                        const float* rel0, float* rel, void* ws, size_t ws_bytes, hipStream_t stream);

/* The "A r" direction: relevance flows from attended tokens to the tokens
 * attending them. Every token i takes the GQA-mean causal softmax average of
 * the previous increment over its prefix,
 *   delta_t(i) = w * mean_g sum_{j<=i} softmax_j(<q_ig,k_j>/sqrt d) delta_{t-1}(j),
 * rel = rel0 + delta_1 + ... (GraceKV page, '03 Bottom-up value flow', read
 * in the other direction of the attention graph). One causal row pass per
 * hop and row block (the row softmax and the value average in the same
 * pass); n_seeds is ignored. */
size_t kvc_propagate_ar_workspace(const kvc_shape* shape, const kvc_params* prm);
int kvc_propagate_ar(const kvc_shape* shape, const kvc_params* prm, const void* K, const void* Qctx,
                     const float* rel0, float* rel, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ A0
 * kvc_partition: slots of each sequence's compressible region.
 * GraceKV page, '01 Curvature-guided partition' (cut where the normalized
 * hidden-state trajectory turns; a DP also weighs within-slot dispersion and
 * slot length; 16-128 tokens, target 64). With prm->slot_len > 0 the slots
 * are fixed-length (the last one shorter) and hidden is not read.
 * mode 0: compute the quantized DP inputs from hidden [T][hidden_dim] (bf16 or
 *   f32 as shape->dtype) and, if dp_cost_q/dp_cut_q are non-NULL, export them;
 * mode 1: read the DP inputs from dp_cost_q/dp_cut_q instead (hidden unused).
 * dp_cost_q [T][slot_max-slot_min+1] int64: row = global index of a slot's last
 *   token, column = n - slot_min, value = round(cost * 2^20) with
 *   cost = sum ||h^_i - mean||^2 + lambda_len*((n-target)/target)^2;
 * dp_cut_q [T] int64 = round(lambda_curv * turning score * 2^20) of a cut
 *   before that token.
 * Outputs: slot_start [S][stride+1] int32 (sequence positions; slot k is
 *   [slot_start[k], slot_start[k+1])), n_slots [S] int32. */
int kvc_partition(const kvc_shape* shape, const kvc_params* prm, const void* hidden,
                  int32_t hidden_dim, int32_t mode, int64_t* dp_cost_q, int64_t* dp_cut_q,
                  int32_t* slot_start, int32_t* n_slots, void* ws, size_t ws_bytes,
                  hipStream_t stream);
/* Slots from several sampled depths and surprisal (GraceKV page, 'Technical
 * details and default settings': turns stabilized across sampled depths and
 * windows, surprisal a smaller auxiliary boundary signal). hidden is
 * [n_depth][T][hidden_dim] (prm->n_depth); the turning score is the mean over
 * every valid (depth, window) pair, the dispersion the mean over depths, and
 * a cut before token b also earns lambda_surp * surprisal[b] / (largest
 * surprisal of its sequence) when that maximum is positive; surprisal [T]
 * fp32 device, nullable. kvc_partition is this call with surprisal NULL. */
int kvc_partition_ex(const kvc_shape* shape, const kvc_params* prm, const void* hidden,
                     int32_t hidden_dim, const float* surprisal, int32_t mode, int64_t* dp_cost_q,
                     int64_t* dp_cut_q, int32_t* slot_start, int32_t* n_slots, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ A4
 * kvc_build_trees: prototype trees per (s, l, h, slot).
 * GraceKV page, '02 Progressively refinable representation', 'Inside one
 * cache entry', '03 Bottom-up value flow', '04 Top-down budget flow' and the
 * technical details (0.25 : 0.75 distortion). Binary midpoint trees (left
 * child ceil(n/2)); per node: rel = sum of children; mu = max(1, n*rho),
 * rho = ||sum k~|| / sum ||k~|| over unrotated keys; prototype key = RoPE(mean
 * k~, a + floor((n-1)/2)); value = sum ((1-beta) r_i/rel + beta/n) v_i;
 * D = min(1, w_attn*e_A + w_value*e_V) over n_dprobe probe rows;
 * op utilities u = s_lh * gain / cost with gain(Add) = rel_root(1-D_root),
 * gain(Split q) = rel_q D_q - sum_c rel_c D_c. rope_cos/sin from
 * kvc_rope_table (n_pos >= max L_s). Outputs into *out (all [Ly][H][2T]);
 * entries outside slots are left untouched. */
int kvc_build_trees(const kvc_shape* shape, const kvc_params* prm, const void* K, const void* V,
                    const void* Qprobe, const float* probe_lse, const float* rel,
                    const float* head_sens, const float* rope_cos, const float* rope_sin,
                    const int32_t* slot_start, const int32_t* n_slots, kvc_trees* out,
                    void* ws, size_t ws_bytes, hipStream_t stream);
/* kvc_build_trees_ex: the same with the tree shapes of prm->split_mode.
 * GraceKV page, 'Technical details and default settings' (tree construction
 * weighs high-curvature split candidates beside the midpoint and may isolate
 * a salient token in a three-way child set). split_mode 1 decides each node
 * [a, a+n), n >= 2, top-down, before any distortion: with i the first
 * position of the node's largest relevance (fp32), the node splits three ways
 * [a, i), {i}, [i+1, a+n) when n >= 3, its relevance S (a left-to-right
 * float64 sum of the fp32 values) is positive, 2 r_i > S and i lies at least
 * max(floor(n/4), 1) tokens from either end; otherwise at one cut among those
 * leaving both children at least ceil(n/4) tokens: the largest dp_cut_q score
 * (ties: the midpoint, then the nearest cut, then the lower one), or the
 * midpoint when dp_cut_q is NULL. A three-way split costs 2 entries and its
 * utility is s_lh * gain / 2. dp_cut_q: [T] int64 device, the partition's
 * quantized cut scores (cut before that token; kvc_partition exports them),
 * nullable; ignored when split_mode = 0. out->node_topo receives the node
 * records (required when split_mode = 1; when non-NULL with split_mode 0 the
 * midpoint trees' records are written). kvc_build_trees is this call with
 * dp_cut_q NULL. */
int kvc_build_trees_ex(const kvc_shape* shape, const kvc_params* prm, const void* K, const void* V,
                       const void* Qprobe, const float* probe_lse, const float* rel,
                       const float* head_sens, const float* rope_cos, const float* rope_sin,
                       const int32_t* slot_start, const int32_t* n_slots, const int64_t* dp_cut_q,
                       kvc_trees* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ A5/A6
 * kvc_auction: spend each sequence's budget.
 * Tree mode: GraceKV page, 'Exact-information safeguard' (singleton floor:
 * the top leaves by s_lh*r_i, scanned in order, each paying its untaken path,
 * while the floor spend stays <= floor_frac * allocatable budget) and '04
 * Top-down budget flow' (best-first greedy: the exposed op with the highest
 * utility, lower op id on ties, is taken next until the budget is spent; an op
 * that costs more than what is left is discarded with its subtree). With
 * prm->split_mode 1 the trees' node_topo records give the tree shapes.
 * Writes op_taken [Ly][H][2T] uint8 (1 = taken; every other byte of the
 * layout is cleared) and spent [S] int64 (entries bought, floor included);
 * spent_floor [S] (nullable) = floor part.
 * Token mode (prm->token_mode): DistillCache Algorithm 1 (deterministic top-B
 * by score); trees, head_sens, slot arrays may be NULL; op_taken is then
 * [Ly][H][T]: the allocatable budget's top tokens by (rel desc, flat index
 * (l*H+h)*T + t asc). NaN utilities or scores rank below everything.
 * Head-level hybrid (prm->hybrid_frac > 0; DistillCache paper, Appendix E.3:
 * the most important heads keep their full cache, token selection runs in
 * the others, at the same overall budget): per sequence the K units of
 * kvc_hybrid_units keep every compressible token (tree mode: all their real
 * ops taken; token mode: all their tokens) and are paid first; the floor,
 * the auction and the token top-B run over the other units with the
 * allocatable budget minus K*C (C = compressible tokens per unit). spent
 * includes the K*C entries; spent_floor does not. head_sens is then needed
 * in token mode too.
 * Tree mode waits on stream twice, mid-call: after two passes of each of its
 * two radix selects (floor leaves, ops) it reads back how many elements are
 * still in the running (a few bytes) to size the remaining passes. */
int kvc_auction(const kvc_shape* shape, const kvc_params* prm, const kvc_trees* trees,
                const float* rel, const float* head_sens, const int32_t* slot_start,
                const int32_t* n_slots, uint8_t* op_taken, int64_t* spent,
                int64_t* spent_floor, void* ws, size_t ws_bytes, hipStream_t stream);

/* Head-level hybrid units (DistillCache paper, Appendix E.3): writes
 * unit_full [S][Ly][H] uint8 (device), 1 for the K units of sequence s with
 * the largest head_sens[s][l][h] (ties to the lower l*H + h; NaN ranks
 * last), K = min(floor(hybrid_frac * Ly*H), floor(alloc / C)) with alloc the
 * allocatable budget of kvc_budgets and C the compressible tokens per unit
 * (K = 0 when hybrid_frac = 0 or C = 0). Requires Ly*H <= 4096. */
int kvc_hybrid_units(const kvc_shape* shape, const kvc_params* prm, const float* head_sens,
                     uint8_t* unit_full, hipStream_t stream);

/* ------------------------------------------------------------------ A7
 * kvc_pack: write the physical ragged cache.
 * GraceKV page, '05 Physical cache packing': per (l, h) an independently
 * sized segment; an unselected root writes nothing, an internal frontier node
 * its prototype (keys/values rounded to the cache dtype, ln mu, p_rep), a
 * leaf the original K/V bits (ln mu 0, its position). Segments are stored in
 * (l, h, s) order; entries in position order: prompt, slot frontiers (kept
 * tokens in token mode), recent window, suffix. out->capacity must be at
 * least kvc_pack_capacity(); seg_off/seg_len/K/V/lnmu/pos are written. With
 * prm->split_mode 1 the trees' node_topo records give the tree shapes and a
 * taken op adds op_cost entries. */
int kvc_pack(const kvc_shape* shape, const kvc_params* prm, const void* K, const void* V,
             const float* rel, const kvc_trees* trees, const uint8_t* op_taken,
             const int32_t* slot_start, const int32_t* n_slots, const float* rope_cos,
             const float* rope_sin, kvc_ragged* out, void* ws, size_t ws_bytes,
             hipStream_t stream);

/* The uncompressed cache as a ragged view: fills seg_off [S][Ly][H] =
 * (l*H+h)*T + cu[s] and seg_len = L_s (device arrays). */
int kvc_full_view(const kvc_shape* shape, int64_t* seg_off, int32_t* seg_len, hipStream_t stream);

/* ------------------------------------------------------------------ A8
 * kvc_decode_attn: one decode step over a ragged cache plus appended tokens.
 * GraceKV page, '05 Physical cache packing' (decode reads the packed cache;
 * new tokens append with multiplicity one); DistillCache Sec. 3.1.3 (teacher
 * and student caches both append each new pair).
 * For every (s, l, h, g): z_e = <q, k_e>/sqrt(d) + ln mu_e over the segment's
 * entries and the tail tokens 0..t_valid-1 (K_tail/V_tail [Ly][H][S][t_cap][d],
 * ln mu 0); o = softmax(z) V. Q is [S][Ly][H*G][d].
 * x_out[s*x_stride + (h*G+g)*d + j] = sum over l (in order) of o.
 * o_out (nullable) [S][Ly][H*G][d]. Split-K: every segment is cut into
 * near-equal pieces of at most 768 (bf16) or 256 (fp32) entries and the tail
 * tokens into pieces of their own; the workspace (device memory, owned by the
 * caller, size from kvc_decode_workspace for the largest t_cap to be used)
 * holds the plan of the pieces, their partials and the merge counters.
 * Requires sum of seg_len <= capacity and seg_off + seg_len <= capacity.
 * All calls are asynchronous on `stream`; errors are argument checks only
 * (KVC_E_INVAL, KVC_E_SHAPE, KVC_E_DTYPE, KVC_E_UNSUPPORTED, KVC_E_WORKSPACE).
 * kvc_decode_attn plans and runs one step. kvc_decode_plan writes the plan
 * of the cache's segments into ws (it depends on seg_len, seg_off and
 * capacity only); kvc_decode_attn_planned runs a step from the plan in ws,
 * which must have been made for the same segments with the same group and
 * t_cap (steps over one cache then skip the plan's launch). Two calls that
 * share a workspace must not overlap. */
size_t kvc_decode_workspace(const kvc_ragged* cache, int32_t group, int32_t t_cap);
int kvc_decode_attn(const kvc_ragged* cache, const void* K_tail, const void* V_tail,
                    int32_t t_valid, int32_t t_cap, const void* Q, int32_t group, float* x_out,
                    int64_t x_stride, float* o_out, void* ws, size_t ws_bytes,
                    hipStream_t stream);
int kvc_decode_plan(const kvc_ragged* cache, int32_t group, int32_t t_cap, void* ws,
                    size_t ws_bytes, hipStream_t stream);
int kvc_decode_attn_planned(const kvc_ragged* cache, const void* K_tail, const void* V_tail,
                            int32_t t_valid, int32_t t_cap, const void* Q, int32_t group,
                            float* x_out, int64_t x_stride, float* o_out, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* kvc_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments and results as kvc_decode_attn (plan and step in one call)
 * without a workspace: the step's workspace is a 64 MiB array in the
 * library's device code, one copy per GPU, held from the first call on that
 * GPU until the process ends. Returns KVC_E_WORKSPACE (nothing launched) when
 * kvc_decode_workspace(cache, group, t_cap) exceeds kvc_decode_static_limit().
 * Calls on one GPU share that array: calls that overlap on one GPU (two
 * streams, two host threads) race and give undefined results. The stream
 * must belong to the current device. Allocates nothing. */
size_t kvc_decode_static_limit(void);
int kvc_decode_attn_static(const kvc_ragged* cache, const void* K_tail, const void* V_tail,
                           int32_t t_valid, int32_t t_cap, const void* Q, int32_t group,
                           float* x_out, int64_t x_stride, float* o_out, hipStream_t stream);

/* ------------------------------------------------------------------ A9
 * kvc_kl: per-row KL(full || compressed) through a vocab projection.
 * DistillCache paper, Sec. 3.1.4 (reward = -KL(P_t || P^_t) between the full-
 * and pruned-cache next-token distributions, with standard stabilization).
 * x^ = x / sqrt(mean(x^2) + 1e-6) rounded to W's dtype; y = x^ W^T with
 * W [vocab][d_model] (KVC_BF16 or KVC_F32); kl[p] = sum_v P_v (y_v - y^_v)
 * - lse(y) + lse(y^), P = softmax(y) of the full row. x_full, x_comp are
 * [n_pairs][d_model] fp32. The logits never reach memory. */
size_t kvc_kl_workspace(int64_t n_pairs, int32_t d_model, int32_t vocab, int32_t w_dtype);
int kvc_kl(int64_t n_pairs, int32_t d_model, int32_t vocab, const float* x_full,
           const float* x_comp, const void* W, int32_t w_dtype, float* kl_out, void* ws,
           size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ step-wise eviction
 * DistillCache paper, Sec. 3.1.1 (per-token state: attention mass, value
 * norm, variance across heads, attention-weighted entropy of the recent
 * queries, position), Sec. 3.1.2 (deterministic top-B by the policy score)
 * and Algorithm 1 (after every decode step the new pair is appended, the
 * cache is scored and pruned to B = max(floor(r * n_seen), B_min), n_seen
 * the tokens seen so far: L before the first step, L + t + 1 after step t).
 * Features of a cached token, over all layers, query heads and the w window
 * queries (each attends the whole current cache): mean attention mass,
 * mean value norm over (l, h), population variance over the Ly*H*G query
 * heads of the window-mean mass, sum a*H(a) / sum a, position /
 * max(n_seen - 1, 1). Score: Linear(5,128) -> LayerNorm -> ReLU ->
 * Linear(128,128) -> LayerNorm -> ReLU -> Linear(128,1), LayerNorm eps 1e-5.
 * Kept: the top-B by (fp32 score desc, position asc); the same tokens leave
 * every (l, h). No region is protected. Window size prm->window (multiple of
 * 8, group * window <= 256, every sequence at least window tokens long). */
typedef struct kvc_policy {
  const float* w1;         /* [128][5] */
  const float* b1;         /* [128] */
  const float* g1;         /* [128] LayerNorm scale */
  const float* be1;        /* [128] LayerNorm shift */
  const float* w2;         /* [128][128] */
  const float* b2, *g2, *be2;  /* [128] each */
  const float* w3;         /* [128] */
  const float* b3;         /* [1] */
} kvc_policy;

typedef struct kvc_student {
  void* K;                 /* [Ly][H][cap_total][d] kept keys (cache dtype), slot order */
  void* V;                 /* [Ly][H][cap_total][d] */
  int32_t* pos;            /* [cap_total] sequence position of each slot's token */
  void* Qwin;              /* [S][Ly][H*G][window][d] window queries (ring, queries dtype) */
  int64_t* seg_off;        /* DEVICE [S][Ly][H] ragged view of the occupied slots (for kvc_decode_attn) */
  int32_t* seg_len;        /* DEVICE [S][Ly][H] */
  const int64_t* seq_off;  /* HOST [S] first slot of sequence s (regions must not overlap) */
  const int32_t* seq_cap;  /* HOST [S] slots of sequence s (kvc_step_capacity) */
  int32_t* seq_len;        /* HOST [S] occupied slots; the calls below update it */
  int64_t cap_total;       /* slots per (l, h) */
} kvc_student;

/* Slots each sequence needs for t_steps decode steps: the largest cache
 * before a prune, min(L + t_steps, max(floor(r (L + t_steps)), B_min) + 1). */
int kvc_step_capacity(const kvc_shape* shape, const kvc_params* prm, int32_t t_steps, int32_t* seq_cap);
size_t kvc_step_workspace(const kvc_shape* shape, const kvc_params* prm, int64_t cap_total);
/* Fill the window with the last `window` prefill queries of every sequence
 * (Qctx [Ly][H*G][T][d]), score the prefill cache (K, V [Ly][H][T][d]), keep
 * the top-B of each sequence and write them to the student in position
 * order; sets seq_len and the ragged view. feats_out [5][T] and scores_out
 * [T] (fp32, nullable) receive the features and scores. */
int kvc_step_init(const kvc_shape* shape, const kvc_params* prm, const void* K, const void* V,
                  const void* Qctx, const kvc_policy* policy, kvc_student* st, float* feats_out,
                  float* scores_out, void* ws, size_t ws_bytes, hipStream_t stream);
/* Step t: append decode token t of every sequence (K_tail/V_tail
 * [Ly][H][S][t_cap][d], position L_s + t) to the student, replace the
 * oldest window query with Q_t ([S][Ly][H*G][d]) and refresh the ragged
 * view; decoding q_t then reads the student through kvc_decode_attn with
 * t_valid = 0. KVC_E_SHAPE if a sequence has no free slot. */
int kvc_step_append(const kvc_shape* shape, const kvc_params* prm, kvc_student* st, const void* K_tail,
                    const void* V_tail, const void* Q_t, int32_t t, int32_t t_cap, hipStream_t stream);
/* Step t: score the student's tokens with the window (n_seen = L + t + 1),
 * keep the top-B of each sequence; an evicted slot below the new length is
 * refilled by a kept token from the slots past it. feats_out [5][cap_total]
 * and scores_out [cap_total] (slot order, nullable). */
int kvc_step_prune(const kvc_shape* shape, const kvc_params* prm, kvc_student* st, int32_t t,
                   const kvc_policy* policy, float* feats_out, float* scores_out, void* ws,
                   size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H_ */
