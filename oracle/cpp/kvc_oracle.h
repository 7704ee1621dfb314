/*
 * kvc_oracle -- plain CPU oracle of the KV-cache compression path, in C++17
 * with OpenMP over (sequence, layer, KV head) units, fp64 arithmetic.
 *
 * TEST INFRASTRUCTURE ONLY. It restates, step by step, what the compression
 * path computes (GraceKV project page: probe relevance, value flow,
 * curvature-guided slots, prototype trees, singleton floor, global Add/Split
 * auction, physical packing; DistillCache paper: features, top-B, decode over
 * the pruned cache, KL between next-token distributions). It shares no code,
 * header or constant with the GPU library; only the tests, the smoke check
 * and the benchmark's CPU-baseline leg load it. The Python oracle in the same
 * directory tree follows the same readings; this library is pinned against
 * it (tests/test_oracle_cpp.py) and against the same closed forms.
 *
 * Every array is host memory in the layouts of the GPU library's C ABI:
 *   K, V    [Ly][H][T][d]        Qp [S][Ly][H*G][P][d]    Qctx [Ly][H*G][T][d]
 *   per-token [Ly][H][T]          tree arrays [Ly][H][2T]  (slot at global
 *   token t0 of unit (l,h): node j at (l*H+h)*2T + 2*t0 + j, op 0 = Add,
 *   op 1+j = Split(node j); node_topo records: bits 0-7 first token - t0,
 *   8-15 length - 1, 16-23 parent + 1, 24-31 next sibling, 0xFFFFFFFF past
 *   the slot's last node; a NULL node_topo means midpoint trees)
 * dtype 1 = bf16 bits (uint16), 0 = fp32. Outputs that feed a decision
 * downstream (relevance, sensitivity, utilities) are rounded to fp32, as the
 * stages hand them over.
 */
#ifndef KVC_ORACLE_H_
#define KVC_ORACLE_H_
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ko_shape {
  int32_t S, Ly, H, G, d, P;
  int32_t dtype;          /* 1 bf16, 0 fp32 (K, V, queries, hidden) */
  int64_t T;
  const int64_t* cu;      /* [S+1] */
} ko_shape;

typedef struct ko_params {
  float budget_ratio;
  int32_t budget_min, prompt_exact, recent_exact, suffix_exact;
  int32_t n_hops, n_seeds;
  float hop_weight;
  int32_t n_dprobe;
  float w_attn, w_value, value_base, floor_frac;
  int32_t token_mode, slot_len, slot_min, slot_max, slot_target;
  float lambda_len, lambda_curv, lambda_surp;
  double rope_base;
  int32_t split_mode;     /* 0 midpoint trees; 1 curvature-candidate cuts + salient three-way splits */
} ko_params;

/* threads the OpenMP loops use */
int ko_threads(void);

/* regions of a sequence of length L: out[4] = prompt_end, comp_start,
 * comp_end, suffix_start */
void ko_regions(int64_t L, const ko_params* p, int64_t* out);
/* per-sequence budget, allocatable budget and floor cap [S] each */
void ko_budgets(const ko_shape* sh, const ko_params* p, int64_t* B, int64_t* alloc, int64_t* floor_cap);

/* probe attention and features (r0, feats nullable, lse, ent, sens) */
void ko_probe_scores(const ko_shape* sh, const void* K, const void* V, const void* Qp, float* r0, float* feats,
                     float* lse, float* ent, float* sens);
/* two-hop value flow over the seeds' causal prefill rows; seeds nullable
 * [hops][S][Ly][H][n_seeds] */
void ko_propagate(const ko_shape* sh, const ko_params* p, const void* K, const void* Qctx, const float* r0,
                  float* rel, int32_t* seeds);
/* quantized slot costs [T][slot_max-slot_min+1] and cut bonuses [T];
 * hidden [n_depth][T][dim] (same dtype as the shape); surprisal [T] fp32 nullable */
void ko_slot_costs(const ko_shape* sh, const ko_params* p, const void* hidden, int32_t dim, int32_t n_depth,
                   const float* surprisal, int64_t* cost_q, int64_t* cut_q);
/* slots of every sequence: slot_start [S][stride+1], n_slots [S]; DP when
 * slot_len == 0 (cost_q/cut_q from ko_slot_costs), fixed lengths otherwise */
void ko_slots(const ko_shape* sh, const ko_params* p, const int64_t* cost_q, const int64_t* cut_q, int32_t stride,
              int32_t* slot_start, int32_t* n_slots);
/* prototype trees: node_rel/node_D/node_mu/op_util f32, op_cost u8, node_topo
 * u32 (nullable), all [Ly][H][2T]; cut_q [T] (nullable) the partition's cut
 * scores for split_mode 1; topo_in (nullable) node records whose tree shapes
 * are used instead of deciding them */
void ko_build_trees(const ko_shape* sh, const ko_params* p, const void* K, const void* V, const void* Qp,
                    const float* lse, const float* rel, const float* sens, const int32_t* slot_start,
                    const int32_t* n_slots, int32_t stride, const int64_t* cut_q, const uint32_t* topo_in,
                    float* node_rel, float* node_D, float* node_mu, float* op_util, uint8_t* op_cost,
                    uint32_t* node_topo);
/* singleton floor: taken [Ly][H][2T] u8 (floor ops), spent [S] */
void ko_floor(const ko_shape* sh, const ko_params* p, const float* rel, const float* sens, const uint8_t* op_cost,
              const uint32_t* node_topo, const int32_t* slot_start, const int32_t* n_slots, int32_t stride,
              uint8_t* taken, int64_t* spent);
/* best-first auction after the floor: taken and spent are updated in place */
void ko_auction(const ko_shape* sh, const ko_params* p, const float* op_util, const uint8_t* op_cost,
                const uint32_t* node_topo, const int32_t* slot_start, const int32_t* n_slots, int32_t stride,
                uint8_t* taken, int64_t* spent);
/* token mode: taken [Ly][H][T], spent [S] */
void ko_token_topk(const ko_shape* sh, const ko_params* p, const float* rel, uint8_t* taken, int64_t* spent);
/* entries pack writes (to size its outputs) */
int64_t ko_pack_count(const ko_shape* sh, const ko_params* p, const uint8_t* taken, const uint32_t* node_topo,
                      const int32_t* slot_start, const int32_t* n_slots, int32_t stride);
/* the packed cache: Kp, Vp [N][d] in the cache dtype, lnmu [N] f32, pos [N]
 * i32, seg_off/seg_len [S][Ly][H] */
void ko_pack(const ko_shape* sh, const ko_params* p, const void* K, const void* V, const float* rel,
             const float* node_rel, const float* node_mu, const uint32_t* node_topo, const uint8_t* taken,
             const int32_t* slot_start,
             const int32_t* n_slots, int32_t stride, void* Kp, void* Vp, float* lnmu, int32_t* pos,
             int64_t* seg_off, int32_t* seg_len);
/* one decode step t over a ragged cache (K/V rows in `dtype`, lnmu nullable)
 * plus the appended tokens 0..t (Kd, Vd [Ly][H][S][T_dec][d]); Qd_t
 * [S][Ly][H*G][d]; x [S][H*G*d] f32 (sum over layers) */
void ko_decode_step(int32_t S, int32_t Ly, int32_t H, int32_t G, int32_t d, int32_t dtype, const void* Kc,
                    const void* Vc, const float* lnmu, const int64_t* seg_off, const int32_t* seg_len,
                    const void* Kd, const void* Vd, int32_t T_dec, int32_t t, const void* Qd_t, float* x);
/* KL(full || compressed) per row: x_full, x_comp [n][dm] f32, W [vocab][dm]
 * (w_dtype 1 bf16 bits, 0 f32); kl [n] f32 */
void ko_kl_rows(int64_t n, int32_t dm, int32_t vocab, const float* x_full, const float* x_comp, const void* W,
                int32_t w_dtype, float* kl);

#ifdef __cplusplus
}
#endif
#endif
