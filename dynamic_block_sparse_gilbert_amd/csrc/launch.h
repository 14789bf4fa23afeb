// Internal launch interface between the C ABI layer (api.cpp) and the kernel
// translation units.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dbs {

struct ReorderArgs {
  const void* x;        // reorder: source [B, N, Hh, d] strided
  void* y;              // reorder: destination; inverse: source (rows)
  void* x_out;          // inverse: destination [B, N, Hh, d] strided
  const void* x2;       // reorder_kv: V source (same strides as x, which is K)
  void* y2;             // reorder_kv: V destination (tiles-transposed); y is K (rows)
  int64_t sb, sn, sh;
  const int32_t* perm;
  int perm_h_stride;    // 0 (shared) or N (per head)
  int B, Hh, N, Npad, d, b;
  bool x_f32, y_f32, tiles_t;
  void* k_g;            // reorder_kv: set (with v_g, n_pool dividing b) to form the ASA_G global tokens too
  void* v_g;
  int n_pool;
  hipStream_t stream;
};

struct MeanpoolArgs {
  const void* k_r;
  const void* v_t;
  void* k_g;
  void* v_g;
  int B, Hh, N, Npad, d, b, n, Ng;
  hipStream_t stream;
};

// Token-order operands of the fused entry points: element (b, i, h, :) of a
// [B, N, Hh, d] tensor at b * sb + perm_h[i] * sn + h * sh, perm_h = perm +
// h * perm_h_stride (curve position i -> token).
struct TokIO {
  const void* q;        // nullable: Q read in token order instead of from q_r
  void* out;            // nullable: output written in token order instead of to o_r
  const int32_t* perm;
  int64_t qsb, qsn, qsh, osb, osn, osh;   // element strides
  int perm_h_stride;
  int q_f32, out_f32;   // element types (float32 when set, else bf16)
};

struct EstimateArgs {
  const void* q_r;
  const void* k_r;
  float* p_imp;
  void* workspace;      // compact Q_s, K_s (bf16) and lse2 (float); see estimate_workspace_bytes
  int B, Hh, N, Npad, d, b, k, nb;
  float scale;
  TokIO tok;            // tok.q set: sampled Q rows gathered in token order (out unused)
  // k_tok set (with tok.perm): the sampled K rows are gathered from K in token
  // order into the workspace (after the estimator's own part; k_r unused)
  const void* k_tok;
  int64_t ksb, ksn, ksh;
  int k_f32;
  const struct MaskArgs* fuse;   // set: the final launch also selects the kept blocks (p_imp nullable)
  hipStream_t stream;
};

struct MaskArgs {
  const float* p_imp;
  int32_t* kv_count;
  int32_t* kv_idx;
  uint8_t* mask;
  int32_t* order;       // nullable: attention work order
  int rows, nb;
  float tau;            // rule 0
  int rule;             // 0 cumulative threshold, 1 top-k, 2 statistical cutoff
  int topk;             // rule 1
  double u;             // rule 2: the quantile in p = mean + std * u
  hipStream_t stream;
};

struct AttnArgs {
  const void* q_r;
  const void* k_r;
  const void* v_t;
  const int32_t* kv_count;
  const int32_t* kv_idx;
  const int32_t* order;  // nullable: work order from build_mask
  const void* k_g;
  const void* v_g;
  void* o_r;
  float* lse;
  int B, Hh, N, Npad, d, b, nb, Ng, n_pool;
  float scale;
  TokIO tok;            // zero: reordered Q in, reordered O out
  const int32_t* q_count;   // set (with rowsel): only the listed query rows of each block (pruned queries)
  const int32_t* rowsel;    // [B * Hh * nb, b] kept reordered rows of each block, ascending
  hipStream_t stream;
};

// Query pruning (BSA notes, key design 1): kept rows of every query block.
struct PruneArgs {
  const void* q;            // token order, element strides qsb / qsn / qsh, d contiguous
  int64_t qsb, qsn, qsh;
  int q_f32;
  const int32_t* perm;      // reordered row -> token
  const int32_t* anchor;    // reordered row -> reordered row of its window centre
  int perm_h_stride;        // 0 (shared) or N (per head), for perm and anchor alike
  int B, Hh, N, Npad, d, b, nb;
  double r;                 // keep ratio in (0, 1]
  int32_t* q_count;         // [B * Hh * nb]
  int32_t* rowsel;          // [B * Hh * nb, b], -1 past the count
  uint8_t* keep;            // [B * Hh * Npad]
  hipStream_t stream;
};

// Pooled block estimate (MEAN / TripPool descriptors, row softmax of their products).
struct PooledArgs {
  const void* q_r;          // reordered rows, when tok.perm is not set
  const void* k_r;          // reordered rows [B, Hh, Npad, d]
  TokIO tok;                // tok.perm set: Q read in token order
  float* p_imp;             // [B, Hh, nb, nb]
  void* workspace;          // pooled_workspace_bytes
  int B, Hh, N, Npad, d, b, nb;
  int kind;                 // 0 MEAN, 1 TRIP (mean, max, min)
  hipStream_t stream;
};

// SICS of every block and the per-head aggregation score; with n_cand > 0,
// of every candidate permutation (and of K too when tensors == 2) and the
// per-head choice.
struct SicsArgs {
  const void* q_r;
  TokIO tok;
  float* sics;              // [B, Hh, nb]; candidates: [n_cand, tensors, B, Hh, nb]
  float* as;                // [B, Hh]; candidates: [n_cand, B, Hh]
  int B, Hh, N, Npad, d, b, nb;
  const void* k;            // candidates: K in token order (tok's strides and type), when tensors == 2
  const int32_t* perms;     // candidates: [n_cand, N]
  int n_cand, tensors;
  int32_t* choice;          // candidates: [B, Hh]
  hipStream_t stream;
};

// Token filling: pruned rows copy their centre's output row (token order).
struct FillArgs {
  void* out;
  int64_t osb, osn, osh;
  int out_f32;
  int row_bytes;            // d * element size, a multiple of 16
  const int32_t* perm;
  const int32_t* anchor;
  int perm_h_stride;
  const uint8_t* keep;
  float* lse;               // nullable, [B * Hh * Npad]
  int B, Hh, N, Npad;
  hipStream_t stream;
};

struct TransposeListsArgs {
  const int32_t* kv_count;
  const int32_t* kv_idx;
  int32_t* kvT_count;
  int32_t* kvT_idx;
  int B, Hh, nb;
  hipStream_t stream;
};

struct AttnBwdArgs {
  const void* q_r;
  const void* k_r;
  const void* v_r;       // V in rows layout
  const void* o_r;
  const void* do_r;
  const float* lse;      // natural log, from the forward
  const int32_t* kv_count;
  const int32_t* kv_idx;
  const int32_t* kvT_count;
  const int32_t* kvT_idx;
  float* dq;
  float* dk;
  float* dv;
  void* workspace;
  int B, Hh, N, Npad, d, b, nb;
  float scale;
  hipStream_t stream;
};

hipError_t launch_reorder(const ReorderArgs& a);
hipError_t launch_reorder_kv(const ReorderArgs& a);
hipError_t launch_inverse_reorder(const ReorderArgs& a);
hipError_t launch_meanpool(const MeanpoolArgs& a);
hipError_t launch_estimate(const EstimateArgs& a);
size_t estimate_workspace_bytes(int B, int Hh, int nb, int k, int d);
// With K in token order: the same, rounded up to 256 bytes, plus the gathered
// sampled K rows (bf16, B * Hh * nsp_pad * d).
size_t estimate_kvtok_workspace_bytes(int B, int Hh, int nb, int k, int d);
hipError_t launch_build_mask(const MaskArgs& a);
hipError_t launch_build_order(const MaskArgs& a);   // a.kv_count -> a.order only
hipError_t launch_query_prune(const PruneArgs& a);
hipError_t launch_fill_pruned(const FillArgs& a);
size_t pooled_workspace_bytes(int B, int Hh, int nb, int d);
hipError_t launch_pooled(const PooledArgs& a);
hipError_t launch_sics(const SicsArgs& a);
hipError_t launch_attn_fwd(const AttnArgs& a);
// Float32 operands (reordered rows; v_t holds V as rows): VALU kernels.
hipError_t launch_estimate_f32(const EstimateArgs& a);
hipError_t launch_attn_fwd_f32(const AttnArgs& a);
hipError_t launch_transpose_lists(const TransposeListsArgs& a);
size_t attn_bwd_workspace_bytes(int B, int Hh, int Npad, int d);
hipError_t launch_attn_bwd(const AttnBwdArgs& a);

}  // namespace dbs
