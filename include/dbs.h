/*
 * dbs.h -- content-adaptive block-sparse attention (ASA / ASA_G), forward pass,
 *          for AMD Instinct MI355X (gfx950).  C ABI (version: DBS_ABI_VERSION).
 *
 * The method: Video-BLADE ("Preprocessing", "Step 1", "Step 2.1", "Step 2.2")
 * and the BLADE notes (key designs 1 and 2).  A layer runs, on one stream:
 *
 *   dbs_reorder(Q), dbs_reorder(K), dbs_reorder(V)     tokens -> curve order
 *   [dbs_meanpool_kv]                                  ASA_G global tokens
 *   dbs_estimate_blocks                                sampled block importance
 *   dbs_build_mask                                     cumulative-threshold mask
 *   dbs_sparse_attn_fwd                                attention over kept tiles
 *   dbs_inverse_reorder(O)                             back to token order
 *
 * or, with the same results, in fewer launches and without the Q and O copies:
 *
 *   dbs_reorder_kv(K, V)                               K, V -> curve order
 *   [dbs_meanpool_kv]
 *   dbs_estimate_blocks_tok                            Q read in token order
 *   dbs_build_mask
 *   dbs_sparse_attn_fwd_tok                            Q read, O written in token order
 *
 * where dbs_estimate_mask_tok may stand for the estimate and mask pair: it
 * selects the kept blocks from each P_imp row on chip (P_imp optional), and
 * dbs_reorder_kv_pool for the reorder and meanpool pair (ASA_G).
 *
 * Beyond the forward layer: the backward of the attention
 * (dbs_transpose_lists, dbs_sparse_attn_bwd), other selection rules
 * (dbs_build_mask_rule), pooled estimates and SICS block-shape scores
 * (dbs_estimate_pooled_tok, dbs_sics_tok), and BSA query pruning with token
 * filling (dbs_prune_anchors, dbs_query_prune, dbs_sparse_attn_fwd_pruned_tok).
 *
 * Conventions for every call:
 * - Device pointers are allocated and owned by the caller and must be 16-byte
 *   aligned.  The library allocates no device memory.  Its only device state
 *   is the static scratch array of dbs_estimate_mask_tok_noalloc.
 * - Device calls are asynchronous on the given stream (NULL: the default
 *   stream) and never synchronise.  Arguments are checked on the host before
 *   any launch; a failed check launches nothing.
 * - The status is returned directly; dbs_last_error() describes the last
 *   failure of the calling thread.  No C++ exception crosses the ABI.
 * - B batch, Hh heads, N true tokens, Npad = N rounded up to a multiple of
 *   the block size b, d head dimension, nb = Npad / b blocks.
 *
 * Tensor layouts (all contiguous unless strides are given):
 *   DBS_ROWS     [B, Hh, Npad, d]            one token per row
 *   DBS_TILES_T  [B, Hh, Npad / b, d, b]     each b-token tile stored d-major
 *                                            (token index fastest); used for V
 *                                            so that the P*V product reads the
 *                                            keys of one channel contiguously.
 *                                            Token offset t of a tile sits in
 *                                            column t with bits 2 and 3 swapped:
 *                                            every 16 tokens are stored in the
 *                                            order 0-3, 8-11, 4-7, 12-15.
 */
#ifndef DBS_H
#define DBS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DBS_ABI_VERSION 13

typedef enum {
  DBS_OK = 0,
  DBS_ERR_INVALID_ARG = -1,  /* null pointer, bad size or range            */
  DBS_ERR_UNSUPPORTED = -2,  /* valid but not implemented (d, b, k, dtype) */
  DBS_ERR_ALIGNMENT = -3,    /* a device pointer is not 16-byte aligned    */
  DBS_ERR_LAUNCH = -4,       /* the kernel launch failed                   */
  DBS_ERR_HIP = -5           /* another HIP runtime call failed            */
} dbs_status;

/* Element type and layout arguments.  The two range enumerators make every
 * int a valid value of the type, so an unknown value passed by a caller is
 * well defined in C++ too and is rejected by the argument checks. */
typedef enum {
  DBS_BF16 = 0,
  DBS_FP32 = 1,
  DBS_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
  DBS_DTYPE_RANGE_MAX_ = 0x7fffffff
} dbs_dtype;
typedef enum {
  DBS_ROWS = 0,
  DBS_TILES_T = 1,
  DBS_LAYOUT_RANGE_MIN_ = -0x7fffffff - 1,
  DBS_LAYOUT_RANGE_MAX_ = 0x7fffffff
} dbs_layout;

/* ABI version of the loaded library (DBS_ABI_VERSION). */
int dbs_abi_version(void);

/* Message for the calling thread's last failed call; "" if none.  Valid until
 * that thread's next call. */
const char* dbs_last_error(void);

/* ---------------------------------------------------------------------------
 * Host permutation helpers (shape only; no device work).
 *
 * perm[new] = old: position `new` of the reordered sequence holds raster
 * token `old` = prefix + (t * H + h) * W + w.  Positions < prefix (text
 * tokens) stay in place.  perm_out must hold prefix + T*H*W entries.
 * ------------------------------------------------------------------------- */

/* Gilbert (generalised Hilbert) curve over the T x H x W latent grid, the
 * locality-preserving order of Video-BLADE "Preprocessing".  The pages name the
 * curve without defining it; the recursion implemented is a corner-to-corner
 * walk that splits the box along its long side, or into a three-piece "U"
 * across the plane of its two longest sides; every step moves to a grid
 * neighbour.  Errors: INVALID_ARG if a side < 1, prefix < 0, perm_out NULL, or
 * the length exceeds INT32_MAX. */
dbs_status dbs_perm_gilbert3d(int T, int H, int W, int prefix, int32_t* perm_out);

/* Cuboid-major order (Bidirectional Sparse Attention notes, "overall
 * framework"; VEDA key design 2 for per-head shapes): cuboids of
 * ct x ch x cw in raster order, raster order inside each cuboid; border
 * cuboids hold fewer tokens.  Errors as above. */
dbs_status dbs_perm_cuboid(int T, int H, int W, int ct, int ch, int cw, int prefix,
                           int32_t* perm_out);

/* inv_out[perm[i]] = i.  INVALID_ARG if perm is not a permutation of 0..n-1. */
dbs_status dbs_perm_invert(const int32_t* perm, int n, int32_t* inv_out);

/* Window centres for query pruning (Bidirectional Sparse Attention notes, key
 * design 1 and "a complete example"), on the host.  Windows of wt x wh x ww
 * tile the T x H x W grid from its origin (border windows are cut); the
 * centre of a window sits at offset (e - 1) / 2 along each axis, e the
 * window's extent there; a text-prefix token is its own centre.
 * anchor_out[i] = the reordered index of the centre of token perm[i], for the
 * reordered sequence given by perm (length prefix + T*H*W).  Errors:
 * INVALID_ARG for a side < 1, a NULL pointer or a perm that is not a
 * permutation. */
dbs_status dbs_prune_anchors(int T, int H, int W, int prefix, int wt, int wh, int ww, const int32_t* perm,
                             int32_t* anchor_out);

/* ---------------------------------------------------------------------------
 * Device calls.
 * ------------------------------------------------------------------------- */

/* Reorder tokens into curve / cuboid order (Video-BLADE "Preprocessing").
 *   y[b, h, i, :] = x[b, perm_h[i], h, :]  for i < N;  rows N..Npad-1 = 0.
 * x: element type x_dt, element strides (sb, sn, sh) for (batch, token, head);
 *    the d channels contiguous.
 * y: element type y_dt (DBS_FP32 -> DBS_BF16 rounds to nearest even; the
 *    reverse is not offered), layout y_layout (DBS_TILES_T tiles of b tokens).
 * perm: device int32, [N] for all heads (perm_per_head = 0) or [Hh, N], a
 *    permutation of 0..N-1 (entries outside [0, N) are clamped into it, which
 *    keeps every access in bounds but is not a meaningful result).
 * Supported: d in {64, 128}; b in {64, 128}; Npad % b == 0; N <= Npad. */
dbs_status dbs_reorder(const void* x, dbs_dtype x_dt, int64_t sb, int64_t sn, int64_t sh,
                       void* y, dbs_dtype y_dt, dbs_layout y_layout,
                       const int32_t* perm, int perm_per_head,
                       int B, int Hh, int N, int Npad, int d, int b, hipStream_t stream);

/* K and V reordered together (Video-BLADE "Preprocessing"), in one launch:
 *   k_r = dbs_reorder(k, rows layout, bf16), v_t = dbs_reorder(v, tiles
 *   layout, bf16), bit for bit.
 * k, v: element type x_dt (DBS_BF16 or DBS_FP32, rounded to bf16 to nearest
 *    even), [B, N, Hh, d] with the same element strides (sb, sn, sh).
 * k_r: device bf16 [B, Hh, Npad, d]; v_t: device bf16 [B, Hh, Npad/b, d, b];
 *    rows and columns N..Npad-1 are zero.
 * perm, sizes and limits as for dbs_reorder. */
dbs_status dbs_reorder_kv(const void* k, const void* v, dbs_dtype x_dt,
                          int64_t sb, int64_t sn, int64_t sh,
                          void* k_r, void* v_t, const int32_t* perm, int perm_per_head,
                          int B, int Hh, int N, int Npad, int d, int b, hipStream_t stream);

/* Inverse of dbs_reorder for the attention output:
 *   x[b, perm_h[i], h, :] = y[b, h, i, :]  for i < N.
 * y: DBS_ROWS, element type y_dt; x: element type x_dt with strides
 * (sb, sn, sh).  DBS_BF16 -> DBS_FP32 widens exactly and DBS_FP32 ->
 * DBS_FP32 copies (DBS_FP32 -> DBS_BF16 is not offered: UNSUPPORTED).  perm
 * as for dbs_reorder (entries clamped into [0, N)). */
dbs_status dbs_inverse_reorder(const void* y, dbs_dtype y_dt, void* x, dbs_dtype x_dt,
                               int64_t sb, int64_t sn, int64_t sh,
                               const int32_t* perm, int perm_per_head,
                               int B, int Hh, int N, int Npad, int d, hipStream_t stream);

/* Bytes of device workspace dbs_estimate_blocks needs: one
 * partial softmax (max, sum) float pair per sampled query and key split (the
 * library splits the sampled keys over up to nb*k/64 workgroups per panel of
 * 256 sampled queries), and per sampled query the maximum raw score over each cell of
 * min(k, 64) sampled keys (B * Hh * nb*k * nb*k/min(k,64) floats; about
 * 50 MB for 12 heads, nb = 256, k = 16), k rounded up to a power of two.
 * Returns 0 for invalid sizes. */
size_t dbs_estimate_workspace_bytes(int B, int Hh, int N, int d, int b, int k);

/* Block-importance estimation (Video-BLADE "Step 1"; BLADE notes key design 1).
 * From every b-token block J, k_J = min(k, L_J) tokens are sampled at offsets
 * floor(t * L_J / k_J), t < k_J (L_J = valid tokens of block J), in Q and K
 * alike.  P_approx = row-softmax(Q_s K_s^T * scale) over all sampled keys of
 * the (batch, head); p_imp[b, h, I, J] = max of P_approx over (samples of I) x
 * (samples of J), float32, [B, Hh, nb, nb].
 * q_r, k_r: DBS_ROWS, type dt.  DBS_BF16: bf16 products with float32
 * accumulation and a float32 softmax; a block's sampled slots are padded to
 * the next power of two (empty slots take no part), so any k in 1..b costs
 * what that power of two costs.  DBS_FP32: float32 operands and float32
 * arithmetic throughout (any k in 1..b), for workloads stored in float32.
 * workspace: device, >= dbs_estimate_workspace_bytes(...) bytes; its contents
 * on entry do not matter.  Q and K must be finite (a NaN input gives an
 * undefined result).  Errors: UNSUPPORTED for d, b, k or dt outside the
 * supported set; INVALID_ARG for a small workspace. */
dbs_status dbs_estimate_blocks(const void* q_r, const void* k_r, dbs_dtype dt,
                               int B, int Hh, int N, int Npad, int d, int b, int k, float scale,
                               float* p_imp, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* dbs_estimate_blocks with Q in token order: the sampled Q rows are read as
 * q[b, perm_h[i], h, :] (element strides sb, sn, sh; d contiguous; perm as
 * for dbs_reorder, entries clamped into [0, N)) instead of from a reordered
 * copy, so the layer need not reorder Q.  q_dt: DBS_BF16, or DBS_FP32 rounded
 * to bf16 (round to nearest even) exactly as dbs_reorder rounds it; the
 * result equals dbs_estimate_blocks on dbs_reorder's output bit for bit.
 * k_r, workspace and the errors as for dbs_estimate_blocks. */
dbs_status dbs_estimate_blocks_tok(const void* q, dbs_dtype q_dt, int64_t sb, int64_t sn, int64_t sh,
                                   const int32_t* perm, int perm_per_head, const void* k_r,
                                   int B, int Hh, int N, int Npad, int d, int b, int k, float scale,
                                   float* p_imp, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* Cumulative-threshold mask (Video-BLADE "Step 2.1").  For every row
 * (b, h, I): order the blocks by p_imp value descending, then index
 * ascending, and keep the fewest m >= 1 whose exact sum reaches
 * tau * (exact row sum); tau >= 1 keeps all nb.  The sums are exact (every
 * float32 is an exact rational), so the result does not depend on summation
 * order.  A row holding a value outside [0, 1] or NaN keeps every block.
 * kv_count[b, h, I] = m; kv_idx[b, h, I, 0..m-1] = kept blocks ascending
 * (entries m..nb-1 are left untouched); mask (nullable) [B, Hh, nb, nb]
 * uint8 1 for kept, 0 otherwise.  tau must be in (0, 1].  nb <= 4096.
 * order (nullable): int32 [B * Hh * nb], a work order for
 * dbs_sparse_attn_fwd, a permutation of the row index (b * Hh + h) * nb + I.
 * The rows are split into eight contiguous ranges (the first
 * (B*Hh*nb) % 8 of them one row longer), one per XCD of the attention launch,
 * and each range lists its rows by kept count descending (equal counts in
 * any order): every XCD starts its longest query blocks first.  Any order
 * gives the same attention result; this one balances the uneven work.
 * Errors: INVALID_ARG for a NULL p_imp / kv_count / kv_idx or tau outside
 * (0, 1]; UNSUPPORTED for nb > 4096; ALIGNMENT for a misaligned pointer. */
dbs_status dbs_build_mask(const float* p_imp, int B, int Hh, int nb, float tau,
                          int32_t* kv_count, int32_t* kv_idx, uint8_t* mask, int32_t* order,
                          hipStream_t stream);

/* The same kept-block lists (and optional mask / work order) under another
 * selection rule (one of dbs_mask_rule), for comparing rules on one P_imp:
 *   DBS_RULE_CUMULATIVE  param = tau: exactly dbs_build_mask.
 *   DBS_RULE_TOPK        param = k (an integer >= 1): the k blocks of largest
 *                        importance, ties by block index (k >= nb keeps all);
 *                        the fixed-budget rule the BSA notes compare against.
 *   DBS_RULE_STAT        param = u: the statistical cutoff of the BSA notes
 *                        (design 2), p = mean + std * u over the row's nb
 *                        scores (population std, float64, fixed summation
 *                        order), read as a per-block cutoff: every block with
 *                        P_imp >= p is kept, and at least the largest one.
 *                        u = U(1 - k/n), the standard normal quantile, keeps
 *                        about k of n blocks on normally spread scores.
 *   DBS_RULE_STAT_K      param = k, 0 < k < nb: DBS_RULE_STAT with
 *                        u = dbs_normal_quantile(1 - k/nb) computed here.
 * Rows holding a value outside [0, 1] or NaN keep every block.  Output as
 * for dbs_build_mask.  INVALID_ARG for an unknown rule or a bad param. */
typedef enum { DBS_RULE_CUMULATIVE = 0, DBS_RULE_TOPK = 1, DBS_RULE_STAT = 2, DBS_RULE_STAT_K = 3 } dbs_mask_rule;
dbs_status dbs_build_mask_rule(const float* p_imp, int B, int Hh, int nb, int rule, double param,
                               int32_t* kv_count, int32_t* kv_idx, uint8_t* mask, int32_t* order,
                               hipStream_t stream);

/* The standard normal quantile U(p) (inverse of the normal distribution
 * function) on the host, as the statistical rule uses it: Wichura's algorithm
 * AS 241 (Applied Statistics 37, 1988), about 16 significant digits.
 * p in (0, 1); U(0) = -inf, U(1) = +inf, NaN outside [0, 1]. */
double dbs_normal_quantile(double p);

/* Estimation and selection in one pass over the estimator's intermediate
 * results (the fusion of the importance estimate with the mask builder that
 * SPADE's fused prepass suggests): the same kv_count / kv_idx / mask / order
 * as dbs_estimate_blocks followed by dbs_build_mask_rule(rule, param), bit for
 * bit, but each P_imp row is formed on chip and handed straight to the
 * selection.  p_imp (nullable): when given, P_imp is written as well, equal
 * to dbs_estimate_blocks' output.  Inputs, workspace and limits as for
 * dbs_estimate_blocks, outputs and rules as for dbs_build_mask_rule
 * (nb <= 4096); the errors of both.  With dt = DBS_FP32 the estimate and the
 * selection are two launches, P_imp held in p_imp or else in the workspace. */
dbs_status dbs_estimate_mask(const void* q_r, const void* k_r, dbs_dtype dt,
                             int B, int Hh, int N, int Npad, int d, int b, int k, float scale,
                             int rule, double param, float* p_imp,
                             int32_t* kv_count, int32_t* kv_idx, uint8_t* mask, int32_t* order,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* dbs_estimate_mask with Q read in token order, as dbs_estimate_blocks_tok
 * reads it (same q, q_dt, strides and perm arguments). */
dbs_status dbs_estimate_mask_tok(const void* q, dbs_dtype q_dt, int64_t sb, int64_t sn, int64_t sh,
                                 const int32_t* perm, int perm_per_head, const void* k_r,
                                 int B, int Hh, int N, int Npad, int d, int b, int k, float scale,
                                 int rule, double param, float* p_imp,
                                 int32_t* kv_count, int32_t* kv_idx, uint8_t* mask, int32_t* order,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace dbs_estimate_mask_kvtok needs:
 * dbs_estimate_workspace_bytes rounded up to 256, plus the sampled K rows it
 * gathers (bf16, B * Hh * P * d with P = nb * k rounded up to a multiple of
 * 64, k rounded up to a power of two).  Returns 0 for invalid sizes. */
size_t dbs_estimate_kvtok_workspace_bytes(int B, int Hh, int N, int d, int b, int k);

/* dbs_estimate_mask_tok with K read in token order as well (Video-BLADE
 * "Step 1" samples K as it samples Q): the sampled K rows are gathered from
 * key[b, perm_h[i], h, :] (element strides ksb, ksn, ksh; d contiguous;
 * key_dt DBS_BF16, or DBS_FP32 rounded to bf16 as dbs_reorder_kv rounds it)
 * into the workspace, so the estimate needs no reordered K.  A layer can then
 * run dbs_reorder_kv on a second stream while this call runs.  The outputs
 * equal dbs_estimate_mask_tok on dbs_reorder_kv's k_r bit for bit.  q, q_dt,
 * its strides, perm and the rest as for dbs_estimate_mask_tok; workspace:
 * device, >= dbs_estimate_kvtok_workspace_bytes(...) bytes.  Errors as for
 * dbs_estimate_mask_tok, and for key as for q. */
dbs_status dbs_estimate_mask_kvtok(const void* q, dbs_dtype q_dt, int64_t qsb, int64_t qsn, int64_t qsh,
                                   const void* key, dbs_dtype key_dt, int64_t ksb, int64_t ksn, int64_t ksh,
                                   const int32_t* perm, int perm_per_head,
                                   int B, int Hh, int N, int Npad, int d, int b, int k, float scale,
                                   int rule, double param, float* p_imp,
                                   int32_t* kv_count, int32_t* kv_idx, uint8_t* mask, int32_t* order,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * dbs_estimate_mask_tok with no workspace argument.  The estimator's
 * intermediate results go to a static device array of
 * DBS_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends; this call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).  The array's address on the
 * stream's device is looked up on the first call there.  Every argument,
 * output and error is dbs_estimate_mask_tok's, plus: UNSUPPORTED, before any
 * device work, when the shape needs more than DBS_NOALLOC_SCRATCH_BYTES
 * (dbs_estimate_workspace_bytes(B, Hh, N, d, b, k) says how much).  Nothing in
 * the array has to start at zero.  All calls on one GPU share its array:
 * calls that overlap on one GPU (on different streams, or from several
 * threads) race and give undefined results. */
#define DBS_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
dbs_status dbs_estimate_mask_tok_noalloc(const void* q, dbs_dtype q_dt, int64_t sb, int64_t sn, int64_t sh,
                                         const int32_t* perm, int perm_per_head, const void* k_r, int B, int Hh,
                                         int N, int Npad, int d, int b, int k, float scale, int rule, double param,
                                         float* p_imp, int32_t* kv_count, int32_t* kv_idx, uint8_t* mask,
                                         int32_t* order, hipStream_t stream);

/* Query pruning (Bidirectional Sparse Attention notes, key design 1): in each
 * query block I (reordered rows I*b .. I*b + n - 1, n valid), a row i whose
 * centre anchor[i] (dbs_prune_anchors) is itself is a centre and always kept;
 * of the other rows the m - c of largest 1 - cos(q[centre], q[i]) are kept
 * (float32 from the bf16 values; ties by smaller row), where c is the block's
 * number of centres and m = min(n, max(ceil(r * n), c)).
 * q: token order [B, N, Hh, d] with element strides sb, sn, sh (d contiguous;
 * bf16, or float32 rounded to bf16), read through perm as for
 * dbs_estimate_blocks_tok; anchor: int32 [N] (or [Hh, N] when perm_per_head),
 * reordered indices.  Outputs: q_count int32 [B, Hh, nb] = m; rowsel int32
 * [B, Hh, nb, b], the kept rows (reordered indices) ascending, -1 after m;
 * keep uint8 [B, Hh, Npad], 1 for a kept row (0 for rows >= N).  r in (0, 1].
 * Errors as for dbs_estimate_blocks_tok, and INVALID_ARG for r. */
dbs_status dbs_query_prune(const void* q, dbs_dtype q_dt, int64_t sb, int64_t sn, int64_t sh,
                           const int32_t* perm, int perm_per_head, const int32_t* anchor,
                           int B, int Hh, int N, int Npad, int d, int b, double r,
                           int32_t* q_count, int32_t* rowsel, uint8_t* keep, hipStream_t stream);

/* dbs_sparse_attn_fwd_tok (plain ASA, no global tokens) for the kept query
 * rows of dbs_query_prune only, then token filling: every row with keep = 0
 * takes the output (and lse) of its centre anchor[i], which the pruning
 * always keeps.  Kept rows get exactly the output dbs_sparse_attn_fwd_tok
 * gives them.  Query work is split into 64-row pieces of each block's kept
 * list, so the attention's cost follows the kept rows.  q_count, rowsel,
 * keep, anchor: as written / read by dbs_query_prune for the same perm.
 * Other arguments and errors as for dbs_sparse_attn_fwd_tok. */
dbs_status dbs_sparse_attn_fwd_pruned_tok(const void* q, dbs_dtype q_dt, int64_t qsb, int64_t qsn, int64_t qsh,
                                          const int32_t* perm, int perm_per_head, const void* k_r,
                                          const void* v_r, int B, int Hh, int N, int Npad, int d, int b,
                                          float scale, const int32_t* kv_count, const int32_t* kv_idx,
                                          const int32_t* order, const int32_t* q_count, const int32_t* rowsel,
                                          const int32_t* anchor, const uint8_t* keep, void* out,
                                          dbs_dtype out_dt, int64_t osb, int64_t osn, int64_t osh, float* lse,
                                          hipStream_t stream);

/* Pooled block estimate, an alternative to dbs_estimate_blocks on the same
 * P_imp boundary (the SPADE notes' MEAN and DSA summaries; VEDA key design 1,
 * TripPool, with its head-specific projections taken as the identity): block
 * J of b reordered tokens (valid ones only) is summarised by
 *   DBS_POOL_MEAN  the mean of its tokens (d values), or
 *   DBS_POOL_TRIP  their mean, channel-wise maximum and minimum (3d values),
 * in float32 from the bf16 values, and
 *   p_imp[b, h, I, J] = softmax over J of desc_q(I) . desc_k(J) / sqrt(d'),
 * d' the descriptor length.  Q in token order as for dbs_estimate_blocks_tok;
 * k_r DBS_ROWS.  workspace >= dbs_pooled_workspace_bytes (2 * B * Hh * nb *
 * 3d floats).  Errors as for dbs_estimate_blocks_tok, INVALID_ARG for kind. */
typedef enum { DBS_POOL_MEAN = 0, DBS_POOL_TRIP = 1 } dbs_pool_kind;
size_t dbs_pooled_workspace_bytes(int B, int Hh, int N, int d, int b);
dbs_status dbs_estimate_pooled_tok(const void* q, dbs_dtype q_dt, int64_t sb, int64_t sn, int64_t sh,
                                   const int32_t* perm, int perm_per_head, const void* k_r,
                                   int B, int Hh, int N, int Npad, int d, int b, int kind,
                                   float* p_imp, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* SICS (the SPADE notes, runtime scheme generation): for the reordering perm
 * (a candidate block shape, e.g. dbs_perm_cuboid), every block of b reordered
 * tokens gets SICS = || sum of its unit-normalised Q rows ||^2 (equal to the
 * sum of all pairwise cosine similarities in the block; a zero row adds
 * nothing), float32, sics [B, Hh, nb]; as_out [B, Hh] = the head's
 * aggregation score, the sum over its blocks in a fixed order.  Choosing, per
 * head, the candidate with the largest score is the notes' scheme choice.
 * Q as for dbs_estimate_blocks_tok. */
dbs_status dbs_sics_tok(const void* q, dbs_dtype q_dt, int64_t sb, int64_t sn, int64_t sh,
                        const int32_t* perm, int perm_per_head, int B, int Hh, int N, int Npad, int d, int b,
                        float* sics, float* as_out, hipStream_t stream);

/* The SPADE notes' scheme choice (runtime scheme generation) over n_cand
 * candidate token orders in one call.  The notes compute the aggregation
 * score of Query and of Key for every candidate; read here as the per-head
 * score AS(Q | c) + AS(K | c), each the sum over the blocks of
 * || sum of the block's unit-normalised rows ||^2 as in dbs_sics_tok.
 * q, k: token order [B, N, Hh, d], type dt (bf16, or float32 rounded to
 *    bf16), element strides sb, sn, sh (d contiguous); k nullable (then Q
 *    alone is scored).
 * perms: device int32 [n_cand, N], candidate c's order perms[c] (shared by
 *    every head), e.g. dbs_perm_cuboid of candidate block shapes; 1 <= n_cand
 *    <= 64.
 * block_scores: device float32 [n_cand, T, B, Hh, nb] (T = 2 with k, else 1),
 *    every block's score; scores: float32 [n_cand, B, Hh], the aggregation
 *    scores (blocks summed in a fixed order); choice: int32 [B, Hh], the
 *    candidate with the largest score, the smallest index among equal ones.
 * Errors as for dbs_sics_tok, INVALID_ARG for n_cand. */
dbs_status dbs_sics_choose(const void* q, const void* k, dbs_dtype dt, int64_t sb, int64_t sn, int64_t sh,
                           const int32_t* perms, int n_cand, int B, int Hh, int N, int Npad, int d, int b,
                           float* block_scores, float* scores, int32_t* choice, hipStream_t stream);

/* ASA_G global tokens (Video-BLADE "Step 2.2 (2)"; BLADE notes key design 2):
 * mean of each window of n consecutive reordered tokens,
 *   k_g[b, h, g, :] = mean(k_r[b, h, g*n .. g*n + r_g - 1, :]),
 *   r_g = min(n, N - g*n),  g < Ng = ceil(N / n),  likewise v_g,
 * accumulated in float32 and rounded to bf16.
 * k_r: DBS_ROWS; v_r: DBS_TILES_T (tiles of b).  k_g: DBS_ROWS
 * [B, Hh, Ngpad, d]; v_g: DBS_TILES_T [B, Hh, Ngpad / b, d, b] with
 * Ngpad = ceil(Ng / b) * b; rows Ng..Ngpad-1 are written as zeros. */
dbs_status dbs_meanpool_kv(const void* k_r, const void* v_r, dbs_dtype dt,
                           int B, int Hh, int N, int Npad, int d, int b, int n,
                           void* k_g, void* v_g, hipStream_t stream);

/* dbs_reorder_kv and dbs_meanpool_kv in one launch (the fusion of the reorder
 * with the ASA_G pooling that SPADE's fused prepass suggests): each tile of b
 * reordered tokens is reordered and, when n divides b, its windows' means are
 * formed from the tile held in LDS, with exactly dbs_meanpool_kv's arithmetic
 * (float32 sums in ascending token order), so k_r, v_t, k_g and v_g equal the
 * two calls' outputs bit for bit.  When n does not divide b the two calls are
 * made.  Arguments as for the two calls; k_g, v_g as for dbs_meanpool_kv. */
dbs_status dbs_reorder_kv_pool(const void* k, const void* v, dbs_dtype x_dt, int64_t sb, int64_t sn, int64_t sh,
                               void* k_r, void* v_t, const int32_t* perm, int perm_per_head,
                               int B, int Hh, int N, int Npad, int d, int b, int n,
                               void* k_g, void* v_g, hipStream_t stream);

/* Block-sparse attention forward (Video-BLADE "Step 2.2").  For every query
 * row q < N of query block I:
 *   O_q = sum_c softmax_c(s_qc) V_c,  s_qc = scale * q . k_c
 * over the tokens c < N of the kept blocks kv_idx[b, h, I, 0..m-1]
 * (m = kv_count[b, h, I]), and, when k_g != NULL (ASA_G), over all Ng global
 * tokens with s = scale * q . k_g + ln(r_g), r_g = min(n_pool, N - g*n_pool).
 * Scores and the softmax are float32; the probabilities are rounded to bf16
 * for the P*V product (float32 accumulation).  Rows with no key at all get
 * O = 0 and lse = -inf.
 * dt = DBS_BF16: q_r, k_r DBS_ROWS bf16; v_r DBS_TILES_T bf16; k_g, v_g as
 * written by dbs_meanpool_kv; o_r DBS_ROWS bf16, rows >= N untouched.
 * dt = DBS_FP32 (workloads stored in float32): q_r, k_r, v_r and o_r all
 * DBS_ROWS float32, every product and the softmax in float32 (P is not
 * rounded); no global tokens (k_g, v_g must be NULL: UNSUPPORTED otherwise).
 * lse (nullable): float32 [B, Hh, Npad], natural-log normaliser of each row < N.
 * kv_count is clamped to [0, nb] and kv_idx entries outside [0, nb) are
 * skipped, so malformed lists cannot read outside the K/V buffers.
 * order (nullable): the work order written by dbs_build_mask for the same
 * kv_count (NULL: rows in index order).  Entries are clamped to
 * [0, B*Hh*nb); an order that is not a permutation computes some rows twice
 * and leaves others untouched, but never reads or writes outside the
 * buffers.  Q, K and V must be finite (a NaN input gives an undefined
 * result).  Returns UNSUPPORTED for nb > 4096 (the kernel keeps a query
 * block's list in LDS) or a head dimension / block size other than 64, 128;
 * INVALID_ARG / ALIGNMENT for bad sizes or pointers. */
dbs_status dbs_sparse_attn_fwd(const void* q_r, const void* k_r, const void* v_r, dbs_dtype dt,
                               int B, int Hh, int N, int Npad, int d, int b, float scale,
                               const int32_t* kv_count, const int32_t* kv_idx, const int32_t* order,
                               const void* k_g, const void* v_g, int Ng, int n_pool,
                               void* o_r, float* lse, hipStream_t stream);

/* dbs_sparse_attn_fwd with Q read and the output written in token order
 * (Video-BLADE "Step 2.2" followed by the return to token order, as one
 * launch): Q row i of head h is q[b, perm_h[i], h, :] and output row i is
 * written to out[b, perm_h[i], h, :] for i < N (element strides qsb/qsn/qsh
 * and osb/osn/osh, d contiguous, 16-byte aligned rows; perm as for
 * dbs_reorder, entries clamped into [0, N), a permutation for a complete
 * output).  q_dt: DBS_BF16, or DBS_FP32 rounded to bf16 as dbs_reorder
 * rounds it; out_dt: DBS_BF16, or DBS_FP32 holding the bf16 result widened
 * exactly.  The output equals dbs_inverse_reorder applied to
 * dbs_sparse_attn_fwd's o_r bit for bit; lse stays in curve order
 * ([B, Hh, Npad]).  Everything else as for dbs_sparse_attn_fwd. */
dbs_status dbs_sparse_attn_fwd_tok(const void* q, dbs_dtype q_dt, int64_t qsb, int64_t qsn, int64_t qsh,
                                   const int32_t* perm, int perm_per_head, const void* k_r, const void* v_r,
                                   int B, int Hh, int N, int Npad, int d, int b, float scale,
                                   const int32_t* kv_count, const int32_t* kv_idx, const int32_t* order,
                                   const void* k_g, const void* v_g, int Ng, int n_pool,
                                   void* out, dbs_dtype out_dt, int64_t osb, int64_t osn, int64_t osh,
                                   float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Backward (plain ASA).  The pages define the forward only (Video-BLADE
 * "Step 2.2"); its gradient is the derivative of that definition, and the
 * key-to-query lists it needs are the reverse scatter of the query-to-key
 * lists that the BSA notes (sparse kernels with forward and backward) use.
 * ------------------------------------------------------------------------- */

/* Key-to-query lists: for every (b, h, J), the query blocks I whose list
 * (kv_count / kv_idx as written by dbs_build_mask) holds J, in ascending
 * order.  kv_count entries are clamped to [0, nb] and kv_idx entries outside
 * [0, nb) skipped, as the attention does; a row's list is taken as a set
 * (a repeated entry counts once; dbs_build_mask never repeats one).
 * kvT_count [B, Hh, nb] int32,
 * kvT_idx [B, Hh, nb, nb] int32 (entries past kvT_count unspecified).
 * UNSUPPORTED for nb > 4096. */
dbs_status dbs_transpose_lists(const int32_t* kv_count, const int32_t* kv_idx, int B, int Hh, int nb,
                               int32_t* kvT_count, int32_t* kvT_idx, hipStream_t stream);

/* Bytes of device workspace dbs_sparse_attn_bwd needs: D = rowsum(dO * O),
 * one float per row (B * Hh * Npad floats).  0 for invalid sizes. */
size_t dbs_attn_bwd_workspace_bytes(int B, int Hh, int Npad, int d);

/* Gradients of dbs_sparse_attn_fwd without global tokens:
 *   P = softmax(Q K^T * scale) over the kept blocks, dV = P^T dO,
 *   dS = P * (dO V^T - rowsum(dO * O)), dQ = dS K * scale, dK = dS^T Q * scale.
 * q_r, k_r, v_r, o_r, do_r: DBS_ROWS bf16 [B, Hh, Npad, d] (note: V in rows
 * layout); rows N..Npad-1 of q_r, k_r, v_r and do_r must be finite
 * (dbs_reorder writes zeros there), o_r's are not read.  lse: the forward's
 * float32 [B, Hh, Npad] (rows < N read).  kv_count / kv_idx: the lists the
 * forward used; kvT_count / kvT_idx: their dbs_transpose_lists.  dq_r, dk_r,
 * dv_r: float32 [B, Hh, Npad, d], rows >= N written as zero; a query block
 * with no kept block gets dQ = 0.  workspace: device, >=
 * dbs_attn_bwd_workspace_bytes(B, Hh, Npad, d) bytes, contents irrelevant.
 * Errors as for dbs_sparse_attn_fwd, and INVALID_ARG for a small workspace. */
dbs_status dbs_sparse_attn_bwd(const void* q_r, const void* k_r, const void* v_r, const void* o_r,
                               const void* do_r, const float* lse,
                               int B, int Hh, int N, int Npad, int d, int b, float scale,
                               const int32_t* kv_count, const int32_t* kv_idx,
                               const int32_t* kvT_count, const int32_t* kvT_idx,
                               float* dq_r, float* dk_r, float* dv_r,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DBS_H */
