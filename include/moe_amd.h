/*
 * moe_amd.h -- C ABI of the single-device Mixture-of-Experts layer hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * The path follows the four stages of an MoE layer described in the Transformer
 * Engine user guide "Mixture of Experts" (section "Introduction"): the router
 * scores the experts and keeps the top-k per token, token dispatch lays the tokens
 * out expert-contiguously, the grouped expert MLP runs over all expert blocks, and
 * token combine merges the per-expert outputs back in token order.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers, row-major, densely packed, owned by
 *    the caller. The library never allocates, frees or synchronises inside these
 *    calls, never reads device data on the host, and enqueues work only on
 *    `stream` (a hipStream_t passed as void*; NULL is the default stream).
 *  - bf16 tensors are passed as void* (IEEE bfloat16 bit patterns); e4m3 tensors
 *    as uint8 codes of the OCP FP8 E4M3 ("fn") format; scales as float32.
 *  - Token counts per expert stay on the device (Transformer Engine guide,
 *    "Grouped GEMM": device-side counts avoid a host synchronisation), so every
 *    call can be captured in a HIP graph.
 *  - Concurrency: the grouped-GEMM launches of moe_forward / moe_backward keep
 *    their tile counters in the layer workspace (zeroed by the forward's dispatch,
 *    left zero by every launch), so layers with their own workspaces may run at
 *    once on different streams, eagerly or as graph replays. A stand-alone
 *    grouped-GEMM entry point takes one of 64 device-side tile-counter slots of the
 *    library, in launch order, and hands it back zeroed when it ends: up to 64 such
 *    launches may be in flight at once on one device; a captured one keeps the slot
 *    it drew at capture, so its replay must not overlap an eager stand-alone launch
 *    that drew the same slot.
 *  - Routing is dropless: routed row buffers always hold T*k rows (guide, "Example:
 *    MoE layer on a single device": num_out_tokens = num_tokens * top_k).
 *  - Errors: host-side argument checks return MOE_ERR_INVALID_ARG (bad pointer,
 *    negative size, k out of range) or MOE_ERR_UNSUPPORTED (a size the kernels do
 *    not handle); a failed kernel launch returns MOE_ERR_HIP; a workspace smaller
 *    than required returns MOE_ERR_WORKSPACE. Nothing is enqueued when a check
 *    fails. T == 0 is a valid no-op. Out-of-range expert ids in topk_idx are the
 *    caller's error and are not checked on the device; so are device group offsets
 *    passed to the grouped GEMMs that are not non-decreasing within [0, rows].
 *  - Supported sizes: 1 <= k <= min(E, 32), E <= 256, H % 64 == 0, I % 64 == 0,
 *    one expert's weight matrix under 4 GiB (and 512 rows of the GEMM's activation
 *    operand under 4 GiB), T*(k+1) + 256*4095 routed rows within int32 (row ids and
 *    offsets are int32), T*k*H <= 2^40, every pointer 16-byte aligned; larger sizes
 *    return MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_AMD_H
#define MOE_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status_t;

typedef enum { MOE_BF16 = 0, MOE_FP8_E4M3 = 1, MOE_FP32 = 2, MOE_MXFP8 = 3 } moe_dtype_t;

/* Score functions (guide, "Router": softmax before or after the top-k, sigmoid,
 * sqrtsoftplus).
 * MOE_SOFTMAX_PRE_RENORM: softmax over all experts, keep the top-k, divide by their
 *   sum (te_mixtral.py, TEMixtralSparseMoeBlock.forward).
 * MOE_SOFTMAX_POST: softmax over the k kept logits (guide, use_pre_softmax=False).
 * MOE_SIGMOID: sigmoid of each kept logit, not renormalised (guide, "Token
 *   combine": sigmoid top-1 weights are not one and must be applied).
 * MOE_SQRTSOFTPLUS: sqrt(log(1 + e^l)) of each kept logit, not renormalised.
 * MOE_SOFTMAX_PRE: softmax over all experts, the kept experts' probabilities as they are,
 *   not renormalised (guide, use_pre_softmax=True; "Token combine": pre-softmax top-1
 *   weights are not one).
 * Selection is on the logits, descending, ties to the lower expert index (with an
 * expert bias: on fp32(score + bias); see moe_router_opts_t). A NaN logit counts as -inf;
 * an expert at -inf is still taken when too few others are left (lowest id first), so
 * the ids are always k distinct experts of [0, E). */
typedef enum {
  MOE_SOFTMAX_PRE_RENORM = 0,
  MOE_SOFTMAX_POST = 1,
  MOE_SIGMOID = 2,
  MOE_SQRTSOFTPLUS = 3,
  MOE_SOFTMAX_PRE = 4
} moe_score_t;

/* Layouts of the grouped GEMM (guide, "Grouped GEMM": Y_i = X_i W_i per expert
 * block, the same result as one product per expert). "rows" is the number of rows
 * of the expert-contiguous buffers; group g owns rows [offsets[g], offsets[g+1]).
 *  MOE_GEMM_NN:    C[rows,N]  = A[rows,K] . B[g][K,N]
 *  MOE_GEMM_NT:    C[rows,N]  = A[rows,K] . B[g][N,K]^T
 *  MOE_GEMM_TN_DW: C[g][M,N]  = A_g[rows_g,M]^T . B_g[rows_g,N]  (weight gradient;
 *                  a group with no rows gets C[g] = 0) */
typedef enum { MOE_GEMM_NN = 0, MOE_GEMM_NT = 1, MOE_GEMM_TN_DW = 2 } moe_gemm_mode_t;

const char* moe_status_str(moe_status_t s);

/* Router: fused score function + top-k (guide, "Router"; all math in fp32).
 *  logits      [T,E] float32 in.
 *  topk_idx    [T,k] int32 out: expert ids, best first.
 *  topk_prob   [T,k] float32 out: routing weights of those experts.
 *  counts      [E]   int32 out: tokens routed to each expert (overwritten).
 *  routing_map [T,E] uint8 out, nullable: 1 at the selected experts, else 0.
 *  probs_dense [T,E] float32 out, nullable: weights at the selected experts, else 0. */
moe_status_t moe_router_topk(const float* logits, int T, int E, int k, int score,
                             int32_t* topk_idx, float* topk_prob, int32_t* counts,
                             uint8_t* routing_map, float* probs_dense, void* stream);

/* Router options (guide, "Router" options and "Load balancing").
 *  expert_bias   [E] float32 or NULL: added to the sigmoid / sqrtsoftplus scores for the
 *                selection only (the weights stay the unbiased scores); with a softmax
 *                score function MOE_ERR_UNSUPPORTED.
 *  num_groups    0 or 1: no grouped routing. Else the experts form num_groups equal
 *                groups of consecutive ids (E % num_groups == 0, num_groups <= 64); a
 *                group's score is the fp32 sum, best first, of the values of its
 *                m = k / group_topk best experts (softmax before the top-k, either
 *                form: the fp32 probabilities; after it: the logits; sigmoid /
 *                sqrtsoftplus: the fp32 scores, plus the bias when given); the
 *                group_topk best groups are kept
 *                and the top-k is taken among their experts (ties to the lower id).
 *  group_topk    groups kept: 1 <= group_topk <= num_groups, k >= group_topk,
 *                k <= group_topk * (E / num_groups).
 *  scaling_factor multiplies the returned weights (0 is taken as 1).
 *  map_format    0: routing_map uint8 [T,E]; 1: bit-packed [T, ceil(E/8)] bytes, bit e%8
 *                of byte e/8 (least significant first) set at the selected experts. */
typedef struct {
  const float* expert_bias;
  int num_groups;
  int group_topk;
  float scaling_factor;
  int map_format;
} moe_router_opts_t;

/* moe_router_topk with options (opts may be NULL: none). Arguments and outputs as
 * moe_router_topk; routing_map in the opts->map_format layout. */
moe_status_t moe_router_topk_ex(const float* logits, int T, int E, int k, int score,
                                const moe_router_opts_t* opts, int32_t* topk_idx,
                                float* topk_prob, int32_t* counts, uint8_t* routing_map,
                                float* probs_dense, void* stream);

/* Auxiliary-loss-free load balancing step (torchtitan pull request 1269,
 * MoE._update_expert_bias; guide, "Load balancing": lower the bias of overloaded experts,
 * raise it for under-used ones), in place on expert_bias [E] float32:
 * bias += coeff * sign(mean(c) - c_e) - mean over experts of that term, c =
 * tokens_per_expert [E] int32 (e.g. the counts of moe_router_topk). The signs are exact
 * (integer comparison); the update is computed in fp64 and rounded once. E <= 256. */
moe_status_t moe_expert_bias_update(float* expert_bias, const int32_t* tokens_per_expert,
                                    int E, float coeff, void* stream);

/* ---- auxiliary load-balancing loss (guide, "Load balancing") --------------------------
 * The loss is the Switch Transformer balance loss (Fedus, Zoph and Shazeer 2021, section
 * 2.2) for top-k routing: coeff * E * sum_e f_e P_e, f_e = c_e / (k T) the fraction of the
 * routed (token, choice) pairs sent to expert e, P_e = sum_t s_te / T the mean dense score:
 *   loss = coeff * E / (k T^2) * sum_e c_e sum_t s_te,  T = total_num_tokens. */

/* Dense scores for the loss (guide: fused_compute_score_for_moe_aux_loss; no expert bias, no
 * grouped routing). logits [T,E] float32 in (a NaN counts as -inf); scores [T,E] float32
 * out, a distribution over the experts per token: the softmax over all experts (any
 * softmax score function), or the sigmoid / sqrtsoftplus scores divided by their sum.
 * routing_map [T,E] uint8 out, nullable: the plain top-k of the logits (as moe_router_topk),
 * which can differ from the real router's when that one uses a bias or groups. */
moe_status_t moe_aux_loss_scores(const float* logits, int T, int E, int k, int score,
                                 float* scores, uint8_t* routing_map, void* stream);

/* Scratch bytes moe_aux_loss needs for (T, E). */
size_t moe_aux_loss_workspace_bytes(int T, int E);

/* The loss (guide: fused_moe_aux_loss). scores [T,E] float32 (moe_aux_loss_scores),
 * tokens_per_expert [E] int32 (the real router's counts), total_num_tokens > 0, coeff the
 * loss weight. loss [1] float32 device out. fp32 column sums over fixed token chunks,
 * added in a fixed order (deterministic). ws: moe_aux_loss_workspace_bytes(T, E). */
moe_status_t moe_aux_loss(const float* scores, const int32_t* tokens_per_expert, int T, int E,
                          int k, int total_num_tokens, float coeff, float* loss, void* ws,
                          size_t ws_bytes, void* stream);

/* Gradient of the loss with respect to every logit, for an upstream gradient d_loss [1]
 * float32 device (NULL: 1). With C = d_loss coeff E / (k T^2), g_e = C c_e and
 * D = sum_i s_i g_i: softmax d_logits[t,e] = s_e (g_e - D); sigmoid / sqrtsoftplus, with r
 * the unnormalised scores, r'(l_e) (g_e - D) / sum_i r_i (r' = r (1 - r), or
 * sigmoid(l) / (2 r)). accumulate = 1 adds to d_logits (e.g. the router backward's), 0
 * overwrites it. */
moe_status_t moe_aux_loss_backward(const float* logits, const int32_t* tokens_per_expert, int T,
                                   int E, int k, int total_num_tokens, float coeff, int score,
                                   const float* d_loss, float* d_logits, int accumulate,
                                   void* stream);

/* Scratch bytes moe_permute needs for (T, E, k). */
size_t moe_permute_workspace_bytes(int T, int E, int k);

/* Token dispatch (guide, "Token dispatch"): expert-contiguous copy of the tokens.
 *  x        [T,H] bf16 in.       topk_idx [T,k] int32 in (ids in [0,E); not checked on the
 *           device: another id makes the kernels write outside the buffers).
 *  out_dtype MOE_BF16: xp [T*k,H] bf16 is a bit copy of the token rows.
 *            MOE_FP8_E4M3: xp [T*k,H] e4m3 codes, xp_scale [T*k] float32: each token
 *            quantised per row, scale = amax/448 (1 for an all-zero row).
 *  offsets  [E+1] int32 out: offsets[e] = rows of experts < e; offsets[E] = T*k.
 *  row_of   [T,k] int32 out: row of token t's j-th choice. Inside a block rows
 *            follow ascending token index.
 *  src_of   [T*k] int32 out: token that fills each row.
 *  ws/ws_bytes: scratch of at least moe_permute_workspace_bytes(T,E,k) bytes. */
moe_status_t moe_permute(const void* x, const int32_t* topk_idx, int T, int H, int E, int k,
                         int out_dtype, void* xp, float* xp_scale, int32_t* offsets,
                         int32_t* row_of, int32_t* src_of, void* ws, size_t ws_bytes,
                         void* stream);

/* moe_permute for callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops or harnesses that forbid hipMalloc): the same arguments and results minus
 * the workspace. The dispatch scratch lives in a device array of the library of
 * moe_permute_noalloc_limit() bytes (4 MiB) that each GPU holds until the process ends; the
 * call allocates nothing. Sizes whose scratch, moe_permute_workspace_bytes(T, E, k), exceeds
 * the limit return MOE_ERR_UNSUPPORTED (e.g. E = 256 allows T*k up to 1048320). Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (several streams, or a
 * graph replay during an eager call) race and must be serialised by the caller. */
moe_status_t moe_permute_noalloc(const void* x, const int32_t* topk_idx, int T, int H, int E,
                                 int k, int out_dtype, void* xp, float* xp_scale,
                                 int32_t* offsets, int32_t* row_of, int32_t* src_of,
                                 void* stream);

/* Bytes of the device scratch array moe_permute_noalloc uses. */
size_t moe_permute_noalloc_limit(void);

/* Rows a padded dispatch needs at most: T*k + E*(align-1) (align > 1), else T*k (guide,
 * "Receive buffer": counts of 129 and 127 need 384 rows at alignment 128). */
size_t moe_padded_rows(int T, int E, int k, int align);

/* Padded token dispatch (guide, "Padding and alignment"): moe_permute with every expert
 * block rounded up to a multiple of `align` rows (1 <= align <= 4096).
 *  xp [moe_padded_rows(T,E,k,align), H] (bf16, or e4m3 with xp_scale): token rows at
 *  row_of, padding rows zero (fp8 scale 1); rows past offsets[E] are not written.
 *  offsets [E+1] out: padded block starts (offsets[E] = the padded total).
 *  pad_offsets [E] out: padding rows before block e (cumulative; 0 for e = 0).
 *  src_of [moe_padded_rows] out: token of each row, -1 for padding rows.
 *  ws: at least moe_permute_workspace_bytes(T,E,k) bytes. Combine needs nothing more:
 *  row_of already points into the padded layout. */
moe_status_t moe_permute_padded(const void* x, const int32_t* topk_idx, int T, int H, int E,
                                int k, int align, int out_dtype, void* xp, float* xp_scale,
                                int32_t* offsets, int32_t* pad_offsets, int32_t* row_of,
                                int32_t* src_of, void* ws, size_t ws_bytes, void* stream);

/* Grouped GEMM1 with the SwiGLU epilogue (guide, "Grouped MLP": FC1 with the
 * activation fused, FC2 separate; te_mixtral.py _expert_ffn: gate/up fused weight,
 * silu(gate) * up).
 *  xp      [rows,H] bf16 (dtype MOE_BF16) or e4m3 codes (MOE_FP8_E4M3) in.
 *  xp_scale [rows] float32 per-row scales (fp8 only, else NULL).
 *  w_gu    bf16: [G,H,2I], gate = columns [0,I), up = columns [I,2I).
 *          fp8:  [G,2I,H] e4m3 codes (output-channel major, as written by
 *                moe_quantize_fp8_weights), w_scale [G,2I] float32.
 *  offsets [G+1] int32 device group boundaries.
 *  h       [rows,I] bf16 out: silu(g) * u, g and u held in fp32.
 *  gu_saved [rows,2I] bf16 out, nullable: g and u rounded to bf16 (for backward).
 *  ws, ws_bytes: nullable split-K space (see moe_grouped_gemm_splitk_workspace_bytes with
 *          ncols = 2I); ignored by shapes that never split; a space smaller than that size
 *          returns MOE_ERR_INVALID_ARG before any launch. */
moe_status_t moe_grouped_gemm_swiglu(const void* xp, const float* xp_scale, const void* w_gu,
                                     const float* w_scale, const int32_t* offsets, int G,
                                     int rows, int H, int I, int dtype, void* h, void* gu_saved,
                                     void* ws, size_t ws_bytes, void* stream);

/* Grouped GEMM (guide, "Grouped GEMM"); see moe_gemm_mode_t for the layouts.
 *  dtype MOE_BF16: A, B bf16.  MOE_FP8_E4M3 (mode NT only): A e4m3 [rows,K] with
 *  a_scale [rows], B e4m3 [G][N,K] with b_scale [G,N]; C = acc * a_scale * b_scale.
 *  c_dtype MOE_BF16 or MOE_FP32 (fp32 accumulation in every case). M is used by
 *  MOE_GEMM_TN_DW only, K by NN/NT only.
 *  ws, ws_bytes: nullable split-K space (moe_grouped_gemm_splitk_workspace_bytes with
 *  ncols = N); ignored by shapes that never split; a space smaller than that size returns
 *  MOE_ERR_INVALID_ARG before any launch. */
moe_status_t moe_grouped_gemm(int mode, const void* A, const float* a_scale, const void* B,
                              const float* b_scale, const int32_t* offsets, int G, int rows,
                              int M, int N, int K, int dtype, void* C, int c_dtype, void* ws,
                              size_t ws_bytes, void* stream);

/* Split-K space of a bf16 NN/NT grouped GEMM (moe_grouped_gemm_swiglu: ncols = 2I;
 * moe_grouped_gemm: ncols = N) over `rows` rows in G groups; 0 for shapes that never split.
 * Only decode-sized launches split (at most 256 rows and at most 32 rows per group on
 * average: one 32-row tile per expert, so a few wide tiles per expert would leave compute
 * units idle): each tile's reduction over K is cut into up to 8 parts, chosen on the device
 * from the exact tile count; the parts' fp32 sums go to this space and a second launch adds
 * them in part order and applies the epilogue. Results equal the unsplit launch's up to the
 * order of the fp32 additions. The caller owns the space; concurrent launches need their
 * own. The layer's forward (moe_forward) keeps its own in the layer workspace. */
size_t moe_grouped_gemm_splitk_workspace_bytes(int rows, int G, int ncols);

/* Backward of GEMM2 + SwiGLU: dh = d_out[rows,H] . W_down[g][I,H]^T (layout NT), then
 *  with the saved bf16 g,u and s = sigmoid(g): dg = dh*u*s*(1+g*(1-s)), du = dh*g*s,
 *  written as dgu [rows,2I] bf16 (dg in [0,I), du in [I,2I)). */
moe_status_t moe_grouped_gemm_swiglu_bwd(const void* d_out, const void* w_down,
                                         const int32_t* offsets, const void* gu_saved, int G,
                                         int rows, int H, int I, void* dgu, void* stream);

/* ScaledSwiGLU (guide, "Grouped MLP": the activation output is multiplied by the routing
 * weights before FC2; with a bias-free FC2 the expert output is then already weighted and
 * the combine sums unweighted). bf16 only. As moe_grouped_gemm_swiglu, with
 * h[r] = bf16(silu(g) u row_scale[r]) (one fp32 product of g, u, weight, one rounding).
 *  row_scale [rows] float32: the routing weight of each routed row (moe_permute_probs). */
moe_status_t moe_grouped_gemm_swiglu_scaled(const void* xp, const void* w_gu,
                                            const int32_t* offsets, const float* row_scale, int G,
                                            int rows, int H, int I, void* h, void* gu_saved,
                                            void* stream);

/* Backward of FC2 + ScaledSwiGLU: dh = d_out . W_down[g]^T (the gradient of the scaled h),
 * then as moe_grouped_gemm_swiglu_bwd with dh * row_scale[r]. d_scale_part [rows, I/64]
 * float32 out, nullable: per row and block of 64 h columns, sum_c dh[r,c] silu(g) u from the
 * saved bf16 g, u (fp32); the weight gradient of row r is the sum of its I/64 values. */
moe_status_t moe_grouped_gemm_swiglu_scaled_bwd(const void* d_out, const void* w_down,
                                                const int32_t* offsets, const void* gu_saved,
                                                const float* row_scale, int G, int rows, int H,
                                                int I, void* dgu, float* d_scale_part,
                                                void* stream);

/* The routing weight of every routed row (guide, "Token dispatch": the permuted
 * probabilities): row_prob[row_of[t,j]] = topk_prob[t,j]. row_of, topk_prob [T,k];
 * row_prob [T*k] float32 out (rows of a padded dispatch's padding are not written). */
moe_status_t moe_permute_probs(const int32_t* row_of, const float* topk_prob, int T, int k,
                               float* row_prob, void* stream);

/* Cap on the persistent grid of every grouped-GEMM launch (the entry points above and
 * the ones inside moe_forward / moe_backward). Each launch runs min(tiles, resident)
 * blocks, resident = compute units x blocks per unit, and every block walks its share of
 * the tiles. max_blocks > 0 lowers the cap to that many blocks (leaving compute units to
 * concurrent work, or forcing many tiles per block); 0 restores the default. Process-wide
 * host setting, read once by each launch as it is enqueued (an atomic: any host thread may
 * set it; launches already enqueued keep the grid they were given). MOE_ERR_INVALID_ARG for
 * max_blocks < 0. */
moe_status_t moe_set_gemm_max_blocks(int max_blocks);

/* Token combine (guide, "Token combine"): y[t] = sum_j p[t,j] * y_perm[row_of[t,j]]
 * (+ shared_out[t]), summed in fp32, one rounding to bf16.
 *  y_perm [T*k,H] bf16, row_of [T,k], topk_prob [T,k] float32 or NULL (unweighted
 *  sum: the dispatch backward), shared_out [T,H] bf16 or NULL, y [T,H] bf16 out. */
moe_status_t moe_unpermute_combine(const void* y_perm, const int32_t* row_of,
                                   const float* topk_prob, const void* shared_out, int T,
                                   int H, int k, void* y, void* stream);

/* Backward of the weighted combine: d_out[row_of[t,j]] = bf16(p[t,j] * dy[t]). */
moe_status_t moe_combine_backward(const void* dy, const int32_t* row_of, const float* topk_prob,
                                  int T, int H, int k, void* d_out, void* stream);

/* Per-row e4m3 quantisation of a bf16 matrix x [R,C]: scale[r] = amax_r/448 (1 for a
 * zero row), q = e4m3(x/scale), nearest-even, saturating. */
moe_status_t moe_quantize_fp8_rows(const void* x, int R, int C, uint8_t* q, float* scale,
                                   void* stream);

/* Offline weight preparation for the fp8 recipe: per-output-channel e4m3
 * quantisation of w [G,K,N] bf16, one scale per (g, n) over K. Writes the codes
 * output-channel major, q [G,N,K], and scale [G,N]. */
moe_status_t moe_quantize_fp8_weights(const void* w, int G, int K, int N, uint8_t* q,
                                      float* scale, void* stream);

/* ---- router projection and router backward -------------------------------------- */

/* Router projection (guide, "Example: MoE layer on a single device": the logits come
 * from a bias-free linear layer of the hidden states; te_mixtral.py,
 * TEMixtralSparseMoeBlock: gate of shape (experts, hidden)).
 *  x [T,H] bf16, w_router [E,H] bf16 in; logits [T,E] float32 out:
 *  logits[t,e] = sum_h x[t,h] w_router[e,h], fp32 accumulation, no bf16 rounding (the
 *  router's math runs in fp32). */
moe_status_t moe_router_logits(const void* x, const void* w_router, int T, int H, int E,
                               float* logits, void* stream);

/* Combine backward with the routing-weight gradient (guide, "Token combine": the merging
 * weights are an input of the differentiable combine; "Router": the score function and
 * top-k are differentiable with fp32 math).
 *  dy [T,H] bf16, expert_out [T*k,H] bf16 (the forward's expert outputs before
 *  weighting), row_of [T,k], topk_idx [T,k], topk_prob [T,k] float32, score as in
 *  the forward. logits [T,E] float32: read for MOE_SOFTMAX_PRE only (else may be NULL).
 *  d_out [T*k,H] bf16 out: d_out[row_of[t,j]] = bf16(p[t,j] * dy[t]).
 *  d_prob [T,k] float32 out, nullable: <dy[t], expert_out[row_of[t,j]]> (fp32 sum).
 *  d_logits [T,E] float32 out: with p = c s (c = scaling_factor, 0 taken as 1; s the
 *  score-function output), at the kept experts softmax (every form) c s_j (d_prob_j -
 *  sum_i s_i d_prob_i), sigmoid c d_prob_j s_j (1 - s_j), sqrtsoftplus
 *  c d_prob_j sigmoid(l_j) / (2 s_j). At the other experts 0 (the top-k choice is
 *  piecewise constant), except for MOE_SOFTMAX_PRE, whose weights are probabilities of
 *  a softmax over every expert: -c p_e sum_i s_i d_prob_i, p_e the softmax of logits. */
moe_status_t moe_combine_backward_router(const void* dy, const void* expert_out,
                                         const int32_t* row_of, const int32_t* topk_idx,
                                         const float* topk_prob, const float* logits, int T,
                                         int H, int E, int k, int score, float scaling_factor,
                                         void* d_out, float* d_prob, float* d_logits,
                                         void* stream);

/* Scratch bytes moe_router_weight_grad needs for (T, H, E). */
size_t moe_router_weight_grad_workspace_bytes(int T, int H, int E);

/* Router weight gradient dw_router [E,H] float32 = d_logits[T,E]^T . x[T,H]. Each d_logits
 * value enters the bf16 matrix-core product as two bf16 halves (hi = bf16(d),
 * lo = bf16(d - hi)), about 16 significant bits; the K = T reduction is split into
 * ranges whose fp32 partial products are summed in a fixed order (deterministic).
 *  ws: at least moe_router_weight_grad_workspace_bytes(T,H,E) bytes. T == 0 writes zeros. */
moe_status_t moe_router_weight_grad(const void* x, const float* d_logits, int T, int H, int E,
                                    float* dw_router, void* ws, size_t ws_bytes, void* stream);

/* Dispatch backward of a layer that owns its router projection: dx[t] =
 * bf16(sum_j dxp[row_of[t,j]] + sum_e d_logits[t,e] w_router[e]), summed in fp32 with one
 * rounding; the router's term runs over the experts whose d_logits is nonzero, in
 * ascending id (the kept ones, topk_idx, for every score function but MOE_SOFTMAX_PRE,
 * whose d_logits reaches every expert). topk_idx is checked but not read. */
moe_status_t moe_dispatch_backward_router(const void* dxp, const int32_t* row_of,
                                          const int32_t* topk_idx, const float* d_logits,
                                          const void* w_router, int T, int H, int E, int k,
                                          void* dx, void* stream);

/* Dispatch backward of a layer whose routing weights scale the expert inputs and which
 * owns its router projection (torchtitan pull request 1269, MoE.forward,
 * scoring_before_experts; the weighted dispatch itself is moe_combine_backward applied to
 * x, and without the router the dispatch backward is moe_unpermute_combine with the
 * weights). dxp [T*k,H] bf16, x [T,H] bf16, row_of, topk_idx, topk_prob [T,k], logits
 * [T,E] float32 (read for MOE_SOFTMAX_PRE only), w_router [E,H] bf16, score /
 * scaling_factor as in the forward.
 *  d_logits [T,E] float32 out: the score-function backward (see
 *  moe_combine_backward_router) of d_prob_j = <dxp[row_of[t,j]], x[t]>.
 *  dx [T,H] bf16 out: bf16(sum_j p_j dxp[row_of[t,j]] + sum_e d_logits[t,e] w_router[e]),
 *  fp32 sum with one rounding. */
moe_status_t moe_dispatch_backward_router_input(const void* dxp, const void* x,
                                                const int32_t* row_of, const int32_t* topk_idx,
                                                const float* topk_prob, const float* logits,
                                                const void* w_router, int T, int H, int E, int k,
                                                int score, float scaling_factor, void* dx,
                                                float* d_logits, void* stream);

/* Dispatch backward of a ScaledSwiGLU layer that owns its router projection: d_prob[t,j] =
 * the sum, in a fixed order, of the I/64 partials d_scale_part [rows, I/64] of row
 * row_of[t,j] (moe_grouped_gemm_swiglu_scaled_bwd); d_logits [T,E] out, its score-function
 * backward (see moe_combine_backward_router; logits read for MOE_SOFTMAX_PRE only);
 * dx [T,H] bf16 out: bf16(sum_j dxp[row_of[t,j]] + sum_e d_logits[t,e] w_router[e]). */
moe_status_t moe_dispatch_backward_router_scaled(const void* dxp, const float* d_scale_part,
                                                 const int32_t* row_of, const int32_t* topk_idx,
                                                 const float* topk_prob, const float* logits,
                                                 const void* w_router, int T, int H, int E, int k,
                                                 int I, int score, float scaling_factor, void* dx,
                                                 float* d_logits, void* stream);

/* ---- MXFP8 (te_mixtral.py's mxfp8 recipe) ------------------------------------------
 * e4m3 codes with one power-of-two scale per block of 32 consecutive values along K,
 * stored as a byte (E8M0: log2(scale) + 127). Conversion of a block (OCP Microscaling
 * v1.0): scale = 2^(floor(log2(amax)) - 8), clamped to [2^-127, 2^127], 2^-127 for an
 * all-zero block; code = e4m3(v / scale), nearest-even, saturating to +-448. */

/* x [R,C] bf16 (C % 32 == 0) -> q [R,C] codes, scale [R,C/32] bytes. */
moe_status_t moe_quantize_mxfp8_rows(const void* x, int R, int C, uint8_t* q, uint8_t* scale,
                                     void* stream);

/* Offline weight preparation: w [G,K,N] bf16 (K % 32 == 0) -> q [G,N,K] codes (output
 * channel major) and scale [G,N,K/32] bytes, blocks along K. */
moe_status_t moe_quantize_mxfp8_weights(const void* w, int G, int K, int N, uint8_t* q,
                                        uint8_t* scale, void* stream);

/* Block-scaled grouped GEMM (layout NT): C[r,n] = sum over K blocks of
 * scale_A[r,b] scale_B[g][n,b] sum_{k in b} A[r,k] B[g][n,k], fp32 accumulation, the scales
 * applied by the matrix-core instruction. A [rows,K] codes + a_scale [rows,K/32]; B [G,N,K]
 * codes + b_scale [G,N,K/32]; offsets [G+1] device. swiglu = 0: C bf16 [rows,N]
 * (N % 64 == 0). swiglu = 1: N = 2I (gate columns [0,I), up [I,2I), I % 64 == 0) and
 * C = h bf16 [rows,I] = silu(g) u. K % 64 == 0. */
moe_status_t moe_grouped_gemm_mxfp8(const uint8_t* A, const uint8_t* a_scale, const uint8_t* B,
                                    const uint8_t* b_scale, const int32_t* offsets, int G,
                                    int rows, int N, int K, int swiglu, void* C, void* stream);

/* MXFP8 backward (the same recipe in the training step). The data-gradient GEMMs take
 * operands quantised along their own K: d_out rows and dgu rows with
 * moe_quantize_mxfp8_rows, and the weights as stored (w_down [E,I,H] as rows of H,
 * w_gu [E,H,2I] as rows of 2I), also with moe_quantize_mxfp8_rows. The weight-gradient
 * GEMMs reduce over each expert's rows, so their operands are quantised along the token
 * axis, in blocks of 32 that start at every expert's first row: expert g's rows go to
 * columns [co[g], co[g] + roundup(n_g, 64)) of a transposed operand [C, Kp], the columns
 * past its rows holding zero codes (as if the expert's rows were padded with zero rows,
 * te_mixtral.py's mxfp8 recipe padding every expert's split). */

/* Columns a transposed operand needs: roundup(R + 63 G, 64) (-1 on bad arguments). */
long long moe_mxfp8_cols_capacity(int R, int G);

/* co [G+1] device out: co[0] = 0, co[g+1] = co[g] + roundup(offsets[g+1] - offsets[g], 64)
 * from the row offsets [G+1] (device). */
moe_status_t moe_mxfp8_col_offsets(const int32_t* offsets, int G, int32_t* col_offsets,
                                   void* stream);

/* x [R,C] bf16 expert-contiguous rows (C % 8 == 0), offsets [G+1] and col_offsets [G+1]
 * (moe_mxfp8_col_offsets) device -> qt [C,Kp] codes and scale_t [C,Kp/32] bytes, the
 * token axis blocked per expert as above. Kp % 64 == 0 and Kp >= moe_mxfp8_cols_capacity;
 * columns at and past co[G] are not written. */
moe_status_t moe_quantize_mxfp8_cols(const void* x, int R, int C, const int32_t* offsets,
                                     const int32_t* col_offsets, int G, int Kp, uint8_t* qt,
                                     uint8_t* scale_t, void* stream);

/* Weight-gradient GEMM: C[g] [M,N] bf16 = sum over the columns k in [co[g], co[g+1]) of
 * scale_A scale_B At[m,k] Bt[n,k] (fp32 accumulation, block scales in the instruction).
 * At [M,Kp] + a_scale [M,Kp/32], Bt [N,Kp] + b_scale [N,Kp/32] (moe_quantize_mxfp8_cols);
 * C [G,M,N]; an expert with no rows gets zeros. M % 64 == 0, N % 64 == 0. */
moe_status_t moe_grouped_gemm_mxfp8_wgrad(const uint8_t* At, const uint8_t* a_scale,
                                          const uint8_t* Bt, const uint8_t* b_scale,
                                          const int32_t* col_offsets, int G, int M, int N, int Kp,
                                          void* C, void* stream);

/* GEMM2 data gradient with the SwiGLU backward: dh = A B^T per expert as in
 * moe_grouped_gemm_mxfp8 (A = d_out codes [rows,K=H], B = w_down codes [G,I,H]), then from
 * the saved gu [rows,2I] bf16 (gate columns first), s = sigmoid(g):
 * dgu [rows,2I] bf16 = [dh u s (1 + g (1 - s)), dh g s]. I % 64 == 0, K % 64 == 0. */
moe_status_t moe_grouped_gemm_mxfp8_swiglu_bwd(const uint8_t* A, const uint8_t* a_scale,
                                               const uint8_t* B, const uint8_t* b_scale,
                                               const int32_t* offsets, int G, int rows, int I,
                                               int K, const void* gu, void* dgu, void* stream);

/* ---- whole layer ------------------------------------------------------------ */

typedef struct {
  int T, H, E, k, I;
  int shared_I;  /* 0: no shared expert; else a dense SwiGLU MLP of width shared_I,
                    unweighted, added in combine (torchtitan pull request 1269,
                    MoE.forward) */
  int score;     /* moe_score_t */
  int dtype;     /* expert GEMMs: MOE_BF16, MOE_FP8_E4M3 (forward only) or MOE_MXFP8 (the
                    weight tensors then hold moe_quantize_mxfp8_weights codes, and the
                    *_scale pointers their scale bytes, [E,2I,H/32] and [E,H,I/32];
                    training also takes the *_bwd copies) */
  int training;  /* 1: keep what moe_backward needs in the workspace */
  int router;    /* 1: the layer owns its router projection: moe_forward computes the
                    logits from x and w_router (into the workspace; t->logits is not
                    read) and moe_backward also returns dw_router and adds the router's
                    term to dx */
  int num_groups;        /* grouped routing, as moe_router_opts_t (0: none) */
  int group_topk;
  float scaling_factor;  /* multiplies the routing weights (0 is taken as 1) */
  int weight_placement;  /* MOE_PLACE_COMBINE (0): the weights scale the expert outputs in
                            the combine; MOE_PLACE_INPUT (1, bf16 only): they scale the
                            routed input rows, xp[r] = bf16(q x[t]), and the combine sums
                            unweighted (torchtitan pull request 1269, MoE.forward,
                            scoring_before_experts); MOE_PLACE_ACTIVATION (2, bf16 only):
                            they scale the SwiGLU output, h = bf16(silu(g) u q), and the
                            combine sums unweighted (guide, "Grouped MLP", ScaledSwiGLU) */
  int align_size;        /* 0 or 1: no padding. Else a padded dispatch (guide, "Padding and
                            alignment"): every expert block starts at a multiple of
                            align_size rows (<= 4096), padding rows are zero; the row
                            buffers hold T*k + E*(align_size-1) rows */
} moe_problem_t;

enum { MOE_PLACE_COMBINE = 0, MOE_PLACE_INPUT = 1, MOE_PLACE_ACTIVATION = 2 };

typedef struct {
  const void* x;              /* [T,H] bf16 */
  const float* logits;        /* [T,E] */
  const void* w_gu;           /* bf16 [E,H,2I]  | fp8 [E,2I,H] codes */
  const float* w_gu_scale;    /* fp8: [E,2I] */
  const void* w_down;         /* bf16 [E,I,H]   | fp8 [E,H,I] codes */
  const float* w_down_scale;  /* fp8: [E,H] */
  const void* shared_gu;      /* bf16 [H,2*shared_I] or NULL */
  const void* shared_down;    /* bf16 [shared_I,H] or NULL */
  void* y;                    /* [T,H] bf16 out */
  const void* w_router;       /* bf16 [E,H] (router = 1), else NULL */
  float* dw_router;           /* [E,H] float32 out of moe_backward (router = 1), else NULL */
  const float* expert_bias;   /* [E] selection bias (sigmoid / sqrtsoftplus) or NULL */
  /* MOE_MXFP8 training: the weights' second MXFP8 copy, blocked along the stored last
     axis, for the data gradients (moe_quantize_mxfp8_rows of w_gu as [E*H,2I] and of
     w_down as [E*I,H]); NULL otherwise */
  const void* w_gu_bwd;             /* [E,H,2I] codes */
  const uint8_t* w_gu_bwd_scale;    /* [E,H,2I/32] */
  const void* w_down_bwd;           /* [E,I,H] codes */
  const uint8_t* w_down_bwd_scale;  /* [E,I,H/32] */
} moe_tensors_t;

/* Device pointers into a forward workspace (all inside ws). */
typedef struct {
  int32_t* topk_idx;   /* [T,k] */
  float* topk_prob;    /* [T,k] */
  int32_t* counts;     /* [E] */
  int32_t* offsets;    /* [E+1] (padded block starts when align_size > 1) */
  int32_t* row_of;     /* [T,k] */
  int32_t* src_of;     /* [T*k] */
  void* xp;            /* [T*k,H] bf16 (or e4m3) */
  float* xp_scale;     /* [T*k] (fp8) */
  void* gu;            /* [T*k,2I] bf16 (training) */
  void* h;             /* [T*k,I] bf16 */
  uint8_t* hq;         /* [T*k,I] e4m3 (fp8) */
  float* h_scale;      /* [T*k] (fp8) */
  void* out;           /* [T*k,H] bf16 */
  void* xq;            /* [rows,H] MXFP8 codes (MOE_MXFP8) */
  uint8_t* xq_scale;   /* [rows,H/32] scale bytes (MOE_MXFP8) */
  uint8_t* hq_scale;   /* [rows,I/32] scale bytes (MOE_MXFP8; codes in hq) */
  void* shared_h;      /* [T,shared_I] bf16 */
  void* shared_out;    /* [T,H] bf16 */
  int32_t* shared_offsets; /* [2] = {0, T} */
  void* d_out;         /* [T*k,H] bf16 (training) */
  void* dgu;           /* [T*k,2I] bf16 (training) */
  void* dxp;           /* [T*k,H] bf16 (training) */
  void* scratch;       /* moe_permute scratch */
  size_t scratch_bytes;
  int32_t* pad_offsets; /* [E] padding before each expert block (align_size > 1) */
  int rows;            /* rows of the expert-contiguous buffers below: T*k (+ padding) */
  float* logits;       /* [T,E] (router = 1) */
  float* d_logits;     /* [T,E] (router = 1, training) */
  void* router_ws;     /* moe_router_weight_grad scratch (router = 1, training) */
  size_t router_ws_bytes;
  /* MOE_MXFP8 training */
  int32_t* mx_col_offsets;  /* [E+1] expert starts along the token axis (multiples of 64) */
  uint8_t* dgq;             /* [rows,2I] dgu codes */
  uint8_t* dgq_scale;       /* [rows,2I/32] */
  uint8_t* mx_ta;           /* [max(H,I),mx_kp] token-axis codes: h, then xp */
  uint8_t* mx_ta_scale;
  uint8_t* mx_tb;           /* [max(H,2I),mx_kp] token-axis codes: d_out, then dgu */
  uint8_t* mx_tb_scale;
  int mx_kp;                /* moe_mxfp8_cols_capacity(rows, E) */
} moe_views_t;

/* Bytes of workspace moe_forward (and, when training, moe_backward) needs. */
size_t moe_workspace_bytes(const moe_problem_t* p);

/* Fill `v` with the pointers of every intermediate inside workspace `ws`. */
moe_status_t moe_workspace_views(const moe_problem_t* p, void* ws, size_t ws_bytes,
                                 moe_views_t* v);

/* Whole forward: router -> dispatch -> grouped SwiGLU MLP -> combine, enqueued on
 * `stream` with no host synchronisation. All intermediates live in `ws`, which
 * moe_backward later reads: keep it untouched between the two calls. */
moe_status_t moe_forward(const moe_problem_t* p, const moe_tensors_t* t, void* ws,
                         size_t ws_bytes, void* stream);

/* Backward of the layer for upstream gradient dy [T,H] bf16 (bf16 or MXFP8 MLP, training=1
 * forward only): dx [T,H] bf16, dw_gu [E,H,2I] bf16, dw_down [E,I,H] bf16. MXFP8: the
 * GEMMs of moe_grouped_gemm_mxfp8_swiglu_bwd, moe_grouped_gemm_mxfp8 and
 * moe_grouped_gemm_mxfp8_wgrad on the operands described above them. With
 * router = 0 the logits are an input of the layer and no gradient flows to the router.
 * With router = 1 (t->x and t->w_router as in the forward) it also writes
 * t->dw_router [E,H] float32 and d_logits into the workspace, and dx includes the
 * router's term; the stages are moe_combine_backward_router, the GEMM backward,
 * moe_router_weight_grad and moe_dispatch_backward_router. */
moe_status_t moe_backward(const moe_problem_t* p, const moe_tensors_t* t, const void* dy,
                          void* dx, void* dw_gu, void* dw_down, void* ws, size_t ws_bytes,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_AMD_H */
