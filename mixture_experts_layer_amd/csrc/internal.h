// Internal launchers (host side) shared by the C-ABI layer. Not exported.
#pragma once

#include "common.h"

namespace moe {

// mx.hip: MXFP8 (e4m3 codes, one E8M0 scale byte per 32 along K)
// The dispatch copy (times prob[t,j] when given) fused with the MXFP8 row quantisation of
// its copies: xp rows (bf16, H values) plus their e4m3 codes q and block scales (H % 32 == 0).
hipError_t launch_scatter_rows_mx(const void* x, const int32_t* row_of, const float* prob, int T,
                                  int H, int k, void* xp, uint8_t* q, uint8_t* scale, hipStream_t s);
hipError_t launch_mx_quantize_rows(const void* x, int R, int C, uint8_t* q, uint8_t* scale,
                                   hipStream_t s);
hipError_t launch_mx_quantize_weights(const void* w, int G, int K, int N, uint8_t* q,
                                      uint8_t* scale, hipStream_t s);
// epi EPI_STORE: C bf16 [rows, N]; EPI_SWIGLU: N = 2I, C = h bf16 [rows, I] (and g,u into
// gu_out [rows, 2I] when not null); EPI_SWIGLU_BWD: N = I, C = dgu bf16 [rows, 2I] from
// dh = A B^T and the saved g,u in gu_in [rows, 2I]
hipError_t launch_mx_gemm(int epi, const void* A, const uint8_t* sa, const void* B,
                          const uint8_t* sb, const int32_t* offsets, int G, int rows, int N,
                          int K, int I, void* C, hipStream_t s, const void* gu_in = nullptr,
                          void* gu_out = nullptr);
// Weight-gradient layout: expert ranges along the token axis padded to multiples of 64.
constexpr int kMxColAlign = 64;
inline long long mx_cols_capacity(long long R, long long G) {
  return (R + (kMxColAlign - 1) * G + kMxColAlign - 1) / kMxColAlign * kMxColAlign;
}
hipError_t launch_mx_col_offsets(const int32_t* offsets, int G, int32_t* col_offsets,
                                 hipStream_t s);
// x [R, C] bf16 expert-contiguous rows -> qt [C, Kp] codes, st [C, Kp/32] scale bytes
hipError_t launch_mx_quantize_cols(const void* x, int R, int C, const int32_t* offsets,
                                   const int32_t* col_offsets, int G, int Kp, uint8_t* qt,
                                   uint8_t* st, hipStream_t s);
// C[g] [M, N] bf16 = At[:, co[g]:co[g+1]] Bt[:, co[g]:co[g+1]]^T with block scales
hipError_t launch_mx_gemm_wgrad(const void* At, const uint8_t* sa, const void* Bt,
                                const uint8_t* sb, const int32_t* col_offsets, int G, int M,
                                int N, int Kp, void* C, hipStream_t s);

// Router options (router_opts.hip). Plain: none of them set.
struct RouterOpts {
  const float* expert_bias;  // [E] or null: added to sigmoid / sqrtsoftplus scores to select
  int num_groups;            // <= 1: no grouped routing
  int group_topk;            // groups kept
  float scaling;             // multiplies the weights
  int bitmap;                // routing_map bit-packed [T, ceil(E/8)]
};
inline bool router_opts_plain(const RouterOpts& o, int score) {
  return o.expert_bias == nullptr && o.num_groups <= 1 && o.scaling == 1.0f && !o.bitmap &&
         score != MOE_SQRTSOFTPLUS;
}
// chunk_tokens > 0: per-chunk histograms into counts[chunk][E] (as launch_router_hist);
// 0: counts [E] zeroed then accumulated.
hipError_t launch_router_ext(const float* logits, int T, int E, int k, int score,
                             const RouterOpts& o, int32_t* topk_idx, float* topk_prob,
                             int32_t* counts, uint8_t* routing_map, float* probs_dense,
                             int chunk_tokens, hipStream_t s);
hipError_t launch_expert_bias_update(float* bias, const int32_t* tokens_per_expert, int E,
                                     float coeff, hipStream_t s);

// aux_loss.hip: the auxiliary load-balancing loss (C = coeff E / (k T^2), host-computed)
hipError_t launch_aux_scores(const float* logits, int T, int E, int k, int score, float* scores,
                             uint8_t* routing_map, hipStream_t s);
size_t aux_loss_scratch_bytes(int T, int E);
hipError_t launch_aux_loss(const float* scores, const int32_t* counts, int T, int E, float C,
                           float* loss, float* part, hipStream_t s);
hipError_t launch_aux_loss_bwd(const float* logits, int T, int E, int score, const int32_t* counts,
                               float C, const float* d_loss, float* d_logits, int accumulate,
                               hipStream_t s);

// noalloc.hip: moe_permute with its scratch in the library's device array
size_t permute_noalloc_scratch_limit();
hipError_t launch_permute_noalloc(const void* x, const int32_t* topk_idx, int T, int H, int E,
                                  int k, int out_dtype, void* xp, float* xp_scale,
                                  int32_t* offsets, int32_t* row_of, int32_t* src_of,
                                  hipStream_t s);

// router.hip
hipError_t launch_router_topk(const float* logits, int T, int E, int k, int score,
                              int32_t* topk_idx, float* topk_prob, int32_t* counts,
                              uint8_t* routing_map, float* probs_dense, hipStream_t s);
// Router that also writes the per-expert histogram of each chunk of `chunk_tokens`
// tokens to partial[chunk][E] (input of launch_dispatch_from_hist).
// Routing, dispatch metadata and row copies of a step of at most 32 tokens and 256
// choices (k <= 16, E <= 256, H % 8 == 0) in one launch, for the plain router options:
// the same topk_idx, topk_prob, counts, offsets (offsets[E + 1] = extra_end when >= 0),
// row_of, src_of and xp as launch_router_hist + launch_dispatch_from_hist +
// launch_scatter_rows; zero16 (nullable): 16 ints set to zero.
bool route_dispatch_small_fits(int T, int E, int k);
hipError_t launch_route_dispatch_small(const float* logits, int T, int E, int k, int score,
                                       int32_t* topk_idx, float* topk_prob, int32_t* counts,
                                       int32_t* offsets, int32_t* row_of, int32_t* src_of,
                                       const void* x, int H, void* xp, int extra_end,
                                       int32_t* zero16, hipStream_t s);
hipError_t launch_router_hist(const float* logits, int T, int E, int k, int score,
                              int32_t* topk_idx, float* topk_prob, int32_t* partial,
                              int chunk_tokens, hipStream_t s);

// permute.hip
constexpr int kPermChunk = 256;  // flattened (token, slot) entries per dispatch chunk
size_t permute_scratch_bytes(int T, int E, int k);
int router_chunk_tokens(int T);
// align > 1: padded dispatch (blocks rounded up to multiples of align; offsets padded,
// pad_offsets [E] = padding before each block when given). extra_end >= 0: also write
// offsets[E + 1] = extra_end (the end of one more group after the experts). zero16: 16 ints
// set to zero (the layer's GEMM tile counters).
hipError_t launch_dispatch_from_hist(const int32_t* topk_idx, int T, int E, int k, int chunk_tokens,
                                     int32_t* partial, int32_t* counts, int32_t* offsets,
                                     int32_t* row_of, int32_t* src_of, hipStream_t s,
                                     int align = 1, int32_t* pad_offsets = nullptr,
                                     int extra_end = -1, int32_t* zero16 = nullptr);
hipError_t launch_dispatch_meta(const int32_t* topk_idx, int T, int E, int k, int32_t* offsets,
                                int32_t* row_of, int32_t* src_of, void* scratch, hipStream_t s,
                                int align = 1, int32_t* pad_offsets = nullptr,
                                int32_t* counts = nullptr);
// zero the padding rows of a padded dispatch (and set their fp8 scale 1 and src_of -1)
hipError_t launch_zero_pad_rows(const int32_t* offsets, const int32_t* counts, int E,
                                int row_bytes, void* rows, float* scale, int32_t* src_of,
                                hipStream_t s);
// with row_w: also row_w[row_of[t,j]] = w[t,j] (the routing weight of each routed row)
hipError_t launch_scatter_rows(const void* x, const int32_t* row_of, const float* prob, int T,
                               int H, int k, void* xp, hipStream_t s, const float* w = nullptr,
                               float* row_w = nullptr);
hipError_t launch_row_weights(const int32_t* row_of, const float* w, int T, int k, float* row_w,
                              hipStream_t s);
hipError_t launch_scatter_rows_fp8(const void* x, const int32_t* row_of, int T, int H, int k,
                                   uint8_t* xq, float* xscale, hipStream_t s);
hipError_t launch_combine(const void* y_perm, const int32_t* row_of, const float* prob,
                          const void* shared, int T, int H, int k, void* y, hipStream_t s);
hipError_t launch_quantize_rows(const void* x, int R, int C, uint8_t* q, float* scale,
                                hipStream_t s);
hipError_t launch_quantize_weights(const void* w, int G, int K, int N, uint8_t* q, float* scale,
                                   hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);
// Dispatch backward with the router's dx term: dx[t] = sum_j dxp[row_of[t,j]] +
// sum_e d_logits[t, e] * w_router[e] (over the nonzero d_logits), fp32 sum, one rounding.
hipError_t launch_dispatch_bwd_router(const void* dxp, const int32_t* row_of,
                                      const int32_t* topk_idx, const float* d_logits,
                                      const void* w_router, int T, int H, int E, int k, void* dx,
                                      hipStream_t s);

// router_proj.hip
hipError_t launch_router_logits(const void* x, const void* w_router, int T, int H, int E,
                                float* logits, hipStream_t s);
// logits [T,E] are read for MOE_SOFTMAX_PRE only (the experts not kept get a gradient).
hipError_t launch_combine_bwd_router(const void* dy, const void* out, const int32_t* row_of,
                                     const int32_t* topk_idx, const float* prob,
                                     const float* logits, int T, int H, int E, int k, int score,
                                     float scaling, void* d_out, float* d_prob, float* d_logits,
                                     uint16_t* dls, int mp, hipStream_t s);
// Dispatch backward when the routing weights scale the expert inputs (with the router
// projection): d_prob = <dxp, x>, d_logits (+ split halves), dx = sum q dxp + router term.
hipError_t launch_dispatch_bwd_router_input(const void* dxp, const void* x, const int32_t* row_of,
                                            const int32_t* topk_idx, const float* prob,
                                            const float* logits, const void* w_router, int T,
                                            int H, int E, int k, int score, float scaling,
                                            void* dx, float* d_logits, uint16_t* dls, int mp,
                                            hipStream_t s);
// Dispatch backward of a layer whose routing weights scale the SwiGLU output (ScaledSwiGLU)
// and which owns its router projection: d_prob[t,j] = sum over the P = I/64 partials of
// row row_of[t,j] (row_part [rows, P], fixed order), d_logits (+ split halves), dx =
// sum_j dxp[row_of[t,j]] + router term.
hipError_t launch_dispatch_bwd_router_act(const void* dxp, const float* row_part, int P,
                                          const int32_t* row_of, const int32_t* topk_idx,
                                          const float* prob, const float* logits,
                                          const void* w_router, int T, int H, int E, int k,
                                          int score, float scaling, void* dx, float* d_logits,
                                          uint16_t* dls, int mp, hipStream_t s);
hipError_t launch_router_wgrad_reduce(const float* part, int S, int E, int H, int mp, float* dw,
                                      hipStream_t s);
hipError_t launch_router_split(const float* d_logits, int T, int E, int mp, uint16_t* dls,
                               hipStream_t s);
// Columns of the split operand (hi and lo halves, padded to the GEMM's 64-column step)
// and the number of K splits of the router weight-gradient GEMM.
inline int router_split_cols(int E) { return (2 * E + 63) / 64 * 64; }
#ifndef MOE_ROUTER_SPLIT_ROWS
#define MOE_ROUTER_SPLIT_ROWS 256
#endif
inline int router_wgrad_splits(int T) {
  const int s = T / MOE_ROUTER_SPLIT_ROWS;  // at least that many rows per split
  return s < 1 ? 1 : (s > 32 ? 32 : s);
}

// gemm.hip
enum GemmEpi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SWIGLU_BWD = 2 };

struct GemmParams {
  int mode;              // moe_gemm_mode_t
  int epi;               // GemmEpi
  int fp8;               // operands e4m3 (NT only) instead of bf16
  const void* A;
  const void* B;
  const float* a_scale;  // fp8: [rows]
  const float* b_scale;  // fp8: [G, Ncols]
  const int32_t* offsets;  // [G+1] device group boundaries; NULL: G even splits of rows
  int G, rows;
  int M, N, K;           // NN/NT: C[rows,N] = A[rows,K] B_g ; DW: C[g][M,N], K ragged
  void* C;
  int c_fp32;
  int I;                 // SwiGLU width (EPI_SWIGLU: N = 2I; EPI_SWIGLU_BWD: N = I)
  void* gu_out;          // EPI_SWIGLU: optional saved g,u [rows,2I]
  const void* gu_in;     // EPI_SWIGLU_BWD: saved g,u [rows,2I]
  int sched_slot;        // tile-counter slot of the launch (set by the launcher)
  int* sched;            // optional: the launch's own tile counters (16 ints, zero when the
                         // launch starts, left zero when it ends); NULL: a library slot
  // NN/NT, bf16, no saved g,u: when A_last is set the last group (G-1) takes its A rows,
  // its weight and its C rows from these tensors (row 0 = the group's first row) instead
  // of from A, B and C. Used to run a dense shared expert as one more group.
  const void* A_last;
  const void* B_last;
  void* C_last;
  // ScaledSwiGLU (bf16 only): EPI_SWIGLU multiplies h by row_scale[row] (not the A_last
  // group's rows); EPI_SWIGLU_BWD multiplies dh by it, and with row_part [rows, I/64]
  // writes per row and 64-column block sum_c dh[row,c] silu(g) u (dh before the scaling).
  const float* row_scale;
  float* row_part;
  // Split-K (bf16 NN/NT launches on 32-row tiles, the decode case, where a few wide tiles
  // per expert leave compute units idle): with `part` set, each tile's K range may be cut
  // into S <= kSplitKMax parts, chosen on the device from the exact tile count. Every part
  // writes its fp32 sums to part[S][rows][ncols] (ncols = 2I for SwiGLU, else N), S goes
  // to *part_s, and a second kernel adds the parts in order and applies the epilogue.
  // NULL: no split. Space: splitk_workspace_bytes.
  float* part;
  int* part_s;
};
constexpr int kSplitKMax = 8;
// Bytes of the split-K space of a bf16 NN/NT grouped GEMM over `rows` rows in G groups with
// ncols output columns before the epilogue (0: the shape never splits). The space holds
// part_s at offset 0 and part at offset 256.
size_t splitk_workspace_bytes(long long rows, int G, long long ncols);
hipError_t launch_grouped_gemm(const GemmParams& p, hipStream_t s);
// Grid cap of the persistent grouped-GEMM launches (0: every resident block).
void set_gemm_max_blocks(int n);

}  // namespace moe
