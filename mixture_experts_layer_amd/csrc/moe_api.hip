// extern "C" entry points declared in include/moe_amd.h: argument checks, workspace
// layout, and the enqueue order of the whole-layer forward and backward.
#include "internal.h"

using namespace moe;

namespace {

inline hipStream_t S(void* s) { return (hipStream_t)s; }
inline moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                           \
  do {                                          \
    hipError_t _e = (expr);                     \
    if (_e != hipSuccess) return MOE_ERR_HIP;   \
  } while (0)

bool ok_ptr(const void* p) { return p != nullptr && moe_aligned16(p); }
bool opt_ptr(const void* p) { return p == nullptr || moe_aligned16(p); }

moe_status_t check_shape(int T, int H, int E, int k) {
  if (T < 0 || H <= 0 || E <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
  if (k > E) return MOE_ERR_INVALID_ARG;
  if (k > 32 || E > 256) return MOE_ERR_UNSUPPORTED;
  if (H % 64) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * k * (long long)(H > 0 ? H : 1) > (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  // routed rows (T k, plus T of a shared expert, plus at most 256 x 4095 of padding) are
  // int32 row ids and offsets
  if ((long long)T * (k + 1) + 256LL * 4095 > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The grouped GEMM addresses one expert's weight matrix (N x K elements of esz bytes) and a
// tile's rows of the activations with 32-bit offsets.
bool gemm_offsets_fit(long long N, long long K, int esz) {
  return N * K * esz < (1LL << 32) && 512LL * K * esz < (1LL << 32);
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace layout of moe_forward / moe_backward. Every region is 256-byte aligned.
struct Layout {
  size_t topk_idx, topk_prob, counts, offsets, pad_offsets, row_of, src_of, shared_offsets;
  size_t xp, xp_scale, gu, h, hq, h_scale, out, shared_h, shared_out, xq, xq_scale, hq_scale;
  size_t d_out, dgu, dxp, scratch, scratch_bytes;
  size_t logits, d_logits, router_ws, router_ws_bytes, total;
  size_t mx_col_offsets, dgq, dgq_scale, mx_ta, mx_ta_scale, mx_tb, mx_tb_scale, mx_kp;
  size_t row_prob, row_part;  // ScaledSwiGLU: weight of each routed row; d_prob partials
  size_t sched;  // tile counters of the layer's grouped-GEMM launches (16 ints)
  size_t splitk, splitk_bytes;  // split-K partial sums of the forward's decode-sized GEMMs
  size_t rows;  // rows of the expert-contiguous buffers
};

// Scratch of the router weight gradient: the split d_logits operand [T, mp] bf16, then the
// fp32 partial products [S, mp, H] of the K splits.
size_t router_wgrad_dls_bytes(int T, int E) { return align_up((size_t)T * router_split_cols(E) * 2); }
size_t router_wgrad_bytes(int T, int H, int E) {
  return router_wgrad_dls_bytes(T, E) +
         (size_t)router_wgrad_splits(T) * router_split_cols(E) * (size_t)H * 4;
}

// A dense shared expert of the routed experts' width runs as one more group of T rows
// (offsets[E+1] = N + T) in the forward's expert GEMM launches, reading x, its own weights
// and its own outputs; other widths, and training, launch it separately.
bool fuses_shared(const moe_problem_t& p) {
  return p.shared_I == p.I && !p.training && p.dtype == MOE_BF16 && p.align_size <= 1;
}

Layout make_layout(const moe_problem_t& p) {
  Layout L{};
  const size_t NT = (size_t)p.T * p.k;  // routed (token, choice) pairs
  // rows of the expert-contiguous buffers: the pairs, plus the padding of a padded dispatch
  const size_t N = NT + (p.align_size > 1 ? (size_t)p.E * (p.align_size - 1) : 0);
  const bool fp8 = p.dtype == MOE_FP8_E4M3;
  const bool mx = p.dtype == MOE_MXFP8;
  const size_t act = fp8 ? 1 : 2;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align_up(bytes);
    return at;
  };
  L.topk_idx = take(NT * 4);
  L.topk_prob = take(NT * 4);
  L.counts = take((size_t)p.E * 4);
  L.offsets = take(((size_t)p.E + 2) * 4);  // one more end for a fused shared group
  L.pad_offsets = take((size_t)p.E * 4);
  L.row_of = take(NT * 4);
  L.src_of = take(N * 4);
  L.shared_offsets = take(2 * 4);
  L.xp = take(N * p.H * act);
  L.xp_scale = take(fp8 ? N * 4 : 0);
  L.gu = take(p.training ? N * 2 * p.I * 2 : 0);
  L.h = take(N * p.I * 2);
  L.hq = take(fp8 || mx ? N * p.I : 0);
  L.xq = take(mx ? N * p.H : 0);
  L.xq_scale = take(mx ? N * (p.H / 32) : 0);
  L.hq_scale = take(mx ? N * (p.I / 32) : 0);
  L.h_scale = take(fp8 ? N * 4 : 0);
  L.out = take(N * p.H * 2);
  L.shared_h = take(p.shared_I ? (size_t)p.T * p.shared_I * 2 : 0);
  L.shared_out = take(p.shared_I ? (size_t)p.T * p.H * 2 : 0);
  L.d_out = take(p.training ? N * p.H * 2 : 0);
  L.dgu = take(p.training ? N * 2 * p.I * 2 : 0);
  L.dxp = take(p.training ? N * p.H * 2 : 0);
  L.scratch_bytes = permute_scratch_bytes(p.T, p.E, p.k);
  L.scratch = take(L.scratch_bytes);
  L.logits = take(p.router ? (size_t)p.T * p.E * 4 : 0);
  L.d_logits = take(p.router && p.training ? (size_t)p.T * p.E * 4 : 0);
  L.router_ws_bytes = p.router && p.training ? router_wgrad_bytes(p.T, p.H, p.E) : 0;
  L.router_ws = take(L.router_ws_bytes);
  const bool at_act = p.weight_placement == MOE_PLACE_ACTIVATION;
  L.row_prob = take(at_act ? N * 4 : 0);
  L.row_part = take(at_act && p.router && p.training ? N * (size_t)(p.I / 64) * 4 : 0);
  L.sched = take(16 * 4);
  // split-K space of the bf16 forward GEMMs (one after the other, so they share it)
  if (p.dtype == MOE_BF16) {
    const long long rows = (long long)N + (fuses_shared(p) ? p.T : 0);
    const int G = p.E + (fuses_shared(p) ? 1 : 0);
    const size_t b1 = splitk_workspace_bytes(rows, G, 2LL * p.I);
    const size_t b2 = splitk_workspace_bytes(rows, G, p.H);
    L.splitk_bytes = b1 > b2 ? b1 : b2;
  }
  L.splitk = take(L.splitk_bytes);
  // MXFP8 training: dgu codes (rows), and the token-axis (transposed) operands of the weight
  // gradients, [C, Kp] codes for C up to max(H, I) (A side) and max(H, 2I) (B side)
  const bool mxt = mx && p.training;
  L.mx_kp = mxt ? (size_t)mx_cols_capacity((long long)N, p.E) : 0;
  const size_t ca = (size_t)(p.H > p.I ? p.H : p.I), cb = (size_t)(p.H > 2 * p.I ? p.H : 2 * p.I);
  L.mx_col_offsets = take(mxt ? ((size_t)p.E + 1) * 4 : 0);
  L.dgq = take(mxt ? N * 2 * p.I : 0);
  L.dgq_scale = take(mxt ? N * 2 * p.I / 32 : 0);
  L.mx_ta = take(ca * L.mx_kp);
  L.mx_ta_scale = take(ca * L.mx_kp / 32);
  L.mx_tb = take(cb * L.mx_kp);
  L.mx_tb_scale = take(cb * L.mx_kp / 32);
  L.total = o;
  L.rows = N;
  return L;
}

bool valid_score(int score) { return score >= MOE_SOFTMAX_PRE_RENORM && score <= MOE_SOFTMAX_PRE; }

// Router options against (E, k, score); fills `o` (scaling 0 is taken as 1).
moe_status_t make_router_opts(int E, int k, int score, const float* expert_bias, int num_groups,
                              int group_topk, float scaling, int map_format, RouterOpts* o) {
  if (!opt_ptr(expert_bias) || num_groups < 0 || (map_format != 0 && map_format != 1))
    return MOE_ERR_INVALID_ARG;
  if (!(scaling == scaling) || scaling == INFINITY || scaling == -INFINITY) return MOE_ERR_INVALID_ARG;
  if (expert_bias && score != MOE_SIGMOID && score != MOE_SQRTSOFTPLUS) return MOE_ERR_UNSUPPORTED;
  if (num_groups > 1) {
    if (num_groups > 64 || E % num_groups) return MOE_ERR_UNSUPPORTED;
    if (group_topk < 1 || group_topk > num_groups || k < group_topk ||
        k > group_topk * (E / num_groups))
      return MOE_ERR_INVALID_ARG;
  }
  o->expert_bias = expert_bias;
  o->num_groups = num_groups > 1 ? num_groups : 0;
  o->group_topk = num_groups > 1 ? group_topk : 0;
  o->scaling = scaling == 0.f ? 1.f : scaling;
  o->bitmap = map_format;
  return MOE_OK;
}

moe_status_t check_problem(const moe_problem_t* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  moe_status_t st = check_shape(p->T, p->H, p->E, p->k);
  if (st != MOE_OK) return st;
  if (p->I <= 0 || p->shared_I < 0) return MOE_ERR_INVALID_ARG;
  if (p->I % 64 || p->shared_I % 64) return MOE_ERR_UNSUPPORTED;
  if (!gemm_offsets_fit(2LL * p->I, p->H, 2) || !gemm_offsets_fit(2LL * p->shared_I, p->H, 2))
    return MOE_ERR_UNSUPPORTED;
  if (!valid_score(p->score)) return MOE_ERR_INVALID_ARG;
  if (p->dtype != MOE_BF16 && p->dtype != MOE_FP8_E4M3 && p->dtype != MOE_MXFP8)
    return MOE_ERR_INVALID_ARG;
  if (p->dtype == MOE_MXFP8 && (p->shared_I || p->weight_placement != MOE_PLACE_COMBINE))
    return MOE_ERR_UNSUPPORTED;
  if (p->router != 0 && p->router != 1) return MOE_ERR_INVALID_ARG;
  RouterOpts o;
  moe_status_t so = make_router_opts(p->E, p->k, p->score, nullptr, p->num_groups, p->group_topk,
                                     p->scaling_factor, 0, &o);
  if (so != MOE_OK) return so;
  if (p->weight_placement != MOE_PLACE_COMBINE && p->weight_placement != MOE_PLACE_INPUT &&
      p->weight_placement != MOE_PLACE_ACTIVATION)
    return MOE_ERR_INVALID_ARG;
  if (p->weight_placement != MOE_PLACE_COMBINE && p->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (p->align_size < 0) return MOE_ERR_INVALID_ARG;
  if (p->align_size > 4096) return MOE_ERR_UNSUPPORTED;
  if (p->dtype == MOE_FP8_E4M3) {
    if (p->H % 128 || p->I % 128) return MOE_ERR_UNSUPPORTED;
    if (p->training || p->shared_I) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// dW_r = d_logits^T x from the split operand dls [T, mp] (hi | lo | 0): a ragged-K
// weight-gradient GEMM over S even splits of the T rows into fp32 partials [S, mp, H],
// then the fixed-order sum of the splits and of the two halves.
hipError_t launch_router_wgrad(const void* x, const uint16_t* dls, int T, int H, int E,
                               float* part, float* dw, hipStream_t s) {
  const int mp = router_split_cols(E), S = router_wgrad_splits(T);
  GemmParams r{};
  r.mode = MOE_GEMM_TN_DW;
  r.epi = EPI_STORE;
  r.A = dls;
  r.B = x;
  r.offsets = nullptr;  // S even splits of the T rows
  r.G = S;
  r.rows = T;
  r.M = mp;
  r.N = H;
  r.C = part;
  r.c_fp32 = 1;
  hipError_t e = launch_grouped_gemm(r, s);
  if (e != hipSuccess) return e;
  return launch_router_wgrad_reduce(part, S, E, H, mp, dw, s);
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status_t moe_set_gemm_max_blocks(int max_blocks) {
  MOE_REQUIRE(max_blocks >= 0, MOE_ERR_INVALID_ARG);
  moe::set_gemm_max_blocks(max_blocks);
  return MOE_OK;
}

moe_status_t moe_router_topk(const float* logits, int T, int E, int k, int score,
                             int32_t* topk_idx, float* topk_prob, int32_t* counts,
                             uint8_t* routing_map, float* probs_dense, void* stream) {
  return moe_router_topk_ex(logits, T, E, k, score, nullptr, topk_idx, topk_prob, counts,
                            routing_map, probs_dense, stream);
}

moe_status_t moe_router_topk_ex(const float* logits, int T, int E, int k, int score,
                                const moe_router_opts_t* opts, int32_t* topk_idx,
                                float* topk_prob, int32_t* counts, uint8_t* routing_map,
                                float* probs_dense, void* stream) {
  moe_status_t st = check_shape(T, 64, E, k);
  if (st != MOE_OK) return st;
  if (!valid_score(score)) return MOE_ERR_INVALID_ARG;
  RouterOpts o;
  st = opts ? make_router_opts(E, k, score, opts->expert_bias, opts->num_groups, opts->group_topk,
                               opts->scaling_factor, opts->map_format, &o)
            : make_router_opts(E, k, score, nullptr, 0, 0, 1.f, 0, &o);
  if (st != MOE_OK) return st;
  if (!ok_ptr(counts)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!ok_ptr(logits) || !ok_ptr(topk_idx) || !ok_ptr(topk_prob)))
    return MOE_ERR_INVALID_ARG;
  if (!opt_ptr(routing_map) || !opt_ptr(probs_dense)) return MOE_ERR_INVALID_ARG;
  if (router_opts_plain(o, score))
    return hip_status(launch_router_topk(logits, T, E, k, score, topk_idx, topk_prob, counts,
                                         routing_map, probs_dense, S(stream)));
  return hip_status(launch_router_ext(logits, T, E, k, score, o, topk_idx, topk_prob, counts,
                                      routing_map, probs_dense, 0, S(stream)));
}

moe_status_t moe_expert_bias_update(float* expert_bias, const int32_t* tokens_per_expert,
                                    int E, float coeff, void* stream) {
  if (E <= 0) return MOE_ERR_INVALID_ARG;
  if (E > 256) return MOE_ERR_UNSUPPORTED;
  if (!ok_ptr(expert_bias) || !ok_ptr(tokens_per_expert)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_expert_bias_update(expert_bias, tokens_per_expert, E, coeff, S(stream)));
}

size_t moe_permute_workspace_bytes(int T, int E, int k) {
  if (T < 0 || E <= 0 || k <= 0) return 0;
  return permute_scratch_bytes(T, E, k);
}

moe_status_t moe_permute(const void* x, const int32_t* topk_idx, int T, int H, int E, int k,
                         int out_dtype, void* xp, float* xp_scale, int32_t* offsets,
                         int32_t* row_of, int32_t* src_of, void* ws, size_t ws_bytes,
                         void* stream) {
  moe_status_t st = check_shape(T, H, E, k);
  if (st != MOE_OK) return st;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  if (!ok_ptr(offsets)) return MOE_ERR_INVALID_ARG;
  if (T > 0) {
    if (!ok_ptr(x) || !ok_ptr(topk_idx) || !ok_ptr(xp) || !ok_ptr(row_of) || !ok_ptr(src_of))
      return MOE_ERR_INVALID_ARG;
    if (out_dtype == MOE_FP8_E4M3 && !ok_ptr(xp_scale)) return MOE_ERR_INVALID_ARG;
    if (!ok_ptr(ws)) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < permute_scratch_bytes(T, E, k)) return MOE_ERR_WORKSPACE;
  }
  hipStream_t s = S(stream);
  MOE_TRY(launch_dispatch_meta(topk_idx, T, E, k, offsets, row_of, src_of, ws, s));
  if (out_dtype == MOE_BF16) MOE_TRY(launch_scatter_rows(x, row_of, nullptr, T, H, k, xp, s));
  else MOE_TRY(launch_scatter_rows_fp8(x, row_of, T, H, k, (uint8_t*)xp, xp_scale, s));
  return MOE_OK;
}

moe_status_t moe_permute_noalloc(const void* x, const int32_t* topk_idx, int T, int H, int E,
                                 int k, int out_dtype, void* xp, float* xp_scale,
                                 int32_t* offsets, int32_t* row_of, int32_t* src_of,
                                 void* stream) {
  moe_status_t st = check_shape(T, H, E, k);
  if (st != MOE_OK) return st;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  if (!ok_ptr(offsets)) return MOE_ERR_INVALID_ARG;
  if (permute_scratch_bytes(T, E, k) > permute_noalloc_scratch_limit())
    return MOE_ERR_UNSUPPORTED;
  if (T > 0) {
    if (!ok_ptr(x) || !ok_ptr(topk_idx) || !ok_ptr(xp) || !ok_ptr(row_of) || !ok_ptr(src_of))
      return MOE_ERR_INVALID_ARG;
    if (out_dtype == MOE_FP8_E4M3 && !ok_ptr(xp_scale)) return MOE_ERR_INVALID_ARG;
  }
  return hip_status(launch_permute_noalloc(x, topk_idx, T, H, E, k, out_dtype, xp, xp_scale,
                                           offsets, row_of, src_of, S(stream)));
}

size_t moe_permute_noalloc_limit(void) { return permute_noalloc_scratch_limit(); }

size_t moe_padded_rows(int T, int E, int k, int align) {
  if (T < 0 || E <= 0 || k <= 0 || align < 0) return 0;
  return (size_t)T * k + (align > 1 ? (size_t)E * (align - 1) : 0);
}

moe_status_t moe_permute_padded(const void* x, const int32_t* topk_idx, int T, int H, int E,
                                int k, int align, int out_dtype, void* xp, float* xp_scale,
                                int32_t* offsets, int32_t* pad_offsets, int32_t* row_of,
                                int32_t* src_of, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_shape(T, H, E, k);
  if (st != MOE_OK) return st;
  if (align < 1) return MOE_ERR_INVALID_ARG;
  if (align > 4096) return MOE_ERR_UNSUPPORTED;
  if (out_dtype != MOE_BF16 && out_dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  if (out_dtype == MOE_FP8_E4M3 && H % 16) return MOE_ERR_UNSUPPORTED;
  if (!ok_ptr(offsets) || !ok_ptr(pad_offsets) || !ok_ptr(ws)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < permute_scratch_bytes(T, E, k)) return MOE_ERR_WORKSPACE;
  if (T > 0) {
    if (!ok_ptr(x) || !ok_ptr(topk_idx) || !ok_ptr(xp) || !ok_ptr(row_of) || !ok_ptr(src_of))
      return MOE_ERR_INVALID_ARG;
    if (out_dtype == MOE_FP8_E4M3 && !ok_ptr(xp_scale)) return MOE_ERR_INVALID_ARG;
  }
  hipStream_t s = S(stream);
  const int nchunks = (T * k + kPermChunk - 1) / kPermChunk;
  int32_t* counts = (int32_t*)ws + (size_t)nchunks * E;  // after the histograms
  MOE_TRY(launch_dispatch_meta(topk_idx, T, E, k, offsets, row_of, src_of, ws, s, align,
                               pad_offsets, counts));
  if (T == 0) return MOE_OK;
  const bool fp8 = out_dtype == MOE_FP8_E4M3;
  if (!fp8) MOE_TRY(launch_scatter_rows(x, row_of, nullptr, T, H, k, xp, s));
  else MOE_TRY(launch_scatter_rows_fp8(x, row_of, T, H, k, (uint8_t*)xp, xp_scale, s));
  MOE_TRY(launch_zero_pad_rows(offsets, counts, E, fp8 ? H : 2 * H, xp, fp8 ? xp_scale : nullptr,
                               src_of, s));
  return MOE_OK;
}

size_t moe_grouped_gemm_splitk_workspace_bytes(int rows, int G, int ncols) {
  return splitk_workspace_bytes(rows, G, ncols);
}

// Optional split-K space of a stand-alone grouped GEMM: NULL, or at least the bytes above.
static moe_status_t take_splitk(GemmParams& p, long long ncols, void* ws, size_t ws_bytes) {
  if (ws == nullptr) return MOE_OK;
  if (!ok_ptr(ws)) return MOE_ERR_INVALID_ARG;
  const size_t need = splitk_workspace_bytes(p.rows, p.G, ncols);
  if (need == 0 || p.fp8 || p.mode == MOE_GEMM_TN_DW) return MOE_OK;  // never splits
  if (ws_bytes < need) return MOE_ERR_INVALID_ARG;
  p.part_s = (int*)ws;
  p.part = (float*)((uint8_t*)ws + 256);
  return MOE_OK;
}

moe_status_t moe_grouped_gemm_swiglu(const void* xp, const float* xp_scale, const void* w_gu,
                                     const float* w_scale, const int32_t* offsets, int G,
                                     int rows, int H, int I, int dtype, void* h, void* gu_saved,
                                     void* ws, size_t ws_bytes, void* stream) {
  if (G <= 0 || rows < 0 || H <= 0 || I <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 64 || I % 64 || G > 256) return MOE_ERR_UNSUPPORTED;
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  const bool fp8 = dtype == MOE_FP8_E4M3;
  if (fp8 && (H % 128)) return MOE_ERR_UNSUPPORTED;
  if (!gemm_offsets_fit(2LL * I, H, fp8 ? 1 : 2)) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!ok_ptr(xp) || !ok_ptr(w_gu) || !ok_ptr(offsets) || !ok_ptr(h) || !opt_ptr(gu_saved))
    return MOE_ERR_INVALID_ARG;
  if (fp8 && (!ok_ptr(xp_scale) || !ok_ptr(w_scale))) return MOE_ERR_INVALID_ARG;
  GemmParams p{};
  p.mode = fp8 ? MOE_GEMM_NT : MOE_GEMM_NN;
  p.epi = EPI_SWIGLU;
  p.fp8 = fp8;
  p.A = xp;
  p.B = w_gu;
  p.a_scale = xp_scale;
  p.b_scale = w_scale;
  p.offsets = offsets;
  p.G = G;
  p.rows = rows;
  p.N = 2 * I;
  p.K = H;
  p.C = h;
  p.I = I;
  p.gu_out = gu_saved;
  const moe_status_t st = take_splitk(p, 2LL * I, ws, ws_bytes);
  if (st != MOE_OK) return st;
  return hip_status(launch_grouped_gemm(p, S(stream)));
}

moe_status_t moe_grouped_gemm(int mode, const void* A, const float* a_scale, const void* B,
                              const float* b_scale, const int32_t* offsets, int G, int rows,
                              int M, int N, int K, int dtype, void* C, int c_dtype, void* ws,
                              size_t ws_bytes, void* stream) {
  if (G <= 0 || rows < 0 || N <= 0) return MOE_ERR_INVALID_ARG;
  if (G > 256) return MOE_ERR_UNSUPPORTED;
  if (mode != MOE_GEMM_NN && mode != MOE_GEMM_NT && mode != MOE_GEMM_TN_DW)
    return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  if (c_dtype != MOE_BF16 && c_dtype != MOE_FP32) return MOE_ERR_INVALID_ARG;
  const bool fp8 = dtype == MOE_FP8_E4M3;
  if (fp8 && mode != MOE_GEMM_NT) return MOE_ERR_UNSUPPORTED;
  if (N % 64) return MOE_ERR_UNSUPPORTED;
  if (mode == MOE_GEMM_TN_DW) {
    if (M <= 0) return MOE_ERR_INVALID_ARG;
    if (M % 64) return MOE_ERR_UNSUPPORTED;
  } else {
    if (K <= 0) return MOE_ERR_INVALID_ARG;
    if (K % (fp8 ? 128 : 64)) return MOE_ERR_UNSUPPORTED;
    if (!gemm_offsets_fit(N, K, fp8 ? 1 : 2)) return MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
  }
  if (!ok_ptr(A) || !ok_ptr(B) || !ok_ptr(offsets) || !ok_ptr(C)) return MOE_ERR_INVALID_ARG;
  if (fp8 && (!ok_ptr(a_scale) || !ok_ptr(b_scale))) return MOE_ERR_INVALID_ARG;
  GemmParams p{};
  p.mode = mode;
  p.epi = EPI_STORE;
  p.fp8 = fp8;
  p.A = A;
  p.B = B;
  p.a_scale = a_scale;
  p.b_scale = b_scale;
  p.offsets = offsets;
  p.G = G;
  p.rows = rows;
  p.M = M;
  p.N = N;
  p.K = K;
  p.C = C;
  p.c_fp32 = c_dtype == MOE_FP32;
  const moe_status_t st = take_splitk(p, N, ws, ws_bytes);
  if (st != MOE_OK) return st;
  return hip_status(launch_grouped_gemm(p, S(stream)));
}

moe_status_t moe_grouped_gemm_swiglu_bwd(const void* d_out, const void* w_down,
                                         const int32_t* offsets, const void* gu_saved, int G,
                                         int rows, int H, int I, void* dgu, void* stream) {
  if (G <= 0 || rows < 0 || H <= 0 || I <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 64 || I % 64 || G > 256) return MOE_ERR_UNSUPPORTED;
  if (!gemm_offsets_fit(I, H, 2)) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!ok_ptr(d_out) || !ok_ptr(w_down) || !ok_ptr(offsets) || !ok_ptr(gu_saved) || !ok_ptr(dgu))
    return MOE_ERR_INVALID_ARG;
  GemmParams p{};
  p.mode = MOE_GEMM_NT;
  p.epi = EPI_SWIGLU_BWD;
  p.A = d_out;
  p.B = w_down;
  p.offsets = offsets;
  p.G = G;
  p.rows = rows;
  p.N = I;
  p.K = H;
  p.C = dgu;
  p.I = I;
  p.gu_in = gu_saved;
  return hip_status(launch_grouped_gemm(p, S(stream)));
}

moe_status_t moe_grouped_gemm_swiglu_scaled(const void* xp, const void* w_gu,
                                            const int32_t* offsets, const float* row_scale, int G,
                                            int rows, int H, int I, void* h, void* gu_saved,
                                            void* stream) {
  if (G <= 0 || rows < 0 || H <= 0 || I <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 64 || I % 64 || G > 256) return MOE_ERR_UNSUPPORTED;
  if (!gemm_offsets_fit(2LL * I, H, 2)) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!ok_ptr(xp) || !ok_ptr(w_gu) || !ok_ptr(offsets) || !ok_ptr(row_scale) || !ok_ptr(h) ||
      !opt_ptr(gu_saved))
    return MOE_ERR_INVALID_ARG;
  GemmParams p{};
  p.mode = MOE_GEMM_NN;
  p.epi = EPI_SWIGLU;
  p.A = xp;
  p.B = w_gu;
  p.offsets = offsets;
  p.G = G;
  p.rows = rows;
  p.N = 2 * I;
  p.K = H;
  p.C = h;
  p.I = I;
  p.gu_out = gu_saved;
  p.row_scale = row_scale;
  return hip_status(launch_grouped_gemm(p, S(stream)));
}

moe_status_t moe_grouped_gemm_swiglu_scaled_bwd(const void* d_out, const void* w_down,
                                                const int32_t* offsets, const void* gu_saved,
                                                const float* row_scale, int G, int rows, int H,
                                                int I, void* dgu, float* d_scale_part,
                                                void* stream) {
  if (G <= 0 || rows < 0 || H <= 0 || I <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 64 || I % 64 || G > 256) return MOE_ERR_UNSUPPORTED;
  if (!gemm_offsets_fit(I, H, 2)) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!ok_ptr(d_out) || !ok_ptr(w_down) || !ok_ptr(offsets) || !ok_ptr(gu_saved) ||
      !ok_ptr(row_scale) || !ok_ptr(dgu) || !opt_ptr(d_scale_part))
    return MOE_ERR_INVALID_ARG;
  GemmParams p{};
  p.mode = MOE_GEMM_NT;
  p.epi = EPI_SWIGLU_BWD;
  p.A = d_out;
  p.B = w_down;
  p.offsets = offsets;
  p.G = G;
  p.rows = rows;
  p.N = I;
  p.K = H;
  p.C = dgu;
  p.I = I;
  p.gu_in = gu_saved;
  p.row_scale = row_scale;
  p.row_part = d_scale_part;
  return hip_status(launch_grouped_gemm(p, S(stream)));
}

moe_status_t moe_permute_probs(const int32_t* row_of, const float* topk_prob, int T, int k,
                               float* row_prob, void* stream) {
  if (T < 0 || k <= 0) return MOE_ERR_INVALID_ARG;
  if (k > 32 || (long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;  // int32 row ids
  if (T == 0) return MOE_OK;
  if (!ok_ptr(row_of) || !ok_ptr(topk_prob) || !ok_ptr(row_prob)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_row_weights(row_of, topk_prob, T, k, row_prob, S(stream)));
}

moe_status_t moe_unpermute_combine(const void* y_perm, const int32_t* row_of,
                                   const float* topk_prob, const void* shared_out, int T,
                                   int H, int k, void* y, void* stream) {
  if (T < 0 || H <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
  if (k > 32 || (long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;  // int32 row ids
  if (H % 64) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(y_perm) || !ok_ptr(row_of) || !ok_ptr(y) || !opt_ptr(topk_prob) ||
      !opt_ptr(shared_out))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(y_perm, row_of, topk_prob, shared_out, T, H, k, y, S(stream)));
}

moe_status_t moe_combine_backward(const void* dy, const int32_t* row_of, const float* topk_prob,
                                  int T, int H, int k, void* d_out, void* stream) {
  if (T < 0 || H <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
  if (k > 32 || (long long)T * k > 0x7fffffffLL) return MOE_ERR_UNSUPPORTED;  // int32 row ids
  if (H % 64) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(dy) || !ok_ptr(row_of) || !ok_ptr(topk_prob) || !ok_ptr(d_out))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_scatter_rows(dy, row_of, topk_prob, T, H, k, d_out, S(stream)));
}

moe_status_t moe_router_logits(const void* x, const void* w_router, int T, int H, int E,
                               float* logits, void* stream) {
  moe_status_t st = check_shape(T, H, E, 1);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(w_router) || !ok_ptr(logits)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_router_logits(x, w_router, T, H, E, logits, S(stream)));
}

moe_status_t moe_combine_backward_router(const void* dy, const void* expert_out,
                                         const int32_t* row_of, const int32_t* topk_idx,
                                         const float* topk_prob, const float* logits, int T,
                                         int H, int E, int k, int score, float scaling_factor,
                                         void* d_out, float* d_prob, float* d_logits,
                                         void* stream) {
  moe_status_t st = check_shape(T, H, E, k);
  if (st != MOE_OK) return st;
  if (!valid_score(score)) return MOE_ERR_INVALID_ARG;
  if (!(scaling_factor == scaling_factor) || scaling_factor == INFINITY || scaling_factor == -INFINITY)
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(dy) || !ok_ptr(expert_out) || !ok_ptr(row_of) || !ok_ptr(topk_idx) ||
      !ok_ptr(topk_prob) || !ok_ptr(d_out) || !opt_ptr(d_prob) || !ok_ptr(d_logits) ||
      (score == MOE_SOFTMAX_PRE && !ok_ptr(logits)))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine_bwd_router(dy, expert_out, row_of, topk_idx, topk_prob, logits,
                                              T, H, E, k, score,
                                              scaling_factor == 0.f ? 1.f : scaling_factor, d_out,
                                              d_prob, d_logits, nullptr, 0, S(stream)));
}

size_t moe_router_weight_grad_workspace_bytes(int T, int H, int E) {
  if (check_shape(T, H, E, 1) != MOE_OK) return 0;
  return router_wgrad_bytes(T, H, E);
}

moe_status_t moe_router_weight_grad(const void* x, const float* d_logits, int T, int H, int E,
                                    float* dw_router, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_shape(T, H, E, 1);
  if (st != MOE_OK) return st;
  if (!ok_ptr(dw_router) || !ok_ptr(ws)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!ok_ptr(x) || !ok_ptr(d_logits))) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < router_wgrad_bytes(T, H, E)) return MOE_ERR_WORKSPACE;
  hipStream_t s = S(stream);
  uint16_t* dls = (uint16_t*)ws;
  MOE_TRY(launch_router_split(d_logits, T, E, router_split_cols(E), dls, s));
  return hip_status(launch_router_wgrad(x, dls, T, H, E,
                                        (float*)((uint8_t*)ws + router_wgrad_dls_bytes(T, E)),
                                        dw_router, s));
}

moe_status_t moe_dispatch_backward_router(const void* dxp, const int32_t* row_of,
                                          const int32_t* topk_idx, const float* d_logits,
                                          const void* w_router, int T, int H, int E, int k,
                                          void* dx, void* stream) {
  moe_status_t st = check_shape(T, H, E, k);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(dxp) || !ok_ptr(row_of) || !ok_ptr(topk_idx) || !ok_ptr(d_logits) ||
      !ok_ptr(w_router) || !ok_ptr(dx))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_dispatch_bwd_router(dxp, row_of, topk_idx, d_logits, w_router, T, H, E,
                                               k, dx, S(stream)));
}

moe_status_t moe_dispatch_backward_router_input(const void* dxp, const void* x,
                                                const int32_t* row_of, const int32_t* topk_idx,
                                                const float* topk_prob, const float* logits,
                                                const void* w_router, int T, int H, int E, int k,
                                                int score, float scaling_factor, void* dx,
                                                float* d_logits, void* stream) {
  moe_status_t st = check_shape(T, H, E, k);
  if (st != MOE_OK) return st;
  if (!valid_score(score)) return MOE_ERR_INVALID_ARG;
  if (!(scaling_factor == scaling_factor) || scaling_factor == INFINITY || scaling_factor == -INFINITY)
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(dxp) || !ok_ptr(x) || !ok_ptr(row_of) || !ok_ptr(topk_idx) || !ok_ptr(topk_prob) ||
      !ok_ptr(w_router) || !ok_ptr(dx) || !ok_ptr(d_logits) ||
      (score == MOE_SOFTMAX_PRE && !ok_ptr(logits)))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_dispatch_bwd_router_input(
      dxp, x, row_of, topk_idx, topk_prob, logits, w_router, T, H, E, k, score,
      scaling_factor == 0.f ? 1.f : scaling_factor, dx, d_logits, nullptr, 0, S(stream)));
}

// ---- auxiliary load-balancing loss -------------------------------------------------------

moe_status_t moe_aux_loss_scores(const float* logits, int T, int E, int k, int score,
                                 float* scores, uint8_t* routing_map, void* stream) {
  moe_status_t st = check_shape(T, 64, E, k);
  if (st != MOE_OK) return st;
  if (!valid_score(score)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(logits) || !ok_ptr(scores) || !opt_ptr(routing_map)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_aux_scores(logits, T, E, k, score, scores, routing_map, S(stream)));
}

size_t moe_aux_loss_workspace_bytes(int T, int E) {
  if (T < 0 || E <= 0 || E > 256) return 0;
  return aux_loss_scratch_bytes(T, E);
}

namespace {
// coeff * E / (k * total^2), in double, rounded once
bool aux_constant(int E, int k, int total, float coeff, float* C) {
  if (total <= 0 || k <= 0 || !(coeff == coeff) || coeff == INFINITY || coeff == -INFINITY)
    return false;
  *C = (float)((double)coeff * E / ((double)k * (double)total * (double)total));
  return true;
}
}  // namespace

moe_status_t moe_aux_loss(const float* scores, const int32_t* tokens_per_expert, int T, int E,
                          int k, int total_num_tokens, float coeff, float* loss, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status_t st = check_shape(T, 64, E, k);
  if (st != MOE_OK) return st;
  float C;
  if (!aux_constant(E, k, total_num_tokens, coeff, &C)) return MOE_ERR_INVALID_ARG;
  if ((T > 0 && !ok_ptr(scores)) || !ok_ptr(tokens_per_expert) || !ok_ptr(loss) || !ok_ptr(ws))
    return MOE_ERR_INVALID_ARG;
  if (ws_bytes < aux_loss_scratch_bytes(T, E)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_aux_loss(scores, tokens_per_expert, T, E, C, loss, (float*)ws,
                                    S(stream)));
}

moe_status_t moe_aux_loss_backward(const float* logits, const int32_t* tokens_per_expert, int T,
                                   int E, int k, int total_num_tokens, float coeff, int score,
                                   const float* d_loss, float* d_logits, int accumulate,
                                   void* stream) {
  moe_status_t st = check_shape(T, 64, E, k);
  if (st != MOE_OK) return st;
  if (!valid_score(score) || (accumulate != 0 && accumulate != 1)) return MOE_ERR_INVALID_ARG;
  float C;
  if (!aux_constant(E, k, total_num_tokens, coeff, &C)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(logits) || !ok_ptr(tokens_per_expert) || !opt_ptr(d_loss) || !ok_ptr(d_logits))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_aux_loss_bwd(logits, T, E, score, tokens_per_expert, C, d_loss,
                                        d_logits, accumulate, S(stream)));
}

moe_status_t moe_dispatch_backward_router_scaled(const void* dxp, const float* d_scale_part,
                                                 const int32_t* row_of, const int32_t* topk_idx,
                                                 const float* topk_prob, const float* logits,
                                                 const void* w_router, int T, int H, int E, int k,
                                                 int I, int score, float scaling_factor, void* dx,
                                                 float* d_logits, void* stream) {
  moe_status_t st = check_shape(T, H, E, k);
  if (st != MOE_OK) return st;
  if (!valid_score(score) || I <= 0) return MOE_ERR_INVALID_ARG;
  if (I % 64) return MOE_ERR_UNSUPPORTED;
  if (!(scaling_factor == scaling_factor) || scaling_factor == INFINITY || scaling_factor == -INFINITY)
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!ok_ptr(dxp) || !ok_ptr(d_scale_part) || !ok_ptr(row_of) || !ok_ptr(topk_idx) ||
      !ok_ptr(topk_prob) || !ok_ptr(w_router) || !ok_ptr(dx) || !ok_ptr(d_logits) ||
      (score == MOE_SOFTMAX_PRE && !ok_ptr(logits)))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_dispatch_bwd_router_act(
      dxp, d_scale_part, I / 64, row_of, topk_idx, topk_prob, logits, w_router, T, H, E, k, score,
      scaling_factor == 0.f ? 1.f : scaling_factor, dx, d_logits, nullptr, 0, S(stream)));
}

moe_status_t moe_quantize_mxfp8_rows(const void* x, int R, int C, uint8_t* q, uint8_t* scale,
                                     void* stream) {
  if (R < 0 || C <= 0) return MOE_ERR_INVALID_ARG;
  if (C % 32) return MOE_ERR_UNSUPPORTED;
  if (R == 0) return MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(q) || scale == nullptr) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_mx_quantize_rows(x, R, C, q, scale, S(stream)));
}

moe_status_t moe_quantize_mxfp8_weights(const void* w, int G, int K, int N, uint8_t* q,
                                        uint8_t* scale, void* stream) {
  if (G <= 0 || K <= 0 || N <= 0) return MOE_ERR_INVALID_ARG;
  if (K % 32) return MOE_ERR_UNSUPPORTED;
  if (!ok_ptr(w) || !ok_ptr(q) || scale == nullptr) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_mx_quantize_weights(w, G, K, N, q, scale, S(stream)));
}

moe_status_t moe_grouped_gemm_mxfp8(const uint8_t* A, const uint8_t* a_scale, const uint8_t* B,
                                    const uint8_t* b_scale, const int32_t* offsets, int G,
                                    int rows, int N, int K, int swiglu, void* C, void* stream) {
  if (G <= 0 || rows < 0 || N <= 0 || K <= 0) return MOE_ERR_INVALID_ARG;
  if (G > 256 || K % 64 || N % (swiglu ? 128 : 64)) return MOE_ERR_UNSUPPORTED;
  if ((long long)N * K >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!ok_ptr(A) || !ok_ptr(B) || !ok_ptr(offsets) || !ok_ptr(C) || a_scale == nullptr ||
      b_scale == nullptr)
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_mx_gemm(swiglu ? EPI_SWIGLU : EPI_STORE, A, a_scale, B, b_scale,
                                   offsets, G, rows, N, K, swiglu ? N / 2 : 0, C, S(stream)));
}

long long moe_mxfp8_cols_capacity(int R, int G) {
  if (R < 0 || G <= 0) return -1;
  return mx_cols_capacity(R, G);
}

moe_status_t moe_mxfp8_col_offsets(const int32_t* offsets, int G, int32_t* col_offsets,
                                   void* stream) {
  if (G <= 0 || !ok_ptr(offsets) || !ok_ptr(col_offsets)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_mx_col_offsets(offsets, G, col_offsets, S(stream)));
}

moe_status_t moe_quantize_mxfp8_cols(const void* x, int R, int C, const int32_t* offsets,
                                     const int32_t* col_offsets, int G, int Kp, uint8_t* qt,
                                     uint8_t* scale_t, void* stream) {
  if (R < 0 || C <= 0 || G <= 0 || Kp < 0) return MOE_ERR_INVALID_ARG;
  if (C % 8 || Kp % kMxColAlign) return MOE_ERR_UNSUPPORTED;
  if (Kp < mx_cols_capacity(R, G)) return MOE_ERR_INVALID_ARG;
  if (Kp == 0) return MOE_OK;
  if ((R > 0 && !ok_ptr(x)) || !ok_ptr(offsets) || !ok_ptr(col_offsets) || !ok_ptr(qt) ||
      scale_t == nullptr)
    return MOE_ERR_INVALID_ARG;
  return hip_status(
      launch_mx_quantize_cols(x, R, C, offsets, col_offsets, G, Kp, qt, scale_t, S(stream)));
}

moe_status_t moe_grouped_gemm_mxfp8_wgrad(const uint8_t* At, const uint8_t* a_scale,
                                          const uint8_t* Bt, const uint8_t* b_scale,
                                          const int32_t* col_offsets, int G, int M, int N, int Kp,
                                          void* C, void* stream) {
  if (G <= 0 || M <= 0 || N <= 0 || Kp < 0) return MOE_ERR_INVALID_ARG;
  if (M % 64 || N % 64 || Kp % kMxColAlign) return MOE_ERR_UNSUPPORTED;
  if (!ok_ptr(At) || !ok_ptr(Bt) || !ok_ptr(col_offsets) || !ok_ptr(C) || a_scale == nullptr ||
      b_scale == nullptr)
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_mx_gemm_wgrad(At, a_scale, Bt, b_scale, col_offsets, G, M, N, Kp, C,
                                         S(stream)));
}

moe_status_t moe_grouped_gemm_mxfp8_swiglu_bwd(const uint8_t* A, const uint8_t* a_scale,
                                               const uint8_t* B, const uint8_t* b_scale,
                                               const int32_t* offsets, int G, int rows, int I,
                                               int K, const void* gu, void* dgu, void* stream) {
  if (G <= 0 || rows < 0 || I <= 0 || K <= 0) return MOE_ERR_INVALID_ARG;
  if (G > 256 || K % 64 || I % 64) return MOE_ERR_UNSUPPORTED;
  if ((long long)I * K >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!ok_ptr(A) || !ok_ptr(B) || !ok_ptr(offsets) || !ok_ptr(gu) || !ok_ptr(dgu) ||
      a_scale == nullptr || b_scale == nullptr)
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_mx_gemm(EPI_SWIGLU_BWD, A, a_scale, B, b_scale, offsets, G, rows, I, K,
                                   I, dgu, S(stream), gu, nullptr));
}

moe_status_t moe_quantize_fp8_rows(const void* x, int R, int C, uint8_t* q, float* scale,
                                   void* stream) {
  if (R < 0 || C <= 0) return MOE_ERR_INVALID_ARG;
  if (C % 64) return MOE_ERR_UNSUPPORTED;
  if (R == 0) return MOE_OK;
  if (!ok_ptr(x) || !ok_ptr(q) || !ok_ptr(scale)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_rows(x, R, C, q, scale, S(stream)));
}

moe_status_t moe_quantize_fp8_weights(const void* w, int G, int K, int N, uint8_t* q,
                                      float* scale, void* stream) {
  if (G <= 0 || K <= 0 || N <= 0) return MOE_ERR_INVALID_ARG;
  if (!ok_ptr(w) || !ok_ptr(q) || !ok_ptr(scale)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_weights(w, G, K, N, q, scale, S(stream)));
}

size_t moe_workspace_bytes(const moe_problem_t* p) {
  if (check_problem(p) != MOE_OK) return 0;
  return make_layout(*p).total;
}

moe_status_t moe_workspace_views(const moe_problem_t* p, void* ws, size_t ws_bytes,
                                 moe_views_t* v) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!v || !ok_ptr(ws)) return MOE_ERR_INVALID_ARG;
  const Layout L = make_layout(*p);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  uint8_t* b = (uint8_t*)ws;
  const bool fp8 = p->dtype == MOE_FP8_E4M3;
  v->topk_idx = (int32_t*)(b + L.topk_idx);
  v->topk_prob = (float*)(b + L.topk_prob);
  v->counts = (int32_t*)(b + L.counts);
  v->offsets = (int32_t*)(b + L.offsets);
  v->pad_offsets = (int32_t*)(b + L.pad_offsets);
  v->rows = (int)(L.rows);
  v->row_of = (int32_t*)(b + L.row_of);
  v->src_of = (int32_t*)(b + L.src_of);
  v->xp = b + L.xp;
  v->xp_scale = fp8 ? (float*)(b + L.xp_scale) : nullptr;
  v->gu = p->training ? b + L.gu : nullptr;
  v->h = b + L.h;
  const bool mx = p->dtype == MOE_MXFP8;
  v->hq = fp8 || mx ? b + L.hq : nullptr;
  v->xq = mx ? b + L.xq : nullptr;
  v->xq_scale = mx ? (uint8_t*)(b + L.xq_scale) : nullptr;
  v->hq_scale = mx ? (uint8_t*)(b + L.hq_scale) : nullptr;
  v->h_scale = fp8 ? (float*)(b + L.h_scale) : nullptr;
  v->out = b + L.out;
  v->shared_h = p->shared_I ? b + L.shared_h : nullptr;
  v->shared_out = p->shared_I ? b + L.shared_out : nullptr;
  v->shared_offsets = (int32_t*)(b + L.shared_offsets);
  v->d_out = p->training ? b + L.d_out : nullptr;
  v->dgu = p->training ? b + L.dgu : nullptr;
  v->dxp = p->training ? b + L.dxp : nullptr;
  v->scratch = b + L.scratch;
  v->scratch_bytes = L.scratch_bytes;
  v->logits = p->router ? (float*)(b + L.logits) : nullptr;
  v->d_logits = p->router && p->training ? (float*)(b + L.d_logits) : nullptr;
  v->router_ws = L.router_ws_bytes ? b + L.router_ws : nullptr;
  v->router_ws_bytes = L.router_ws_bytes;
  const bool mxt = mx && p->training;
  v->mx_col_offsets = mxt ? (int32_t*)(b + L.mx_col_offsets) : nullptr;
  v->dgq = mxt ? b + L.dgq : nullptr;
  v->dgq_scale = mxt ? b + L.dgq_scale : nullptr;
  v->mx_ta = mxt ? b + L.mx_ta : nullptr;
  v->mx_ta_scale = mxt ? b + L.mx_ta_scale : nullptr;
  v->mx_tb = mxt ? b + L.mx_tb : nullptr;
  v->mx_tb_scale = mxt ? b + L.mx_tb_scale : nullptr;
  v->mx_kp = (int)L.mx_kp;
  return MOE_OK;
}

moe_status_t moe_forward(const moe_problem_t* p, const moe_tensors_t* t, void* ws,
                         size_t ws_bytes, void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!t) return MOE_ERR_INVALID_ARG;
  if (p->T == 0) return MOE_OK;
  const bool fp8 = p->dtype == MOE_FP8_E4M3;
  if (!ok_ptr(t->x) || !ok_ptr(t->w_gu) || !ok_ptr(t->w_down) || !ok_ptr(t->y))
    return MOE_ERR_INVALID_ARG;
  if (p->router ? !ok_ptr(t->w_router) : !ok_ptr(t->logits)) return MOE_ERR_INVALID_ARG;
  {
    RouterOpts chk;
    moe_status_t so = make_router_opts(p->E, p->k, p->score, t->expert_bias, p->num_groups,
                                       p->group_topk, p->scaling_factor, 0, &chk);
    if (so != MOE_OK) return so;
  }
  const bool mx = p->dtype == MOE_MXFP8;
  if ((fp8 || mx) && (!ok_ptr(t->w_gu_scale) || !ok_ptr(t->w_down_scale)))
    return MOE_ERR_INVALID_ARG;
  if (p->shared_I && (!ok_ptr(t->shared_gu) || !ok_ptr(t->shared_down)))
    return MOE_ERR_INVALID_ARG;
  moe_views_t v;
  st = moe_workspace_views(p, ws, ws_bytes, &v);
  if (st != MOE_OK) return st;
  hipStream_t s = S(stream);
  const int T = p->T, H = p->H, E = p->E, k = p->k, I = p->I;
  const int N = v.rows;  // T*k, plus the padding rows of a padded dispatch
  const int align = p->align_size > 1 ? p->align_size : 1;

  // 1. router (projection first when the layer owns it), writing per-chunk expert
  //    histograms (no atomics)
  const float* logits = t->logits;
  if (p->router) {
    MOE_TRY(launch_router_logits(t->x, t->w_router, T, H, E, v.logits, s));
    logits = v.logits;
  }
  const int chunk_tokens = router_chunk_tokens(T);
  RouterOpts ro;
  st = make_router_opts(E, k, p->score, t->expert_bias, p->num_groups, p->group_topk,
                        p->scaling_factor, 0, &ro);
  if (st != MOE_OK) return st;
  const bool fuse_shared = fuses_shared(*p);
  // The layer's grouped-GEMM launches (forward and backward) keep their tile counters in
  // the workspace: the dispatch zeroes them, each launch leaves them zero.
  int32_t* const sched = (int32_t*)((uint8_t*)ws + make_layout(*p).sched);
  const bool at_input = p->weight_placement == MOE_PLACE_INPUT;
  const bool at_act = p->weight_placement == MOE_PLACE_ACTIVATION;
  float* row_prob = at_act ? (float*)((uint8_t*)ws + make_layout(*p).row_prob) : nullptr;
  const bool plain = router_opts_plain(ro, p->score);
  bool xq_done = false;  // MXFP8: the row copies were quantised as they were written
  if (plain && route_dispatch_small_fits(T, E, k) && align == 1 && !fp8 && !at_input && !at_act) {
    // a decode-sized step: routing, dispatch and row copies in one launch
    MOE_TRY(launch_route_dispatch_small(logits, T, E, k, p->score, v.topk_idx, v.topk_prob,
                                        v.counts, v.offsets, v.row_of, v.src_of, t->x, H, v.xp,
                                        fuse_shared ? N + T : -1, sched, s));
  } else {
    if (plain)
      MOE_TRY(launch_router_hist(logits, T, E, k, p->score, v.topk_idx, v.topk_prob,
                                 (int32_t*)v.scratch, chunk_tokens, s));
    else
      MOE_TRY(launch_router_ext(logits, T, E, k, p->score, ro, v.topk_idx, v.topk_prob,
                                (int32_t*)v.scratch, nullptr, nullptr, chunk_tokens, s));
    // 2. dispatch: counts, offsets (and the shared group's end), row maps from the
    //    histograms, then the row copies
    MOE_TRY(launch_dispatch_from_hist(v.topk_idx, T, E, k, chunk_tokens, (int32_t*)v.scratch,
                                      v.counts, v.offsets, v.row_of, v.src_of, s, align,
                                      v.pad_offsets, fuse_shared ? N + T : -1, sched));
    if (align > 1)  // zero padding rows (fp8 scale / ScaledSwiGLU weight 1), src_of -1
      MOE_TRY(launch_zero_pad_rows(v.offsets, v.counts, E, fp8 ? H : 2 * H, v.xp,
                                   fp8 ? v.xp_scale : row_prob, v.src_of, s));
    if (fp8) {
      MOE_TRY(launch_scatter_rows_fp8(t->x, v.row_of, T, H, k, (uint8_t*)v.xp, v.xp_scale, s));
    } else if (mx && align == 1 && !at_act) {
      MOE_TRY(launch_scatter_rows_mx(t->x, v.row_of, at_input ? v.topk_prob : nullptr, T, H, k, v.xp,
                                     (uint8_t*)v.xq, v.xq_scale, s));
      xq_done = true;
    } else {
      MOE_TRY(launch_scatter_rows(t->x, v.row_of, at_input ? v.topk_prob : nullptr, T, H, k, v.xp, s,
                                  v.topk_prob, row_prob));
    }
  }
  if (mx) {
    // MXFP8 (te_mixtral's mxfp8 recipe): rows quantised per 32-element block, block-scaled
    // GEMMs; the weight arguments hold codes and scale bytes (moe_quantize_mxfp8_weights)
    if (!xq_done) MOE_TRY(launch_mx_quantize_rows(v.xp, N, H, (uint8_t*)v.xq, v.xq_scale, s));
    MOE_TRY(launch_mx_gemm(EPI_SWIGLU, v.xq, v.xq_scale, t->w_gu, (const uint8_t*)t->w_gu_scale,
                           v.offsets, E, N, 2 * I, H, I, v.h, s, nullptr,
                           p->training ? v.gu : nullptr));
    MOE_TRY(launch_mx_quantize_rows(v.h, N, I, (uint8_t*)v.hq, v.hq_scale, s));
    MOE_TRY(launch_mx_gemm(EPI_STORE, v.hq, v.hq_scale, t->w_down,
                           (const uint8_t*)t->w_down_scale, v.offsets, E, N, H, I, 0, v.out, s));
    MOE_TRY(launch_combine(v.out, v.row_of, v.topk_prob, nullptr, T, H, k, t->y, s));
    return MOE_OK;
  }
  // 3. grouped MLP (with the fused shared group when there is one)
  GemmParams g1{};
  g1.sched = sched;
  g1.mode = fp8 ? MOE_GEMM_NT : MOE_GEMM_NN;
  g1.epi = EPI_SWIGLU;
  g1.fp8 = fp8;
  g1.A = v.xp;
  g1.a_scale = v.xp_scale;
  g1.B = t->w_gu;
  g1.b_scale = t->w_gu_scale;
  g1.offsets = v.offsets;
  g1.G = E;
  g1.rows = N;
  g1.N = 2 * I;
  g1.K = H;
  g1.C = v.h;
  g1.I = I;
  g1.gu_out = p->training ? v.gu : nullptr;
  g1.row_scale = row_prob;  // ScaledSwiGLU: h of routed rows times their weight
  if (fuse_shared) {
    g1.G = E + 1;
    g1.rows = N + T;
    g1.A_last = t->x;
    g1.B_last = t->shared_gu;
    g1.C_last = v.shared_h;
  }
  // decode-sized launches may split K (partial sums in the workspace)
  const Layout L = make_layout(*p);
  float* const part = L.splitk_bytes ? (float*)((uint8_t*)ws + L.splitk + 256) : nullptr;
  int32_t* const part_s = (int32_t*)((uint8_t*)ws + L.splitk);
  if (!fp8 && part && splitk_workspace_bytes(g1.rows, g1.G, 2LL * I) != 0) {
    g1.part = part;
    g1.part_s = part_s;
  }
  MOE_TRY(launch_grouped_gemm(g1, s));
  GemmParams g2{};
  g2.sched = sched;
  g2.mode = fp8 ? MOE_GEMM_NT : MOE_GEMM_NN;
  g2.epi = EPI_STORE;
  g2.fp8 = fp8;
  if (fp8) {
    MOE_TRY(launch_quantize_rows(v.h, N, I, v.hq, v.h_scale, s));
    g2.A = v.hq;
    g2.a_scale = v.h_scale;
  } else {
    g2.A = v.h;
  }
  g2.B = t->w_down;
  g2.b_scale = t->w_down_scale;
  g2.offsets = v.offsets;
  g2.G = E;
  g2.rows = N;
  g2.N = H;
  g2.K = I;
  g2.C = v.out;
  if (fuse_shared) {
    g2.G = E + 1;
    g2.rows = N + T;
    g2.A_last = v.shared_h;
    g2.B_last = t->shared_down;
    g2.C_last = v.shared_out;
  }
  if (!fp8 && part && splitk_workspace_bytes(g2.rows, g2.G, H) != 0) {
    g2.part = part;
    g2.part_s = part_s;
  }
  MOE_TRY(launch_grouped_gemm(g2, s));
  // shared expert: one dense group over all T tokens, read straight from x
  if (p->shared_I && !fuse_shared) {
    MOE_TRY(launch_fill_i32(v.shared_offsets, 1, 0, s));
    MOE_TRY(launch_fill_i32(v.shared_offsets + 1, 1, T, s));
    GemmParams s1{};
  s1.sched = sched;
    s1.mode = MOE_GEMM_NN;
    s1.epi = EPI_SWIGLU;
    s1.A = t->x;
    s1.B = t->shared_gu;
    s1.offsets = v.shared_offsets;
    s1.G = 1;
    s1.rows = T;
    s1.N = 2 * p->shared_I;
    s1.K = H;
    s1.C = v.shared_h;
    s1.I = p->shared_I;
    MOE_TRY(launch_grouped_gemm(s1, s));
    GemmParams s2{};
  s2.sched = sched;
    s2.mode = MOE_GEMM_NN;
    s2.epi = EPI_STORE;
    s2.A = v.shared_h;
    s2.B = t->shared_down;
    s2.offsets = v.shared_offsets;
    s2.G = 1;
    s2.rows = T;
    s2.N = H;
    s2.K = p->shared_I;
    s2.C = v.shared_out;
    MOE_TRY(launch_grouped_gemm(s2, s));
  }
  // 4. combine (unweighted when the weights already scaled the inputs or the SwiGLU output)
  MOE_TRY(launch_combine(v.out, v.row_of, at_input || at_act ? nullptr : v.topk_prob,
                         p->shared_I ? v.shared_out : nullptr, T, H, k, t->y, s));
  return MOE_OK;
}

moe_status_t moe_backward(const moe_problem_t* p, const moe_tensors_t* t, const void* dy,
                          void* dx, void* dw_gu, void* dw_down, void* ws, size_t ws_bytes,
                          void* stream) {
  moe_status_t st = check_problem(p);
  if (st != MOE_OK) return st;
  if (!t || !p->training || p->dtype == MOE_FP8_E4M3) return MOE_ERR_INVALID_ARG;
  const bool mx = p->dtype == MOE_MXFP8;
  if (mx && (!ok_ptr(t->w_gu_bwd) || !ok_ptr(t->w_down_bwd) || t->w_gu_bwd_scale == nullptr ||
             t->w_down_bwd_scale == nullptr))
    return MOE_ERR_INVALID_ARG;
  if (p->shared_I) return MOE_ERR_UNSUPPORTED;
  if (!ok_ptr(t->w_gu) || !ok_ptr(t->w_down) || !ok_ptr(dw_gu) || !ok_ptr(dw_down))
    return MOE_ERR_INVALID_ARG;
  if (p->T > 0 && (!ok_ptr(dy) || !ok_ptr(dx))) return MOE_ERR_INVALID_ARG;
  if (p->router && (!ok_ptr(t->w_router) || !ok_ptr(t->dw_router) || !ok_ptr(t->x)))
    return MOE_ERR_INVALID_ARG;
  moe_views_t v;
  st = moe_workspace_views(p, ws, ws_bytes, &v);
  if (st != MOE_OK) return st;
  hipStream_t s = S(stream);
  const int T = p->T, H = p->H, E = p->E, k = p->k, I = p->I;
  const int N = v.rows;  // T*k, plus the padding rows of a padded dispatch
  const bool at_input = p->weight_placement == MOE_PLACE_INPUT;
  const bool at_act = p->weight_placement == MOE_PLACE_ACTIVATION;
  const Layout L = make_layout(*p);
  float* const row_prob = at_act ? (float*)((uint8_t*)ws + L.row_prob) : nullptr;
  float* const row_part = at_act && p->router ? (float*)((uint8_t*)ws + L.row_part) : nullptr;
  int32_t* const gsched = (int32_t*)((uint8_t*)ws + L.sched);  // zero since the forward
  // MXFP8 without padding: the d_out copies are quantised as they are written
  const bool dq_fused = mx && p->align_size <= 1;
  bool dq_done = false;
  if (T == 0) {
    // no routed rows: the weight gradients are zero (the dW GEMMs see empty groups)
    MOE_TRY(launch_fill_i32(v.offsets, E + 1, 0, s));
  } else if (at_input || at_act) {
    // the combine was unweighted: d_out[row_of[t,j]] = dy[t]
    if (dq_fused)
      MOE_TRY(launch_scatter_rows_mx(dy, v.row_of, nullptr, T, H, k, v.d_out, (uint8_t*)v.xq,
                                     v.xq_scale, s));
    else MOE_TRY(launch_scatter_rows(dy, v.row_of, nullptr, T, H, k, v.d_out, s));
    dq_done = dq_fused;
  } else if (p->router) {
    // combine backward with the routing-weight gradient: d_out, d_logits and the split
    // operand of the router weight gradient
    MOE_TRY(launch_combine_bwd_router(dy, v.out, v.row_of, v.topk_idx, v.topk_prob, v.logits, T, H, E, k,
                                      p->score, p->scaling_factor == 0.f ? 1.f : p->scaling_factor,
                                      v.d_out, nullptr, v.d_logits, (uint16_t*)v.router_ws,
                                      router_split_cols(E), s));
  } else {
    // combine backward: d_out[row_of[t,j]] = bf16(p[t,j] * dy[t])
    if (dq_fused)
      MOE_TRY(launch_scatter_rows_mx(dy, v.row_of, v.topk_prob, T, H, k, v.d_out, (uint8_t*)v.xq,
                                     v.xq_scale, s));
    else MOE_TRY(launch_scatter_rows(dy, v.row_of, v.topk_prob, T, H, k, v.d_out, s));
    dq_done = dq_fused;
  }
  float* const r_part = p->router ? (float*)((uint8_t*)v.router_ws + router_wgrad_dls_bytes(T, E))
                                   : nullptr;
  const float r_scale = p->scaling_factor == 0.f ? 1.f : p->scaling_factor;
  if (p->router && !at_input && !at_act)
    MOE_TRY(launch_router_wgrad(t->x, (const uint16_t*)v.router_ws, T, H, E, r_part, t->dw_router, s));
  if (p->align_size > 1 && T > 0)  // the padding rows of d_out are zero
    MOE_TRY(launch_zero_pad_rows(v.offsets, v.counts, E, 2 * H, v.d_out, nullptr, nullptr, s));
  if (mx) {
    // MXFP8: data gradients with operands blocked along their K (d_out and dgu rows; the
    // weights' second copy, blocked along the stored last axis), weight gradients with
    // operands blocked along each expert's tokens
    const int Kp = v.mx_kp;
    if (N > 0) {
      if (!dq_done) MOE_TRY(launch_mx_quantize_rows(v.d_out, N, H, (uint8_t*)v.xq, v.xq_scale, s));
      MOE_TRY(launch_mx_gemm(EPI_SWIGLU_BWD, v.xq, v.xq_scale, t->w_down_bwd, t->w_down_bwd_scale,
                             v.offsets, E, N, I, H, I, v.dgu, s, v.gu, nullptr));
      MOE_TRY(launch_mx_quantize_rows(v.dgu, N, 2 * I, v.dgq, v.dgq_scale, s));
      MOE_TRY(launch_mx_gemm(EPI_STORE, v.dgq, v.dgq_scale, t->w_gu_bwd, t->w_gu_bwd_scale,
                             v.offsets, E, N, H, 2 * I, 0, v.dxp, s));
    }
    MOE_TRY(launch_mx_col_offsets(v.offsets, E, v.mx_col_offsets, s));
    MOE_TRY(launch_mx_quantize_cols(v.h, N, I, v.offsets, v.mx_col_offsets, E, Kp, v.mx_ta,
                                    v.mx_ta_scale, s));
    MOE_TRY(launch_mx_quantize_cols(v.d_out, N, H, v.offsets, v.mx_col_offsets, E, Kp, v.mx_tb,
                                    v.mx_tb_scale, s));
    MOE_TRY(launch_mx_gemm_wgrad(v.mx_ta, v.mx_ta_scale, v.mx_tb, v.mx_tb_scale, v.mx_col_offsets,
                                 E, I, H, Kp, dw_down, s));
    MOE_TRY(launch_mx_quantize_cols(v.xp, N, H, v.offsets, v.mx_col_offsets, E, Kp, v.mx_ta,
                                    v.mx_ta_scale, s));
    MOE_TRY(launch_mx_quantize_cols(v.dgu, N, 2 * I, v.offsets, v.mx_col_offsets, E, Kp, v.mx_tb,
                                    v.mx_tb_scale, s));
    MOE_TRY(launch_mx_gemm_wgrad(v.mx_ta, v.mx_ta_scale, v.mx_tb, v.mx_tb_scale, v.mx_col_offsets,
                                 E, H, 2 * I, Kp, dw_gu, s));
  } else {
  // GEMM2 backward: dgu = SwiGLU'(d_out . W_down^T), dW_down = h^T . d_out
  GemmParams a{};
  a.sched = gsched;
  a.mode = MOE_GEMM_NT;
  a.epi = EPI_SWIGLU_BWD;
  a.A = v.d_out;
  a.B = t->w_down;
  a.offsets = v.offsets;
  a.G = E;
  a.rows = N;
  a.N = I;
  a.K = H;
  a.C = v.dgu;
  a.I = I;
  a.gu_in = v.gu;
  a.row_scale = row_prob;  // ScaledSwiGLU: dh times the row's weight
  a.row_part = row_part;   // and the weight gradient's partials (router projection)
  if (N > 0) MOE_TRY(launch_grouped_gemm(a, s));
  GemmParams b{};
  b.sched = gsched;
  b.mode = MOE_GEMM_TN_DW;
  b.epi = EPI_STORE;
  b.A = v.h;
  b.B = v.d_out;
  b.offsets = v.offsets;
  b.G = E;
  b.rows = N;
  b.M = I;
  b.N = H;
  b.C = dw_down;
  MOE_TRY(launch_grouped_gemm(b, s));
  // GEMM1 backward: dxp = dgu . W_gu^T, dW_gu = xp^T . dgu
  GemmParams c{};
  c.sched = gsched;
  c.mode = MOE_GEMM_NT;
  c.epi = EPI_STORE;
  c.A = v.dgu;
  c.B = t->w_gu;
  c.offsets = v.offsets;
  c.G = E;
  c.rows = N;
  c.N = H;
  c.K = 2 * I;
  c.C = v.dxp;
  if (N > 0) MOE_TRY(launch_grouped_gemm(c, s));
  GemmParams d{};
  d.sched = gsched;
  d.mode = MOE_GEMM_TN_DW;
  d.epi = EPI_STORE;
  d.A = v.xp;
  d.B = v.dgu;
  d.offsets = v.offsets;
  d.G = E;
  d.rows = N;
  d.M = H;
  d.N = 2 * I;
  d.C = dw_gu;
  MOE_TRY(launch_grouped_gemm(d, s));
  }
  // dispatch backward: dx[t] = sum_j dxp[row_of[t,j]] (weighted when the weights scaled the
  // inputs; + the router's term)
  if (p->router && at_input) {
    MOE_TRY(launch_dispatch_bwd_router_input(v.dxp, t->x, v.row_of, v.topk_idx, v.topk_prob, v.logits,
                                             t->w_router, T, H, E, k, p->score, r_scale, dx,
                                             v.d_logits, (uint16_t*)v.router_ws,
                                             router_split_cols(E), s));
    MOE_TRY(launch_router_wgrad(t->x, (const uint16_t*)v.router_ws, T, H, E, r_part, t->dw_router, s));
  } else if (p->router && at_act) {
    MOE_TRY(launch_dispatch_bwd_router_act(v.dxp, row_part, I / 64, v.row_of, v.topk_idx,
                                           v.topk_prob, v.logits, t->w_router, T, H, E, k,
                                           p->score, r_scale, dx, v.d_logits,
                                           (uint16_t*)v.router_ws, router_split_cols(E), s));
    MOE_TRY(launch_router_wgrad(t->x, (const uint16_t*)v.router_ws, T, H, E, r_part, t->dw_router, s));
  } else if (p->router) {
    MOE_TRY(launch_dispatch_bwd_router(v.dxp, v.row_of, v.topk_idx, v.d_logits, t->w_router, T, H,
                                       E, k, dx, s));
  } else {
    MOE_TRY(launch_combine(v.dxp, v.row_of, at_input ? v.topk_prob : nullptr, nullptr, T, H, k, dx,
                           s));
  }
  return MOE_OK;
}

}  // extern "C"
