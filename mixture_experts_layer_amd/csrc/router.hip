// Router: fused score function + top-k, one wavefront per token.
//
// Transformer Engine guide "Mixture of Experts", section "Router": the score function
// and the top-k run in one kernel with fp32 math; outputs are the selected expert ids,
// their routing weights, and optionally the [T,E] mask and dense weights.
//
// Selection works on the logits (softmax and sigmoid are strictly increasing, so they
// select the same experts): k rounds of a wave-wide arg-max with the lower expert id
// winning a tie, each lane holding up to four experts (E <= 256) in registers. A NaN logit
// counts as -inf, and each round takes the best available expert even when every one
// left is at -inf, so the ids are always k distinct experts of [0, E).
// Weights: for softmax before the top-k with renormalisation, or after the top-k,
// q_j = exp(l_j - l_max) / sum over the k kept logits -- the full-softmax denominator
// cancels in the renormalisation; for softmax before the top-k without renormalisation
// q_j = exp(l_j - l_max) / sum over all E logits; sigmoid(l_j) without renormalisation
// for the sigmoid score.
#include "internal.h"

namespace moe {

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_i32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

// HIST = false: a grid-stride loop over tokens; per-expert counts are summed in LDS and
//   added to `counts` with one atomic per (block, expert).
// HIST = true: block c owns the chunk of `chunk_tokens` tokens starting at c*chunk_tokens
//   and writes that chunk's per-expert histogram to partial[c][0..E) (no atomics); the
//   dispatch scan turns these rows into counts, offsets and per-chunk row bases.
template <int EPL, bool HIST>  // experts per lane: ceil(E / 64)
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int score, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_prob, int32_t* __restrict__ counts, uint8_t* __restrict__ routing_map,
    float* __restrict__ probs_dense, int chunk_tokens) {
  __shared__ int hist[256];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int waves = blockDim.x >> 6;
  int t0, t_end, t_step;
  if (HIST) {
    t0 = blockIdx.x * chunk_tokens + (threadIdx.x >> 6);
    t_end = min(T, (blockIdx.x + 1) * chunk_tokens);
    t_step = waves;
  } else {
    t0 = blockIdx.x * waves + (threadIdx.x >> 6);
    t_end = T;
    t_step = gridDim.x * waves;
  }
  for (int t = t0; t < t_end; t += t_step) {
    const float* row = logits + (size_t)t * E;
    float v[EPL];
    bool taken[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      int e = lane + 64 * i;
      taken[i] = e >= E;
      v[i] = taken[i] ? 0.f : nan_to_ninf(row[e]);
    }
    // softmax before the top-k without renormalisation: every expert's exp(l - l_max)
    float zall = 0.f, vmax = -__builtin_inff();
    if (score == MOE_SOFTMAX_PRE) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (!taken[i]) vmax = fmaxf(vmax, v[i]);
      vmax = wave_max(vmax);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (!taken[i]) zall += expf(v[i] - vmax);
      zall = wave_sum(zall);
    }
    int my_e = 0;
    float my_v = 0.f;
    for (int j = 0; j < k; ++j) {
      float bv = 0.f;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {  // ascending id: strict > keeps the lower id on a tie
        if (!taken[i] && (be == 0x7fffffff || v[i] > bv)) {
          bv = v[i];
          be = lane + 64 * i;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(bv, o, 64);
        int oe = __shfl_xor(be, o, 64);
        bool other = (be == 0x7fffffff) ||
                     (oe != 0x7fffffff && (ov > bv || (ov == bv && oe < be)));
        if (other) {
          bv = ov;
          be = oe;
        }
      }
      if (lane == j) {
        my_e = be;
        my_v = bv;
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (be == lane + 64 * i) taken[i] = true;
    }
    float q;
    if (score == MOE_SIGMOID) {
      q = 1.0f / (1.0f + expf(-my_v));
    } else if (score == MOE_SOFTMAX_PRE) {
      q = expf(my_v - vmax) / zall;
    } else {
      float m = __shfl(my_v, 0, 64);  // the best logit is the first choice
      float z = lane < k ? expf(my_v - m) : 0.f;
      q = z / wave_sum(z);
    }
    if (lane < k) {
      topk_idx[(size_t)t * k + lane] = my_e;
      topk_prob[(size_t)t * k + lane] = q;
      atomicAdd(&hist[my_e], 1);
    }
    if (routing_map || probs_dense) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        int e = lane + 64 * i;
        if (e < E) {
          if (routing_map) routing_map[(size_t)t * E + e] = taken[i] ? 1 : 0;
          if (probs_dense && !taken[i]) probs_dense[(size_t)t * E + e] = 0.f;
        }
      }
      if (probs_dense && lane < k) probs_dense[(size_t)t * E + my_e] = q;
    }
  }
  __syncthreads();
  if (HIST) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts[(size_t)blockIdx.x * E + e] = hist[e];
  } else {
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      if (hist[e]) atomicAdd(&counts[e], hist[e]);
  }
}

// Router for k <= 16: one token per 16-lane row (four tokens per wave), each lane holding
// the logits of experts r, r+16, ... (EPR of them). A round's arg-max is a local pass over
// the lane's untaken experts and four DPP row rotations (8, 4, 2, 1 lanes) combining
// (value, id) pairs under "larger value, then lower id" -- a total order, so every lane of
// the row ends with the same winner. Blocks of 512 threads take 32 tokens per step. HIST as
// in router_topk_kernel (tokens_per_block tokens per block, a multiple of 32).
MOE_DEV int dpp_ror(int v, int ctrl_sel) {
  switch (ctrl_sel) {  // row_ror:N is DPP control 0x120 + N
    case 8: return __builtin_amdgcn_update_dpp(v, v, 0x128, 0xf, 0xf, false);
    case 4: return __builtin_amdgcn_update_dpp(v, v, 0x124, 0xf, 0xf, false);
    case 2: return __builtin_amdgcn_update_dpp(v, v, 0x122, 0xf, 0xf, false);
    default: return __builtin_amdgcn_update_dpp(v, v, 0x121, 0xf, 0xf, false);
  }
}

// One token's routing on its 16-lane row (lane r holds experts r, r+16, ...): k rounds of
// arg-max, then the weight of the lane's choice (lanes r < k: choice r). `avail` ends with
// bit i clear where expert r + 16 i was taken.
template <int EPR>
MOE_DEV void route_row(const float* __restrict__ lrow, int E, int k, int score, int r, int& my_e,
                       float& q, int& avail) {
  float v[EPR];
  avail = 0;  // bit i: expert r + 16 i exists and is not taken
#pragma unroll
  for (int i = 0; i < EPR; ++i) {
    const int e = r + 16 * i;
    v[i] = e < E ? nan_to_ninf(lrow[e]) : 0.f;
    if (e < E) avail |= 1 << i;
  }
  const int exists = avail;
  my_e = 0;
  float my_v = 0.f, top_v = 0.f;
  for (int j = 0; j < k; ++j) {
    // branch-free: a lane with no candidate holds (-inf, INT_MAX), which every available
    // expert beats (an available one at -inf by its lower id), so the winner is always a
    // real expert; the lane's first available expert is taken whatever its value
    float bv = -__builtin_inff();
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPR; ++i) {  // ascending id: strict > keeps the lower id on a tie
      const bool take = ((avail >> i) & 1) & ((be == 0x7fffffff) | (v[i] > bv));
      bv = take ? v[i] : bv;
      be = take ? r + 16 * i : be;
    }
#pragma unroll
    for (int sh = 8; sh > 0; sh >>= 1) {
      const float ov = __int_as_float(dpp_ror(__float_as_int(bv), sh));
      const int oe = dpp_ror(be, sh);
      const bool other = (ov > bv) | ((ov == bv) & (oe < be));
      bv = other ? ov : bv;
      be = other ? oe : be;
    }
    if (j == 0) top_v = bv;
    if (r == j) {
      my_e = be;
      my_v = bv;
    }
    if ((be & 15) == r) avail &= ~(1 << (be >> 4));
  }
  if (score == MOE_SIGMOID) {
    q = 1.0f / (1.0f + expf(-my_v));
  } else if (score == MOE_SOFTMAX_PRE) {
    // the full softmax: every expert's exp(l - l_max) summed over the row's 16 lanes
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < EPR; ++i)
      if ((exists >> i) & 1) sum += expf(v[i] - top_v);
#pragma unroll
    for (int sh = 8; sh > 0; sh >>= 1) sum += __int_as_float(dpp_ror(__float_as_int(sum), sh));
    q = expf(my_v - top_v) / sum;
  } else {
    const float z = r < k ? expf(my_v - top_v) : 0.f;  // the best logit is the first choice
    float sum = z;
#pragma unroll
    for (int sh = 8; sh > 0; sh >>= 1) sum += __int_as_float(dpp_ror(__float_as_int(sum), sh));
    q = z / sum;
  }
}

template <int EPR, bool HIST>  // experts per lane: ceil(E / 16)
__global__ __launch_bounds__(512) void router_row_kernel(
    const float* __restrict__ logits, int T, int E, int k, int score, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_prob, int32_t* __restrict__ counts, uint8_t* __restrict__ routing_map,
    float* __restrict__ probs_dense, int tokens_per_block) {
  __shared__ int hist[256];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int r = threadIdx.x & 15;            // lane within the token's row
  const int row = threadIdx.x >> 4;          // 32 rows per block
  int t_begin, t_end, t_step;
  if (HIST) {
    t_begin = blockIdx.x * tokens_per_block;
    t_end = min(T, t_begin + tokens_per_block);
    t_step = 32;
  } else {
    t_begin = blockIdx.x * 32;
    t_end = T;
    t_step = gridDim.x * 32;
  }
  for (int t0 = t_begin; t0 < t_end; t0 += t_step) {
    const int t = t0 + row;
    const bool live = t < t_end;
    const float* lrow = logits + (size_t)(live ? t : t0) * E;
    int my_e, avail;
    float q;
    route_row<EPR>(lrow, E, k, score, r, my_e, q, avail);
    if (live) {
      if (r < k) {
        topk_idx[(size_t)t * k + r] = my_e;
        topk_prob[(size_t)t * k + r] = q;
        atomicAdd(&hist[my_e], 1);
      }
      if (routing_map || probs_dense) {
#pragma unroll
        for (int i = 0; i < EPR; ++i) {
          const int e = r + 16 * i;
          if (e < E) {
            const bool taken = !(avail >> i & 1);
            if (routing_map) routing_map[(size_t)t * E + e] = taken ? 1 : 0;
            if (probs_dense && !taken) probs_dense[(size_t)t * E + e] = 0.f;
          }
        }
      }
    }
    // kept experts were not zeroed above, so no ordering is needed
    if (live && probs_dense && r < k) probs_dense[(size_t)t * E + my_e] = q;
  }
  __syncthreads();
  if (HIST) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) counts[(size_t)blockIdx.x * E + e] = hist[e];
  } else {
    for (int e = threadIdx.x; e < E; e += blockDim.x)
      if (hist[e]) atomicAdd(&counts[e], hist[e]);
  }
}

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int score,
                              int32_t* topk_idx, float* topk_prob, int32_t* counts,
                              uint8_t* routing_map, float* probs_dense, hipStream_t s) {
  hipError_t err = launch_fill_i32(counts, E, 0, s);
  if (err != hipSuccess || T == 0) return err;
  if (k <= 16) {
    int blocks = (T + 31) / 32;
    if (blocks > 2048) blocks = 2048;
    const int epr = (E + 15) / 16;
#define MOE_ROUTER_ROW(n)                                                                       \
  case n:                                                                                       \
    router_row_kernel<n, false><<<blocks, 512, 0, s>>>(logits, T, E, k, score, topk_idx,         \
                                                       topk_prob, counts, routing_map,           \
                                                       probs_dense, 0);                          \
    break;
    switch ((epr + 3) / 4 * 4) {
      MOE_ROUTER_ROW(4)
      MOE_ROUTER_ROW(8)
      MOE_ROUTER_ROW(12)
      MOE_ROUTER_ROW(16)
      default:
        return hipErrorInvalidValue;
    }
#undef MOE_ROUTER_ROW
    return hipGetLastError();
  }
  int blocks = (T + 3) / 4;
  if (blocks > 2048) blocks = 2048;
  int epl = (E + 63) / 64;
#define MOE_ROUTER_CASE(n)                                                                    \
  case n:                                                                                     \
    router_topk_kernel<n, false><<<blocks, 256, 0, s>>>(logits, T, E, k, score, topk_idx,      \
                                                        topk_prob, counts, routing_map,        \
                                                        probs_dense, 0);                       \
    break;
  switch (epl) {
    MOE_ROUTER_CASE(1)
    MOE_ROUTER_CASE(2)
    MOE_ROUTER_CASE(3)
    MOE_ROUTER_CASE(4)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_ROUTER_CASE
  return hipGetLastError();
}

// A step of at most 32 tokens and 256 choices (decode) in one block: the routing above
// (one token per 16-lane row), then the dispatch metadata -- counts, offsets (and the end
// of one more group after the experts), each choice's row in expert-contiguous order, the
// stable counting sort of the flattened choices, with a choice's rank the number of
// earlier choices of the same expert -- and the row copies xp[row_of[f]] = x[f / k]. The
// results are those of the router, dispatch and scatter launches of larger steps.
template <int EPR>
__global__ __launch_bounds__(512) void route_dispatch_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int score, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_prob, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_of, int32_t* __restrict__ src_of, const u32x4_t* __restrict__ x,
    int H8, u32x4_t* __restrict__ xp, int extra_end, int32_t* __restrict__ zero16) {
  __shared__ int hist[256], base[256], s_idx[256], s_row[256], wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int r = tid & 15, t = tid >> 4;
  if (t < T) {  // whole 16-lane rows: the row's rotations stay among live lanes
    int my_e, avail;
    float q;
    route_row<EPR>(logits + (size_t)t * E, E, k, score, r, my_e, q, avail);
    if (r < k) {
      topk_idx[(size_t)t * k + r] = my_e;
      topk_prob[(size_t)t * k + r] = q;
      s_idx[t * k + r] = my_e;
      atomicAdd(&hist[my_e], 1);
    }
  }
  __syncthreads();
  // exclusive scan of the counts over the experts (E <= 256: the first four waves)
  int cnt = tid < E ? hist[tid] : 0, incl = cnt;
  if (wave < 4) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
  }
  __syncthreads();
  if (wave < 4) {
    for (int w = 0; w < wave; ++w) incl += wsum[w];
    if (tid < E) {
      base[tid] = incl - cnt;
      offsets[tid] = incl - cnt;
      counts[tid] = cnt;
    }
    if (tid == 255) offsets[E] = incl;  // threads past E add nothing: incl is the total
    if (tid == 0 && extra_end >= 0) offsets[E + 1] = extra_end;
    if (zero16 && tid < 16) zero16[tid] = 0;
  }
  __syncthreads();
  const int n = T * k;
  if (tid < n) {
    const int e = s_idx[tid];
    int rank = 0;
    for (int f = 0; f < tid; ++f) rank += s_idx[f] == e ? 1 : 0;
    const int row = base[e] + rank;
    s_row[tid] = row;
    row_of[tid] = row;
    src_of[row] = tid / k;
  }
  __syncthreads();
  // the row copies, eight 16-byte pieces per thread requested before any is stored (one
  // load latency per batch instead of one per piece)
  const int total = n * H8;
  for (int i0 = tid; i0 < total; i0 += 8 * blockDim.x) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * (int)blockDim.x;
      if (i < total) {
        const int f = i / H8, c = i - f * H8;
        v[u] = x[(size_t)(f / k) * H8 + c];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * (int)blockDim.x;
      if (i < total) {
        const int f = i / H8, c = i - f * H8;
        __builtin_nontemporal_store(v[u], &xp[(size_t)s_row[f] * H8 + c]);
      }
    }
  }
}

bool route_dispatch_small_fits(int T, int E, int k) {
  return T >= 1 && T <= 32 && k >= 1 && k <= 16 && T * k <= 256 && E >= 1 && E <= 256;
}

hipError_t launch_route_dispatch_small(const float* logits, int T, int E, int k, int score,
                                       int32_t* topk_idx, float* topk_prob, int32_t* counts,
                                       int32_t* offsets, int32_t* row_of, int32_t* src_of,
                                       const void* x, int H, void* xp, int extra_end,
                                       int32_t* zero16, hipStream_t s) {
  if (!route_dispatch_small_fits(T, E, k) || H % 8) return hipErrorInvalidValue;
  const int epr = (E + 15) / 16;
#define MOE_ROUTE_SMALL(n)                                                                      \
  case n:                                                                                      \
    route_dispatch_small_kernel<n><<<1, 512, 0, s>>>(logits, T, E, k, score, topk_idx, topk_prob, \
                                                     counts, offsets, row_of, src_of,          \
                                                     (const u32x4_t*)x, H / 8, (u32x4_t*)xp,    \
                                                     extra_end, zero16);                       \
    break;
  switch ((epr + 3) / 4 * 4) {
    MOE_ROUTE_SMALL(4)
    MOE_ROUTE_SMALL(8)
    MOE_ROUTE_SMALL(12)
    MOE_ROUTE_SMALL(16)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_ROUTE_SMALL
  return hipGetLastError();
}

hipError_t launch_router_hist(const float* logits, int T, int E, int k, int score,
                              int32_t* topk_idx, float* topk_prob, int32_t* partial,
                              int chunk_tokens, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int blocks = (T + chunk_tokens - 1) / chunk_tokens;
  if (k <= 16 && chunk_tokens % 32 == 0) {
    const int epr = (E + 15) / 16;
#define MOE_ROUTER_ROW(n)                                                                       \
  case n:                                                                                       \
    router_row_kernel<n, true><<<blocks, 512, 0, s>>>(logits, T, E, k, score, topk_idx,          \
                                                      topk_prob, partial, nullptr, nullptr,      \
                                                      chunk_tokens);                             \
    break;
    switch ((epr + 3) / 4 * 4) {
      MOE_ROUTER_ROW(4)
      MOE_ROUTER_ROW(8)
      MOE_ROUTER_ROW(12)
      MOE_ROUTER_ROW(16)
      default:
        return hipErrorInvalidValue;
    }
#undef MOE_ROUTER_ROW
    return hipGetLastError();
  }
  int epl = (E + 63) / 64;
#define MOE_ROUTER_CASE(n)                                                                     \
  case n:                                                                                      \
    router_topk_kernel<n, true><<<blocks, 256, 0, s>>>(logits, T, E, k, score, topk_idx,        \
                                                       topk_prob, partial, nullptr, nullptr,    \
                                                       chunk_tokens);                          \
    break;
  switch (epl) {
    MOE_ROUTER_CASE(1)
    MOE_ROUTER_CASE(2)
    MOE_ROUTER_CASE(3)
    MOE_ROUTER_CASE(4)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_ROUTER_CASE
  return hipGetLastError();
}

}  // namespace moe
