// Auxiliary load-balancing loss.
//
// Transformer Engine guide "Mixture of Experts", section "Load balancing": a helper returns
// dense routing scores (one per expert, ignoring expert bias and grouped routing) with a
// plain top-k routing map, and the loss takes those scores with the per-expert token
// counts of the real router, so it has a gradient for every expert's logit.
// The loss is the Switch Transformer balance loss (Fedus, Zoph and Shazeer 2021, section
// 2.2), coeff * E * sum_e f_e P_e, with f_e = c_e / (k T) the fraction of routed
// (token, choice) pairs that went to expert e and P_e = sum_t s_te / T the mean score:
//   loss = coeff * E / (k T^2) * sum_e c_e sum_t s_te.
// The scores of a token form a distribution over the experts: the softmax over all experts
// for the softmax score functions, the sigmoid / sqrtsoftplus scores divided by their sum.
//
// Kernels: dense scores, one wave per token (four tokens per block); the loss as per-block
// column sums over fixed token chunks and one block that adds them in a fixed order
// (deterministic); the gradient, one wave per token, recomputing the scores.
#include "internal.h"

namespace moe {

namespace {

MOE_DEV float softplus_aux(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }

// The token's values r (EPL per lane, 0 past E) and their sum: softmax -> exp(l - l_max),
// sigmoid -> sigmoid(l), sqrtsoftplus -> sqrt(softplus(l)). The scores are r / sum.
template <int EPL>
MOE_DEV float aux_values(const float* row, int E, int score, int lane, float (&v)[EPL],
                         float (&r)[EPL]) {
  const bool smax = score == MOE_SOFTMAX_PRE_RENORM || score == MOE_SOFTMAX_POST ||
                    score == MOE_SOFTMAX_PRE;
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? nan_to_ninf(row[e]) : -__builtin_inff();
    m = fmaxf(m, v[i]);
  }
  if (smax) m = wave_max(m);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    float x = 0.f;
    if (e < E) {
      if (smax) x = expf(v[i] - m);
      else if (score == MOE_SIGMOID) x = 1.0f / (1.0f + expf(-v[i]));
      else x = sqrtf(softplus_aux(v[i]));
    }
    r[i] = x;
    sum += x;
  }
  return wave_sum(sum);
}

}  // namespace

template <int EPL>
__global__ __launch_bounds__(256) void aux_scores_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int score,
                                                         float* __restrict__ scores,
                                                         uint8_t* __restrict__ routing_map) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // the whole wave
  const float* row = logits + (size_t)t * E;
  float v[EPL], r[EPL];
  const float sum = aux_values<EPL>(row, E, score, lane, v, r);
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) scores[(size_t)t * E + e] = r[i] / sum;
  }
  if (!routing_map) return;
  // the plain top-k on the logits (no bias, no groups): k rounds of a wave arg-max, the
  // best available expert first, the lower id on a tie
  bool taken[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) taken[i] = lane + 64 * i >= E;
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (!taken[i] && (be == 0x7fffffff || v[i] > bv)) {
        bv = v[i];
        be = lane + 64 * i;
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      const bool other = (be == 0x7fffffff) ||
                         (oe != 0x7fffffff && (ov > bv || (ov == bv && oe < be)));
      bv = other ? ov : bv;
      be = other ? oe : be;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (be == lane + 64 * i) taken[i] = true;
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) routing_map[(size_t)t * E + e] = taken[i] ? 1 : 0;
  }
}

// Column sums of the scores over token chunk b: part[b][e] (thread e, rows in order).
__global__ __launch_bounds__(256) void aux_colsum_kernel(const float* __restrict__ scores, int T,
                                                         int E, int chunk,
                                                         float* __restrict__ part) {
  const int b = blockIdx.x, e = threadIdx.x;
  if (e >= E) return;
  const int t0 = b * chunk, t1 = min(T, t0 + chunk);
  float acc = 0.f;
  // rows 8 at a time, requested before any is added; the sum still runs in row order
  for (int ta = t0; ta < t1; ta += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ta + j < t1 ? scores[(size_t)(ta + j) * E + e] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (ta + j < t1) acc += v[j];
  }
  part[(size_t)b * E + e] = acc;
}

// loss = C * sum_e c_e * (sum over chunks, in order, of part[b][e]); one block of 256.
__global__ __launch_bounds__(256) void aux_loss_final_kernel(const float* __restrict__ part, int B,
                                                             int E,
                                                             const int32_t* __restrict__ counts,
                                                             float C, float* __restrict__ loss) {
  __shared__ float red[4];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  float x = 0.f;
  if (e < E) {
    float col = 0.f;
    for (int b = 0; b < B; ++b) col += part[(size_t)b * E + e];
    x = (float)counts[e] * col;
  }
  x = wave_sum(x);
  if (lane == 0) red[wave] = x;
  __syncthreads();
  if (e == 0) loss[0] = C * ((red[0] + red[1]) + (red[2] + red[3]));
}

// d_logits (= or +=) the gradient of the loss for the upstream d_loss: g_e = C d c_e,
// D = sum_i s_i g_i; softmax: s_e (g_e - D); sigmoid: r_e (1 - r_e) (g_e - D) / sum r;
// sqrtsoftplus: sigmoid(l_e) / (2 r_e) (g_e - D) / sum r.
template <int EPL>
__global__ __launch_bounds__(256) void aux_loss_bwd_kernel(const float* __restrict__ logits, int T,
                                                           int E, int score,
                                                           const int32_t* __restrict__ counts,
                                                           float C, const float* __restrict__ d_loss,
                                                           float* __restrict__ d_logits,
                                                           int accumulate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float cd = C * (d_loss ? d_loss[0] : 1.0f);
  float v[EPL], r[EPL], g[EPL];
  const float sum = aux_values<EPL>(logits + (size_t)t * E, E, score, lane, v, r);
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    g[i] = e < E ? cd * (float)counts[e] : 0.f;
    dot = fmaf(r[i] / sum, g[i], dot);
  }
  dot = wave_sum(dot);
  const bool smax = score == MOE_SOFTMAX_PRE_RENORM || score == MOE_SOFTMAX_POST ||
                    score == MOE_SOFTMAX_PRE;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e >= E) continue;
    float d;
    if (smax) {
      d = (r[i] / sum) * (g[i] - dot);
    } else {
      const float dr = score == MOE_SIGMOID ? r[i] * (1.0f - r[i])
                                            : (1.0f / (1.0f + expf(-v[i]))) / (2.0f * r[i]);
      d = dr * (g[i] - dot) / sum;
    }
    float* o = d_logits + (size_t)t * E + e;
    *o = accumulate ? *o + d : d;
  }
}

int aux_chunk_tokens(int T) {
  const int c = (T + 511) / 512;  // at most 512 chunks
  return c < 64 ? 64 : c;
}

size_t aux_loss_scratch_bytes(int T, int E) {
  const int c = aux_chunk_tokens(T);
  const size_t B = T > 0 ? (size_t)(T + c - 1) / c : 1;
  return B * (size_t)E * sizeof(float);
}

#define MOE_AUX_EPL(launch)         \
  switch ((E + 63) / 64) {          \
    case 1: launch(1); break;       \
    case 2: launch(2); break;       \
    case 3: launch(3); break;       \
    case 4: launch(4); break;       \
    default: return hipErrorInvalidValue; \
  }

hipError_t launch_aux_scores(const float* logits, int T, int E, int k, int score, float* scores,
                             uint8_t* routing_map, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int blocks = (T + 3) / 4;
#define L(n) aux_scores_kernel<n><<<blocks, 256, 0, s>>>(logits, T, E, k, score, scores, routing_map)
  MOE_AUX_EPL(L)
#undef L
  return hipGetLastError();
}

hipError_t launch_aux_loss(const float* scores, const int32_t* counts, int T, int E, float C,
                           float* loss, float* part, hipStream_t s) {
  const int chunk = aux_chunk_tokens(T);
  const int B = T > 0 ? (T + chunk - 1) / chunk : 0;
  if (B > 0) {
    aux_colsum_kernel<<<B, 256, 0, s>>>(scores, T, E, chunk, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  aux_loss_final_kernel<<<1, 256, 0, s>>>(part, B, E, counts, C, loss);
  return hipGetLastError();
}

hipError_t launch_aux_loss_bwd(const float* logits, int T, int E, int score, const int32_t* counts,
                               float C, const float* d_loss, float* d_logits, int accumulate,
                               hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int blocks = (T + 3) / 4;
#define L(n) aux_loss_bwd_kernel<n><<<blocks, 256, 0, s>>>(logits, T, E, score, counts, C, d_loss, \
                                                           d_logits, accumulate)
  MOE_AUX_EPL(L)
#undef L
  return hipGetLastError();
}

#undef MOE_AUX_EPL

}  // namespace moe
