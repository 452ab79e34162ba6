// Router with its options, and the expert-bias update.
//
// Transformer Engine guide "Mixture of Experts", section "Router": besides softmax (before
// or after the top-k) and sigmoid, the score function may be sqrtsoftplus,
// sqrt(log(1 + e^l)); an expert bias is added to the scores for the selection only
// (sigmoid and sqrtsoftplus, section "Load balancing"); grouped routing splits the experts
// into equal groups, scores each group by the sum of its best expert scores, keeps the
// best groups and takes the top-k among their experts; a scaling factor multiplies the
// returned weights; the routing map may be bit-packed. torchtitan pull request 1269,
// MoE._update_expert_bias: the auxiliary-loss-free bias step.
//
// One wavefront per token. Each lane holds experts lane, lane+64, ... (EPL of them). The
// selection key is the logit, except with an expert bias, where it is fp32(score + bias);
// grouped routing sums, per group, the values of its m = k / group_topk best experts
// (softmax before the top-k, renormalised or not: the fp32 probabilities; after it: the
// logits; sigmoid and
// sqrtsoftplus: the fp32 scores, plus the bias when there is one), best first, in fp32.
// The wave writes the keys and values of its token to LDS, lane g < num_groups scores
// group g, group_topk rounds of a wave arg-max keep the groups, and the experts of the
// other groups are excluded before the k rounds of arg-max on the key (lower id first on
// a tie throughout).
#include "internal.h"

namespace moe {

namespace {

MOE_DEV float softplus_f(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }

// wave-wide arg-max of (value, id) pairs, larger value first, then the lower id;
// id 0x7fffffff marks a lane with no candidate
MOE_DEV void wave_argmax(float& bv, int& be) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oe = __shfl_xor(be, o, 64);
    const bool other = (be == 0x7fffffff) ||
                       (oe != 0x7fffffff && (ov > bv || (ov == bv && oe < be)));
    if (other) {
      bv = ov;
      be = oe;
    }
  }
}

}  // namespace

template <int EPL, bool HIST>  // experts per lane: ceil(E / 64)
__global__ __launch_bounds__(256) void router_ext_kernel(
    const float* __restrict__ logits, int T, int E, int k, int score, RouterOpts o,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_prob, int32_t* __restrict__ counts,
    uint8_t* __restrict__ routing_map, float* __restrict__ probs_dense, int chunk_tokens) {
  __shared__ int hist[256];
  __shared__ float sk[4][256], sg[4][256];  // per wave: the token's keys and group values
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  int t0, t_end, t_step;
  if (HIST) {
    t0 = blockIdx.x * chunk_tokens + wv;
    t_end = min(T, (blockIdx.x + 1) * chunk_tokens);
    t_step = waves;
  } else {
    t0 = blockIdx.x * waves + wv;
    t_end = T;
    t_step = gridDim.x * waves;
  }
  const bool per_expert = score == MOE_SIGMOID || score == MOE_SQRTSOFTPLUS;
  const bool biased = per_expert && o.expert_bias != nullptr;
  for (int t = t0; t < t_end; t += t_step) {
    const float* row = logits + (size_t)t * E;
    float key[EPL], gv[EPL];
    bool taken[EPL], chosen[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      taken[i] = e >= E;
      chosen[i] = false;
      key[i] = taken[i] ? 0.f : nan_to_ninf(row[e]);
      gv[i] = key[i];
    }
    const bool pre = score == MOE_SOFTMAX_PRE_RENORM || score == MOE_SOFTMAX_PRE;
    // softmax before the top-k without renormalisation: the weights divide by every
    // expert's exp(l - l_max)
    float zall = 0.f, vmax = -INFINITY;
    if (score == MOE_SOFTMAX_PRE) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (!taken[i]) vmax = fmaxf(vmax, key[i]);
      vmax = wave_max(vmax);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (!taken[i]) zall += expf(key[i] - vmax);
      zall = wave_sum(zall);
    }
    if (pre && o.num_groups > 1) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (!taken[i]) m = fmaxf(m, key[i]);
      m = wave_max(m);
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        gv[i] = taken[i] ? 0.f : expf(key[i] - m);
        z += gv[i];
      }
      z = wave_sum(z);
#pragma unroll
      for (int i = 0; i < EPL; ++i) gv[i] = gv[i] / z;
    } else if (per_expert) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const float l = key[i];
        const float sc = score == MOE_SIGMOID ? 1.0f / (1.0f + expf(-l)) : sqrtf(softplus_f(l));
        gv[i] = sc;
        if (biased && !taken[i]) {
          key[i] = sc + o.expert_bias[lane + 64 * i];
          gv[i] = key[i];
        }
      }
    }
    if (o.num_groups > 1) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (!taken[i]) {
          sk[wv][lane + 64 * i] = key[i];
          sg[wv][lane + 64 * i] = gv[i];
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int gsz = E / o.num_groups, m = k / o.group_topk;
      float gscore = 0.f;
      if (lane < o.num_groups) {
        // the m best (key, id) of group `lane`, each the best strictly after the previous
        float pk = 0.f, acc = 0.f;
        int pi = -1;
        for (int j = 0; j < m; ++j) {
          float bk = 0.f;
          int bi = -1;
          for (int x = 0; x < gsz; ++x) {
            const int e = lane * gsz + x;
            const float kx = sk[wv][e];
            const bool after = pi < 0 || kx < pk || (kx == pk && e > pi);
            if (after && (bi < 0 || kx > bk)) {
              bk = kx;
              bi = e;
            }
          }
          acc += sg[wv][bi];
          pk = bk;
          pi = bi;
        }
        gscore = nan_to_ninf(acc);  // a row of -inf logits: every group ties, lowest id first
      }
      uint64_t kept = 0;
      bool gdone = lane >= o.num_groups;
      for (int r = 0; r < o.group_topk; ++r) {
        float bv = gdone ? 0.f : gscore;
        int be = gdone ? 0x7fffffff : lane;
        wave_argmax(bv, be);
        kept |= 1ull << be;
        if (lane == be) gdone = true;
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (!taken[i] && !((kept >> (e / gsz)) & 1ull)) taken[i] = true;
      }
      // the next token's keys overwrite this wave's LDS rows only after these reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      float bv = 0.f;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {  // ascending id: strict > keeps the lower id on a tie
        if (!taken[i] && (be == 0x7fffffff || key[i] > bv)) {
          bv = key[i];
          be = lane + 64 * i;
        }
      }
      wave_argmax(bv, be);
      if (lane == j) my_e = be;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (be == lane + 64 * i) {
          taken[i] = true;
          chosen[i] = true;
        }
    }
    // weights from the chosen experts' logits
    const float lsel = lane < k ? nan_to_ninf(row[my_e]) : 0.f;
    float q;
    if (score == MOE_SIGMOID) {
      q = 1.0f / (1.0f + expf(-lsel));
    } else if (score == MOE_SQRTSOFTPLUS) {
      q = sqrtf(softplus_f(lsel));
    } else if (score == MOE_SOFTMAX_PRE) {
      q = expf(lsel - vmax) / zall;
    } else {
      // the largest kept logit: with grouping the first choice need not be the largest
      float mx = lane < k ? lsel : -INFINITY;
      mx = wave_max(mx);
      const float z = lane < k ? expf(lsel - mx) : 0.f;
      q = z / wave_sum(z);
    }
    q *= o.scaling;
    if (lane < k) {
      topk_idx[(size_t)t * k + lane] = my_e;
      topk_prob[(size_t)t * k + lane] = q;
      atomicAdd(&hist[my_e], 1);
    }
    if (routing_map) {
      if (o.bitmap) {
        const int nbytes = (E + 7) / 8;
        uint32_t byte = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          const uint64_t mk = __ballot(chosen[i]);
          if (lane / 8 == i) byte = (uint32_t)(mk >> (8 * (lane % 8))) & 0xffu;
        }
        if (lane < nbytes) routing_map[(size_t)t * nbytes + lane] = (uint8_t)byte;
      } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          const int e = lane + 64 * i;
          if (e < E) routing_map[(size_t)t * E + e] = chosen[i] ? 1 : 0;
        }
      }
    }
    if (probs_dense) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E && !chosen[i]) probs_dense[(size_t)t * E + e] = 0.f;
      }
      if (lane < k) probs_dense[(size_t)t * E + my_e] = q;
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

hipError_t launch_router_ext(const float* logits, int T, int E, int k, int score,
                             const RouterOpts& o, int32_t* topk_idx, float* topk_prob,
                             int32_t* counts, uint8_t* routing_map, float* probs_dense,
                             int chunk_tokens, hipStream_t s) {
  const bool hist = chunk_tokens > 0;
  if (!hist) {
    hipError_t err = launch_fill_i32(counts, E, 0, s);
    if (err != hipSuccess) return err;
  }
  if (T == 0) return hipSuccess;
  // without histograms: 16 tokens per block (four per wave), so the per-block count
  // atomics at the end stay few
  int blocks = hist ? (T + chunk_tokens - 1) / chunk_tokens : (T + 15) / 16;
  if (!hist && blocks > 2048) blocks = 2048;
#define MOE_ROUTER_EXT(n)                                                                   \
  case n:                                                                                   \
    if (hist)                                                                               \
      router_ext_kernel<n, true><<<blocks, 256, 0, s>>>(logits, T, E, k, score, o, topk_idx, \
                                                        topk_prob, counts, routing_map,      \
                                                        probs_dense, chunk_tokens);          \
    else                                                                                    \
      router_ext_kernel<n, false><<<blocks, 256, 0, s>>>(logits, T, E, k, score, o,          \
                                                         topk_idx, topk_prob, counts,        \
                                                         routing_map, probs_dense, 0);       \
    break;
  switch ((E + 63) / 64) {
    MOE_ROUTER_EXT(1)
    MOE_ROUTER_EXT(2)
    MOE_ROUTER_EXT(3)
    MOE_ROUTER_EXT(4)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_ROUTER_EXT
  return hipGetLastError();
}

// ---- expert-bias update ------------------------------------------------------------------
// One block of 256 threads (E <= 256). sign(mean - c_e) is taken exactly as
// sign(S - c_e E) on integers (S = the token total); delta = coeff * sign minus its mean,
// and bias + delta, in fp64 with one rounding to fp32.
__global__ __launch_bounds__(256) void expert_bias_update_kernel(float* __restrict__ bias,
                                                                 const int32_t* __restrict__ tpe,
                                                                 int E, float coeff) {
  __shared__ long long part[4];
  __shared__ int net[4];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const long long c = t < E ? tpe[t] : 0;
  long long sum = c;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (lane == 0) part[wv] = sum;
  __syncthreads();
  const long long S = part[0] + part[1] + part[2] + part[3];
  const long long diff = S - c * E;
  const int sg = t < E ? (diff > 0) - (diff < 0) : 0;
  int n = sg;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, 64);
  if (lane == 0) net[wv] = n;
  __syncthreads();
  if (t < E) {
    const int nt = net[0] + net[1] + net[2] + net[3];
    const double d = (double)coeff * sg;
    const double mean = ((double)coeff * nt) / E;
    bias[t] = (float)((double)bias[t] + (d - mean));
  }
}

hipError_t launch_expert_bias_update(float* bias, const int32_t* tokens_per_expert, int E,
                                     float coeff, hipStream_t s) {
  expert_bias_update_kernel<<<1, 256, 0, s>>>(bias, tokens_per_expert, E, coeff);
  return hipGetLastError();
}

}  // namespace moe
