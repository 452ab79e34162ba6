// Router projection and router backward.
//
// Transformer Engine guide "Mixture of Experts", section "Example: MoE layer on a single
// device": the logits the router scores come from a bias-free linear layer of the hidden
// states (te_mixtral.py, TEMixtralSparseMoeBlock: a gate of shape (experts, hidden));
// section "Router": score function and top-k form one differentiable step with fp32 math;
// section "Token combine": the merging weights are an input of the differentiable
// combine, so they receive a gradient.
//
//  logits    = x . W_r^T                    x [T,H] bf16, W_r [E,H] bf16, logits fp32
//  d_prob    = <dy[t], out[row_of[t,j]]>    per routed pair, fp32
//  d_logits  = score-function backward of d_prob at the kept experts, 0 elsewhere:
//              softmax (before or after the top-k: the same function of the kept
//              logits) q_j (d_prob_j - sum_i q_i d_prob_i); sigmoid d_prob_j q_j (1-q_j)
//  dW_r      = d_logits^T . x               (split-K weight-gradient GEMM + reduce)
//  dx       += d_logits . W_r               (folded into the dispatch backward)
#include "internal.h"

namespace moe {

// ---- logits = x . W_r^T ------------------------------------------------------------
// One block per 32 tokens, four waves; wave w owns the 32-expert blocks w and w+4
// (E <= 256). Both operands are K-contiguous, so each lane loads its 16-byte MFMA
// fragment (8 bf16 of one row) straight from memory: the token rows stream from HBM once
// per block, the router weight (E*H*2 bytes) is served from L2.
// v_mfma_f32_32x32x16_bf16 with the weight fragment as the first operand: lane l holds
// token row l%32 and experts 8*(v/4) + 4*(l/32) + v%4 of its 32-expert block.
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ w, int T,
                                                            int H, int E,
                                                            float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 32;
  const int r = lane & 31, kq = (lane >> 5) * 8;
  const int tm = min(t0 + r, T - 1);  // rows past T read the last row; never stored
  const bf16x8_t* xa = (const bf16x8_t*)(x + (size_t)tm * H + kq);
  const bool live0 = wave * 32 < E, live1 = (wave + 4) * 32 < E;  // wave-uniform
  const int n0 = min(wave * 32 + r, E - 1), n1 = min((wave + 4) * 32 + r, E - 1);
  const bf16x8_t* wb0 = (const bf16x8_t*)(w + (size_t)n0 * H + kq);
  const bf16x8_t* wb1 = (const bf16x8_t*)(w + (size_t)n1 * H + kq);
  f32x16_t acc0 = {}, acc1 = {};
  if (!live0) return;
  // H % 64 == 0: four 16-wide K steps per iteration, loads issued before the multiplies
  for (int k = 0; k < H; k += 64) {
    bf16x8_t a[4], b0[4], b1[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = xa[(k + 16 * s) / 8];
#pragma unroll
    for (int s = 0; s < 4; ++s) b0[s] = wb0[(k + 16 * s) / 8];
    if (live1) {
#pragma unroll
      for (int s = 0; s < 4; ++s) b1[s] = wb1[(k + 16 * s) / 8];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0[s], a[s], acc0, 0, 0, 0);
    if (live1) {
#pragma unroll
      for (int s = 0; s < 4; ++s) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1[s], a[s], acc1, 0, 0, 0);
    }
  }
  if (t0 + r >= T) return;
  float* row = logits + (size_t)(t0 + r) * E;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int e = 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
    if (wave * 32 + e < E) row[wave * 32 + e] = acc0[v];
    if (live1 && (wave + 4) * 32 + e < E) row[(wave + 4) * 32 + e] = acc1[v];
  }
}

hipError_t launch_router_logits(const void* x, const void* w_router, int T, int H, int E,
                                float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  router_logits_kernel<<<(T + 31) / 32, 256, 0, s>>>((const uint16_t*)x, (const uint16_t*)w_router,
                                                     T, H, E, logits);
  return hipGetLastError();
}

// ---- combine backward with the routing-weight gradient --------------------------------
// One block per token (256 threads). Reads dy[t] once and the token's k expert output
// rows, writes the k rows d_out = bf16(q_j dy[t]), and reduces the k dot products
// d_prob_j = <dy[t], out_j> (fp32 partial sums per thread in slot order, then a wave and
// a block reduction). The score-function backward then runs on the k values, and the
// token's dense d_logits row is written (0 at the experts not kept). With `dls` the same
// values are also written as two bf16 halves, hi = bf16(d) at column e and
// lo = bf16(d - hi) at column E + e of a row of `mp` columns (zero past 2E): the operand
// of the router weight-gradient GEMM, which so keeps about 16 bits of each value.
template <int KM>  // a bound on k: 8 or 32
__global__ __launch_bounds__(256) void combine_bwd_router_kernel(
    const u32x4_t* __restrict__ dy, const u32x4_t* __restrict__ out,
    const int32_t* __restrict__ row_of, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ prob, int H8, int E, int k, int score, u32x4_t* __restrict__ d_out,
    float* __restrict__ d_prob, float* __restrict__ d_logits, uint16_t* __restrict__ dls, int mp) {
  __shared__ int rows[32], ids[32];
  __shared__ float p[32], red[4][32], dl_s[32];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < k) {
    rows[tid] = row_of[(size_t)t * k + tid];
    ids[tid] = topk_idx[(size_t)t * k + tid];
    p[tid] = prob[(size_t)t * k + tid];
  }
  __syncthreads();
  float dot[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) dot[j] = 0.f;
  for (int v = tid; v < H8; v += 256) {
    const u32x4_t g = dy[(size_t)t * H8 + v];
#pragma unroll
    for (int j0 = 0; j0 < KM; j0 += 8) {
      if (j0 >= k) continue;  // (continue, not break: the loop stays unrolled)
      u32x4_t o[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (j0 + jj < k) o[jj] = __builtin_nontemporal_load(&out[(size_t)rows[j0 + jj] * H8 + v]);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj >= k) continue;
        float s = dot[j0 + jj];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          s = fmaf(bf16lo(g[d]), bf16lo(o[jj][d]), s);
          s = fmaf(bf16hi(g[d]), bf16hi(o[jj][d]), s);
        }
        dot[j0 + jj] = s;
        const float q = p[j0 + jj];
        u32x4_t w;
#pragma unroll
        for (int d = 0; d < 4; ++d) w[d] = pack_bf16x2(q * bf16lo(g[d]), q * bf16hi(g[d]));
        __builtin_nontemporal_store(w, &d_out[(size_t)rows[j0 + jj] * H8 + v]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j >= k) continue;
    const float s = wave_sum(dot[j]);
    if (lane == 0) red[wave][j] = s;
  }
  __syncthreads();
  if (tid < k) {
    const float dq = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
    if (d_prob) d_prob[(size_t)t * k + tid] = dq;
    red[0][tid] = dq;  // only thread tid reads or writes red[*][tid] here
  }
  __syncthreads();
  if (tid < k) {
    const float q = p[tid], dq = red[0][tid];
    float dl;
    if (score == MOE_SIGMOID) {
      dl = dq * q * (1.0f - q);
    } else {  // both softmax orders: the same function of the kept logits
      float sdot = 0.f;
      for (int j = 0; j < k; ++j) sdot = fmaf(p[j], red[0][j], sdot);
      dl = q * (dq - sdot);
    }
    dl_s[tid] = dl;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    float v = 0.f;
    for (int j = 0; j < k; ++j) v = ids[j] == e ? dl_s[j] : v;
    d_logits[(size_t)t * E + e] = v;
    if (dls) {
      const uint32_t hi = f32_to_bf16(v);
      dls[(size_t)t * mp + e] = (uint16_t)hi;
      dls[(size_t)t * mp + E + e] = (uint16_t)f32_to_bf16(v - bf16_to_f32((uint16_t)hi));
    }
  }
  if (dls)
    for (int c = 2 * E + tid; c < mp; c += 256) dls[(size_t)t * mp + c] = 0;
}

hipError_t launch_combine_bwd_router(const void* dy, const void* out, const int32_t* row_of,
                                     const int32_t* topk_idx, const float* prob, int T, int H,
                                     int E, int k, int score, void* d_out, float* d_prob,
                                     float* d_logits, uint16_t* dls, int mp, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (k <= 8)
    combine_bwd_router_kernel<8><<<T, 256, 0, s>>>((const u32x4_t*)dy, (const u32x4_t*)out, row_of,
                                                   topk_idx, prob, H / 8, E, k, score,
                                                   (u32x4_t*)d_out, d_prob, d_logits, dls, mp);
  else
    combine_bwd_router_kernel<32><<<T, 256, 0, s>>>((const u32x4_t*)dy, (const u32x4_t*)out, row_of,
                                                    topk_idx, prob, H / 8, E, k, score,
                                                    (u32x4_t*)d_out, d_prob, d_logits, dls, mp);
  return hipGetLastError();
}

// ---- d_logits -> the two bf16 halves of the weight-gradient operand ---------------------
// (for a d_logits that did not come from combine_bwd_router_kernel)
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ d_logits,
                                                           int T, int E, int mp,
                                                           uint16_t* __restrict__ dls) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)T * mp) return;
  const int t = (int)(i / mp), c = (int)(i % mp);
  uint32_t v = 0;
  if (c < E) {
    v = f32_to_bf16(d_logits[(size_t)t * E + c]);
  } else if (c < 2 * E) {
    const float d = d_logits[(size_t)t * E + c - E];
    v = f32_to_bf16(d - bf16_to_f32((uint16_t)f32_to_bf16(d)));
  }
  dls[i] = (uint16_t)v;
}

hipError_t launch_router_split(const float* d_logits, int T, int E, int mp, uint16_t* dls,
                               hipStream_t s) {
  const size_t n = (size_t)T * mp;
  if (n == 0) return hipSuccess;
  router_split_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(d_logits, T, E, mp, dls);
  return hipGetLastError();
}

// ---- dW_r from the split-K partials ------------------------------------------------------
// part [S, mp, H] fp32: rows [0,E) hold hi^T x and rows [E,2E) lo^T x of each K split.
// dw[e,h] = sum over s in order of (hi part + lo part). Four columns per thread.
__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(const f32x4_t* __restrict__ part,
                                                                  int S, int E, int H4, int mp,
                                                                  f32x4_t* __restrict__ dw) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= E * H4) return;
  const int e = i / H4, c = i % H4;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const f32x4_t a = part[((size_t)s * mp + e) * H4 + c];
    const f32x4_t b = part[((size_t)s * mp + E + e) * H4 + c];
    acc += a + b;
  }
  dw[i] = acc;
}

hipError_t launch_router_wgrad_reduce(const float* part, int S, int E, int H, int mp, float* dw,
                                      hipStream_t s) {
  const int n = E * (H / 4);
  router_wgrad_reduce_kernel<<<(n + 255) / 256, 256, 0, s>>>((const f32x4_t*)part, S, E, H / 4, mp,
                                                            (f32x4_t*)dw);
  return hipGetLastError();
}

}  // namespace moe
