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
//  d_logits  = score-function backward of d_prob at the kept experts, 0 elsewhere. With
//              the weights q = c s (c the scaling factor, s the score-function output):
//              softmax (before or after the top-k: the same function of the kept
//              logits) c s_j (d_prob_j - sum_i s_i d_prob_i); sigmoid c d_prob_j s_j (1-s_j);
//              sqrtsoftplus c d_prob_j sigmoid(l_j) / (2 s_j), where s^2 = softplus(l)
//              gives sigmoid(l) = 1 - e^(-s^2)
//  dW_r      = d_logits^T . x               (split-K weight-gradient GEMM + reduce)
//  dx       += d_logits . W_r               (folded into the dispatch backward)
#include "internal.h"

namespace moe {

// ---- logits = x . W_r^T ------------------------------------------------------------
// One block per 16 tokens and 16*NB experts (blockIdx.y picks the expert range; NB is the
// power of two that covers E, at most 8), eight waves splitting K: wave w multiplies the
// pairs of 32-wide K chunks w, w+8, ... for every 16-expert tile of the block, and the
// eight partial tiles are summed in LDS in wave order (deterministic).
// Both operands are K-contiguous and are loaded straight into registers: lane l reads 16
// bytes of row l/4 (piece l%4 of the row's 64-byte K chunk), so every quad of lanes reads
// one contiguous 64-byte segment, and one ds_bpermute per dword then moves piece p of row
// r to lane r + 16p, the MFMA operand layout. The two chunks of a pair use two fragment
// sets in turn, each reloaded with the next pair as soon as it has been multiplied, so one
// set's loads are in flight while the other multiplies; every load is unconditional (the
// prefetch past the last pair re-reads it), so the compiler waits for exactly the set in
// use. The token rows stream from HBM once; the router weight (E*H*2 bytes) comes from L2,
// once per 16 tokens (blocks of 32 or 64 tokens, which read it less often, measured
// slower: half or a quarter of the blocks, and the same wave-serial load chain).
// v_mfma_f32_16x16x32_bf16 with the weight fragment as the first operand: lane l holds
// token l%16 and experts 4*(l/16) + q, q < 4, of its tile.
constexpr int kLogitWaves = 8;
template <int NB>
__global__ __launch_bounds__(kLogitWaves * 64) void router_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T, int H, int E,
    float* __restrict__ logits) {
  constexpr int MT = 1;  // 16-token tiles per block
  __shared__ float red[kLogitWaves][16][16 * NB + 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16 * NB;
  // rows past T or E read the last row; their results are never stored
  const int lr = lane >> 2, lp = (lane & 3) * 8;
  const int src = (4 * (lane & 15) + (lane >> 4)) * 4;  // byte address of the source lane
  const uint16_t* xa[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xa[m] = x + (size_t)min(t0 + 16 * m + lr, T - 1) * H + lp;
  const uint16_t* wb[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) wb[j] = w + (size_t)min(e0 + 16 * j + lr, E - 1) * H + lp;
  auto perm = [&](const bf16x8_t& v) __attribute__((always_inline)) -> bf16x8_t {
    typedef __attribute__((ext_vector_type(4))) int i4;
    i4 u = __builtin_bit_cast(i4, v), o;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = __builtin_amdgcn_ds_bpermute(src, u[d]);
    return __builtin_bit_cast(bf16x8_t, o);
  };
  f32x4_t acc[MT][NB];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bf16x8_t a0[MT], b0[NB], a1[MT], b1[NB];
  auto load = [&](int c, bf16x8_t* a, bf16x8_t* b) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < MT; ++m) a[m] = *(const bf16x8_t*)(xa[m] + 32 * c);
#pragma unroll
    for (int j = 0; j < NB; ++j) b[j] = *(const bf16x8_t*)(wb[j] + 32 * c);
  };
  auto mul = [&](const bf16x8_t* a, const bf16x8_t* b) __attribute__((always_inline)) {
    bf16x8_t ap[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) ap[m] = perm(a[m]);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const bf16x8_t bp = perm(b[j]);
#pragma unroll
      for (int m = 0; m < MT; ++m)
        acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bp, ap[m], acc[m][j], 0, 0, 0);
    }
  };
  const int npair = H / 64;  // H % 64 == 0
  if (wave < npair) {
    load(2 * wave, a0, b0);
    load(2 * wave + 1, a1, b1);
    for (int p = wave; p < npair; p += kLogitWaves) {
      const int pn = min(p + kLogitWaves, npair - 1);
      // scheduling barriers keep each set's loads right after its multiplies (the
      // scheduler would otherwise sink them next to their use, one latency per pair)
      mul(a0, b0);
      load(2 * pn, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mul(a1, b1);
      load(2 * pn + 1, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[wave][lane & 15][16 * j + 4 * (lane >> 4) + q] = acc[0][j][q];
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * 16 * NB; i += kLogitWaves * 64) {
    const int tr = i / (16 * NB), col = i % (16 * NB);
    float v = red[0][tr][col];
#pragma unroll
    for (int ww = 1; ww < kLogitWaves; ++ww) v += red[ww][tr][col];
    if (t0 + tr < T && e0 + col < E) logits[(size_t)(t0 + tr) * E + e0 + col] = v;
  }
}

hipError_t launch_router_logits(const void* x, const void* w_router, int T, int H, int E,
                                float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const unsigned bx = (T + 15) / 16;
  auto go = [&](auto kern, int nb) {
    kern<<<dim3(bx, (E + 16 * nb - 1) / (16 * nb)), kLogitWaves * 64, 0, s>>>(
        (const uint16_t*)x, (const uint16_t*)w_router, T, H, E, logits);
    return hipGetLastError();
  };
  if (E <= 16) return go(router_logits_kernel<1>, 1);
  if (E <= 32) return go(router_logits_kernel<2>, 2);
  if (E <= 64) return go(router_logits_kernel<4>, 4);
  return go(router_logits_kernel<8>, 8);
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

// The block's k partial dot products -> d_prob (optional), the score-function backward
// -> dl_s[k] in LDS, the token's d_logits row (also kept in LDS, dl_row[E]) and its split
// halves. Every thread calls it. Softmax before the top-k without renormalisation also
// moves the logits of the experts not kept: with u_j the kept probabilities and
// S = sum_j u_j d_prob_j, expert e gets -c p_e S, p_e = exp(l_e - l_max) / sum over the
// token's logits (read from `logits`, block max and sum).
template <int KM>
MOE_DEV void router_score_bwd(const float (&dot)[KM], int t, int E, int k, int score,
                              float scaling, const float* p, const int* ids, float (*red)[32],
                              float* dl_s, float* dl_row, const float* __restrict__ logits,
                              float* __restrict__ d_prob, float* __restrict__ d_logits,
                              uint16_t* __restrict__ dls, int mp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // softmax before the top-k: this token's logit, the block max and the block sum
  float pe = 0.f;
  if (score == MOE_SOFTMAX_PRE) {
    const float l = tid < E ? nan_to_ninf(logits[(size_t)t * E + tid]) : -__builtin_inff();
    const float wm = wave_max(l);
    if (lane == 0) red[wave][31] = wm;
    __syncthreads();
    const float m = fmaxf(fmaxf(red[0][31], red[1][31]), fmaxf(red[2][31], red[3][31]));
    const float z = tid < E ? expf(l - m) : 0.f;
    __syncthreads();
    const float ws = wave_sum(z);
    if (lane == 0) red[wave][31] = ws;
    __syncthreads();
    pe = z / ((red[0][31] + red[1][31]) + (red[2][31] + red[3][31]));
    __syncthreads();
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
    const float sv = p[tid] / scaling, dq = red[0][tid];
    float dl;
    if (score == MOE_SIGMOID) {
      dl = scaling * dq * sv * (1.0f - sv);
    } else if (score == MOE_SQRTSOFTPLUS) {
      dl = scaling * dq * (-expm1f(-sv * sv)) / (2.0f * sv);
    } else {  // softmax: both renormalised orders are the same function of the kept
              // logits; without renormalisation the same form with the full probabilities
      float sdot = 0.f;
      for (int j = 0; j < k; ++j) sdot = fmaf(p[j] / scaling, red[0][j], sdot);
      dl = scaling * sv * (dq - sdot);
      if (tid == 0) red[1][31] = sdot;  // S, for the experts not kept
    }
    dl_s[tid] = dl;
  }
  __syncthreads();
  const float off = score == MOE_SOFTMAX_PRE ? -scaling * red[1][31] : 0.f;
  for (int e = tid; e < E; e += 256) {
    float v = off * pe;  // e < 256: thread e holds p_e
    for (int j = 0; j < k; ++j) v = ids[j] == e ? dl_s[j] : v;
    d_logits[(size_t)t * E + e] = v;
    dl_row[e] = v;
    if (dls) {
      const uint32_t hi = f32_to_bf16(v);
      dls[(size_t)t * mp + e] = (uint16_t)hi;
      dls[(size_t)t * mp + E + e] = (uint16_t)f32_to_bf16(v - bf16_to_f32((uint16_t)hi));
    }
  }
  if (dls)
    for (int c = 2 * E + tid; c < mp; c += 256) dls[(size_t)t * mp + c] = 0;
  __syncthreads();  // dl_row complete
}

// The nonzero entries of the token's d_logits row, ascending expert id, compacted into
// nz_e / nz_v (LDS); returns their number. Every thread calls it (E <= 256 = blockDim).
MOE_DEV int compact_nonzero(const float* dl_row, int E, int* nz_e, float* nz_v, int* wcount) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float v = tid < E ? dl_row[tid] : 0.f;
  const bool nz = v != 0.f;
  const uint64_t b = __ballot(nz);
  if (lane == 0) wcount[wave] = __popcll(b);
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? wcount[w] : 0;
    total += wcount[w];
  }
  if (nz) {
    const int at = before + __popcll(b & lanemask_lt());
    nz_e[at] = tid;
    nz_v[at] = v;
  }
  __syncthreads();
  return total;
}

template <int KM>  // a bound on k: 8 or 32
__global__ __launch_bounds__(256) void combine_bwd_router_kernel(
    const u32x4_t* __restrict__ dy, const u32x4_t* __restrict__ out,
    const int32_t* __restrict__ row_of, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ prob, const float* __restrict__ logits, int H8, int E, int k,
    int score, float scaling, u32x4_t* __restrict__ d_out,
    float* __restrict__ d_prob, float* __restrict__ d_logits, uint16_t* __restrict__ dls, int mp) {
  __shared__ int rows[32], ids[32];
  __shared__ float p[32], red[4][32], dl_s[32], dl_row[256];
  const int t = blockIdx.x, tid = threadIdx.x;
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
  router_score_bwd<KM>(dot, t, E, k, score, scaling, p, ids, red, dl_s, dl_row, logits, d_prob,
                       d_logits, dls, mp);
}

// ---- dispatch backward of a layer that weights the expert inputs ---------------------------
// torchtitan pull request 1269, MoE.forward with scoring_before_experts: xp = q x, so
// dx[t] = sum_j q_j dxp[row_j] and d_prob_j = <dxp[row_j], x[t]>. One block per token:
// pass 1 reads x[t] and the k dxp rows and reduces the k dot products, the score-function
// backward follows (router_score_bwd), and pass 2 writes dx[t] = bf16(sum_j q_j dxp[row_j]
// + sum_j d_logits[t,e_j] W_r[e_j]) (fp32 sum, one rounding; the dxp rows were just read,
// so the second read comes from cache).
// ACT (ScaledSwiGLU: the weights scaled the SwiGLU output): d_prob_j is the sum of the P
// per-64-column partials of row row_of[t,j] written by the SwiGLU-backward epilogue
// (threads take slots tid, tid + 256, ...; the block reduction adds them in a fixed
// order), and dx[t] = bf16(sum_j dxp[row_j] + router term), unweighted.
template <int KM, bool ACT>
__global__ __launch_bounds__(256) void dispatch_bwd_router_input_kernel(
    const u32x4_t* __restrict__ dxp, const u32x4_t* __restrict__ x,
    const float* __restrict__ row_part, int P,
    const int32_t* __restrict__ row_of, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ prob, const float* __restrict__ logits,
    const u32x4_t* __restrict__ w_router, int H8, int E, int k, int score, float scaling,
    u32x4_t* __restrict__ dx, float* __restrict__ d_logits, uint16_t* __restrict__ dls, int mp) {
  __shared__ int rows[32], ids[32], nz_e[256], wcount[4];
  __shared__ float p[32], red[4][32], dl_s[32], dl_row[256], nz_v[256];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < k) {
    rows[tid] = row_of[(size_t)t * k + tid];
    ids[tid] = topk_idx[(size_t)t * k + tid];
    p[tid] = prob[(size_t)t * k + tid];
  }
  __syncthreads();
  float dot[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) dot[j] = 0.f;
  if constexpr (ACT) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j >= k) continue;
      float a = 0.f;
      for (int q = tid; q < P; q += 256) a += row_part[(size_t)rows[j] * P + q];
      dot[j] = a;
    }
  }
  for (int v = tid; v < (ACT ? 0 : H8); v += 256) {
    const u32x4_t xv = x[(size_t)t * H8 + v];
#pragma unroll
    for (int j0 = 0; j0 < KM; j0 += 8) {
      if (j0 >= k) continue;
      u32x4_t o[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (j0 + jj < k) o[jj] = dxp[(size_t)rows[j0 + jj] * H8 + v];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj >= k) continue;
        float s = dot[j0 + jj];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          s = fmaf(bf16lo(xv[d]), bf16lo(o[jj][d]), s);
          s = fmaf(bf16hi(xv[d]), bf16hi(o[jj][d]), s);
        }
        dot[j0 + jj] = s;
      }
    }
  }
  router_score_bwd<KM>(dot, t, E, k, score, scaling, p, ids, red, dl_s, dl_row, logits, nullptr,
                       d_logits, dls, mp);
  // the router's dx term over the experts with a nonzero d_logits (the kept ones, or every
  // expert for softmax before the top-k without renormalisation)
  const int nnz = compact_nonzero(dl_row, E, nz_e, nz_v, wcount);
  for (int v = tid; v < H8; v += 256) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // rows 8 at a time, requested before any is added; the sums keep slot order, then
    // ascending expert id
    for (int j0 = 0; j0 < k; j0 += 8) {
      u32x4_t o[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (j0 + jj < k) o[jj] = dxp[(size_t)rows[j0 + jj] * H8 + v];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj >= k) break;
        const float q = ACT ? 1.f : p[j0 + jj];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc[2 * d] = fmaf(q, bf16lo(o[jj][d]), acc[2 * d]);
          acc[2 * d + 1] = fmaf(q, bf16hi(o[jj][d]), acc[2 * d + 1]);
        }
      }
    }
    for (int j0 = 0; j0 < nnz; j0 += 8) {
      u32x4_t wv[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (j0 + jj < nnz) wv[jj] = w_router[(size_t)nz_e[j0 + jj] * H8 + v];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj >= nnz) break;
        const float g = nz_v[j0 + jj];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc[2 * d] = fmaf(g, bf16lo(wv[jj][d]), acc[2 * d]);
          acc[2 * d + 1] = fmaf(g, bf16hi(wv[jj][d]), acc[2 * d + 1]);
        }
      }
    }
    u32x4_t ov;
#pragma unroll
    for (int d = 0; d < 4; ++d) ov[d] = pack_bf16x2(acc[2 * d], acc[2 * d + 1]);
    dx[(size_t)t * H8 + v] = ov;
  }
}

hipError_t launch_dispatch_bwd_router_input(const void* dxp, const void* x, const int32_t* row_of,
                                            const int32_t* topk_idx, const float* prob,
                                            const float* logits, const void* w_router, int T,
                                            int H, int E, int k, int score, float scaling,
                                            void* dx, float* d_logits, uint16_t* dls, int mp,
                                            hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (k <= 8)
    dispatch_bwd_router_input_kernel<8, false><<<T, 256, 0, s>>>(
        (const u32x4_t*)dxp, (const u32x4_t*)x, nullptr, 0, row_of, topk_idx, prob, logits,
        (const u32x4_t*)w_router, H / 8, E, k, score, scaling, (u32x4_t*)dx, d_logits, dls, mp);
  else
    dispatch_bwd_router_input_kernel<32, false><<<T, 256, 0, s>>>(
        (const u32x4_t*)dxp, (const u32x4_t*)x, nullptr, 0, row_of, topk_idx, prob, logits,
        (const u32x4_t*)w_router, H / 8, E, k, score, scaling, (u32x4_t*)dx, d_logits, dls, mp);
  return hipGetLastError();
}

hipError_t launch_dispatch_bwd_router_act(const void* dxp, const float* row_part, int P,
                                          const int32_t* row_of, const int32_t* topk_idx,
                                          const float* prob, const float* logits,
                                          const void* w_router, int T, int H, int E, int k,
                                          int score, float scaling, void* dx, float* d_logits,
                                          uint16_t* dls, int mp, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (k <= 8)
    dispatch_bwd_router_input_kernel<8, true><<<T, 256, 0, s>>>(
        (const u32x4_t*)dxp, nullptr, row_part, P, row_of, topk_idx, prob, logits,
        (const u32x4_t*)w_router, H / 8, E, k, score, scaling, (u32x4_t*)dx, d_logits, dls, mp);
  else
    dispatch_bwd_router_input_kernel<32, true><<<T, 256, 0, s>>>(
        (const u32x4_t*)dxp, nullptr, row_part, P, row_of, topk_idx, prob, logits,
        (const u32x4_t*)w_router, H / 8, E, k, score, scaling, (u32x4_t*)dx, d_logits, dls, mp);
  return hipGetLastError();
}

hipError_t launch_combine_bwd_router(const void* dy, const void* out, const int32_t* row_of,
                                     const int32_t* topk_idx, const float* prob,
                                     const float* logits, int T, int H, int E, int k, int score,
                                     float scaling, void* d_out, float* d_prob, float* d_logits,
                                     uint16_t* dls, int mp, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (k <= 8)
    combine_bwd_router_kernel<8><<<T, 256, 0, s>>>((const u32x4_t*)dy, (const u32x4_t*)out, row_of,
                                                   topk_idx, prob, logits, H / 8, E, k, score,
                                                   scaling, (u32x4_t*)d_out, d_prob, d_logits,
                                                   dls, mp);
  else
    combine_bwd_router_kernel<32><<<T, 256, 0, s>>>((const u32x4_t*)dy, (const u32x4_t*)out, row_of,
                                                    topk_idx, prob, logits, H / 8, E, k, score,
                                                    scaling, (u32x4_t*)d_out, d_prob, d_logits,
                                                    dls, mp);
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
  // eight splits' partials requested before any is added; the sum keeps split order
  for (int s0 = 0; s0 < S; s0 += 8) {
    f32x4_t a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) {
        a[j] = part[((size_t)(s0 + j) * mp + e) * H4 + c];
        b[j] = part[((size_t)(s0 + j) * mp + E + e) * H4 + c];
      }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) acc += a[j] + b[j];
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
