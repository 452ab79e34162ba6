// Token dispatch and combine (HBM-bound side of the path).
//
// Transformer Engine guide "Mixture of Experts", sections "Token dispatch" and "Token
// combine": dispatch lays the routed (token, choice) pairs out expert-contiguously,
// combine returns the expert outputs to token order and merges a token's k
// contributions with the routing weights in the same pass.
//
// Dispatch metadata is a stable counting sort of the flattened [T,k] choices by expert:
//   1. per-chunk histograms over experts: dispatch_hist (chunks of 1024 entries, LDS
//      atomics) for a given topk_idx, or written by the router itself inside the layer
//      (chunks of whole tokens, see router.hip);
//   2. dispatch_scan  : one block; per-expert totals (the counts), offsets[e] = their
//                       exclusive scan, and each chunk's starting row per expert;
//   3. dispatch_rank  : one wave per chunk walks its entries in order; lanes that chose
//                       the same expert find each other with 9 ballots (one per bit of the
//                       id), so a row is chunk_base + rank among the earlier lanes.
// No atomics decide any order, so the layout is deterministic and matches a stable sort.
// Row copies read each token row once and write its k destination rows with 16-byte
// vector accesses (scatter form: x is read exactly once).
#include "internal.h"

namespace moe {

int router_chunk_tokens(int T) {
  // whole-token chunks for the fused router histogram: at most 512 chunks, a multiple of
  // 32 tokens (one router block step)
  int c = (T + 511) / 512;
  return (c + 31) / 32 * 32;
}

size_t permute_scratch_bytes(int T, int E, int k) {
  const size_t n = (size_t)T * k;
  const size_t a = (n + kPermChunk - 1) / kPermChunk;
  const int ct = router_chunk_tokens(T);
  const size_t b = ((size_t)T + ct - 1) / ct;
  // per-chunk histograms and row bases, then the per-expert counts of a padded dispatch
  return (2 * (a > b ? a : b) + 1) * (size_t)E * sizeof(int32_t);
}

__global__ __launch_bounds__(256) void dispatch_hist_kernel(const int32_t* __restrict__ idx, int n,
                                                            int E, int32_t* __restrict__ partial) {
  __shared__ int h[256];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kPermChunk;
  for (int i = threadIdx.x; i < kPermChunk; i += 256) {
    int f = base + i;
    if (f < n) atomicAdd(&h[idx[f]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) partial[(size_t)blockIdx.x * E + e] = h[e];
}

// One block of 1024 threads: thread (part, e), e < EP (E rounded up to 64, 128 or 256),
// part < 1024/EP, owns a contiguous run of the chunks of expert e. It loads its run in
// batches of SCAN_BATCH independent loads (kept in registers when the run fits one batch),
// sums them; totals -> counts and offsets (exclusive scan over e); then each thread writes
// the running row base of its chunks.
constexpr int SCAN_BATCH = 64;
// align > 1 (padded dispatch, guide "Padding and alignment"): every expert block is
// rounded up to a multiple of align rows; offsets are the padded block starts and
// pad_offsets[e] (when given) the padding before block e.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ partial,
                                                             int nchunks, int E,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ chunk_base,
                                                             int align,
                                                             int32_t* __restrict__ pad_offsets) {
  __shared__ int psum[1024];
  __shared__ int s[256];
  const int EP = E <= 64 ? 64 : (E <= 128 ? 128 : 256);
  const int P = 1024 / EP;
  const int e = threadIdx.x % EP, part = threadIdx.x / EP;
  const int L = (nchunks + P - 1) / P;
  const int c0 = part * L, c1 = min(nchunks, c0 + L);
  int v[SCAN_BATCH];
  int sum = 0;
  if (e < E) {
    for (int b = c0; b < c1; b += SCAN_BATCH) {
#pragma unroll
      for (int i = 0; i < SCAN_BATCH; ++i) v[i] = b + i < c1 ? partial[(size_t)(b + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < SCAN_BATCH; ++i) sum += v[i];
    }
  }
  psum[threadIdx.x] = sum;
  __syncthreads();
  int tot = 0, before = 0;
  for (int q = 0; q < P; ++q) {
    const int x = psum[q * EP + e];
    tot += x;
    if (q < part) before += x;
  }
  // inclusive scan over e of the (padded) block sizes: within each wave by shuffles, then
  // the wave totals (at most four waves: EP <= 256) added from LDS
  __shared__ int wtot[4];
  const int ptot = align > 1 ? (tot + align - 1) / align * align : tot;
  auto scan = [&](int val) -> int {  // returns the inclusive scan, s[] holds it for every e
    int incl = e < E ? val : 0;
    if (part == 0) {
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if ((e & 63) >= o) incl += y;
      }
      if ((e & 63) == 63) wtot[e >> 6] = incl;
    }
    __syncthreads();
    if (part == 0) {
      for (int q = 0; q < (e >> 6); ++q) incl += wtot[q];
      s[e] = incl;
    }
    __syncthreads();
    return s[e];
  };
  if (pad_offsets) {
    const int pincl = scan(ptot - tot);
    if (part == 0 && e < E) pad_offsets[e] = pincl - (ptot - tot);
    __syncthreads();
  }
  const int excl = scan(ptot) - ptot;
  if (part == 0 && e < E) {
    offsets[e] = excl;
    if (counts) counts[e] = tot;
  }
  if ((int)threadIdx.x == EP - 1) offsets[E] = s[EP - 1];
  if (e < E) {
    int run = excl + before;
    if (c1 - c0 <= SCAN_BATCH) {  // the run is still in registers
#pragma unroll
      for (int i = 0; i < SCAN_BATCH; ++i)
        if (c0 + i < c1) {
          chunk_base[(size_t)(c0 + i) * E + e] = run;
          run += v[i];
        }
    } else {
      for (int c = c0; c < c1; ++c) {
        chunk_base[(size_t)c * E + e] = run;
        run += partial[(size_t)c * E + e];
      }
    }
  }
}

__global__ __launch_bounds__(64) void dispatch_rank_kernel(const int32_t* __restrict__ idx, int n,
                                                           int k, int E, int chunk_entries,
                                                           const int32_t* __restrict__ chunk_base,
                                                           int32_t* __restrict__ row_of,
                                                           int32_t* __restrict__ src_of) {
  __shared__ int base[256];
  const int lane = threadIdx.x;
  const int c = blockIdx.x;
  for (int e = lane; e < E; e += 64) base[e] = chunk_base[(size_t)c * E + e];
  __syncthreads();
  const uint64_t lt = lanemask_lt();
  const int iters = (chunk_entries + 63) / 64;
  for (int it = 0; it < iters; ++it) {
    const int off = it * 64 + lane;
    const int f = c * chunk_entries + off;
    const bool valid = off < chunk_entries && f < n;
    const int e = valid ? idx[f] : 0x1ff;  // 9-bit sentinel never equals a real id (< 256)
    uint64_t peers = ~0ull;
#pragma unroll
    for (int b = 0; b < 9; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt);
    if (valid) {
      const int r = base[e] + rank;
      row_of[f] = r;
      src_of[r] = f / k;
    }
    __syncthreads();
    if (valid && (peers >> lane) == 1ull) base[e] += __popcll(peers);  // last lane of the group
    __syncthreads();
  }
}

hipError_t launch_dispatch_meta(const int32_t* topk_idx, int T, int E, int k, int32_t* offsets,
                                int32_t* row_of, int32_t* src_of, void* scratch, hipStream_t s,
                                int align, int32_t* pad_offsets, int32_t* counts) {
  const int n = T * k;
  const int nchunks = (n + kPermChunk - 1) / kPermChunk;
  int32_t* partial = (int32_t*)scratch;
  int32_t* chunk_base = partial + (size_t)nchunks * E;
  if (n == 0) {
    hipError_t e = pad_offsets ? launch_fill_i32(pad_offsets, E, 0, s) : hipSuccess;
    if (e == hipSuccess && counts) e = launch_fill_i32(counts, E, 0, s);
    return e == hipSuccess ? launch_fill_i32(offsets, E + 1, 0, s) : e;
  }
  dispatch_hist_kernel<<<nchunks, 256, 0, s>>>(topk_idx, n, E, partial);
  dispatch_scan_kernel<<<1, 1024, 0, s>>>(partial, nchunks, E, counts, offsets, chunk_base, align,
                                          pad_offsets);
  dispatch_rank_kernel<<<nchunks, 64, 0, s>>>(topk_idx, n, k, E, kPermChunk, chunk_base, row_of,
                                              src_of);
  return hipGetLastError();
}

hipError_t launch_dispatch_from_hist(const int32_t* topk_idx, int T, int E, int k, int chunk_tokens,
                                     int32_t* partial, int32_t* counts, int32_t* offsets,
                                     int32_t* row_of, int32_t* src_of, hipStream_t s, int align,
                                     int32_t* pad_offsets) {
  const int n = T * k;
  if (n == 0) {
    hipError_t e = pad_offsets ? launch_fill_i32(pad_offsets, E, 0, s) : hipSuccess;
    return e == hipSuccess ? launch_fill_i32(offsets, E + 1, 0, s) : e;
  }
  const int nchunks = (T + chunk_tokens - 1) / chunk_tokens;
  int32_t* chunk_base = partial + (size_t)nchunks * E;
  dispatch_scan_kernel<<<1, 1024, 0, s>>>(partial, nchunks, E, counts, offsets, chunk_base, align,
                                          pad_offsets);
  dispatch_rank_kernel<<<nchunks, 64, 0, s>>>(topk_idx, n, k, E, chunk_tokens * k, chunk_base,
                                              row_of, src_of);
  return hipGetLastError();
}

// ---- row movement ----------------------------------------------------------

// xp[row_of[t,j]] = x[t] (prob == NULL), or bf16(prob[t,j] * x[t]) (combine backward).
__global__ __launch_bounds__(256) void scatter_rows_kernel(const u32x4_t* __restrict__ x,
                                                           const int32_t* __restrict__ row_of,
                                                           const float* __restrict__ prob, int H8,
                                                           int k, u32x4_t* __restrict__ xp) {
  __shared__ int rows[32];
  __shared__ float p[32];
  const int t = blockIdx.x;
  if ((int)threadIdx.x < k) {
    rows[threadIdx.x] = row_of[(size_t)t * k + threadIdx.x];
    p[threadIdx.x] = prob ? prob[(size_t)t * k + threadIdx.x] : 1.f;
  }
  __syncthreads();
  for (int v = threadIdx.x; v < H8; v += blockDim.x) {
    const u32x4_t val = x[(size_t)t * H8 + v];
    for (int j = 0; j < k; ++j) {
      u32x4_t o = val;
      if (prob) {
        const float q = p[j];
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(q * bf16lo(val[d]), q * bf16hi(val[d]));
      }
      __builtin_nontemporal_store(o, &xp[(size_t)rows[j] * H8 + v]);
    }
  }
}

hipError_t launch_scatter_rows(const void* x, const int32_t* row_of, const float* prob, int T,
                               int H, int k, void* xp, hipStream_t s) {
  if (T == 0) return hipSuccess;
  scatter_rows_kernel<<<T, 256, 0, s>>>((const u32x4_t*)x, row_of, prob, H / 8, k, (u32x4_t*)xp);
  return hipGetLastError();
}

// Padding rows of a padded dispatch (guide, "Padding and alignment"): block e's rows
// [offsets[e] + counts[e], offsets[e+1]) get zeros (row16 16-byte words each), scale 1
// (fp8) and src_of -1. One block per expert.
__global__ __launch_bounds__(256) void zero_pad_rows_kernel(const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ counts,
                                                            int row16, u32x4_t* __restrict__ rows,
                                                            float* __restrict__ scale,
                                                            int32_t* __restrict__ src_of) {
  const int e = blockIdx.x;
  const int r0 = offsets[e] + counts[e], r1 = offsets[e + 1];
  const size_t n = (size_t)(r1 - r0) * row16;
  const u32x4_t z = {0u, 0u, 0u, 0u};
  if (rows)
    for (size_t i = threadIdx.x; i < n; i += 256) rows[(size_t)r0 * row16 + i] = z;
  for (int r = r0 + (int)threadIdx.x; r < r1; r += 256) {
    if (scale) scale[r] = 1.f;
    if (src_of) src_of[r] = -1;
  }
}

hipError_t launch_zero_pad_rows(const int32_t* offsets, const int32_t* counts, int E,
                                int row_bytes, void* rows, float* scale, int32_t* src_of,
                                hipStream_t s) {
  zero_pad_rows_kernel<<<E, 256, 0, s>>>(offsets, counts, row_bytes / 16, (u32x4_t*)rows, scale,
                                         src_of);
  return hipGetLastError();
}

MOE_DEV float block_max_256(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// Row-wise e4m3 quantisation helper: 8 bf16 values -> 8 codes (two u32 words).
MOE_DEV u32x2_t quant8(const u32x4_t val, float s) {
  u32x2_t o;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    o[d] = pack_e4m3x4(bf16lo(val[2 * d]) / s, bf16hi(val[2 * d]) / s, bf16lo(val[2 * d + 1]) / s,
                       bf16hi(val[2 * d + 1]) / s);
  }
  return o;
}

MOE_DEV float amax8(const u32x4_t val) {
  float a = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) a = fmaxf(a, fmaxf(fabsf(bf16lo(val[d])), fabsf(bf16hi(val[d]))));
  return a;
}

// Dispatch with dynamic per-token e4m3 quantisation: scale = amax/448 (1 for a zero row).
__global__ __launch_bounds__(256) void scatter_rows_fp8_kernel(const u32x4_t* __restrict__ x,
                                                               const int32_t* __restrict__ row_of,
                                                               int H8, int k,
                                                               u32x2_t* __restrict__ xq,
                                                               float* __restrict__ xscale) {
  __shared__ int rows[32];
  __shared__ float red[8];
  const int t = blockIdx.x;
  if ((int)threadIdx.x < k) rows[threadIdx.x] = row_of[(size_t)t * k + threadIdx.x];
  float a = 0.f;
  for (int v = threadIdx.x; v < H8; v += blockDim.x) a = fmaxf(a, amax8(x[(size_t)t * H8 + v]));
  a = block_max_256(a, red);
  const float sc = a == 0.f ? 1.f : a / 448.0f;
  for (int v = threadIdx.x; v < H8; v += blockDim.x) {
    const u32x2_t q = quant8(x[(size_t)t * H8 + v], sc);
    for (int j = 0; j < k; ++j) xq[(size_t)rows[j] * H8 + v] = q;
  }
  if ((int)threadIdx.x < k) xscale[rows[threadIdx.x]] = sc;
}

hipError_t launch_scatter_rows_fp8(const void* x, const int32_t* row_of, int T, int H, int k,
                                   uint8_t* xq, float* xscale, hipStream_t s) {
  if (T == 0) return hipSuccess;
  scatter_rows_fp8_kernel<<<T, 256, 0, s>>>((const u32x4_t*)x, row_of, H / 8, k, (u32x2_t*)xq,
                                            xscale);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void quantize_rows_kernel(const u32x4_t* __restrict__ x, int C8,
                                                            u32x2_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  __shared__ float red[8];
  const size_t r = blockIdx.x;
  float a = 0.f;
  for (int v = threadIdx.x; v < C8; v += blockDim.x) a = fmaxf(a, amax8(x[r * C8 + v]));
  a = block_max_256(a, red);
  const float sc = a == 0.f ? 1.f : a / 448.0f;
  for (int v = threadIdx.x; v < C8; v += blockDim.x) q[r * C8 + v] = quant8(x[r * C8 + v], sc);
  if (threadIdx.x == 0) scale[r] = sc;
}

// One wave per P rows (4P rows per block) for rows of at most 512 vectors of 8 values: the
// rows are loaded once into registers (V vectors per lane and row, all requested before any
// is used), each row's amax reduced within the wave, and the codes written from the
// registers. Same scale and codes as the block kernel.
template <int V, int P>
__global__ __launch_bounds__(256) void quantize_rows_wave_kernel(const u32x4_t* __restrict__ x, int R,
                                                                 int C8, u32x2_t* __restrict__ q,
                                                                 float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * P;
  if (r0 >= R) return;  // the whole wave
  u32x4_t v[P][V];
#pragma unroll
  for (int j = 0; j < P; ++j)
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int c = lane + 64 * i;
      if (r0 + j < R && c < C8) v[j][i] = x[(size_t)(r0 + j) * C8 + c];
    }
#pragma unroll
  for (int j = 0; j < P; ++j) {
    if (r0 + j >= R) break;
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (lane + 64 * i < C8) a = fmaxf(a, amax8(v[j][i]));
    a = wave_max(a);
    const float sc = a == 0.f ? 1.f : a / 448.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int c = lane + 64 * i;
      if (c < C8) q[(size_t)(r0 + j) * C8 + c] = quant8(v[j][i], sc);
    }
    if (lane == 0) scale[r0 + j] = sc;
  }
}

hipError_t launch_quantize_rows(const void* x, int R, int C, uint8_t* q, float* scale,
                                hipStream_t s) {
  if (R == 0) return hipSuccess;
  const int C8 = C / 8;
  constexpr int P = 1;  // rows per wave (2 and 4 measured no faster)
  const int blocks = (R + 4 * P - 1) / (4 * P);
  const auto xx = (const u32x4_t*)x;
  const auto qq = (u32x2_t*)q;
  if (C8 <= 64) quantize_rows_wave_kernel<1, P><<<blocks, 256, 0, s>>>(xx, R, C8, qq, scale);
  else if (C8 <= 128) quantize_rows_wave_kernel<2, P><<<blocks, 256, 0, s>>>(xx, R, C8, qq, scale);
  else if (C8 <= 256) quantize_rows_wave_kernel<4, P><<<blocks, 256, 0, s>>>(xx, R, C8, qq, scale);
  else if (C8 <= 512) quantize_rows_wave_kernel<8, P><<<blocks, 256, 0, s>>>(xx, R, C8, qq, scale);
  else quantize_rows_kernel<<<R, 256, 0, s>>>((const u32x4_t*)x, C8, (u32x2_t*)q, scale);
  return hipGetLastError();
}

// Per-output-channel weight quantisation w[g][K][N] -> q[g][N][K], scale[g][N].
// One block per (g, 64 columns): a column-amax pass, then 64x64 tiles transposed
// through LDS so both the reads and the code writes are coalesced.
__global__ __launch_bounds__(256) void quantize_weights_kernel(const uint16_t* __restrict__ w, int K,
                                                               int N, uint8_t* __restrict__ q,
                                                               float* __restrict__ scale) {
  __shared__ float part[4][64];
  __shared__ float sc[64];
  __shared__ float tile[64][65];
  const int g = blockIdx.y;
  const int n0 = blockIdx.x * 64;
  const uint16_t* wg = w + (size_t)g * K * N;
  const int c = threadIdx.x & 63, r4 = threadIdx.x >> 6;
  float a = 0.f;
  if (n0 + c < N)
    for (int kk = r4; kk < K; kk += 4) a = fmaxf(a, fabsf(bf16_to_f32(wg[(size_t)kk * N + n0 + c])));
  part[r4][c] = a;
  __syncthreads();
  if (threadIdx.x < 64) {
    float m = fmaxf(fmaxf(part[0][c], part[1][c]), fmaxf(part[2][c], part[3][c]));
    float s = m == 0.f ? 1.f : m / 448.0f;
    sc[c] = s;
    if (n0 + c < N) scale[(size_t)g * N + n0 + c] = s;
  }
  __syncthreads();
  uint8_t* qg = q + (size_t)g * N * K;
  for (int k0 = 0; k0 < K; k0 += 64) {
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
      int kk = i / 64, cc = i % 64;
      tile[kk][cc] = (k0 + kk < K && n0 + cc < N) ? bf16_to_f32(wg[(size_t)(k0 + kk) * N + n0 + cc]) : 0.f;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
      int cc = i / 64, kk = i % 64;
      if (k0 + kk < K && n0 + cc < N)
        qg[(size_t)(n0 + cc) * K + k0 + kk] = (uint8_t)f32_to_e4m3(tile[kk][cc] / sc[cc]);
    }
    __syncthreads();
  }
}

hipError_t launch_quantize_weights(const void* w, int G, int K, int N, uint8_t* q, float* scale,
                                   hipStream_t s) {
  if (G == 0 || N == 0) return hipSuccess;
  dim3 grid((N + 63) / 64, G);
  quantize_weights_kernel<<<grid, 256, 0, s>>>((const uint16_t*)w, K, N, q, scale);
  return hipGetLastError();
}

// y[t] = sum_j p[t,j] * y_perm[row_of[t,j]] (+ shared[t]); fp32 sum in slot order, one
// rounding to bf16. prob == NULL gives the unweighted sum used by the dispatch backward.
// ROUTER (dispatch backward of a layer that owns its router projection): the router's dx
// term sum_j d_logits[t, e_j] * W_r[e_j] over the kept experts e_j is added after the k
// rows, before the rounding (the other experts' d_logits are 0).
template <bool ROUTER>
__global__ __launch_bounds__(256) void combine_kernel(const u32x4_t* __restrict__ yp,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ prob,
                                                      const u32x4_t* __restrict__ shared, int H8,
                                                      int k, u32x4_t* __restrict__ y,
                                                      const int32_t* __restrict__ topk_idx = nullptr,
                                                      const float* __restrict__ d_logits = nullptr,
                                                      const u32x4_t* __restrict__ w_router = nullptr,
                                                      int E = 0) {
  __shared__ int rows[32], ids[32];
  __shared__ float p[32], dl[32];
  const int t = blockIdx.x;
  if ((int)threadIdx.x < k) {
    rows[threadIdx.x] = row_of[(size_t)t * k + threadIdx.x];
    p[threadIdx.x] = prob ? prob[(size_t)t * k + threadIdx.x] : 1.f;
    if constexpr (ROUTER) {
      const int e = topk_idx[(size_t)t * k + threadIdx.x];
      ids[threadIdx.x] = e;
      dl[threadIdx.x] = d_logits[(size_t)t * E + e];
    }
  }
  __syncthreads();
  for (int v = threadIdx.x; v < H8; v += blockDim.x) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // the k row pieces are requested 8 at a time before any is summed, so their latencies
    // overlap; the sum still runs in slot order
    for (int j0 = 0; j0 < k; j0 += 8) {
      u32x4_t val[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (j0 + jj < k) val[jj] = __builtin_nontemporal_load(&yp[(size_t)rows[j0 + jj] * H8 + v]);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj >= k) break;
        const float q = p[j0 + jj];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc[2 * d] = fmaf(q, bf16lo(val[jj][d]), acc[2 * d]);
          acc[2 * d + 1] = fmaf(q, bf16hi(val[jj][d]), acc[2 * d + 1]);
        }
      }
    }
    if constexpr (ROUTER) {
      for (int j = 0; j < k; ++j) {
        const u32x4_t wv = w_router[(size_t)ids[j] * H8 + v];
        const float g = dl[j];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc[2 * d] = fmaf(g, bf16lo(wv[d]), acc[2 * d]);
          acc[2 * d + 1] = fmaf(g, bf16hi(wv[d]), acc[2 * d + 1]);
        }
      }
    }
    if (shared) {
      const u32x4_t sv = shared[(size_t)t * H8 + v];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        acc[2 * d] += bf16lo(sv[d]);
        acc[2 * d + 1] += bf16hi(sv[d]);
      }
    }
    u32x4_t o;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(acc[2 * d], acc[2 * d + 1]);
    y[(size_t)t * H8 + v] = o;
  }
}

hipError_t launch_combine(const void* y_perm, const int32_t* row_of, const float* prob,
                          const void* shared, int T, int H, int k, void* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  combine_kernel<false><<<T, 256, 0, s>>>((const u32x4_t*)y_perm, row_of, prob,
                                          (const u32x4_t*)shared, H / 8, k, (u32x4_t*)y);
  return hipGetLastError();
}

hipError_t launch_dispatch_bwd_router(const void* dxp, const int32_t* row_of,
                                      const int32_t* topk_idx, const float* d_logits,
                                      const void* w_router, int T, int H, int E, int k, void* dx,
                                      hipStream_t s) {
  if (T == 0) return hipSuccess;
  combine_kernel<true><<<T, 256, 0, s>>>((const u32x4_t*)dxp, row_of, nullptr, nullptr, H / 8, k,
                                         (u32x4_t*)dx, topk_idx, d_logits,
                                         (const u32x4_t*)w_router, E);
  return hipGetLastError();
}

}  // namespace moe
