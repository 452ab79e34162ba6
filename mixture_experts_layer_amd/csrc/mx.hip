// MXFP8 recipe: e4m3 elements with one power-of-two (E8M0) scale per block of 32 along K.
//
// te_mixtral.py names the mxfp8 recipe (FP8GlobalStateManager.get_fp8_recipe().mxfp8());
// the conversion of a block follows the OCP Microscaling (MX) v1.0 format: X =
// 2^(floor(log2(amax)) - 8), 8 being the largest e4m3 exponent, clamped to [2^-127, 2^127]
// (an all-zero block takes 2^-127); codes = e4m3(v / X), nearest-even, saturating to
// +-448; the scale byte is log2(X) + 127.
//
// The grouped GEMM multiplies e4m3 tiles on the matrix cores with the block scales applied
// inside the instruction (v_mfma_scale_f32_32x32x64_f8f6f4: each lane hands the scale of
// one 32-element K block of its row, for both operands), so no per-element dequantisation
// runs.
// Layout: A [rows, K] codes with scales [rows, K/32]; B [G, N, K] codes (output-channel
// major) with scales [G, N, K/32].
//
// Tiles: BM rows x BN B rows per block (320 or 256 x 256, eight waves of 160 or 128 x 64 as
// 5 or 4 x 2 blocks of 32x32), K in steps of 64 bytes through a double-buffered LDS stage
// loaded by all threads (16-byte loads into registers, then LDS), the next stage's loads in
// flight during the multiply. SwiGLU: a block's first BN/2 B rows are gate columns and the last BN/2 the
// matching up columns, and a wave's B blocks pair a gate block with its up block, so
// h = silu(g) u is formed in registers. One block per tile; the grid covers an upper bound
// of the tile count and the extra blocks exit.
#include "internal.h"

namespace moe {

namespace {

// log2 of the block scale from the block's largest magnitude (fp32 bits; exact)
MOE_DEV int mx_scale_exp(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xff);
  if (e == 0) return -127;  // zero or fp32-subnormal: floor(log2) - 8 < -127
  const int se = e - 127 - 8;
  return se < -127 ? -127 : (se > 127 ? 127 : se);
}
MOE_DEV float exp2i(int n) { return __uint_as_float((uint32_t)(n + 127) << 23); }  // n in [-126, 127]

}  // namespace

// ---- quantisation -------------------------------------------------------------------------
// Rows: four threads per block of 32 (eight bf16 each); the block's amax by two shuffles.
__global__ __launch_bounds__(256) void mx_quantize_rows_kernel(const u32x4_t* __restrict__ x,
                                                               size_t n8, int C8,
                                                               uint32_t* __restrict__ q,
                                                               uint8_t* __restrict__ scale) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = i < n8;
  const u32x4_t v = live ? x[i] : u32x4_t{0u, 0u, 0u, 0u};
  float f[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f[2 * d] = bf16lo(v[d]);
    f[2 * d + 1] = bf16hi(v[d]);
  }
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(f[e]));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  const int se = mx_scale_exp(m);
  const float inv = exp2i(-se);
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = fminf(fmaxf(f[4 * h + e] * inv, -448.f), 448.f);
    w[h] = pack_e4m3x4(t[0], t[1], t[2], t[3]);
  }
  if (live) {
    q[2 * i] = w[0];
    q[2 * i + 1] = w[1];
    if ((i & 3) == 0) {
      const size_t r = i / C8, c = i % C8;  // C8 % 4 == 0: a block never straddles rows
      scale[r * (C8 / 4) + c / 4] = (uint8_t)(se + 127);
    }
  }
}

namespace {
// One 16-byte piece (8 bf16) of a 32-value block whose four pieces sit in four neighbouring
// lanes (all four lanes call this together): the block scale exponent and the 8 codes, as
// mx_quantize_rows_kernel forms them.
MOE_DEV void mx_quant8(const u32x4_t v, uint32_t (&w)[2], int& se) {
  float f[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f[2 * d] = bf16lo(v[d]);
    f[2 * d + 1] = bf16hi(v[d]);
  }
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(f[e]));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  se = mx_scale_exp(m);
  const float inv = exp2i(-se);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = fminf(fmaxf(f[4 * h + e] * inv, -448.f), 448.f);
    w[h] = pack_e4m3x4(t[0], t[1], t[2], t[3]);
  }
}
}  // namespace

// The dispatch copy fused with the MXFP8 row quantisation of its copies: each token's row
// is read once; each of its k copies (times prob[t,j] and rounded to bf16 when prob is
// given) goes to xp[row_of[t,j]] as bf16 and to q / scale as e4m3 codes and block scales,
// equal to what mx_quantize_rows_kernel makes of that xp row. TPB tokens per block.
template <int TPB>
__global__ __launch_bounds__(256) void scatter_rows_mx_kernel(const u32x4_t* __restrict__ x,
                                                              const int32_t* __restrict__ row_of,
                                                              const float* __restrict__ prob, int T,
                                                              int H8, int k, u32x4_t* __restrict__ xp,
                                                              uint32_t* __restrict__ q,
                                                              uint8_t* __restrict__ scale) {
  __shared__ int rows[TPB][32];
  __shared__ float pw[TPB][32];
  const int t0 = blockIdx.x * TPB;
  if ((int)threadIdx.x < TPB * k) {
    const int b = threadIdx.x / k, j = threadIdx.x - b * k, t = t0 + b;
    if (t < T) {
      rows[b][j] = row_of[(size_t)t * k + j];
      pw[b][j] = prob ? prob[(size_t)t * k + j] : 1.f;
    }
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < TPB; ++b) {
    const int t = t0 + b;
    if (t >= T) break;
    // every lane of a 32-value block (four neighbouring lanes) runs the same iterations
    for (int v = threadIdx.x; v < H8; v += blockDim.x) {
      const u32x4_t val = x[(size_t)t * H8 + v];
      uint32_t w[2];
      int se = 0;
      if (!prob) mx_quant8(val, w, se);
      for (int j = 0; j < k; ++j) {
        const size_t r = (size_t)rows[b][j];
        u32x4_t o = val;
        if (prob) {
          const float g = pw[b][j];
#pragma unroll
          for (int d = 0; d < 4; ++d) o[d] = pack_bf16x2(g * bf16lo(val[d]), g * bf16hi(val[d]));
          mx_quant8(o, w, se);
        }
        __builtin_nontemporal_store(o, &xp[r * H8 + v]);
        *(u32x2_t*)&q[(r * H8 + v) * 2] = u32x2_t{w[0], w[1]};
        if ((v & 3) == 0) scale[r * (H8 / 4) + v / 4] = (uint8_t)(se + 127);
      }
    }
  }
}

hipError_t launch_scatter_rows_mx(const void* x, const int32_t* row_of, const float* prob, int T,
                                  int H, int k, void* xp, uint8_t* q, uint8_t* scale, hipStream_t s) {
  if (T == 0) return hipSuccess;
  constexpr int TPB = 2;
  scatter_rows_mx_kernel<TPB><<<(T + TPB - 1) / TPB, 256, 0, s>>>(
      (const u32x4_t*)x, row_of, prob, T, H / 8, k, (u32x4_t*)xp, (uint32_t*)q, scale);
  return hipGetLastError();
}

hipError_t launch_mx_quantize_rows(const void* x, int R, int C, uint8_t* q, uint8_t* scale,
                                   hipStream_t s) {
  const size_t n8 = (size_t)R * C / 8;
  if (n8 == 0) return hipSuccess;
  mx_quantize_rows_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(
      (const u32x4_t*)x, n8, C / 8, (uint32_t*)q, scale);
  return hipGetLastError();
}

// Weights w [G, K, N] bf16 -> codes [G, N, K] and scales [G, N, K/32]: one thread per
// (g, n, 32-block of K); neighbouring threads take neighbouring n, so the strided reads of
// a K block are coalesced across the wave.
__global__ __launch_bounds__(256) void mx_quantize_weights_kernel(const uint16_t* __restrict__ w,
                                                                  int G, int K, int N,
                                                                  uint8_t* __restrict__ q,
                                                                  uint8_t* __restrict__ scale) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int KB = K / 32;
  if (i >= (size_t)G * KB * N) return;
  const int n = (int)(i % N);
  const size_t gk = i / N;
  const int kb = (int)(gk % KB), g = (int)(gk / KB);
  const uint16_t* src = w + ((size_t)g * K + (size_t)kb * 32) * N + n;
  float f[32];
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    f[e] = bf16_to_f32(src[(size_t)e * N]);
    m = fmaxf(m, fabsf(f[e]));
  }
  const int se = mx_scale_exp(m);
  const float inv = exp2i(-se);
  u32x4_t o[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float t[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = fminf(fmaxf(f[16 * h + 4 * d + e] * inv, -448.f), 448.f);
      o[h][d] = pack_e4m3x4(t[0], t[1], t[2], t[3]);
    }
  u32x4_t* dst = (u32x4_t*)(q + ((size_t)g * N + n) * K + (size_t)kb * 32);
  dst[0] = o[0];
  dst[1] = o[1];
  scale[((size_t)g * N + n) * KB + kb] = (uint8_t)(se + 127);
}

hipError_t launch_mx_quantize_weights(const void* w, int G, int K, int N, uint8_t* q,
                                      uint8_t* scale, hipStream_t s) {
  const size_t n = (size_t)G * (K / 32) * N;
  if (n == 0) return hipSuccess;
  mx_quantize_weights_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((const uint16_t*)w, G, K,
                                                                        N, q, scale);
  return hipGetLastError();
}

// ---- token-axis (transposed) quantisation for the weight gradients ---------------------------
// Expert e's rows [off[e], off[e+1]) go to columns [co[e], co[e] + roundup(n_e, 64)) of the
// transposed codes qt [C, Kp]: blocks of 32 start at the expert's first row and the rows past
// its end read as zero, so no block holds two experts' rows.
// One block of 256 threads: thread t sums the padded sizes of experts [t*per, (t+1)*per),
// a block-wide exclusive scan of those sums, then each thread writes its experts' starts.
__global__ __launch_bounds__(256) void mx_col_offsets_kernel(const int32_t* __restrict__ off,
                                                             int G, int32_t* __restrict__ co) {
  __shared__ int s_sum[256];
  const int t = threadIdx.x, per = (G + 255) / 256;
  const int g0 = min(G, t * per), g1 = min(G, g0 + per);
  auto padded = [&](int g) {
    return (off[g + 1] - off[g] + kMxColAlign - 1) / kMxColAlign * kMxColAlign;
  };
  int mine = 0;
  for (int g = g0; g < g1; ++g) mine += padded(g);
  s_sum[t] = mine;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {  // inclusive scan (Hillis-Steele)
    const int v = t >= d ? s_sum[t - d] : 0;
    __syncthreads();
    s_sum[t] += v;
    __syncthreads();
  }
  int acc = s_sum[t] - mine;
  for (int g = g0; g < g1; ++g) {
    co[g] = acc;
    acc += padded(g);
  }
  if (t == 255) co[G] = s_sum[255];
}

hipError_t launch_mx_col_offsets(const int32_t* offsets, int G, int32_t* col_offsets,
                                 hipStream_t s) {
  mx_col_offsets_kernel<<<1, 256, 0, s>>>(offsets, G, col_offsets);
  return hipGetLastError();
}

// One block per (64 token columns, 64 channels): a 64-column span lies inside one expert's
// range (every range is a multiple of 64 long). The bf16 rows are staged in LDS (rows of 66
// values, so the column reads below fall in distinct banks); thread t then takes channel
// t/4 and rows 16*(t%4) .. +16 (half a block: the block amax by one shuffle) and writes
// 16 code bytes, four threads covering one channel's 64 contiguous bytes.
constexpr int kColTile = 64, kColLd = 66;
__global__ __launch_bounds__(256) void mx_quantize_cols_kernel(
    const uint16_t* __restrict__ x, int R, int C, const int32_t* __restrict__ off,
    const int32_t* __restrict__ co, int G, int Kp, uint8_t* __restrict__ qt,
    uint8_t* __restrict__ st) {
  __shared__ uint16_t s_x[kColTile * kColLd];
  const int tid = threadIdx.x;
  // channel tiles vary fastest over the grid, so blocks that run together read neighbouring
  // 128-byte pieces of the same rows (measured 8-17 % faster than token tiles fastest)
  const int p0 = blockIdx.y * kColTile, c0 = blockIdx.x * kColTile;
  if (p0 >= co[G]) return;  // past the last expert's range (uniform per block)
  int lo = 0, hi = G - 1;   // the expert whose range holds p0: co[e] <= p0 < co[e+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (co[mid] <= p0) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int n_e = off[e + 1] - off[e];
  const int local0 = p0 - co[e];
  // stage: 64 rows x 64 channels, thread t loads 8 channels of rows t/8 and t/8 + 32
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = (tid >> 3) + 32 * h, c = (tid & 7) * 8;
    const int li = local0 + r;
    const long long src = (long long)off[e] + li;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (li < n_e && src < R && c0 + c < C) v = *(const u32x4_t*)(x + (size_t)src * C + c0 + c);
    uint32_t* d = (uint32_t*)&s_x[r * kColLd + c];
#pragma unroll
    for (int w = 0; w < 4; ++w) d[w] = v[w];
  }
  __syncthreads();
  const int ch = tid >> 2, q = tid & 3;
  if (c0 + ch >= C) return;  // no barrier follows
  float f[16];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f[i] = bf16_to_f32(s_x[(16 * q + i) * kColLd + ch]);
    m = fmaxf(m, fabsf(f[i]));
  }
  m = fmaxf(m, __shfl_xor(m, 1, 64));  // the other half of the 32-row block
  const int se = mx_scale_exp(m);
  const float inv = exp2i(-se);
  u32x4_t o;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = fminf(fmaxf(f[4 * d + i] * inv, -448.f), 448.f);
    o[d] = pack_e4m3x4(t[0], t[1], t[2], t[3]);
  }
  const size_t row = (size_t)(c0 + ch);
  *(u32x4_t*)(qt + row * Kp + p0 + 16 * q) = o;
  if ((q & 1) == 0) st[row * (Kp / 32) + p0 / 32 + q / 2] = (uint8_t)(se + 127);
}

hipError_t launch_mx_quantize_cols(const void* x, int R, int C, const int32_t* offsets,
                                   const int32_t* col_offsets, int G, int Kp, uint8_t* qt,
                                   uint8_t* st, hipStream_t s) {
  if (Kp == 0 || C == 0) return hipSuccess;
  const dim3 grid((unsigned)((C + kColTile - 1) / kColTile), (unsigned)(Kp / kColTile));
  mx_quantize_cols_kernel<<<grid, 256, 0, s>>>((const uint16_t*)x, R, C, offsets, col_offsets,
                                               G, Kp, qt, st);
  return hipGetLastError();
}

// ---- grouped GEMM ---------------------------------------------------------------------------
constexpr int kMxBK = 64;  // K bytes (e4m3 values) per stage: two scale blocks
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3), read off the hardware with a
// one-hot probe: lane l holds row l%32; its bytes 0-15 are k 16*(l/32) .. +16 (K block 0)
// and bytes 16-31 are k 32 + 16*(l/32) .. +16 (K block 1); the scale of block b of row r
// comes from lane r + 32*b (byte 0 of its scale register).
MOE_DEV int mx_lane_scale(uint16_t two_blocks, int kh) { return (two_blocks >> (8 * kh)) & 0xff; }

// Two ways of grouping: by rows (the forward and the data gradients: group g owns rows
// [off[g], off[g+1]) of A and its own B [N, K]) or by K (the weight gradients: A [M, K] and
// B [N, K] are shared, group g owns K columns [off[g], off[g+1]), a multiple of 64, and
// writes C[g] [M, N]).
struct MxArgs {
  const uint8_t* A;
  const uint8_t* sa;
  const uint8_t* B;
  const uint8_t* sb;
  const int32_t* offsets;
  int G, M, N, K, I;  // by rows: M unused; by K: K is the row length of A and B (Kp)
  uint16_t* C;
  const uint16_t* gu_in;  // SwiGLU backward: the saved g,u [rows, 2I]
  uint16_t* gu_out;       // SwiGLU forward: g,u [rows, 2I] (training) or null
};

// Tile BM x BN, WM x WN waves, each wave (BM/WM) x (BN/WN) outputs as 32x32 blocks. The LDS
// traffic per matrix instruction falls as the wave tile grows (a 128x64 wave tile reads six
// 2 KB fragments per eight instructions, a 64x64 one four per four), so the wide tiles run
// the long launches. SwiGLU: the tile's first BN/2 B rows are gate columns, the last BN/2
// the matching up columns, and a wave's N blocks are NB/2 gate blocks then their up blocks.
template <int EPI, bool KGRP, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64, 2) void mx_gemm_kernel(MxArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int MB = BM / WM / 32, NB = BN / WN / 32, NH = NB / 2, HB = BN / 2;
  // 16-byte chunks per thread (the last round partial when BM * 4 is not a multiple of NT)
  constexpr int A_PER = (BM * 4 + NT - 1) / NT, B_PER = (BN * 4 + NT - 1) / NT;
  static_assert(BN * 4 % NT == 0 && BM % 32 == 0, "load split");
  static_assert(EPI != EPI_SWIGLU || NB % 2 == 0, "SwiGLU pairs gate and up blocks");
  // Row-grouped: a ring of three stage buffers, stage kt+2 written while stage kt is
  // multiplied, into the buffer of stage kt-1, which every wave finished reading before the
  // last barrier (one barrier per K step). By K (4-5 K steps per tile): two buffers, the
  // next stage written between two barriers (measured faster there).
  constexpr int NSTG = KGRP ? 2 : 3;
  __shared__ __attribute__((aligned(16))) uint8_t s_a[NSTG][BM * kMxBK];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[NSTG][BN * kMxBK];
  __shared__ uint16_t s_sa[NSTG][BM], s_sb[NSTG][BN];  // two block scales per row per stage
  __shared__ int s_off[264], s_pref[264];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int K = p.K, I = p.I, N = p.N;
  const int KB = K / 32;
  // ---- tile decode (blocks in tile order: an XCD-contiguous remapping of the tiles measured
  // no faster, dW_down 7 % faster and dW_gu 5 % slower) ----
  int g, ntile, m0, rows_valid, k0, nk;
  if constexpr (KGRP) {
    const int mt = (p.M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
    const int tile = blockIdx.x;
    g = tile / (mt * ntn);
    const int local = tile - g * (mt * ntn);
    ntile = local / mt;
    m0 = (local % mt) * BM;
    rows_valid = min(BM, p.M - m0);
    k0 = min(p.offsets[g], K);  // clamped to the operands' row length
    nk = max(0, min(p.offsets[g + 1], K) - k0) / kMxBK;
  } else {
    // groups' M-tile prefix, then (group, n-tile, m-tile)
    const int ntn = EPI == EPI_SWIGLU ? (I + HB - 1) / HB : (N + BN - 1) / BN;
    for (int x = tid; x <= p.G; x += NT) s_off[x] = p.offsets[x];
    __syncthreads();
    if (wave == 0) {  // the prefix by one wave: up to five groups per lane, then a lane scan
      const int per = (p.G + 63) / 64;
      int loc[5];
      int sum = 0;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int x = lane * per + i;
        int mtx = 0;
        if (i < per && x < p.G) mtx = (s_off[x + 1] - s_off[x] + BM - 1) / BM;
        sum += mtx;
        loc[i] = sum;
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      if (lane == 0) s_pref[0] = 0;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int x = lane * per + i;
        if (i < per && x < p.G) s_pref[x + 1] = incl - sum + loc[i];
      }
    }
    __syncthreads();
    const int tile = blockIdx.x;
    if (tile >= s_pref[p.G] * ntn) return;
    {  // the tile's group: the last g with s_pref[g] * ntn <= tile (binary search)
      int lo = 0, hi = p.G;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pref[mid] * ntn <= tile) lo = mid;
        else hi = mid - 1;
      }
      g = lo;
    }
    const int local = tile - s_pref[g] * ntn;
    const int mt = s_pref[g + 1] - s_pref[g];
    ntile = local / mt;
    m0 = s_off[g] + (local % mt) * BM;
    rows_valid = min(BM, s_off[g + 1] - m0);
    k0 = 0;
    nk = K / kMxBK;
  }
  // ---- loaders: chunk c (of BM*4 for A, BN*4 for B) = row c/4, 16-byte piece c%4; thread t
  // takes chunks t, t + NT, ...; scales: thread t < BM takes A row t, then B rows ----
  auto brow_of = [&](int r) -> int {  // B row (output channel) of LDS B row r
    if constexpr (EPI == EPI_SWIGLU) {
      int hcol = ntile * HB + (r < HB ? r : r - HB);
      hcol = hcol < I ? hcol : ntile * HB;  // past I: outputs never stored
      return r < HB ? hcol : I + hcol;
    } else {
      const int c = ntile * BN + r;
      return c < N ? c : ntile * BN;
    }
  };
  const uint8_t* bg = KGRP ? p.B : p.B + (size_t)g * N * K;
  const uint8_t* sbg = KGRP ? p.sb : p.sb + (size_t)g * N * KB;
  const uint8_t* pa[A_PER];
  const uint8_t* pb[B_PER];
#pragma unroll
  for (int h = 0; h < A_PER; ++h) {
    const int c = tid + NT * h, r = c >> 2;  // c >= BM * 4: no chunk (pa unused)
    pa[h] = p.A + (size_t)(m0 + (r < rows_valid ? r : 0)) * K + k0 + (c & 3) * 16;  // dead rows: the first
  }
#pragma unroll
  for (int h = 0; h < B_PER; ++h) {
    const int c = tid + NT * h;
    pb[h] = bg + (size_t)brow_of(c >> 2) * K + k0 + (c & 3) * 16;
  }
  constexpr int SC_PER = (BM + BN + NT - 1) / NT;
  const uint8_t* psc[SC_PER];
#pragma unroll
  for (int h = 0; h < SC_PER; ++h) {
    const int r = tid + NT * h;
    if (r < BM) psc[h] = p.sa + (size_t)(m0 + (r < rows_valid ? r : 0)) * KB + k0 / 32;
    else if (r < BM + BN) psc[h] = sbg + (size_t)brow_of(r - BM) * KB + k0 / 32;
    else psc[h] = nullptr;
  }
  // LDS rows of 64 bytes, the 16-byte chunk index XORed with (row/4)%4 so the fragment
  // reads of 32 consecutive rows spread over the banks
  auto chunk_at = [](int row, int c) { return row * kMxBK + ((c ^ ((row >> 2) & 3)) << 4); };
  u32x4_t ra[A_PER], rb[B_PER];
  uint16_t rs[SC_PER];
  auto gload = [&](int kt) {
#pragma unroll
    for (int h = 0; h < A_PER; ++h)
      if (BM * 4 % NT == 0 || tid + NT * h < BM * 4) ra[h] = *(const u32x4_t*)(pa[h] + (size_t)kt * kMxBK);
#pragma unroll
    for (int h = 0; h < B_PER; ++h) rb[h] = *(const u32x4_t*)(pb[h] + (size_t)kt * kMxBK);
#pragma unroll
    for (int h = 0; h < SC_PER; ++h)
      if (psc[h]) rs[h] = (uint16_t)(psc[h][2 * kt] | (psc[h][2 * kt + 1] << 8));
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < A_PER; ++h) {
      const int c = tid + NT * h;
      if (BM * 4 % NT == 0 || c < BM * 4) *(u32x4_t*)&s_a[buf][chunk_at(c >> 2, c & 3)] = ra[h];
    }
#pragma unroll
    for (int h = 0; h < B_PER; ++h) {
      const int c = tid + NT * h;
      *(u32x4_t*)&s_b[buf][chunk_at(c >> 2, c & 3)] = rb[h];
    }
#pragma unroll
    for (int h = 0; h < SC_PER; ++h) {
      const int r = tid + NT * h;
      if (r < BM) s_sa[buf][r] = rs[h];
      else if (r < BM + BN) s_sb[buf][r - BM] = rs[h];
    }
  };
  // B row (within the tile) of N block j of this wave
  auto bcol0 = [&](int j) {
    if constexpr (EPI == EPI_SWIGLU) return j < NH ? (wn * NH + j) * 32 : HB + (wn * NH + j - NH) * 32;
    return (wn * NB + j) * 32;
  };
  f32x16_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int l32 = lane & 31, kh = lane >> 5;
  // M blocks of this wave holding a valid row (wave-uniform): the others skip the multiply
  const int mlive = __builtin_amdgcn_readfirstlane(
      min(MB, max(0, (rows_valid - wm * (BM / WM) + 31) / 32)));
  if (nk > 0) {  // uniform per block
    gload(0);
    lstore(0);
    if (NSTG == 3 && nk > 1) {
      gload(1);
      lstore(1);
    }
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt % NSTG;
    if (kt + NSTG - 1 < nk) gload(kt + NSTG - 1);
    i32x8_t bf[NB];
    int bs[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int r = bcol0(j) + l32;
      const u32x4_t lo = *(const u32x4_t*)&s_b[buf][chunk_at(r, kh)];
      const u32x4_t hi = *(const u32x4_t*)&s_b[buf][chunk_at(r, 2 + kh)];
      bf[j] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      bs[j] = mx_lane_scale(s_sb[buf][r], kh);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (i < mlive) {
        const int r = wm * (BM / WM) + 32 * i + l32;
        const u32x4_t lo = *(const u32x4_t*)&s_a[buf][chunk_at(r, kh)];
        const u32x4_t hi = *(const u32x4_t*)&s_a[buf][chunk_at(r, 2 + kh)];
        const i32x8_t af = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        const int as = mx_lane_scale(s_sa[buf][r], kh);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j], af, acc[i][j], 0, 0,
                                                                      0, bs[j], 0, as);
      }
    }
    if constexpr (NSTG == 3) {
      if (kt + 2 < nk) lstore((kt + 2) % 3);  // stage kt-1's buffer: read before the last barrier
      __syncthreads();  // stage kt+1 (written one step ago) is visible; stage kt is read
    } else {
      if (kt + 1 < nk) {
        __syncthreads();  // every wave is done with the other buffer (read two steps ago)
        lstore(buf ^ 1);
        __syncthreads();
      }
    }
  }
  // ---- epilogues: lane l holds row l%32 of its M block and, per j, columns
  // 8*(v/4) + 4*(l/32) + v%4 of its 32-column B block. Each goes through LDS areas of the
  // wave's own in a stage buffer no wave reads any more (three buffers: every K step ends
  // with a barrier, so buffer 0; two: the one the last K step did not use, which every wave
  // finished reading before the barrier that preceded the last stage's LDS writes, or never
  // written with a single K step), so that global memory sees row segments of 64 or 128
  // bytes ----
  constexpr int NA = BM * kMxBK / 4096;  // 4 KB areas in the A half of a stage buffer
  static_assert(NA + BN * kMxBK / 4096 >= WM * WN, "staging areas: one of 4 KB per wave");
  const int sb_ = NSTG == 3 ? 0 : (nk & 1);
  uint8_t* const stg = wave < NA ? s_a[sb_] + wave * 4096 : s_b[sb_] + (wave - NA) * 4096;
  // 32 rows of 64 bytes, 16-byte chunks XORed with (row/4)%4
  auto at = [](int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); };
  if constexpr (EPI == EPI_SWIGLU) {
    // per M block and gate block: h = silu(g) u (and, training, g and u) as bf16 32 x 32
    // tiles, written in the accumulator layout and read back as 16-byte row pieces
    uint8_t* const s0 = stg;
    uint8_t* const s1 = stg + 2048;
    auto put = [&](uint8_t* area, int q4, float a0, float a1, float a2, float a3) {
      *(u32x2_t*)(area + at(l32, q4) + 8 * kh) = u32x2_t{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
    };
    auto sync_wave = [&]() {
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
    };
    auto out = [&](const uint8_t* area, uint16_t* base, size_t ld, int r0, int col) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int pc = lane + 64 * h, rr = pc >> 2, ch = pc & 3;
        const u32x4_t v = *(const u32x4_t*)(area + at(rr, ch));
        if (r0 + rr < rows_valid) *(u32x4_t*)(base + ((size_t)m0 + r0 + rr) * ld + col + ch * 8) = v;
      }
    };
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int r0 = wm * (BM / WM) + 32 * i;
      if (r0 >= rows_valid) continue;  // wave-uniform
#pragma unroll
      for (int jj = 0; jj < NH; ++jj) {
        const int hc = ntile * HB + (wn * NH + jj) * 32;
        if (hc >= I) continue;  // I % 64 == 0: a 32-column block is wholly in or out
        const f32x16_t& ga = acc[i][jj];
        const f32x16_t& ua = acc[i][jj + NH];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gg = ga[4 * q4 + r], uu = ua[4 * q4 + r];
            hv[r] = gg * sigmoid_fast(gg) * uu;
          }
          put(s0, q4, hv[0], hv[1], hv[2], hv[3]);
          if (p.gu_out) put(s1, q4, ga[4 * q4], ga[4 * q4 + 1], ga[4 * q4 + 2], ga[4 * q4 + 3]);
        }
        sync_wave();
        out(s0, p.C, (size_t)I, r0, hc);
        if (p.gu_out) out(s1, p.gu_out, 2 * (size_t)I, r0, hc);
        sync_wave();
        if (p.gu_out) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) put(s0, q4, ua[4 * q4], ua[4 * q4 + 1], ua[4 * q4 + 2], ua[4 * q4 + 3]);
          sync_wave();
          out(s0, p.gu_out, 2 * (size_t)I, r0, I + hc);
          sync_wave();
        }
      }
    }
  }
  if constexpr (EPI == EPI_SWIGLU_BWD) {
    // acc = dh[row, c] (fp32), c < I; with s = sigmoid(g), from the saved bf16 g,u:
    // dgu[row] = [dh u s (1 + g (1 - s)), dh g s]. Per M block and 32-column N block, the
    // wave moves g,u in and dg,du out as 64-byte row segments through the two 2 KB halves
    // of its area, converting between them and the accumulator layout there.
    uint8_t* const sgv = stg;
    uint8_t* const suv = stg + 2048;
    const size_t twoI = 2 * (size_t)I;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int r0 = wm * (BM / WM) + 32 * i;
      if (r0 >= rows_valid) continue;  // wave-uniform
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int cb = ntile * BN + bcol0(j);  // 32 dh columns (I % 64 == 0: all or none)
        if (cb >= N) continue;
        // g, u in: piece p = lane + 64 h is row p/4, 16-byte chunk p%4
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int pc = lane + 64 * h, rr = pc >> 2, ch = pc & 3;
          u32x4_t gv = u32x4_t{0u, 0u, 0u, 0u}, uv = gv;
          if (r0 + rr < rows_valid) {
            const uint16_t* src = p.gu_in + ((size_t)m0 + r0 + rr) * twoI + cb + ch * 8;
            gv = *(const u32x4_t*)src;
            uv = *(const u32x4_t*)(src + I);
          }
          *(u32x4_t*)(sgv + at(rr, ch)) = gv;
          *(u32x4_t*)(suv + at(rr, ch)) = uv;
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        // accumulator layout: row l32, columns 8 q4 + 4 kh .. +4 (chunk q4, byte 8 kh)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2_t* gp = (u32x2_t*)(sgv + at(l32, q4) + 8 * kh);
          u32x2_t* up = (u32x2_t*)(suv + at(l32, q4) + 8 * kh);
          const u32x2_t gw = *gp, uw = *up;
          float dg[4], du[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gg = (e & 1) ? bf16hi(gw[e >> 1]) : bf16lo(gw[e >> 1]);
            const float uu = (e & 1) ? bf16hi(uw[e >> 1]) : bf16lo(uw[e >> 1]);
            const float dh = acc[i][j][4 * q4 + e];
            const float sg = sigmoid_fast(gg);
            dg[e] = dh * uu * sg * (1.0f + gg * (1.0f - sg));
            du[e] = dh * gg * sg;
          }
          *gp = u32x2_t{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
          *up = u32x2_t{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        // dg, du out
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int pc = lane + 64 * h, rr = pc >> 2, ch = pc & 3;
          const u32x4_t gv = *(const u32x4_t*)(sgv + at(rr, ch));
          const u32x4_t uv = *(const u32x4_t*)(suv + at(rr, ch));
          if (r0 + rr < rows_valid) {
            uint16_t* dst = p.C + ((size_t)m0 + r0 + rr) * twoI + cb + ch * 8;
            *(u32x4_t*)dst = gv;
            *(u32x4_t*)(dst + I) = uv;
          }
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
      }
    }
  }
  if constexpr (EPI == EPI_STORE) {
    // Whole 128-byte lines: per M block, the wave writes its 32 rows x 64 columns (bf16)
    // into its 4 KB area, the 16-byte chunk index XORed with row%8, and reads them back as
    // 16 consecutive bytes of one row per lane.
    static_assert(NB == 2, "a wave's 64 output columns");
    uint16_t* cg = KGRP ? p.C + (size_t)g * p.M * N : p.C;
    const int c0 = ntile * BN + bcol0(0);  // this wave's 64 columns (N % 64 == 0: all or none)
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int r0 = wm * (BM / WM) + 32 * i;
      if (r0 >= rows_valid || c0 >= N) continue;  // wave-uniform
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16_t& a = acc[i][j];
          const int chunk = 4 * j + q4;  // columns 32 j + 8 q4 .. +8: 16-byte chunk 4 j + q4
          *(u32x2_t*)(stg + l32 * 128 + ((chunk ^ (l32 & 7)) << 4) + 8 * kh) =
              u32x2_t{pack_bf16x2(a[4 * q4], a[4 * q4 + 1]), pack_bf16x2(a[4 * q4 + 2], a[4 * q4 + 3])};
        }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int r = pass * 8 + (lane >> 3), piece = lane & 7;
        const u32x4_t v = *(const u32x4_t*)(stg + r * 128 + ((piece ^ (r & 7)) << 4));
        if (r0 + r < rows_valid)
          *(u32x4_t*)(cg + ((size_t)m0 + r0 + r) * N + c0 + piece * 8) = v;
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
    }
  }
}

// Tile configurations (BM, BN, WM, WN): the SwiGLU forward and backward and the plain
// store by rows, and the weight gradients by K. Eight waves of 128x64 or 160x64 (measured on
// the Qwen3-shaped stages, one process per build: with exactly 256 rows per expert 1.59 ms
// for the six at 256x256 against 1.80 with 128x128 tiles of four 64x64 waves and 2.19 with
// 256x128 or 128x256 tiles of four waves; 4x2 waves the same as 2x4). With the routed
// (ragged) rows, 320-row tiles keep most experts to one M tile: the four row-grouped
// launches 0.89 ms against 1.12 with 256 rows.
#ifndef MOE_MX_TILE_ROWS
#define MOE_MX_TILE_ROWS 320, 256, 2, 4
#endif
#ifndef MOE_MX_TILE_SWIGLU
#define MOE_MX_TILE_SWIGLU 320, 256, 2, 4
#endif
#ifndef MOE_MX_TILE_SWIGLU_BWD
#define MOE_MX_TILE_SWIGLU_BWD 320, 256, 2, 4
#endif
#ifndef MOE_MX_TILE_WGRAD
#define MOE_MX_TILE_WGRAD 256, 256, 2, 4
#endif

namespace {
template <int EPI, bool KGRP, int BM, int BN, int WM, int WN>
hipError_t mx_launch(const MxArgs& a, int rows, hipStream_t s) {
  long long tiles;
  if (KGRP) tiles = (long long)a.G * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  else tiles = ((long long)rows / BM + a.G) *
               (EPI == EPI_SWIGLU ? (a.I + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN);
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  mx_gemm_kernel<EPI, KGRP, BM, BN, WM, WN><<<(unsigned)tiles, WM * WN * 64, 0, s>>>(a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_mx_gemm(int epi, const void* A, const uint8_t* sa, const void* B,
                          const uint8_t* sb, const int32_t* offsets, int G, int rows, int N,
                          int K, int I, void* C, hipStream_t s, const void* gu_in,
                          void* gu_out) {
  MxArgs a{(const uint8_t*)A, sa, (const uint8_t*)B, sb, offsets, G, 0, N, K, I, (uint16_t*)C,
           (const uint16_t*)gu_in, (uint16_t*)gu_out};
  if (epi == EPI_SWIGLU) return mx_launch<EPI_SWIGLU, false, MOE_MX_TILE_SWIGLU>(a, rows, s);
  if (epi == EPI_SWIGLU_BWD) return mx_launch<EPI_SWIGLU_BWD, false, MOE_MX_TILE_SWIGLU_BWD>(a, rows, s);
  return mx_launch<EPI_STORE, false, MOE_MX_TILE_ROWS>(a, rows, s);
}

hipError_t launch_mx_gemm_wgrad(const void* At, const uint8_t* sa, const void* Bt,
                                const uint8_t* sb, const int32_t* col_offsets, int G, int M,
                                int N, int Kp, void* C, hipStream_t s) {
  MxArgs a{(const uint8_t*)At, sa, (const uint8_t*)Bt, sb, col_offsets, G, M, N, Kp, 0,
           (uint16_t*)C, nullptr, nullptr};
  return mx_launch<EPI_STORE, true, MOE_MX_TILE_WGRAD>(a, 0, s);
}

}  // namespace moe
