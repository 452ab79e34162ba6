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
// Tiles: 128 rows x 128 B rows per block, four waves of 64 x 64 (2 x 2 blocks of 32x32),
// K in steps of 64 bytes through a double-buffered LDS stage loaded by all threads (16-byte
// loads into registers, then LDS), the next stage's loads in flight during the multiply.
// SwiGLU: a block's 128 B rows are 64 gate columns and the 64 matching up columns, and a
// wave's two B blocks are a gate block and its up block, so h = silu(g) u is formed in
// registers. One block per tile; the grid covers an upper bound of the tile count and the
// extra blocks exit.
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

// ---- grouped GEMM ---------------------------------------------------------------------------
constexpr int kMxBM = 128, kMxBN = 128, kMxBK = 64;
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3), read off the hardware with a
// one-hot probe: lane l holds row l%32; its bytes 0-15 are k 16*(l/32) .. +16 (K block 0)
// and bytes 16-31 are k 32 + 16*(l/32) .. +16 (K block 1); the scale of block b of row r
// comes from lane r + 32*b (byte 0 of its scale register).
MOE_DEV int mx_lane_scale(uint16_t two_blocks, int kh) { return (two_blocks >> (8 * kh)) & 0xff; }

template <int EPI>  // EPI_STORE (C bf16 [rows, N]) or EPI_SWIGLU (h bf16 [rows, I])
__global__ __launch_bounds__(256) void mx_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ sa, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ sb, const int32_t* __restrict__ offsets, int G, int N, int K,
    int I, uint16_t* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][kMxBM * kMxBK];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][kMxBN * kMxBK];
  __shared__ uint16_t s_sa[2][kMxBM], s_sb[2][kMxBN];  // two block scales per row per stage
  __shared__ int s_off[264], s_pref[264];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // ---- tile decode: groups' M-tile prefix, then (group, n-tile, m-tile) ----
  const int ntn = EPI == EPI_SWIGLU ? I / 64 : (N + kMxBN - 1) / kMxBN;
  for (int g = tid; g <= G; g += 256) s_off[g] = offsets[g];
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    s_pref[0] = 0;
    for (int g = 0; g < G; ++g) {
      acc += (s_off[g + 1] - s_off[g] + kMxBM - 1) / kMxBM;
      s_pref[g + 1] = acc;
    }
  }
  __syncthreads();
  const int tile = blockIdx.x;
  if (tile >= s_pref[G] * ntn) return;
  int g = 0;
  while (s_pref[g + 1] * ntn <= tile) ++g;
  const int local = tile - s_pref[g] * ntn;
  const int mt = s_pref[g + 1] - s_pref[g];
  const int ntile = local / mt, mtile = local % mt;
  const int m0 = s_off[g] + mtile * kMxBM;
  const int rows_valid = min(kMxBM, s_off[g + 1] - m0);
  const int KB = K / 32;
  // ---- loaders: thread t loads 16 bytes of two A rows and two B rows per stage ----
  // A row r = t / 4 (+64), 16-byte chunk t % 4; B rows likewise; scales: t < 128 -> A row
  // t, else B row t - 128 (two bytes: the stage's two 32-element blocks).
  auto brow_of = [&](int r) -> int {  // B row (output channel) of LDS B row r
    if constexpr (EPI == EPI_SWIGLU) {
      const int hcol = ntile * 64 + (r & 63);
      return r < 64 ? hcol : I + hcol;
    } else {
      const int c = ntile * kMxBN + r;
      return c < N ? c : ntile * kMxBN;
    }
  };
  const uint8_t* bg = B + (size_t)g * N * K;
  const uint8_t* sbg = sb + (size_t)g * N * KB;
  const int lr = tid >> 2, lc = (tid & 3) * 16;
  const uint8_t* pa[2];
  const uint8_t* pb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = lr + 64 * h;
    pa[h] = A + (size_t)(m0 + (r < rows_valid ? r : 0)) * K + lc;  // dead rows: the first
    pb[h] = bg + (size_t)brow_of(r) * K + lc;
  }
  const uint8_t* psc;
  if (tid < kMxBM) psc = sa + (size_t)(m0 + (tid < rows_valid ? tid : 0)) * KB;
  else psc = sbg + (size_t)brow_of(tid - kMxBM) * KB;
  // LDS rows of 64 bytes, the 16-byte chunk index XORed with (row/4)%4 so the fragment
  // reads of 32 consecutive rows spread over the banks
  auto chunk_at = [](int row, int c) { return row * kMxBK + ((c ^ ((row >> 2) & 3)) << 4); };
  u32x4_t ra[2], rb[2];
  uint16_t rs;
  auto gload = [&](int kt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ra[h] = *(const u32x4_t*)(pa[h] + (size_t)kt * kMxBK);
      rb[h] = *(const u32x4_t*)(pb[h] + (size_t)kt * kMxBK);
    }
    rs = (uint16_t)(psc[2 * kt] | (psc[2 * kt + 1] << 8));
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *(u32x4_t*)&s_a[buf][chunk_at(lr + 64 * h, lc >> 4)] = ra[h];
      *(u32x4_t*)&s_b[buf][chunk_at(lr + 64 * h, lc >> 4)] = rb[h];
    }
    if (tid < kMxBM) s_sa[buf][tid] = rs;
    else s_sb[buf][tid - kMxBM] = rs;
  };
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int l32 = lane & 31, kh = lane >> 5;
  const int nk = K / kMxBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    i32x8_t af[2], bf[2];
    int as[2], bs[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + 32 * i + l32;
      const u32x4_t lo = *(const u32x4_t*)&s_a[buf][chunk_at(r, kh)];
      const u32x4_t hi = *(const u32x4_t*)&s_a[buf][chunk_at(r, 2 + kh)];
      af[i] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      as[i] = mx_lane_scale(s_sa[buf][r], kh);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = EPI == EPI_SWIGLU ? 64 * j + 32 * wn + l32 : wn * 64 + 32 * j + l32;
      const u32x4_t lo = *(const u32x4_t*)&s_b[buf][chunk_at(r, kh)];
      const u32x4_t hi = *(const u32x4_t*)&s_b[buf][chunk_at(r, 2 + kh)];
      bf[j] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      bs[j] = mx_lane_scale(s_sb[buf][r], kh);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j], af[i], acc[i][j], 0, 0,
                                                                    0, bs[j], 0, as[i]);
    if (kt + 1 < nk) {
      __syncthreads();  // every wave is done with the other buffer (read two steps ago)
      lstore(buf ^ 1);
      __syncthreads();
    }
  }
  // ---- epilogue: lane l holds row l%32 of its M block and, per j, columns
  // 8*(v/4) + 4*(l/32) + v%4 of its 32-column B block ----
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rloc = wm * 64 + 32 * i + l32;
    if (rloc >= rows_valid) continue;
    const size_t row = (size_t)m0 + rloc;
    if constexpr (EPI == EPI_SWIGLU) {
      uint16_t* hr = C + row * I + ntile * 64 + 32 * wn;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gg = acc[i][0][4 * q4 + r], uu = acc[i][1][4 * q4 + r];
          hv[r] = gg * sigmoid_fast(gg) * uu;
        }
        *(u32x2_t*)(hr + 8 * q4 + 4 * kh) = u32x2_t{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c0 = ntile * kMxBN + wn * 64 + 32 * j;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int c = c0 + 8 * q4 + 4 * kh;
          if (c >= N) continue;
          const f32x16_t& a = acc[i][j];
          *(u32x2_t*)(C + row * N + c) =
              u32x2_t{pack_bf16x2(a[4 * q4], a[4 * q4 + 1]), pack_bf16x2(a[4 * q4 + 2], a[4 * q4 + 3])};
        }
      }
    }
  }
}

hipError_t launch_mx_gemm(int epi, const void* A, const uint8_t* sa, const void* B,
                          const uint8_t* sb, const int32_t* offsets, int G, int rows, int N,
                          int K, int I, void* C, hipStream_t s) {
  const int ntn = epi == EPI_SWIGLU ? I / 64 : (N + kMxBN - 1) / kMxBN;
  const long long tiles = ((long long)rows / kMxBM + G) * ntn;  // upper bound
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU)
    mx_gemm_kernel<EPI_SWIGLU><<<(unsigned)tiles, 256, 0, s>>>(
        (const uint8_t*)A, sa, (const uint8_t*)B, sb, offsets, G, N, K, I, (uint16_t*)C);
  else
    mx_gemm_kernel<EPI_STORE><<<(unsigned)tiles, 256, 0, s>>>(
        (const uint8_t*)A, sa, (const uint8_t*)B, sb, offsets, G, N, K, I, (uint16_t*)C);
  return hipGetLastError();
}

}  // namespace moe
