// Grouped GEMM on the CDNA4 matrix cores (gfx950), bf16 or e4m3 operands, fp32 accumulate.
//
// Transformer Engine guide "Mixture of Experts", section "Grouped GEMM": one call runs
// the per-expert products Y_e = X_e W_e over expert-contiguous row blocks, with the
// per-expert row counts kept on the device. Section "Grouped MLP": FC1 carries the
// activation in its epilogue (here SwiGLU, te_mixtral.py _expert_ffn: silu(gate) * up
// on a fused gate/up weight) and FC2 is a separate grouped GEMM.
//
// Design (gfx950, wave64):
//  * 128x128 output tile per 256-thread block, four waves in a 2x2 grid, each wave a
//    64x64 sub-tile of four 32x32 MFMA blocks (v_mfma_f32_32x32x16_bf16, or
//    v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales for e4m3).
//  * K is staged 128 bytes at a time (64 bf16 or 128 e4m3) through two LDS buffers
//    (double buffering: the next tile's global loads are in flight while the MFMAs
//    consume the current one). Rows are padded to 144 bytes so the 16-byte fragment
//    reads of 16 consecutive rows hit distinct banks.
//  * Both operands are stored K-contiguous in LDS. Operands that are contiguous along
//    M or N in memory (the weight of the NN forward, both operands of the weight
//    gradient) are loaded as 8x8 bf16 blocks and transposed in registers before the
//    LDS write.
//  * Tile schedule on the device: every block rebuilds the prefix of per-group M-tile
//    counts from offsets[] in LDS, so any row split works with no host sync and no
//    padding. Tiles are ordered (group, N-tile, M-tile) so the M-tiles that share one
//    weight panel are neighbours, and block ids are remapped so that neighbours land
//    on the same XCD (blocks are dispatched round-robin over the 8 XCDs, each with
//    its own L2).
#include "internal.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 128;
constexpr int BKB = 128;                    // K bytes per stage
constexpr int PITCH = BKB + 16;             // padded LDS row pitch, bytes
constexpr int REGION_A = BM * PITCH;
constexpr int STAGE = (BM + BN) * PITCH;    // 36864 bytes
constexpr int NT = 256;

MOE_DEV uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
MOE_DEV uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// 8x8 bf16 transpose: in[i] holds columns 0..7 of row i; out[j] holds rows 0..7 of column j.
MOE_DEV void transpose8x8(const u32x4_t in[8], u32x4_t out[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t a = in[2 * d][j >> 1], b = in[2 * d + 1][j >> 1];
      out[j][d] = (j & 1) ? hi_pair(a, b) : lo_pair(a, b);
    }
  }
}

struct Tile {
  int g;
  int m0;          // first row (NN/NT: absolute row of the buffer; DW: first M index)
  int n0;          // first output column (SWIGLU: first h column)
  int rows_valid;  // NN/NT: rows of this tile inside the group
  int kcount;      // DW: rows of the group (the reduction length)
  int kbase;       // DW: first row of the group
};

template <int MODE, int EPI>
MOE_DEV int n_tiles(const GemmParams& p) {
  if (EPI == EPI_SWIGLU) return p.I / (BN / 2);
  return (p.N + BN - 1) / BN;
}

// Column of the B operand held by LDS row c of this tile.
template <int EPI>
MOE_DEV int bcol(const GemmParams& p, int n0, int c) {
  if (EPI == EPI_SWIGLU) return c < BN / 2 ? n0 + c : p.I + n0 + c - BN / 2;
  return n0 + c;
}

}  // namespace

template <int MODE, int EPI, bool FP8>
__global__ __launch_bounds__(NT, 2) void grouped_gemm_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ int s_pref[264];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = n_tiles<MODE, EPI>(p);

  // ---- tile schedule ------------------------------------------------------------
  int total;
  if (MODE != MOE_GEMM_TN_DW) {
    if (wave == 0) {
      const int per = (p.G + 63) / 64;
      int loc[5];
      int sum = 0;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int g = lane * per + i;
        int mt = 0;
        if (i < per && g < p.G) {
          const int cnt = p.offsets[g + 1] - p.offsets[g];
          mt = (cnt + BM - 1) / BM;
        }
        sum += mt;
        loc[i] = sum;
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      const int excl = incl - sum;
      if (lane == 0) s_pref[0] = 0;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int g = lane * per + i;
        if (i < per && g < p.G) s_pref[g + 1] = excl + loc[i];
      }
    }
    __syncthreads();
    total = s_pref[p.G] * ntn;
  } else {
    total = p.G * ((p.M + BM - 1) / BM) * ntn;
  }
  const int b = blockIdx.x;
  if (b >= total) return;
  int tile;
  {
    const int xcd = b & 7, i = b >> 3, base = total >> 3, rem = total & 7;
    tile = xcd * base + (xcd < rem ? xcd : rem) + i;
  }
  Tile t;
  if (MODE != MOE_GEMM_TN_DW) {
    int lo = 0, hi = p.G;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] * ntn <= tile) lo = mid;
      else hi = mid - 1;
    }
    const int g = lo;
    const int mt = s_pref[g + 1] - s_pref[g];
    const int local = tile - s_pref[g] * ntn;
    const int ntile = local / mt, mtile = local % mt;
    const int gbeg = p.offsets[g], cnt = p.offsets[g + 1] - gbeg;
    t.g = g;
    t.m0 = gbeg + mtile * BM;
    t.rows_valid = min(BM, cnt - mtile * BM);
    t.n0 = ntile * (EPI == EPI_SWIGLU ? BN / 2 : BN);
    t.kcount = p.K;
    t.kbase = 0;
  } else {
    const int mtn = (p.M + BM - 1) / BM;
    const int g = tile / (mtn * ntn), rem = tile % (mtn * ntn);
    t.g = g;
    t.m0 = (rem / ntn) * BM;
    t.n0 = (rem % ntn) * BN;
    t.rows_valid = BM;
    t.kbase = p.offsets[g];
    t.kcount = p.offsets[g + 1] - t.kbase;
  }

  // ---- operand addressing ---------------------------------------------------------
  // Each thread stages eight 16-byte global loads per K step.
  //  NT: all threads: rows (i*32 + tid/8) of A (i < 4) and of B (i >= 4), chunk tid%8.
  //  NN: threads 0..127 load one 8(k) x 8(n) block of B_g[K,N] (k block tid%8, column
  //      block tid/8) and transpose it; threads 128..255 load eight K-contiguous
  //      chunks of A, rows (tid-128)/8 + 16*i, chunk (tid-128)%8.
  //  DW: threads 0..127 transpose an 8x8 block of A[rows,M], threads 128..255 one of
  //      B[rows,N] (the reduction runs over the group's rows).
  const int q = tid & 127;
  const bool lower = tid < 128;
  const int kb = q & 7, nb = q >> 3;          // 8x8 block coordinates
  const int esz = FP8 ? 1 : 2;
  const uint8_t* src[8];                      // K-contiguous row pointers
  const uint16_t* blk = nullptr;              // 8x8 block source (row kb*8 of the tile)
  int blk_ld = 0;                             // its leading dimension, elements
  bool blk_ok = true;
  int nk;
  if (MODE != MOE_GEMM_TN_DW) {
    const size_t lda = (size_t)p.K * esz;
    const uint8_t* bg = (const uint8_t*)p.B + (size_t)t.g * p.N * lda;
    if (MODE == MOE_GEMM_NT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = min(i * 32 + (tid >> 3), t.rows_valid - 1);
        src[i] = (const uint8_t*)p.A + (size_t)(t.m0 + r) * lda + (tid & 7) * 16;
        const int c = min(bcol<EPI>(p, t.n0, i * 32 + (tid >> 3)), p.N - 1);
        src[4 + i] = bg + (size_t)c * lda + (tid & 7) * 16;
      }
    } else if (lower) {  // NN, B block
      const int c = bcol<EPI>(p, t.n0, nb * 8);
      blk_ok = c < p.N;
      blk_ld = p.N;
      blk = (const uint16_t*)p.B + (size_t)t.g * p.K * p.N + (size_t)(kb * 8) * p.N + (blk_ok ? c : 0);
    } else {             // NN, A chunks
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = min((q >> 3) + 16 * i, t.rows_valid - 1);
        src[i] = (const uint8_t*)p.A + (size_t)(t.m0 + r) * lda + (q & 7) * 16;
      }
    }
    nk = (int)(lda / BKB);
  } else {
    const int ld = lower ? p.M : p.N;
    const int c = (lower ? t.m0 : t.n0) + nb * 8;
    blk_ok = c < ld;
    blk_ld = ld;
    blk = (const uint16_t*)(lower ? p.A : p.B) + (size_t)(t.kbase + kb * 8) * ld + (blk_ok ? c : 0);
    nk = (t.kcount + 63) / 64;
  }

  u32x4_t st[8];

  auto load_stage = [&](int kt) {
    const bool is_blk = (MODE == MOE_GEMM_TN_DW) || (MODE == MOE_GEMM_NN && lower);
    if (!is_blk) {
      const size_t kbyte = (size_t)kt * BKB;
#pragma unroll
      for (int i = 0; i < 8; ++i) st[i] = *(const u32x4_t*)(src[i] + kbyte);
    } else {
      const uint16_t* s0 = blk + (size_t)kt * 64 * blk_ld;
      const int krow = kt * 64 + kb * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool in = blk_ok && (MODE != MOE_GEMM_TN_DW || krow + i < t.kcount);
        st[i] = in ? *(const u32x4_t*)(s0 + (size_t)i * blk_ld) : u32x4_t{0, 0, 0, 0};
      }
    }
  };

  auto store_stage = [&](int buf) {
    uint8_t* sa = smem + buf * STAGE;
    uint8_t* sb = sa + REGION_A;
    if (MODE == MOE_GEMM_NT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *(u32x4_t*)(sa + (i * 32 + (tid >> 3)) * PITCH + (tid & 7) * 16) = st[i];
        *(u32x4_t*)(sb + (i * 32 + (tid >> 3)) * PITCH + (tid & 7) * 16) = st[4 + i];
      }
    } else if (MODE == MOE_GEMM_NN && !lower) {
#pragma unroll
      for (int i = 0; i < 8; ++i) *(u32x4_t*)(sa + ((q >> 3) + 16 * i) * PITCH + (q & 7) * 16) = st[i];
    } else {
      uint8_t* dst = (MODE == MOE_GEMM_NN || !lower) ? sb : sa;
      u32x4_t tr[8];
      transpose8x8(st, tr);
#pragma unroll
      for (int j = 0; j < 8; ++j) *(u32x4_t*)(dst + (nb * 8 + j) * PITCH + kb * 16) = tr[j];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // LDS rows of this lane's fragments
  const int arow0 = wm * 64 + (lane & 31);
  int brow[2];
  if (EPI == EPI_SWIGLU) {
    brow[0] = wn * 32 + (lane & 31);            // gate columns
    brow[1] = BN / 2 + wn * 32 + (lane & 31);   // up columns
  } else {
    brow[0] = wn * 64 + (lane & 31);
    brow[1] = wn * 64 + 32 + (lane & 31);
  }
  const int khalf = lane >> 5;

  auto compute_stage = [&](int buf) {
    const uint8_t* sa = smem + buf * STAGE;
    const uint8_t* sb = sa + REGION_A;
    if (!FP8) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8_t af[2], bfr[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          af[mi] = *(const bf16x8_t*)(sa + (arow0 + mi * 32) * PITCH + ks * 32 + khalf * 16);
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          bfr[ni] = *(const bf16x8_t*)(sb + brow[ni] * PITCH + ks * 32 + khalf * 16);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        i32x8_t af[2], bfr[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const uint8_t* src = sa + (arow0 + mi * 32) * PITCH + ks * 64 + khalf * 32;
          const u32x4_t x0 = *(const u32x4_t*)src, x1 = *(const u32x4_t*)(src + 16);
          af[mi] = i32x8_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                           (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const uint8_t* src = sb + brow[ni] * PITCH + ks * 64 + khalf * 32;
          const u32x4_t x0 = *(const u32x4_t*)src, x1 = *(const u32x4_t*)(src + 16);
          bfr[ni] = i32x8_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                            (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[mi], bfr[ni], acc[mi][ni], 0, 0, 0, 127, 0, 127);
      }
    }
  };

  // ---- main loop: double-buffered LDS ---------------------------------------------
  if (nk > 0) {
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) load_stage(kt + 1);
      compute_stage(kt & 1);
      if (more) store_stage((kt + 1) & 1);
      __syncthreads();
    }
  }

  // ---- epilogue -------------------------------------------------------------------
  // 32x32 accumulator layout: lane l, element v -> column l%32,
  // row 8*(v/4) + 4*(l/32) + v%4.
  const int lcol = lane & 31;
  const int rbase = 4 * (lane >> 5);
  if (EPI == EPI_SWIGLU) {
    const int hcol = t.n0 + wn * 32 + lcol;
    uint16_t* h = (uint16_t*)p.C;
    uint16_t* gu = (uint16_t*)p.gu_out;
    const size_t twoI = 2 * (size_t)p.I;
    float sg = 1.f, su = 1.f;
    if (FP8) {
      sg = p.b_scale[(size_t)t.g * twoI + hcol];
      su = p.b_scale[(size_t)t.g * twoI + p.I + hcol];
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + mi * 32 + 8 * (v >> 2) + rbase + (v & 3);
        if (r < t.rows_valid) {
          const size_t row = (size_t)t.m0 + r;
          float g = acc[mi][0][v], u = acc[mi][1][v];
          if (FP8) {
            const float sa = p.a_scale[row];
            g = g * sa * sg;
            u = u * sa * su;
          }
          const float hv = g / (1.0f + expf(-g)) * u;
          h[row * p.I + hcol] = (uint16_t)f32_to_bf16(hv);
          if (gu) {
            gu[row * twoI + hcol] = (uint16_t)f32_to_bf16(g);
            gu[row * twoI + p.I + hcol] = (uint16_t)f32_to_bf16(u);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int col = t.n0 + wn * 64 + ni * 32 + lcol;
      if (col >= p.N) continue;
      float sb = 1.f;
      if (FP8) sb = p.b_scale[(size_t)t.g * p.N + col];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * 64 + mi * 32 + 8 * (v >> 2) + rbase + (v & 3);
          float val = acc[mi][ni][v];
          if (MODE == MOE_GEMM_TN_DW) {
            const int m = t.m0 + r;
            if (m >= p.M) continue;
            const size_t o = (size_t)t.g * p.M * p.N + (size_t)m * p.N + col;
            if (p.c_fp32) ((float*)p.C)[o] = val;
            else ((uint16_t*)p.C)[o] = (uint16_t)f32_to_bf16(val);
          } else {
            if (r >= t.rows_valid) continue;
            const size_t row = (size_t)t.m0 + r;
            if (FP8) val = val * p.a_scale[row] * sb;
            if (EPI == EPI_SWIGLU_BWD) {
              // val = dh[row, col], col < I; saved g, u are bf16
              const uint16_t* gu = (const uint16_t*)p.gu_in;
              const size_t twoI = 2 * (size_t)p.I;
              const float g = bf16_to_f32(gu[row * twoI + col]);
              const float u = bf16_to_f32(gu[row * twoI + p.I + col]);
              const float s = 1.0f / (1.0f + expf(-g));
              const float dg = val * u * s * (1.0f + g * (1.0f - s));
              const float du = val * g * s;
              uint16_t* dgu = (uint16_t*)p.C;
              dgu[row * twoI + col] = (uint16_t)f32_to_bf16(dg);
              dgu[row * twoI + p.I + col] = (uint16_t)f32_to_bf16(du);
            } else {
              const size_t o = row * p.N + col;
              if (p.c_fp32) ((float*)p.C)[o] = val;
              else ((uint16_t*)p.C)[o] = (uint16_t)f32_to_bf16(val);
            }
          }
        }
      }
    }
  }
}

hipError_t launch_grouped_gemm(const GemmParams& p, hipStream_t s) {
  if (p.G <= 0) return hipSuccess;
  // Upper bound of the tile count; the surplus blocks exit at once (the real count
  // lives on the device).
  long long blocks;
  int ntn = p.epi == EPI_SWIGLU ? p.I / (BN / 2) : (p.N + BN - 1) / BN;
  if (p.mode == MOE_GEMM_TN_DW) blocks = (long long)p.G * ((p.M + BM - 1) / BM) * ntn;
  else blocks = ((long long)(p.rows + BM - 1) / BM + p.G) * ntn;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(NT);
#define MOE_GG(MODE, EPI, F8) grouped_gemm_kernel<MODE, EPI, F8><<<grid, block, 0, s>>>(p)
  if (p.fp8) {
    if (p.mode != MOE_GEMM_NT) return hipErrorInvalidValue;
    if (p.epi == EPI_SWIGLU) MOE_GG(MOE_GEMM_NT, EPI_SWIGLU, true);
    else MOE_GG(MOE_GEMM_NT, EPI_STORE, true);
  } else if (p.mode == MOE_GEMM_NN) {
    if (p.epi == EPI_SWIGLU) MOE_GG(MOE_GEMM_NN, EPI_SWIGLU, false);
    else MOE_GG(MOE_GEMM_NN, EPI_STORE, false);
  } else if (p.mode == MOE_GEMM_NT) {
    if (p.epi == EPI_SWIGLU_BWD) MOE_GG(MOE_GEMM_NT, EPI_SWIGLU_BWD, false);
    else MOE_GG(MOE_GEMM_NT, EPI_STORE, false);
  } else {
    MOE_GG(MOE_GEMM_TN_DW, EPI_STORE, false);
  }
#undef MOE_GG
  return hipGetLastError();
}

}  // namespace moe
