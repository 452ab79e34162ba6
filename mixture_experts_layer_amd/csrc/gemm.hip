// Grouped GEMM on the CDNA4 matrix cores (gfx950), bf16 or e4m3 operands, fp32 accumulate.
//
// Transformer Engine guide "Mixture of Experts", section "Grouped GEMM": one call runs
// the per-expert products Y_e = X_e W_e over expert-contiguous row blocks, with the
// per-expert row counts kept on the device. Section "Grouped MLP": FC1 carries the
// activation in its epilogue (here SwiGLU, te_mixtral.py _expert_ffn: silu(gate) * up
// on a fused gate/up weight) and FC2 is a separate grouped GEMM.
//
// Design (gfx950, wave64):
//  * Block tile BM x BN, WM x WN waves; each wave owns (BM/WM) x (BN/WN) outputs as
//    32x32 MFMA blocks (v_mfma_f32_32x32x16_bf16, or v_mfma_scale_f32_32x32x64_f8f6f4
//    with unit scales for e4m3). A wave's M blocks are interleaved (wave wm takes
//    blocks wm, wm+WM, ...) so the blocks past a group's last row, which are skipped,
//    are spread over the waves.
//  * K advances 128 bytes per stage (64 bf16 or 128 e4m3). Operands go from global
//    memory straight into an LDS ring of STAGES buffers with 16-byte
//    global_load_lds (no staging registers, no VALU copies); the loads for stage
//    kt+STAGES-1 are in flight while stage kt is multiplied.
//  * LDS layouts. K-contiguous operands: rows of 128 bytes, the 16-byte chunk index
//    XORed with (row/2)%8, so the fragment reads of 16 consecutive rows hit distinct
//    banks. M- or N-contiguous operands (the bf16 weight of the NN forward, both
//    operands of the weight gradient): rows of k, the 64-byte segment index XORed with
//    k%4, read with ds_read_b64_tr_b16, which hands each lane 4 consecutive k of one
//    column (two reads form the 8-element MFMA operand). The swizzles are applied on
//    the global side because global_load_lds places lane l's 16 bytes at base + 16*l.
//  * Rows past a group's end and columns past N load from a zero block; the weight
//    gradient's ragged reduction is zero-padded the same way.
//  * Epilogue through LDS: accumulators (converted, or consumed by SwiGLU / SwiGLU
//    backward) are staged row-major and written with 16-byte stores.
//  * Tile schedule on the device: every block rebuilds the prefix of per-group M-tile
//    counts from offsets[] in LDS, so any row split works with no host sync and no
//    padding. Tiles are ordered (group, N-tile, M-tile) so the M-tiles that share one
//    weight panel are neighbours, and block ids are remapped so that neighbours land
//    on the same XCD (blocks are dispatched round-robin over the 8 XCDs, each with
//    its own L2).
#include <type_traits>

#include "internal.h"

namespace moe {

namespace {

__device__ __attribute__((aligned(256))) uint8_t g_zero_block[4096];  // stays zero

typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Workgroup barrier for the LDS ring. The memory clobbers keep the compiler from moving
// LDS accesses across it without emitting any wait: the producers' completion is
// established by the explicit vmcnt wait before it (global_load_lds) and by the
// consumers' own lgkmcnt waits (their fragments feed MFMAs issued before it).
MOE_DEV void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
MOE_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}

// 16 bytes per lane from global memory straight into LDS at M0 + 16*lane.
// Issued from inline asm so the compiler does not track it as an LDS write (its
// conservative tracking would wait for every DMA in flight before any LDS read); the
// instruction has no result registers, and its address and M0 are read at issue. The
// kernel orders these writes itself with explicit vmcnt waits and barriers.
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
MOE_DEV void load_lds16(const void* g, uint8_t* lds) {
  const unsigned m0 = (unsigned)(uintptr_t)((lds_u8_t*)lds);
  // one wait state between the M0 write and the LDS-DMA that reads it
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}

template <int BM, int BN, int WM, int WN, int STAGES, int BKB_>
struct Cfg {
  static constexpr int BKB = BKB_;      // K bytes per stage: 64 or 128
  static constexpr int KR = BKB / 2;    // bf16 k rows of an M/N-contiguous stage tile
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int MB = TM / 32, NB = TN / 32;
  static constexpr int A_BYTES = BM * BKB, B_BYTES = BN * BKB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int SMEM = STAGE * STAGES;
  static constexpr int A_LOADS = A_BYTES / 1024 / NW, B_LOADS = B_BYTES / 1024 / NW;  // per wave
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static_assert(BKB == 64 || BKB == 128, "stage depth");
  static_assert(MB >= 1 && NB >= 1, "wave tile");
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "load split");
};

// Rows of an epilogue slice: the tallest of BM, 128, 64, 32 whose staging fits `cap` bytes.
constexpr int slice_rows(int bm, int row_bytes, int cap) {
  return bm * row_bytes <= cap ? bm : 128 * row_bytes <= cap ? 128 : 64 * row_bytes <= cap ? 64 : 32;
}

struct Tile {
  int g;
  int m0;          // NN/NT: first buffer row of the tile; DW: first M index
  int n0;          // first output column (SWIGLU: first h column)
  int rows_valid;  // NN/NT: rows of this tile inside the group; DW: BM
  int kcount;      // DW: rows of the group (the reduction length)
  int kbase;       // DW: first row of the group
};

// K-contiguous operand tile: rows of BKB bytes, the 16-byte chunk index XORed with a
// function of the row so the fragment reads of 16 consecutive rows hit distinct banks:
// BKB = 128: 8 chunks, XOR (row/2)%8; BKB = 64: 4 chunks, XOR (row/4)%4.
template <int BKB>
MOE_DEV int kc_swz(int row) { return BKB == 128 ? (row >> 1) & 7 : (row >> 2) & 3; }
// One 1 KB chunk-load: lane l fills LDS row (chunk*rows + l/slots), physical 16-byte slot
// l%slots; the logical chunk it must hold is slot ^ swz(row).
template <int BKB>
MOE_DEV int kc_row(int chunk, int lane) { return chunk * (1024 / BKB) + lane / (BKB / 16); }
template <int BKB>
MOE_DEV int kc_logical(int row, int lane) { return (lane & (BKB / 16 - 1)) ^ kc_swz<BKB>(row); }

// M/N-contiguous operand tile: KR k-rows of W bytes (W = 2*cols), made of 64-byte
// segments. The physical segment of (k, logical segment s) is s ^ mn_swz(k), chosen so
// the ds_read_b64_tr_b16 pattern (rows k..k+3 and k+8..k+11, one segment each) spreads
// over the four 16-bank groups: W >= 256: s ^ (k & 3); W = 128 (two segments per row,
// row k starting at bank group 2k mod 4): s ^ ((k >> 1) & 1).
template <int COLS>
MOE_DEV int mn_swz(int k) {
  static_assert(COLS * 2 >= 128, "rows of at least two 64-byte segments");
  return COLS * 2 >= 256 ? (k & 3) : ((k >> 1) & 1);
}
// Lane l of chunk c fills row (c*1024 + 16*l) / W at physical offset (16*l) % W.
template <int COLS>
MOE_DEV void mn_slot(int chunk, int lane, int& k, int& logical_byte) {
  constexpr int W = COLS * 2;
  const int byte = chunk * 1024 + lane * 16;
  k = byte / W;
  const int phys = byte % W;
  logical_byte = (((phys >> 6) ^ mn_swz<COLS>(k)) << 6) | (phys & 63);
}

// LDS byte offset of element (k, col) in an M/N-contiguous tile.
template <int COLS>
MOE_DEV int mn_offset(int k, int col) {
  const int byte = col * 2;
  return k * (COLS * 2) + ((((byte >> 6) ^ mn_swz<COLS>(k)) << 6) | (byte & 63));
}

}  // namespace

template <int MODE, int EPI, bool FP8, int BM, int BN, int WM, int WN, int STAGES, int BKB_>
__global__ __launch_bounds__(WM* WN * 64, 1) void grouped_gemm_kernel(const GemmParams p) {
  using C = Cfg<BM, BN, WM, WN, STAGES, BKB_>;
  constexpr int BKB = C::BKB, KR = C::KR;
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");
  // The LDS ring: stage kt lives in buffer kt % STAGES. The DMA writes are issued from
  // inline asm, so the compiler's own LDS-DMA tracking never serialises reads behind them.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::SMEM];
  __shared__ int s_pref[264];
  static_assert(EPI != EPI_SWIGLU || C::NB % 2 == 0, "SwiGLU wave tile: gate blocks + as many up blocks");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases stay scalar
  const int wm = wave / WN, wn = wave % WN;
  constexpr bool DW = MODE == MOE_GEMM_TN_DW;
  constexpr bool B_MN = (MODE == MOE_GEMM_NN) || DW;  // B tile M/N-contiguous in memory
  constexpr int HB = BN / 2;                           // SwiGLU: h columns per tile
  const int ntn = EPI == EPI_SWIGLU ? (p.I + HB - 1) / HB : (p.N + BN - 1) / BN;

  // ---- tile schedule ------------------------------------------------------------
  int total;
  if (!DW) {
    if (wave == 0) {
      const int per = (p.G + 63) / 64;
      int loc[5];
      int sum = 0;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int g = lane * per + i;
        int mt = 0;
        if (i < per && g < p.G) mt = (p.offsets[g + 1] - p.offsets[g] + BM - 1) / BM;
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
  if (!DW) {
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
    t.n0 = ntile * (EPI == EPI_SWIGLU ? HB : BN);
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

  t.g = __builtin_amdgcn_readfirstlane(t.g);
  t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
  t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
  t.rows_valid = __builtin_amdgcn_readfirstlane(t.rows_valid);
  t.kcount = __builtin_amdgcn_readfirstlane(t.kcount);
  t.kbase = __builtin_amdgcn_readfirstlane(t.kbase);

  // ---- load descriptors: a global pointer per 1 KB chunk-load, advanced per stage ----
  const int esz = FP8 ? 1 : 2;
  const uint8_t* zero = g_zero_block;
  const uint8_t* a_src[C::A_LOADS];
  const uint8_t* b_src[C::B_LOADS];
  size_t a_step, b_step;      // bytes per stage
  int a_krow[C::A_LOADS], b_krow[C::B_LOADS];  // DW: k row of the chunk lane (zero past kcount)
  int nk;
  if constexpr (!DW) {
    const size_t lda = (size_t)p.K * esz;
    nk = (int)(lda / BKB);
    a_step = BKB;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      const int chunk = wave + C::NW * i;
      const int row = kc_row<BKB>(chunk, lane);
      a_src[i] = row < t.rows_valid
                     ? (const uint8_t*)p.A + (size_t)(t.m0 + row) * lda + kc_logical<BKB>(row, lane) * 16
                     : zero;
      a_krow[i] = 0;
    }
    if constexpr (!B_MN) {  // NT: B_g is [N, K]
      b_step = BKB;
      const uint8_t* bg = (const uint8_t*)p.B + (size_t)t.g * p.N * lda;
#pragma unroll
      for (int i = 0; i < C::B_LOADS; ++i) {
        const int chunk = wave + C::NW * i;
        const int row = kc_row<BKB>(chunk, lane);
        int col = row;
        bool ok;
        if (EPI == EPI_SWIGLU) {
          const int hcol = t.n0 + (row < HB ? row : row - HB);
          col = row < HB ? hcol : p.I + hcol;
          ok = hcol < p.I;
        } else {
          col = t.n0 + row;
          ok = col < p.N;
        }
        b_src[i] = ok ? bg + (size_t)col * lda + kc_logical<BKB>(row, lane) * 16 : zero;
        b_krow[i] = 0;
      }
    } else {      // NN: B_g is [K, N]
      b_step = (size_t)KR * p.N * 2;
      const uint8_t* bg = (const uint8_t*)p.B + (size_t)t.g * p.K * p.N * 2;
#pragma unroll
      for (int i = 0; i < C::B_LOADS; ++i) {
        const int chunk = wave + C::NW * i;
        int k, lb;
        mn_slot<BN>(chunk, lane, k, lb);
        const int c = lb / 2;  // column within the tile
        int col;
        bool ok;
        if (EPI == EPI_SWIGLU) {
          const int hcol = t.n0 + (c < HB ? c : c - HB);
          col = c < HB ? hcol : p.I + hcol;
          ok = hcol < p.I;
        } else {
          col = t.n0 + c;
          ok = col < p.N;
        }
        b_src[i] = ok ? bg + ((size_t)k * p.N + col) * 2 : zero;
        b_krow[i] = 0;
      }
    }
  } else {
    nk = (t.kcount + KR - 1) / KR;
    a_step = (size_t)KR * p.M * 2;
    b_step = (size_t)KR * p.N * 2;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      const int chunk = wave + C::NW * i;
      int k, lb;
      mn_slot<BM>(chunk, lane, k, lb);
      const int col = t.m0 + lb / 2;
      a_krow[i] = col < p.M ? k : 0x40000000;  // never valid when the column is out of range
      a_src[i] = (const uint8_t*)p.A + ((size_t)(t.kbase + k) * p.M + (col < p.M ? col : 0)) * 2;
    }
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
      const int chunk = wave + C::NW * i;
      int k, lb;
      mn_slot<BN>(chunk, lane, k, lb);
      const int col = t.n0 + lb / 2;
      b_krow[i] = col < p.N ? k : 0x40000000;
      b_src[i] = (const uint8_t*)p.B + ((size_t)(t.kbase + k) * p.N + (col < p.N ? col : 0)) * 2;
    }
  }

  // Load slot i < LOADS of stage kt: A chunk-loads first, then B.
  auto issue_one = [&](int kt, uint8_t* sa, int i) __attribute__((always_inline)) {
    if (i < C::A_LOADS) {
      const uint8_t* src;
      if (DW) src = (kt * KR + a_krow[i] < t.kcount) ? a_src[i] + (size_t)kt * a_step : zero;
      else src = a_src[i] == zero ? zero : a_src[i] + (size_t)kt * a_step;
      load_lds16(src, sa + (wave + C::NW * i) * 1024);
    } else {
      const int j = i - C::A_LOADS;
      const uint8_t* src;
      if (DW) src = (kt * KR + b_krow[j] < t.kcount) ? b_src[j] + (size_t)kt * b_step : zero;
      else src = b_src[j] == zero ? zero : b_src[j] + (size_t)kt * b_step;
      load_lds16(src, sa + C::A_BYTES + (wave + C::NW * j) * 1024);
    }
  };
  auto issue_stage = [&](int kt, uint8_t* sa) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) issue_one(kt, sa, i);
  };

  // ---- fragments --------------------------------------------------------------------
  f32x16_t acc[C::MB][C::NB];
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < C::NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // M blocks of this wave that hold at least one valid row (wave-uniform)
  int mb_live = 0;
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
    if ((wm + WM * i) * 32 < t.rows_valid) mb_live = i + 1;
  mb_live = __builtin_amdgcn_readfirstlane(mb_live);
  nk = __builtin_amdgcn_readfirstlane(nk);

  // B block column (within the tile) of N block j of this wave. SwiGLU: the first NB/2
  // blocks are gate columns, the last NB/2 the matching up columns (offset HB).
  auto bcol0 = [&](int j) __attribute__((always_inline)) {
    if (EPI == EPI_SWIGLU) {
      constexpr int NH = C::NB / 2;
      return j < NH ? (wn * NH + j) * 32 : HB + (wn * NH + j - NH) * 32;
    }
    return (wn * C::NB + j) * 32;
  };

  const int l32 = lane & 31, khalf = lane >> 5;
  // tr16 address pattern: row (k) and column offset of this lane's 4-element source
  const int tr_k = khalf * 8 + ((lane & 15) >> 2);
  const int tr_c = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;

  auto kc_frag = [&](const uint8_t* base, int row, int chunk) __attribute__((always_inline)) -> u32x4_t {
    return *(const u32x4_t*)(base + row * BKB + ((chunk ^ kc_swz<BKB>(row)) << 4));
  };
  // Fragment loads of k sub-step ks into registers.
  auto load_frags = [&](auto MBL_c, const uint8_t* sa, int ks, auto& af, auto& bfr) __attribute__((always_inline)) {
    constexpr int MBL = decltype(MBL_c)::value;
    const uint8_t* sb = sa + C::A_BYTES;
    if constexpr (!FP8) {
#pragma unroll
      for (int i = 0; i < MBL; ++i) {
        const int r0 = (wm + WM * i) * 32;
        if constexpr (!DW) {
          af[i] = __builtin_bit_cast(bf16x8_t, kc_frag(sa, r0 + l32, ks * 2 + khalf));
        } else {
          const int k = ks * 16 + tr_k;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(sa + mn_offset<BM>(k, r0 + tr_c)));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(sa + mn_offset<BM>(k + 4, r0 + tr_c)));
          af[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
#pragma unroll
      for (int j = 0; j < C::NB; ++j) {
        const int c0 = bcol0(j);
        if constexpr (!B_MN) {
          bfr[j] = __builtin_bit_cast(bf16x8_t, kc_frag(sb, c0 + l32, ks * 2 + khalf));
        } else {
          const int k = ks * 16 + tr_k;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(sb + mn_offset<BN>(k, c0 + tr_c)));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_t*)(sb + mn_offset<BN>(k + 4, c0 + tr_c)));
          bfr[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < MBL; ++i) {
        const int r = (wm + WM * i) * 32 + l32;
        const u32x4_t x0 = kc_frag(sa, r, ks * 4 + khalf * 2);
        const u32x4_t x1 = kc_frag(sa, r, ks * 4 + khalf * 2 + 1);
        af[i] = i32x8_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                        (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      }
#pragma unroll
      for (int j = 0; j < C::NB; ++j) {
        const int r = bcol0(j) + l32;
        const u32x4_t x0 = kc_frag(sb, r, ks * 4 + khalf * 2);
        const u32x4_t x1 = kc_frag(sb, r, ks * 4 + khalf * 2 + 1);
        bfr[j] = i32x8_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                         (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      }
    }
  };
  auto mfmas = [&](auto MBL_c, const auto& af, const auto& bfr) __attribute__((always_inline)) {
    constexpr int MBL = decltype(MBL_c)::value;
#pragma unroll
    for (int i = 0; i < MBL; ++i)
#pragma unroll
      for (int j = 0; j < C::NB; ++j) {
        if constexpr (!FP8)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], acc[i][j],
                                                                       0, 0, 0, 127, 0, 127);
      }
  };
  // One ring stage: KS k sub-steps; while sub-step ks multiplies, the fragments of ks+1
  // are read and a slice of the loads of stage kt+2 (into `nxt`) is issued.
  auto compute_stage = [&](auto MBL_c, const uint8_t* sa, int kt_next, uint8_t* nxt) __attribute__((always_inline)) {
    constexpr int KS = FP8 ? BKB / 64 : BKB / 32;
    constexpr int PER = (C::LOADS + KS - 1) / KS;
    using frag_t = typename std::conditional<FP8, i32x8_t, bf16x8_t>::type;
    frag_t af[2][C::MB], bfr[2][C::NB];
    load_frags(MBL_c, sa, 0, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) load_frags(MBL_c, sa, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
      if (kt_next >= 0) {
#pragma unroll
        for (int q = ks * PER; q < (ks + 1) * PER && q < C::LOADS; ++q) issue_one(kt_next, nxt, q);
      }
      mfmas(MBL_c, af[ks & 1], bfr[ks & 1]);
    }
  };

  // ---- main loop: ring of three LDS buffers, unrolled so each buffer is static ------
  // step(kt): stage kt is complete in `cur` once this wave's loads for it have landed
  // (at most the next stage's loads still in flight) and every wave passed the barrier;
  // the loads for stage kt+2 go to `nxt`, which held stage kt-1, spread over the
  // sub-steps of this stage's multiply.
  auto buf = [&](int kt) __attribute__((always_inline)) { return smem + (kt % STAGES) * C::STAGE; };
  auto main_loop = [&](auto MBL_c) __attribute__((always_inline)) {
    constexpr int LEAD = STAGES - 1;  // stages in flight ahead of the one being multiplied
#pragma unroll
    for (int s0 = 0; s0 < LEAD; ++s0)
      if (s0 < nk) issue_stage(s0, buf(s0));
    for (int kt = 0; kt < nk; ++kt) {
      // stage kt has landed once at most the later issued stages are still in flight
      const int later = min(LEAD - 1, nk - 1 - kt);
      if (LEAD - 1 >= 2 && later >= 2) wait_vmcnt<(LEAD >= 3 ? 2 : 0) * C::LOADS>();
      else if (LEAD - 1 >= 1 && later >= 1) wait_vmcnt<C::LOADS>();
      else wait_vmcnt<0>();
      ring_barrier();  // every wave's loads for stage kt landed; stage kt-1 fully read
      compute_stage(MBL_c, buf(kt), kt + LEAD < nk ? kt + LEAD : -1, buf(kt + LEAD));
    }
  };
  static_assert(C::MB <= 4, "live-block dispatch below covers up to four M blocks per wave");
  // Every wave runs the loop: it issues its share of each stage's loads and takes part
  // in every barrier even when none of its M blocks holds a valid row (MBL = 0).
  switch (mb_live) {
    case 0: main_loop(std::integral_constant<int, 0>{}); break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (C::MB >= 2) main_loop(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (C::MB >= 3) main_loop(std::integral_constant<int, 3>{}); break;
    default: if constexpr (C::MB >= 4) main_loop(std::integral_constant<int, 4>{}); break;
  }
  wait_vmcnt<0>();
  __syncthreads();

  // ---- epilogue: stage row slices of the tile in LDS, then 16-byte stores ----------
  // 32x32 accumulator layout: lane l, element v -> column l%32, row 8*(v/4) + 4*(l/32) + v%4.
  // A slice of PR rows holds the M blocks (wm + WM*i) whose rows fall inside it.
  const int rb = 4 * khalf;
  if (EPI == EPI_SWIGLU) {
    // h slice [PR][HB] bf16 in the first half of the ring, g,u slice [PR][BN] in the second
    constexpr int HP = HB * 2 + 16, GP = BN * 2 + 16;
    constexpr int PR = slice_rows(BM, GP, C::SMEM / 2);
    static_assert(PR * GP <= C::SMEM / 2 && PR * HP <= C::SMEM / 2, "slice");
    uint8_t* sh = smem;
    uint8_t* sgu = smem + C::SMEM / 2;
    constexpr int NH = C::NB / 2;
    const size_t twoI = 2 * (size_t)p.I;
    for (int r0 = 0; r0 < t.rows_valid; r0 += PR) {
#pragma unroll
      for (int jg = 0; jg < NH; ++jg) {
        const int hc = (wn * NH + jg) * 32 + l32;   // h column within the tile
        float sg = 1.f, su = 1.f;
        if (FP8 && t.n0 + hc < p.I) {
          sg = p.b_scale[(size_t)t.g * twoI + t.n0 + hc];
          su = p.b_scale[(size_t)t.g * twoI + p.I + t.n0 + hc];
        }
#pragma unroll
        for (int i = 0; i < C::MB; ++i) {
          const int blk = (wm + WM * i) * 32;
          if (i >= mb_live || blk < r0 || blk >= r0 + PR) continue;
#pragma unroll
          for (int v = 0; v < 16; v += 2) {  // rows r and r+1 share one packed convert
            const int r = blk + 8 * (v >> 2) + rb + (v & 3);
            float g0 = acc[i][jg][v], u0 = acc[i][jg + NH][v];
            float g1 = acc[i][jg][v + 1], u1 = acc[i][jg + NH][v + 1];
            if (FP8) {
              const float sa0 = r < t.rows_valid ? p.a_scale[t.m0 + r] : 0.f;
              const float sa1 = r + 1 < t.rows_valid ? p.a_scale[t.m0 + r + 1] : 0.f;
              g0 *= sa0 * sg;
              u0 *= sa0 * su;
              g1 *= sa1 * sg;
              u1 *= sa1 * su;
            }
            const uint32_t hv = pack_bf16x2(g0 * sigmoid_fast(g0) * u0, g1 * sigmoid_fast(g1) * u1);
            uint8_t* hrow = sh + (r - r0) * HP + hc * 2;
            *(uint16_t*)hrow = (uint16_t)hv;
            *(uint16_t*)(hrow + HP) = (uint16_t)(hv >> 16);
            if (p.gu_out) {
              const uint32_t gv = pack_bf16x2(g0, g1), uv = pack_bf16x2(u0, u1);
              uint8_t* grow = sgu + (r - r0) * GP + hc * 2;
              *(uint16_t*)grow = (uint16_t)gv;
              *(uint16_t*)(grow + GP) = (uint16_t)(gv >> 16);
              *(uint16_t*)(grow + HB * 2) = (uint16_t)uv;
              *(uint16_t*)(grow + GP + HB * 2) = (uint16_t)(uv >> 16);
            }
          }
        }
      }
      __syncthreads();
      constexpr int HV = HB / 8;  // 16-byte vectors per h row
      for (int idx = tid; idx < PR * HV; idx += C::NT) {
        const int r = idx / HV, c = idx % HV;
        if (r0 + r < t.rows_valid && t.n0 + c * 8 < p.I) {
          const u32x4_t v = *(const u32x4_t*)(sh + r * HP + c * 16);
          *(u32x4_t*)((uint16_t*)p.C + (size_t)(t.m0 + r0 + r) * p.I + t.n0 + c * 8) = v;
        }
      }
      if (p.gu_out) {
        constexpr int GV = BN / 8;
        for (int idx = tid; idx < PR * GV; idx += C::NT) {
          const int r = idx / GV, c = idx % GV;
          const int hcol = t.n0 + (c < HV ? c : c - HV) * 8;
          if (r0 + r < t.rows_valid && hcol < p.I) {
            const u32x4_t v = *(const u32x4_t*)(sgu + r * GP + c * 16);
            const int col = c < HV ? hcol : p.I + hcol;
            *(u32x4_t*)((uint16_t*)p.gu_out + (size_t)(t.m0 + r0 + r) * twoI + col) = v;
          }
        }
      }
      __syncthreads();
    }
  } else if (EPI == EPI_SWIGLU_BWD || p.c_fp32) {
    // fp32 slice [PR][BN] in the ring
    constexpr int FP = BN * 4 + 16;
    constexpr int PR = slice_rows(BM, FP, C::SMEM);
    static_assert(PR * FP <= C::SMEM, "slice");
    uint8_t* sf = smem;
    for (int r0 = 0; r0 < t.rows_valid; r0 += PR) {
#pragma unroll
      for (int i = 0; i < C::MB; ++i) {
        const int blk = (wm + WM * i) * 32;
        if (i >= mb_live || blk < r0 || blk >= r0 + PR) continue;
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
          const int c = bcol0(j) + l32;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = blk + 8 * (v >> 2) + rb + (v & 3);
            *(float*)(sf + (r - r0) * FP + c * 4) = acc[i][j][v];
          }
        }
      }
      __syncthreads();
      constexpr int V8 = BN / 8;  // 8-column groups per row
      for (int idx = tid; idx < PR * V8; idx += C::NT) {
        const int r = idx / V8, c8 = idx % V8;
        const int col = t.n0 + c8 * 8;
        const int rr = r0 + r;
        if (rr >= t.rows_valid || col >= p.N) continue;
        if (DW && t.m0 + rr >= p.M) continue;
        const f32x4_t x0 = *(const f32x4_t*)(sf + r * FP + c8 * 32);
        const f32x4_t x1 = *(const f32x4_t*)(sf + r * FP + c8 * 32 + 16);
        float val[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        if (EPI == EPI_SWIGLU_BWD) {
          const size_t twoI = 2 * (size_t)p.I;
          const size_t row = (size_t)t.m0 + rr;
          const u32x4_t gv = *(const u32x4_t*)((const uint16_t*)p.gu_in + row * twoI + col);
          const u32x4_t uv = *(const u32x4_t*)((const uint16_t*)p.gu_in + row * twoI + p.I + col);
          u32x4_t dg, du;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            float o[4];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const float g = h2 ? bf16hi(gv[d]) : bf16lo(gv[d]);
              const float u = h2 ? bf16hi(uv[d]) : bf16lo(uv[d]);
              const float dh = val[2 * d + h2];
              const float sgm = sigmoid_fast(g);
              o[h2] = dh * u * sgm * (1.0f + g * (1.0f - sgm));
              o[2 + h2] = dh * g * sgm;
            }
            dg[d] = pack_bf16x2(o[0], o[1]);
            du[d] = pack_bf16x2(o[2], o[3]);
          }
          *(u32x4_t*)((uint16_t*)p.C + row * twoI + col) = dg;
          *(u32x4_t*)((uint16_t*)p.C + row * twoI + p.I + col) = du;
        } else {
          const size_t o = DW ? (size_t)t.g * p.M * p.N + (size_t)(t.m0 + rr) * p.N + col
                              : (size_t)(t.m0 + rr) * p.N + col;
          if (FP8) {
            const float sa = p.a_scale[t.m0 + rr];
#pragma unroll
            for (int e = 0; e < 8; ++e) val[e] *= sa * p.b_scale[(size_t)t.g * p.N + col + e];
          }
          *(f32x4_t*)((float*)p.C + o) = f32x4_t{val[0], val[1], val[2], val[3]};
          *(f32x4_t*)((float*)p.C + o + 4) = f32x4_t{val[4], val[5], val[6], val[7]};
        }
      }
      __syncthreads();
    }
  } else {
    // bf16 slice [PR][BN] in the ring
    constexpr int CP = BN * 2 + 16;
    constexpr int PR = slice_rows(BM, CP, C::SMEM);
    static_assert(PR * CP <= C::SMEM, "slice");
    uint8_t* sc = smem;
    for (int r0 = 0; r0 < t.rows_valid; r0 += PR) {
#pragma unroll
      for (int i = 0; i < C::MB; ++i) {
        const int blk = (wm + WM * i) * 32;
        if (i >= mb_live || blk < r0 || blk >= r0 + PR) continue;
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
          const int c = bcol0(j) + l32;
          float sb = 1.f;
          if (FP8) sb = (t.n0 + c < p.N) ? p.b_scale[(size_t)t.g * p.N + t.n0 + c] : 0.f;
#pragma unroll
          for (int v = 0; v < 16; v += 2) {  // rows r and r+1 share one packed convert
            const int r = blk + 8 * (v >> 2) + rb + (v & 3);
            float v0 = acc[i][j][v], v1 = acc[i][j][v + 1];
            if (FP8) {
              v0 = r < t.rows_valid ? v0 * p.a_scale[t.m0 + r] * sb : 0.f;
              v1 = r + 1 < t.rows_valid ? v1 * p.a_scale[t.m0 + r + 1] * sb : 0.f;
            }
            const uint32_t pk = pack_bf16x2(v0, v1);
            uint8_t* crow = sc + (r - r0) * CP + c * 2;
            *(uint16_t*)crow = (uint16_t)pk;
            *(uint16_t*)(crow + CP) = (uint16_t)(pk >> 16);
          }
        }
      }
      __syncthreads();
      constexpr int V8 = BN / 8;
      for (int idx = tid; idx < PR * V8; idx += C::NT) {
        const int r = idx / V8, c8 = idx % V8;
        const int col = t.n0 + c8 * 8;
        const int rr = r0 + r;
        if (rr >= t.rows_valid || col >= p.N) continue;
        if (DW && t.m0 + rr >= p.M) continue;
        const size_t o = DW ? (size_t)t.g * p.M * p.N + (size_t)(t.m0 + rr) * p.N + col
                            : (size_t)(t.m0 + rr) * p.N + col;
        *(u32x4_t*)((uint16_t*)p.C + o) = *(const u32x4_t*)(sc + r * CP + c8 * 16);
      }
      __syncthreads();
    }
  }
}

namespace {

template <int MODE, int EPI, bool FP8, int BM, int BN, int WM, int WN, int STAGES, int BKB>
hipError_t launch_cfg(const GemmParams& p, hipStream_t s) {
  using C = Cfg<BM, BN, WM, WN, STAGES, BKB>;
  auto kern = grouped_gemm_kernel<MODE, EPI, FP8, BM, BN, WM, WN, STAGES, BKB>;
  static_assert(C::SMEM + 264 * 4 <= 160 * 1024, "LDS budget");
  const int ntn = EPI == EPI_SWIGLU ? (p.I + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
  long long blocks;
  if (MODE == MOE_GEMM_TN_DW) blocks = (long long)p.G * ((p.M + BM - 1) / BM) * ntn;
  else blocks = ((long long)(p.rows + BM - 1) / BM + p.G) * ntn;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  kern<<<dim3((unsigned)blocks), dim3(C::NT), 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

// Tile configurations (BM, BN, WM, WN, STAGES, K bytes per stage), chosen by
// measurement on the Qwen3- and Mixtral-shaped expert GEMMs: bf16 uses 256x256 tiles with
// eight waves (two per SIMD, 128x64 each) and a four-stage ring of 64-byte K steps (three
// stages of loads in flight); e4m3 uses 256x128 tiles with four waves and a three-stage
// ring of 128-byte steps (its eight-wave build does not fit the register file).
#ifndef MOE_GEMM_TILE_BF16
#define MOE_GEMM_TILE_BF16 256, 256, 2, 4, 4, 64
#endif
#ifndef MOE_GEMM_TILE_FP8
#define MOE_GEMM_TILE_FP8 256, 128, 2, 2, 3, 128
#endif
// Small-M tiles (decode: a handful of rows per expert): 32-row tiles, 64 output columns
// per block (one wave), a four-stage ring of 64-byte K steps; many blocks per CU so that
// enough waves stream the weights.
#ifndef MOE_GEMM_TILE_SMALL_M
#define MOE_GEMM_TILE_SMALL_M 32, 64, 1, 1, 4, 64
#endif
namespace {
template <int MODE, int EPI, bool F8>
hipError_t launch_sel(const GemmParams& p, hipStream_t s) {
  if constexpr (F8) {
    return launch_cfg<MODE, EPI, true, MOE_GEMM_TILE_FP8>(p, s);
  } else {
    // every group fits one 32-row tile when the whole buffer has at most 32 rows per group
    // on average and at most 256 rows: the decode case
    if constexpr (MODE != MOE_GEMM_TN_DW) {
      if (p.rows <= 256 && p.rows <= 32 * p.G)
        return launch_cfg<MODE, EPI, false, MOE_GEMM_TILE_SMALL_M>(p, s);
    }
    return launch_cfg<MODE, EPI, false, MOE_GEMM_TILE_BF16>(p, s);
  }
}
}  // namespace

hipError_t launch_grouped_gemm(const GemmParams& p, hipStream_t s) {
  if (p.G <= 0) return hipSuccess;
#define MOE_GG(MODE, EPI, F8) return launch_sel<MODE, EPI, F8>(p, s)
  if (p.fp8) {
    if (p.mode != MOE_GEMM_NT) return hipErrorInvalidValue;
    if (p.epi == EPI_SWIGLU) MOE_GG(MOE_GEMM_NT, EPI_SWIGLU, true);
    MOE_GG(MOE_GEMM_NT, EPI_STORE, true);
  }
  if (p.mode == MOE_GEMM_NN) {
    if (p.epi == EPI_SWIGLU) MOE_GG(MOE_GEMM_NN, EPI_SWIGLU, false);
    MOE_GG(MOE_GEMM_NN, EPI_STORE, false);
  }
  if (p.mode == MOE_GEMM_NT) {
    if (p.epi == EPI_SWIGLU_BWD) MOE_GG(MOE_GEMM_NT, EPI_SWIGLU_BWD, false);
    MOE_GG(MOE_GEMM_NT, EPI_STORE, false);
  }
  MOE_GG(MOE_GEMM_TN_DW, EPI_STORE, false);
#undef MOE_GG
}

}  // namespace moe
