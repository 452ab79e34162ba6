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
//  * K advances 64 or 128 bytes per stage (32 or 64 bf16, 64 e4m3). Operands go from
//    global memory straight into an LDS ring of STAGES buffers with 16-byte
//    global_load_lds (no staging registers, no VALU copies); the loads for stage
//    kt+STAGES-1 are in flight while stage kt is multiplied.
//  * LDS layouts. K-contiguous operands: rows of 64 or 128 bytes, the 16-byte chunk
//    index XORed with (row/4)%4 or (row/2)%8, so the fragment reads of 16 consecutive
//    rows hit distinct banks. M- or N-contiguous operands (the bf16 weight of the NN forward, both
//    operands of the weight gradient): rows of k, the 64-byte segment index XORed with
//    k%4, read with ds_read_b64_tr_b16, which hands each lane 4 consecutive k of one
//    column (two reads form the 8-element MFMA operand). The swizzles are applied on
//    the global side because global_load_lds places lane l's 16 bytes at base + 16*l.
//  * Rows past a group's end and columns past N load the tile's first row or column:
//    they only feed outputs that are never stored. The weight gradient's ragged
//    reduction is zero-padded from a zero block.
//  * Epilogue through LDS: accumulators (converted, or consumed by SwiGLU / SwiGLU
//    backward) are staged row-major and written with 16-byte stores.
//  * Tile schedule on the device: every block rebuilds the prefix of per-group M-tile
//    counts from offsets[] in LDS, so any row split works with no host sync and no
//    padding; a group's rows are spread evenly over its M tiles. Tiles are ordered
//    (group, N-tile, M-tile) so the M-tiles that share one weight panel are neighbours.
//    The grid is persistent (every resident block); XCD x (blocks are dispatched
//    round-robin over the 8 XCDs, each with its own L2) serves the x-th eighth of the
//    tile range, from a per-XCD ticket counter (ragged rows) or with a fixed stride
//    (weight gradients), and the load of a block's next tile starts while the current
//    one is still being multiplied.
#include <atomic>
#include <type_traits>

#include "internal.h"

// Split-K of the 32-row (decode) tiles, per epilogue: bit 0 the SwiGLU GEMM, bit 1 the
// store GEMM.
#ifndef MOE_GEMM_SPLITK
#define MOE_GEMM_SPLITK 3
#endif

namespace moe {

namespace {

__device__ __attribute__((aligned(256))) uint8_t g_zero_block[4096];  // stays zero

// Tile counters of the persistent launches: one counter per XCD ([0..8)) and the count of
// finished blocks ([8]). The last block of a launch to finish puts them back to zero, so the
// next launch that uses them starts from zero. The layer's launches bring their own (in
// the layer workspace, zeroed by its dispatch); the stand-alone entry points take the
// library's slots in turn (kSchedSlots of them), so launches in flight at the same time
// on one device use different slots as long as fewer than kSchedSlots overlap.
constexpr int kSchedSlots = 64;
__device__ int g_sched[kSchedSlots][16];

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

// The same from a wave-uniform base (SGPR pair) plus a 32-bit per-lane byte offset.
// One 4-byte LDS-DMA per lane: lane l fills lds + 4 l.
MOE_DEV void load_lds4(const void* g, uint8_t* lds) {
  const unsigned m0 = (unsigned)(uintptr_t)((lds_u8_t*)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}
MOE_DEV void load_lds16_s(const void* base, uint32_t off, uint8_t* lds) {
  const unsigned m0 = (unsigned)(uintptr_t)((lds_u8_t*)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}
// The same with the non-temporal cache policy, for data streamed once.
MOE_DEV void load_lds16_s_nt(const void* base, uint32_t off, uint8_t* lds) {
  const unsigned m0 = (unsigned)(uintptr_t)((lds_u8_t*)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}

template <int BM, int BN, int WM, int WN, int STAGES, int BKB_>
struct Cfg {
  static constexpr int BKB = BKB_;      // K bytes per stage: 64 or 128
  static constexpr int KR = BKB / 2;    // bf16 k rows of an M/N-contiguous stage tile
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int MB = TM / 32, NB = TN / 32;
  // A chunk-loads per wave: a whole number, so with BM * BKB not a multiple of NW KB the
  // last rows of the A area are loaded (from the tile's first row) and never read
  static constexpr int A_LOADS = (BM * BKB / 1024 + NW - 1) / NW;
  static constexpr int A_BYTES = A_LOADS * NW * 1024, B_BYTES = BN * BKB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int SMEM = STAGE * STAGES;
  static constexpr int B_LOADS = B_BYTES / 1024 / NW;  // per wave
  static constexpr int LOADS = A_LOADS + B_LOADS;
  static_assert(BKB == 64 || BKB == 128, "stage depth");
  static_assert(MB >= 1 && NB >= 1, "wave tile");
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "load split");
};

struct Tile {
  int g;
  int m0;          // NN/NT: first buffer row of the tile; DW: first M index
  int n0;          // first output column (SWIGLU: first h column)
  int rows_valid;  // NN/NT: rows of this tile inside the group; DW: BM
  int kcount;      // DW: rows of the group (the reduction length)
  int kbase;       // first row of the group
  int nst;         // NN/NT: K stages of the tile (of its K part when split)
  int kst0;        // NN/NT: first K stage
  int ks;          // NN/NT: K part
};

// Split-K: the number of K parts per tile for `base` tiles of nk stages on `blocks`
// persistent blocks. The decode launches stream weights, and measurement on them showed
// the memory system saturating with about half of the compute units streaming wide weight
// strips (more streams, from more tiles or from K parts, made the launch no faster, and the
// parts' partial sums and second launch cost extra). So only launches that leave more than
// 1 - 1/MOE_SPLITK_SPARSE of the blocks without a tile split, into the fewest parts that
// give half of the blocks one; parts keep at least four stages.
#ifndef MOE_SPLITK_SPARSE
#define MOE_SPLITK_SPARSE 2
#endif
MOE_DEV int choose_ksplit(int base, int blocks, int nk) {
  if (base <= 0 || (long long)base * MOE_SPLITK_SPARSE >= blocks) return 1;
  int s = (blocks / 2 + base - 1) / base;
  s = s < kSplitKMax ? s : kSplitKMax;
  while (s > 1 && nk / s < 4) --s;
  return s;
}

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

namespace {

// Buffer resource over one output tile: stores whose byte offset is kOutOfRange (at or past
// the record count) are dropped by the hardware range check, so masked lanes still issue
// their store and every wave issues the same number of stores per epilogue.
constexpr int kOutOfRange = 0x7fffffff;
MOE_DEV __amdgpu_buffer_rsrc_t tile_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, kOutOfRange, 0x00020000);
}

// s_waitcnt vmcnt for "stage landed": `pend` later stages (LOADS each) and, with allow > 0,
// one epilogue's stores (S1 or S2 instructions) were issued after the stage's loads. The
// counter drains in issue order, so any allowance not above the younger operations is safe.
template <int LOADS, int S1, int S2>
MOE_DEV void wait_stage(int pend, int allow) {
  constexpr int A = S1 < 63 ? S1 : 63, B = S2 < 63 ? S2 : 63;
  constexpr int A1 = LOADS + S1 < 63 ? LOADS + S1 : 63, B1 = LOADS + S2 < 63 ? LOADS + S2 : 63;
  constexpr int A2 = 2 * LOADS + S1 < 63 ? 2 * LOADS + S1 : 63;
  constexpr int B2 = 2 * LOADS + S2 < 63 ? 2 * LOADS + S2 : 63;
  if (allow == 0) {
    if (pend >= 2) wait_vmcnt<2 * LOADS>();
    else if (pend == 1) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
  } else if (allow == 1) {
    if (pend >= 2) wait_vmcnt<A2>();
    else if (pend == 1) wait_vmcnt<A1>();
    else wait_vmcnt<A>();
  } else {
    if (pend >= 2) wait_vmcnt<B2>();
    else if (pend == 1) wait_vmcnt<B1>();
    else wait_vmcnt<B>();
  }
}

}  // namespace

// BNT (NN only): the launch streams each weight panel once (its groups average at most one
// M tile), so the weight tiles are loaded with the non-temporal policy and leave the caches
// to the activation rows that several N tiles re-read. An NN weight tile is read as whole
// runs of its columns per stage (256 or 512 contiguous bytes: every line used once); an NT
// operand's 64-byte pieces share lines with the next stage, so NT keeps the default policy.
template <int MODE, int EPI, bool FP8, int BM, int BN, int WM, int WN, int STAGES, int BKB_,
          bool BNT = false>
__global__ __launch_bounds__(WM* WN * 64, 1) void grouped_gemm_kernel(const GemmParams p) {
  using C = Cfg<BM, BN, WM, WN, STAGES, BKB_>;
  static_assert(!BNT || MODE == MOE_GEMM_NN, "non-temporal weight loads: NN only");
  constexpr int BKB = C::BKB, KR = C::KR;
  constexpr int LEAD = STAGES - 1;  // stages in flight ahead of the one being multiplied
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");
  // The LDS ring: stream stage s lives in buffer s % STAGES. The DMA writes are issued from
  // inline asm, so the compiler's own LDS-DMA tracking never serialises reads behind them.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::SMEM];
  __shared__ int s_pref[264];  // NN/NT: prefix of the per-group M-tile counts
  __shared__ int s_off[264];   // offsets[0..G]
  // per-wave epilogue staging: 32 rows of SB bytes (128 when it fits the LDS budget)
  constexpr int SB = C::SMEM + 2 * 264 * 4 + 64 + C::NW * 4096 <= 160 * 1024 &&
                             (EPI == EPI_SWIGLU ? (C::NB / 2) % 2 == 0 : C::NB % 2 == 0)
                         ? 128 : 64;
  __shared__ __attribute__((aligned(16))) uint8_t s_epi[C::NW * 32 * SB];
  __shared__ int s_tk[8];      // published tile tickets
  // e4m3: each tile's row and column scales, DMA'd when the load cursor reaches the tile
  // (so they land before its first stage is read), one slot per tile the cursor can be ahead
  constexpr int SC_SLOTS = LEAD + 1;
  __shared__ __attribute__((aligned(16))) float s_fsc[FP8 ? SC_SLOTS : 1][FP8 ? BM + BN : 1];
  static_assert(EPI != EPI_SWIGLU || C::NB % 2 == 0, "SwiGLU wave tile: gate blocks + as many up blocks");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases stay scalar
  const int wm = wave / WN, wn = wave % WN;
  constexpr bool DW = MODE == MOE_GEMM_TN_DW;
  constexpr bool B_MN = (MODE == MOE_GEMM_NN) || DW;  // B tile M/N-contiguous in memory
  constexpr int HB = BN / 2;                           // SwiGLU: h columns per tile
  const int ntn = EPI == EPI_SWIGLU ? (p.I + HB - 1) / HB : (p.N + BN - 1) / BN;
  // split-K is built for the 32-row bf16 tiles (decode) only
  constexpr bool SPLITK = !DW && !FP8 && BM == 32 && EPI != EPI_SWIGLU_BWD &&
                          (MOE_GEMM_SPLITK & (EPI == EPI_SWIGLU ? 1 : 2)) != 0;
  const int esz = FP8 ? 1 : 2;
  const size_t lda = (size_t)p.K * esz;
  const int nk_fixed = DW ? 0 : (int)(lda / BKB);  // NN/NT: K stages of a whole tile

  // ---- group offsets and tile count ----------------------------------------------
  // no offsets: G groups split the rows evenly (split-K weight gradients)
  for (int g = tid; g <= p.G; g += C::NT)
    s_off[g] = p.offsets ? p.offsets[g] : (int)((long long)g * p.rows / p.G);
  __syncthreads();
  int total;
  if constexpr (!DW) {
    if (wave == 0) {
      const int per = (p.G + 63) / 64;
      int loc[5];
      int sum = 0;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int g = lane * per + i;
        int mt = 0;
        if (i < per && g < p.G) mt = (s_off[g + 1] - s_off[g] + BM - 1) / BM;
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
  total = __builtin_amdgcn_readfirstlane(total);
  // split-K: ksn copies of the tile range, one per K part (part-major, so the blocks that
  // run at the same time read neighbouring weight columns over the same K rows). With one
  // part the tiles write their outputs themselves and the second launch does nothing.
  int ksn = 1;
  const int base_total = total;
  if (SPLITK && p.part != nullptr) {
    ksn = choose_ksplit(total, (int)gridDim.x, nk_fixed);
    ksn = __builtin_amdgcn_readfirstlane(ksn);
    total *= ksn;
    if (blockIdx.x == 0 && tid == 0) *p.part_s = ksn;
  }
  const bool split = SPLITK && ksn > 1;

  // ---- this block's tiles ------------------------------------------------------------
  // The grid is persistent. Tiles are ordered (group, N-tile, M-tile); blocks are handed
  // out round-robin over the 8 XCDs, so XCD x serves the x-th eighth of the tile range and
  // neighbours that share weight panels run at the same time on one XCD (one L2).
  // NN/NT (ragged rows, uneven tile costs): each XCD's blocks take tickets from its own
  // counter as they free up. A block holds three tickets at start (from its index); at the
  // end of each epilogue wave 0 publishes the ticket requested one tile earlier (so the
  // atomic's latency is never waited for) and requests the next.
  // Weight gradients (equal tiles): a fixed stride through the XCD's eighth.
  constexpr bool DYN = !DW;
  const int nx = (gridDim.x & 7) == 0 ? 8 : 1;
  const int xcd = nx == 8 ? (int)(blockIdx.x & 7) : 0;
  int r_start, r_end;
  {
    const int base = total / nx, rem = total % nx;
    r_start = xcd * base + (xcd < rem ? xcd : rem);
    r_end = r_start + base + (xcd < rem ? 1 : 0);
  }
  const int seq_first = r_start + (int)(blockIdx.x / nx), seq_stride = (int)gridDim.x / nx;
  int* const sched = p.sched ? p.sched : g_sched[p.sched_slot];
  int* const ctr = &sched[xcd];
  int n_pub = 0x40000000;     // tickets published in s_tk (a ring of 8); unbounded when static
  bool sched_open = false;    // later tickets may still hold tiles
  int pend_tk = 0;            // wave 0 holds a requested, unpublished ticket
  int tk = 0;                 // wave 0, lane 0: that ticket
  if constexpr (DYN) {
    // The three starting tickets follow the block index (blocks are spread over the CUs in
    // index order, so the first tiles are too); later tickets come from the counter, past
    // the 3 BX starting ones.
    if (tid == 0) {
      const int t0 = 3 * (int)(blockIdx.x / nx);
      s_tk[0] = t0;
      s_tk[1] = t0 + 1;
      s_tk[2] = t0 + 2;
#pragma unroll
      for (int i = 3; i < 8; ++i) s_tk[i] = 0x40000000;  // never a tile
    }
    __syncthreads();
    n_pub = 3;
    // tickets past the first 3 BX map to themselves: more grabs pay off while they can
    // still land inside the range
    sched_open = 3 * ((int)gridDim.x / nx) < r_end - r_start;
  }
  // The sequence ends at the first index without a tile; past the published tickets there
  // is none (a block whose last published ticket is valid stops there).
  auto tile_of = [&](int j) __attribute__((always_inline)) -> int {
    int t;
    if constexpr (DYN) {
      if (j >= n_pub) return -1;
      // The first 3*BX tickets of an XCD (three per block, taken at start) are spread so
      // that blocks start on consecutive tiles, and a range shorter than 3 BX still gives
      // every block its share: ticket 3i+k -> tile i + BX*k. Later tickets map to
      // themselves.
      const int BX = (int)gridDim.x / nx;
      t = s_tk[j & 7];
      if (t < 3 * BX) t = t / 3 + BX * (t % 3);  // a bijection of [0, 3 BX)
      t += r_start;
      t = t < r_end ? t : -1;
    } else {
      t = seq_first + j * seq_stride;
      t = t < r_end ? t : -1;
    }
    return __builtin_amdgcn_readfirstlane(t);
  };
  // Tile fields from the tile index (LDS reads only: no global loads while DMAs fly).
  auto decode = [&](int tile) __attribute__((always_inline)) -> Tile {
    Tile t;
    if constexpr (!DW) {
      int ks = 0;
      if (SPLITK && ksn > 1) {
        ks = tile / base_total;
        tile -= ks * base_total;
      }
      t.ks = ks;
      t.kst0 = ks * nk_fixed / ksn;
      t.nst = (ks + 1) * nk_fixed / ksn - t.kst0;
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
      const int gbeg = s_off[g], cnt = s_off[g + 1] - gbeg;
      // the group's rows are spread evenly over its M tiles (in 32-row steps), so a group a
      // little over BM rows takes two part tiles rather than a full one and a sliver
      const int per = ((cnt + mt - 1) / mt + 31) & ~31;
      t.g = g;
      t.m0 = gbeg + mtile * per;
      t.rows_valid = min(per, cnt - mtile * per);
      t.n0 = ntile * (EPI == EPI_SWIGLU ? HB : BN);
      t.kcount = p.K;
      t.kbase = gbeg;
    } else {
      const int mtn = (p.M + BM - 1) / BM;
      const int g = tile / (mtn * ntn), rem = tile % (mtn * ntn);
      t.g = g;
      t.m0 = (rem / ntn) * BM;
      t.n0 = (rem % ntn) * BN;
      t.rows_valid = BM;
      t.kbase = s_off[g];
      t.kcount = s_off[g + 1] - t.kbase;
    }
    t.g = __builtin_amdgcn_readfirstlane(t.g);
    t.m0 = __builtin_amdgcn_readfirstlane(t.m0);
    t.n0 = __builtin_amdgcn_readfirstlane(t.n0);
    t.rows_valid = __builtin_amdgcn_readfirstlane(t.rows_valid);
    t.kcount = __builtin_amdgcn_readfirstlane(t.kcount);
    t.kbase = __builtin_amdgcn_readfirstlane(t.kbase);
    if constexpr (!DW) {
      t.ks = __builtin_amdgcn_readfirstlane(t.ks);
      t.kst0 = __builtin_amdgcn_readfirstlane(t.kst0);
      t.nst = __builtin_amdgcn_readfirstlane(t.nst);
    }
    return t;
  };

  // The last group's own A, weight and C tensors (a dense shared expert), when given.
  auto last_group = [&](const Tile& t) __attribute__((always_inline)) {
    return !DW && p.A_last != nullptr && t.g == p.G - 1;
  };
  auto c_base = [&](const Tile& t) __attribute__((always_inline)) -> const uint16_t* {
    return (const uint16_t*)(last_group(t) ? p.C_last : p.C);
  };
  auto c_row = [&](const Tile& t) __attribute__((always_inline)) -> size_t {
    return (size_t)(last_group(t) ? t.m0 - t.kbase : t.m0);
  };

  // ---- load descriptors: a global pointer per 1 KB chunk-load, advanced per stage ----
  const uint8_t* zero = g_zero_block;
  const uint32_t lda32 = (uint32_t)lda;
  size_t a_step, b_step;  // bytes per stage
  if constexpr (!DW) {
    a_step = BKB;
    b_step = B_MN ? (size_t)KR * p.N * 2 : (size_t)BKB;
  } else {
    a_step = (size_t)KR * p.M * 2;
    b_step = (size_t)KR * p.N * 2;
  }
  auto stages_of = [&](const Tile& t) __attribute__((always_inline)) {
    return DW ? (t.kcount + KR - 1) / KR : t.nst;
  };
  // NN/NT: a wave-uniform base per operand (stage lk at base + lk * step) and a 32-bit byte
  // offset per lane and chunk-load (the host keeps one expert's operands under 4 GiB).
  // DW: full pointers plus the stage index.
  const uint8_t* a_base = nullptr;
  const uint8_t* b_base = nullptr;
  uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
  const uint8_t* a_src[DW ? C::A_LOADS : 1];
  const uint8_t* b_src[DW ? C::B_LOADS : 1];
  int a_krow[C::A_LOADS], b_krow[C::B_LOADS];  // DW: k row of the chunk lane (zero past kcount)
  auto setup_loads = [&](const Tile& t) __attribute__((always_inline)) {
    if constexpr (!DW) {
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i) {
        const int chunk = wave + C::NW * i;
        const int row = kc_row<BKB>(chunk, lane);
        const bool ok = row < t.rows_valid;
        // rows past the group's end read the tile's first row: they only feed output rows
        // that are never stored
        a_off[i] = (uint32_t)(ok ? row : 0) * lda32 + kc_logical<BKB>(row, lane) * 16;
        a_krow[i] = 0;
      }
      const bool lastg = last_group(t);
      a_base = lastg ? (const uint8_t*)p.A_last + (size_t)(t.m0 - t.kbase) * lda
                     : (const uint8_t*)p.A + (size_t)t.m0 * lda;
      if constexpr (!B_MN) {  // NT: B_g is [N, K]
        const uint8_t* bg = lastg ? (const uint8_t*)p.B_last : (const uint8_t*)p.B + (size_t)t.g * p.N * lda;
        b_base = bg;
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i) {
          const int chunk = wave + C::NW * i;
          const int row = kc_row<BKB>(chunk, lane);
          int col;
          bool ok;
          if (EPI == EPI_SWIGLU) {
            const int hcol = t.n0 + (row < HB ? row : row - HB);
            col = row < HB ? hcol : p.I + hcol;
            ok = hcol < p.I;
          } else {
            col = t.n0 + row;
            ok = col < p.N;
          }
          // columns past the end read the tile's first column (outputs never stored)
          b_off[i] = (uint32_t)(ok ? col : t.n0) * lda32 + kc_logical<BKB>(row, lane) * 16;
          b_krow[i] = 0;
        }
      } else {  // NN: B_g is [K, N]
        const uint8_t* bg = lastg ? (const uint8_t*)p.B_last : (const uint8_t*)p.B + (size_t)t.g * p.K * p.N * 2;
        b_base = bg;
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
          b_off[i] = ((uint32_t)k * p.N + (ok ? col : t.n0)) * 2u;
          b_krow[i] = 0;
        }
      }
      if constexpr (SPLITK) {  // the tile's K part starts kst0 stages in
        a_base += (size_t)t.kst0 * a_step;
        b_base += (size_t)t.kst0 * b_step;
      }
    } else {
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
  };

  // e4m3: the tile's BM row scales and BN column scales (in B-tile row order: for SwiGLU
  // the gate columns, then the up columns) into slot j % SC_SLOTS, 64 values per
  // wave-uniform DMA; rows and columns past the tile's valid ones read the zero block (their
  // outputs are never stored).
  auto issue_scales = [&](const Tile& t, int j) __attribute__((always_inline)) {
    if constexpr (FP8) {
      static_assert((BM + BN) % 64 == 0, "whole 64-value scale DMAs");
      constexpr int PARTS = (BM + BN) / 64;
      float* slot = s_fsc[j % SC_SLOTS];
      for (int part = wave; part < PARTS; part += C::NW) {
        const int idx = part * 64 + lane;
        const void* src = zero;
        if (idx < BM) {
          if (idx < t.rows_valid) src = p.a_scale + t.m0 + idx;
        } else {
          const int r = idx - BM;
          if (EPI == EPI_SWIGLU) {
            const int hcol = t.n0 + (r < HB ? r : r - HB);
            if (hcol < p.I) src = p.b_scale + (size_t)t.g * (2 * p.I) + (r < HB ? hcol : p.I + hcol);
          } else {
            const int col = t.n0 + r;
            if (col < p.N) src = p.b_scale + (size_t)t.g * p.N + col;
          }
        }
        load_lds4(src, (uint8_t*)(slot + part * 64));
      }
    }
  };

  // ---- load cursor: walks this block's tiles ahead of the multiply ---------------------
  Tile lt;              // tile whose stages are being loaded
  int lj = -1;          // its index in this block's sequence
  int lk = 0, lnk = 0;  // next stage to load, stages of the tile
  // Cursor state, one variable (separate flags end up in scratch memory once the compiler
  // merges their stores): a stage is available to load, the next tile's ticket is not
  // published yet, or the block's tiles are all loaded.
  enum { L_END = 0, L_LIVE = 1, L_BLOCKED = 2 };
  int l_state = L_END;
  auto cursor_advance = [&]() __attribute__((always_inline)) {
    int st = L_END;
    for (;;) {
      if (lj + 1 >= n_pub) {
        st = L_BLOCKED;
        break;
      }
      ++lj;
      const int tl = tile_of(lj);
      if (tl < 0) break;
      lt = decode(tl);
      lnk = stages_of(lt);
      lk = 0;
      if (lnk > 0) {
        setup_loads(lt);
        issue_scales(lt, lj);
        st = L_LIVE;
        break;
      }
    }
    l_state = __builtin_amdgcn_readfirstlane(st);
  };
  // Load slot i < LOADS of the cursor's stage lk: A chunk-loads first, then B.
  auto issue_one = [&](uint8_t* sa, int i) __attribute__((always_inline)) {
    if (i < C::A_LOADS) {
      uint8_t* dst = sa + (wave + C::NW * i) * 1024;
      if constexpr (DW) {
        load_lds16((lk * KR + a_krow[i] < lt.kcount) ? a_src[i] + (size_t)lk * a_step : zero, dst);
      } else {
        load_lds16_s(a_base + (size_t)lk * a_step, a_off[i], dst);
      }
    } else {
      const int j = i - C::A_LOADS;
      uint8_t* dst = sa + C::A_BYTES + (wave + C::NW * j) * 1024;
      if constexpr (DW) {
        load_lds16((lk * KR + b_krow[j] < lt.kcount) ? b_src[j] + (size_t)lk * b_step : zero, dst);
      } else {
        if constexpr (BNT) load_lds16_s_nt(b_base + (size_t)lk * b_step, b_off[j], dst);
        else load_lds16_s(b_base + (size_t)lk * b_step, b_off[j], dst);
      }
    }
  };

  // ---- fragments ----------------------------------------------------------------------
  // The MFMA takes the B fragment as its first operand, so each accumulator block holds
  // C^T: lane l, element v -> output row l%32 of the block, output column
  // 8*(v/4) + 4*(l/32) + v%4. Each lane thus owns runs of 4 consecutive output columns,
  // which the epilogue writes straight from registers.
  f32x16_t acc[C::MB][C::NB];

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
  using frag_t = typename std::conditional<FP8, i32x8_t, bf16x8_t>::type;
  // A fragment of M block i of this wave, k sub-step ks.
  auto load_a = [&](const uint8_t* sa, int ks, int i) __attribute__((always_inline)) -> frag_t {
    const int r0 = (wm + WM * i) * 32;
    if constexpr (FP8) {
      const u32x4_t x0 = kc_frag(sa, r0 + l32, ks * 4 + khalf * 2);
      const u32x4_t x1 = kc_frag(sa, r0 + l32, ks * 4 + khalf * 2 + 1);
      return i32x8_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                     (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    } else if constexpr (!DW) {
      return __builtin_bit_cast(bf16x8_t, kc_frag(sa, r0 + l32, ks * 2 + khalf));
    } else {
      const int k = ks * 16 + tr_k;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(sa + mn_offset<BM>(k, r0 + tr_c)));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(sa + mn_offset<BM>(k + 4, r0 + tr_c)));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  // B fragments of this wave's N blocks, k sub-step ks.
  auto load_b = [&](const uint8_t* sa, int ks, frag_t* bfr) __attribute__((always_inline)) {
    const uint8_t* sb = sa + C::A_BYTES;
#pragma unroll
    for (int j = 0; j < C::NB; ++j) {
      const int c0 = bcol0(j);
      if constexpr (FP8) {
        const u32x4_t x0 = kc_frag(sb, c0 + l32, ks * 4 + khalf * 2);
        const u32x4_t x1 = kc_frag(sb, c0 + l32, ks * 4 + khalf * 2 + 1);
        bfr[j] = i32x8_t{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                         (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      } else if constexpr (!B_MN) {
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
  };
  // Fragment loads of k sub-step ks into registers.
  auto load_frags = [&](auto MBL_c, const uint8_t* sa, int ks, auto& af, auto& bfr) __attribute__((always_inline)) {
    constexpr int MBL = decltype(MBL_c)::value;
#pragma unroll
    for (int i = 0; i < MBL; ++i) af[i] = load_a(sa, ks, i);
    load_b(sa, ks, bfr);
  };
  auto mfma1 = [&](int i, int j, const frag_t& a, const frag_t& b) __attribute__((always_inline)) {
    if constexpr (!FP8)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc[i][j], 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, acc[i][j], 0, 0, 0, 127, 0, 127);
  };
  auto mfmas = [&](auto MBL_c, const auto& af, const auto& bfr) __attribute__((always_inline)) {
    constexpr int MBL = decltype(MBL_c)::value;
#pragma unroll
    for (int i = 0; i < MBL; ++i)
#pragma unroll
      for (int j = 0; j < C::NB; ++j) mfma1(i, j, af[i], bfr[j]);
  };
  // One ring stage: KS k sub-steps; while sub-step ks multiplies, the fragments of ks+1
  // are read and a slice of the cursor's next stage (into `nxt`) is issued.
  // Five M blocks per wave, or e4m3 fragments (8 registers each) with eight waves, leave no
  // room for a whole sub-step of A fragments in flight: there A fragments are read one M
  // block ahead of the multiply instead. The weight gradients take the same order (measured
  // 3 % faster than reading the whole next sub-step ahead; their fragments come from
  // transposing LDS reads).
  constexpr bool APIPE = C::MB >= 5 || (FP8 && C::NW == 8) || DW;
  auto compute_stage = [&](auto MBL_c, const uint8_t* sa, bool iss, uint8_t* nxt) __attribute__((always_inline)) {
    constexpr int KS = FP8 ? BKB / 64 : BKB / 32;
    constexpr int PER = (C::LOADS + KS - 1) / KS;
    // e4m3 (one sub-step per stage): the next stage's loads go out between the M blocks'
    // multiplies rather than together (measured 1.5-2.5 % faster there, 1-3 % slower on the
    // bf16 tiles)
    constexpr bool SPREAD = FP8;
    if constexpr (APIPE) {
      constexpr int MBL = decltype(MBL_c)::value;
      frag_t af[2], bfr[2][C::NB];
      load_b(sa, 0, bfr[0]);
      if constexpr (MBL > 0) af[0] = load_a(sa, 0, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) load_b(sa, ks + 1, bfr[(ks + 1) & 1]);
        if (iss && !(SPREAD && MBL > 0)) {
#pragma unroll
          for (int q = ks * PER; q < (ks + 1) * PER && q < C::LOADS; ++q) issue_one(nxt, q);
        }
#pragma unroll
        for (int i = 0; i < MBL; ++i) {
          if (SPREAD && iss) {
#pragma unroll
            for (int j = 0; j < PER; ++j)
              if (j * MBL / PER == i && ks * PER + j < C::LOADS) issue_one(nxt, ks * PER + j);
          }
          const int f = ks * MBL + i;  // fragment f sits in af[f & 1]
          if (i + 1 < MBL) af[(f + 1) & 1] = load_a(sa, ks, i + 1);
          else if (ks + 1 < KS) af[(f + 1) & 1] = load_a(sa, ks + 1, 0);
          // keep the read of the next fragment ahead of this block's multiplies: left
          // alone, the scheduler sinks it below them into the same registers, and every
          // pair of multiplies then waits for a read issued just before it
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < C::NB; ++j) mfma1(i, j, af[f & 1], bfr[ks & 1][j]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      return;
    }
    frag_t af[2][C::MB], bfr[2][C::NB];
    load_frags(MBL_c, sa, 0, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) load_frags(MBL_c, sa, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
      if (iss) {
#pragma unroll
        for (int q = ks * PER; q < (ks + 1) * PER && q < C::LOADS; ++q) issue_one(nxt, q);
      }
      mfmas(MBL_c, af[ks & 1], bfr[ks & 1]);
    }
  };

  // ---- epilogue: per-wave staging, 16-byte row stores -------------------------------
  // Each wave owns an LDS area outside the ring of 32 rows x SB bytes (SB = 128 when the
  // budget allows: two 32-column bf16 blocks side by side, so every store covers whole
  // 128-byte lines; else 64). Values go in as 8- or 16-byte pieces from the C^T layout, the
  // 16-byte chunk index XORed with a row function so both the writes and the row reads are
  // conflict-free, and come back as 16 consecutive bytes of one row per lane. Only this
  // wave touches its area and LDS accesses of a wave complete in order: no barrier needed.
  uint8_t* stg = s_epi + wave * (32 * SB);
  constexpr int LPR = SB / 16, RPI = 64 / LPR, NRI = 32 / RPI;  // lanes/row, rows/read, reads
  constexpr int PB = SB / 64;                                   // bf16 blocks per group
  auto stg_addr = [&](int r, int chunk) __attribute__((always_inline)) -> uint8_t* {
    const int sw = SB == 128 ? (r >> 1) & 7 : (r >> 2) & 3;
    return stg + r * SB + ((chunk ^ sw) << 4);
  };
  // Store instructions per wave and epilogue (bf16 output; SwiGLU without / with g,u),
  // the same for every tile: masked lanes store out of range instead of branching.
  constexpr int NH_ = EPI == EPI_SWIGLU ? C::NB / 2 : 1;
  constexpr int S_STORE = C::MB * (C::NB / PB) * NRI;
  constexpr int S_SWIGLU = C::MB * (NH_ / PB) * NRI;
  constexpr int S_SWIGLU_GU = 3 * S_SWIGLU;
  constexpr int S1 = EPI == EPI_SWIGLU ? S_SWIGLU : S_STORE;
  constexpr int S2 = EPI == EPI_SWIGLU ? S_SWIGLU_GU : S_STORE;
  static_assert((EPI == EPI_SWIGLU ? NH_ : C::NB) % PB == 0, "staging groups");
  auto epilogue = [&](const Tile& t, int sc) __attribute__((always_inline)) {  // sc: scale slot
    // Lane-derived row and column parts, made opaque so the address arithmetic below is
    // not hoisted out of the tile loop (where it would sit in registers the whole time).
    int l32 = lane & 31, kh = lane >> 5, rr = lane / LPR, cc = lane % LPR;
    asm volatile("" : "+v"(l32), "+v"(kh), "+v"(rr), "+v"(cc));
    // Stage a group of PB bf16 blocks (`val(b, q)`: the packed values of block b, 4-column
    // run q) and store its 32 rows of PB*32 columns.
    auto group_bf16 = [&](auto val, auto row_ok, auto col_ok, auto offset, const __amdgpu_buffer_rsrc_t& rs)
        __attribute__((always_inline)) {
#pragma unroll
      for (int b = 0; b < PB; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int piece = 8 * b + 2 * q + kh;  // 8-byte piece of the staged row
          *(u32x2_t*)(stg_addr(l32, piece >> 1) + (piece & 1) * 8) = val(b, q);
        }
#pragma unroll
      for (int h = 0; h < NRI; ++h) {
        const int r = rr + RPI * h;
        const u32x4_t v = *(const u32x4_t*)stg_addr(r, cc);
        const bool ok = row_ok(r) && col_ok(8 * cc);
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, ok ? offset(r, 8 * cc) : kOutOfRange, 0, 0);
      }
    };
    // Stage one fp32 block in 128 / SB passes of SB/4 columns; `use(r, c, v)` gets row r,
    // first column c and the 4 values of each lane's 16-byte piece.
    auto block_f32 = [&](const f32x16_t& a, auto use) __attribute__((always_inline)) {
      constexpr int NP = 128 / SB, QP = 4 / NP;  // passes, 4-column runs per pass
#pragma unroll
      for (int ps = 0; ps < NP; ++ps) {
#pragma unroll
        for (int q = ps * QP; q < ps * QP + QP; ++q)
          *(u32x4_t*)stg_addr(l32, 2 * (q - ps * QP) + kh) =
              u32x4_t{__float_as_uint(a[4 * q]), __float_as_uint(a[4 * q + 1]),
                      __float_as_uint(a[4 * q + 2]), __float_as_uint(a[4 * q + 3])};
#pragma unroll
        for (int h = 0; h < NRI; ++h) {
          const int r = rr + RPI * h;
          use(ps * NRI + h, r, ps * (SB / 4) + 4 * cc, *(const u32x4_t*)stg_addr(r, cc));
        }
      }
    };
    if constexpr (SPLITK) {
      if (split) {
        // this K part's fp32 sums of the tile's valid rows and columns, into part ks laid
        // out [rows, pc] (SwiGLU: the gate columns, then the up columns from I on)
        const int pc = EPI == EPI_SWIGLU ? 2 * p.I : p.N;
        const auto pr = tile_rsrc(p.part + ((size_t)t.ks * p.rows + t.m0) * pc);
#pragma unroll
        for (int i = 0; i < C::MB; ++i) {
          const int r0 = (wm + WM * i) * 32;
#pragma unroll
          for (int j = 0; j < C::NB; ++j) {
            const int c0 = bcol0(j);  // first column of the block within the tile
            // the block's first output column (SwiGLU: h column) and where it goes in part
            const int oc = t.n0 + (EPI == EPI_SWIGLU && c0 >= HB ? c0 - HB : c0);
            const int lim = EPI == EPI_SWIGLU ? p.I : p.N;
            const int pcol = EPI == EPI_SWIGLU && c0 >= HB ? p.I + oc : oc;
            block_f32(acc[i][j], [&](int, int r, int c, u32x4_t x) {
              const bool ok = r0 + r < t.rows_valid && oc + c < lim;
              __builtin_amdgcn_raw_buffer_store_b128(x, pr, ok ? ((r0 + r) * pc + pcol + c) * 4 : kOutOfRange,
                                                     0, 0);
            });
          }
        }
        return;
      }
    }
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int NH = C::NB / 2;
      const int twoI = 2 * p.I;
      const auto hr = tile_rsrc(c_base(t) + c_row(t) * p.I + t.n0);
      const auto gr = tile_rsrc(p.gu_out ? (const uint16_t*)p.gu_out + (size_t)t.m0 * twoI + t.n0
                                         : (const uint16_t*)p.C);
      const bool scaled = !FP8 && p.row_scale != nullptr && !last_group(t);
#pragma unroll
      for (int i = 0; i < C::MB; ++i) {
        const int r0 = (wm + WM * i) * 32;
        float sa = 1.f;
        if (FP8) sa = s_fsc[sc][r0 + l32];
        // ScaledSwiGLU: the routing weight of this lane's row (lane l holds row l % 32)
        float rs = 1.f;
        if (scaled) rs = p.row_scale[t.m0 + (r0 + l32 < t.rows_valid ? r0 + l32 : 0)];
        auto row_ok = [&](int r) { return r0 + r < t.rows_valid; };
#pragma unroll
        for (int jg0 = 0; jg0 < NH; jg0 += PB) {
          const int hb = (wn * NH + jg0) * 32;  // first h column of the group within the tile
          auto col_ok = [&](int c) { return t.n0 + hb + c < p.I; };
          float g[PB][16], u[PB][16];
#pragma unroll
          for (int b = 0; b < PB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              g[b][v] = acc[i][jg0 + b][v];
              u[b][v] = acc[i][jg0 + b + NH][v];
            }
          if (FP8) {
            const float* bs = &s_fsc[sc][BM];  // gate columns, then HB up columns
#pragma unroll
            for (int b = 0; b < PB; ++b)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int c = hb + 32 * b + 8 * q + 4 * kh;  // h column within the tile
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  g[b][4 * q + r] *= sa * bs[c + r];
                  u[b][4 * q + r] *= sa * bs[HB + c + r];
                }
              }
          }
          group_bf16([&](int b, int q) {
                       float hv[4];
#pragma unroll
                       for (int r = 0; r < 4; ++r) {
                         const float gg = g[b][4 * q + r];
                         hv[r] = gg * sigmoid_fast(gg) * u[b][4 * q + r];
                         if (scaled) hv[r] *= rs;
                       }
                       return u32x2_t{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
                     },
                     row_ok, col_ok, [&](int r, int c) { return ((r0 + r) * p.I + hb + c) * 2; }, hr);
          if (p.gu_out) {
            group_bf16([&](int b, int q) {
                         return u32x2_t{pack_bf16x2(g[b][4 * q], g[b][4 * q + 1]),
                                        pack_bf16x2(g[b][4 * q + 2], g[b][4 * q + 3])};
                       },
                       row_ok, col_ok, [&](int r, int c) { return ((r0 + r) * twoI + hb + c) * 2; }, gr);
            group_bf16([&](int b, int q) {
                         return u32x2_t{pack_bf16x2(u[b][4 * q], u[b][4 * q + 1]),
                                        pack_bf16x2(u[b][4 * q + 2], u[b][4 * q + 3])};
                       },
                       row_ok, col_ok, [&](int r, int c) { return ((r0 + r) * twoI + p.I + hb + c) * 2; }, gr);
          }
        }
      }
    } else if constexpr (EPI == EPI_SWIGLU_BWD) {
      // acc = dh[m, hcol] (fp32); with s = sigmoid(g): dgu[m] = [dh u s (1 + g (1 - s)), dh g s]
      const int twoI = 2 * p.I;
      const size_t org = (size_t)t.m0 * twoI + t.n0;
      const auto dr = tile_rsrc((const uint16_t*)p.C + org);
      const auto gi = tile_rsrc((const uint16_t*)p.gu_in + org);
      // ScaledSwiGLU: dh of the scaled h is multiplied by the row's weight before the SwiGLU
      // backward, and the weight's gradient sum_c dh silu(g) u is accumulated per row over
      // this wave's 64 columns (one partial per row and 64-column block)
      const bool scaled = p.row_scale != nullptr;
      const bool parts = p.row_part != nullptr;
      static_assert(C::TN == 64, "one 64-column block of partials per wave");
#pragma unroll
      for (int i = 0; i < C::MB; ++i) {
        const int r0 = (wm + WM * i) * 32;
        float rsv[NRI], part[NRI];
#pragma unroll
        for (int h = 0; h < NRI; ++h) {
          const int r = rr + RPI * h;
          rsv[h] = scaled ? p.row_scale[t.m0 + (r0 + r < t.rows_valid ? r0 + r : 0)] : 1.f;
          part[h] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
          const int c0 = bcol0(j);
          // the saved g,u of the block's lanes, loaded up front (latency paid once per block)
          constexpr int NPIECE = (128 / SB) * NRI;
          int go[NPIECE], uo[NPIECE];
          u32x2_t gv[NPIECE], uv[NPIECE];
#pragma unroll
          for (int x = 0; x < NPIECE; ++x) {
            const int r = rr + RPI * (x % NRI);
            const int c = (x / NRI) * (SB / 4) + 4 * cc;
            const bool ok = r0 + r < t.rows_valid && t.n0 + c0 + c < p.N;
            go[x] = ok ? ((r0 + r) * twoI + c0 + c) * 2 : kOutOfRange;
            uo[x] = ok ? go[x] + p.I * 2 : kOutOfRange;
            gv[x] = __builtin_amdgcn_raw_buffer_load_b64(gi, go[x], 0, 0);
            uv[x] = __builtin_amdgcn_raw_buffer_load_b64(gi, uo[x], 0, 0);
          }
          block_f32(acc[i][j], [&](int x, int, int, u32x4_t dv) {
            float dg[4], du[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t gw = gv[x][e >> 1], uw = uv[x][e >> 1];
              const float gg = (e & 1) ? bf16hi(gw) : bf16lo(gw);
              const float uu = (e & 1) ? bf16hi(uw) : bf16lo(uw);
              const float dhs = __uint_as_float(dv[e]);
              const float sg = sigmoid_fast(gg);
              if (parts) part[x % NRI] = fmaf(dhs, gg * sg * uu, part[x % NRI]);
              const float dh = scaled ? dhs * rsv[x % NRI] : dhs;
              dg[e] = dh * uu * sg * (1.0f + gg * (1.0f - sg));
              du[e] = dh * gg * sg;
            }
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])},
                                                  dr, go[x], 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])},
                                                  dr, uo[x], 0, 0);
          });
        }
        if (parts) {
          // the LPR lanes of a row group hold its row's pieces: sum them (fixed xor order),
          // then the group's first lane stores the row's partial of this 64-column block
          const int slot = (t.n0 + wn * C::TN) / 64, P = p.I / 64;
#pragma unroll
          for (int h = 0; h < NRI; ++h) {
            float v = part[h];
#pragma unroll
            for (int o = 1; o < LPR; o <<= 1) v += __shfl_xor(v, o, 64);
            const int r = rr + RPI * h;
            if (cc == 0 && r0 + r < t.rows_valid && t.n0 + wn * C::TN < p.I)
              p.row_part[(size_t)(t.m0 + r0 + r) * P + slot] = v;
          }
        }
      }
    } else {
      const int mlim = DW ? p.M - t.m0 : t.rows_valid;
      const size_t org = DW ? (size_t)t.g * p.M * p.N + (size_t)t.m0 * p.N + t.n0
                            : c_row(t) * p.N + t.n0;
#pragma unroll
      for (int i = 0; i < C::MB; ++i) {
        const int r0 = (wm + WM * i) * 32;
        float sa = 1.f;
        if (FP8) sa = s_fsc[sc][r0 + l32];
        auto row_ok = [&](int r) { return r0 + r < mlim; };
        float v[C::NB][16];
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
#pragma unroll
          for (int e = 0; e < 16; ++e) v[j][e] = acc[i][j][e];
          if (FP8) {
            const int c0 = bcol0(j);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float* bs = &s_fsc[sc][BM + c0 + 8 * q + 4 * kh];
#pragma unroll
              for (int r = 0; r < 4; ++r) v[j][4 * q + r] *= sa * bs[r];
            }
          }
        }
        if (p.c_fp32) {
          const auto cr = tile_rsrc((const float*)(const void*)c_base(t) + org);
#pragma unroll
          for (int j = 0; j < C::NB; ++j) {
            const int c0 = bcol0(j);
            f32x16_t a;
#pragma unroll
            for (int e = 0; e < 16; ++e) a[e] = v[j][e];
            block_f32(a, [&](int, int r, int c, u32x4_t x) {
              const bool ok = row_ok(r) && t.n0 + c0 + c < p.N;
              __builtin_amdgcn_raw_buffer_store_b128(x, cr, ok ? ((r0 + r) * p.N + c0 + c) * 4 : kOutOfRange, 0, 0);
            });
          }
        } else {
          const auto cr = tile_rsrc(c_base(t) + org);
#pragma unroll
          for (int j0 = 0; j0 < C::NB; j0 += PB) {
            const int c0 = bcol0(j0);
            auto col_ok = [&](int c) { return t.n0 + c0 + c < p.N; };
            group_bf16([&](int b, int q) {
                         return u32x2_t{pack_bf16x2(v[j0 + b][4 * q], v[j0 + b][4 * q + 1]),
                                        pack_bf16x2(v[j0 + b][4 * q + 2], v[j0 + b][4 * q + 3])};
                       },
                       row_ok, col_ok, [&](int r, int c) { return ((r0 + r) * p.N + c0 + c) * 2; }, cr);
          }
        }
      }
    }
  };

  // ---- the stage stream -----------------------------------------------------------------
  // Stream stages are numbered over all of this block's tiles: gs is the next stage to
  // multiply, gl the next to load, gl - gs <= LEAD. With `cross`, the cursor runs into the
  // next tile while the current one finishes, so the next tile's first stages are in flight
  // during the epilogue (whose stores then sit between those loads and their wait). The e4m3
  // scales of a tile are staged into LDS when the cursor reaches it, so those epilogues read
  // no global memory either. Without it (the SwiGLU backward, which reads h and the routing
  // weights) each tile starts with its own prologue after the previous epilogue.
  constexpr bool CROSS = EPI != EPI_SWIGLU_BWD;
  // (split-K epilogues only store fp32 partial sums: more stores than S1, S2 count, which
  // only makes the waits below wait longer)
  const bool cross = CROSS && (split || (!p.c_fp32 && !(EPI == EPI_SWIGLU && p.row_scale)));
  const int s_allow = (EPI == EPI_SWIGLU && p.gu_out) ? 2 : 1;
  auto buf = [&](int s) __attribute__((always_inline)) { return smem + (s % STAGES) * C::STAGE; };
  int gs = 0, gl = 0;
  int epi1 = -1, epi2 = -1;  // gl at the last two epilogues: stages below were loaded before their stores
  int cj = 0;
  auto run_tile = [&](auto MBL_c, int cnk) __attribute__((always_inline)) {
    for (int kt = 0; kt < cnk; ++kt) {
      const int pend = gl - gs - 1;  // stages loaded after this one
      const int allow = gs < epi2 ? 0 : (gs < epi1 ? s_allow : 0);
      wait_stage<C::LOADS, S1, S2>(pend, allow);
      ring_barrier();  // every wave's loads for stage gs landed; stage gs-1 fully read
      const bool iss = l_state == L_LIVE && (cross || lj == cj);
      compute_stage(MBL_c, buf(gs), iss, buf(gl));
      if (iss) {
        ++gl;
        if (++lk == lnk) cursor_advance();
      }
      ++gs;
    }
  };
  static_assert(C::MB <= 5, "live-block dispatch below covers up to five M blocks per wave");

  cursor_advance();
  for (;; ++cj) {
    const int tc = tile_of(cj);
    if (tc < 0) break;
    const Tile ct = decode(tc);
    const int cnk = stages_of(ct);
    // prologue: fill the ring up to LEAD stages ahead (a no-op while the stream is primed)
    while (l_state == L_LIVE && (cross || lj == cj) && gl < gs + LEAD) {
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) issue_one(buf(gl), i);
      ++gl;
      if (++lk == lnk) cursor_advance();
    }
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
      if ((wm + WM * i) * 32 < ct.rows_valid) mb_live = i + 1;
    mb_live = __builtin_amdgcn_readfirstlane(mb_live);
    // Every wave runs the stages: it issues its share of each stage's loads and takes part
    // in every barrier even when none of its M blocks holds a valid row (MBL = 0).
    switch (mb_live) {
      case 0: run_tile(std::integral_constant<int, 0>{}, cnk); break;
      case 1: run_tile(std::integral_constant<int, 1>{}, cnk); break;
      case 2: if constexpr (C::MB >= 2) run_tile(std::integral_constant<int, 2>{}, cnk); break;
      case 3: if constexpr (C::MB >= 3) run_tile(std::integral_constant<int, 3>{}, cnk); break;
      case 4: if constexpr (C::MB >= 4) run_tile(std::integral_constant<int, 4>{}, cnk); break;
      default: if constexpr (C::MB >= 5) run_tile(std::integral_constant<int, 5>{}, cnk); break;
    }
    epilogue(ct, cj % SC_SLOTS);
    epi2 = epi1;
    epi1 = gl;
    if constexpr (DYN) {
      if (wave == 0) {
        // this wave's stores and the ticket requested one epilogue ago have landed
        wait_vmcnt<0>();
        if (lane == 0) {
          // the counter value is kept as returned and offset only here, so nothing waits
          // for the atomic before this point
          if (pend_tk) s_tk[n_pub & 7] = 3 * ((int)gridDim.x / nx) + tk;
          if (sched_open) tk = atomicAdd(ctr, 1);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the ticket is in LDS before the barrier
      }
      if (pend_tk) ++n_pub;
      pend_tk = sched_open ? 1 : 0;
      ring_barrier();
      if (sched_open) sched_open = s_tk[(n_pub - 1) & 7] + 1 < r_end - r_start;
      if (l_state == L_BLOCKED) cursor_advance();
    }
  }
  // the last block to finish resets the launch's counters for the next user of the slot
  if constexpr (DYN) {
    if (tid == 0) {
      wait_vmcnt<0>();
      __threadfence();
      if (atomicAdd(&sched[8], 1) == (int)gridDim.x - 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sched[i] = 0;
        sched[8] = 0;
        __threadfence();
      }
    }
  }
}

// Split-K finish: out[row, c] from the S fp32 partial sums of the launch (added in part
// order), then the epilogue of the unsplit launch: SwiGLU h = silu(g) u (times row_scale
// outside the last group's own rows when given) and the optional bf16 g, u; or the plain
// bf16 / fp32 store. One thread per 8 output columns of a row; rows outside
// [offsets[0], offsets[G]) are left alone, as the GEMM leaves them.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_finish_kernel(const GemmParams p) {
  const int S = *p.part_s;
  if (S <= 1) return;  // the launch did not split: its tiles wrote the outputs
  const int oc = EPI == EPI_SWIGLU ? p.I : p.N;  // output columns
  const int pc = EPI == EPI_SWIGLU ? 2 * p.I : p.N;
  const int r_lo = p.offsets ? p.offsets[0] : 0;
  const int r_hi = p.offsets ? p.offsets[p.G] : p.rows;
  const int last0 = p.A_last == nullptr ? 0x7fffffff
                    : p.offsets ? p.offsets[p.G - 1] : (int)((long long)(p.G - 1) * p.rows / p.G);
  const int vpr = oc / 8;
  const size_t pstride = (size_t)p.rows * pc;
  const long long n = (long long)p.rows * vpr;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < n; idx += (long long)gridDim.x * 256) {
    const int row = (int)(idx / vpr), c = (int)(idx % vpr) * 8;
    if (row < r_lo || row >= r_hi) continue;
    const bool lastg = row >= last0;
    const float* src = p.part + (size_t)row * pc + c;
    if constexpr (EPI == EPI_SWIGLU) {
      float g[8], u[8];
      for (int e = 0; e < 8; ++e) g[e] = u[e] = 0.f;
      for (int k = 0; k < S; ++k) {
        const f32x4_t* pg = (const f32x4_t*)(src + (size_t)k * pstride);
        const f32x4_t* pu = (const f32x4_t*)(src + (size_t)k * pstride + p.I);
        const f32x4_t g0 = pg[0], g1 = pg[1], u0 = pu[0], u1 = pu[1];
        for (int e = 0; e < 4; ++e) {
          g[e] += g0[e];
          g[4 + e] += g1[e];
          u[e] += u0[e];
          u[4 + e] += u1[e];
        }
      }
      const float rs = p.row_scale != nullptr && !lastg ? p.row_scale[row] : 1.f;
      uint32_t hv[4];
      for (int e = 0; e < 4; ++e) {
        float h0 = g[2 * e] * sigmoid_fast(g[2 * e]) * u[2 * e];
        float h1 = g[2 * e + 1] * sigmoid_fast(g[2 * e + 1]) * u[2 * e + 1];
        if (p.row_scale != nullptr && !lastg) {
          h0 *= rs;
          h1 *= rs;
        }
        hv[e] = pack_bf16x2(h0, h1);
      }
      uint16_t* dst = lastg ? (uint16_t*)p.C_last + (size_t)(row - last0) * p.I : (uint16_t*)p.C + (size_t)row * p.I;
      *(u32x4_t*)(dst + c) = u32x4_t{hv[0], hv[1], hv[2], hv[3]};
      if (p.gu_out) {
        uint16_t* gd = (uint16_t*)p.gu_out + (size_t)row * pc + c;
        *(u32x4_t*)gd = u32x4_t{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                                pack_bf16x2(g[6], g[7])};
        *(u32x4_t*)(gd + p.I) = u32x4_t{pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]),
                                        pack_bf16x2(u[4], u[5]), pack_bf16x2(u[6], u[7])};
      }
    } else {
      float v[8];
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
      for (int k = 0; k < S; ++k) {
        const f32x4_t* pv = (const f32x4_t*)(src + (size_t)k * pstride);
        const f32x4_t v0 = pv[0], v1 = pv[1];
        for (int e = 0; e < 4; ++e) {
          v[e] += v0[e];
          v[4 + e] += v1[e];
        }
      }
      const size_t orow = lastg ? (size_t)(row - last0) : (size_t)row;
      if (p.c_fp32) {
        float* dst = (float*)(lastg ? p.C_last : p.C) + orow * p.N + c;
        *(f32x4_t*)dst = f32x4_t{v[0], v[1], v[2], v[3]};
        *(f32x4_t*)(dst + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
      } else {
        uint16_t* dst = (uint16_t*)(lastg ? p.C_last : p.C) + orow * p.N + c;
        *(u32x4_t*)dst = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                 pack_bf16x2(v[6], v[7])};
      }
    }
  }
}

namespace {

// Resident blocks of one kernel on the current device (compute units x blocks per CU),
// queried once per device and kernel: `cache` belongs to the caller's instantiation. The
// entries are atomics so that launches from several host threads may fill them (every
// thread computes the same value).
template <typename K>
int persistent_blocks(K kern, int threads, std::atomic<int> (&cache)[64]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, 0) != hipSuccess) return 0;
    v = cus * (occ > 0 ? occ : 1);
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Compute units of the current device (cached per device; 0 when the query fails).
int device_cus() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// grid cap set through moe_set_gemm_max_blocks (0: none); atomic so that a launch on one
// host thread may read it while another thread sets it (each launch reads it once)
std::atomic<int> g_max_blocks{0};
std::atomic<unsigned> g_launch_seq{0};  // picks the tile-counter slot of each launch

template <int MODE, int EPI, bool FP8, int BM, int BN, int WM, int WN, int STAGES, int BKB,
          bool BNT = false>
hipError_t launch_cfg(const GemmParams& p, hipStream_t s) {
  using C = Cfg<BM, BN, WM, WN, STAGES, BKB>;
  auto kern = grouped_gemm_kernel<MODE, EPI, FP8, BM, BN, WM, WN, STAGES, BKB, BNT>;
  static_assert(C::SMEM + 2 * 264 * 4 + 64 + C::NW * 2048 <= 160 * 1024, "LDS budget");
  const int ntn = EPI == EPI_SWIGLU ? (p.I + BN / 2 - 1) / (BN / 2) : (p.N + BN - 1) / BN;
  // upper bound of the tile count (the exact count depends on offsets[], read on the device)
  long long tiles;
  if (MODE == MOE_GEMM_TN_DW) tiles = (long long)p.G * ((p.M + BM - 1) / BM) * ntn;
  else tiles = ((long long)(p.rows + BM - 1) / BM + p.G) * ntn;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  // epilogue offsets are 32-bit byte offsets from a tile's first output element
  const long long row_bytes = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_BWD) ? 4LL * p.I
                                                                          : (long long)p.N * (p.c_fp32 ? 4 : 2);
  if ((long long)BM * row_bytes >= kOutOfRange) return hipErrorInvalidValue;
  static std::atomic<int> resident_cache[64];  // one per instantiation of launch_cfg
  const int resident = persistent_blocks(kern, C::NT, resident_cache);
  const int max_blocks = g_max_blocks.load(std::memory_order_relaxed);
  if (resident <= 0) return hipErrorInvalidValue;
  // split-K (32-row bf16 tiles): up to kSplitKMax parts per tile, fp32 partial rows of
  // 2I (SwiGLU) or N columns. Offered to the device only when even the most tiles the rows
  // can make (each M tile holds a row) leave blocks without one.
  constexpr bool SPLITK = MODE != MOE_GEMM_TN_DW && !FP8 && BM == 32 && EPI != EPI_SWIGLU_BWD &&
                          (MOE_GEMM_SPLITK & (EPI == EPI_SWIGLU ? 1 : 2)) != 0;
  bool split = false;
  if (SPLITK && p.part != nullptr) {
    if (p.part_s == nullptr) return hipErrorInvalidValue;
    const long long pc = EPI == EPI_SWIGLU ? 2LL * p.I : (long long)p.N;
    if ((long long)BM * pc * 4 >= kOutOfRange) return hipErrorInvalidValue;
    const long long mt = (long long)(p.rows + BM - 1) / BM + p.G;
    const long long most = (mt < p.rows ? mt : (long long)p.rows) * ntn;
    int blocks = resident;
    if (max_blocks > 0 && max_blocks < blocks) blocks = max_blocks;
    split = most < blocks;
    if (split) tiles *= kSplitKMax;
  }
  long long grid = tiles < resident ? tiles : resident;
  if (max_blocks > 0 && grid > max_blocks) grid = max_blocks;
  GemmParams q = p;
  if (!split) q.part = nullptr;
  q.sched_slot = (int)(g_launch_seq.fetch_add(1, std::memory_order_relaxed) % kSchedSlots);
  kern<<<dim3((unsigned)grid), dim3(C::NT), 0, s>>>(q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  const long long oc = EPI == EPI_SWIGLU ? p.I : p.N;
  const long long n = (long long)p.rows * (oc / 8);
  long long fb = (n + 255) / 256;
  if (fb > 8192) fb = 8192;
  if (fb < 1) return hipSuccess;
  splitk_finish_kernel<EPI == EPI_SWIGLU ? EPI_SWIGLU : EPI_STORE><<<dim3((unsigned)fb), dim3(256), 0, s>>>(q);
  return hipGetLastError();
}

}  // namespace

// Tile configurations (BM, BN, WM, WN, STAGES, K bytes per stage), chosen by
// measurement on the Qwen3- and Mixtral-shaped expert GEMMs. bf16 NN/NT and the SwiGLU
// forward: 320x256 tiles with eight waves (two per SIMD, 160x64 each) and a three-stage
// ring of 64-byte K steps; weight gradients 256x256 tiles with a four-stage ring (measured
// 1-2 % faster than three stages, one process per build). SwiGLU backward
// (whose epilogue reads the saved g,u): the same 320x256 tiles when they still give every
// CU at least four tiles, else 320x128 tiles with four waves and a four-stage ring (fewer
// tiles per CU leave too many CUs idle at the end). e4m3: 256x256 tiles with eight waves
// and a four-stage ring of 64-byte (64-element) K steps (1-2 % faster than three), A
// fragments read one M block ahead of the multiply so that the 8-register e4m3 fragments
// fit.
#ifndef MOE_GEMM_TILE_BF16
#define MOE_GEMM_TILE_BF16 320, 256, 2, 4, 3, 64
#endif
#ifndef MOE_GEMM_TILE_BF16_DW
#define MOE_GEMM_TILE_BF16_DW 256, 256, 2, 4, 4, 64
#endif
#ifndef MOE_GEMM_TILE_BF16_SWIGLU
#define MOE_GEMM_TILE_BF16_SWIGLU 320, 256, 2, 4, 3, 64
#endif
#ifndef MOE_GEMM_TILE_BF16_SWIGLU_BWD
#define MOE_GEMM_TILE_BF16_SWIGLU_BWD 320, 256, 2, 4, 3, 64
#endif
#ifndef MOE_GEMM_TILE_BF16_SWIGLU_BWD_NARROW
#define MOE_GEMM_TILE_BF16_SWIGLU_BWD_NARROW 320, 128, 2, 2, 4, 64
#endif
#ifndef MOE_GEMM_TILE_FP8
#define MOE_GEMM_TILE_FP8 256, 256, 2, 4, 4, 64
#endif
// Small-M tiles (decode: a handful of rows per expert): 32-row tiles, since a decode step
// only streams weights. The store GEMM: 128 output columns per block (two waves) and four
// stages of 128-byte K steps, 64 KB in flight per CU (measured best on Llama4-shaped decode
// among 32x64 to 32x512 tiles with one to eight waves and three or four stages). The SwiGLU
// GEMM: 512 columns (256 gate, 256 up: 512-byte weight-row pieces) with eight waves and
// three stages of 64-byte K steps; on the Llama4-shaped step it takes 147 us against 193 for
// 32x256 tiles (half as many tiles, each streaming twice the bytes per weight row).
#ifndef MOE_GEMM_TILE_SMALL_M
#define MOE_GEMM_TILE_SMALL_M 32, 128, 1, 2, 4, 128
#endif
#ifndef MOE_GEMM_TILE_SMALL_M_SWIGLU
#define MOE_GEMM_TILE_SMALL_M_SWIGLU 32, 512, 1, 8, 3, 64
#endif
namespace {
// every group fits one 32-row tile when the whole buffer has at most 32 rows per group on
// average and at most 256 rows: the decode case
bool small_m_rows(long long rows, int G) { return rows <= 256 && rows <= 32LL * G; }

// The M-tile height of a tile configuration.
constexpr int tile_rows(int bm, int, int, int, int, int) { return bm; }

template <int MODE, int EPI, bool F8>
hipError_t launch_sel(const GemmParams& p, hipStream_t s) {
  // NN launches whose groups average at most one M tile stream each weight panel once
  const auto nn_once = [&](int bm) { return (long long)p.rows <= (long long)p.G * bm; };
  if constexpr (F8) {
    return launch_cfg<MODE, EPI, true, MOE_GEMM_TILE_FP8>(p, s);
  } else {
    if constexpr (MODE != MOE_GEMM_TN_DW) {
      if (small_m_rows(p.rows, p.G)) {  // (at most 32 rows per group on average)
        constexpr bool NT_W = MODE == MOE_GEMM_NN;
        if constexpr (EPI == EPI_SWIGLU) return launch_cfg<MODE, EPI, false, MOE_GEMM_TILE_SMALL_M_SWIGLU, NT_W>(p, s);
        else return launch_cfg<MODE, EPI, false, MOE_GEMM_TILE_SMALL_M, NT_W>(p, s);
      }
    }
    if constexpr (EPI == EPI_SWIGLU_BWD) {
      // upper bound of the wide tiles (BM = 320, BN = 256), as the launcher counts them,
      // against the blocks a launch can have
      const long long wide = ((long long)(p.rows + 319) / 320 + p.G) * ((p.N + 255) / 256);
      int blocks = device_cus();
      const int max_blocks = g_max_blocks.load(std::memory_order_relaxed);
      if (max_blocks > 0 && max_blocks < blocks) blocks = max_blocks;
      if (wide >= 4LL * blocks) return launch_cfg<MODE, EPI, false, MOE_GEMM_TILE_BF16_SWIGLU_BWD>(p, s);
      return launch_cfg<MODE, EPI, false, MOE_GEMM_TILE_BF16_SWIGLU_BWD_NARROW>(p, s);
    }
    else if constexpr (EPI == EPI_SWIGLU) {
      if constexpr (MODE == MOE_GEMM_NN)
        if (nn_once(tile_rows(MOE_GEMM_TILE_BF16_SWIGLU)))
          return launch_cfg<MODE, EPI, false, MOE_GEMM_TILE_BF16_SWIGLU, true>(p, s);
      return launch_cfg<MODE, EPI, false, MOE_GEMM_TILE_BF16_SWIGLU>(p, s);
    }
    else if constexpr (MODE == MOE_GEMM_TN_DW) return launch_cfg<MODE, EPI, false, MOE_GEMM_TILE_BF16_DW>(p, s);
    else {
      if constexpr (MODE == MOE_GEMM_NN)
        if (nn_once(tile_rows(MOE_GEMM_TILE_BF16))) return launch_cfg<MODE, EPI, false, MOE_GEMM_TILE_BF16, true>(p, s);
      return launch_cfg<MODE, EPI, false, MOE_GEMM_TILE_BF16>(p, s);
    }
  }
}
}  // namespace

void set_gemm_max_blocks(int n) { g_max_blocks.store(n, std::memory_order_relaxed); }

size_t splitk_workspace_bytes(long long rows, int G, long long ncols) {
  if (rows <= 0 || G <= 0 || ncols <= 0 || !small_m_rows(rows, G)) return 0;
  return 256 + (size_t)kSplitKMax * (size_t)rows * (size_t)ncols * 4;
}

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
