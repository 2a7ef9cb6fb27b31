// Grouped SwiGLU, bf16 path on the CDNA4 matrix cores.
//
// Method: Sparse MoE routing-math page (arman1o1.github.io), section 0
// (SwiGLU(h) = (SiLU(h W_gate) * (h W_up)) W_down), section 3 (all local
// experts in one grouped GEMM over variable-sized token buckets, no padding).
//
// Two launches over the device-built tile list:
//   gate/up: act[r, n] = SiLU(x_r . Wg[n]) * (x_r . Wu[n])     K = d_model
//            x rows gathered on load through row_index (no x_perm copy);
//            the B tile stacks 128 W_gate rows over the same 128 W_up rows,
//            so each lane holds matching gate and up accumulators.
//   down:    y[r, n] = (act_r . Wd[n]) * row_scale[r]          K = d_ffn
// The training form of gate/up (a compile-time variant) also writes a = x.Wg
// and u = x.Wu to au [rows, 2 d_ffn] from the same accumulators, in extra
// passes of its epilogue, for the backward pass.
//
// Tile: 256 grouped rows x 256 weight rows x 64 k, eight waves (two per
// SIMD) in a 4 x 2 layout, each wave 64 rows x 128 weight rows as 2 x 4
// blocks of v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  A 256-row tile
// covers a whole expert whenever it has <= 256 rows (the DeepSeek-V3 prefill
// and decode shapes), so each weight slice is streamed from HBM once; a wave
// skips the MFMAs of 32-row blocks that hold no row of the group, and rows
// past the group are neither loaded nor staged.  256 weight rows per tile
// halve the re-reads of the gathered x rows (once per column tile) compared
// with 128.  The global loads of the next 64-k slice stay in flight while the
// current one is multiplied out of LDS (two register sets, two 64 KB LDS
// stages; 16-byte chunks XOR-swizzled per row so fragment reads and staging
// writes are bank-conflict free).  This shape measured fastest for both the
// weight-streaming (few rows per expert) and the matrix-core-bound shapes.
//
// Four kernels share the tile: a one-tile-per-workgroup kernel (any shape),
// and three persistent streaming kernels for K and N that fit whole slices
// and column tiles: an LDS-fed one (operands loaded straight into LDS) for
// groups of at least 256 rows on average, where the matrix cores bound the
// products; for smaller groups, where streaming the weights from HBM bounds
// them, one that sends the weights straight into a three-stage LDS ring and
// keeps the x rows on the register path (inference forms), and the
// register-staged one (both operands through registers; the training form
// and the down product with a row scale).
//
// Work order: by group, then blocks of up to four row tiles by all column
// tiles, row tile fastest (item_tile); block ids are remapped so each XCD
// walks a contiguous run of it: the row tiles of one (expert, column tile)
// run side by side on one XCD and share the weight slice through its L2, and
// the column tiles of the same row tiles reuse their gathered x rows from it.
#include "swiglu_tiles.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;         // k per LDS stage (8 chunks of 16 B per row)
constexpr int kRowBytes = kBK * 2;                     // 128 B
constexpr int kNumXcd = 8;

// Row and column tile of item `local` of a group with nmt row tiles and NT
// column tiles.  Items run in blocks of kItemRows row tiles by all column
// tiles, row tile fastest inside a block, so the items an XCD's workgroups
// take side by side (consecutive items) cover a few row tiles by several
// column tiles and share both operands' slices through its L2; groups of at
// most kItemRows row tiles keep plain row-tile-fastest order.
constexpr int kItemRows = 4;
__device__ __forceinline__ void item_tile(int local, int nmt, int NT, int& mt, int& nt) {
  if (nmt <= kItemRows) {  // one block: a single division
    nt = local / nmt;
    mt = local - nt * nmt;
    return;
  }
  const int full = nmt / kItemRows;
  const int span = kItemRows * NT;
  if (local < full * span) {
    const int sr = local / span, j = local - sr * span;
    mt = sr * kItemRows + j % kItemRows;
    nt = j / kItemRows;
  } else {
    const int j = local - full * span, rl = nmt - full * kItemRows;
    mt = full * kItemRows + j % rl;
    nt = j / rl;
  }
}
constexpr int kBufferFlags = 0x00020000;               // raw buffer, 32-bit data format

// LDS byte offset of 16-byte chunk c of tile row r.  The chunk index is XORed
// with (r & 7) ^ ((r >> 3) & 1): a fragment read (32 consecutive rows, one
// chunk) and a staging write (8 lanes per row) then hit distinct banks whether
// the LDS serves 8 lanes x 16 B or 16 lanes x 16 B per cycle.
__device__ __forceinline__ int swz(int r, int c) {
  return r * kRowBytes + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4);
}

template <int BM, int BNW, int NTHR>
struct Tile {
  static constexpr int kThreads = NTHR;
  static constexpr int kWaves = NTHR / 64;
  static constexpr int kWavesM = BM / 64;              // waves along rows
  static constexpr int kWavesN = kWaves / kWavesM;     // waves along weight rows
  static constexpr int kNB = BNW / kWavesN / 32;       // 32-wide weight blocks per wave
  static constexpr int kABytes = BM * kRowBytes;
  static constexpr int kStageBytes = (BM + BNW) * kRowBytes;
  static constexpr int kRowsPerPass = NTHR / 8;        // rows one load pass covers
  static constexpr int kALoads = BM / kRowsPerPass;
  static constexpr int kBLoads = BNW / kRowsPerPass;
  // waves per SIMD: workgroups per CU x waves per workgroup / 4 SIMDs
  static constexpr int kWavesPerEU = ((BM + BNW <= 256) ? 2 : 1) * kWaves / 4;
};

// GATEUP: 64 act columns per tile, W0 = W_gate, W1 = W_up
// DOWN:   128 y columns per tile,  W0 = W_down
template <bool GATEUP, int BM, int BNW, int NTHR, int NSETS, bool AU = false>
__global__ __launch_bounds__(NTHR)
__attribute__((amdgpu_waves_per_eu(Tile<BM, BNW, NTHR>::kWavesPerEU,
                                   Tile<BM, BNW, NTHR>::kWavesPerEU)))
void bf16_tile_kernel(
    int Kdim, int N, int x_rows, int NT, const TileInfo* __restrict__ tiles,
    const int32_t* __restrict__ meta, const int32_t* __restrict__ row_index,
    const uint16_t* __restrict__ A, const WeightSet W, const float* __restrict__ row_scale,
    uint16_t* __restrict__ out, uint16_t* __restrict__ au) {
  using TL = Tile<BM, BNW, NTHR>;
  constexpr int kALoads = TL::kALoads;
  constexpr int kBLoads = TL::kBLoads;
  constexpr int kNB = TL::kNB;
  __shared__ __attribute__((aligned(16))) char smem[2 * TL::kStageBytes];

  // ---- block -> (group, column tile, row tile), XCD-contiguous
  const int total = meta[0] * NT;
  const int xcd = blockIdx.x % kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int w = xcd * per_xcd + slot;
  if (slot >= per_xcd || w >= total) return;
  // a group's items are the NT column tiles of each of its tiles, so tile
  // w / NT belongs to the group of work item w; its record holds the group's
  // first tile and tile count, and the group's weight index
  const TileInfo t0 = tiles[w / NT];
  const int g = t0.group;
  const int gstart = t0.gstart;
  const int nmt = max(t0.ntiles, 1);
  int mtile, ntile;
  item_tile(w - gstart * NT, nmt, NT, mtile, ntile);
  const TileInfo ti = tiles[gstart + mtile];
  const int nrows = min(ti.m1 - ti.m0, BM);

  constexpr int kCols = GATEUP ? BNW / 2 : BNW;
  const int n0 = ntile * kCols;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int wm = wave / TL::kWavesN, wn = wave % TL::kWavesN;

  // ---- per-thread load slots (row lr + 32 i, 16-byte chunk lc of the k-slice).
  // Buffer loads: an offset past the end of the buffer reads zeros without a
  // memory access, so rows past the group, rows with an out-of-range source
  // and columns past N need no branch -- the loop stays straight-line and the
  // loads of later slices stay in flight across the LDS stores.  The per-lane
  // offsets are loop-invariant; the k position goes in the uniform soffset.
  const int lc = tid & 7;
  const int lr = tid >> 3;  // 0 .. kRowsPerPass-1
  constexpr int kRP = TL::kRowsPerPass;
  constexpr uint32_t kOff = 0x80000000u;  // beyond every buffer (sizes < 2 GiB)
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A), 0, static_cast<int>(static_cast<uint32_t>(x_rows) * Kdim * 2u),
      kBufferFlags);
  uint32_t a_off[kALoads];
#pragma unroll
  for (int i = 0; i < kALoads; ++i) {
    const int r = lr + kRP * i;
    int sr = -1;
    if (r < nrows) {
      const int gr = ti.m0 + r;
      sr = row_index ? row_index[gr] : gr;
      if (sr < 0 || sr >= x_rows) sr = -1;
    }
    a_off[i] = (sr >= 0) ? (static_cast<uint32_t>(sr) * Kdim + lc * 8) * 2u : kOff;
  }
  const int wbytes = static_cast<int>(static_cast<uint32_t>(N) * Kdim * 2u);
  const size_t wmat = static_cast<size_t>(N) * Kdim;
  const __amdgpu_buffer_rsrc_t rsB0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W.base(false, g, wmat)), 0, wbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsB1 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W.base(GATEUP, g, wmat)), 0, wbytes, kBufferFlags);
  uint32_t b_off[kBLoads];
#pragma unroll
  for (int i = 0; i < kBLoads; ++i) {
    const int r = lr + kRP * i;  // 0..BNW-1
    const int n = GATEUP ? n0 + (r % (BNW / 2)) : n0 + r;
    b_off[i] = (n < N) ? (static_cast<uint32_t>(n) * Kdim + lc * 8) * 2u : kOff;
  }

#define MOE_LOAD_SLICE(SA, SB, K0)                                                      \
  do {                                                                                 \
    const uint32_t kb_ = static_cast<uint32_t>(K0) * 2u;                               \
    _Pragma("unroll") for (int i = 0; i < kALoads; ++i) SA[i] =                        \
        __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsA, a_off[i], kb_, 0)); \
    _Pragma("unroll") for (int i = 0; i < kBLoads; ++i) SB[i] = __builtin_bit_cast(     \
        uint4, __builtin_amdgcn_raw_buffer_load_b128((!GATEUP || i < kBLoads / 2) ? rsB0 : rsB1, \
                                                     b_off[i], kb_, 0));               \
  } while (0)
#define MOE_STORE_SLICE(SA, SB, STAGE)                                                  \
  do {                                                                                 \
    char* as_ = smem + (STAGE) * TL::kStageBytes;                                      \
    char* bs_ = as_ + TL::kABytes;                                                     \
    _Pragma("unroll") for (int i = 0; i < kALoads; ++i)                                \
        if (lr + kRP * i < nrows)                                                      \
          *reinterpret_cast<uint4*>(as_ + swz(lr + kRP * i, lc)) = SA[i];              \
    _Pragma("unroll") for (int i = 0; i < kBLoads; ++i)                                \
        *reinterpret_cast<uint4*>(bs_ + swz(lr + kRP * i, lc)) = SB[i];                \
  } while (0)

  // B-tile rows of this wave's 32-wide weight blocks.  GATEUP: the first half
  // of the blocks are W_gate rows, the second half the matching W_up rows.
  int brow[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    if (GATEUP) {
      const int half = kNB / 2;
      const int base = wn * (BNW / 2 / TL::kWavesN);
      brow[nb] = (nb < half) ? base + nb * 32 : BNW / 2 + base + (nb - half) * 32;
    } else {
      brow[nb] = wn * (BNW / TL::kWavesN) + nb * 32;
    }
  }

  f32x16_t acc[2][kNB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mb][nb][q] = 0.0f;

  // wave-uniform: which of this wave's two 32-row blocks hold rows of the group
  const bool mb0 = wm * 64 < nrows;
  const bool mb1 = wm * 64 + 32 < nrows;
  const int fr = lane & 31;  // fragment row within a 32-block
  const int fh = lane >> 5;  // which 8-wide k half of a 16-k step

  auto compute = [&](int stage) {
    if (!mb0) return;
    const char* as = smem + stage * TL::kStageBytes;
    const char* bs = as + TL::kABytes;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int c = kk * 2 + fh;
      bf16x8_t af[2], bfr[kNB];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        bfr[nb] = *reinterpret_cast<const bf16x8_t*>(bs + swz(brow[nb] + fr, c));
      af[0] = *reinterpret_cast<const bf16x8_t*>(as + swz(wm * 64 + fr, c));
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], bfr[nb], acc[0][nb], 0, 0, 0);
      if (mb1) {
        af[1] = *reinterpret_cast<const bf16x8_t*>(as + swz(wm * 64 + 32 + fr, c));
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1], bfr[nb], acc[1][nb], 0, 0, 0);
      }
    }
  };

  // ---- main loop: NSETS register sets rotate through the global loads, so
  // slices kt+1 .. kt+NSETS are in flight while slice kt is multiplied out of
  // one of two LDS stages.  Every step issues its prefetch unconditionally
  // (past the end it re-reads the last slice, an L2 hit), so the wait before
  // each LDS store counts only the slice being stored and the newer slices
  // stay in flight.  Rows past the group are neither loaded nor stored: their
  // LDS rows hold stale values, which only reach output rows masked at the end.
  const int nk = Kdim / kBK;
  uint4 sa0[kALoads], sb0[kBLoads], sa1[kALoads], sb1[kBLoads];
  uint4 sa2[NSETS > 2 ? kALoads : 1], sb2[NSETS > 2 ? kBLoads : 1];
  uint4 sa3[NSETS > 3 ? kALoads : 1], sb3[NSETS > 3 ? kBLoads : 1];
  MOE_LOAD_SLICE(sa0, sb0, 0);
  MOE_LOAD_SLICE(sa1, sb1, min(1, nk - 1) * kBK);
  if constexpr (NSETS > 2) MOE_LOAD_SLICE(sa2, sb2, min(2, nk - 1) * kBK);
  if constexpr (NSETS > 3) MOE_LOAD_SLICE(sa3, sb3, min(3, nk - 1) * kBK);
  MOE_STORE_SLICE(sa0, sb0, 0);
  __syncthreads();
  // step J multiplies slice J (stage J % 2), refills its register set with
  // slice J + NSETS and stores slice J + 1 (the next set) to the other stage
#define MOE_STEP(J, LA, LB, STAGE, SA, SB)                                              \
  MOE_LOAD_SLICE(LA, LB, min((J) + NSETS, nk - 1) * kBK);                              \
  compute(STAGE);                                                                      \
  if ((J) + 1 >= nk) break;                                                            \
  MOE_STORE_SLICE(SA, SB, (STAGE) ^ 1);                                                \
  __syncthreads();
  if constexpr (NSETS == 2) {
    for (int kt = 0;; kt += 2) {
      MOE_STEP(kt + 0, sa0, sb0, 0, sa1, sb1)
      MOE_STEP(kt + 1, sa1, sb1, 1, sa0, sb0)
    }
  } else if constexpr (NSETS == 3) {
    for (int kt = 0;; kt += 6) {
      MOE_STEP(kt + 0, sa0, sb0, 0, sa1, sb1)
      MOE_STEP(kt + 1, sa1, sb1, 1, sa2, sb2)
      MOE_STEP(kt + 2, sa2, sb2, 0, sa0, sb0)
      MOE_STEP(kt + 3, sa0, sb0, 1, sa1, sb1)
      MOE_STEP(kt + 4, sa1, sb1, 0, sa2, sb2)
      MOE_STEP(kt + 5, sa2, sb2, 1, sa0, sb0)
    }
  } else {
    for (int kt = 0;; kt += 4) {
      MOE_STEP(kt + 0, sa0, sb0, 0, sa1, sb1)
      MOE_STEP(kt + 1, sa1, sb1, 1, sa2, sb2)
      MOE_STEP(kt + 2, sa2, sb2, 0, sa3, sb3)
      MOE_STEP(kt + 3, sa3, sb3, 1, sa0, sb0)
    }
  }
#undef MOE_STEP
#undef MOE_LOAD_SLICE
#undef MOE_STORE_SLICE

  // ---- epilogue: the bf16 tile is staged in LDS (both stages are free now)
  // and written as whole 16-byte chunks of each output row; the MFMA layout
  // alone would give 2-byte stores scattered over 32 rows per instruction.
  // D[row][col] of a 32x32 block sits in lane (col + 32*((row/4)%2)),
  // register (row%4) + 4*(row/8).  Staging layout: row-major bf16 rows of
  // kCols, the 16-byte chunk index XORed with (row & 4) so the two half-waves
  // (rows r and r+4) write disjoint banks.
  static_assert(BM * kCols * 2 <= 2 * TL::kStageBytes, "output tile exceeds LDS");
  constexpr int kOutRowBytes = kCols * 2;
  constexpr int kOutChunks = kCols / 8;
  // Gate/up with AU: pass 0 also stages a in the second half of the LDS (the
  // gate accumulators are then dead for the read-outs), pass 1 stages u; both
  // go to au [rows, 2N].
  static_assert(!AU || 2 * BM * kCols * 2 <= 2 * TL::kStageBytes, "a|u tiles exceed LDS");
  constexpr int npass = (GATEUP && AU) ? 2 : 1;
  constexpr int kHalf = BM * kOutRowBytes;
#pragma unroll
  for (int pass = 0; pass < npass; ++pass) {
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = wm * 64 + mb * 32 + 8 * (q >> 2) + 4 * fh + (q & 3);
      if (row >= nrows) continue;
      char* orow = smem + row * kOutRowBytes;
      const int sw = row & 4;
      if (GATEUP) {
#pragma unroll
        for (int nb = 0; nb < kNB / 2; ++nb) {
          const int c = brow[nb] + fr;
          const int co = (((c >> 3) ^ sw) << 4) + (c & 7) * 2;
          const float gv = acc[mb][nb][q], uv = acc[mb][nb + kNB / 2][q];
          if (pass == 0) {
            *reinterpret_cast<uint16_t*>(orow + co) = f32_to_bf16(silu(gv) * uv);
            if (AU) *reinterpret_cast<uint16_t*>(orow + kHalf + co) = f32_to_bf16(gv);
          } else {
            *reinterpret_cast<uint16_t*>(orow + co) = f32_to_bf16(uv);
          }
        }
      } else {
        const float sc = row_scale ? row_scale[ti.m0 + row] : 1.0f;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const int c = brow[nb] + fr;
          *reinterpret_cast<uint16_t*>(orow + (((c >> 3) ^ sw) << 4) + (c & 7) * 2) =
              f32_to_bf16(acc[mb][nb][q] * sc);
        }
      }
    }
  }
  __syncthreads();
  // pass 0: half 0 -> out (and, with AU, half 1 -> a); pass 1: half 0 -> u
  constexpr int kHalves = AU ? 2 : 1;
#pragma unroll
  for (int hf = 0; hf < kHalves; ++hf) {
    if (pass == 1 && hf == 1) break;
    const size_t ldo = (pass == 0 && hf == 0) ? static_cast<size_t>(N) : 2 * static_cast<size_t>(N);
    uint16_t* const ob = (pass == 0 && hf == 0) ? out : au + (pass == 1 ? N : 0);
#pragma unroll
    for (int it = 0; it < BM * kOutChunks / NTHR; ++it) {
      const int idx = it * NTHR + tid;
      const int r = idx / kOutChunks;
      const int c = idx % kOutChunks;
      if (r < nrows && n0 + c * 8 < N) {
        const uint4 v = *reinterpret_cast<const uint4*>(smem + hf * kHalf + r * kOutRowBytes +
                                                       ((c ^ (r & 4)) << 4));
        *reinterpret_cast<uint4*>(ob + static_cast<size_t>(ti.m0 + r) * ldo + n0 + c * 8) = v;
      }
    }
  }
  }
}

// ---------------------------------------------------------------- streaming, LDS-fed
//
// One workgroup per CU, each walking a fixed list of work items: the items of
// an XCD (the same XCD-contiguous runs as above) are dealt round-robin to its
// workgroups, and a workgroup streams the k-slices of its items back to back,
// so the first slices of the next item are already in flight while the last
// one of the current item is multiplied and its output tile written.
//
// Operand slices go from HBM/L2 straight into LDS (buffer loads with an LDS
// destination: no staging registers, no LDS store instructions).  The stages
// rotate with kStages - 1 slices in flight: step j waits for its own slice,
// meets the other waves at one barrier (after which the stage multiplied at
// step j - 1 is free in every wave), sends the loads of the next slice into
// that stage and multiplies slice j.  The wait and the barrier are one asm
// statement, so every wave's share of the slice has landed before any wave
// reads it.  The stages are separate LDS objects and the stage of a step is a
// compile-time choice (the step loop is unrolled by the stage count), which
// lets the compiler count the loads each LDS read waits for exactly.  The
// explicit wait counts only the newer slices' loads, so it is exact whatever
// else was issued in between: loads complete in order, and any extra newer
// load only makes the wait longer.
//
// The next item's tile records arrive through scalar loads two steps apart,
// its gathered row indices (gate/up) through a small LDS DMA, so the loop has
// no vector loads besides the slices.  Down: each item's row scales are sent
// into LDS (by item parity) when its loads start and read by its epilogue.
// Used when K is a multiple of 128 with at least kMinStreamSlices slices and N
// is a multiple of the column tile, for groups of at least a full row tile on
// average (matrix-core-bound products).  With 64-k slices a stage holds 64 KB,
// so one slice is in flight per step: enough where the products are bound by
// the matrix cores, too little for weight streaming, which the register-staged
// kernel below handles with two slices in flight.
// Stage geometry of the streaming kernel for k-slices of BK (32 or 64): tile
// rows of 2 BK bytes, 256 A rows + 256 B rows per stage, 4 stages of 32 KB or 2
// of 64 KB.  A slice load covers RPI whole rows per wave instruction.
template <int BK>
struct StreamGeom {
  static_assert(BK == 32 || BK == 64, "32 or 64 k per stage");
  static constexpr int kRow = BK * 2;               // bytes per tile row
  static constexpr int kChunks = BK / 8;            // 16-byte chunks per row
  static constexpr int kTileBytes = 256 * kRow;     // one operand tile
  static constexpr int kStageBytes = 2 * kTileBytes;
  static constexpr int kStages = BK == 32 ? 4 : 2;
  static constexpr int kRPI = 64 / kChunks;         // rows per load instruction
  static constexpr int kNI = 256 / kRPI / 8;        // load instructions per wave and operand
  // LDS byte offset of 16-byte k chunk c of tile row r.  64-byte rows: the
  // chunk is XORed with ((r >> 1) & 3) ^ ((r >> 3) & 1), 128-byte rows with
  // (r & 7) ^ ((r >> 3) & 1): a fragment read (32 consecutive rows, one chunk)
  // then puts any 8 consecutive rows in distinct 16-byte bank groups of a
  // 128-byte window and any 16 in distinct groups of a 256-byte one.
  static __device__ __forceinline__ int swz(int r, int c) {
    const int x = BK == 32 ? ((r >> 1) & 3) ^ ((r >> 3) & 1) : (r & 7) ^ ((r >> 3) & 1);
    return r * kRow + ((c ^ x) << 4);
  }
};
constexpr int kMinStreamSlices = 8;
constexpr int kStreamBK = 64;             // k per stage of the LDS-fed streaming kernel
constexpr int kDmaMinRowsPerGroup = 256;  // average rows per group that select it

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes),
                                           kBufferFlags);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer load of BYTES per lane into LDS: lane l's data lands at lds + l * BYTES
// (lds is wave-uniform).  Only voffset takes part in the range check, so an
// out-of-range voffset reads zeros while the uniform soffset moves along k.
// Cache policy of the weight loads: non-temporal.  Within a launch each
// weight slice is needed only by the row tiles of its expert that run side by
// side (at most a few, on one XCD), so the expert weights -- gigabytes per
// launch -- are streamed past the caches instead of displacing the gathered
// token rows and activations that every column tile re-reads.  Measured:
// decode-shape gate/up 2.10 -> 1.90 ms, down 1.11 -> 1.03 ms; Mixtral down
// 1.18 -> 1.11 ms; prefill unchanged.
constexpr int kWeightPolicy = 2;

template <int BYTES, int AUX = 0>
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff,
                                    uint32_t soff) {
  static_assert(BYTES == 4 || BYTES == 16, "dword or 16-byte loads");
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds, 16, voff, soff, 0, AUX);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds, 4, voff, soff, 0, AUX);
}

// The same load with the LDS destination passed through an empty asm: the
// compiler then cannot tie the load to an LDS object and inserts no wait for
// it before LDS reads.  For kernels whose own explicit waits and barriers
// order every such load before the reads of its data.
template <int AUX = 0>
__device__ __forceinline__ void dma16_unscoped(__amdgpu_buffer_rsrc_t rs, void* lds, uint32_t voff,
                                               uint32_t soff) {
  lds_ptr_t l = (lds_ptr_t)lds;
  asm volatile("" : "+s"(l));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, l, 16, voff, soff, 0, AUX);
}

template <bool GATEUP, int BK, bool AU = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bf16_stream_kernel(
    int Kdim, int N, int x_rows, int rows, int NT, const TileInfo* __restrict__ tiles,
    const int32_t* __restrict__ meta, const int32_t* __restrict__ row_index,
    const uint16_t* __restrict__ A, const WeightSet W, const float* __restrict__ row_scale,
    uint16_t* __restrict__ out, uint16_t* __restrict__ au) {
  using G = StreamGeom<BK>;
  constexpr int BM = 256, BNW = 256, NTHR = 512;
  constexpr int kWavesN = 2;                  // waves: 4 along rows x 2 along weight rows
  constexpr int kNB = BNW / kWavesN / 32;     // 32-wide weight blocks per wave
  constexpr int kCols = GATEUP ? BNW / 2 : BNW;
  constexpr int kNI = G::kNI, kRPI = G::kRPI;
  constexpr uint32_t kOff = 0x80000000u;      // beyond every buffer (sizes < 2 GiB)
  constexpr int kS0 = G::kStageBytes;
  constexpr int kS2 = G::kStages == 4 ? G::kStageBytes : 16;
  __shared__ __attribute__((aligned(16))) char st0[kS0];
  __shared__ __attribute__((aligned(16))) char st1[kS0];
  __shared__ __attribute__((aligned(16))) char st2[kS2];
  __shared__ __attribute__((aligned(16))) char st3[kS2];
  __shared__ __attribute__((aligned(16))) int32_t ri_lds[8 * 64];     // next item's source rows
  __shared__ __attribute__((aligned(16))) float sc_lds[2 * 8 * 64];   // row scales by item parity
  char* const st_last = G::kStages == 4 ? st3 : st1;

  // ---- this workgroup's items: first, first + nslot, ... below end
  const int total = meta[0] * NT;
  const int nslot = gridDim.x / kNumXcd;
  const int xcd = blockIdx.x % kNumXcd;
  const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int first = xcd * per_xcd + static_cast<int>(blockIdx.x) / kNumXcd;
  const int end = min(total, (xcd + 1) * per_xcd);
  if (first >= end) return;
  const int n_items = (end - first + nslot - 1) / nslot;
  const int nk = Kdim / BK;  // a multiple of 4 / BK * 32 stages... a multiple of the stage count

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: scalar
  const int lane = tid % kWave;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  // Slice loads: load instruction i of a wave sends tile rows kRPI (wave + 8 i)
  // + drow of A and of B; lane l lands at LDS chunk l % kChunks of its row, so
  // it loads the k chunk that the swizzle stores there.
  const int drow = lane / G::kChunks;
  const int dchunk =
      (lane % G::kChunks) ^ (BK == 32 ? ((drow >> 1) & 3) ^ ((drow >> 3) & 1) : drow ^ (wave & 1));
  const uint32_t rowbytes = static_cast<uint32_t>(Kdim) * 2u;
  const uint32_t wbytes = static_cast<uint32_t>(N) * rowbytes;
  const __amdgpu_buffer_rsrc_t rsA = buffer_rsrc(A, static_cast<uint32_t>(x_rows) * rowbytes);
  // gate/up gathers x rows through row_index (NULL: grouped row r is x row r)
  const bool gather = GATEUP && row_index != nullptr;
  const __amdgpu_buffer_rsrc_t rsR =
      buffer_rsrc(row_index, gather ? static_cast<uint32_t>(rows) * 4u : 0u);
  const bool has_scale = !GATEUP && row_scale != nullptr;
  const __amdgpu_buffer_rsrc_t rsS =
      buffer_rsrc(row_scale, has_scale ? static_cast<uint32_t>(rows) * 4u : 0u);

  auto a_offset = [&](int i, int nrows, int sr) -> uint32_t {
    return (kRPI * (wave + 8 * i) + drow < nrows && sr >= 0 && sr < x_rows)
               ? static_cast<uint32_t>(sr) * rowbytes + static_cast<uint32_t>(dchunk) * 16u
               : kOff;
  };

  // ---- load-side item
  int l_item = 0, l_g, l_ntile, l_m0, l_nrows;
  {
    const TileInfo t0 = tiles[first / NT];
    int mt;
    item_tile(first - t0.gstart * NT, max(t0.ntiles, 1), NT, mt, l_ntile);
    const TileInfo ti = tiles[t0.gstart + mt];
    l_g = t0.group;
    l_m0 = ti.m0;
    l_nrows = min(ti.m1 - ti.m0, BM);
  }
  uint32_t a_off[kNI];
#pragma unroll
  for (int i = 0; i < kNI; ++i) {
    const int r = kRPI * (wave + 8 * i) + drow;
    const int sr = gather ? (r < l_nrows ? row_index[l_m0 + r] : -1) : l_m0 + r;
    a_off[i] = a_offset(i, l_nrows, sr);
  }
  __amdgpu_buffer_rsrc_t rb0, rb1;
  uint32_t bcol;
  const uint32_t b_off = static_cast<uint32_t>(kRPI * wave + drow) * rowbytes +
                         static_cast<uint32_t>(dchunk) * 16u;
  auto set_weights = [&]() {
    rb0 = buffer_rsrc(W.base(false, l_g, static_cast<size_t>(N) * Kdim), wbytes);
    rb1 = buffer_rsrc(W.base(GATEUP, l_g, static_cast<size_t>(N) * Kdim), wbytes);
    bcol = static_cast<uint32_t>(l_ntile * kCols) * rowbytes;
  };
  set_weights();
  const uint32_t kb_end = static_cast<uint32_t>(nk) * G::kRow;
  uint32_t kb = 0;  // byte offset of the load side's next k-slice

  // ---- next item, fetched ahead: group record at slice 0 of the current
  // load-side item, row-tile record at slice 2, row indices sent at slice 4
  int nw = first + min(1, n_items - 1) * nslot;
  int f_group = 0, f_gstart = 0, f_ntiles = 1, f_m0 = 0, f_m1 = 0;
  int n_g = l_g, n_ntile = l_ntile, n_m0 = l_m0, n_nrows = l_nrows;

  // Moves the load side on by one slice into stage st.
  auto issue = [&](char* st) {
    if (kb == kb_end) {
      if (l_item + 1 < n_items) {
        ++l_item;
        kb = 0;
        l_g = n_g; l_ntile = n_ntile; l_m0 = n_m0; l_nrows = n_nrows;
        set_weights();
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
          const int sr = gather ? ri_lds[wave * 64 + kRPI * i + drow]
                                : l_m0 + kRPI * (wave + 8 * i) + drow;
          a_off[i] = a_offset(i, l_nrows, sr);
        }
        nw = first + min(l_item + 1, n_items - 1) * nslot;
      } else {
        kb = kb_end - G::kRow;  // past the last item: re-read its last slice (an L2 hit)
      }
    }
    const uint32_t lk = kb / G::kRow;
    if (lk == 0) {
      const TileInfo t = tiles[nw / NT];
      f_group = t.group;
      f_gstart = t.gstart;
      f_ntiles = max(t.ntiles, 1);
    } else if (lk == 2) {
      int mt;
      item_tile(nw - f_gstart * NT, f_ntiles, NT, mt, n_ntile);
      n_g = f_group;
      const TileInfo u = tiles[f_gstart + mt];
      f_m0 = u.m0;
      f_m1 = u.m1;
    } else if (lk == 4) {
      n_m0 = f_m0;
      n_nrows = min(f_m1 - f_m0, BM);
      if (GATEUP) {
        // lane l < 32: row kRPI * (wave + 8 * (l / kRPI)) + l % kRPI
        const int r = kRPI * (wave + 8 * (lane / kRPI)) + lane % kRPI;
        dma<4>(rsR, ri_lds + wave * 64,
               (lane < 32 && r < n_nrows) ? static_cast<uint32_t>(n_m0 + r) * 4u : kOff, 0);
      } else {
        const int r = wm * 64 + lane;
        dma<4>(rsS, sc_lds + (l_item & 1) * 512 + wave * 64,
               r < l_nrows ? static_cast<uint32_t>(l_m0 + r) * 4u : kOff, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < kNI; ++i)
      dma<16>(rsA, st + kRPI * (wave + 8 * i) * G::kRow, a_off[i], kb);
    // B tile row kRPI (wave + 8 i) + drow: W_gate rows over the matching W_up
    // rows (gate/up), or 256 consecutive W_down rows
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      const int add = GATEUP ? kRPI * 8 * (i % (kNI / 2)) : kRPI * 8 * i;
      dma<16, kWeightPolicy>((GATEUP && i >= kNI / 2) ? rb1 : rb0,
                             st + G::kTileBytes + kRPI * (wave + 8 * i) * G::kRow, b_off,
              bcol + static_cast<uint32_t>(add) * rowbytes + kb);
    }
    kb += G::kRow;
  };

  // ---- compute side (trails the load side by kStages - 1 slices)
  int c_item = 0, c_m0 = l_m0, c_nrows = l_nrows, c_n0 = l_ntile * kCols;

  int brow[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    if (GATEUP) {
      const int half = kNB / 2;
      const int base = wn * (BNW / 2 / kWavesN);
      brow[nb] = (nb < half) ? base + nb * 32 : BNW / 2 + base + (nb - half) * 32;
    } else {
      brow[nb] = wn * (BNW / kWavesN) + nb * 32;
    }
  }

  f32x16_t acc[2][kNB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mb][nb][q] = 0.0f;

  const int fr = lane & 31;
  const int fh = lane >> 5;

  // Wave (wm, wn) multiplies the 32-row blocks 2 wm and 2 wm + 1 (a block
  // with no row of the item is skipped) against its kNB weight blocks.
  //
  // Both 32-row blocks of a busy wave are multiplied (rows past the group hold
  // zeros in LDS and are never written out), so a step is one basic block:
  // the fragment reads of its second 32-k half are issued between the MFMAs
  // of the first half (one read after each MFMA), where their LDS latency is
  // covered, instead of after them.
  auto compute = [&](const char* st) {
    if (wm * 64 >= c_nrows) return;
    const char* bs = st + G::kTileBytes;
    bf16x8_t bq[BK / 32][2][kNB], aq[BK / 32][2][2];
#pragma unroll
    for (int kh = 0; kh < BK / 32; ++kh)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int c = kh * 4 + kk * 2 + fh;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          bq[kh][kk][nb] = *reinterpret_cast<const bf16x8_t*>(bs + G::swz(brow[nb] + fr, c));
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          aq[kh][kk][mb] = *reinterpret_cast<const bf16x8_t*>(st + G::swz(wm * 64 + mb * 32 + fr, c));
      }
#pragma unroll
    for (int kh = 0; kh < BK / 32; ++kh)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[kh][kk][mb], bq[kh][kk][nb],
                                                                  acc[mb][nb], 0, 0, 0);
    // order: the first 16-k step's reads, then each 16-k step's MFMAs with
    // the next step's reads one after each MFMA, then the last step's MFMAs
    constexpr int kReadsKK = kNB + 2;       // fragment reads of one 16-k step
    constexpr int kMfmaKK = 2 * kNB;        // its MFMAs
    constexpr int kSteps = BK / 16;
    static_assert(kReadsKK <= kMfmaKK, "one read after each MFMA of the step before");
    __builtin_amdgcn_sched_group_barrier(0x100, kReadsKK, 0);
#pragma unroll
    for (int st = 0; st + 1 < kSteps; ++st) {
#pragma unroll
      for (int i = 0; i < kReadsKK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kMfmaKK - kReadsKK, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfmaKK, 0);
  };

  // Output tile of the compute-side item, staged through the last stage (free
  // once every wave has multiplied it; the next slice into it is sent only
  // after the next step's barrier) in rounds of kRoundRows rows: bf16 rows of
  // kCols with the 16-byte chunk index XORed with (row & 4), then written as
  // whole 16-byte chunks.  D[row][col] of a 32x32 block sits in lane
  // (col + 32*((row/4)%2)), register (row%4) + 4*(row/8).
  constexpr int kOutRowBytes = kCols * 2;
  constexpr int kRoundRows =
      G::kStageBytes / kOutRowBytes < BM ? G::kStageBytes / kOutRowBytes : BM;
  constexpr int kOutChunks = kCols / 8;
  constexpr int kReadRows = NTHR / kOutChunks;
  static_assert(kRoundRows % 64 == 0 && BM % kRoundRows == 0, "rounds hold whole waves' rows");
  static_assert(NTHR % kOutChunks == 0 && kReadRows % 8 == 0, "read-out rows keep row & 4");
  auto epilogue = [&]() {
    // Lane constants are rederived here from the hardware lane id: hoisted
    // out of the item loop they would stay live through the inner loop.
    int ez = 0;  // opaque zero: keeps the lane-id computation inside the loop
    asm volatile("" : "+v"(ez));
    const int e_lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, ez));
    const int etid = wave * kWave + e_lane;
    const int e_fr = e_lane & 31, e_fh = e_lane >> 5;
    const float* sc = sc_lds + (c_item & 1) * 512 + wave * 64;
    char* const ot = st_last;
    // every wave has multiplied the last stage
    asm volatile("s_barrier" ::: "memory");
    // gate/up with AU: two more passes write a and u to au [rows, 2N]
    constexpr int npass = (GATEUP && AU) ? 3 : 1;
    for (int pass = 0; pass < npass; ++pass) {
#pragma unroll
    for (int r0 = 0; r0 < BM; r0 += kRoundRows) {
      if (r0 >= c_nrows) break;
      {
        int cofs[kNB];
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const int c = (GATEUP ? (nb < kNB / 2 ? wn * (BNW / 2 / kWavesN) + nb * 32
                                                : BNW / 2 + wn * (BNW / 2 / kWavesN) +
                                                      (nb - kNB / 2) * 32)
                                : wn * (BNW / kWavesN) + nb * 32) +
                        e_fr;
          cofs[nb] = (((c >> 3) ^ (4 * e_fh)) << 4) + (c & 7) * 2;
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          if (wm * 64 < r0 || wm * 64 >= r0 + kRoundRows) break;  // rows of another round
          // block row base, relative to the round, plus this lane's half (4 * fh)
          const int base = wm * 64 + mb * 32 - r0 + 4 * e_fh;
          char* ob = ot + base * kOutRowBytes;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            float4 s4 = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            if (has_scale)
              s4 = *reinterpret_cast<const float4*>(sc + mb * 32 + 8 * q4 + 4 * e_fh);
            const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int q1 = 0; q1 < 4; ++q1) {
              const int q = 4 * q4 + q1;
              // rows past the item are staged too (never written out)
              char* orow = ob + (8 * q4 + q1) * kOutRowBytes;
              if (GATEUP) {
#pragma unroll
                for (int nb = 0; nb < kNB / 2; ++nb) {
                  const float gv = acc[mb][nb][q], uv = acc[mb][nb + kNB / 2][q];
                  const float v = pass == 0 ? silu(gv) * uv : (pass == 1 ? gv : uv);
                  *reinterpret_cast<uint16_t*>(orow + cofs[nb]) = f32_to_bf16(v);
                }
              } else {
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb)
                  *reinterpret_cast<uint16_t*>(orow + cofs[nb]) =
                      f32_to_bf16(acc[mb][nb][q] * sv[q1]);
              }
            }
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const int rl = etid / kOutChunks, cl = etid % kOutChunks;
      const char* src = ot + rl * kOutRowBytes + ((cl ^ (rl & 4)) << 4);
      const size_t ldo = pass == 0 ? static_cast<size_t>(N) : 2 * static_cast<size_t>(N);
      uint16_t* dst = (pass == 0 ? out : au + (pass == 2 ? N : 0)) +
                      static_cast<size_t>(c_m0 + r0 + rl) * ldo + c_n0 + cl * 8;
#pragma unroll
      for (int it = 0; it < kRoundRows / kReadRows; ++it) {
        if (rl < c_nrows - r0 - it * kReadRows)
          *reinterpret_cast<uint4*>(dst + static_cast<size_t>(it) * kReadRows * ldo) =
              *reinterpret_cast<const uint4*>(src + it * kReadRows * kOutRowBytes);
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    }
  };

  // ---- stream: the first kStages - 1 slices in flight, then per step: wait
  // for this step's slice (the newer slices, 2 kNI loads per lane each, may
  // stay in flight), barrier, send the next slice into the stage freed by the
  // previous step, multiply.  nk is a multiple of the stage count, so every
  // item starts on stage 0 and ends on the last.
#define MOE_STEP(CUR, NEXT)                                                                 \
  if constexpr (G::kStages == 4)                                                            \
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(4 * kNI) : "memory");             \
  else                                                                                      \
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");                           \
  issue(NEXT);                                                                              \
  compute(CUR);
  if constexpr (G::kStages == 4) {
    issue(st0);
    issue(st1);
    issue(st2);
  } else {
    issue(st0);
  }
  for (int j = 0; j < n_items; ++j) {
    if constexpr (G::kStages == 4) {
      for (int kt = 0; kt < nk; kt += 4) {
        MOE_STEP(st0, st3)
        MOE_STEP(st1, st0)
        MOE_STEP(st2, st1)
        MOE_STEP(st3, st2)
      }
    } else {
      for (int kt = 0; kt < nk; kt += 2) {
        MOE_STEP(st0, st1)
        MOE_STEP(st1, st0)
      }
    }
    epilogue();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.0f;
    ++c_item;
    c_m0 = l_m0;
    c_nrows = l_nrows;
    c_n0 = l_ntile * kCols;
  }
#undef MOE_STEP
  // the re-read slices of the last steps must land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Shapes the streaming kernel takes: K a multiple of 128 with at least
// kMinStreamSlices slices, N a multiple of its column tile.
bool stream_shape(int K, int N, int cols) {
  return K % 128 == 0 && K / kStreamBK >= kMinStreamSlices && N % cols == 0;
}

// ---------------------------------------------------------------- streaming, register-staged
//
// One workgroup per CU, each walking a fixed list of work items: the items of
// an XCD (the same XCD-contiguous runs as above) are dealt round-robin to its
// workgroups.  A workgroup streams the k-slices of its items back to back
// through the same two register sets and two LDS stages, so the first slices
// of the next item are in flight while the last slice of the current one is
// multiplied and its output tile written: no CU idles through an item's
// set-up loads or its epilogue, and there is no launch gap between items.
// The next item's tile records and gathered row indices are fetched a few
// slices ahead by loads issued on every step (branch-free, so the compiler's
// wait counts stay exact).  Used when K is an even number of at least
// kMinStreamSlices slices and N is a multiple of the column tile.

template <bool GATEUP, int BM, int BNW, int NTHR, bool AU = false>
__global__ __launch_bounds__(NTHR)
__attribute__((amdgpu_waves_per_eu(Tile<BM, BNW, NTHR>::kWavesPerEU,
                                   Tile<BM, BNW, NTHR>::kWavesPerEU)))
void bf16_regs_stream_kernel(
    int Kdim, int N, int x_rows, int rows, int max_tiles, int NT,
    const TileInfo* __restrict__ tiles, const int32_t* __restrict__ meta,
    const int32_t* __restrict__ row_index, const uint16_t* __restrict__ A, const WeightSet W,
    const float* __restrict__ row_scale, uint16_t* __restrict__ out, uint16_t* __restrict__ au) {
  using TL = Tile<BM, BNW, NTHR>;
  constexpr int kALoads = TL::kALoads;
  constexpr int kBLoads = TL::kBLoads;
  constexpr int kNB = TL::kNB;
  constexpr int kRP = TL::kRowsPerPass;
  constexpr int kCols = GATEUP ? BNW / 2 : BNW;
  constexpr uint32_t kOff = 0x80000000u;  // beyond every buffer (sizes < 2 GiB)
  static_assert(kCols % kRP == 0, "a load pass must not straddle the gate/up halves");
  __shared__ __attribute__((aligned(16))) char smem[2 * TL::kStageBytes];

  // ---- this workgroup's items: first, first + nslot, ... below end
  const int total = meta[0] * NT;
  const int nslot = gridDim.x / kNumXcd;
  const int xcd = blockIdx.x % kNumXcd;
  const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int first = xcd * per_xcd + static_cast<int>(blockIdx.x) / kNumXcd;
  const int end = min(total, (xcd + 1) * per_xcd);
  if (first >= end) return;
  const int n_items = (end - first + nslot - 1) / nslot;
  const int nk = Kdim / kBK;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: scalar
  const int lane = tid % kWave;
  const int wm = wave / TL::kWavesN, wn = wave % TL::kWavesN;
  const int lc = tid & 7;
  const int lr = tid >> 3;  // 0 .. kRP-1
  const uint32_t rowbytes = static_cast<uint32_t>(Kdim) * 2u;
  const uint32_t wbytes = static_cast<uint32_t>(N) * rowbytes;
  const __amdgpu_buffer_rsrc_t rsA = buffer_rsrc(A, static_cast<uint32_t>(x_rows) * rowbytes);
  const __amdgpu_buffer_rsrc_t rsT =
      buffer_rsrc(tiles, static_cast<uint32_t>(max_tiles) * sizeof(TileInfo));
  // gate/up gathers x rows through row_index (NULL: grouped row r is x row r);
  // without it every row-index load is out of range and reads nothing
  const bool gather = GATEUP && row_index != nullptr;
  const __amdgpu_buffer_rsrc_t rsR =
      buffer_rsrc(row_index, gather ? static_cast<uint32_t>(rows) * 4u : 0u);

  // A-tile offset of load slot i (tile row lr + kRP * i, source row sr) of an
  // item with nrows rows; the row test is written as lr < nrows - kRP * i so
  // that no per-slot row value has to stay in a register.
  auto a_offset = [&](int i, int nrows, int sr) -> uint32_t {
    return (lr < nrows - kRP * i && sr >= 0 && sr < x_rows)
               ? static_cast<uint32_t>(sr) * rowbytes + static_cast<uint32_t>(lc) * 16u
               : kOff;
  };

  // ---- load-side item: its group, column tile, rows and per-lane offsets
  int l_item = 0, l_g, l_ntile, l_m0, l_nrows;
  {
    const int w = first;
    const TileInfo t0 = tiles[w / NT];
    int mt;
    item_tile(w - t0.gstart * NT, max(t0.ntiles, 1), NT, mt, l_ntile);
    const TileInfo ti = tiles[t0.gstart + mt];
    l_g = t0.group;
    l_m0 = ti.m0;
    l_nrows = min(ti.m1 - ti.m0, BM);
  }
  uint32_t a_off[kALoads];
#pragma unroll
  for (int i = 0; i < kALoads; ++i) {
    const int r = lr + kRP * i;
    int sr = l_m0 + r;
    if (gather) sr = (r < l_nrows) ? row_index[l_m0 + r] : -1;
    a_off[i] = a_offset(i, l_nrows, sr);
  }
  // B-tile row of load slot i is lr + boff(i); GATEUP stacks gate rows over
  // the matching up rows, so slots of the second half repeat the first's rows.
  auto b_row_add = [&](int i) -> uint32_t {
    const int add = GATEUP ? (kRP * i) % (BNW / 2) : kRP * i;
    return static_cast<uint32_t>(add) * rowbytes;
  };

  // Weights of the load-side item and the byte offset of its column tile
  // (set per item); the lane's own B row and chunk stay in bb.
  __amdgpu_buffer_rsrc_t rb0, rb1;
  uint32_t bcol;
  const uint32_t bb = static_cast<uint32_t>(lr) * rowbytes + static_cast<uint32_t>(lc) * 16u;
  auto set_weights = [&]() {
    rb0 = buffer_rsrc(W.base(false, l_g, static_cast<size_t>(N) * Kdim), wbytes);
    rb1 = buffer_rsrc(W.base(GATEUP, l_g, static_cast<size_t>(N) * Kdim), wbytes);
    bcol = static_cast<uint32_t>(l_ntile * kCols) * rowbytes;
  };
  set_weights();
  const uint32_t kb_end = static_cast<uint32_t>(nk) * kBK * 2u;
  uint32_t kb = 0;  // byte offset of the load side's next k-slice

#define MOE_LOAD_SLICE(SA, SB)                                                               \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < kALoads; ++i) SA[i] =                             \
        __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsA, a_off[i], kb, 0)); \
    _Pragma("unroll") for (int i = 0; i < kBLoads; ++i) SB[i] = __builtin_bit_cast(          \
        uint4, __builtin_amdgcn_raw_buffer_load_b128((!GATEUP || i < kBLoads / 2) ? rb0 : rb1, \
                                                     bb, bcol + kb + b_row_add(i),         \
                                                     kWeightPolicy));                      \
    kb += kBK * 2;                                                                          \
  } while (0)
#define MOE_STORE_SLICE(SA, SB, STAGE)                                                      \
  do {                                                                                      \
    char* as_ = smem + (STAGE) * TL::kStageBytes;                                           \
    char* bs_ = as_ + TL::kABytes;                                                          \
    _Pragma("unroll") for (int i = 0; i < kALoads; ++i)                                     \
        *reinterpret_cast<uint4*>(as_ + swz(lr + kRP * i, lc)) = SA[i];                     \
    _Pragma("unroll") for (int i = 0; i < kBLoads; ++i)                                     \
        *reinterpret_cast<uint4*>(bs_ + swz(lr + kRP * i, lc)) = SB[i];                     \
  } while (0)
  // ---- next item, fetched ahead.  p holds, in lane l, dword (l & 7) of the
  // tile record of the next item's group start (lanes with l & 8 == 0) or of
  // its row tile (l & 8 != 0); ri holds, in lane j + 8 i, the source row of
  // tile row 8 * wave + j + kRP * i (the rows this wave's load slots need).
  // Both are refetched on every other step, after that step's slice loads,
  // and read back two steps later: a wait for them then covers only slices
  // that were due anyway, and the loop stays branch-free around its loads
  // (so the compiler's wait counts stay exact).  After the next item changes,
  // the group record is read one fetch later, the row-tile record two and the
  // row indices three.
  static_assert(kALoads * 8 <= kWave, "one lane per gathered row of the wave");
  int p = 0, ri = -1;
  int n_g = 0, n_ntile = 0, n_m0 = 0, n_nrows = 0;
  int nw = first + min(1, n_items - 1) * nslot;  // next item
  int t0rec = nw / NT;                           // a tile of its group
  int rec = 0;                                   // its row tile
  int fa = 0;                                    // fetches since nw changed

  // Read the records fetched two steps ago, and move the load side to the
  // next item once all slices of the current one are issued.
#define MOE_ADVANCE()                                                                       \
  do {                                                                                      \
    if (fa == 1) { /* the group record just arrived: locate the row tile */                 \
      const int gstart_ = __builtin_amdgcn_readlane(p, 3);                                  \
      const int gnt_ = max(__builtin_amdgcn_readlane(p, 4), 1);                             \
      int mt_;                                                                              \
      item_tile(nw - gstart_ * NT, gnt_, NT, mt_, n_ntile);                                 \
      n_g = __builtin_amdgcn_readlane(p, 0);                                                \
      rec = gstart_ + mt_;                                                                  \
    }                                                                                       \
    n_m0 = __builtin_amdgcn_readlane(p, 9);                                                 \
    n_nrows = min(__builtin_amdgcn_readlane(p, 10) - n_m0, BM);                             \
    if (kb == kb_end) {                                                                     \
      if (l_item + 1 < n_items) {                                                           \
        ++l_item;                                                                           \
        kb = 0;                                                                             \
        l_g = n_g; l_ntile = n_ntile; l_m0 = n_m0; l_nrows = n_nrows;                       \
        set_weights();                                                                      \
        _Pragma("unroll") for (int i = 0; i < kALoads; ++i) {                               \
          const int sr_ = gather ? __builtin_amdgcn_ds_bpermute(((lane >> 3) + 8 * i) * 4, ri) \
                                 : l_m0 + kRP * i + lr;                                     \
          a_off[i] = a_offset(i, l_nrows, sr_);                                             \
        }                                                                                   \
        nw = first + min(l_item + 1, n_items - 1) * nslot;                                  \
        t0rec = nw / NT;                                                                    \
        fa = 0;                                                                             \
      } else {                                                                              \
        kb = kb_end - kBK * 2; /* past the last item: re-read its last slice (an L2 hit) */ \
      }                                                                                     \
    }                                                                                       \
  } while (0)
  // Refetch the next item's records and row indices (the lane id is
  // recomputed rather than kept in a register through the loop).
#define MOE_FETCH()                                                                         \
  do {                                                                                      \
    int z_ = 0;                                                                             \
    asm volatile("" : "+v"(z_));                                                            \
    const int ln_ = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, z_));     \
    if (GATEUP) { /* without row_index every load is out of range: no branch */             \
      const int r_ = wave * 8 + (ln_ & 7) + kRP * ((ln_ >> 3) & (kALoads - 1));             \
      ri = __builtin_amdgcn_raw_buffer_load_b32(                                            \
          rsR, r_ < n_nrows ? static_cast<uint32_t>(n_m0 + r_) * 4u : kOff, 0, 0);          \
    }                                                                                       \
    p = __builtin_amdgcn_raw_buffer_load_b32(                                               \
        rsT, static_cast<uint32_t>((ln_ & 8) ? rec : t0rec) * 32u + (ln_ & 7) * 4u, 0, 0);  \
    fa = min(fa + 1, 3);                                                                    \
  } while (0)

  // ---- compute-side item (trails the load side by two slices)
  int c_m0 = l_m0, c_nrows = l_nrows, c_n0 = l_ntile * kCols;

  int brow[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    if (GATEUP) {
      const int half = kNB / 2;
      const int base = wn * (BNW / 2 / TL::kWavesN);
      brow[nb] = (nb < half) ? base + nb * 32 : BNW / 2 + base + (nb - half) * 32;
    } else {
      brow[nb] = wn * (BNW / TL::kWavesN) + nb * 32;
    }
  }

  f32x16_t acc[2][kNB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mb][nb][q] = 0.0f;

  const int fr = lane & 31;
  const int fh = lane >> 5;

  // Wave (wm, wn) multiplies the 32-row blocks 2 wm and 2 wm + 1.  The LDS
  // fragments of k-step kk + 1 are read while the MFMAs of kk run (two
  // fragment buffers), so the LDS latency is not exposed per k-step.
  auto compute = [&](int stage) {
    const bool mb0 = wm * 64 < c_nrows;
    const bool mb1 = wm * 64 + 32 < c_nrows;
    if (!mb0) return;
    const char* as = smem + stage * TL::kStageBytes;
    const char* bs = as + TL::kABytes;
    bf16x8_t bq[2][kNB], aq[2][2];
#define MOE_FRAGS(KK, BUF)                                                                  \
  do {                                                                                      \
    const int c_ = (KK) * 2 + fh;                                                           \
    _Pragma("unroll") for (int nb = 0; nb < kNB; ++nb) bq[BUF][nb] =                        \
        *reinterpret_cast<const bf16x8_t*>(bs + swz(brow[nb] + fr, c_));                    \
    aq[BUF][0] = *reinterpret_cast<const bf16x8_t*>(as + swz(wm * 64 + fr, c_));            \
    if (mb1) aq[BUF][1] = *reinterpret_cast<const bf16x8_t*>(as + swz(wm * 64 + 32 + fr, c_)); \
  } while (0)
    MOE_FRAGS(0, 0);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < kBK / 16) MOE_FRAGS(kk + 1, cur ^ 1);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        acc[0][nb] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[cur][0], bq[cur][nb], acc[0][nb], 0, 0, 0);
      if (mb1) {
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[cur][1], bq[cur][nb],
                                                               acc[1][nb], 0, 0, 0);
      }
    }
#undef MOE_FRAGS
  };

  // Output tile of the compute-side item, staged through LDS stage `stage`
  // (free once every wave has multiplied it) in rounds of kRoundRows rows:
  // bf16 rows of kCols with the 16-byte chunk index XORed with (row & 4), then
  // written as whole 16-byte chunks.  D[row][col] of a 32x32 block sits in
  // lane (col + 32*((row/4)%2)), register (row%4) + 4*(row/8).
  constexpr int kOutRowBytes = kCols * 2;
  constexpr int kRoundRows = (BM * kOutRowBytes <= TL::kStageBytes) ? BM
                                                                    : TL::kStageBytes / kOutRowBytes;
  constexpr int kOutChunks = kCols / 8;
  static_assert(kRoundRows % 64 == 0 && BM % kRoundRows == 0, "rounds hold whole waves' rows");
  // Row of (mb, q) is wm*64 + mb*32 + 8*(q/4) + 4*fh + q%4, so (row & 4) is
  // 4*fh in every register and each LDS write is a per-lane base plus a
  // constant; the read-out rows of iteration `it` are it * (NTHR / kOutChunks)
  // + tid / kOutChunks, again a per-lane base plus a constant.
  auto epilogue = [&](int stage) {
    // Lane constants are rederived here from the hardware lane id: hoisted
    // out of the item loop they would stay live through the inner loop, which
    // needs every register.
    int ez = 0;  // opaque zero: keeps the lane-id computation inside the loop
    asm volatile("" : "+v"(ez));
    const int e_lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, ez));
    const int e_wave = wave;
    const int etid = e_wave * kWave + e_lane;
    const int e_wm = e_wave / TL::kWavesN, e_wn = e_wave % TL::kWavesN;
    const int e_fr = e_lane & 31, e_fh = e_lane >> 5;
    char* ot = smem + stage * TL::kStageBytes;
    constexpr int kReadRows = NTHR / kOutChunks;
    static_assert(NTHR % kOutChunks == 0 && kReadRows % 8 == 0, "read-out rows keep row & 4");
    static_assert(kRoundRows % 64 == 0 && BM % kRoundRows == 0, "rounds hold whole waves' rows");
    // gate/up with AU: two more passes write a and u to au [rows, 2N]
    constexpr int npass = (GATEUP && AU) ? 3 : 1;
    for (int pass = 0; pass < npass; ++pass) {
#pragma unroll
    for (int r0 = 0; r0 < BM; r0 += kRoundRows) {
      if (r0 >= c_nrows) break;
      {
        int cofs[kNB];
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const int c = (GATEUP ? (nb < kNB / 2 ? e_wn * (BNW / 2 / TL::kWavesN) + nb * 32
                                                : BNW / 2 + e_wn * (BNW / 2 / TL::kWavesN) +
                                                      (nb - kNB / 2) * 32)
                                : e_wn * (BNW / TL::kWavesN) + nb * 32) +
                        e_fr;
          cofs[nb] = (((c >> 3) ^ (4 * e_fh)) << 4) + (c & 7) * 2;
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          if (e_wm * 64 < r0 || e_wm * 64 >= r0 + kRoundRows) break;  // rows of another round
          // block row base, relative to the round, plus this lane's half (4 * fh)
          const int base = e_wm * 64 + mb * 32 - r0 + 4 * e_fh;
          char* ob = ot + base * kOutRowBytes;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            // rows past the item are staged too (never written out)
            const int rr = 8 * (q >> 2) + (q & 3);
            char* orow = ob + rr * kOutRowBytes;
            if (GATEUP) {
#pragma unroll
              for (int nb = 0; nb < kNB / 2; ++nb) {
                const float gv = acc[mb][nb][q], uv = acc[mb][nb + kNB / 2][q];
                const float v = pass == 0 ? silu(gv) * uv : (pass == 1 ? gv : uv);
                *reinterpret_cast<uint16_t*>(orow + cofs[nb]) = f32_to_bf16(v);
              }
            } else if (row_scale == nullptr) {
#pragma unroll
              for (int nb = 0; nb < kNB; ++nb)
                *reinterpret_cast<uint16_t*>(orow + cofs[nb]) = f32_to_bf16(acc[mb][nb][q]);
            } else {  // waits on its loads, so stalls the stream once per item
              // (row < c_nrows) as (lane base < c_nrows - rr): no per-row registers
              const int row0 = base + r0;
              const float sc = row0 < c_nrows - rr ? row_scale[c_m0 + row0 + rr] : 1.0f;
#pragma unroll
              for (int nb = 0; nb < kNB; ++nb)
                *reinterpret_cast<uint16_t*>(orow + cofs[nb]) = f32_to_bf16(acc[mb][nb][q] * sc);
            }
          }
        }
      }
      __syncthreads();
      const int rl = etid / kOutChunks, cl = etid % kOutChunks;
      const char* src = ot + rl * kOutRowBytes + ((cl ^ (rl & 4)) << 4);
      const size_t ldo = pass == 0 ? static_cast<size_t>(N) : 2 * static_cast<size_t>(N);
      uint16_t* dst = (pass == 0 ? out : au + (pass == 2 ? N : 0)) +
                      static_cast<size_t>(c_m0 + r0 + rl) * ldo + c_n0 + cl * 8;
#pragma unroll
      for (int it = 0; it < kRoundRows / kReadRows; ++it) {
        if (rl < c_nrows - r0 - it * kReadRows)
          *reinterpret_cast<uint4*>(dst + static_cast<size_t>(it) * kReadRows * ldo) =
              *reinterpret_cast<const uint4*>(src + it * kReadRows * kOutRowBytes);
      }
      __syncthreads();
    }
    }
  };

  // ---- stream: each step loads the slice two ahead into the register set
  // stored by the previous step, stores the next slice (loaded one step ago)
  // to the other LDS stage, and multiplies one slice out of its stage; the LDS
  // writes drain under the MFMAs, and the stored set is free during them.  nk is even, so every item starts on
  // stage 1 and ends on stage 0, where its output tile is then staged (at LDS
  // offset 0, so the staging offsets fit the instructions' 16-bit immediate).
  uint4 sa0[kALoads], sb0[kBLoads], sa1[kALoads], sb1[kBLoads];
  MOE_LOAD_SLICE(sa0, sb0);
  MOE_LOAD_SLICE(sa1, sb1);
  MOE_STORE_SLICE(sa0, sb0, 1);
  __syncthreads();
  // The load side changes item only on the first step of a pair (nk is even),
  // so that step also advances and refetches the fetch-ahead.
  for (int j = 0; j < n_items; ++j) {
    for (int kt = 0; kt < nk; kt += 2) {
      MOE_ADVANCE();
      MOE_LOAD_SLICE(sa0, sb0);
      MOE_FETCH();
      MOE_STORE_SLICE(sa1, sb1, 0);
      compute(1);
      __syncthreads();
      MOE_LOAD_SLICE(sa1, sb1);
      MOE_STORE_SLICE(sa0, sb0, 1);
      compute(0);
      __syncthreads();
    }
    epilogue(0);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.0f;
    c_m0 = l_m0;
    c_nrows = l_nrows;
    c_n0 = l_ntile * kCols;
  }
#undef MOE_ADVANCE
#undef MOE_FETCH
#undef MOE_LOAD_SLICE
#undef MOE_STORE_SLICE
}

// ---------------------------------------------------------------- streaming, weights by LDS DMA
//
// The register-staged kernel with its weight side moved out of registers:
// each weight slice (256 rows x 64 k, 32 KB) goes from memory straight into
// one of three LDS stages by buffer loads with an LDS destination, two slices
// ahead of the multiply, while the x rows keep the register path (coalesced
// 16-byte loads, one register set, two LDS stages).  A step stores the x rows
// of the next slice (loaded one step earlier) to LDS, loads the rows of the
// slice after it, sends that slice's weights, multiplies, then waits for the
// weights of the next slice and meets the barrier.  Loads complete in order
// and each step issues its row loads before its weight loads, so neither
// wait covers the newest weight slice: every weight slice has about two steps
// to arrive (the register-staged kernel gives it one).  The weight stages
// rotate through the slices of all items back to back (the step loop is
// unrolled over the three stages, so the stage of each step is known when
// compiling), and an item may end on any of the three: each unrolled step
// closes the item when its last slice has been multiplied.  The row stages
// alternate at run time.  The MFMAs take the weight fragment first,
// so the epilogue packs four consecutive output columns per 8-byte LDS write.
// Every LDS access keeps its alias scope: an LDS access the compiler cannot
// tell apart from the weight stages would wait for every weight slice in
// flight.  Used for groups of fewer rows than a tile on average (weight
// streaming) when K has at least kWdmaMinSlices slices.
constexpr int kWdmaStages = 3;
// The next item's records are fetched on every third step and reach the load
// side through three dependent fetches (group record, row-tile record, row
// indices), the first of them up to two steps after the item changed: the
// load side may move on again 11 steps after it last did, so an item needs at
// least that many slices.
constexpr int kWdmaMinSlices = 12;

template <bool GATEUP, bool AU = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bf16_wdma_kernel(
    int Kdim, int N, int x_rows, int rows, int max_tiles, int NT,
    const TileInfo* __restrict__ tiles, const int32_t* __restrict__ meta,
    const int32_t* __restrict__ row_index, const uint16_t* __restrict__ A, const WeightSet W,
    uint16_t* __restrict__ out, uint16_t* __restrict__ au) {
  using G = StreamGeom<64>;
  using TL = Tile<256, 256, 512>;
  constexpr int BM = 256, BNW = 256, NTHR = 512;
  constexpr int kALoads = TL::kALoads;
  constexpr int kNB = TL::kNB;
  constexpr int kRP = TL::kRowsPerPass;
  constexpr int kWavesN = TL::kWavesN;
  constexpr int kCols = GATEUP ? BNW / 2 : BNW;
  constexpr int kNI = G::kNI, kRPI = G::kRPI;  // weight loads per wave and slice, rows per load
  constexpr uint32_t kOff = 0x80000000u;       // beyond every buffer (sizes < 2 GiB)
  constexpr int kTile = G::kTileBytes;         // one 256-row operand tile of a slice
  static_assert(kWdmaStages == 3, "the step loop is unrolled over three weight stages");
  __shared__ __attribute__((aligned(16))) char a_st[2 * kTile];  // x-row stages (LDS writes)
  __shared__ __attribute__((aligned(16))) char b0[kTile];        // weight stages (LDS DMA)
  __shared__ __attribute__((aligned(16))) char b1[kTile];
  __shared__ __attribute__((aligned(16))) char b2[kTile];

  // ---- this workgroup's items: first, first + nslot, ... below end
  const int total = meta[0] * NT;
  const int nslot = gridDim.x / kNumXcd;
  const int xcd = blockIdx.x % kNumXcd;
  const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int first = xcd * per_xcd + static_cast<int>(blockIdx.x) / kNumXcd;
  const int end = min(total, (xcd + 1) * per_xcd);
  if (first >= end) return;
  const int n_items = (end - first + nslot - 1) / nslot;
  const int nk = Kdim / kBK;  // at least kWdmaMinSlices

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: scalar
  const int lane = tid % kWave;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int lc = tid & 7;
  const int lr = tid >> 3;  // 0 .. kRP-1
  const uint32_t rowbytes = static_cast<uint32_t>(Kdim) * 2u;
  const uint32_t wbytes = static_cast<uint32_t>(N) * rowbytes;
  const uint32_t kb_end = static_cast<uint32_t>(nk) * kBK * 2u;  // past the last slice
  const __amdgpu_buffer_rsrc_t rsA = buffer_rsrc(A, static_cast<uint32_t>(x_rows) * rowbytes);
  const __amdgpu_buffer_rsrc_t rsT =
      buffer_rsrc(tiles, static_cast<uint32_t>(max_tiles) * sizeof(TileInfo));
  const bool gather = GATEUP && row_index != nullptr;
  const __amdgpu_buffer_rsrc_t rsR =
      buffer_rsrc(row_index, gather ? static_cast<uint32_t>(rows) * 4u : 0u);

  // x-row offset of load slot i (tile row lr + kRP * i, source row sr)
  auto a_offset = [&](int i, int nrows, int sr) -> uint32_t {
    return (lr < nrows - kRP * i && sr >= 0 && sr < x_rows)
               ? static_cast<uint32_t>(sr) * rowbytes + static_cast<uint32_t>(lc) * 16u
               : kOff;
  };

  // ---- load-side item
  int l_item = 0, l_g, l_ntile, l_m0, l_nrows;
  {
    const TileInfo t0 = tiles[first / NT];
    int mt;
    item_tile(first - t0.gstart * NT, max(t0.ntiles, 1), NT, mt, l_ntile);
    const TileInfo ti = tiles[t0.gstart + mt];
    l_g = t0.group;
    l_m0 = ti.m0;
    l_nrows = min(ti.m1 - ti.m0, BM);
  }
  // x-row loads a step issues for the load-side item: only those of row
  // passes that hold rows of the item (a load whose every lane is out of range
  // still costs an issue slot and address-unit time).  The rows of the passes
  // left out keep stale values in LDS; only waves with no row of the item
  // would read them, and those skip their multiply.
  static_assert(kALoads == 4, "the step's waits below are written for four row passes");
  auto x_loads = [](int nrows) { return min(max((nrows + kRP - 1) / kRP, 1), kALoads); };
  int l_na = x_loads(l_nrows);
  uint32_t a_off[kALoads];
#pragma unroll
  for (int i = 0; i < kALoads; ++i) {
    const int r = lr + kRP * i;
    int sr = l_m0 + r;
    if (gather) sr = (r < l_nrows) ? row_index[l_m0 + r] : -1;
    a_off[i] = a_offset(i, l_nrows, sr);
  }
  // Weight-slice load i of a wave sends tile rows kRPI (wave + 8 i) + drow;
  // lane l lands at LDS chunk l % 8 of its row, so it loads the k chunk that
  // the swizzle stores there.
  const int drow = lane / G::kChunks;
  const int dchunk = (lane % G::kChunks) ^ drow ^ (wave & 1);
  const uint32_t b_off = static_cast<uint32_t>(kRPI * wave + drow) * rowbytes +
                         static_cast<uint32_t>(dchunk) * 16u;
  __amdgpu_buffer_rsrc_t rb0, rb1;
  uint32_t bcol;
  auto set_weights = [&]() {
    rb0 = buffer_rsrc(W.base(false, l_g, static_cast<size_t>(N) * Kdim), wbytes);
    rb1 = buffer_rsrc(W.base(GATEUP, l_g, static_cast<size_t>(N) * Kdim), wbytes);
    bcol = static_cast<uint32_t>(l_ntile * kCols) * rowbytes;
  };
  set_weights();
  uint32_t kb = 0;  // byte offset of the load side's next k-slice

  // Loads the x rows of the load side's slice into sa, then sends its weight
  // slice into stage ST.
  uint4 sa[kALoads] = {};
#define MOE_WLOAD(ST)                                                                        \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < kALoads; ++i) if (i < l_na) sa[i] =               \
        __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsA, a_off[i], kb, 0)); \
    __builtin_amdgcn_sched_barrier(0); /* rows before weights: see the step's waits */      \
    _Pragma("unroll") for (int i = 0; i < kNI; ++i) {                                       \
      const int add_ = GATEUP ? kRPI * 8 * (i % (kNI / 2)) : kRPI * 8 * i;                  \
      dma16_unscoped<kWeightPolicy>((GATEUP && i >= kNI / 2) ? rb1 : rb0,                   \
                             (ST) + kRPI * (wave + 8 * i) * G::kRow, b_off,                   \
                             bcol + static_cast<uint32_t>(add_) * rowbytes + kb);           \
    }                                                                                       \
    kb += kBK * 2;                                                                          \
  } while (0)
#define MOE_WSTORE(AST)                                                                      \
  do {                                                                                      \
    char* as_ = a_st + (AST) * kTile;                                                       \
    _Pragma("unroll") for (int i = 0; i < kALoads; ++i)                                     \
        *reinterpret_cast<uint4*>(as_ + swz(lr + kRP * i, lc)) = sa[i];                     \
  } while (0)

  // ---- next item, fetched ahead (as in the register-staged kernel): p holds,
  // in lane l, dword (l & 7) of the tile record of the next item's group
  // start (l & 8 == 0) or of its row tile (l & 8 != 0); ri holds, in lane
  // j + 8 i, the source row of tile row 8 * wave + j + kRP * i.  Refetched on
  // every third step, after that step's loads, and read three steps later
  // (ri into ri_l, which the load side takes when it changes item, on any
  // step).  After the next item changes, the group record is read one fetch
  // later, the row-tile record two and the row indices three.
  static_assert(kALoads * 8 <= kWave, "one lane per gathered row of the wave");
  int p = 0, ri = -1, ri_l = -1;
  int n_g = 0, n_ntile = 0, n_m0 = 0, n_nrows = 0;
  int nw = first + min(1, n_items - 1) * nslot;  // next item
  int t0rec = nw / NT;                           // a tile of its group
  int rec = 0;                                   // its row tile
  int fa = 0;                                    // fetches since nw changed

  // Read the records and row indices fetched three steps ago.
#define MOE_WDECODE()                                                                        \
  do {                                                                                      \
    if (fa == 1) { /* the group record just arrived: locate the row tile */                 \
      const int gstart_ = __builtin_amdgcn_readlane(p, 3);                                  \
      const int gnt_ = max(__builtin_amdgcn_readlane(p, 4), 1);                             \
      int mt_;                                                                              \
      item_tile(nw - gstart_ * NT, gnt_, NT, mt_, n_ntile);                                 \
      n_g = __builtin_amdgcn_readlane(p, 0);                                                \
      rec = gstart_ + mt_;                                                                  \
    }                                                                                       \
    n_m0 = __builtin_amdgcn_readlane(p, 9);                                                 \
    n_nrows = min(__builtin_amdgcn_readlane(p, 10) - n_m0, BM);                             \
    if (GATEUP) /* a register of its own: ri's is then free for the next fetch */            \
      asm volatile("v_mov_b32 %0, %1" : "=&v"(ri_l) : "v"(ri));                             \
  } while (0)
  // Move the load side to the next item once all slices of the current one
  // are issued.
#define MOE_WSWITCH()                                                                        \
  do {                                                                                      \
    if (kb == kb_end) {                                                                     \
      if (l_item + 1 < n_items) {                                                           \
        ++l_item;                                                                           \
        kb = 0;                                                                             \
        l_g = n_g; l_ntile = n_ntile; l_m0 = n_m0; l_nrows = n_nrows;                       \
        l_na = x_loads(l_nrows);                                                            \
        set_weights();                                                                      \
        _Pragma("unroll") for (int i = 0; i < kALoads; ++i) {                               \
          const int sr_ = gather ? __builtin_amdgcn_ds_bpermute(((lane >> 3) + 8 * i) * 4, ri_l) \
                                 : l_m0 + kRP * i + lr;                                     \
          a_off[i] = a_offset(i, l_nrows, sr_);                                             \
        }                                                                                   \
        nw = first + min(l_item + 1, n_items - 1) * nslot;                                  \
        t0rec = nw / NT;                                                                    \
        fa = 0;                                                                             \
      } else {                                                                              \
        kb = kb_end - kBK * 2; /* past the last item: its last slice again */               \
      }                                                                                     \
    }                                                                                       \
  } while (0)
#define MOE_WFETCH()                                                                         \
  do {                                                                                      \
    int z_ = 0;                                                                             \
    asm volatile("" : "+v"(z_));                                                            \
    const int ln_ = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, z_));     \
    if (GATEUP) { /* without row_index every load is out of range: no branch */             \
      const int r_ = wave * 8 + (ln_ & 7) + kRP * ((ln_ >> 3) & (kALoads - 1));             \
      ri = __builtin_amdgcn_raw_buffer_load_b32(                                            \
          rsR, r_ < n_nrows ? static_cast<uint32_t>(n_m0 + r_) * 4u : kOff, 0, 0);          \
    }                                                                                       \
    p = __builtin_amdgcn_raw_buffer_load_b32(                                               \
        rsT, static_cast<uint32_t>((ln_ & 8) ? rec : t0rec) * 32u + (ln_ & 7) * 4u, 0, 0);  \
    fa = min(fa + 1, 3);                                                                    \
  } while (0)

  // ---- compute side (trails the load side by two slices)
  int c_m0 = l_m0, c_nrows = l_nrows, c_n0 = l_ntile * kCols;
  int gk = 0;  // steps so far: the x-row stage of step gk is gk & 1

  int brow[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    if (GATEUP) {
      const int half = kNB / 2;
      const int base = wn * (BNW / 2 / kWavesN);
      brow[nb] = (nb < half) ? base + nb * 32 : BNW / 2 + base + (nb - half) * 32;
    } else {
      brow[nb] = wn * (BNW / kWavesN) + nb * 32;
    }
  }

  f32x16_t acc[2][kNB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mb][nb][q] = 0.0f;

  const int fr = lane & 31;
  const int fh = lane >> 5;
  constexpr int kSteps = kBK / 16;

  // Wave (wm, wn) multiplies its two 32-row blocks (rows past the item hold
  // zeros or stale rows, never written out) by its kNB weight blocks; a wave
  // with no row of the item skips.  MFMAs weight block by weight block, both
  // row blocks each, the weight fragment first; the fragments of 16-k step
  // kk + 1 are read between the MFMAs of step kk.
  auto compute = [&](const char* as, const char* bs) {
    if (wm * 64 >= c_nrows) return;
    bf16x8_t bq[kSteps][kNB], aq[kSteps][2];
#pragma unroll
    for (int kk = 0; kk < kSteps; ++kk) {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        bq[kk][nb] = *reinterpret_cast<const bf16x8_t*>(bs + swz(brow[nb] + fr, kk * 2 + fh));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        aq[kk][mb] = *reinterpret_cast<const bf16x8_t*>(as + swz(wm * 64 + mb * 32 + fr, kk * 2 + fh));
    }
#pragma unroll
    for (int kk = 0; kk < kSteps; ++kk)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq[kk][nb], aq[kk][mb],
                                                                acc[mb][nb], 0, 0, 0);
    // the first step's reads, then per step: (2 MFMAs, 1 read) x kNB for the
    // next step's weight fragments, its two row fragments after them
    __builtin_amdgcn_sched_group_barrier(0x100, kNB + 2, 0);
#pragma unroll
    for (int st = 0; st + 1 < kSteps; ++st) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int i = 2; i < kNB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kNB, 0);
  };

  // Output tile of the compute-side item, staged through the x-row stage it
  // was last multiplied from (free until the next item's second store) in
  // rounds of kRoundRows rows.  Block (mb, nb) of a lane holds tile row
  // wm*64 + mb*32 + (lane & 31) at the four consecutive weight columns
  // 8*(q/4) + 4*(lane/32) + 0..3 of registers q: one 8-byte LDS write each,
  // at 16-byte chunk (col / 8) XOR (row & 15) of a bf16 row of kCols, read
  // back as whole 16-byte chunks.
  constexpr int kOutRowBytes = kCols * 2;
  constexpr int kRoundRows = kTile / kOutRowBytes < BM ? kTile / kOutRowBytes : BM;
  constexpr int kOutChunks = kCols / 8;
  constexpr int kReadRows = NTHR / kOutChunks;
  static_assert(kRoundRows % 64 == 0 && BM % kRoundRows == 0, "rounds hold whole waves' rows");
  static_assert(NTHR % kOutChunks == 0 && kReadRows % 16 == 0, "read-out rows keep row & 15");
  auto epilogue = [&](int obase) {  // obase: byte offset of the staging stage in a_st
    int ez = 0;  // opaque zero: keeps the lane-id computation inside the loop
    asm volatile("" : "+v"(ez));
    const int e_lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, ez));
    const int etid = wave * kWave + e_lane;
    const int e_fr = e_lane & 31, e_fh = e_lane >> 5;
    constexpr int npass = (GATEUP && AU) ? 3 : 1;
    for (int pass = 0; pass < npass; ++pass) {
#pragma unroll
    for (int r0 = 0; r0 < BM; r0 += kRoundRows) {
      if (r0 >= c_nrows) break;
      if (wm * 64 >= r0 && wm * 64 < r0 + kRoundRows) {  // a wave's 64 rows lie in one round
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          // rows past the item are staged too (never written out)
          const int R = wm * 64 + mb * 32 + e_fr - r0;
          int roff = obase + R * kOutRowBytes;
          asm("" : "+v"(roff));  // one opaque offset: keeps each store's pointer chain short
#pragma unroll
          for (int nb = 0; nb < (GATEUP ? kNB / 2 : kNB); ++nb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int col = (GATEUP ? wn * (BNW / 2 / kWavesN) : wn * (BNW / kWavesN)) + nb * 32 +
                              8 * g + 4 * e_fh;
              float v[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float gv = acc[mb][nb][4 * g + j];
                if (GATEUP) {
                  const float uv = acc[mb][nb + kNB / 2][4 * g + j];
                  v[j] = pass == 0 ? silu(gv) * uv : (pass == 1 ? gv : uv);
                } else {
                  v[j] = gv;
                }
              }
              // one 64-bit store (two 32-bit ones get merged without their alias
              // scope), a few pointer steps from a_st (a longer chain of them
              // loses it too)
              *reinterpret_cast<uint64_t*>(
                  a_st + (roff + ((((col >> 3) ^ (R & 15)) << 4) + (col & 4) * 2))) =
                  static_cast<uint64_t>(pack_bf16x2(v[0], v[1])) |
                  (static_cast<uint64_t>(pack_bf16x2(v[2], v[3])) << 32);
            }
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const int rl = etid / kOutChunks, cl = etid % kOutChunks;
      int soff = obase + rl * kOutRowBytes + ((cl ^ (rl & 15)) << 4);
      asm("" : "+v"(soff));
      const size_t ldo = pass == 0 ? static_cast<size_t>(N) : 2 * static_cast<size_t>(N);
      uint16_t* dst = (pass == 0 ? out : au + (pass == 2 ? N : 0)) +
                      static_cast<size_t>(c_m0 + r0 + rl) * ldo + c_n0 + cl * 8;
#pragma unroll
      for (int it = 0; it < kRoundRows / kReadRows; ++it) {
        if (rl < c_nrows - r0 - it * kReadRows)
        {
          // vector copies: a uint4 assignment is a memcpy, whose LDS load
          // carries no alias scope.  The down product's rows (y_perm, read
          // once by the combine) leave through non-temporal stores.
          const bf16x8_t v_ =
              *reinterpret_cast<const bf16x8_t*>(a_st + (soff + it * kReadRows * kOutRowBytes));
          bf16x8_t* d_ = reinterpret_cast<bf16x8_t*>(dst + static_cast<size_t>(it) * kReadRows * ldo);
          if (GATEUP)
            *d_ = v_;
          else
            __builtin_nontemporal_store(v_, d_);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    }
  };

  // ---- stream.  Prologue: rows and weights of slice 0 in LDS, those of
  // slice 1 in flight.  Step gk (compute slice k, weight stage k % 3): store
  // the rows of slice k + 1, load the rows of slice k + 2 and send its
  // weights, multiply slice k, wait for slice k + 1's weights, barrier.  The
  // wait leaves in flight what was issued after those weights: this step's
  // row and weight loads (l_na + kNI) and the fetch loads of the steps
  // between (position 1 of each three issues them).  A step that multiplied
  // an item's last slice writes its output tile before the next step.
  constexpr int kNF = GATEUP ? 2 : 1;  // fetch loads
  // (slice 1's loads go last, as in a step, so that the loop sees the same
  // loads in flight from the prologue as from its own last step)
  MOE_WLOAD(b0);
  MOE_WSTORE(0);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  MOE_WLOAD(b1);
  // the compiler may sink slice 1's row loads below its weight loads (they
  // read memory nothing here writes); using them here keeps them first
  asm volatile("" ::"v"(sa[0].x), "v"(sa[1].x), "v"(sa[2].x), "v"(sa[3].x) : "memory");
  int kc = 0;  // slices of the compute-side item multiplied
  int jc = 0;  // items finished
#define MOE_WWAIT(N)                                                                         \
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory")
#define MOE_WSTEP(U, BCUR, BNEXT, WAITB)                                                     \
  if ((U) == 1) MOE_WDECODE();                                                              \
  MOE_WSWITCH();                                                                            \
  MOE_WSTORE((gk + 1) & 1);                                                                 \
  __builtin_amdgcn_sched_barrier(0); /* the stores' waits must not cover the new loads */   \
  MOE_WLOAD(BNEXT);                                                                         \
  if ((U) == 1) MOE_WFETCH();                                                               \
  compute(a_st + (gk & 1) * kTile, BCUR);                                                   \
  if (l_na == 4)                                                                            \
    MOE_WWAIT((WAITB) + 4);                                                                 \
  else if (l_na == 3)                                                                       \
    MOE_WWAIT((WAITB) + 3);                                                                 \
  else if (l_na == 2)                                                                       \
    MOE_WWAIT((WAITB) + 2);                                                                 \
  else                                                                                      \
    MOE_WWAIT((WAITB) + 1);                                                                 \
  ++gk;                                                                                     \
  if (++kc == nk) {                                                                         \
    epilogue(((gk + 1) & 1) * kTile);                                                       \
    _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                        \
        _Pragma("unroll") for (int nb = 0; nb < kNB; ++nb)                                  \
            _Pragma("unroll") for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.0f;           \
    c_m0 = l_m0;                                                                            \
    c_nrows = l_nrows;                                                                      \
    c_n0 = l_ntile * kCols;                                                                 \
    kc = 0;                                                                                 \
    if (++jc == n_items) break;                                                             \
  }
  for (;;) {
    MOE_WSTEP(0, b0, b2, kNI)
    MOE_WSTEP(1, b1, b0, kNI + kNF)
    MOE_WSTEP(2, b2, b1, kNI + kNF)
  }
#undef MOE_WSTEP
#undef MOE_WWAIT
#undef MOE_WDECODE
#undef MOE_WSWITCH
#undef MOE_WFETCH
#undef MOE_WLOAD
#undef MOE_WSTORE
  // the trailing weight slices still write LDS: drain them before exit
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------- streaming, both operands by LDS DMA
//
// The weight-DMA kernel with the x rows sent into LDS by buffer loads with an
// LDS destination too, into three stages of their own, so both operands of a
// slice are issued two slices ahead of its multiply and the rows need no
// staging registers or LDS stores.  The LDS holds three weight stages (256
// rows x 64 k, 32 KB each) and three x-row stages of kXdmaRows rows (21 KB
// each): the tile list for this kernel is built with row tiles of at most
// kXdmaRows rows (a group with more rows gets further row tiles, which read
// its weights again).  A step sends the x rows of the slice two ahead (only
// the 8-row loads that hold rows of the item, so each wave issues 0 to 3 of
// them), then its weights, multiplies its own slice, waits for the next
// slice and meets the barrier; the stage of every step is a compile-time LDS
// object.  Rows kXdmaRows..191 of the third wave row do not exist: lanes of
// its second row block read the stage's last row for them, and their results
// belong to rows past the item, never written out.  The output tile is staged
// through the weight stage just multiplied (free until the next step sends
// a slice into it).  Used for groups of at most 128 rows on average when K
// has at least kWdmaMinSlices slices: the inference forms of both products,
// and the backward's activation-gradient products.
constexpr int kXdmaRows = 168;

template <bool GATEUP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bf16_xdma_kernel(
    int Kdim, int N, int x_rows, int rows, int max_tiles, int NT,
    const TileInfo* __restrict__ tiles, const int32_t* __restrict__ meta,
    const int32_t* __restrict__ row_index, const uint16_t* __restrict__ A, const WeightSet W,
    uint16_t* __restrict__ out) {
  using G = StreamGeom<64>;
  constexpr int BNW = 256, NTHR = 512;
  constexpr int kWavesN = 2;                   // waves: 4 along rows x 2 along weight rows
  constexpr int kNB = BNW / kWavesN / 32;      // 32-wide weight blocks per wave
  constexpr int kCols = GATEUP ? BNW / 2 : BNW;
  constexpr int kNI = G::kNI, kRPI = G::kRPI;  // weight loads per wave and slice, rows per load
  constexpr int kXI = 3;                       // x-row load slots per wave
  constexpr int kXLoads = kXdmaRows / kRPI;    // 8-row x loads per slice (20)
  constexpr uint32_t kOff = 0x80000000u;       // beyond every buffer (sizes < 2 GiB)
  constexpr int kTile = G::kTileBytes;         // one weight slice stage
  constexpr int kXTile = kXdmaRows * G::kRow;  // one x-row slice stage
  static_assert(kWdmaStages == 3, "the step loop is unrolled over three stages");
  static_assert(kXLoads <= 8 * kXI && kXLoads > 8 * (kXI - 1), "three load slots per wave");
  static_assert(kXdmaRows % kRPI == 0 && kXdmaRows > 160 && kXdmaRows <= 192,
                "the third wave row holds the rows past 128, its second block some of them");
  __shared__ __attribute__((aligned(16))) char a0[kXTile];  // x-row stages
  __shared__ __attribute__((aligned(16))) char a1[kXTile];
  __shared__ __attribute__((aligned(16))) char a2[kXTile];
  __shared__ __attribute__((aligned(16))) char b0[kTile];   // weight stages
  __shared__ __attribute__((aligned(16))) char b1[kTile];
  __shared__ __attribute__((aligned(16))) char b2[kTile];

  // ---- this workgroup's items: first, first + nslot, ... below end
  const int total = meta[0] * NT;
  const int nslot = gridDim.x / kNumXcd;
  const int xcd = blockIdx.x % kNumXcd;
  const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int first = xcd * per_xcd + static_cast<int>(blockIdx.x) / kNumXcd;
  const int end = min(total, (xcd + 1) * per_xcd);
  if (first >= end) return;
  const int n_items = (end - first + nslot - 1) / nslot;
  const int nk = Kdim / kBK;  // at least kWdmaMinSlices

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: scalar
  const int lane = tid % kWave;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const uint32_t rowbytes = static_cast<uint32_t>(Kdim) * 2u;
  const uint32_t wbytes = static_cast<uint32_t>(N) * rowbytes;
  const uint32_t kb_end = static_cast<uint32_t>(nk) * kBK * 2u;  // past the last slice
  const __amdgpu_buffer_rsrc_t rsA = buffer_rsrc(A, static_cast<uint32_t>(x_rows) * rowbytes);
  const __amdgpu_buffer_rsrc_t rsT =
      buffer_rsrc(tiles, static_cast<uint32_t>(max_tiles) * sizeof(TileInfo));
  const bool gather = GATEUP && row_index != nullptr;
  const __amdgpu_buffer_rsrc_t rsR =
      buffer_rsrc(row_index, gather ? static_cast<uint32_t>(rows) * 4u : 0u);

  // Load slot i of a wave sends tile rows kRPI (wave + 8 i) + drow (x rows)
  // or weight rows kRPI (wave + 8 i) + drow; lane l lands at LDS chunk l % 8
  // of its row, so it loads the k chunk that the swizzle stores there.
  const int drow = lane / G::kChunks;
  const int dchunk = (lane % G::kChunks) ^ drow ^ (wave & 1);
  auto a_offset = [&](int i, int nrows, int sr) -> uint32_t {
    return (kRPI * (wave + 8 * i) + drow < nrows && sr >= 0 && sr < x_rows)
               ? static_cast<uint32_t>(sr) * rowbytes + static_cast<uint32_t>(dchunk) * 16u
               : kOff;
  };
  // x-row loads this wave issues per slice for an item of nrows rows: the
  // slots whose 8 rows start below nrows
  auto x_loads = [&](int nrows) {
    const int m = min((nrows + kRPI - 1) / kRPI, kXLoads);
    int n = 0;
#pragma unroll
    for (int i = 0; i < kXI; ++i) n += (wave + 8 * i < m) ? 1 : 0;
    return n;
  };

  // ---- load-side item
  int l_item = 0, l_g, l_ntile, l_m0, l_nrows;
  {
    const TileInfo t0 = tiles[first / NT];
    int mt;
    item_tile(first - t0.gstart * NT, max(t0.ntiles, 1), NT, mt, l_ntile);
    const TileInfo ti = tiles[t0.gstart + mt];
    l_g = t0.group;
    l_m0 = ti.m0;
    l_nrows = min(ti.m1 - ti.m0, kXdmaRows);
  }
  int l_nx = x_loads(l_nrows);
  uint32_t a_off[kXI];
#pragma unroll
  for (int i = 0; i < kXI; ++i) {
    const int r = kRPI * (wave + 8 * i) + drow;
    int sr = l_m0 + r;
    if (gather) sr = (r < l_nrows) ? row_index[l_m0 + r] : -1;
    a_off[i] = a_offset(i, l_nrows, sr);
  }
  const uint32_t b_off = static_cast<uint32_t>(kRPI * wave + drow) * rowbytes +
                         static_cast<uint32_t>(dchunk) * 16u;
  __amdgpu_buffer_rsrc_t rb0, rb1;
  uint32_t bcol;
  auto set_weights = [&]() {
    rb0 = buffer_rsrc(W.base(false, l_g, static_cast<size_t>(N) * Kdim), wbytes);
    rb1 = buffer_rsrc(W.base(GATEUP, l_g, static_cast<size_t>(N) * Kdim), wbytes);
    bcol = static_cast<uint32_t>(l_ntile * kCols) * rowbytes;
  };
  set_weights();
  uint32_t kb = 0;  // byte offset of the load side's next k-slice

  // Sends the x rows of the load side's slice into x stage AST, then its
  // weights into weight stage BST.
#define MOE_XLOAD(AST, BST)                                                                  \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < kXI; ++i) if (i < l_nx)                           \
        dma16_unscoped<0>(rsA, (AST) + kRPI * (wave + 8 * i) * G::kRow, a_off[i], kb);      \
    __builtin_amdgcn_sched_barrier(0); /* rows before weights: see the step's waits */      \
    _Pragma("unroll") for (int i = 0; i < kNI; ++i) {                                       \
      const int add_ = GATEUP ? kRPI * 8 * (i % (kNI / 2)) : kRPI * 8 * i;                  \
      dma16_unscoped<kWeightPolicy>((GATEUP && i >= kNI / 2) ? rb1 : rb0,                   \
                                    (BST) + kRPI * (wave + 8 * i) * G::kRow, b_off,          \
                                    bcol + static_cast<uint32_t>(add_) * rowbytes + kb);    \
    }                                                                                       \
    kb += kBK * 2;                                                                          \
  } while (0)

  // ---- next item, fetched ahead as in the weight-DMA kernel (p: tile
  // records, ri: in lane j + 8 i the source row of tile row 8 wave + j + 64 i)
  int p = 0, ri = -1, ri_l = -1;
  int n_g = 0, n_ntile = 0, n_m0 = 0, n_nrows = 0;
  int nw = first + min(1, n_items - 1) * nslot;  // next item
  int t0rec = nw / NT;                           // a tile of its group
  int rec = 0;                                   // its row tile
  int fa = 0;                                    // fetches since nw changed

#define MOE_XDECODE()                                                                        \
  do {                                                                                      \
    if (fa == 1) { /* the group record just arrived: locate the row tile */                 \
      const int gstart_ = __builtin_amdgcn_readlane(p, 3);                                  \
      const int gnt_ = max(__builtin_amdgcn_readlane(p, 4), 1);                             \
      int mt_;                                                                              \
      item_tile(nw - gstart_ * NT, gnt_, NT, mt_, n_ntile);                                 \
      n_g = __builtin_amdgcn_readlane(p, 0);                                                \
      rec = gstart_ + mt_;                                                                  \
    }                                                                                       \
    n_m0 = __builtin_amdgcn_readlane(p, 9);                                                 \
    n_nrows = min(__builtin_amdgcn_readlane(p, 10) - n_m0, kXdmaRows);                      \
    if (GATEUP) /* a register of its own: ri's is then free for the next fetch */            \
      asm volatile("v_mov_b32 %0, %1" : "=&v"(ri_l) : "v"(ri));                             \
  } while (0)
#define MOE_XSWITCH()                                                                        \
  do {                                                                                      \
    if (kb == kb_end) {                                                                     \
      if (l_item + 1 < n_items) {                                                           \
        ++l_item;                                                                           \
        kb = 0;                                                                             \
        l_g = n_g; l_ntile = n_ntile; l_m0 = n_m0; l_nrows = n_nrows;                       \
        l_nx = x_loads(l_nrows);                                                            \
        set_weights();                                                                      \
        _Pragma("unroll") for (int i = 0; i < kXI; ++i) {                                   \
          const int sr_ = gather ? __builtin_amdgcn_ds_bpermute(((lane >> 3) + 8 * i) * 4, ri_l) \
                                 : l_m0 + kRPI * (wave + 8 * i) + drow;                     \
          a_off[i] = a_offset(i, l_nrows, sr_);                                             \
        }                                                                                   \
        nw = first + min(l_item + 1, n_items - 1) * nslot;                                  \
        t0rec = nw / NT;                                                                    \
        fa = 0;                                                                             \
      } else {                                                                              \
        kb = kb_end - kBK * 2; /* past the last item: its last slice again */               \
      }                                                                                     \
    }                                                                                       \
  } while (0)
#define MOE_XFETCH()                                                                         \
  do {                                                                                      \
    int z_ = 0;                                                                             \
    asm volatile("" : "+v"(z_));                                                            \
    const int ln_ = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, z_));     \
    if (GATEUP) { /* without row_index every load is out of range: no branch */             \
      const int r_ = wave * 8 + (ln_ & 7) + 64 * ((ln_ >> 3) & 3);                          \
      ri = __builtin_amdgcn_raw_buffer_load_b32(                                            \
          rsR, r_ < n_nrows ? static_cast<uint32_t>(n_m0 + r_) * 4u : kOff, 0, 0);          \
    }                                                                                       \
    p = __builtin_amdgcn_raw_buffer_load_b32(                                               \
        rsT, static_cast<uint32_t>((ln_ & 8) ? rec : t0rec) * 32u + (ln_ & 7) * 4u, 0, 0);  \
    fa = min(fa + 1, 3);                                                                    \
  } while (0)

  // ---- compute side (trails the load side by two slices)
  int c_m0 = l_m0, c_nrows = l_nrows, c_n0 = l_ntile * kCols;

  int brow[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    if (GATEUP) {
      const int half = kNB / 2;
      const int base = wn * (BNW / 2 / kWavesN);
      brow[nb] = (nb < half) ? base + nb * 32 : BNW / 2 + base + (nb - half) * 32;
    } else {
      brow[nb] = wn * (BNW / kWavesN) + nb * 32;
    }
  }
  // tile rows of this lane's fragment in the wave's two 32-row blocks (rows
  // past kXdmaRows are not in the stage: the third wave row's second block
  // reads its last row instead, for results that are never written out)
  const int arow0 = wm * 64 + (lane & 31);
  const int arow1 = min(wm * 64 + 32 + (lane & 31), kXdmaRows - 1);

  f32x16_t acc[2][kNB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mb][nb][q] = 0.0f;

  const int fr = lane & 31;
  const int fh = lane >> 5;
  constexpr int kSteps = kBK / 16;

  // As in the weight-DMA kernel: both row blocks of a busy wave, weight block
  // by weight block, the weight fragment first; the fragments of 16-k step
  // kk + 1 are read between the MFMAs of step kk.
  auto compute = [&](const char* as, const char* bs) {
    if (wm * 64 >= c_nrows) return;
    bf16x8_t bq[kSteps][kNB], aq[kSteps][2];
#pragma unroll
    for (int kk = 0; kk < kSteps; ++kk) {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        bq[kk][nb] = *reinterpret_cast<const bf16x8_t*>(bs + swz(brow[nb] + fr, kk * 2 + fh));
      aq[kk][0] = *reinterpret_cast<const bf16x8_t*>(as + swz(arow0, kk * 2 + fh));
      aq[kk][1] = *reinterpret_cast<const bf16x8_t*>(as + swz(arow1, kk * 2 + fh));
    }
#pragma unroll
    for (int kk = 0; kk < kSteps; ++kk)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq[kk][nb], aq[kk][mb],
                                                                acc[mb][nb], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, kNB + 2, 0);
#pragma unroll
    for (int st = 0; st + 1 < kSteps; ++st) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int i = 2; i < kNB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kNB, 0);
  };

  // Output tile of the compute-side item, staged through the weight stage
  // stg (just multiplied) in rounds of kRoundRows rows.  Block (mb, nb) of a
  // lane holds tile row wm*64 + mb*32 + (lane & 31) at the four consecutive
  // weight columns 8*(q/4) + 4*(lane/32) + 0..3 of registers q: one 8-byte
  // LDS write each, at 16-byte chunk (col / 8) XOR (row & 15) of a bf16 row
  // of kCols, read back as whole 16-byte chunks.
  constexpr int kOutRowBytes = kCols * 2;
  constexpr int kRoundRows = kTile / kOutRowBytes;
  constexpr int kOutChunks = kCols / 8;
  constexpr int kReadRows = NTHR / kOutChunks;
  static_assert(kRoundRows % 64 == 0, "rounds hold whole waves' rows");
  static_assert(NTHR % kOutChunks == 0 && kReadRows % 16 == 0, "read-out rows keep row & 15");
  auto epilogue = [&](char* stg) {
    int ez = 0;  // opaque zero: keeps the lane-id computation inside the loop
    asm volatile("" : "+v"(ez));
    const int e_lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, ez));
    const int etid = wave * kWave + e_lane;
    const int e_fr = e_lane & 31, e_fh = e_lane >> 5;
#pragma unroll
    for (int r0 = 0; r0 < kXdmaRows; r0 += kRoundRows) {
      if (r0 >= c_nrows) break;
      if (wm * 64 >= r0 && wm * 64 < r0 + kRoundRows) {  // a wave's 64 rows lie in one round
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          // rows past the item are staged too (never written out)
          const int R = wm * 64 + mb * 32 + e_fr - r0;
          int roff = R * kOutRowBytes;
          asm("" : "+v"(roff));  // one opaque offset: keeps each store's pointer chain short
#pragma unroll
          for (int nb = 0; nb < (GATEUP ? kNB / 2 : kNB); ++nb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int col = (GATEUP ? wn * (BNW / 2 / kWavesN) : wn * (BNW / kWavesN)) + nb * 32 +
                              8 * g + 4 * e_fh;
              float v[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float gv = acc[mb][nb][4 * g + j];
                v[j] = GATEUP ? silu(gv) * acc[mb][nb + kNB / 2][4 * g + j] : gv;
              }
              // one 64-bit store (two 32-bit ones get merged without their alias
              // scope), a few pointer steps from the stage
              *reinterpret_cast<uint64_t*>(
                  stg + (roff + ((((col >> 3) ^ (R & 15)) << 4) + (col & 4) * 2))) =
                  static_cast<uint64_t>(pack_bf16x2(v[0], v[1])) |
                  (static_cast<uint64_t>(pack_bf16x2(v[2], v[3])) << 32);
            }
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const int rl = etid / kOutChunks, cl = etid % kOutChunks;
      int soff = rl * kOutRowBytes + ((cl ^ (rl & 15)) << 4);
      asm("" : "+v"(soff));
      uint16_t* dst = out + static_cast<size_t>(c_m0 + r0 + rl) * N + c_n0 + cl * 8;
#pragma unroll
      for (int it = 0; it < kRoundRows / kReadRows; ++it) {
        if (rl < c_nrows - r0 - it * kReadRows) {
          // vector copies (a uint4 assignment is a memcpy, whose LDS load
          // carries no alias scope); both products' rows leave through
          // non-temporal stores (measured at the prefill shape: the gate/up
          // launch 0.04 ms faster, the down launch that reads its rows back
          // 0.02 ms slower)
          const bf16x8_t v_ =
              *reinterpret_cast<const bf16x8_t*>(stg + (soff + it * kReadRows * kOutRowBytes));
          bf16x8_t* d_ = reinterpret_cast<bf16x8_t*>(dst + static_cast<size_t>(it) * kReadRows * N);
          __builtin_nontemporal_store(v_, d_);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };

  // ---- stream.  Prologue: slice 0 in LDS, slice 1 in flight.  Step k
  // (stages k % 3): send slice k + 2, multiply slice k, wait for slice k + 1,
  // barrier.  The wait leaves in flight what was issued after slice k + 1's
  // weights: this step's x-row and weight loads (l_nx + kNI), after the fetch
  // loads that position 1 of each three issues first (so that the records
  // they bring have three steps of loads behind them when read).
  constexpr int kNF = GATEUP ? 2 : 1;  // fetch loads
  MOE_XLOAD(a0, b0);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  MOE_XLOAD(a1, b1);
  int kc = 0;  // slices of the compute-side item multiplied
  int jc = 0;  // items finished
#define MOE_XWAIT(N)                                                                         \
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory")
#define MOE_XSTEP(U, ACUR, BCUR, ANEXT, BNEXT, WAITB)                                        \
  if ((U) == 1) MOE_XDECODE();                                                              \
  MOE_XSWITCH();                                                                            \
  if ((U) == 1) MOE_XFETCH();                                                               \
  MOE_XLOAD(ANEXT, BNEXT);                                                                  \
  compute(ACUR, BCUR);                                                                      \
  if (l_nx == 3)                                                                            \
    MOE_XWAIT((WAITB) + 3);                                                                 \
  else if (l_nx == 2)                                                                       \
    MOE_XWAIT((WAITB) + 2);                                                                 \
  else if (l_nx == 1)                                                                       \
    MOE_XWAIT((WAITB) + 1);                                                                 \
  else                                                                                      \
    MOE_XWAIT(WAITB);                                                                       \
  if (++kc == nk) {                                                                         \
    epilogue(BCUR);                                                                         \
    _Pragma("unroll") for (int mb = 0; mb < 2; ++mb)                                        \
        _Pragma("unroll") for (int nb = 0; nb < kNB; ++nb)                                  \
            _Pragma("unroll") for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.0f;           \
    c_m0 = l_m0;                                                                            \
    c_nrows = l_nrows;                                                                      \
    c_n0 = l_ntile * kCols;                                                                 \
    kc = 0;                                                                                 \
    if (++jc == n_items) break;                                                             \
  }
  for (;;) {
    MOE_XSTEP(0, a0, b0, a2, b2, kNI)
    MOE_XSTEP(1, a1, b1, a0, b0, kNI + kNF)
    MOE_XSTEP(2, a2, b2, a1, b1, kNI)
  }
#undef MOE_XSTEP
#undef MOE_XWAIT
#undef MOE_XDECODE
#undef MOE_XSWITCH
#undef MOE_XFETCH
#undef MOE_XLOAD
  // the trailing slices still write LDS: drain them before exit
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Shapes the weight-DMA streaming kernel takes (K of whole slices, at least
// kWdmaMinSlices of them; N of whole column tiles).
bool wdma_shape(int K, int N, int cols) {
  return K % kBK == 0 && K / kBK >= kWdmaMinSlices && N % cols == 0;
}

// Workgroups of the streaming kernels: one per CU, a multiple of the XCD count.
int stream_grid() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < kNumXcd)
      cus = 256;
    cached[dev] = cus / kNumXcd * kNumXcd;
  }
  return cached[dev];
}

// The down-direction product over the tile list in w (built for BM rows):
// C[r, n] = (A_r . W[g][n]) * (row_scale ? row_scale[r] : 1), K-contiguous A
// [rows, K] and W [n_groups, N, K], C [rows, N].  The streaming kernels when
// the shape allows (LDS-fed for groups of at least a row tile on average),
// else the one-tile-per-workgroup kernel.
template <int BM, int BNW, int NTHR, int NSETS>
hipError_t launch_down(int n_groups, int K, int N, int rows, bool mfma_bound,
                       const SwigluWorkspace& w, const uint16_t* A, const WeightSet& W,
                       const float* row_scale, uint16_t* C, const char* name, hipStream_t s,
                       int tile_rows = BM) {
  const int max_tiles = max_tiles_for(rows, n_groups, tile_rows);
  const int nt = (N + BNW - 1) / BNW;
  ProfScope prof_(s, name);
  if (tile_rows == kXdmaRows && BNW == 256 && row_scale == nullptr && wdma_shape(K, N, 256)) {
    hipLaunchKernelGGL((bf16_xdma_kernel<false>), dim3(stream_grid()), dim3(512), 0, s, K, N,
                       rows, rows, max_tiles, nt, w.tiles, w.meta, nullptr, A, W, C);
  } else if (stream_shape(K, N, 256) && mfma_bound) {
    hipLaunchKernelGGL((bf16_stream_kernel<false, kStreamBK>), dim3(stream_grid()), dim3(512), 0,
                       s, K, N, rows, rows, nt, w.tiles, w.meta, nullptr, A, W, row_scale, C,
                       nullptr);
  } else if (BM == 256 && BNW == 256 && row_scale == nullptr && wdma_shape(K, N, 256)) {
    hipLaunchKernelGGL((bf16_wdma_kernel<false>), dim3(stream_grid()), dim3(512), 0, s, K, N,
                       rows, rows, max_tiles, nt, w.tiles, w.meta, nullptr, A, W, C, nullptr);
  } else if (stream_shape(K, N, BNW)) {
    hipLaunchKernelGGL((bf16_regs_stream_kernel<false, BM, BNW, NTHR>), dim3(stream_grid()),
                       dim3(NTHR), 0, s, K, N, rows, rows, max_tiles, nt, w.tiles, w.meta,
                       nullptr, A, W, row_scale, C, nullptr);
  } else {
    long blocks = static_cast<long>(max_tiles) * nt;
    blocks = (blocks + kNumXcd - 1) / kNumXcd * kNumXcd;
    hipLaunchKernelGGL((bf16_tile_kernel<false, BM, BNW, NTHR, NSETS>),
                       dim3(static_cast<unsigned>(blocks)), dim3(NTHR), 0, s, K, N, rows, nt,
                       w.tiles, w.meta, nullptr, A, W, row_scale, C, nullptr);
  }
  return hipGetLastError();
}

// The gate/up product act = SiLU(x W_gate^T) * (x W_up^T) over the tile list
// in w; with AU the gate and up values also go to au [rows, 2 d_ffn].
// Groups of at least a full row tile on average make the products matrix-core
// bound: LDS-fed kernel.  Fewer rows make them weight-streaming bound: the
// weight-DMA kernel, or for the training form the register-staged one.
template <int BM, int BNW, int NTHR, int NSETS, bool AU>
hipError_t launch_gateup(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                         bool mfma_bound, const int32_t* row_index, const uint16_t* x,
                         const WeightSet& W, uint16_t* act, uint16_t* au,
                         const SwigluWorkspace& w, hipStream_t s, int tile_rows = BM,
                         const char* prof_name = "gateup_bf16") {
  const int max_tiles = max_tiles_for(rows, n_groups, tile_rows);
  const int nt1 = (d_ffn + BNW / 2 - 1) / (BNW / 2);
  ProfScope prof_(s, prof_name);
  if (!AU && tile_rows == kXdmaRows && BNW == 256 && wdma_shape(d_model, d_ffn, 128)) {
    hipLaunchKernelGGL((bf16_xdma_kernel<true>), dim3(stream_grid()), dim3(512), 0, s, d_model,
                       d_ffn, x_rows, rows, max_tiles, nt1, w.tiles, w.meta, row_index, x, W,
                       act);
  } else if (stream_shape(d_model, d_ffn, 128) && mfma_bound) {
    hipLaunchKernelGGL((bf16_stream_kernel<true, kStreamBK, AU>), dim3(stream_grid()), dim3(512),
                       0, s, d_model, d_ffn, x_rows, rows, nt1, w.tiles, w.meta, row_index, x, W,
                       nullptr, act, au);
  } else if (!AU && BM == 256 && BNW == 256 && wdma_shape(d_model, d_ffn, 128)) {
    hipLaunchKernelGGL((bf16_wdma_kernel<true, false>), dim3(stream_grid()), dim3(512), 0, s,
                       d_model, d_ffn, x_rows, rows, max_tiles, nt1, w.tiles, w.meta, row_index,
                       x, W, act, nullptr);
  } else if (stream_shape(d_model, d_ffn, BNW / 2)) {
    hipLaunchKernelGGL((bf16_regs_stream_kernel<true, BM, BNW, NTHR, AU>), dim3(stream_grid()),
                       dim3(NTHR), 0, s, d_model, d_ffn, x_rows, rows, max_tiles, nt1, w.tiles,
                       w.meta, row_index, x, W, nullptr, act, au);
  } else {
    long blocks1 = static_cast<long>(max_tiles) * nt1;
    blocks1 = (blocks1 + kNumXcd - 1) / kNumXcd * kNumXcd;
    hipLaunchKernelGGL((bf16_tile_kernel<true, BM, BNW, NTHR, NSETS, AU>),
                       dim3(static_cast<unsigned>(blocks1)), dim3(NTHR), 0, s, d_model, d_ffn,
                       x_rows, nt1, w.tiles, w.meta, row_index, x, W, nullptr, act, au);
  }
  return hipGetLastError();
}

// Both products over the tile list already in w (n_groups: the number of
// groups the list was built for).
template <int BM, int BNW, int NTHR, int NSETS>
hipError_t launch_products(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                           const int32_t* row_index, const uint16_t* x, const WeightSet& Wgu,
                           const WeightSet& Wd, const float* row_scale, uint16_t* y,
                           uint16_t* au, const SwigluWorkspace& w, hipStream_t s,
                           int tile_rows = BM) {
  uint16_t* act = static_cast<uint16_t*>(w.act);
  const bool mfma_bound = rows >= kDmaMinRowsPerGroup * static_cast<long>(n_groups);
  hipError_t err =
      au != nullptr
          ? launch_gateup<BM, BNW, NTHR, NSETS, true>(n_groups, d_model, d_ffn, rows, x_rows,
                                                      mfma_bound, row_index, x, Wgu, act, au, w,
                                                      s, tile_rows)
          : launch_gateup<BM, BNW, NTHR, NSETS, false>(n_groups, d_model, d_ffn, rows, x_rows,
                                                       mfma_bound, row_index, x, Wgu, act,
                                                       nullptr, w, s, tile_rows);
  if (err != hipSuccess) return err;
  return launch_down<BM, BNW, NTHR, NSETS>(n_groups, d_ffn, d_model, rows, mfma_bound, w, act, Wd,
                                           row_scale, y, "down_bf16", s, tile_rows);
}

// Row-tile size of the tile list for both products: kXdmaRows when the groups
// average at most kXdmaMaxAvgRows rows (so that few of them need a second row
// tile, which reads their weights again) and both products take the kernel
// that sends both operands by LDS DMA (inference forms), else 256.
constexpr int kXdmaMaxAvgRows = 128;
int products_tile_rows(int n_groups, int d_model, int d_ffn, int rows, bool au,
                       bool row_scale) {
  return (rows <= kXdmaMaxAvgRows * static_cast<long>(n_groups) && !au && !row_scale &&
          wdma_shape(d_model, d_ffn, 128) && wdma_shape(d_ffn, d_model, 256))
             ? kXdmaRows
             : 256;
}

// Matrix-core-bound inference forms (groups of at least 256 rows on average):
// a row tile of the LDS-fed kernel costs about as much with a few rows as
// with 256 (its steps wait on the slice loads, not on the multiply), so each
// group's last rows, when fewer than kSplitRows, go to a second launch of the
// kernel that sends both operands by LDS DMA, which streams such tiles about
// twice as fast.  Both products need whole slices and column tiles for it.
constexpr int kSplitRows = 128;
bool split_remainders(int n_groups, int d_model, int d_ffn, int rows, bool au, bool row_scale) {
  // one group (a shared expert): its remainder is known here
  if (n_groups == 1 && (rows % 256 == 0 || rows % 256 >= kSplitRows)) return false;
  return !au && !row_scale && rows >= kDmaMinRowsPerGroup * static_cast<long>(n_groups) &&
         stream_shape(d_model, d_ffn, 128) && stream_shape(d_ffn, d_model, 256) &&
         wdma_shape(d_model, d_ffn, 128) && wdma_shape(d_ffn, d_model, 256) &&
         static_cast<long long>(rows) * d_model * 2 < (1ll << 31) &&
         static_cast<long long>(rows) * d_ffn * 2 < (1ll << 31) &&
         max_tiles_for(rows, n_groups, 256) + n_groups <= max_tiles_for(rows, n_groups, 32);
}

// The products over the two tile lists of launch_build_split_tiles: the full
// tiles on the LDS-fed kernel, then the remainders on the both-operands-by-DMA
// kernel, each product's two launches timed as one.
hipError_t launch_products_split(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                                 const int32_t* offsets, const int32_t* row_index,
                                 const uint16_t* x, const WeightSet& Wgu, const WeightSet& Wd,
                                 uint16_t* y, const SwigluWorkspace& w, hipStream_t s) {
  const int off2 = max_tiles_for(rows, n_groups, 256);
  hipError_t err = launch_build_split_tiles(n_groups, rows, kSplitRows, off2, offsets, w, s);
  if (err != hipSuccess) return err;
  SwigluWorkspace w2 = w;
  w2.tiles = w.tiles + off2;
  w2.meta = w.meta + 2;
  uint16_t* act = static_cast<uint16_t*>(w.act);
  {
    ProfScope prof_(s, "gateup_bf16");
    err = launch_gateup<256, 256, 512, 2, false>(n_groups, d_model, d_ffn, rows, x_rows, true,
                                                 row_index, x, Wgu, act, nullptr, w, s, 256,
                                                 nullptr);
    if (err != hipSuccess) return err;
    err = launch_gateup<256, 256, 512, 2, false>(n_groups, d_model, d_ffn, rows, x_rows, true,
                                                 row_index, x, Wgu, act, nullptr, w2, s,
                                                 kXdmaRows, nullptr);
    if (err != hipSuccess) return err;
  }
  ProfScope prof_(s, "down_bf16");
  err = launch_down<256, 256, 512, 2>(n_groups, d_ffn, d_model, rows, true, w, act, Wd, nullptr,
                                      y, nullptr, s, 256);
  if (err != hipSuccess) return err;
  return launch_down<256, 256, 512, 2>(n_groups, d_ffn, d_model, rows, true, w2, act, Wd,
                                       nullptr, y, nullptr, s, kXdmaRows);
}

}  // namespace

hipError_t launch_grouped_nt_bf16(int n_groups, int K, int N, int rows, const int32_t* offsets,
                                  const SwigluWorkspace& w, const uint16_t* A, const uint16_t* W,
                                  uint16_t* C, const char* name, hipStream_t s,
                                  bool tiles_built, int tile_rows) {
  if (tile_rows != 256 && tile_rows != kXdmaRows) return hipErrorInvalidValue;
  if (!tiles_built) {
    hipError_t err = launch_build_tiles(n_groups, rows, tile_rows, offsets, w, s);
    if (err != hipSuccess) return err;
  }
  const bool mfma_bound = rows >= kDmaMinRowsPerGroup * static_cast<long>(n_groups);
  return launch_down<256, 256, 512, 2>(n_groups, K, N, rows, mfma_bound, w, A,
                                       WeightSet::one(W, W), nullptr, C, name, s, tile_rows);
}

int grouped_nt_tile_rows(int n_groups, int rows, int K1, int N1, int K2, int N2) {
  const auto fits = [&](int K, int N) {
    return wdma_shape(K, N, 256) &&
           static_cast<long long>(rows) * N * 2 < (1ll << 31);  // 32-bit buffer offsets
  };
  return (rows <= kXdmaMaxAvgRows * static_cast<long>(n_groups) && fits(K1, N1) && fits(K2, N2))
             ? kXdmaRows
             : 256;
}

hipError_t launch_swiglu_bf16(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                              const int32_t* offsets, const int32_t* row_index,
                              const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                              const uint16_t* wd, const float* row_scale, uint16_t* y,
                              uint16_t* au, void* ws, hipStream_t s) {
  SwigluWorkspace w = swiglu_layout(ws, n_groups, d_ffn, rows, 2, 32);
  if (split_remainders(n_groups, d_model, d_ffn, rows, au != nullptr, row_scale != nullptr))
    return launch_products_split(n_groups, d_model, d_ffn, rows, x_rows, offsets, row_index, x,
                                 WeightSet::one(wg, wu), WeightSet::one(wd, wd), y, w, s);
  const int bm = products_tile_rows(n_groups, d_model, d_ffn, rows, au != nullptr,
                                    row_scale != nullptr);
  hipError_t err = launch_build_tiles(n_groups, rows, bm, offsets, w, s);
  if (err != hipSuccess) return err;
  return launch_products<256, 256, 512, 2>(n_groups, d_model, d_ffn, rows, x_rows, row_index, x,
                                           WeightSet::one(wg, wu), WeightSet::one(wd, wd),
                                           row_scale, y, au, w, s, bm);
}

hipError_t launch_experts_bf16(int E_r, int E_s, int T, int K, int d_model, int d_ffn,
                               const int32_t* offsets, const int32_t* row_token,
                               const uint16_t* h, const uint16_t* wg, const uint16_t* wu,
                               const uint16_t* wd, const uint16_t* wsg, const uint16_t* wsu,
                               const uint16_t* wsd, uint16_t* y, void* ws, hipStream_t s) {
  const ExpertsLayout L = experts_layout(ws, E_r, E_s, T, K, d_ffn);
  hipError_t err = launch_build_tiles_experts(E_r, E_s, T, K, L.shared_rows_per_group, offsets,
                                              row_token, L.row_index, L.sw, s);
  if (err != hipSuccess) return err;
  return launch_products<256, 256, 512, 2>(L.n_groups, d_model, d_ffn, L.rows, T, L.row_index, h,
                                           WeightSet{wg, wu, wsg, wsu, E_r},
                                           WeightSet{wd, wd, wsd, wsd, E_r}, nullptr, y, nullptr,
                                           L.sw, s);
}

}  // namespace moe
