// Grouped SwiGLU, bf16 path on the CDNA4 matrix cores.
//
// Method: Sparse MoE routing-math page (arman1o1.github.io), section 0
// (SwiGLU(h) = (SiLU(h W_gate) * (h W_up)) W_down), section 3 (all local
// experts in one grouped GEMM over variable-sized token buckets, no padding).
//
// Two launches over the device-built tile list:
//   gate/up: act[r, n] = SiLU(x_r . Wg[n]) * (x_r . Wu[n])     K = d_model
//            x rows gathered on load through row_index (no x_perm copy);
//            the B tile stacks 64 W_gate rows over the same 64 W_up rows,
//            so each lane holds matching gate and up accumulators.
//   down:    y[r, n] = (act_r . Wd[n]) * row_scale[r]          K = d_ffn
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
// writes are bank-conflict free).  The kernel is templated on the tile shape
// and the number of register sets; this shape measured fastest for both the
// weight-streaming (few rows per expert) and the matrix-core-bound shapes.
//
// Work order: (group, column tile, row tile); block ids are remapped so each
// XCD walks a contiguous run of it: row tiles of one (expert, column tile) run
// side by side on one XCD and share the weight slice through its L2, and the
// column tiles of one expert reuse its gathered x rows from that L2.
#include "swiglu_tiles.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;         // k per LDS stage (8 chunks of 16 B per row)
constexpr int kRowBytes = kBK * 2;                     // 128 B
constexpr int kNumXcd = 8;
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
template <bool GATEUP, int BM, int BNW, int NTHR, int NSETS>
__global__ __launch_bounds__(NTHR)
__attribute__((amdgpu_waves_per_eu(Tile<BM, BNW, NTHR>::kWavesPerEU,
                                   Tile<BM, BNW, NTHR>::kWavesPerEU)))
void bf16_tile_kernel(
    int Kdim, int N, int x_rows, int n_groups, int NT, const TileInfo* __restrict__ tiles,
    const int32_t* __restrict__ gts, const int32_t* __restrict__ meta,
    const int32_t* __restrict__ row_index, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
    const float* __restrict__ row_scale, uint16_t* __restrict__ out) {
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
  int lo = 0, hi = n_groups;  // largest g with gts[g] * NT <= w (that group has tiles)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (gts[mid] * NT <= w) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int gstart = gts[g];
  const int nmt = gts[g + 1] - gstart;
  const int local = w - gstart * NT;
  const int ntile = local / nmt;
  const TileInfo ti = tiles[gstart + local % nmt];
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
  const __amdgpu_buffer_rsrc_t rsB0 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W0 + static_cast<size_t>(g) * N * Kdim), 0, wbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rsB1 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(GATEUP ? W1 + static_cast<size_t>(g) * N * Kdim : W0), 0, wbytes,
      kBufferFlags);
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

  // ---- epilogue: D[row][col] of a 32x32 block sits in lane (col + 32*((row/4)%2)),
  // register (row%4) + 4*(row/8).
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = wm * 64 + mb * 32 + 8 * (q >> 2) + 4 * fh + (q & 3);
      if (row >= nrows) continue;
      const int gr = ti.m0 + row;
      if (GATEUP) {
#pragma unroll
        for (int nb = 0; nb < kNB / 2; ++nb) {
          const int col = n0 + brow[nb] + fr;
          if (col < N) {
            const float v = silu(acc[mb][nb][q]) * acc[mb][nb + kNB / 2][q];
            out[static_cast<size_t>(gr) * N + col] = f32_to_bf16(v);
          }
        }
      } else {
        const float sc = row_scale ? row_scale[gr] : 1.0f;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const int col = n0 + brow[nb] + fr;
          if (col < N) out[static_cast<size_t>(gr) * N + col] = f32_to_bf16(acc[mb][nb][q] * sc);
        }
      }
    }
  }
}

template <int BM, int BNW, int NTHR, int NSETS>
hipError_t launch_tiles(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                        const int32_t* offsets, const int32_t* row_index, const uint16_t* x,
                        const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                        const float* row_scale, uint16_t* y, const SwigluWorkspace& w,
                        hipStream_t s) {
  hipError_t err = launch_build_tiles(n_groups, rows, BM, offsets, w, s);
  if (err != hipSuccess) return err;
  const int max_tiles = max_tiles_for(rows, n_groups, BM);
  uint16_t* act = static_cast<uint16_t*>(w.act);

  const int nt1 = (d_ffn + BNW / 2 - 1) / (BNW / 2);
  long blocks1 = static_cast<long>(max_tiles) * nt1;
  blocks1 = (blocks1 + kNumXcd - 1) / kNumXcd * kNumXcd;
  {
    ProfScope prof_(s, "gateup_bf16");
    hipLaunchKernelGGL((bf16_tile_kernel<true, BM, BNW, NTHR, NSETS>),
                       dim3(static_cast<unsigned>(blocks1)), dim3(NTHR), 0, s, d_model, d_ffn, x_rows, n_groups, nt1, w.tiles,
                       w.group_tile_start, w.meta, row_index, x, wg, wu, nullptr, act);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  const int nt2 = (d_model + BNW - 1) / BNW;
  long blocks2 = static_cast<long>(max_tiles) * nt2;
  blocks2 = (blocks2 + kNumXcd - 1) / kNumXcd * kNumXcd;
  {
    ProfScope prof_(s, "down_bf16");
    hipLaunchKernelGGL((bf16_tile_kernel<false, BM, BNW, NTHR, NSETS>),
                       dim3(static_cast<unsigned>(blocks2)), dim3(NTHR), 0, s, d_ffn, d_model, rows, n_groups, nt2, w.tiles,
                       w.group_tile_start, w.meta, nullptr, act, wd, nullptr, row_scale, y);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swiglu_bf16(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                              const int32_t* offsets, const int32_t* row_index,
                              const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                              const uint16_t* wd, const float* row_scale, uint16_t* y,
                              void* ws, hipStream_t s) {
  SwigluWorkspace w = swiglu_layout(ws, n_groups, d_ffn, rows, 2, 32);
  return launch_tiles<256, 256, 512, 2>(n_groups, d_model, d_ffn, rows, x_rows, offsets,
                                        row_index, x, wg, wu, wd, row_scale, y, w, s);
}

}  // namespace moe
