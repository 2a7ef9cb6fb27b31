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
// Tile: 128 rows x 256 weight rows x 64 k, four waves in a 2 x 2 layout, each
// wave 2 x 4 blocks of v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  Global
// 16-byte loads for the next k-slice are in flight while the current slice is
// multiplied out of LDS (two LDS stages, XOR-swizzled 16-byte chunks so the
// fragment reads are bank-conflict free).
//
// Work order: (group, column tile, row tile), and block ids are remapped so
// each XCD takes a contiguous run of that order: the row tiles of one
// (expert, column tile) run side by side on one XCD and share the weight
// slice through its L2, and the column tiles of one expert share its x rows.
#include "swiglu_tiles.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;        // grouped rows per tile
constexpr int kBNW = 256;       // weight rows per tile
constexpr int kBK = 64;         // k per LDS stage (8 chunks of 16 B per row)
constexpr int kThreads = 256;
constexpr int kRowBytes = kBK * 2;                     // 128 B
constexpr int kStageBytes = (kBM + kBNW) * kRowBytes;  // 48 KB
constexpr int kNumXcd = 8;

__device__ __forceinline__ int swz(int r, int c) { return r * kRowBytes + ((c ^ (r & 7)) << 4); }

// GATEUP: columns per tile = 128 (act columns), W0 = W_gate, W1 = W_up
// DOWN:   columns per tile = 256 (y columns),   W0 = W_down
template <bool GATEUP>
__global__ __launch_bounds__(kThreads) void bf16_tile_kernel(
    int Kdim, int N, int x_rows, int n_groups, int NT, const TileInfo* __restrict__ tiles,
    const int32_t* __restrict__ gts, const int32_t* __restrict__ meta,
    const int32_t* __restrict__ row_index, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
    const float* __restrict__ row_scale, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];

  // ---- block -> (group, column tile, row tile), XCD-contiguous
  const int total = meta[0] * NT;
  const int xcd = blockIdx.x % kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  const int per_xcd = (total + kNumXcd - 1) / kNumXcd;
  const int w = xcd * per_xcd + slot;
  if (slot >= per_xcd || w >= total) return;
  int lo = 0, hi = n_groups;  // largest g with gts[g] * NT <= w
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

  constexpr int kCols = GATEUP ? 128 : 256;
  const int n0 = ntile * kCols;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- per-thread load slots: 4 A chunks, 8 B chunks per k-slice
  const int lc = tid & 7;          // 16-byte chunk within the 128-byte k-slice row
  const int lr = tid >> 3;         // 0..31
  const uint16_t* a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int gr = ti.m0 + lr + 32 * i;
    int sr = -1;
    if (gr < ti.m1) {
      sr = row_index ? row_index[gr] : gr;
      if (sr < 0 || sr >= x_rows) sr = -1;
    }
    a_src[i] = (sr >= 0) ? A + static_cast<size_t>(sr) * Kdim + lc * 8 : nullptr;
  }
  const size_t wexp = static_cast<size_t>(g) * N * Kdim;
  const uint16_t* b_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = lr + 32 * i;  // 0..255
    const uint16_t* base;
    int n;
    if (GATEUP) {
      base = (r < 128) ? W0 : W1;
      n = n0 + (r & 127);
    } else {
      base = W0;
      n = n0 + r;
    }
    b_src[i] = (n < N) ? base + wexp + static_cast<size_t>(n) * Kdim + lc * 8 : nullptr;
  }

  uint4 ra[4], rb[8];
  auto load_slice = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = a_src[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rb[i] = b_src[i] ? *reinterpret_cast<const uint4*>(b_src[i] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto store_slice = [&](int stage) {
    char* as = smem + stage * kStageBytes;
    char* bs = as + kBM * kRowBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(as + swz(lr + 32 * i, lc)) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(bs + swz(lr + 32 * i, lc)) = rb[i];
  };

  // B-tile rows of this wave's four 32-wide column blocks
  int brow[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    brow[nb] = GATEUP ? ((nb >> 1) * 128 + wn * 64 + (nb & 1) * 32) : (wn * 128 + nb * 32);

  f32x16_t acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mb][nb][q] = 0.0f;

  const int nk = Kdim / kBK;
  load_slice(0);
  store_slice(0);
  __syncthreads();
  const int fr = lane & 31;        // fragment row within a 32-block
  const int fh = lane >> 5;        // which 8-wide k half of the 16-k step
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_slice((kt + 1) * kBK);
    const char* as = smem + cur * kStageBytes;
    const char* bs = as + kBM * kRowBytes;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int c = kk * 2 + fh;
      bf16x8_t af[2], bfr[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        int r = wm * 64 + mb * 32 + fr;
        af[mb] = *reinterpret_cast<const bf16x8_t*>(as + swz(r, c));
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        int r = brow[nb] + fr;
        bfr[nb] = *reinterpret_cast<const bf16x8_t*>(bs + swz(r, c));
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
    }
    if (kt + 1 < nk) store_slice(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: D[row][col] of a 32x32 block sits in lane (col + 32*((row/4)%2)),
  // register (row%4) + 4*(row/8).
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = wm * 64 + mb * 32 + 8 * (q >> 2) + 4 * fh + (q & 3);
      const int gr = ti.m0 + row;
      if (gr >= ti.m1) continue;
      if (GATEUP) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col = n0 + wn * 64 + nb * 32 + fr;
          if (col < N) {
            float v = silu(acc[mb][nb][q]) * acc[mb][nb + 2][q];
            out[static_cast<size_t>(gr) * N + col] = f32_to_bf16(v);
          }
        }
      } else {
        const float sc = row_scale ? row_scale[gr] : 1.0f;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int col = n0 + wn * 128 + nb * 32 + fr;
          if (col < N) out[static_cast<size_t>(gr) * N + col] = f32_to_bf16(acc[mb][nb][q] * sc);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_swiglu_bf16(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                              const int32_t* offsets, const int32_t* row_index,
                              const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                              const uint16_t* wd, const float* row_scale, uint16_t* y,
                              void* ws, hipStream_t s) {
  SwigluWorkspace w = swiglu_layout(ws, n_groups, d_ffn, rows, 2, 32);
  hipError_t err = launch_build_tiles(n_groups, rows, kBM, offsets, w, s);
  if (err != hipSuccess) return err;
  const int max_tiles = max_tiles_for(rows, n_groups, kBM);
  uint16_t* act = static_cast<uint16_t*>(w.act);

  const int nt1 = (d_ffn + 127) / 128;
  long blocks1 = static_cast<long>(max_tiles) * nt1;
  blocks1 = (blocks1 + kNumXcd - 1) / kNumXcd * kNumXcd;
  {
    ProfScope prof_(s, "gateup_bf16");
    hipLaunchKernelGGL((bf16_tile_kernel<true>), dim3(static_cast<unsigned>(blocks1)),
                       dim3(kThreads), 0, s, d_model, d_ffn, x_rows, n_groups, nt1, w.tiles,
                       w.group_tile_start, w.meta, row_index, x, wg, wu, nullptr, act);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  const int nt2 = (d_model + 255) / 256;
  long blocks2 = static_cast<long>(max_tiles) * nt2;
  blocks2 = (blocks2 + kNumXcd - 1) / kNumXcd * kNumXcd;
  {
    ProfScope prof_(s, "down_bf16");
    hipLaunchKernelGGL((bf16_tile_kernel<false>), dim3(static_cast<unsigned>(blocks2)),
                       dim3(kThreads), 0, s, d_ffn, d_model, rows, n_groups, nt2, w.tiles,
                       w.group_tile_start, w.meta, nullptr, act, wd, nullptr, row_scale, y);
  }
  return hipGetLastError();
}

}  // namespace moe
