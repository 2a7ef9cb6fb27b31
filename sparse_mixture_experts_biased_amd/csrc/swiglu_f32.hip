// Grouped SwiGLU, fp32 path, plus the device-side tile-list builder shared
// with the bf16 path.
//
// Method: Sparse MoE routing-math page (arman1o1.github.io), section 0
// (SwiGLU(h) = (SiLU(h W_gate) * (h W_up)) W_down) and section 3 (all local
// experts in one grouped GEMM over variable-sized token buckets).
//
// fp32 tiles are 64 rows x 64 columns on the vector ALUs (fp32 FMA); each
// thread owns a 4 x 4 block (and, for the gate/up kernel, the matching 4 x 4
// block of W_up so SiLU(gate) * up is formed in registers).
#include "swiglu_tiles.h"

namespace moe {
namespace {

// ---------------------------------------------------------------- tile list

// Tile counts come from caller-provided offsets: every index is clamped to
// max_tiles, so even inconsistent offsets cannot write past the tile list.
__global__ __launch_bounds__(1024) void build_tiles_kernel(int n_groups, int rows, int bm,
                                                           int max_tiles,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ gts,
                                                           TileInfo* __restrict__ tiles,
                                                           int32_t* __restrict__ meta) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry_s;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  for (int g0 = 0; g0 < n_groups; g0 += 1024) {
    const int g = g0 + threadIdx.x;
    int lo = 0, hi = 0, nt = 0;
    if (g < n_groups) {
      lo = min(max(offsets[g], 0), rows);
      hi = min(max(offsets[g + 1], lo), rows);
      nt = (hi - lo + bm - 1) / bm;
    }
    part[threadIdx.x] = nt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int v = (threadIdx.x >= static_cast<unsigned>(off)) ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    const int carry = carry_s;
    const int start = carry + part[threadIdx.x] - nt;
    if (g < n_groups) {
      gts[g] = min(start, max_tiles);
      for (int i = 0; i < nt && start + i < max_tiles; ++i)
        tiles[start + i] = TileInfo{g, lo + i * bm, hi, start, min(nt, max_tiles - start), {0, 0, 0}};
    }
    __syncthreads();
    if (threadIdx.x == 1023) carry_s = carry + part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    gts[n_groups] = min(carry_s, max_tiles);
    meta[0] = min(carry_s, max_tiles);
  }
}

// The split lists of launch_build_split_tiles, one workgroup: group g of m
// rows has r = m % 256 rows past its last full 256-row tile; with 0 < r <
// small_rows those rows form one tile of the second list, else they end the
// first list's tiles of g as a partial tile.  Each list is in group order with
// its own group starts.
__global__ __launch_bounds__(1024) void build_split_tiles_kernel(
    int n_groups, int rows, int small_rows, int off2, const int32_t* __restrict__ offsets,
    TileInfo* __restrict__ tiles, int32_t* __restrict__ meta) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry1_s, carry2_s;
  if (threadIdx.x == 0) carry1_s = carry2_s = 0;
  __syncthreads();
  for (int g0 = 0; g0 < n_groups; g0 += 1024) {
    const int g = g0 + threadIdx.x;
    int lo = 0, hi = 0, n1 = 0, n2 = 0;
    if (g < n_groups) {
      lo = min(max(offsets[g], 0), rows);
      hi = min(max(offsets[g + 1], lo), rows);
      const int m = hi - lo, full = m / 256, r = m - full * 256;
      n2 = (r > 0 && r < small_rows) ? 1 : 0;
      n1 = full + ((r > 0 && n2 == 0) ? 1 : 0);
    }
    // inclusive scans of n1, then n2
    part[threadIdx.x] = n1;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = threadIdx.x >= static_cast<unsigned>(off) ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    const int c1 = carry1_s, s1 = c1 + part[threadIdx.x] - n1, t1 = c1 + part[1023];
    __syncthreads();
    part[threadIdx.x] = n2;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = threadIdx.x >= static_cast<unsigned>(off) ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    const int c2 = carry2_s, s2 = c2 + part[threadIdx.x] - n2, t2 = c2 + part[1023];
    if (g < n_groups) {
      for (int i = 0; i < n1; ++i)
        tiles[s1 + i] = TileInfo{g, lo + i * 256, hi, s1, n1, {0, 0, 0}};
      if (n2) tiles[off2 + s2] = TileInfo{g, lo + (hi - lo) / 256 * 256, hi, s2, 1, {0, 0, 0}};
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      carry1_s = t1;
      carry2_s = t2;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    meta[0] = carry1_s;
    meta[2] = carry2_s;
  }
}

// ---------------------------------------------------------------- fp32 GEMM tiles

constexpr int kBM = 64, kBN = 64, kBK = 16, kThreads = 256;

// GATEUP: act[r, n] = SiLU(x_r . Wg[n]) * (x_r . Wu[n]), K = d_model, N = d_ffn
// else  :   y[r, n] = (act_r . Wd[n]) * scale[r],          K = d_ffn,  N = d_model
template <bool GATEUP>
__global__ __launch_bounds__(kThreads) void f32_tile_kernel(
    int Kdim, int N, int x_rows, const TileInfo* __restrict__ tiles,
    const int32_t* __restrict__ meta, const int32_t* __restrict__ row_index,
    const float* __restrict__ A, const float* __restrict__ W0, const float* __restrict__ W1,
    const float* __restrict__ row_scale, float* __restrict__ out) {
  __shared__ float as[kBK][kBM + 4];
  __shared__ float b0s[kBK][kBN + 4];
  __shared__ float b1s[GATEUP ? kBK : 1][kBN + 4];

  const int tile_id = blockIdx.x;
  if (tile_id >= meta[0]) return;
  const TileInfo ti = tiles[tile_id];
  const int n0 = blockIdx.y * kBN;
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  const size_t wbase = static_cast<size_t>(ti.group) * N * Kdim;

  // source row of each of this thread's load slots (4 rows per thread)
  int src_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = (tid + kThreads * i) / kBK;
    int gr = ti.m0 + r;
    int sr = -1;
    if (gr < ti.m1) {
      sr = row_index ? row_index[gr] : gr;
      if (sr < 0 || sr >= x_rows) sr = -1;
    }
    src_row[i] = sr;
  }

  float acc0[4][4] = {}, acc1[4][4] = {};
  for (int k0 = 0; k0 < Kdim; k0 += kBK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int q = tid + kThreads * i;
      int r = q / kBK, c = q % kBK;
      as[c][r] = (src_row[i] >= 0) ? A[static_cast<size_t>(src_row[i]) * Kdim + k0 + c] : 0.0f;
      int n = n0 + r;
      b0s[c][r] = (n < N) ? W0[wbase + static_cast<size_t>(n) * Kdim + k0 + c] : 0.0f;
      if (GATEUP) b1s[c][r] = (n < N) ? W1[wbase + static_cast<size_t>(n) * Kdim + k0 + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK; ++kk) {
      float a[4], w0[4], w1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = as[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w0[j] = b0s[kk][tx * 4 + j];
        if (GATEUP) w1[j] = b1s[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc0[i][j] = fmaf(a[i], w0[j], acc0[i][j]);
          if (GATEUP) acc1[i][j] = fmaf(a[i], w1[j], acc1[i][j]);
        }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int gr = ti.m0 + ty * 4 + i;
    if (gr >= ti.m1) continue;
    float sc = 1.0f;
    if (!GATEUP && row_scale) sc = row_scale[gr];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float v = GATEUP ? silu(acc0[i][j]) * acc1[i][j] : acc0[i][j] * sc;
      out[static_cast<size_t>(gr) * N + n] = v;
    }
  }
}

// Grouped row r of the combined routed + shared launch reads token
// row_token[r] (r < T*K) or token (r - T*K) % T (the shared experts' rows).
// sh_off (or NULL): [E_s + 1] the shared rows' offsets j*T, for the fp32 path
// that runs them as a launch of their own.
__global__ __launch_bounds__(256) void experts_rows_kernel(int TK, int T, int E_s,
                                                           const int32_t* __restrict__ row_token,
                                                           int32_t* __restrict__ row_index,
                                                           int32_t* __restrict__ sh_off) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r < TK) row_index[r] = row_token[r];
  else if (r < TK + E_s * T) row_index[r] = (r - TK) % T;
  if (sh_off != nullptr && r <= E_s) sh_off[r] = r * T;
}

// Tile list of the combined launch, one workgroup.  Routed expert g and the
// q-th shared row group (shared expert q / per, part q % per) take the
// positions g + ceil(g Q / E_r) and floor(q E_r / Q) + 1 + q, Q = E_s * per
// (together a permutation of 0 .. E_r + Q - 1: the shared groups spread
// evenly among the routed experts); tiles are laid out in position order and
// carry their weight index (g, or E_r + q / per) as the group.
__global__ __launch_bounds__(1024) void build_tiles_experts_kernel(
    int E_r, int E_s, int per, int srows, int T, int TK, int bm, int max_tiles,
    const int32_t* __restrict__ offsets, TileInfo* __restrict__ tiles,
    int32_t* __restrict__ meta) {
  __shared__ int32_t lo_s[kMaxExpertGroups], hi_s[kMaxExpertGroups], wi_s[kMaxExpertGroups];
  __shared__ int32_t cnt[kMaxExpertGroups];
  __shared__ int32_t part[1024];
  const int Q = E_s * per, G = E_r + Q;
  for (int x = threadIdx.x; x < G; x += 1024) {
    int p, lo, hi, wi;
    if (x < E_r) {
      p = x + static_cast<int>((static_cast<long long>(x) * Q + E_r - 1) / E_r);
      lo = min(max(offsets[x], 0), TK);
      hi = min(max(offsets[x + 1], lo), TK);
      wi = x;
    } else {
      const int q = x - E_r, j = q / per, i = q % per;
      p = static_cast<int>(static_cast<long long>(q) * E_r / Q) + 1 + q;
      lo = TK + j * T + i * srows;
      hi = min(lo + srows, TK + (j + 1) * T);
      wi = E_r + j;
    }
    lo_s[p] = lo;
    hi_s[p] = hi;
    wi_s[p] = wi;
    cnt[p] = (hi - lo + bm - 1) / bm;
  }
  __syncthreads();
  // exclusive prefix of cnt over positions: thread i owns positions 2i, 2i+1
  const int i0 = 2 * threadIdx.x;
  const int c0 = i0 < G ? cnt[i0] : 0, c1 = i0 + 1 < G ? cnt[i0 + 1] : 0;
  part[threadIdx.x] = c0 + c1;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = threadIdx.x >= static_cast<unsigned>(off) ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  const int base = part[threadIdx.x] - c0 - c1;
  const int starts[2] = {base, base + c0};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p = i0 + u;
    if (p >= G) continue;
    const int start = starts[u], nt = u == 0 ? c0 : c1;
    for (int t = 0; t < nt && start + t < max_tiles; ++t)
      tiles[start + t] = TileInfo{wi_s[p], lo_s[p] + t * bm, hi_s[p], start,
                                  min(nt, max_tiles - start), {0, 0, 0}};
  }
  if (threadIdx.x == 1023) meta[0] = min(part[1023], max_tiles);
}

}  // namespace

hipError_t launch_build_tiles_experts(int E_r, int E_s, int T, int K, int shared_rows_per_group,
                                      const int32_t* offsets, const int32_t* row_token,
                                      int32_t* row_index, const SwigluWorkspace& w,
                                      hipStream_t s) {
  const int TK = T * K, rows = TK + E_s * T;
  const int per = (T + shared_rows_per_group - 1) / shared_rows_per_group;
  ProfScope prof_(s, "tiles");
  hipLaunchKernelGGL(experts_rows_kernel, dim3((rows + 255) / 256), dim3(256), 0, s, TK, T, E_s,
                     row_token, row_index, nullptr);
  hipLaunchKernelGGL(build_tiles_experts_kernel, dim3(1), dim3(1024), 0, s, E_r, E_s, per,
                     shared_rows_per_group, T, TK, 256, max_tiles_for(rows, E_r + E_s * per, 256),
                     offsets, w.tiles, w.meta);
  return hipGetLastError();
}

hipError_t launch_experts_rows(int T, int K, int E_s, const int32_t* row_token,
                               int32_t* row_index, int32_t* sh_off, hipStream_t s) {
  const int rows = T * K + E_s * T;
  hipLaunchKernelGGL(experts_rows_kernel, dim3((max(rows, E_s + 1) + 255) / 256), dim3(256), 0, s,
                     T * K, T, E_s, row_token, row_index, sh_off);
  return hipGetLastError();
}

hipError_t launch_build_tiles(int n_groups, int rows, int bm, const int32_t* offsets,
                              const SwigluWorkspace& w, hipStream_t s) {
  {
    ProfScope prof_(s, "tiles");
    hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(1024), 0, s, n_groups, rows, bm,
                       max_tiles_for(rows, n_groups, bm), offsets, w.group_tile_start, w.tiles,
                       w.meta);
  }
  return hipGetLastError();
}

hipError_t launch_build_split_tiles(int n_groups, int rows, int small_rows, int off2,
                                    const int32_t* offsets, const SwigluWorkspace& w,
                                    hipStream_t s) {
  {
    ProfScope prof_(s, "tiles");
    hipLaunchKernelGGL(build_split_tiles_kernel, dim3(1), dim3(1024), 0, s, n_groups, rows,
                       small_rows, off2, offsets, w.tiles, w.meta);
  }
  return hipGetLastError();
}

hipError_t launch_swiglu_f32(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                             const int32_t* offsets, const int32_t* row_index, const float* x,
                             const float* wg, const float* wu, const float* wd,
                             const float* row_scale, float* y, void* ws, hipStream_t s) {
  SwigluWorkspace w = swiglu_layout(ws, n_groups, d_ffn, rows, 4, 32);
  hipError_t err = launch_build_tiles(n_groups, rows, kBM, offsets, w, s);
  if (err != hipSuccess) return err;
  const int max_tiles = max_tiles_for(rows, n_groups, kBM);
  float* act = static_cast<float*>(w.act);
  {
    ProfScope prof_(s, "gateup_f32");
    hipLaunchKernelGGL((f32_tile_kernel<true>), dim3(max_tiles, (d_ffn + kBN - 1) / kBN),
                       dim3(kThreads), 0, s, d_model, d_ffn, x_rows, w.tiles, w.meta, row_index,
                       x, wg, wu, nullptr, act);
  }
  {
    ProfScope prof_(s, "down_f32");
    hipLaunchKernelGGL((f32_tile_kernel<false>), dim3(max_tiles, (d_model + kBN - 1) / kBN),
                       dim3(kThreads), 0, s, d_ffn, d_model, rows, w.tiles, w.meta, nullptr, act,
                       wd, nullptr, row_scale, y);
  }
  return hipGetLastError();
}

}  // namespace moe
