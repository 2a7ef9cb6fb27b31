// Workspace layout and the device-side tile list of the grouped SwiGLU.
//
// The groups' row counts live on the device (they come from the router), so
// the host never reads them: a one-workgroup kernel turns the offsets into a
// list of row tiles, and the GEMM grids are sized for the worst case
// (ceil(rows / BM) + n_groups tiles); blocks past the real tile count exit.
#pragma once

#include "common.h"

namespace moe {

struct TileInfo {
  int32_t group;
  int32_t m0;      // first grouped row of the tile
  int32_t m1;      // one past the group's last row (rows >= m1 are masked)
  int32_t gstart;  // index of the group's first tile
  int32_t ntiles;  // number of tiles of the group
  int32_t pad[3];
};
static_assert(sizeof(TileInfo) == 32, "TileInfo is read as eight dwords");

struct SwigluWorkspace {
  void* act;                  // [rows, d_ffn] SiLU(gate) * up
  int32_t* group_tile_start;  // [n_groups + 1] prefix count of tiles per group
  TileInfo* tiles;            // [max_tiles]
  int32_t* meta;              // [0] = number of tiles
  size_t bytes;
};

inline int max_tiles_for(int rows, int n_groups, int bm) { return (rows + bm - 1) / bm + n_groups; }

// The expert weights of one bf16 launch ([n, N, K] stacks).  A tile's group
// field is its weight index g: g < n_first takes expert g of w0 (w1: the W_up
// stack of gate/up), a later g takes expert g - n_first of s0 / s1 (shared
// experts appended to a routed launch).
struct WeightSet {
  const uint16_t* w0;
  const uint16_t* w1;
  const uint16_t* s0;
  const uint16_t* s1;
  int n_first;
  static WeightSet one(const uint16_t* a, const uint16_t* b) {
    return WeightSet{a, b, a, b, 0x7fffffff};
  }
  __device__ __forceinline__ const uint16_t* base(bool second, int g, size_t mat) const {
    return g < n_first ? (second ? w1 : w0) + static_cast<size_t>(g) * mat
                       : (second ? s1 : s0) + static_cast<size_t>(g - n_first) * mat;
  }
};

// Carve the caller's workspace; `base` may be nullptr to only size it.
inline SwigluWorkspace swiglu_layout(void* base, int n_groups, int d_ffn, int rows,
                                     int elem_bytes, int min_bm) {
  SwigluWorkspace w{};
  size_t off = 0;
  auto take = [&](size_t n) {
    size_t at = off;
    off = align_up(off + n, 256);
    return base ? static_cast<char*>(base) + at : nullptr;
  };
  w.act = take(static_cast<size_t>(rows) * d_ffn * elem_bytes);
  w.group_tile_start = reinterpret_cast<int32_t*>(take((n_groups + 1) * sizeof(int32_t)));
  w.tiles = reinterpret_cast<TileInfo*>(
      take(static_cast<size_t>(max_tiles_for(rows, n_groups, min_bm)) * sizeof(TileInfo)));
  w.meta = reinterpret_cast<int32_t*>(take(4 * sizeof(int32_t)));
  w.bytes = off;
  return w;
}

// Backward pass (backward.hip): scratch layout and launches (bf16 only).
struct BwdWorkspace {
  struct {
    TileInfo* tiles;
    int32_t* group_tile_start;
    int32_t* meta;
  } tiles, tiles256;        // 128- and 256-row tiles of the grouped rows
  int32_t* kpad;            // [n_groups + 1] expert rows padded to 64, prefix sums
  uint16_t* au;             // [rows, 2f]  a | u, when the backward recomputes them
  uint16_t* dadu;           // [rows, 2f]  da | du
  uint16_t *xT, *dyT;       // per-expert [d, mpad] blocks
  uint16_t *actT, *daT, *duT;  // per-expert [f, mpad] blocks
  size_t bytes;
};
BwdWorkspace bwd_layout(void* base, int n_groups, int d, int f, int rows);
size_t bwd_workspace_bytes(int n_groups, int d, int f, int rows);
size_t bwd_rpad_max(int n_groups, int rows);
hipError_t launch_swiglu_backward(int n_groups, int d, int f, int rows, int x_rows,
                                  const int32_t* offsets, const int32_t* row_index,
                                  const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                                  const uint16_t* wgu_t, const uint16_t* wd_t,
                                  const uint16_t* dy, const uint16_t* au, uint16_t* dx,
                                  uint16_t* dwg, uint16_t* dwu, uint16_t* dwd, void* ws,
                                  hipStream_t s);
hipError_t launch_combine_backward(int T, int d, int K, const uint16_t* dy, const uint16_t* yp,
                                   const int32_t* slot_row, const float* gates, uint16_t* dyp,
                                   float* dg, hipStream_t s);
hipError_t launch_route_backward(int T, int d, int E, int K, int fn, const uint16_t* h,
                                 const float* e, const int32_t* idx, const float* dg,
                                 const int32_t* offsets, const int32_t* row_token, float* dz,
                                 uint16_t* dh, float* de, hipStream_t s);
hipError_t launch_transpose_experts(int n, int rows, int cols, const uint16_t* src,
                                    uint16_t* dst, int ld, int col_off, hipStream_t s);

hipError_t launch_build_tiles(int n_groups, int rows, int bm, const int32_t* offsets,
                              const SwigluWorkspace& w, hipStream_t s);

// Two tile lists for matrix-core-bound launches: 256-row tiles in w.tiles
// (count in w.meta[0]) except each group's last rows when they are fewer than
// small_rows, which get one tile of their own in a second list at
// w.tiles + off2 (count in w.meta[2]), for a kernel that streams such tiles
// faster.  off2 >= max_tiles_for(rows, n_groups, 256); w's tile array must
// hold off2 + n_groups tiles.
hipError_t launch_build_split_tiles(int n_groups, int rows, int small_rows, int off2,
                                    const int32_t* offsets, const SwigluWorkspace& w,
                                    hipStream_t s);

// Routed and shared experts in one grouped launch (moe_experts_swiglu).
// Grouped rows: the T*K routed rows (expert g on offsets[g] .. offsets[g+1]-1,
// gathered through row_token), then shared expert j on rows T*K + j*T + t
// (token t).  Each shared expert's rows are cut into groups of
// shared_rows_per_group rows, and the tile list places those groups evenly
// among the routed experts, so that each XCD's contiguous run of work items
// (the persistent kernels' order) holds about the same share of them.
struct ExpertsLayout {
  int n_groups;                // E_r + E_s * groups per shared expert
  int rows;                    // T*K + E_s*T
  int shared_rows_per_group;
  int32_t* row_index;          // [rows]: row_token, then the token of each shared row
  SwigluWorkspace sw;          // activations and the tile list
  size_t bytes;
};
inline int experts_shared_rows_per_group(int T) {
  // about one group per XCD: ceil(T / 8) rounded up to a 256-row tile
  return ((T + 8 * 256 - 1) / (8 * 256)) * 256;
}
inline ExpertsLayout experts_layout(void* base, int E_r, int E_s, int T, int K, int d_ffn) {
  ExpertsLayout L{};
  L.shared_rows_per_group = experts_shared_rows_per_group(T);
  const int per = (T + L.shared_rows_per_group - 1) / L.shared_rows_per_group;
  L.n_groups = E_r + E_s * per;
  L.rows = T * K + E_s * T;
  const size_t ri = align_up(static_cast<size_t>(L.rows) * sizeof(int32_t), 256);
  L.row_index = base ? static_cast<int32_t*>(base) : nullptr;
  L.sw = swiglu_layout(base ? static_cast<char*>(base) + ri : nullptr, L.n_groups, d_ffn, L.rows,
                       2, 256);
  L.bytes = ri + L.sw.bytes;
  return L;
}
constexpr int kMaxExpertGroups = 2048;
// Fills L.row_index and builds the 256-row tile list of the combined groups.
hipError_t launch_build_tiles_experts(int E_r, int E_s, int T, int K, int shared_rows_per_group,
                                      const int32_t* offsets, const int32_t* row_token,
                                      int32_t* row_index, const SwigluWorkspace& w,
                                      hipStream_t s);
hipError_t launch_experts_rows(int T, int K, int E_s, const int32_t* row_token,
                               int32_t* row_index, int32_t* sh_off, hipStream_t s);
hipError_t launch_experts_bf16(int E_r, int E_s, int T, int K, int d_model, int d_ffn,
                               const int32_t* offsets, const int32_t* row_token,
                               const uint16_t* h, const uint16_t* wg, const uint16_t* wu,
                               const uint16_t* wd, const uint16_t* wsg, const uint16_t* wsu,
                               const uint16_t* wsd, uint16_t* y, void* ws, hipStream_t s);

// Grouped C = A W[g]^T over the rows of each group (bf16, fp32 accumulation):
// A [rows, K], W [n_groups, N, K], C [rows, N]; K a multiple of 64.  Builds a
// tile list of tile_rows-row tiles into w's tile arrays (sized by
// swiglu_layout with min_bm <= tile_rows; tiles_built: w already holds that
// list for these offsets) and runs the grouped SwiGLU's down-direction
// kernels.  tile_rows is 256 or what grouped_nt_tile_rows returns.  `name`
// tags the launch in the profile records.
hipError_t launch_grouped_nt_bf16(int n_groups, int K, int N, int rows, const int32_t* offsets,
                                  const SwigluWorkspace& w, const uint16_t* A, const uint16_t* W,
                                  uint16_t* C, const char* name, hipStream_t s,
                                  bool tiles_built = false, int tile_rows = 256);

// Row-tile size for a pair of such products over the same groups, (K1, N1)
// and (K2, N2): the rows of the kernel that sends both operands by LDS DMA
// when the groups average at most 128 rows and both shapes fit it, else 256.
int grouped_nt_tile_rows(int n_groups, int rows, int K1, int N1, int K2, int N2);

}  // namespace moe
