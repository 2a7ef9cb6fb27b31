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

// Grouped C = A W[g]^T over the rows of each group (bf16, fp32 accumulation):
// A [rows, K], W [n_groups, N, K], C [rows, N]; K a multiple of 64.  Builds a
// 256-row tile list into w's tile arrays (sized by swiglu_layout with min_bm
// <= 256) and runs the grouped SwiGLU's down-direction kernels.  `name` tags
// the launch in the profile records.
hipError_t launch_grouped_nt_bf16(int n_groups, int K, int N, int rows, const int32_t* offsets,
                                  const SwigluWorkspace& w, const uint16_t* A, const uint16_t* W,
                                  uint16_t* C, const char* name, hipStream_t s);

}  // namespace moe
