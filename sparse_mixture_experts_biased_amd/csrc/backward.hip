// Backward pass of the layer (bf16 operands, fp32 accumulation).
//
// Method: the chain rule applied to the layer-output, SwiGLU, gate and score
// equations of the Sparse MoE routing-math page (arman1o1.github.io),
// sections 0 and 2, with the routing decisions of the forward pass fixed.
// With a = x W_gate^T, u = x W_up^T, act = SiLU(a) u, per expert:
//   d act = dy W_down;  da = d act * u * SiLU'(a);  du = d act * SiLU(a)
//   dx = da W_gate + du W_up
//   dW_down = dy^T act;  dW_gate = da^T x;  dW_up = du^T x
// SiLU'(a) = sigma(a) (1 + a (1 - sigma(a))).  The gate gradient reaches the
// router only through the unbiased scores s (section 2: the bias picks, it
// gets no gradient).
//
// Every product is an "NT" grouped GEMM (both operands K-contiguous) on
// v_mfma_f32_32x32x16_bf16: transposed weight copies W_down^T [f, d] and
// [W_gate^T | W_up^T] [d, 2f] (built once per weight update) serve the
// activation gradients, which run on the forward pass's down-direction
// streaming kernels (with the SwiGLU derivative as a separate elementwise
// pass), and per-expert transposed activations (each expert's rows padded to
// a multiple of 64 and laid out as its own [C, rows] block) serve the weight
// gradients, whose K is the expert's row count (kernels below).
#include "swiglu_tiles.h"

#include <algorithm>

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 64;  // tile
constexpr int kThreads = 256;                   // 4 waves, 2 x 2, 64 x 64 each
constexpr int kRowBytes = kBK * 2;
constexpr int kBufferFlags = 0x00020000;
constexpr uint32_t kOff = 0x80000000u;          // beyond every buffer (< 2 GiB)
constexpr int kPad = 64;                         // expert rows padded to this in the
                                                 // transposed layouts
constexpr int kNumXcdB = 8;                      // XCDs (L2 domains) of the chip

__device__ __forceinline__ int swz(int r, int c) {
  return r * kRowBytes + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes),
                                           kBufferFlags);
}

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Arguments of the two backward GEMMs: "Rows" = bwd_gemm_kernel (products
// over the grouped rows), "Kvar" = kvar_stream_kernel (weight gradients).
struct GemmArgs {
  int M, N, K;             // Rows: N, K used (rows from the tile list); Kvar: M, N
  int NT, MT;              // column / row tiles per group
  int n_groups;
  const TileInfo* tiles;   // Rows
  const int32_t* meta;     // Rows: meta[0] = tiles
  const int32_t* kpad;     // Kvar: padded row offsets [n_groups + 1]
  const int32_t* row_index;  // Rows: A row gather (NULL: grouped row itself)
  int a_rows;              // Rows: rows of A (bound of the gather)
  const uint16_t* A;       // Rows: [a_rows, lda]; Kvar: per-group blocks [M, mpad]
  int lda;
  const uint16_t* B;       // Rows: per-group [N, ldb] at B + g * b_stride; Kvar: blocks [N, mpad]
  int ldb;
  size_t b_stride;
  uint16_t* C;             // Rows: [rows, ldc]; Kvar: per group [M, ldc] at C + g * c_stride
  int ldc;
  size_t c_stride;
};

// C = A B^T over one 128 x 128 tile of the grouped rows (the a, u recompute);
// K in 64-wide slices.  Three register sets rotate through the global loads,
// so up to three slices are in flight while one is multiplied out of LDS.
// Four waves in a 2 x 2 layout, each 64 x 64.
constexpr int kSets = 3;

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_gemm_kernel(GemmArgs p) {
  constexpr int BM = kBM, BN = kBN;
  constexpr int kWN = 2;                           // waves along N (2 x 2 waves)
  constexpr int kNB = BN / kWN / 32;               // 32-wide column blocks per wave
  constexpr int kWNC = BN / kWN;                   // columns per wave
  constexpr int kAP = BM / 32, kBP = BN / 32;      // load passes (32 rows each)
  constexpr int kStageT = (BM + BN) * kRowBytes;
  // operand stages, and the output tile staged by the epilogue
  constexpr int kSmem0 = 2 * kStageT;
  constexpr int kSmem1 = BM * BN * 2;
  __shared__ __attribute__((aligned(16))) char smem[kSmem0 > kSmem1 ? kSmem0 : kSmem1];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int wm = wave / kWN, wn = wave % kWN;
  const int lc = tid & 7, lr = tid >> 3;  // 32 rows per load pass

  const int w = blockIdx.x;
  if (w >= p.meta[0] * p.NT) return;
  const TileInfo ti = p.tiles[w / p.NT];
  const int g = ti.group;
  const int m0 = ti.m0;
  const int nrows = min(ti.m1 - ti.m0, BM);
  const int n0 = (w % p.NT) * BN;
  const int nk = p.K / kBK;

  // ---- operand sources
  __amdgpu_buffer_rsrc_t rsA, rsB;
  uint32_t a_off[kAP], b_off[kBP];
  rsA = rsrc(p.A, static_cast<uint32_t>(p.a_rows) * p.lda * 2u);
#pragma unroll
  for (int i = 0; i < kAP; ++i) {
    const int r = lr + 32 * i;
    int sr = -1;
    if (r < nrows) {
      sr = p.row_index ? p.row_index[m0 + r] : m0 + r;
      if (sr < 0 || sr >= p.a_rows) sr = -1;
    }
    a_off[i] = sr >= 0 ? (static_cast<uint32_t>(sr) * p.lda + lc * 8) * 2u : kOff;
  }
  rsB = rsrc(p.B + static_cast<size_t>(g) * p.b_stride, static_cast<uint32_t>(p.N) * p.ldb * 2u);
#pragma unroll
  for (int i = 0; i < kBP; ++i) {
    const int n = n0 + lr + 32 * i;
    b_off[i] = n < p.N ? (static_cast<uint32_t>(n) * p.ldb + lc * 8) * 2u : kOff;
  }

  f32x16_t acc[2][kNB];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < kNB; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.0f;

  auto load = [&](uint4 (&sa)[kAP], uint4 (&sb)[kBP], int kt) {
    const uint32_t kb = static_cast<uint32_t>(kt) * kBK * 2u;
#pragma unroll
    for (int i = 0; i < kAP; ++i)
      sa[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsA, a_off[i], kb, 0));
#pragma unroll
    for (int i = 0; i < kBP; ++i)
      sb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsB, b_off[i], kb, 0));
  };
  auto store = [&](const uint4 (&sa)[kAP], const uint4 (&sb)[kBP], int stage) {
    char* as = smem + stage * kStageT;
    char* bs = as + BM * kRowBytes;
#pragma unroll
    for (int i = 0; i < kAP; ++i) *reinterpret_cast<uint4*>(as + swz(lr + 32 * i, lc)) = sa[i];
#pragma unroll
    for (int i = 0; i < kBP; ++i) *reinterpret_cast<uint4*>(bs + swz(lr + 32 * i, lc)) = sb[i];
  };
  const int fr = lane & 31, fh = lane >> 5;
  const bool busy = wm * 64 < nrows;
  auto compute = [&](int stage) {
    if (!busy) return;
    const char* as = smem + stage * kStageT;
    const char* bs = as + BM * kRowBytes;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int c = kk * 2 + fh;
      bf16x8_t af[2], bq[kNB];
#pragma unroll
      for (int x = 0; x < 2; ++x)
        af[x] = *reinterpret_cast<const bf16x8_t*>(as + swz(wm * 64 + x * 32 + fr, c));
#pragma unroll
      for (int x = 0; x < kNB; ++x)
        bq[x] = *reinterpret_cast<const bf16x8_t*>(bs + swz(wn * kWNC + x * 32 + fr, c));
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < kNB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bq[b], acc[a][b], 0, 0, 0);
    }
  };

  // Step J multiplies slice J (LDS stage J % 2), refills the register set
  // that held it with slice J + 3 (past the end it re-reads the last slice, an
  // L2 hit, so every step issues the same loads and the waits stay exact) and
  // stores slice J + 1 to the other stage.
  if (nk > 0) {
    static_assert(kSets == 3, "the step sequence below rotates three sets");
    uint4 sa0[kAP], sb0[kBP], sa1[kAP], sb1[kBP], sa2[kAP], sb2[kBP];
    load(sa0, sb0, 0);
    load(sa1, sb1, min(1, nk - 1));
    load(sa2, sb2, min(2, nk - 1));
    store(sa0, sb0, 0);
    __syncthreads();
#define MOE_BSTEP(J, LA, LB, STAGE, SA, SB) \
  load(LA, LB, min((J) + kSets, nk - 1));   \
  compute(STAGE);                           \
  if ((J) + 1 >= nk) break;                 \
  store(SA, SB, (STAGE) ^ 1);               \
  __syncthreads();
    for (int kt = 0;; kt += 6) {
      MOE_BSTEP(kt + 0, sa0, sb0, 0, sa1, sb1)
      MOE_BSTEP(kt + 1, sa1, sb1, 1, sa2, sb2)
      MOE_BSTEP(kt + 2, sa2, sb2, 0, sa0, sb0)
      MOE_BSTEP(kt + 3, sa0, sb0, 1, sa1, sb1)
      MOE_BSTEP(kt + 4, sa1, sb1, 0, sa2, sb2)
      MOE_BSTEP(kt + 5, sa2, sb2, 1, sa0, sb0)
    }
#undef MOE_BSTEP
    __syncthreads();
  }

  // ---- epilogue through LDS (both stages are free after the last barrier):
  // the tile is staged as bf16 rows of 128 columns (16-byte chunk index XORed
  // with row & 4, which separates the two half-waves) and written as whole
  // 16-byte row chunks.  D[row][col] of a 32x32 block is in lane
  // col + 32*((row/4)%2), register (row%4) + 4*(row/8).
  constexpr int kORow = BN * 2;                   // bytes per staged row
  constexpr int kOC = BN / 8;                     // 16-byte chunks per row
  constexpr int kORP = kThreads / kOC;            // rows per read-out pass
  static_assert(kORP % 8 == 0, "read-out rows keep row & 4");
  static_assert(BM * kORow <= sizeof(smem), "staging fits");
  char* o0 = smem;                                // [BM][BN] bf16
  auto opos = [&](int row, int col) {
    return row * kORow + ((((col >> 3) ^ (row & 4))) << 4) + (col & 7) * 2;
  };
  const int rl = tid / kOC, cl = tid % kOC;       // read-out position
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = wm * 64 + a * 32 + 8 * (q >> 2) + 4 * fh + (q & 3);
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        const int col = wn * kWNC + b * 32 + fr;
        *reinterpret_cast<uint16_t*>(o0 + opos(row, col)) = f32_to_bf16(acc[a][b][q]);
      }
    }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < BM / kORP; ++it) {
    const int row = it * kORP + rl;
    if (row >= nrows || n0 + cl * 8 >= p.N) continue;
    const size_t r = static_cast<size_t>(m0 + row);
    const int sw = (cl ^ (row & 4)) << 4;
    *reinterpret_cast<uint4*>(p.C + r * p.ldc + n0 + cl * 8) =
        *reinterpret_cast<const uint4*>(o0 + row * kORow + sw);
  }
}

// SwiGLU derivative, elementwise over [rows, f] in 8-column pieces: with
// a | u = au[r], s = sigma(a): da = d act * u * s (1 + a (1 - s)),
// du = d act * a * s, written as dadu[r] = da | du.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(int rows, int f,
                                                         const uint16_t* __restrict__ dact,
                                                         const uint16_t* __restrict__ au,
                                                         uint16_t* __restrict__ dadu) {
  const int f8 = f / 8;
  const long n8 = static_cast<long>(rows) * f8;
  for (long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x; i < n8;
       i += static_cast<long>(gridDim.x) * 256) {
    const long r = i / f8;
    const int c = static_cast<int>(i - r * f8) * 8;
    const uint4 gv = *reinterpret_cast<const uint4*>(dact + r * f + c);
    const uint4 av = *reinterpret_cast<const uint4*>(au + r * 2 * f + c);
    const uint4 uv = *reinterpret_cast<const uint4*>(au + r * 2 * f + f + c);
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, aw[4] = {av.x, av.y, av.z, av.w},
                   uw[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t da[4], du[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float dv[2], dd[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float g = __uint_as_float(h ? (gw[j] & 0xffff0000u) : (gw[j] << 16));
        const float a = __uint_as_float(h ? (aw[j] & 0xffff0000u) : (aw[j] << 16));
        const float u = __uint_as_float(h ? (uw[j] & 0xffff0000u) : (uw[j] << 16));
        const float sg = sigm(a);
        dv[h] = g * u * sg * (1.0f + a * (1.0f - sg));
        dd[h] = g * a * sg;
      }
      da[j] = pack_bf16x2(dv[0], dv[1]);
      du[j] = pack_bf16x2(dd[0], dd[1]);
    }
    *reinterpret_cast<uint4*>(dadu + r * 2 * f + c) = make_uint4(da[0], da[1], da[2], da[3]);
    *reinterpret_cast<uint4*>(dadu + r * 2 * f + f + c) = make_uint4(du[0], du[1], du[2], du[3]);
  }
}

// kpad[g] = sum over groups before g of their rows rounded up to kPad.
__global__ __launch_bounds__(1024) void pad_offsets_kernel(int n_groups, int rows,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ kpad) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry_s;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  for (int g0 = 0; g0 < n_groups; g0 += 1024) {
    const int g = g0 + threadIdx.x;
    int m = 0;
    if (g < n_groups) {
      const int lo = min(max(offsets[g], 0), rows);
      const int hi = min(max(offsets[g + 1], lo), rows);
      m = (hi - lo + kPad - 1) / kPad * kPad;
    }
    part[threadIdx.x] = m;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = threadIdx.x >= static_cast<unsigned>(off) ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    const int carry = carry_s;
    if (g < n_groups) kpad[g] = carry + part[threadIdx.x] - m;
    __syncthreads();
    if (threadIdx.x == 1023) carry_s = carry + part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) kpad[n_groups] = carry_s;
}

enum { kTrCopy = 0, kTrAct = 1 };

// Transposes the rows of one 256-row tile (rows m0 .. m0 + nr of one expert)
// and 64 source columns into the expert's [C, mpad] block: block column = the
// row's position inside its expert.  The expert's last tile also writes the
// zero padding columns.  kTrAct: the source value is SiLU(a) * u from src =
// [a | u] (ld 2C).  Grid (tiles, C / 64), 256 threads.
//
// Load: each thread takes one 8-column piece (16 bytes) of 8 rows -- rows 2p,
// 2p + 1 of four 64-row bands -- with all eight loads issued before any is
// used.  LDS: [64 columns][256 rows], element (c, r) at row position
// r ^ (16 (c >> 3)); a thread writes each of its columns for its row pair as
// one 32-bit word, and the XOR puts the 64 lanes' words of one write in 64
// distinct banks.  The XOR leaves bits 0-2 of r alone, so any 8 consecutive
// rows of a column stay one aligned 16-byte piece.  Store: 16-byte pieces of
// the block rows, consecutive lanes along a row.
template <int TR>
__global__ __launch_bounds__(256) void pad_transpose_kernel(
    int C, int rows, int src_rows, const TileInfo* __restrict__ tiles,
    const int32_t* __restrict__ meta, const int32_t* __restrict__ kpad,
    const int32_t* __restrict__ row_index, const uint16_t* __restrict__ src, int ld_src,
    uint16_t* __restrict__ dst) {
  constexpr int kTM = 256;  // rows of a tile
  __shared__ __attribute__((aligned(16))) uint16_t t[64][kTM];
  if (static_cast<int>(blockIdx.x) >= meta[0]) return;
  const TileInfo ti = tiles[blockIdx.x];
  const int g = ti.group;
  const int m0 = ti.m0;
  const int nr = min(ti.m1 - ti.m0, kTM);
  const int c0 = blockIdx.y * 64;
  const int p0 = m0 - tiles[ti.gstart].m0;  // first block column of this tile (a multiple of 256)
  const int mpad = kpad[g + 1] - kpad[g];
  uint16_t* blk = dst + static_cast<size_t>(kpad[g]) * C;  // [C, mpad]
  const int tid = threadIdx.x;
  const int c8 = tid & 7;     // 8-column piece
  const int pr = tid >> 3;    // row pair 0..31
  // Branch-free loads, so that a thread's eight index loads, then its eight
  // data loads, are in flight together: a row past the tile, a piece past C
  // or an invalid source row loads from a valid address (the tile's first row,
  // source row 0) and is zeroed afterwards.
  const bool col_ok = c0 + 8 * c8 < C && src_rows > 0;
  const int col = col_ok ? c0 + 8 * c8 : 0;
  int sr[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 64 * i + 2 * pr + h;
      const int gr = m0 + (r < nr ? r : 0);  // nr >= 1: m0 is a row of the tile
      sr[i][h] = row_index ? row_index[gr] : gr;
    }
  bool ok[4][2];
  uint4 av[4][2], uv[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 64 * i + 2 * pr + h;
      ok[i][h] = r < nr && col_ok && sr[i][h] >= 0 && sr[i][h] < src_rows;
      const uint16_t* sp =
          src + (ok[i][h] ? static_cast<size_t>(sr[i][h]) * ld_src + col : static_cast<size_t>(0));
      av[i][h] = *reinterpret_cast<const uint4*>(sp);
      if (TR == kTrAct) uv[i][h] = *reinterpret_cast<const uint4*>(sp + C);
    }
  uint4 v[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 x = av[i][h];
      if (TR == kTrAct) {
        const uint4 u4 = uv[i][h];
        const uint32_t aw[4] = {x.x, x.y, x.z, x.w}, uw[4] = {u4.x, u4.y, u4.z, u4.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = silu(__uint_as_float(aw[q] << 16)) * __uint_as_float(uw[q] << 16);
          const float hi =
              silu(__uint_as_float(aw[q] & 0xffff0000u)) * __uint_as_float(uw[q] & 0xffff0000u);
          o[q] = pack_bf16x2(lo, hi);
        }
        x = make_uint4(o[0], o[1], o[2], o[3]);
      }
      v[i][h] = ok[i][h] ? x : make_uint4(0, 0, 0, 0);
    }
  const int swz = 16 * c8;  // the XOR of every column this thread writes (c >> 3 == c8)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo[4] = {v[i][0].x, v[i][0].y, v[i][0].z, v[i][0].w};
    const uint32_t hi[4] = {v[i][1].x, v[i][1].y, v[i][1].z, v[i][1].w};
    const int rpos = (64 * i + 2 * pr) ^ swz;  // even: the pair is one aligned word
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t a = (j & 1) ? (lo[j / 2] >> 16) : (lo[j / 2] & 0xffffu);
      const uint32_t b = (j & 1) ? (hi[j / 2] >> 16) : (hi[j / 2] & 0xffffu);
      *reinterpret_cast<uint32_t*>(&t[8 * c8 + j][rpos]) = a | (b << 16);
    }
  }
  __syncthreads();
  const bool last = ti.m1 - m0 <= kTM;
  // the last tile also writes the padding: width = mpad - p0 <= 256, a multiple
  // of 64; LDS rows past nr hold the zeros loaded for them
  const int width = last ? mpad - p0 : nr;
  const int w8 = width / 8;
  for (int q = tid; q < 64 * w8; q += 256) {
    const int c = q / w8, r8 = q - c * w8;
    if (c0 + c >= C) continue;
    const int pos = (8 * r8) ^ (16 * (c >> 3));
    *reinterpret_cast<uint4*>(blk + static_cast<size_t>(c0 + c) * mpad + p0 + 8 * r8) =
        *reinterpret_cast<const uint4*>(&t[c][pos]);
  }
}

// Combine backward, one wave per token: dy_perm[slot] = g * dy_t (output
// rows of dropped copies are not written) and dg[t, k] = <dy_t, y_perm[slot]>
// (0 for a dropped copy).  16-byte pieces: per piece of dy_t all K rows are
// loaded before any is used; a dropped slot reads zeros and writes nothing
// through an out-of-range buffer offset.  The K dot products are reduced
// across the wave once at the end.
constexpr uint32_t kOffNoRow = 0x80000000u;

__global__ __launch_bounds__(256) void combine_bwd_kernel(int T, int d, int K, int TK,
                                                          const uint16_t* __restrict__ dy,
                                                          const uint16_t* __restrict__ yp,
                                                          const int32_t* __restrict__ slot_row,
                                                          const float* __restrict__ gates,
                                                          uint16_t* __restrict__ dyp,
                                                          float* __restrict__ dg) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  if (t >= T) return;
  const int vecs = d / 8;
  const uint32_t bytes = static_cast<uint32_t>(TK) * d * 2u;
  const __amdgpu_buffer_rsrc_t rsY = rsrc(yp, bytes), rsO = rsrc(dyp, bytes);
  const int sl = lane < K ? slot_row[static_cast<size_t>(t) * K + lane] : -1;
  const float gl = lane < K ? gates[static_cast<size_t>(t) * K + lane] : 0.0f;
  uint32_t off[MOE_MAX_TOPK_DEV];
  float g[MOE_MAX_TOPK_DEV], dot[MOE_MAX_TOPK_DEV];
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) {
    const int sk = __builtin_amdgcn_readlane(sl, k);
    off[k] = (k < K && sk >= 0 && sk < TK) ? static_cast<uint32_t>(sk) * d * 2u : kOffNoRow;
    g[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gl), k));
    dot[k] = 0.0f;
  }
  const uint4* dyr = reinterpret_cast<const uint4*>(dy + static_cast<size_t>(t) * d);
  for (int c = lane; c < vecs; c += kWave) {
    const uint4 dv = dyr[c];
    const uint32_t cb = static_cast<uint32_t>(c) * 16u;
    uint4 yv[MOE_MAX_TOPK_DEV];
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
      if (k < K)
        yv[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsY, off[k] + cb, 0, 0));
    const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
    float df[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      df[2 * i] = __uint_as_float(dw[i] << 16);
      df[2 * i + 1] = __uint_as_float(dw[i] & 0xffff0000u);
    }
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) {
      if (k < K) {
        const uint32_t yw[4] = {yv[k].x, yv[k].y, yv[k].z, yv[k].w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dot[k] = fmaf(df[2 * i], __uint_as_float(yw[i] << 16), dot[k]);
          dot[k] = fmaf(df[2 * i + 1], __uint_as_float(yw[i] & 0xffff0000u), dot[k]);
          o[i] = pack_bf16x2(g[k] * df[2 * i], g[k] * df[2 * i + 1]);
        }
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int,
                               make_uint4(o[0], o[1], o[2], o[3])),
            rsO, off[k] + cb, 0, 0);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) {
    if (k < K) {
      float v = dot[k];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
      if (lane == 0) dg[static_cast<size_t>(t) * K + k] = v;
    }
  }
}

// Router backward, one wave per token: logits of the K picks, dz, and
// dh_t += sum_k dz_k e_k (dh in the tokens' dtype).  Each lane takes 8
// consecutive columns per step (16 bytes of h or dh, 32 of each centroid row),
// with the K centroid pieces loaded before any is used; the K logits are
// reduced across the wave once.
__global__ __launch_bounds__(256) void route_bwd_token_kernel(
    int T, int d, int E, int K, int fn, const uint16_t* __restrict__ h, const float* __restrict__ e,
    const int32_t* __restrict__ idx, const float* __restrict__ dg, float* __restrict__ dz_out,
    uint16_t* __restrict__ dh) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  if (t >= T) return;
  const int vecs = d / 8;
  const int il = lane < K ? idx[static_cast<size_t>(t) * K + lane] : -1;
  const float dgl = lane < K ? dg[static_cast<size_t>(t) * K + lane] : 0.0f;
  int id[MOE_MAX_TOPK_DEV];
  float z[MOE_MAX_TOPK_DEV], w[MOE_MAX_TOPK_DEV], dgk[MOE_MAX_TOPK_DEV];
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) {
    const int i = __builtin_amdgcn_readlane(il, k);
    id[k] = (k < K && i >= 0 && i < E) ? i : -1;
    dgk[k] = id[k] >= 0 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                        __builtin_bit_cast(int, dgl), k))
                        : 0.0f;
    z[k] = 0.0f;
  }
  const uint4* hr = reinterpret_cast<const uint4*>(h + static_cast<size_t>(t) * d);
  auto h8 = [](const uint4& v, float (&f)[8]) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  };
  for (int c = lane; c < vecs; c += kWave) {
    float hf[8];
    h8(hr[c], hf);
    float4 ev[MOE_MAX_TOPK_DEV][2];
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
      if (id[k] >= 0) {
        const float4* er = reinterpret_cast<const float4*>(e + static_cast<size_t>(id[k]) * d) + 2 * c;
        ev[k][0] = er[0];
        ev[k][1] = er[1];
      }
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
      if (id[k] >= 0) {
        const float ef[8] = {ev[k][0].x, ev[k][0].y, ev[k][0].z, ev[k][0].w,
                             ev[k][1].x, ev[k][1].y, ev[k][1].z, ev[k][1].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) z[k] = fmaf(hf[j], ef[j], z[k]);
      }
  }
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
    if (id[k] >= 0) {
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) z[k] += __shfl_xor(z[k], m, kWave);
    }
  // g over the picks and dz (wave-uniform scalars)
  float gsum = 0.0f, zmax = -INFINITY;
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
    if (id[k] >= 0) zmax = fmaxf(zmax, z[k]);
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) {
    w[k] = 0.0f;
    if (id[k] >= 0) w[k] = fn == 0 ? sigm(z[k]) : __expf(z[k] - zmax);
    gsum += w[k];
  }
  gsum = fmaxf(gsum, 1e-12f);
  float gdg = 0.0f;
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) gdg += (w[k] / gsum) * dgk[k];
  float dz[MOE_MAX_TOPK_DEV];
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) {
    dz[k] = 0.0f;
    if (id[k] < 0) continue;
    const float gk = w[k] / gsum;
    dz[k] = fn == 0 ? (dgk[k] - gdg) / gsum * w[k] * (1.0f - w[k]) : gk * (dgk[k] - gdg);
  }
  if (lane < K) {
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
      if (k == lane) v = dz[k];
    dz_out[static_cast<size_t>(t) * K + lane] = v;
  }
  uint4* dhr = reinterpret_cast<uint4*>(dh + static_cast<size_t>(t) * d);
  for (int c = lane; c < vecs; c += kWave) {
    float acc[8];
    h8(dhr[c], acc);
    float4 ev[MOE_MAX_TOPK_DEV][2];
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
      if (id[k] >= 0) {
        const float4* er = reinterpret_cast<const float4*>(e + static_cast<size_t>(id[k]) * d) + 2 * c;
        ev[k][0] = er[0];
        ev[k][1] = er[1];
      }
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
      if (id[k] >= 0) {
        const float ef[8] = {ev[k][0].x, ev[k][0].y, ev[k][0].z, ev[k][0].w,
                             ev[k][1].x, ev[k][1].y, ev[k][1].z, ev[k][1].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(dz[k], ef[j], acc[j]);
      }
    dhr[c] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                        pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

// de_i = sum over expert i's copies (uncapped dispatch, ascending token) of
// dz * h_t; one workgroup per expert: the copies' weights dz are looked up
// once into LDS, then each thread accumulates 8 columns of h rows (16-byte
// loads) in the segment's order -- a fixed order, so deterministic.
__global__ __launch_bounds__(256) void route_bwd_de_kernel(int T, int d, int E, int K,
                                                           const uint16_t* __restrict__ h,
                                                           const int32_t* __restrict__ idx,
                                                           const float* __restrict__ dz,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ row_token,
                                                           float* __restrict__ de) {
  constexpr int kRows = 512;                 // copies staged per pass
  __shared__ float wr[kRows];
  __shared__ int tr[kRows];
  const int i = blockIdx.x;
  const int lo = offsets[i], hi = offsets[i + 1];
  const int nv = d / 8;                      // 16-byte vectors per row
  for (int v0 = 0; v0 < nv; v0 += 256) {
    const int v = v0 + threadIdx.x;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int r0 = lo; r0 < hi; r0 += kRows) {
      const int n = min(kRows, hi - r0);
      __syncthreads();
      for (int q = threadIdx.x; q < n; q += 256) {
        const int t = row_token[r0 + q];
        float w = 0.0f;
        if (t >= 0 && t < T)
          for (int k = 0; k < K; ++k)
            if (idx[static_cast<size_t>(t) * K + k] == i) w = dz[static_cast<size_t>(t) * K + k];
        wr[q] = w;
        tr[q] = (t >= 0 && t < T) ? t : -1;
      }
      __syncthreads();
      if (v < nv)
        for (int q = 0; q < n; ++q) {
          if (tr[q] < 0) continue;
          const uint4 hv = *reinterpret_cast<const uint4*>(h + static_cast<size_t>(tr[q]) * d + v * 8);
          const uint32_t u[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[2 * c] += wr[q] * __uint_as_float(u[c] << 16);
            acc[2 * c + 1] += wr[q] * __uint_as_float(u[c] & 0xffff0000u);
          }
        }
    }
    if (v < nv) {
      float4* out = reinterpret_cast<float4*>(de + static_cast<size_t>(i) * d + v * 8);
      out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

// out[n][c][ld * ? ] : dst[e * cols * ld + c * ld + col_off + r] = src[e][r][c]
__global__ __launch_bounds__(256) void transpose_experts_kernel(int rows, int cols,
                                                                const uint16_t* __restrict__ src,
                                                                uint16_t* __restrict__ dst, int ld,
                                                                int col_off) {
  __shared__ uint16_t t[64][65];
  const int e = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const uint16_t* s = src + static_cast<size_t>(e) * rows * cols;
  uint16_t* o = dst + static_cast<size_t>(e) * cols * ld;
  for (int q = threadIdx.x; q < 64 * 64; q += 256) {
    const int r = q / 64, c = q % 64;
    t[c][r] = (r0 + r < rows && c0 + c < cols) ? s[static_cast<size_t>(r0 + r) * cols + c0 + c] : 0;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 64 * 64; q += 256) {
    const int c = q / 64, r = q % 64;
    if (r0 + r < rows && c0 + c < cols)
      o[static_cast<size_t>(c0 + c) * ld + col_off + r0 + r] = t[c][r];
  }
}


// ---------------------------------------------------------------- weight gradients, streamed
//
// C[g] [M, N] = A_g [M, K_g] B_g [N, K_g]^T for every group g, K_g = the
// group's padded row count (two or three 64-k slices at 128 rows per expert),
// over 256 x 256 output tiles.  One tile's own work is short, so a workgroup
// per tile waits out its first loads every time.  Here one persistent
// workgroup per CU walks an XCD-contiguous run of tiles as one continuous
// stream of k-slices, laid out like the forward pass's register-staged
// streaming kernel: two register sets keep the two slices after the current
// one in flight (also across tiles), two LDS stages alternate, and after a
// tile's last slice its output leaves through the stage that slice used, in
// two rounds of 128 rows.  Eight waves, 4 along M x 2 along N, each 64 x 128
// (2 x 4 blocks of v_mfma_f32_32x32x16_bf16).  A group without rows still
// gets one slice (every load out of range: zeros), so its tiles are written
// as zeros.  Past the last tile the load side re-reads its last slice (an L2
// hit), so every step issues the same loads.
constexpr int kVM = 256, kVN = 256, kVThreads = 512;

__global__ __launch_bounds__(kVThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void kvar_stream_kernel(GemmArgs p, const int32_t* __restrict__ kpad) {
  constexpr int kWNw = 2;                          // waves along N
  constexpr int kNB = kVN / kWNw / 32;             // 32-wide column blocks per wave
  constexpr int kWNC = kVN / kWNw;                 // columns per wave
  constexpr int kRP = kVThreads / 8;               // rows per load pass
  constexpr int kAP = kVM / kRP, kBP = kVN / kRP;  // load passes per operand
  constexpr int kStage = (kVM + kVN) * kRowBytes;  // one k-slice of both operands
  constexpr int kORow = kVN * 2;                   // bytes per staged output row
  constexpr int kOC = kVN / 8;                     // 16-byte chunks per output row
  constexpr int kORP = kVThreads / kOC;            // rows per read-out pass
  constexpr int kRound = kStage / kORow;           // output rows per round
  static_assert(kVM % kRound == 0 && kRound % 64 == 0, "rounds hold whole waves' rows");
  static_assert(kRound % kORP == 0 && kOC == 32, "read-out rows; 32 chunks per staged row");
  __shared__ __attribute__((aligned(16))) char st0[kStage];
  __shared__ __attribute__((aligned(16))) char st1[kStage];

  // ---- this workgroup's tiles: first, first + nslot, ... below end
  const int total = p.n_groups * p.MT * p.NT;
  const int nslot = gridDim.x / kNumXcdB;
  const int xcd = blockIdx.x % kNumXcdB;
  const int per_xcd = (total + kNumXcdB - 1) / kNumXcdB;
  const int first = xcd * per_xcd + static_cast<int>(blockIdx.x) / kNumXcdB;
  const int end = min(total, (xcd + 1) * per_xcd);
  if (first >= end) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int wm = wave / kWNw, wn = wave % kWNw;
  const int lc = tid & 7, lr = tid >> 3;

  // tile w: group, first row and column, slices
  auto tile = [&](int w, int& g, int& m0, int& n0, int& nk, int& kbeg, int& mpad) {
    w = __builtin_amdgcn_readfirstlane(w);
    g = w / (p.MT * p.NT);
    const int rem = w - g * (p.MT * p.NT);
    m0 = (rem / p.NT) * kVM;
    n0 = (rem % p.NT) * kVN;
    kbeg = kpad[g];
    mpad = kpad[g + 1] - kbeg;
    nk = max(mpad / kBK, 1);
  };

  // ---- load side: the slice after next in the stream
  int l_w = first, l_j = 0, l_nk, l_g, l_m0, l_n0;
  __amdgpu_buffer_rsrc_t rsA, rsB;
  uint32_t a_off[kAP], b_off[kBP];
  auto set_load_tile = [&]() {
    int kbeg, mpad;
    tile(l_w, l_g, l_m0, l_n0, l_nk, kbeg, mpad);
    rsA = rsrc(p.A + static_cast<size_t>(kbeg) * p.M, static_cast<uint32_t>(p.M) * mpad * 2u);
    rsB = rsrc(p.B + static_cast<size_t>(kbeg) * p.N, static_cast<uint32_t>(p.N) * mpad * 2u);
#pragma unroll
    for (int i = 0; i < kAP; ++i) {
      const int m = l_m0 + lr + kRP * i;
      a_off[i] = m < p.M ? (static_cast<uint32_t>(m) * mpad + lc * 8) * 2u : kOff;
    }
#pragma unroll
    for (int i = 0; i < kBP; ++i) {
      const int n = l_n0 + lr + kRP * i;
      b_off[i] = n < p.N ? (static_cast<uint32_t>(n) * mpad + lc * 8) * 2u : kOff;
    }
  };
  set_load_tile();
  // loads the load side's slice into (SA, SB) and moves it on
#define MOE_VLOAD(SA, SB)                                                                    \
  do {                                                                                      \
    const uint32_t kb_ = static_cast<uint32_t>(l_j) * kBK * 2u;                             \
    _Pragma("unroll") for (int i = 0; i < kAP; ++i) SA[i] = __builtin_bit_cast(             \
        uint4, __builtin_amdgcn_raw_buffer_load_b128(rsA, a_off[i], kb_, 0));               \
    _Pragma("unroll") for (int i = 0; i < kBP; ++i) SB[i] = __builtin_bit_cast(             \
        uint4, __builtin_amdgcn_raw_buffer_load_b128(rsB, b_off[i], kb_, 0));               \
    if (l_j + 1 < l_nk) {                                                                   \
      ++l_j;                                                                                \
    } else if (l_w + nslot < end) {                                                         \
      l_w += nslot;                                                                         \
      l_j = 0;                                                                              \
      set_load_tile();                                                                      \
    }                                                                                       \
  } while (0)
#define MOE_VSTORE(SA, SB, ST)                                                               \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < kAP; ++i)                                         \
        *reinterpret_cast<uint4*>((ST) + swz(lr + kRP * i, lc)) = SA[i];                    \
    _Pragma("unroll") for (int i = 0; i < kBP; ++i)                                         \
        *reinterpret_cast<uint4*>((ST) + kVM * kRowBytes + swz(lr + kRP * i, lc)) = SB[i];  \
  } while (0)

  // ---- compute side
  int c_w = first, c_j = 0, c_nk, c_g, c_m0, c_n0;
  {
    int kbeg, mpad;
    tile(c_w, c_g, c_m0, c_n0, c_nk, kbeg, mpad);
  }
  f32x16_t acc[2][kNB];
  auto zero = [&]() {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.0f;
  };
  zero();
  const int fr = lane & 31, fh = lane >> 5;
  auto compute = [&](const char* st) {
    const bool busy = c_m0 + wm * 64 < p.M;
    if (!busy) return;
    const char* bs = st + kVM * kRowBytes;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int c = kk * 2 + fh;
      bf16x8_t af[2], bq[kNB];
#pragma unroll
      for (int x = 0; x < 2; ++x)
        af[x] = *reinterpret_cast<const bf16x8_t*>(st + swz(wm * 64 + x * 32 + fr, c));
#pragma unroll
      for (int x = 0; x < kNB; ++x)
        bq[x] = *reinterpret_cast<const bf16x8_t*>(bs + swz(wn * kWNC + x * 32 + fr, c));
      // B A^T: acc[a][b] holds the block transposed, so a lane's registers
      // run along an output row (see the epilogue)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < kNB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq[b], af[a], acc[a][b], 0, 0, 0);
    }
  };

  // Output tile through the free stage ot, in rounds of kRound rows: round r
  // holds the rows of the waves with wm * 64 in it, staged as bf16 rows of
  // 256 columns and written as whole 16-byte row chunks by buffer stores (an
  // out-of-range offset drops one, so every lane issues the same stores).
  // The blocks were multiplied as B A^T, so output [row][col] of a 32x32
  // block is in lane row + 32*((col/4)%2), register (col%4) + 4*(col/8): a
  // lane holds four consecutive columns per register quad and stages them
  // with one 8-byte write.  The 16-byte chunk index of a staged row is XORed
  // with row % 32, so the 32 rows of one write instruction fall on distinct
  // chunks.
  auto epilogue = [&](char* ot) {
    // lane constants rederived from the hardware lane id (an opaque zero keeps
    // them from being hoisted and held through the slice loop)
    int ez = 0;
    asm volatile("" : "+v"(ez));
    const int e_lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, ez));
    const int e_tid = wave * kWave + e_lane;
    const int e_fr = e_lane & 31, e_fh = e_lane >> 5;
    const __amdgpu_buffer_rsrc_t rsC = rsrc(p.C + static_cast<size_t>(c_g) * p.c_stride,
                                            static_cast<uint32_t>(p.M) * p.ldc * 2u);
    const int rl = e_tid / kOC, cl = e_tid % kOC;
#pragma unroll
    for (int r = 0; r < kVM / kRound; ++r) {
      if (wm * 64 >= r * kRound && wm * 64 < (r + 1) * kRound) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int row = wm * 64 - r * kRound + a * 32 + e_fr;
          char* orow = ot + row * kORow;
#pragma unroll
          for (int b = 0; b < kNB; ++b)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int col = wn * kWNC + b * 32 + 8 * qq + 4 * e_fh;
              const uint2 v = make_uint2(
                  pack_bf16x2(acc[a][b][4 * qq], acc[a][b][4 * qq + 1]),
                  pack_bf16x2(acc[a][b][4 * qq + 2], acc[a][b][4 * qq + 3]));
              *reinterpret_cast<uint2*>(orow + (((col >> 3) ^ (row & 31)) << 4) + (col & 4) * 2) = v;
            }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int it = 0; it < kRound / kORP; ++it) {
        const int row = it * kORP + rl;
        const int m = c_m0 + r * kRound + row;
        const uint32_t off = (m < p.M && c_n0 + cl * 8 < p.N)
                                 ? (static_cast<uint32_t>(m) * p.ldc + c_n0 + cl * 8) * 2u
                                 : kOff;
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4_t, *reinterpret_cast<const uint4*>(
                                            ot + row * kORow + ((cl ^ (row & 31)) << 4))),
            rsC, off, 0, 2 /* streaming: not read again here */);
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };

  // ---- the stream.  Slice s sits in register set s % 2 and LDS stage s % 2.
  // Step j: load slice j + 2 into the set that held slice j (stored to LDS in
  // step j - 1), multiply slice j, store slice j + 1 to the other stage,
  // barrier; after a tile's last slice, write its output through stage j % 2.
  uint4 sa0[kAP], sb0[kBP], sa1[kAP], sb1[kBP];
  MOE_VLOAD(sa0, sb0);
  MOE_VLOAD(sa1, sb1);
  MOE_VSTORE(sa0, sb0, st0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#define MOE_VSTEP(LA, LB, CS, SA, SB, SS)                                                    \
  MOE_VLOAD(LA, LB);                                                                        \
  compute(CS);                                                                              \
  MOE_VSTORE(SA, SB, SS);                                                                   \
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                           \
  if (++c_j >= c_nk) {                                                                      \
    epilogue(CS);                                                                           \
    if (c_w + nslot >= end) break;                                                          \
    c_w += nslot;                                                                           \
    c_j = 0;                                                                                \
    int kbeg_, mpad_;                                                                       \
    tile(c_w, c_g, c_m0, c_n0, c_nk, kbeg_, mpad_);                                         \
    zero();                                                                                 \
  }
  for (;;) {
    MOE_VSTEP(sa0, sb0, st0, sa1, sb1, st1)
    MOE_VSTEP(sa1, sb1, st1, sa0, sb0, st0)
  }
#undef MOE_VSTEP
#undef MOE_VLOAD
#undef MOE_VSTORE
  // the last loads and the output stores complete before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Workgroups of the streamed weight-gradient kernel: one per CU, a multiple of
// the XCD count.
int persistent_grid() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < kNumXcdB)
      cus = 256;
    cached[dev] = cus / kNumXcdB * kNumXcdB;
  }
  return cached[dev];
}

hipError_t kvar_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.n_groups * a.MT * a.NT == 0) return hipSuccess;
  hipLaunchKernelGGL(kvar_stream_kernel, dim3(persistent_grid()), dim3(kVThreads), 0, s, a,
                     a.kpad);
  return hipGetLastError();
}

hipError_t rows_gemm(const GemmArgs& a, unsigned blocks, hipStream_t s) {
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_gemm_kernel, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------- workspace

BwdWorkspace bwd_layout(void* base, int n_groups, int d, int f, int rows) {
  BwdWorkspace w{};
  size_t off = 0;
  auto take = [&](size_t n) {
    size_t at = off;
    off = align_up(off + n, 256);
    return base ? static_cast<char*>(base) + at : nullptr;
  };
  const size_t rpad = static_cast<size_t>(rows) + static_cast<size_t>(kPad) * n_groups;
  w.tiles.tiles = reinterpret_cast<TileInfo*>(
      take(static_cast<size_t>(max_tiles_for(rows, n_groups, kBM)) * sizeof(TileInfo)));
  w.tiles.group_tile_start = reinterpret_cast<int32_t*>(take((n_groups + 1) * sizeof(int32_t)));
  w.tiles.meta = reinterpret_cast<int32_t*>(take(4 * sizeof(int32_t)));
  w.tiles256.tiles = reinterpret_cast<TileInfo*>(
      take(static_cast<size_t>(max_tiles_for(rows, n_groups, 256)) * sizeof(TileInfo)));
  w.tiles256.group_tile_start =
      reinterpret_cast<int32_t*>(take((n_groups + 1) * sizeof(int32_t)));
  w.tiles256.meta = reinterpret_cast<int32_t*>(take(4 * sizeof(int32_t)));
  w.kpad = reinterpret_cast<int32_t*>(take((n_groups + 1) * sizeof(int32_t)));
  w.au = reinterpret_cast<uint16_t*>(take(static_cast<size_t>(rows) * 2 * f * 2));
  w.dadu = reinterpret_cast<uint16_t*>(take(static_cast<size_t>(rows) * 2 * f * 2));
  w.xT = reinterpret_cast<uint16_t*>(take(rpad * d * 2));
  w.dyT = reinterpret_cast<uint16_t*>(take(rpad * d * 2));
  w.actT = reinterpret_cast<uint16_t*>(take(rpad * f * 2));
  w.daT = reinterpret_cast<uint16_t*>(take(rpad * f * 2));
  w.duT = reinterpret_cast<uint16_t*>(take(rpad * f * 2));
  w.bytes = off;
  return w;
}

size_t bwd_workspace_bytes(int n_groups, int d, int f, int rows) {
  return bwd_layout(nullptr, n_groups, d, f, rows).bytes;
}

size_t bwd_rpad_max(int n_groups, int rows) {
  return static_cast<size_t>(rows) + static_cast<size_t>(kPad) * n_groups;
}

hipError_t launch_swiglu_backward(int n_groups, int d, int f, int rows, int x_rows,
                                  const int32_t* offsets, const int32_t* row_index,
                                  const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                                  const uint16_t* wgu_t, const uint16_t* wd_t,
                                  const uint16_t* dy, const uint16_t* au, uint16_t* dx,
                                  uint16_t* dwg, uint16_t* dwu, uint16_t* dwd, void* ws,
                                  hipStream_t s) {
  BwdWorkspace w = bwd_layout(ws, n_groups, d, f, rows);
  // one 256-row tile list serves the activation-gradient products and the
  // transposes; the 128-row list only the a | u recompute
  SwigluWorkspace t256{};
  t256.tiles = w.tiles256.tiles;
  t256.group_tile_start = w.tiles256.group_tile_start;
  t256.meta = w.tiles256.meta;
  hipError_t err = launch_build_tiles(n_groups, rows, 256, offsets, t256, s);
  if (err != hipSuccess) return err;
  const int max_tiles256 = max_tiles_for(rows, n_groups, 256);
  ProfScope prof_(s, "swiglu_backward");
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(1024), 0, s, n_groups, rows, offsets,
                     w.kpad);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  // 1. a = x W_gate^T, u = x W_up^T  -> au [rows, 2f], unless the forward
  //    pass stored them
  if (au == nullptr) {
    SwigluWorkspace tl{};
    tl.tiles = w.tiles.tiles;
    tl.group_tile_start = w.tiles.group_tile_start;
    tl.meta = w.tiles.meta;
    if ((err = launch_build_tiles(n_groups, rows, kBM, offsets, tl, s)) != hipSuccess) return err;
    const int max_tiles = max_tiles_for(rows, n_groups, kBM);
    GemmArgs a{};
    a.tiles = tl.tiles;
    a.meta = tl.meta;
    a.n_groups = n_groups;
    a.row_index = row_index;
    a.a_rows = x_rows;
    a.N = f; a.K = d; a.NT = (f + kBN - 1) / kBN;
    a.A = x; a.lda = d;
    a.ldb = d; a.b_stride = static_cast<size_t>(f) * d;
    a.ldc = 2 * f;
    a.B = wg; a.C = w.au;
    if ((err = rows_gemm(a, max_tiles * a.NT, s)) != hipSuccess) return err;
    a.B = wu; a.C = w.au + f;
    if ((err = rows_gemm(a, max_tiles * a.NT, s)) != hipSuccess) return err;
    au = w.au;
  }
  // The activation-gradient products of steps 2 and 3 run over the 256-row
  // tiles, or, for groups of at most 128 rows on average, over tiles for the
  // kernel that sends both operands by LDS DMA, built into the 128-row list's
  // arrays (sized for more tiles; step 1 is done with them by then).
  const int nt_rows = grouped_nt_tile_rows(n_groups, rows, d, f, 2 * f, d);
  SwigluWorkspace tnt = t256;
  if (nt_rows != 256) {
    tnt.tiles = w.tiles.tiles;
    tnt.group_tile_start = w.tiles.group_tile_start;
    tnt.meta = w.tiles.meta;
    if ((err = launch_build_tiles(n_groups, rows, nt_rows, offsets, tnt, s)) != hipSuccess)
      return err;
  }
  // 2. d act = dy W_down (B = W_down^T [f, d]) -> [rows, f], held in the daT
  //    region (rpad >= rows; daT is written only in step 4), with the forward
  //    pass's down-direction kernels; then da, du -> dadu
  uint16_t* dact = w.daT;
  if ((err = launch_grouped_nt_bf16(n_groups, d, f, rows, offsets, tnt, dy, wd_t, dact,
                                    "bwd_dact_bf16", s, /*tiles_built=*/true, nt_rows)) !=
      hipSuccess)
    return err;
  {
    const long n8 = static_cast<long>(rows) * (f / 8);
    const unsigned blocks = static_cast<unsigned>(std::min<long>((n8 + 255) / 256, 65536));
    if (blocks > 0)
      hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(blocks), dim3(256), 0, s, rows, f, dact, au,
                         w.dadu);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // 3. dx = [da | du] [W_gate^T | W_up^T]^T  (K = 2f, B = [d, 2f]) -> dx [rows, d]
  if ((err = launch_grouped_nt_bf16(n_groups, 2 * f, d, rows, offsets, tnt, w.dadu, wgu_t, dx,
                                    "bwd_dx_bf16", s, /*tiles_built=*/true, nt_rows)) !=
      hipSuccess)
    return err;
  // 4. per-expert transposed activations (rows padded to 64 per expert)
  {
    ProfScope pt_(s, "bwd_transpose");
    dim3 gd(max_tiles256, (d + 63) / 64), gf(max_tiles256, (f + 63) / 64);
    hipLaunchKernelGGL(pad_transpose_kernel<kTrCopy>, gd, dim3(256), 0, s, d, rows, x_rows,
                       t256.tiles, t256.meta, w.kpad, row_index, x, d, w.xT);
    hipLaunchKernelGGL(pad_transpose_kernel<kTrCopy>, gd, dim3(256), 0, s, d, rows, rows,
                       t256.tiles, t256.meta, w.kpad, nullptr, dy, d, w.dyT);
    hipLaunchKernelGGL(pad_transpose_kernel<kTrAct>, gf, dim3(256), 0, s, f, rows, rows,
                       t256.tiles, t256.meta, w.kpad, nullptr, au, 2 * f, w.actT);
    hipLaunchKernelGGL(pad_transpose_kernel<kTrCopy>, gf, dim3(256), 0, s, f, rows, rows,
                       t256.tiles, t256.meta, w.kpad, nullptr, w.dadu, 2 * f, w.daT);
    hipLaunchKernelGGL(pad_transpose_kernel<kTrCopy>, gf, dim3(256), 0, s, f, rows, rows,
                       t256.tiles, t256.meta, w.kpad, nullptr, w.dadu + f, 2 * f, w.duT);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // 5. weight gradients, K = the expert's (padded) rows
  GemmArgs k{};
  k.n_groups = n_groups;
  k.kpad = w.kpad;
  //    dW_gate [f, d] = da^T x ; dW_up = du^T x
  k.M = f; k.N = d; k.MT = (f + kVM - 1) / kVM; k.NT = (d + kVN - 1) / kVN;
  k.B = w.xT; k.ldc = d; k.c_stride = static_cast<size_t>(f) * d;
  k.A = w.daT; k.C = dwg;
  if ((err = kvar_gemm(k, s)) != hipSuccess) return err;
  k.A = w.duT; k.C = dwu;
  if ((err = kvar_gemm(k, s)) != hipSuccess) return err;
  //    dW_down [d, f] = dy^T act
  k.M = d; k.N = f; k.MT = (d + kVM - 1) / kVM; k.NT = (f + kVN - 1) / kVN;
  k.A = w.dyT; k.B = w.actT; k.C = dwd; k.ldc = f; k.c_stride = static_cast<size_t>(d) * f;
  return kvar_gemm(k, s);
}

hipError_t launch_combine_backward(int T, int d, int K, const uint16_t* dy, const uint16_t* yp,
                                   const int32_t* slot_row, const float* gates, uint16_t* dyp,
                                   float* dg, hipStream_t s) {
  ProfScope prof_(s, "combine_backward");
  hipLaunchKernelGGL(combine_bwd_kernel, dim3((T + 3) / 4), dim3(256), 0, s, T, d, K, T * K, dy,
                     yp, slot_row, gates, dyp, dg);
  return hipGetLastError();
}

hipError_t launch_route_backward(int T, int d, int E, int K, int fn, const uint16_t* h,
                                 const float* e, const int32_t* idx, const float* dg,
                                 const int32_t* offsets, const int32_t* row_token, float* dz,
                                 uint16_t* dh, float* de, hipStream_t s) {
  ProfScope prof_(s, "route_backward");
  hipLaunchKernelGGL(route_bwd_token_kernel, dim3((T + 3) / 4), dim3(256), 0, s, T, d, E, K, fn,
                     h, e, idx, dg, dz, dh);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_bwd_de_kernel, dim3(E), dim3(256), 0, s, T, d, E, K, h, idx, dz,
                     offsets, row_token, de);
  return hipGetLastError();
}

hipError_t launch_transpose_experts(int n, int rows, int cols, const uint16_t* src,
                                    uint16_t* dst, int ld, int col_off, hipStream_t s) {
  dim3 grid((cols + 63) / 64, (rows + 63) / 64, n);
  hipLaunchKernelGGL(transpose_experts_kernel, grid, dim3(256), 0, s, rows, cols, src, dst, ld,
                     col_off);
  return hipGetLastError();
}

}  // namespace moe
