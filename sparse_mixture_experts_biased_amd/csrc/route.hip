// Router: z = h . e (fp32 accuracy), score function, biased top-K, unbiased
// gates and the load histogram.
//
// Method: Sparse MoE routing-math page (arman1o1.github.io), section 2
// (I_t = TopK(s + b, K), g = s / sum_{I_t} s, sigmoid affinity) and the
// classical-router listing of section 1 (softmax, top-K, renormalise, clamp
// 1e-12); section 4 item 2 keeps the router in fp32.
//
// bf16 tokens (the large workloads): the logits run on the matrix cores.  The
// fp32 centroids are split exactly into three bf16 parts, e = e_hi + e_mid +
// e_lo (truncate, truncate, remainder: 8 + 8 + 8 significant bits), so every
// product h * e_part is exact in fp32 and the MFMA accumulates in fp32 --
// fp32 accuracy at bf16 matrix-core rate (the bf16x3 split of Henry, Tang and
// Heinecke, "Leveraging the bfloat16 Artificial Intelligence Datatype For
// Higher-Precision Computations", 2019).  The d_model loop is split S ways
// across workgroups into fixed partial sums; the top-K kernel adds them in a
// fixed order, so z is deterministic.
// fp32 tokens (the tiny workload): one fused kernel with fp32 FMA.
//
// Selection (both paths): one wave per token, E/64 experts per lane, K rounds
// of a wave-wide arg-max over v = s + b (equal v -> lower expert id), a sort of
// the K picks by expert id, and the gate denominator summed in that order, so
// the gates depend only on the picked set.
//
// Diagnostics (optional, same page, section 1: Switch P_i and the router
// z-loss): the selection wave also writes the token's softmax row p_t and
// logsumexp(z_t)^2; two reduction kernels average them over the tokens in a
// fixed order (deterministic).
#include "common.h"

#include <math.h>

namespace moe {
namespace {

constexpr int kSent = 0x7fffffff;  // "no expert"

// Arg-max over the wave: larger v wins, equal v -> smaller expert id; a real
// expert id always beats the sentinel.
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    float ov = __shfl_xor(v, m, kWave);
    int oid = __shfl_xor(id, m, kWave);
    if (oid != kSent && (id == kSent || ov > v || (ov == v && oid < id))) {
      v = ov;
      id = oid;
    }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Scores, biased top-K, gates and load counts of token t; z[j] is the logit of
// expert lane + 64 j (ignored for experts >= E).  Called by a whole wave.
template <int EJ>
__device__ __forceinline__ void select_token(int t, int E, int K, int fn, const float (&z)[EJ],
                                             const float (&bias)[EJ], int32_t* __restrict__ idx_out,
                                             float* __restrict__ gate_out,
                                             int32_t* __restrict__ loads, int lstride,
                                             float* __restrict__ prow,
                                             float* __restrict__ lsq) {
  const int lane = threadIdx.x % kWave;
  if (prow != nullptr) {  // diagnostics: softmax row and logsumexp^2 of token t
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < EJ; ++j)
      if (lane + kWave * j < E) m = fmaxf(m, z[j]);
    m = wave_max(m);
    float ez[EJ], part = 0.0f;
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
      ez[j] = (lane + kWave * j < E) ? expf(z[j] - m) : 0.0f;
      part += ez[j];
    }
    const float tot = wave_sum(part);
#pragma unroll
    for (int j = 0; j < EJ; ++j)
      if (lane + kWave * j < E) prow[static_cast<size_t>(t) * E + lane + kWave * j] = ez[j] / tot;
    if (lane == 0) {
      const float lse = m + logf(tot);
      lsq[t] = lse * lse;
    }
  }
  float s[EJ], v[EJ];
  if (fn == 0) {
#pragma unroll
    for (int j = 0; j < EJ; ++j) s[j] = 1.0f / (1.0f + expf(-z[j]));
  } else {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < EJ; ++j)
      if (lane + kWave * j < E) m = fmaxf(m, z[j]);
    m = wave_max(m);
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
      s[j] = (lane + kWave * j < E) ? expf(z[j] - m) : 0.0f;
      part += s[j];
    }
    const float tot = wave_sum(part);
#pragma unroll
    for (int j = 0; j < EJ; ++j) s[j] = s[j] / tot;
  }
#pragma unroll
  for (int j = 0; j < EJ; ++j) v[j] = s[j] + bias[j];

  // K rounds of arg-max; sel / sv hold the picks (wave-uniform).
  int sel[MOE_MAX_TOPK_DEV];
  float sv[MOE_MAX_TOPK_DEV];
  unsigned taken = 0u;
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) {
    sel[k] = kSent;
    sv[k] = 0.0f;
    if (k < K) {
      float bv = -INFINITY;
      int be = kSent;
#pragma unroll
      for (int j = 0; j < EJ; ++j) {
        const int ex = lane + kWave * j;
        const bool ok = ex < E && !((taken >> j) & 1u);
        // the first free candidate is always taken, so a NaN score cannot
        // leave the pick without an expert id
        if (ok && (be == kSent || v[j] > bv || (v[j] == bv && ex < be))) {
          bv = v[j];
          be = ex;
        }
      }
      wave_argmax(bv, be);
      if (be < 0 || be >= E) be = 0;  // only reachable with non-finite scores
      const int jw = be / kWave;      // wave-uniform
      float sj = 0.0f;
#pragma unroll
      for (int j = 0; j < EJ; ++j)
        if (j == jw) sj = s[j];
      sj = __shfl(sj, be % kWave, kWave);
      if (lane == be % kWave) taken |= 1u << jw;
      sel[k] = be;
      sv[k] = sj;
    }
  }
  // ascending expert id: lane k < K takes pick k and counts the picks that
  // order before it (a tie, reachable only with non-finite scores, goes by
  // pick order), then one lane permute puts pick k on the lane of its rank
  int my_id = 0;
  float my_s = 0.0f;
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
    if (k == lane) {
      my_id = sel[k];
      my_s = sv[k];
    }
  int rank = lane;  // lanes >= K keep their place
  if (lane < K) {
    rank = 0;
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
      if (k < K) rank += (sel[k] < my_id || (sel[k] == my_id && k < lane)) ? 1 : 0;
  }
  my_id = __builtin_amdgcn_ds_permute(rank * 4, my_id);
  my_s = __int_as_float(__builtin_amdgcn_ds_permute(rank * 4, __float_as_int(my_s)));
  // the gate denominator in ascending id order
  float den = 0.0f;
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
    if (k < K) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
  den = fmaxf(den, 1e-12f);
  if (lane < K) {
    idx_out[static_cast<size_t>(t) * K + lane] = my_id;
    gate_out[static_cast<size_t>(t) * K + lane] = my_s / den;
    if (my_id >= 0 && my_id < E) atomicAdd(&loads[my_id * lstride], 1);
  }
}

// ------------------------------------------------------------ fp32 tokens: fused

constexpr int kBT = 16;       // tokens per workgroup
constexpr int kBK = 32;       // d_model slice per LDS stage
constexpr int kThreads = 256;
constexpr int kTokPerWave = kBT / 4;

template <int EJ>
__global__ __launch_bounds__(kThreads) void route_f32_kernel(
    int T, int d, int E, int K, int fn, const float* __restrict__ h, const float* __restrict__ e,
    const float* __restrict__ b, int32_t* __restrict__ idx_out, float* __restrict__ gate_out,
    int32_t* __restrict__ loads, float* __restrict__ prow, float* __restrict__ lsq) {
  extern __shared__ float smem[];
  float* hs = smem;                       // [kBT][kBK]
  float* es = smem + kBT * kBK;           // [E][kBK + 1]
  float* zs = es;                         // reused after the d loop: [kBT][E]

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int t0 = blockIdx.x * kBT;

  float acc[kTokPerWave][EJ];
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i)
#pragma unroll
    for (int j = 0; j < EJ; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < d; k0 += kBK) {
    for (int q = tid; q < kBT * kBK; q += kThreads) {
      int r = q / kBK, c = q % kBK;
      int t = t0 + r, k = k0 + c;
      hs[q] = (t < T && k < d) ? h[static_cast<size_t>(t) * d + k] : 0.0f;
    }
    for (int q = tid; q < E * kBK; q += kThreads) {
      int r = q / kBK, c = q % kBK;
      int k = k0 + c;
      es[r * (kBK + 1) + c] = (k < d) ? e[static_cast<size_t>(r) * d + k] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < kBK; ++c) {
      float hv[kTokPerWave];
#pragma unroll
      for (int i = 0; i < kTokPerWave; ++i) hv[i] = hs[(wave * kTokPerWave + i) * kBK + c];
#pragma unroll
      for (int j = 0; j < EJ; ++j) {
        int ex = lane + kWave * j;
        float ev = (ex < E) ? es[ex * (kBK + 1) + c] : 0.0f;
#pragma unroll
        for (int i = 0; i < kTokPerWave; ++i) acc[i][j] = fmaf(hv[i], ev, acc[i][j]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i)
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
      int ex = lane + kWave * j;
      if (ex < E) zs[(wave * kTokPerWave + i) * E + ex] = acc[i][j];
    }
  __syncthreads();

  float bias[EJ];
#pragma unroll
  for (int j = 0; j < EJ; ++j) {
    int ex = lane + kWave * j;
    bias[j] = (b != nullptr && ex < E) ? b[ex] : 0.0f;
  }
  for (int i = 0; i < kTokPerWave; ++i) {
    const int r = wave * kTokPerWave + i;
    const int t = t0 + r;
    if (t >= T) break;  // wave-uniform
    float z[EJ];
#pragma unroll
    for (int j = 0; j < EJ; ++j) {
      int ex = lane + kWave * j;
      z[j] = (ex < E) ? zs[r * E + ex] : 0.0f;
    }
    select_token<EJ>(t, E, K, fn, z, bias, idx_out, gate_out, loads, 1, prow, lsq);
  }
}

// ------------------------------------------------------------ bf16 tokens: MFMA

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kZT = 128;   // tokens per workgroup tile
constexpr int kZE = 128;   // experts per workgroup tile
// The T*K load increments of the split path go to counters 256 bytes apart
// (then compacted into loads): packed into one 1 KB block, the same-line
// atomics queue on one or two L2 channels.
constexpr int kLoadStride = 64;

__device__ __forceinline__ uint32_t pack2(uint32_t lo_bits, uint32_t hi_bits) {
  return (lo_bits >> 16) | (hi_bits & 0xffff0000u);
}

// Exact three-way bf16 split of 8 fp32 values: x = hi + mid + lo.
__device__ __forceinline__ void split3(const float4& p, const float4& q, bf16x8_t& hi,
                                       bf16x8_t& mid, bf16x8_t& lo) {
  const float x[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
  uint32_t h[8], m[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t xb = __float_as_uint(x[i]);
    h[i] = xb & 0xffff0000u;                                  // truncate: top 8 bits
    const float r1 = x[i] - __uint_as_float(h[i]);            // exact
    m[i] = __float_as_uint(r1) & 0xffff0000u;                 // next 8 bits
    const float r2 = r1 - __uint_as_float(m[i]);              // exact, <= 8 bits left
    l[i] = __float_as_uint(r2);                               // exact in bf16
  }
  uint4 hv, mv, lv;
  hv.x = pack2(h[0], h[1]); hv.y = pack2(h[2], h[3]); hv.z = pack2(h[4], h[5]); hv.w = pack2(h[6], h[7]);
  mv.x = pack2(m[0], m[1]); mv.y = pack2(m[2], m[3]); mv.z = pack2(m[4], m[5]); mv.w = pack2(m[6], m[7]);
  lv.x = pack2(l[0], l[1]); lv.y = pack2(l[2], l[3]); lv.z = pack2(l[4], l[5]); lv.w = pack2(l[6], l[7]);
  hi = __builtin_bit_cast(bf16x8_t, hv);
  mid = __builtin_bit_cast(bf16x8_t, mv);
  lo = __builtin_bit_cast(bf16x8_t, lv);
}

// zpart[s][t][i] = sum over k in split s of h[t][k] * e[i][k].
// Workgroup: 128 tokens x 128 experts, eight waves in 2 x 4, each 64 x 32 as
// two blocks of 32 x 32; two waves per SIMD, so one wave's centroid split
// (vector ALU) runs while the other's products occupy the matrix core.  k in
// 64-wide slices staged through LDS with coalesced 16-byte loads (h: eight
// lanes per 128-byte row of a slice; e in fp32: sixteen lanes per 256-byte
// row), double-buffered: the next slice's loads are in flight in registers
// while the current one is multiplied.  (Fragment loads straight from global
// memory touch one cache line per row for every 16 bytes they bring, and that
// request rate bounded the kernel.)  The 16-byte chunks of a row are
// XOR-swizzled so fragment reads (32 rows, one chunk) and staging writes are
// bank-conflict free; each centroid fragment (8 fp32) is split exactly into
// its three bf16 parts after the read.
constexpr int kZK = 64;       // k per slice
constexpr int kZThreads = 512;
__device__ __forceinline__ int zswz_h(int r, int c) {  // 128-byte rows, 8 chunks
  return r * 128 + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4);
}
__device__ __forceinline__ int zswz_e(int r, int c) {  // 256-byte rows, 16 chunks
  return r * 256 + ((c ^ (r & 15)) << 4);
}

__global__ __launch_bounds__(kZThreads) void route_logits_mfma_kernel(int T, int d, int E, int klen,
                                                                const uint16_t* __restrict__ h,
                                                                const float* __restrict__ e,
                                                                float* __restrict__ zpart,
                                                                int32_t* __restrict__ lpad) {
  constexpr int kHB = kZT * kZK * 2, kEB = kZE * kZK * 4, kStage = kHB + kEB;
  __shared__ __attribute__((aligned(16))) char lds[2 * kStage];
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int fr = lane & 31, fh = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;
  const int t0 = blockIdx.x * kZT, x0 = blockIdx.y * kZE;
  const int split = blockIdx.z;
  const size_t k_begin = static_cast<size_t>(split) * klen;
  // the first workgroup clears the padded load counters the selection counts into
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = tid; i < E; i += kZThreads) lpad[static_cast<size_t>(i) * kLoadStride] = 0;

  // Buffer descriptors based at the tile's first row: a row past T (or E)
  // is past the descriptor's range and reads zeros, without a branch.  k past
  // klen (the upper half of a last 32-wide slice) reads the next split's
  // values, or zeros, and is replaced by zeros on the way into LDS.
  const int h_rows = min(kZT, T - t0), e_rows = min(kZE, E - x0);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(h + static_cast<size_t>(t0) * d + k_begin), 0,
      h_rows * d * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(e + static_cast<size_t>(x0) * d + k_begin), 0, e_rows * d * 4,
      0x00020000);
  // staging slots: h rows hr + 64 p (chunk hc), e rows er + 32 p (chunk ec)
  const int hr = tid >> 3, hc = tid & 7;
  const int er = tid >> 4, ec = tid & 15;
  uint4 hv[2], ev[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
      hv[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rh, ((hr + 64 * p) * d + k0 + hc * 8) * 2, 0, 0));
#pragma unroll
    for (int p = 0; p < 4; ++p)
      ev[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            re, ((er + 32 * p) * d + k0 + ec * 4) * 4, 0, 0));
  };
  auto masked = [](const uint4& v, uint32_t m) {
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
  };
  auto store = [&](char* st, int k0) {
    const uint32_t hm = k0 + hc * 8 < klen ? ~0u : 0u, em = k0 + ec * 4 < klen ? ~0u : 0u;
#pragma unroll
    for (int p = 0; p < 2; ++p)
      *reinterpret_cast<uint4*>(st + zswz_h(hr + 64 * p, hc)) = masked(hv[p], hm);
#pragma unroll
    for (int p = 0; p < 4; ++p)
      *reinterpret_cast<uint4*>(st + kHB + zswz_e(er + 32 * p, ec)) = masked(ev[p], em);
  };

  f32x16_t acc[2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[a][q] = 0.0f;

  // klen is a multiple of 32.  Slice j + 1 is
  // written to the other stage while slice j is multiplied: that stage was
  // last read in step j - 1, which every wave finished before the barrier
  // that ended it.
  const int n_slices = (klen + kZK - 1) / kZK;
  load(0);
  store(lds, 0);
  __syncthreads();
  for (int j = 0; j < n_slices; ++j) {
    const char* hs = lds + (j & 1) * kStage;
    const char* es = hs + kHB;
    const bool more = j + 1 < n_slices;
    if (more) load((j + 1) * kZK);
    // 16-k step st: A = tokens wm*64 + a*32 + fr (chunk 2st + fh), B =
    // experts wn*32 + fr (fp32 chunks 4st + 2fh, 4st + 2fh + 1)
#pragma unroll
    for (int st = 0; st < kZK / 16; ++st) {
      bf16x8_t af[2], bh, bm, bl;
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = *reinterpret_cast<const bf16x8_t*>(
            hs + zswz_h(wm * 64 + a * 32 + fr, 2 * st + fh));
      const int r = wn * 32 + fr;
      const float4 p0 = *reinterpret_cast<const float4*>(es + zswz_e(r, 4 * st + 2 * fh));
      const float4 p1 = *reinterpret_cast<const float4*>(es + zswz_e(r, 4 * st + 2 * fh + 1));
      split3(p0, p1, bh, bm, bl);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bl, acc[a], 0, 0, 0);
        acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bm, acc[a], 0, 0, 0);
        acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bh, acc[a], 0, 0, 0);
      }
    }
    if (more) store(lds + ((j + 1) & 1) * kStage, (j + 1) * kZK);
    __syncthreads();
  }
  // D[row = token][col = expert]: lane (col + 32*((row/4)%2)), register (row%4) + 4*(row/8)
  float* zs = zpart + static_cast<size_t>(split) * T * E;
  const int ex = x0 + wn * 32 + fr;
  if (ex < E) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int t = t0 + wm * 64 + a * 32 + 8 * (q >> 2) + 4 * fh + (q & 3);
        if (t < T) zs[static_cast<size_t>(t) * E + ex] = acc[a][q];
      }
  }
}

// One wave per token: z = sum_s zpart[s] (fixed order), then selection.
template <int EJ>
__global__ __launch_bounds__(256) void route_topk_kernel(int T, int E, int K, int fn, int S,
                                                         const float* __restrict__ zpart,
                                                         const float* __restrict__ b,
                                                         int32_t* __restrict__ idx_out,
                                                         float* __restrict__ gate_out,
                                                         int32_t* __restrict__ loads,
                                                         float* __restrict__ prow,
                                                         float* __restrict__ lsq) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (t >= T) return;  // wave-uniform
  float z[EJ], bias[EJ];
#pragma unroll
  for (int j = 0; j < EJ; ++j) {
    const int ex = lane + kWave * j;
    z[j] = 0.0f;
    bias[j] = (b != nullptr && ex < E) ? b[ex] : 0.0f;
  }
  // partials of four splits in flight at once, added in split order
  for (int s0 = 0; s0 < S; s0 += 4) {
    float v[4][EJ];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < EJ; ++j) {
        const int ex = lane + kWave * j;
        v[u][j] = (s0 + u < S && ex < E)
                      ? zpart[(static_cast<size_t>(s0 + u) * T + t) * E + ex]
                      : 0.0f;
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < EJ; ++j)
        if (s0 + u < S) z[j] += v[u][j];
  }
  select_token<EJ>(t, E, K, fn, z, bias, idx_out, gate_out, loads, kLoadStride, prow, lsq);
}

// loads[e] = the strided counter of expert e.
__global__ __launch_bounds__(256) void compact_loads_kernel(int E, const int32_t* __restrict__ lpad,
                                                            int32_t* __restrict__ loads) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < E) loads[e] = lpad[static_cast<size_t>(e) * kLoadStride];
}

// Zeroes the strided counters.
// ------------------------------------------------------------ diagnostics

constexpr int kStatChunk = 64;  // tokens per partial sum

// part[c][e] = sum of p_te over tokens of chunk c (e < E); part[c][E] = sum of
// logsumexp^2 over the chunk.  Grid (ceil((E + 1) / 256), chunks).
__global__ __launch_bounds__(256) void stats_partial_kernel(int T, int E,
                                                            const float* __restrict__ prow,
                                                            const float* __restrict__ lsq,
                                                            float* __restrict__ part) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int t0 = blockIdx.y * kStatChunk;
  const int t1 = min(T, t0 + kStatChunk);
  if (e > E) return;
  float acc = 0.0f;
  if (e < E)
    for (int t = t0; t < t1; ++t) acc += prow[static_cast<size_t>(t) * E + e];
  else
    for (int t = t0; t < t1; ++t) acc += lsq[t];
  part[static_cast<size_t>(blockIdx.y) * (E + 1) + e] = acc;
}

// p_mean[e] = (1/T) sum_c part[c][e]; zsq_mean = (1/T) sum_c part[c][E].
__global__ __launch_bounds__(1024) void stats_final_kernel(int T, int E, int n_chunks,
                                                           const float* __restrict__ part,
                                                           float* __restrict__ p_mean,
                                                           float* __restrict__ zsq_mean) {
  for (int e = threadIdx.x; e <= E; e += 1024) {
    float acc = 0.0f;
    for (int c = 0; c < n_chunks; ++c) acc += part[static_cast<size_t>(c) * (E + 1) + e];
    const float v = acc / static_cast<float>(T);
    if (e < E) p_mean[e] = v; else *zsq_mean = v;
  }
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, size_t n) {
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------ launch helpers

template <int EJ>
const void* f32_kernel_ptr() { return reinterpret_cast<const void*>(route_f32_kernel<EJ>); }

hipError_t launch_route_f32(int T, int d, int E, int K, int fn, const float* h, const float* e,
                            const float* b, int32_t* idx, float* gates, int32_t* loads,
                            float* prow, float* lsq, hipStream_t s) {
  dim3 grid((T + kBT - 1) / kBT), block(kThreads);
  const size_t es_floats = static_cast<size_t>(E) * (kBK + 1);
  const size_t zs_floats = static_cast<size_t>(kBT) * E;
  const size_t shmem = (kBT * kBK + (es_floats > zs_floats ? es_floats : zs_floats)) * sizeof(float);
  const int ej = (E + kWave - 1) / kWave;
  if (shmem > 64 * 1024) {
    const void* f = ej <= 1 ? f32_kernel_ptr<1>() : ej <= 2 ? f32_kernel_ptr<2>()
                  : ej <= 4 ? f32_kernel_ptr<4>() : f32_kernel_ptr<8>();
    hipError_t err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (err != hipSuccess) return err;
  }
  ProfScope prof_(s, "route_f32");
  if (ej <= 1)
    hipLaunchKernelGGL(route_f32_kernel<1>, grid, block, shmem, s, T, d, E, K, fn, h, e, b, idx, gates, loads, prow, lsq);
  else if (ej <= 2)
    hipLaunchKernelGGL(route_f32_kernel<2>, grid, block, shmem, s, T, d, E, K, fn, h, e, b, idx, gates, loads, prow, lsq);
  else if (ej <= 4)
    hipLaunchKernelGGL(route_f32_kernel<4>, grid, block, shmem, s, T, d, E, K, fn, h, e, b, idx, gates, loads, prow, lsq);
  else
    hipLaunchKernelGGL(route_f32_kernel<8>, grid, block, shmem, s, T, d, E, K, fn, h, e, b, idx, gates, loads, prow, lsq);
  return hipGetLastError();
}

}  // namespace

// Number of d_model splits of the matrix-core logits (0: that path is not used).
int route_splits(int T, int d, int E, int h_bf16) {
  if (!h_bf16 || d % 32 != 0) return 0;
  const int tiles = ((T + kZT - 1) / kZT) * ((E + kZE - 1) / kZE);
  int S = 1;
  while (tiles * S < 256 && S < 16 && d % (32 * 2 * S) == 0) S *= 2;
  return S;
}

// Split-K logit partials [S][T][E], then one load counter per 256 bytes
// (none without splits: the fp32 path counts into loads directly).
size_t route_workspace_bytes(int T, int d, int E, int h_bf16) {
  const int S = route_splits(T, d, E, h_bf16);
  if (S == 0) return 0;
  return align_up(static_cast<size_t>(S) * T * E * sizeof(float), 256) +
         align_up(static_cast<size_t>(E) * kLoadStride * sizeof(int32_t), 256);
}

// Diagnostics scratch after the logits: p rows [T][E], logsumexp^2 [T],
// partial sums [chunks][E + 1].
size_t route_stats_workspace_bytes(int T, int d, int E, int h_bf16) {
  const size_t n_chunks = (static_cast<size_t>(T) + kStatChunk - 1) / kStatChunk;
  return route_workspace_bytes(T, d, E, h_bf16) +
         align_up(static_cast<size_t>(T) * E * sizeof(float), 256) +
         align_up(static_cast<size_t>(T) * sizeof(float), 256) +
         align_up(n_chunks * (E + 1) * sizeof(float), 256);
}

hipError_t launch_route_stats(int T, int E, const float* prow, const float* lsq, float* part,
                              float* p_mean, float* zsq_mean, hipStream_t s) {
  const int n_chunks = (T + kStatChunk - 1) / kStatChunk;
  {
    ProfScope prof_(s, "route_stats");
    hipLaunchKernelGGL(stats_partial_kernel, dim3((E + 1 + 255) / 256, n_chunks), dim3(256), 0, s,
                       T, E, prow, lsq, part);
    hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(1024), 0, s, T, E, n_chunks, part, p_mean,
                       zsq_mean);
  }
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  {
    ProfScope prof_(s, "fill_i32");
    hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, v, n);
  }
  return hipGetLastError();
}

hipError_t launch_route(int T, int d, int E, int K, int fn, const void* h, int h_bf16,
                        const float* e, const float* b, int32_t* idx, float* gates,
                        int32_t* loads, void* ws, float* p_mean, float* zsq_mean,
                        hipStream_t s) {
  hipError_t err;
  const int S = route_splits(T, d, E, h_bf16);
  float* prow = nullptr;
  float* lsq = nullptr;
  float* part = nullptr;
  if (p_mean != nullptr) {
    char* base = static_cast<char*>(ws) + route_workspace_bytes(T, d, E, h_bf16);
    prow = reinterpret_cast<float*>(base);
    lsq = reinterpret_cast<float*>(base + align_up(static_cast<size_t>(T) * E * sizeof(float), 256));
    part = reinterpret_cast<float*>(reinterpret_cast<char*>(lsq) +
                                    align_up(static_cast<size_t>(T) * sizeof(float), 256));
  }
  if (S == 0) {
    if (h_bf16) return hipErrorInvalidValue;  // rejected on the host before this point
    err = launch_fill_i32(loads, 0, static_cast<size_t>(E), s);
    if (err != hipSuccess) return err;
    err = launch_route_f32(T, d, E, K, fn, static_cast<const float*>(h), e, b, idx, gates,
                           loads, prow, lsq, s);
    if (err != hipSuccess || p_mean == nullptr) return err;
    return launch_route_stats(T, E, prow, lsq, part, p_mean, zsq_mean, s);
  }
  float* zpart = static_cast<float*>(ws);
  int32_t* lpad = reinterpret_cast<int32_t*>(
      static_cast<char*>(ws) + align_up(static_cast<size_t>(S) * T * E * sizeof(float), 256));
  {
    ProfScope prof_(s, "route_logits");
    dim3 grid((T + kZT - 1) / kZT, (E + kZE - 1) / kZE, S);
    hipLaunchKernelGGL(route_logits_mfma_kernel, grid, dim3(kZThreads), 0, s, T, d, E, d / S,
                       static_cast<const uint16_t*>(h), e, zpart, lpad);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    ProfScope prof_(s, "route_topk");
    const int ej = (E + kWave - 1) / kWave;
    dim3 grid((T + 3) / 4), block(256);
    const float* zp = zpart;
    if (ej <= 1)
      hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, T, E, K, fn, S, zp, b, idx, gates, lpad, prow, lsq);
    else if (ej <= 2)
      hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, T, E, K, fn, S, zp, b, idx, gates, lpad, prow, lsq);
    else if (ej <= 4)
      hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, T, E, K, fn, S, zp, b, idx, gates, lpad, prow, lsq);
    else
      hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, T, E, K, fn, S, zp, b, idx, gates, lpad, prow, lsq);
  }
  hipLaunchKernelGGL(compact_loads_kernel, dim3((E + 255) / 256), dim3(256), 0, s, E, lpad, loads);
  err = hipGetLastError();
  if (err != hipSuccess || p_mean == nullptr) return err;
  return launch_route_stats(T, E, prow, lsq, part, p_mean, zsq_mean, s);
}

}  // namespace moe
