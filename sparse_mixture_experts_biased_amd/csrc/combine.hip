// Combine: y_t = h_t + sum_j y_shared[j, t] + sum_k g_{t,k} * y_perm[slot_row[t,k]].
//
// Method: Sparse MoE routing-math page (arman1o1.github.io), section 0
// (layer-output equation: residual + always-active shared experts + gated
// routed experts) and section 3 (un-permute and accumulate the gate-weighted
// sum).
//
// Token-major: one wave per token row, 16-byte vector loads, all of an
// iteration's loads in flight before the first is used; every output element
// is accumulated in fp32 in a fixed order (h, shared experts, then k =
// 0..K-1), so the result is deterministic.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kWave;
constexpr int kChunksPerIter = 2;  // 16-byte chunks of a row per lane and iteration

__device__ __forceinline__ void add_bf16x8(float (&acc)[8], const uint4& v, float w) {
  const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(w, __uint_as_float(p[i] << 16), acc[2 * i]);
    acc[2 * i + 1] = fmaf(w, __uint_as_float(p[i] & 0xffff0000u), acc[2 * i + 1]);
  }
}

// U 16-byte chunks of the row per lane per iteration.  The loads of an
// iteration -- h, the first shared expert's row, the K gathered rows -- are
// all issued before any of them is used, so a wave keeps U * (K + 2) loads in
// flight.  The gathered rows go through buffer loads whose offset is out of
// range (reads zeros, no memory access) for a dropped or invalid slot, so no
// branch sits between them.  The sum is taken in the fixed order h, shared
// experts 0..E_s-1, k = 0..K-1.
constexpr uint32_t kOffNone = 0x80000000u;  // beyond every buffer (sizes < 2 GiB)

template <int U>
__global__ __launch_bounds__(kThreads) void combine_bf16_kernel(
    int T, int d, int K, int E_s, const uint16_t* __restrict__ h,
    const uint16_t* __restrict__ ysh, const uint16_t* __restrict__ yp,
    const int32_t* __restrict__ slot_row, const float* __restrict__ gates,
    uint16_t* __restrict__ y) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * kRowsPerBlock + threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  if (t >= T) return;
  const int TK = T * K;
  const int vecs = d / 8;
  const __amdgpu_buffer_rsrc_t rsP = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(yp), 0, static_cast<int>(static_cast<uint32_t>(TK) * d * 2u),
      0x00020000);
  // the token's slots and gates: lane k holds entry k, then each is broadcast
  const int sl = lane < K ? slot_row[static_cast<size_t>(t) * K + lane] : -1;
  const float gl = lane < K ? gates[static_cast<size_t>(t) * K + lane] : 0.0f;
  uint32_t poff[MOE_MAX_TOPK_DEV];
  float g[MOE_MAX_TOPK_DEV];
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) {
    const int s = __builtin_amdgcn_readlane(sl, k);
    g[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gl), k));
    poff[k] = (k < K && s >= 0 && s < TK) ? static_cast<uint32_t>(s) * d * 2u : kOffNone;
  }
  const uint4* hr = reinterpret_cast<const uint4*>(h + static_cast<size_t>(t) * d);
  const uint4* s0 = reinterpret_cast<const uint4*>(ysh + static_cast<size_t>(t) * d);
  uint4* yr = reinterpret_cast<uint4*>(y + static_cast<size_t>(t) * d);
  for (int c0 = lane; c0 < vecs; c0 += U * kWave) {
    // a chunk past the row end (only when U * kWave does not divide d / 8)
    // reads whatever the buffer bounds allow and is never stored
    bool ok[U];
    uint32_t cb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ok[u] = c0 + u * kWave < vecs;
      cb[u] = static_cast<uint32_t>(c0 + u * kWave) * 16u;
    }
    uint4 vh[U], vs[U], vp[MOE_MAX_TOPK_DEV][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      vh[u] = ok[u] ? hr[c0 + u * kWave] : make_uint4(0, 0, 0, 0);
      vs[u] = (ok[u] && E_s > 0) ? s0[c0 + u * kWave] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
      if (k < K)
#pragma unroll
        for (int u = 0; u < U; ++u)
          vp[k][u] = __builtin_bit_cast(
              uint4, __builtin_amdgcn_raw_buffer_load_b128(rsP, poff[k] + cb[u], 0, 0));
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = 0.0f;
      add_bf16x8(acc[u], vh[u], 1.0f);
      if (E_s > 0) add_bf16x8(acc[u], vs[u], 1.0f);
    }
    for (int j = 1; j < E_s; ++j) {
      const uint4* sr = reinterpret_cast<const uint4*>(ysh + (static_cast<size_t>(j) * T + t) * d);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (ok[u]) add_bf16x8(acc[u], sr[c0 + u * kWave], 1.0f);
    }
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
      if (k < K)
#pragma unroll
        for (int u = 0; u < U; ++u) add_bf16x8(acc[u], vp[k][u], g[k]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ok[u]) {
        uint4 o;
        o.x = pack_bf16x2(acc[u][0], acc[u][1]);
        o.y = pack_bf16x2(acc[u][2], acc[u][3]);
        o.z = pack_bf16x2(acc[u][4], acc[u][5]);
        o.w = pack_bf16x2(acc[u][6], acc[u][7]);
        yr[c0 + u * kWave] = o;
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void combine_f32_kernel(
    int T, int d, int K, int E_s, const float* __restrict__ h, const float* __restrict__ ysh,
    const float* __restrict__ yp, const int32_t* __restrict__ slot_row,
    const float* __restrict__ gates, float* __restrict__ y) {
  const int t = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (t >= T) return;
  const int TK = T * K;
  const int vecs = d / 4;
  for (int c = lane; c < vecs; c += kWave) {
    float4 a = reinterpret_cast<const float4*>(h + static_cast<size_t>(t) * d)[c];
    for (int j = 0; j < E_s; ++j) {
      float4 v = reinterpret_cast<const float4*>(ysh + (static_cast<size_t>(j) * T + t) * d)[c];
      a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
    }
    for (int k = 0; k < K; ++k) {
      int s = slot_row[static_cast<size_t>(t) * K + k];
      if (s < 0 || s >= TK) continue;
      float gk = gates[static_cast<size_t>(t) * K + k];
      float4 v = reinterpret_cast<const float4*>(yp + static_cast<size_t>(s) * d)[c];
      a.x = fmaf(gk, v.x, a.x); a.y = fmaf(gk, v.y, a.y);
      a.z = fmaf(gk, v.z, a.z); a.w = fmaf(gk, v.w, a.w);
    }
    reinterpret_cast<float4*>(y + static_cast<size_t>(t) * d)[c] = a;
  }
}

}  // namespace

hipError_t launch_combine(int T, int d, int K, int E_s, const void* h, const void* y_shared,
                          const void* y_perm, const int32_t* slot_row, const float* gates,
                          int bf16, void* y, hipStream_t s) {
  dim3 grid((T + kRowsPerBlock - 1) / kRowsPerBlock), block(kThreads);
  ProfScope prof_(s, "combine");
  if (bf16)
    hipLaunchKernelGGL(combine_bf16_kernel<kChunksPerIter>, grid, block, 0, s, T, d, K, E_s,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(y_shared),
                       static_cast<const uint16_t*>(y_perm), slot_row, gates,
                       static_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL(combine_f32_kernel, grid, block, 0, s, T, d, K, E_s,
                       static_cast<const float*>(h), static_cast<const float*>(y_shared),
                       static_cast<const float*>(y_perm), slot_row, gates,
                       static_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace moe
