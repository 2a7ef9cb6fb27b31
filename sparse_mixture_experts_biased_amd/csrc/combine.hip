// Combine: y_t = h_t + sum_j y_shared[j, t] + sum_k g_{t,k} * y_perm[slot_row[t,k]].
//
// Method: Sparse MoE routing-math page (arman1o1.github.io), section 0
// (layer-output equation: residual + always-active shared experts + gated
// routed experts) and section 3 (un-permute and accumulate the gate-weighted
// sum).
//
// Token-major: one wave per token row, 16-byte vector loads; every output
// element is accumulated in fp32 in a fixed order (h, shared experts, then
// k = 0..K-1), so the result is deterministic.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kWave;

__device__ __forceinline__ void add_bf16x8(float (&acc)[8], const uint4& v, float w) {
  const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(w, __uint_as_float(p[i] << 16), acc[2 * i]);
    acc[2 * i + 1] = fmaf(w, __uint_as_float(p[i] & 0xffff0000u), acc[2 * i + 1]);
  }
}

__global__ __launch_bounds__(kThreads) void combine_bf16_kernel(
    int T, int d, int K, int E_s, const uint16_t* __restrict__ h,
    const uint16_t* __restrict__ ysh, const uint16_t* __restrict__ yp,
    const int32_t* __restrict__ slot_row, const float* __restrict__ gates,
    uint16_t* __restrict__ y) {
  const int t = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (t >= T) return;
  const int TK = T * K;
  const int vecs = d / 8;
  int slot[MOE_MAX_TOPK_DEV];
  float g[MOE_MAX_TOPK_DEV];
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) {
    slot[k] = -1;
    g[k] = 0.0f;
    if (k < K) {
      int s = slot_row[static_cast<size_t>(t) * K + k];
      slot[k] = (s >= 0 && s < TK) ? s : -1;
      g[k] = gates[static_cast<size_t>(t) * K + k];
    }
  }
  for (int c = lane; c < vecs; c += kWave) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    add_bf16x8(acc, reinterpret_cast<const uint4*>(h + static_cast<size_t>(t) * d)[c], 1.0f);
    for (int j = 0; j < E_s; ++j)
      add_bf16x8(acc,
                 reinterpret_cast<const uint4*>(ysh + (static_cast<size_t>(j) * T + t) * d)[c],
                 1.0f);
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
      if (k < K && slot[k] >= 0)
        add_bf16x8(acc, reinterpret_cast<const uint4*>(yp + static_cast<size_t>(slot[k]) * d)[c],
                   g[k]);
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    reinterpret_cast<uint4*>(y + static_cast<size_t>(t) * d)[c] = o;
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
    hipLaunchKernelGGL(combine_bf16_kernel, grid, block, 0, s, T, d, K, E_s,
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
