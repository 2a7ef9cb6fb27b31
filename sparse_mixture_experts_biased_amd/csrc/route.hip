// Router: z = h . e (fp32), score function, biased top-K, unbiased gates and
// the load histogram, fused in one kernel.
//
// Method: Sparse MoE routing-math page (arman1o1.github.io), section 2
// (I_t = TopK(s + b, K), g = s / sum_{I_t} s, sigmoid affinity) and the
// classical-router listing of section 1 (softmax, top-K, renormalise, clamp
// 1e-12); section 4 item 2 keeps the router in fp32.
//
// Layout: one workgroup of 256 threads owns BT = 16 tokens and all E experts.
// The z tile [16 x E] is built from LDS-staged h and e slices (fp32 FMA), then
// each wave ranks four tokens: K rounds of a wave-wide arg-max over v = s + b
// (equal v -> lower expert id), a sort of the K picks by expert id, and the
// gate denominator summed in that order, so the gates depend only on the
// picked set.
#include "common.h"

#include <math.h>

namespace moe {
namespace {

constexpr int kBT = 16;       // tokens per workgroup
constexpr int kBK = 32;       // d_model slice per LDS stage
constexpr int kThreads = 256;
constexpr int kTokPerWave = kBT / 4;

template <typename TIn>
__device__ __forceinline__ float load_in(const TIn* p, size_t i);
template <>
__device__ __forceinline__ float load_in<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_in<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

// Arg-max over the wave: larger v wins, equal v -> smaller expert id.
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    float ov = __shfl_xor(v, m, kWave);
    int oid = __shfl_xor(id, m, kWave);
    // a real expert id always beats the "none" sentinel
    if (oid != 0x7fffffff && (id == 0x7fffffff || ov > v || (ov == v && oid < id))) {
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

template <typename TIn, int EJ>
__global__ __launch_bounds__(kThreads) void route_kernel(
    int T, int d, int E, int K, int fn, const TIn* __restrict__ h,
    const float* __restrict__ e, const float* __restrict__ b, int32_t* __restrict__ idx_out,
    float* __restrict__ gate_out, int32_t* __restrict__ loads) {
  extern __shared__ float smem[];
  float* hs = smem;                       // [kBT][kBK]
  float* es = smem + kBT * kBK;           // [E][kBK + 1]
  float* zs = es;                         // reused after the K loop: [kBT][E]

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
      hs[q] = (t < T && k < d) ? load_in<TIn>(h, static_cast<size_t>(t) * d + k) : 0.0f;
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

  // z tile to LDS (the e slice is no longer needed).
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
    float s[EJ], v[EJ];
    if (fn == 0) {
#pragma unroll
      for (int j = 0; j < EJ; ++j) {
        int ex = lane + kWave * j;
        float z = (ex < E) ? zs[r * E + ex] : 0.0f;
        s[j] = 1.0f / (1.0f + expf(-z));
      }
    } else {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < EJ; ++j) {
        int ex = lane + kWave * j;
        if (ex < E) m = fmaxf(m, zs[r * E + ex]);
      }
      m = wave_max(m);
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < EJ; ++j) {
        int ex = lane + kWave * j;
        s[j] = (ex < E) ? expf(zs[r * E + ex] - m) : 0.0f;
        part += s[j];
      }
      float tot = wave_sum(part);
#pragma unroll
      for (int j = 0; j < EJ; ++j) s[j] = s[j] / tot;
    }
#pragma unroll
    for (int j = 0; j < EJ; ++j) v[j] = s[j] + bias[j];

    // K rounds of arg-max; sel/sv hold the picks (wave-uniform).
    int sel[MOE_MAX_TOPK_DEV];
    float sv[MOE_MAX_TOPK_DEV];
    unsigned taken = 0u;
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) {
      sel[k] = 0x7fffffff;
      sv[k] = 0.0f;
      if (k < K) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < EJ; ++j) {
          int ex = lane + kWave * j;
          bool ok = ex < E && !((taken >> j) & 1u);
          // the first free candidate is always taken, so a NaN score cannot
          // leave the pick without an expert id
          if (ok && (be == 0x7fffffff || v[j] > bv || (v[j] == bv && ex < be))) {
            bv = v[j];
            be = ex;
          }
        }
        wave_argmax(bv, be);
        if (be < 0 || be >= E) be = 0;      // only reachable with non-finite scores
        const int jw = be / kWave;          // uniform
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
    // ascending expert id (sentinel ids sort last)
#pragma unroll
    for (int a = 0; a < MOE_MAX_TOPK_DEV - 1; ++a)
#pragma unroll
      for (int c = 0; c < MOE_MAX_TOPK_DEV - 1 - a; ++c)
        if (sel[c] > sel[c + 1]) {
          int ti = sel[c]; sel[c] = sel[c + 1]; sel[c + 1] = ti;
          float tf = sv[c]; sv[c] = sv[c + 1]; sv[c + 1] = tf;
        }
    float den = 0.0f;
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
      if (k < K) den += sv[k];
    den = fmaxf(den, 1e-12f);
    int my_id = 0;
    float my_s = 0.0f;
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
      if (k == lane) {
        my_id = sel[k];
        my_s = sv[k];
      }
    if (lane < K) {
      idx_out[static_cast<size_t>(t) * K + lane] = my_id;
      gate_out[static_cast<size_t>(t) * K + lane] = my_s / den;
      if (my_id >= 0 && my_id < E) atomicAdd(&loads[my_id], 1);
    }
  }
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, size_t n) {
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <typename TIn>
hipError_t launch_typed(int T, int d, int E, int K, int fn, const TIn* h, const float* e,
                        const float* b, int32_t* idx, float* gates, int32_t* loads,
                        hipStream_t s) {
  dim3 grid((T + kBT - 1) / kBT), block(kThreads);
  size_t es_floats = static_cast<size_t>(E) * (kBK + 1);
  size_t zs_floats = static_cast<size_t>(kBT) * E;
  size_t shmem = (kBT * kBK + (es_floats > zs_floats ? es_floats : zs_floats)) * sizeof(float);
  int ej = (E + kWave - 1) / kWave;
  if (shmem > 64 * 1024) {
    hipError_t err = hipSuccess;
    if (ej <= 1)
      err = hipFuncSetAttribute(reinterpret_cast<const void*>(route_kernel<TIn, 1>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    else if (ej <= 2)
      err = hipFuncSetAttribute(reinterpret_cast<const void*>(route_kernel<TIn, 2>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    else if (ej <= 4)
      err = hipFuncSetAttribute(reinterpret_cast<const void*>(route_kernel<TIn, 4>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    else
      err = hipFuncSetAttribute(reinterpret_cast<const void*>(route_kernel<TIn, 8>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (err != hipSuccess) return err;
  }
  ProfScope prof_(s, "route");
  if (ej <= 1)
    hipLaunchKernelGGL((route_kernel<TIn, 1>), grid, block, shmem, s, T, d, E, K, fn, h, e, b,
                       idx, gates, loads);
  else if (ej <= 2)
    hipLaunchKernelGGL((route_kernel<TIn, 2>), grid, block, shmem, s, T, d, E, K, fn, h, e, b,
                       idx, gates, loads);
  else if (ej <= 4)
    hipLaunchKernelGGL((route_kernel<TIn, 4>), grid, block, shmem, s, T, d, E, K, fn, h, e, b,
                       idx, gates, loads);
  else
    hipLaunchKernelGGL((route_kernel<TIn, 8>), grid, block, shmem, s, T, d, E, K, fn, h, e, b,
                       idx, gates, loads);
  return hipGetLastError();
}

}  // namespace

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
                        int32_t* loads, hipStream_t s) {
  hipError_t err = launch_fill_i32(loads, 0, static_cast<size_t>(E), s);
  if (err != hipSuccess) return err;
  if (h_bf16)
    return launch_typed<uint16_t>(T, d, E, K, fn, static_cast<const uint16_t*>(h), e, b, idx,
                                  gates, loads, s);
  return launch_typed<float>(T, d, E, K, fn, static_cast<const float*>(h), e, b, idx, gates,
                             loads, s);
}

}  // namespace moe
