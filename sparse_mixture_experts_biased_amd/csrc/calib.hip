// Measurement aid (not part of the layer): the rate at which this chip's
// matrix cores run bf16 products with no memory traffic at all, the ceiling
// that the grouped SwiGLU kernels' matrix-core fractions are read against.
//
// Each wave issues the MFMA sequence of one wave of the grouped SwiGLU tile
// (2 row blocks x 4 weight blocks of v_mfma_f32_32x32x16_bf16 per 16-k step,
// 8 independent accumulators) on two sets of fragments held in registers,
// loaded once from the caller's operands (random in practice) and used on
// alternate k-steps, so the operands change between steps as they do in a
// real product.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kMB = 2, kNB = 4;      // accumulator blocks of one wave
constexpr int kChains = kMB * kNB;   // independent accumulation chains
constexpr int kSets = 2;             // fragment sets, alternated per k-step
constexpr int kVecs = kSets * (kMB + kNB);  // 16-byte operand vectors per thread

__global__ __launch_bounds__(256) void mfma_loop_kernel(const uint4* __restrict__ ops, int iters,
                                                        float* __restrict__ out) {
  const size_t t = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  bf16x8_t a[kSets][kMB], b[kSets][kNB];
#pragma unroll
  for (int k = 0; k < kSets; ++k) {
#pragma unroll
    for (int m = 0; m < kMB; ++m)
      a[k][m] = __builtin_bit_cast(bf16x8_t, ops[t * kVecs + k * (kMB + kNB) + m]);
#pragma unroll
    for (int n = 0; n < kNB; ++n)
      b[k][n] = __builtin_bit_cast(bf16x8_t, ops[t * kVecs + k * (kMB + kNB) + kMB + n]);
  }
  f32x16_t acc[kMB][kNB];
#pragma unroll
  for (int m = 0; m < kMB; ++m)
#pragma unroll
    for (int n = 0; n < kNB; ++n)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[m][n][q] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kSets; ++k)
#pragma unroll
      for (int m = 0; m < kMB; ++m)
#pragma unroll
        for (int n = 0; n < kNB; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k][m], b[k][n], acc[m][n], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < kMB; ++m)
#pragma unroll
    for (int n = 0; n < kNB; ++n)
#pragma unroll
      for (int q = 0; q < 16; ++q) s += acc[m][n][q];
  out[t] = s;
}

// Streaming read: every thread reads 16-byte vectors in a grid-stride loop,
// eight in flight per iteration, and folds them into one word it writes out.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src,
                                                          size_t n_vec, uint32_t* __restrict__ out) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n_vec; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n_vec; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(int workgroups, const void* src, size_t bytes, uint32_t* out,
                              hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(256), 0, s,
                     static_cast<const uint4*>(src), bytes / 16, out);
  return hipGetLastError();
}

double mfma_loop_flops(int workgroups, int iters) {
  return static_cast<double>(workgroups) * (256 / kWave) * iters * kSets * kChains * 2.0 * 32 *
         32 * 16;
}

hipError_t launch_mfma_loop(int workgroups, int iters, const uint16_t* ops, float* out,
                            hipStream_t s) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(ops), iters, out);
  return hipGetLastError();
}

}  // namespace moe
