// Auxiliary-loss-free bias update and load statistics.
//
// Method: Sparse MoE routing-math page (arman1o1.github.io), section 2:
// b_i <- b_i + gamma * sign(cbar - c_i) with cbar = K T / E_r, applied once per
// step after the batch's loads are counted; section 4 item 1: MaxVio =
// (max_i c_i - cbar) / cbar.  The Mixture of Experts designs page
// (raminaeye.github.io), section 1 worked example, leaves a bias unchanged
// when its expert sits exactly at the fair share (sign 0).
//
// sign(cbar - c_i) = sign(K*T - E_r*c_i) is decided in 64-bit integers, and
// gamma * sign is exact, so the update is a single fp32 add: bit-reproducible.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(1024) void bias_update_kernel(int T, int E, int K, float gamma,
                                                          const int32_t* __restrict__ loads,
                                                          float* __restrict__ b,
                                                          BiasStats* __restrict__ stats) {
  __shared__ int32_t smax[1024], smin[1024];
  const int i = threadIdx.x;
  int c = 0;
  if (i < E) {
    c = loads[i];
    const long long diff = static_cast<long long>(K) * T - static_cast<long long>(E) * c;
    const float sgn = static_cast<float>((diff > 0) - (diff < 0));
    b[i] = b[i] + gamma * sgn;
  }
  if (stats == nullptr) return;
  smax[i] = (i < E) ? c : INT32_MIN;
  smin[i] = (i < E) ? c : INT32_MAX;
  __syncthreads();
  for (int off = 512; off >= 1; off >>= 1) {
    if (i < off) {
      smax[i] = max(smax[i], smax[i + off]);
      smin[i] = min(smin[i], smin[i + off]);
    }
    __syncthreads();
  }
  if (i == 0) {
    const long long kt = static_cast<long long>(K) * T;
    const long long num = static_cast<long long>(E) * smax[0] - kt;
    BiasStats st;
    st.max_load = smax[0];
    st.min_load = smin[0];
    st.max_vio = static_cast<float>(static_cast<double>(num) / static_cast<double>(kt));
    st.reserved = 0;
    *stats = st;
  }
}

}  // namespace

hipError_t launch_bias_update(int T, int E, int K, float gamma, const int32_t* loads, float* b,
                              BiasStats* stats, hipStream_t s) {
  {
    ProfScope prof_(s, "bias_update");
    hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(1024), 0, s, T, E, K, gamma, loads, b,
                       stats);
  }
  return hipGetLastError();
}

}  // namespace moe
