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
//
// Router diagnostics (forward values): routing-math page, section 1 (Switch
// f_i = E_r/(K T) c_i times the mean probability P_i, summed; router z-loss)
// and the designs page's per-layer log (MaxVio, dropped-copy rate, entropy of
// the load share with the share clamped at 1e-9 inside the log).  One
// workgroup, fixed-order tree reductions: deterministic.
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

template <typename V, typename Op>
__device__ __forceinline__ V block_reduce(V* sh, V v, Op op) {
  const int i = threadIdx.x;
  sh[i] = v;
  __syncthreads();
  for (int off = 512; off >= 1; off >>= 1) {
    if (i < off) sh[i] = op(sh[i], sh[i + off]);
    __syncthreads();
  }
  const V r = sh[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void router_diag_kernel(int T, int E, int K,
                                                          const int32_t* __restrict__ loads,
                                                          const float* __restrict__ p_mean,
                                                          const float* __restrict__ zsq_mean,
                                                          const int32_t* __restrict__ offsets,
                                                          float* __restrict__ f_out,
                                                          RouterDiag* __restrict__ diag) {
  __shared__ float shf[1024];
  __shared__ int shi[1024];
  const int i = threadIdx.x;
  const int c = (i < E) ? loads[i] : 0;
  const double kt = static_cast<double>(K) * T;
  const float f = (i < E) ? static_cast<float>(static_cast<double>(E) * c / kt) : 0.0f;
  if (f_out != nullptr && i < E) f_out[i] = f;
  const float fP = block_reduce(shf, (i < E) ? f * p_mean[i] : 0.0f,
                                [](float a, float b) { return a + b; });
  const int csum = block_reduce(shi, c, [](int a, int b) { return a + b; });
  const int cmax = block_reduce(shi, (i < E) ? c : INT32_MIN, [](int a, int b) { return max(a, b); });
  float h = 0.0f;
  if (i < E && csum > 0) {
    const float share = static_cast<float>(c) / static_cast<float>(csum);
    h = -share * logf(fmaxf(share, 1e-9f));
  }
  const float ent = block_reduce(shf, h, [](float a, float b) { return a + b; });
  if (i == 0) {
    RouterDiag d;
    d.switch_fP = fP;
    d.z_loss = *zsq_mean;
    d.load_entropy = ent;
    d.max_vio = static_cast<float>((static_cast<double>(E) * cmax - kt) / kt);
    d.dropped = offsets ? static_cast<float>(1.0 - static_cast<double>(offsets[E]) / kt) : 0.0f;
    d.reserved[0] = d.reserved[1] = d.reserved[2] = 0.0f;
    *diag = d;
  }
}

}  // namespace

hipError_t launch_router_diag(int T, int E, int K, const int32_t* loads, const float* p_mean,
                              const float* zsq_mean, const int32_t* offsets, float* f,
                              RouterDiag* diag, hipStream_t s) {
  {
    ProfScope prof_(s, "router_diag");
    hipLaunchKernelGGL(router_diag_kernel, dim3(1), dim3(1024), 0, s, T, E, K, loads, p_mean,
                       zsq_mean, offsets, f, diag);
  }
  return hipGetLastError();
}

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
