// Shared device helpers and the launch-side declarations of every kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest even; gfx950 converts in hardware
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 -> a bf16 pair (lo in the low half), one v_cvt_pk_bf16_f32.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// SiLU(x) = x * sigma(x), with the hardware reciprocal (about 1 ulp) in place
// of an IEEE division: the products are rounded to bf16 or summed in fp32 far
// above that error, and x -> -inf still gives -0 (rcp(inf) = 0).
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// ---------------------------------------------------------------- sizes

constexpr int kWave = 64;
#define MOE_MAX_TOPK_DEV 16

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- launches
// Each returns the hipError_t of its last launch.

// router
int route_splits(int T, int d, int E, int h_bf16);
size_t route_workspace_bytes(int T, int d, int E, int h_bf16);
// p_mean / zsq_mean non-NULL: also the diagnostics (workspace of
// route_stats_workspace_bytes); else the workspace of route_workspace_bytes.
hipError_t launch_route(int T, int d, int E, int K, int fn, const void* h, int h_bf16,
                        const float* e, const float* b, int32_t* idx, float* gates,
                        int32_t* loads, void* ws, float* p_mean, float* zsq_mean,
                        hipStream_t s);
size_t route_stats_workspace_bytes(int T, int d, int E, int h_bf16);
hipError_t launch_route_stats(int T, int E, const float* prow, const float* lsq, float* part,
                              float* p_mean, float* zsq_mean, hipStream_t s);
struct RouterDiag {  // layout of moe_router_diag
  float switch_fP, z_loss, load_entropy, max_vio, dropped, reserved[3];
};
hipError_t launch_router_diag(int T, int E, int K, const int32_t* loads, const float* p_mean,
                              const float* zsq_mean, const int32_t* offsets, float* f,
                              RouterDiag* diag, hipStream_t s);

// dispatch
constexpr int kPermChunk = 256;  // tokens per histogram / rank chunk
size_t permute_workspace_bytes(int T, int E);
// cap < 0: every copy is kept; cap >= 0: at most cap rows per expert.
hipError_t launch_permute(int T, int d, int E, int K, int cap, const int32_t* idx,
                          const void* h, int elem_bytes, int32_t* offsets, int32_t* row_token,
                          int32_t* slot_row, void* x_perm, void* ws, hipStream_t s);

// grouped SwiGLU
size_t swiglu_workspace_bytes(int n_groups, int d_model, int d_ffn, int rows, int bf16);
hipError_t launch_swiglu_f32(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                             const int32_t* offsets, const int32_t* row_index, const float* x,
                             const float* wg, const float* wu, const float* wd,
                             const float* row_scale, float* y, void* ws, hipStream_t s);
hipError_t launch_swiglu_bf16(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                              const int32_t* offsets, const int32_t* row_index,
                              const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                              const uint16_t* wd, const float* row_scale, uint16_t* y,
                              uint16_t* au, void* ws, hipStream_t s);

// combine
hipError_t launch_combine(int T, int d, int K, int E_s, const void* h, const void* y_shared,
                          const void* y_perm, const int32_t* slot_row, const float* gates,
                          int bf16, void* y, hipStream_t s);

// bias update
struct BiasStats {
  int32_t max_load, min_load;
  float max_vio;
  int32_t reserved;
};
hipError_t launch_bias_update(int T, int E, int K, float gamma, const int32_t* loads, float* b,
                              BiasStats* stats, hipStream_t s);

// measurement aid: independent MFMA chains on register operands
double mfma_loop_flops(int workgroups, int iters);
hipError_t launch_mfma_loop(int workgroups, int iters, const uint16_t* ops, float* out,
                            hipStream_t s);
hipError_t launch_stream_read(int workgroups, const void* src, size_t bytes, uint32_t* out,
                              hipStream_t s);

// small utilities
hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s);

// Optional event timing of the library's kernels (off unless enabled through
// moe_profile_enable).  prof_begin returns a token for prof_end, or -1.
int prof_begin(hipStream_t s, const char* name);
void prof_end(int token, hipStream_t s);

struct ProfScope {
  int tok;
  hipStream_t s;
  // name nullptr: no record (a caller's own scope covers the launch)
  ProfScope(hipStream_t st, const char* name) : tok(name ? prof_begin(st, name) : -1), s(st) {}
  ~ProfScope() { prof_end(tok, s); }
};

}  // namespace moe
