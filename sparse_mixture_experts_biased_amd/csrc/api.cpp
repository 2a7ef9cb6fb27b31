// C ABI of the MoE layer library: host-side argument validation, then the
// asynchronous kernel launches.  Nothing here allocates device memory,
// synchronises with the device or copies data back to the host.
#include <cmath>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "common.h"
#include "swiglu_tiles.h"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

moe_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool valid_dtype(moe_dtype d) { return d == MOE_F32 || d == MOE_BF16; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

static_assert(sizeof(moe_bias_stats) == sizeof(moe::BiasStats), "stats layout");

extern "C" {

const char* moe_last_error(void) { return g_err; }

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

size_t moe_route_workspace_size(int T, int d_model, int E_r, moe_dtype h_dtype) {
  if (T < 1 || d_model < 1 || E_r < 1 || !valid_dtype(h_dtype)) return 0;
  return moe::route_workspace_bytes(T, d_model, E_r, h_dtype == MOE_BF16);
}

namespace {

moe_status route_checked(const char* name, int T, int d_model, int E_r, int K, moe_score_fn fn,
                         const void* h, moe_dtype h_dtype, const float* e, const float* b,
                         int32_t* topk_idx, float* gates, int32_t* loads, float* p_mean,
                         float* zsq_mean, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (T < 1 || d_model < 1 || E_r < 1 || K < 1)
    return fail(MOE_ERR_INVALID_ARG, "%s: T=%d d_model=%d E_r=%d K=%d must be >= 1", name, T,
                d_model, E_r, K);
  if (K > E_r) return fail(MOE_ERR_INVALID_ARG, "%s: K=%d > E_r=%d", name, K, E_r);
  if (K > MOE_MAX_TOPK)
    return fail(MOE_ERR_INVALID_ARG, "%s: K=%d > %d", name, K, MOE_MAX_TOPK);
  if (E_r > 512) return fail(MOE_ERR_UNSUPPORTED, "%s: E_r=%d > 512", name, E_r);
  if (fn != MOE_SIGMOID && fn != MOE_SOFTMAX)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown score function %d", name, (int)fn);
  if (!valid_dtype(h_dtype)) return fail(MOE_ERR_INVALID_ARG, "%s: bad dtype", name);
  if (d_model % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: d_model=%d not a multiple of 8", name, d_model);
  if (h_dtype == MOE_BF16 && d_model % 32 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 tokens need d_model %% 32 == 0 (got %d)", name,
                d_model);
  if (h_dtype == MOE_BF16 && d_model > (1 << 20))
    return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 tokens need d_model <= 1048576 (got %d)", name,
                d_model);
  if (!h || !e || !topk_idx || !gates || !loads)
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", name);
  const bool stats = p_mean != nullptr;
  const size_t need = stats ? moe::route_stats_workspace_bytes(T, d_model, E_r, h_dtype == MOE_BF16)
                            : moe::route_workspace_bytes(T, d_model, E_r, h_dtype == MOE_BF16);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace %zu < %zu bytes", name, workspace_bytes, need);
  if (static_cast<long long>(T) * K > INT32_MAX || static_cast<long long>(T) * d_model > (1LL << 40) ||
      static_cast<long long>(T) * E_r > (1LL << 31))
    return fail(MOE_ERR_INVALID_ARG, "%s: sizes overflow", name);
  return hip_status(moe::launch_route(T, d_model, E_r, K, (int)fn, h, h_dtype == MOE_BF16, e, b,
                                      topk_idx, gates, loads, workspace, p_mean, zsq_mean,
                                      as_stream(stream)),
                    name);
}

}  // namespace

moe_status moe_route(int T, int d_model, int E_r, int K, moe_score_fn fn, const void* h,
                     moe_dtype h_dtype, const float* e, const float* b, int32_t* topk_idx,
                     float* gates, int32_t* loads, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return route_checked("moe_route", T, d_model, E_r, K, fn, h, h_dtype, e, b, topk_idx, gates,
                       loads, nullptr, nullptr, workspace, workspace_bytes, stream);
}

size_t moe_route_stats_workspace_size(int T, int d_model, int E_r, moe_dtype h_dtype) {
  if (T < 1 || d_model < 1 || E_r < 1 || !valid_dtype(h_dtype)) return 0;
  return moe::route_stats_workspace_bytes(T, d_model, E_r, h_dtype == MOE_BF16);
}

moe_status moe_route_stats(int T, int d_model, int E_r, int K, moe_score_fn fn, const void* h,
                           moe_dtype h_dtype, const float* e, const float* b, int32_t* topk_idx,
                           float* gates, int32_t* loads, float* p_mean, float* zsq_mean,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!p_mean || !zsq_mean) return fail(MOE_ERR_INVALID_ARG, "moe_route_stats: null pointer");
  return route_checked("moe_route_stats", T, d_model, E_r, K, fn, h, h_dtype, e, b, topk_idx,
                       gates, loads, p_mean, zsq_mean, workspace, workspace_bytes, stream);
}

moe_status moe_router_diag(int T, int E_r, int K, const int32_t* loads, const float* p_mean,
                           const float* zsq_mean, const int32_t* offsets, float* f,
                           moe_router_diag_values* diag, void* stream) {
  if (T < 1 || E_r < 1 || K < 1 || K > E_r)
    return fail(MOE_ERR_INVALID_ARG, "moe_router_diag: T=%d E_r=%d K=%d", T, E_r, K);
  if (E_r > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "moe_router_diag: E_r=%d > %d", E_r, MOE_MAX_EXPERTS);
  if (static_cast<long long>(T) * K > INT32_MAX)
    return fail(MOE_ERR_INVALID_ARG, "moe_router_diag: T*K overflows int32");
  if (!loads || !p_mean || !zsq_mean || !diag)
    return fail(MOE_ERR_INVALID_ARG, "moe_router_diag: null pointer");
  static_assert(sizeof(moe_router_diag_values) == sizeof(moe::RouterDiag), "diag layout");
  return hip_status(moe::launch_router_diag(T, E_r, K, loads, p_mean, zsq_mean, offsets, f,
                                            reinterpret_cast<moe::RouterDiag*>(diag),
                                            as_stream(stream)),
                    "moe_router_diag");
}

size_t moe_permute_workspace_size(int T, int E_r) {
  if (T < 1 || E_r < 1) return 0;
  return moe::permute_workspace_bytes(T, E_r);
}

namespace {

moe_status permute_checked(const char* fn, int T, int d_model, int E_r, int K, int cap,
                           const int32_t* topk_idx, const void* h, moe_dtype dtype,
                           int32_t* offsets, int32_t* row_token, int32_t* slot_row, void* x_perm,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 1 || E_r < 1 || K < 1 || d_model < 1)
    return fail(MOE_ERR_INVALID_ARG, "%s: T=%d d_model=%d E_r=%d K=%d must be >= 1", fn, T,
                d_model, E_r, K);
  if (K > E_r || K > MOE_MAX_TOPK) return fail(MOE_ERR_INVALID_ARG, "%s: K=%d out of range", fn, K);
  if (E_r > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E_r=%d > %d", fn, E_r, MOE_MAX_EXPERTS);
  if (static_cast<long long>(T) * K > INT32_MAX)
    return fail(MOE_ERR_INVALID_ARG, "%s: T*K overflows int32", fn);
  if (!topk_idx || !offsets || !row_token || !slot_row || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (workspace_bytes < moe::permute_workspace_bytes(T, E_r))
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace %zu < %zu bytes", fn, workspace_bytes,
                moe::permute_workspace_bytes(T, E_r));
  if (x_perm) {
    if (!h) return fail(MOE_ERR_INVALID_ARG, "%s: x_perm needs h", fn);
    if (!valid_dtype(dtype)) return fail(MOE_ERR_INVALID_ARG, "%s: bad dtype", fn);
    if (d_model % 8 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "%s: d_model=%d not a multiple of 8", fn, d_model);
  }
  const int eb = dtype == MOE_BF16 ? 2 : 4;
  return hip_status(moe::launch_permute(T, d_model, E_r, K, cap, topk_idx, h, eb, offsets,
                                        row_token, slot_row, x_perm, workspace,
                                        as_stream(stream)),
                    fn);
}

}  // namespace

moe_status moe_permute(int T, int d_model, int E_r, int K, const int32_t* topk_idx,
                       const void* h, moe_dtype dtype, int32_t* offsets, int32_t* row_token,
                       int32_t* slot_row, void* x_perm, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return permute_checked("moe_permute", T, d_model, E_r, K, -1, topk_idx, h, dtype, offsets,
                         row_token, slot_row, x_perm, workspace, workspace_bytes, stream);
}

int moe_expert_capacity(int T, int K, int E_r, double capacity_factor) {
  if (T < 1 || K < 1 || E_r < 1 || !(capacity_factor >= 0.0)) return -1;
  const double c = std::ceil(capacity_factor * static_cast<double>(static_cast<long long>(T) * K) /
                             static_cast<double>(E_r));
  if (c > static_cast<double>(INT32_MAX)) return -1;
  return static_cast<int>(c);
}

moe_status moe_permute_capacity(int T, int d_model, int E_r, int K, int capacity,
                                const int32_t* topk_idx, const void* h, moe_dtype dtype,
                                int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                                void* x_perm, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (capacity < 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_permute_capacity: capacity=%d must be >= 0", capacity);
  return permute_checked("moe_permute_capacity", T, d_model, E_r, K, capacity, topk_idx, h, dtype,
                         offsets, row_token, slot_row, x_perm, workspace, workspace_bytes, stream);
}

size_t moe_grouped_swiglu_workspace_size(int n_groups, int d_model, int d_ffn, int rows,
                                         moe_dtype dtype) {
  (void)d_model;
  if (n_groups < 1 || d_ffn < 1 || rows < 0 || !valid_dtype(dtype)) return 0;
  return moe::swiglu_workspace_bytes(n_groups, d_model, d_ffn, rows, dtype == MOE_BF16);
}

namespace {

// Shared by the inference and training forms; au (bf16 only) also receives the
// gate and up projections.
moe_status grouped_swiglu(const char* fn, int n_groups, int d_model, int d_ffn, int rows,
                          int x_rows, const int32_t* offsets, const int32_t* row_index,
                          const void* x, moe_dtype dtype, const void* w_gate, const void* w_up,
                          const void* w_down, const float* row_scale, void* y, void* au,
                          void* workspace, size_t workspace_bytes, void* stream,
                          bool launch = true) {
  if (n_groups < 1 || d_model < 1 || d_ffn < 1 || rows < 0 || x_rows < 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: n_groups=%d d_model=%d d_ffn=%d rows=%d x_rows=%d", fn,
                n_groups, d_model, d_ffn, rows, x_rows);
  if (n_groups > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "%s: n_groups=%d > %d", fn, n_groups, MOE_MAX_EXPERTS);
  if (!valid_dtype(dtype)) return fail(MOE_ERR_INVALID_ARG, "%s: bad dtype", fn);
  if (!offsets || !x || !w_gate || !w_up || !w_down || !y || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (row_index == nullptr && x_rows < rows)
    return fail(MOE_ERR_INVALID_ARG, "%s: x_rows=%d < rows=%d without row_index", fn, x_rows,
                rows);
  const int align = dtype == MOE_BF16 ? 64 : 16;
  if (d_model % align || d_ffn % align)
    return fail(MOE_ERR_UNSUPPORTED, "%s: d_model=%d and d_ffn=%d must be multiples of %d", fn,
                d_model, d_ffn, align);
  if (static_cast<long long>(rows) * d_ffn > (1LL << 40) ||
      static_cast<long long>(d_model) * d_ffn > INT32_MAX)
    return fail(MOE_ERR_INVALID_ARG, "%s: sizes overflow", fn);
  if (dtype == MOE_BF16) {
    // the matrix-core path addresses each operand with 32-bit buffer offsets
    const long long lim = (1LL << 31) - 1;
    if (2LL * x_rows * d_model > lim || 2LL * rows * d_ffn > lim || 2LL * d_model * d_ffn > lim)
      return fail(MOE_ERR_UNSUPPORTED,
                  "%s: bf16 operands must each be under 2 GiB "
                  "(x %lld, activations %lld, one weight matrix %lld bytes)",
                  fn, 2LL * x_rows * d_model, 2LL * rows * d_ffn, 2LL * d_model * d_ffn);
  }
  const size_t need = moe::swiglu_workspace_bytes(n_groups, d_model, d_ffn, rows, dtype == MOE_BF16);
  if (workspace_bytes < need)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  if (!launch) return MOE_OK;
  if (rows == 0) return MOE_OK;
  hipError_t err;
  if (dtype == MOE_BF16)
    err = moe::launch_swiglu_bf16(n_groups, d_model, d_ffn, rows, x_rows, offsets, row_index,
                                  static_cast<const uint16_t*>(x),
                                  static_cast<const uint16_t*>(w_gate),
                                  static_cast<const uint16_t*>(w_up),
                                  static_cast<const uint16_t*>(w_down), row_scale,
                                  static_cast<uint16_t*>(y), static_cast<uint16_t*>(au), workspace,
                                  as_stream(stream));
  else
    err = moe::launch_swiglu_f32(n_groups, d_model, d_ffn, rows, x_rows, offsets, row_index,
                                 static_cast<const float*>(x), static_cast<const float*>(w_gate),
                                 static_cast<const float*>(w_up),
                                 static_cast<const float*>(w_down), row_scale,
                                 static_cast<float*>(y), workspace, as_stream(stream));
  return hip_status(err, fn);
}

}  // namespace

moe_status moe_grouped_swiglu(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                              const int32_t* offsets, const int32_t* row_index, const void* x,
                              moe_dtype dtype, const void* w_gate, const void* w_up,
                              const void* w_down, const float* row_scale, void* y,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return grouped_swiglu("moe_grouped_swiglu", n_groups, d_model, d_ffn, rows, x_rows, offsets,
                        row_index, x, dtype, w_gate, w_up, w_down, row_scale, y, nullptr,
                        workspace, workspace_bytes, stream);
}

// ---- routed and shared experts in one call

namespace {

// fp32: the combined row index, the shared offsets, then one grouped
// workspace that the routed and the shared launches use in turn.
struct ExpertsF32Layout {
  int32_t* row_index;
  int32_t* sh_off;
  void* ws;
  size_t bytes;
};
ExpertsF32Layout experts_f32_layout(void* base, int E_r, int E_s, int T, int K, int d_model,
                                    int d_ffn) {
  const int TK = T * K, rows = TK + E_s * T;
  const size_t ri = moe::align_up(static_cast<size_t>(rows) * 4, 256);
  const size_t so = moe::align_up(static_cast<size_t>(E_s + 1) * 4, 256);
  size_t w = moe::swiglu_workspace_bytes(E_r, d_model, d_ffn, TK, 0);
  if (E_s > 0) w = std::max(w, moe::swiglu_workspace_bytes(E_s, d_model, d_ffn, E_s * T, 0));
  char* b = static_cast<char*>(base);
  return ExpertsF32Layout{b ? reinterpret_cast<int32_t*>(b) : nullptr,
                          b ? reinterpret_cast<int32_t*>(b + ri) : nullptr,
                          b ? b + ri + so : nullptr, ri + so + w};
}

size_t experts_workspace_bytes(int E_r, int E_s, int T, int K, int d_model, int d_ffn,
                               moe_dtype dtype) {
  if (dtype == MOE_BF16) return moe::experts_layout(nullptr, E_r, E_s, T, K, d_ffn).bytes;
  return experts_f32_layout(nullptr, E_r, E_s, T, K, d_model, d_ffn).bytes;
}

bool experts_shape_ok(int E_r, int E_s, int T, int K, int d_model, int d_ffn) {
  return E_r >= 1 && E_s >= 0 && T >= 1 && K >= 1 && K <= E_r && d_model >= 1 && d_ffn >= 1 &&
         E_r <= MOE_MAX_EXPERTS && E_s <= MOE_MAX_EXPERTS &&
         static_cast<long long>(T) * (K + E_s) <= INT32_MAX;
}

}  // namespace

size_t moe_experts_swiglu_workspace_size(int E_r, int E_s, int T, int K, int d_model, int d_ffn,
                                         moe_dtype dtype) {
  if (!experts_shape_ok(E_r, E_s, T, K, d_model, d_ffn) || !valid_dtype(dtype)) return 0;
  return experts_workspace_bytes(E_r, E_s, T, K, d_model, d_ffn, dtype);
}

moe_status moe_experts_swiglu(int E_r, int E_s, int T, int K, int d_model, int d_ffn,
                              const int32_t* offsets, const int32_t* row_token, const void* h,
                              moe_dtype dtype, const void* w_gate, const void* w_up,
                              const void* w_down, const void* ws_gate, const void* ws_up,
                              const void* ws_down, void* y, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const char* fn = "moe_experts_swiglu";
  if (!experts_shape_ok(E_r, E_s, T, K, d_model, d_ffn))
    return fail(MOE_ERR_INVALID_ARG,
                "%s: E_r=%d E_s=%d T=%d K=%d d_model=%d d_ffn=%d (need E_r, T, K, d_model, d_ffn "
                ">= 1, E_s >= 0, K <= E_r, E_r and E_s <= %d, T*(K+E_s) <= INT32_MAX)",
                fn, E_r, E_s, T, K, d_model, d_ffn, MOE_MAX_EXPERTS);
  if (!valid_dtype(dtype)) return fail(MOE_ERR_INVALID_ARG, "%s: bad dtype", fn);
  if (!offsets || !row_token || !h || !w_gate || !w_up || !w_down || !y || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (E_s > 0 && (!ws_gate || !ws_up || !ws_down))
    return fail(MOE_ERR_INVALID_ARG, "%s: null shared-expert weights with E_s=%d", fn, E_s);
  const int TK = T * K, rows = TK + E_s * T;
  const int align = dtype == MOE_BF16 ? 64 : 16;
  if (d_model % align || d_ffn % align)
    return fail(MOE_ERR_UNSUPPORTED, "%s: d_model=%d and d_ffn=%d must be multiples of %d", fn,
                d_model, d_ffn, align);
  if (static_cast<long long>(rows) * d_ffn > (1LL << 40) ||
      static_cast<long long>(d_model) * d_ffn > INT32_MAX)
    return fail(MOE_ERR_INVALID_ARG, "%s: sizes overflow", fn);
  if (dtype == MOE_BF16) {
    const long long lim = (1LL << 31) - 1;
    if (2LL * T * d_model > lim || 2LL * rows * d_ffn > lim || 2LL * d_model * d_ffn > lim)
      return fail(MOE_ERR_UNSUPPORTED,
                  "%s: bf16 operands must each be under 2 GiB "
                  "(h %lld, activations %lld, one weight matrix %lld bytes)",
                  fn, 2LL * T * d_model, 2LL * rows * d_ffn, 2LL * d_model * d_ffn);
    const int n_groups = moe::experts_layout(nullptr, E_r, E_s, T, K, d_ffn).n_groups;
    if (n_groups > moe::kMaxExpertGroups)
      return fail(MOE_ERR_UNSUPPORTED, "%s: %d row groups > %d (E_r=%d, E_s=%d)", fn, n_groups,
                  moe::kMaxExpertGroups, E_r, E_s);
  }
  const size_t need = experts_workspace_bytes(E_r, E_s, T, K, d_model, d_ffn, dtype);
  if (workspace_bytes < need)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  hipStream_t s = as_stream(stream);
  hipError_t err;
  if (dtype == MOE_BF16) {
    err = moe::launch_experts_bf16(
        E_r, E_s, T, K, d_model, d_ffn, offsets, row_token, static_cast<const uint16_t*>(h),
        static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up),
        static_cast<const uint16_t*>(w_down), static_cast<const uint16_t*>(ws_gate),
        static_cast<const uint16_t*>(ws_up), static_cast<const uint16_t*>(ws_down),
        static_cast<uint16_t*>(y), workspace, s);
    return hip_status(err, fn);
  }
  // fp32: the routed experts, then the shared ones, as two grouped launches
  const ExpertsF32Layout L = experts_f32_layout(workspace, E_r, E_s, T, K, d_model, d_ffn);
  err = moe::launch_experts_rows(T, K, E_s, row_token, L.row_index, L.sh_off, s);
  if (err == hipSuccess)
    err = moe::launch_swiglu_f32(E_r, d_model, d_ffn, TK, T, offsets, L.row_index,
                                 static_cast<const float*>(h), static_cast<const float*>(w_gate),
                                 static_cast<const float*>(w_up),
                                 static_cast<const float*>(w_down), nullptr,
                                 static_cast<float*>(y), L.ws, s);
  if (err == hipSuccess && E_s > 0)
    err = moe::launch_swiglu_f32(E_s, d_model, d_ffn, E_s * T, T, L.sh_off, L.row_index + TK,
                                 static_cast<const float*>(h), static_cast<const float*>(ws_gate),
                                 static_cast<const float*>(ws_up),
                                 static_cast<const float*>(ws_down), nullptr,
                                 static_cast<float*>(y) + static_cast<size_t>(TK) * d_model,
                                 L.ws, s);
  return hip_status(err, fn);
}

// ---- the form that allocates nothing: its workspace is one file-scope device
// array per GPU, found once per device with hipGetSymbolAddress.  In host code
// `scratch` only names the symbol; kernels get the address from g_scratch.

static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this GPU's scratch array (the current device's), looked up
// on the first call on that device.
moe_status scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device %d beyond %d devices", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    if (p == nullptr) return fail(MOE_ERR_HIP, "%s: scratch array has no device address", fn);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

moe_status moe_grouped_swiglu_noalloc(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                                      const int32_t* offsets, const int32_t* row_index,
                                      const void* x, moe_dtype dtype, const void* w_gate,
                                      const void* w_up, const void* w_down,
                                      const float* row_scale, void* y, void* stream) {
  const char* fn = "moe_grouped_swiglu_noalloc";
  const size_t cap = MOE_NOALLOC_SCRATCH_BYTES;
  if (n_groups >= 1 && d_model >= 1 && d_ffn >= 1 && rows >= 0 && valid_dtype(dtype)) {
    const size_t need =
        moe::swiglu_workspace_bytes(n_groups, d_model, d_ffn, rows, dtype == MOE_BF16);
    if (need > cap)
      return fail(MOE_ERR_UNSUPPORTED,
                  "%s: rows=%d x d_ffn=%d needs %zu bytes of scratch, more than the %zu this "
                  "form holds per GPU; call moe_grouped_swiglu with a workspace instead",
                  fn, rows, d_ffn, need, cap);
  }
  // every argument is checked before the scratch address is looked up
  void* const probe = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  moe_status st = grouped_swiglu(fn, n_groups, d_model, d_ffn, rows, x_rows, offsets, row_index,
                                 x, dtype, w_gate, w_up, w_down, row_scale, y, nullptr, probe, cap,
                                 stream, /*launch=*/false);
  if (st != MOE_OK) return st;
  void* ws = nullptr;
  st = scratch_address(fn, &ws);
  if (st != MOE_OK) return st;
  return grouped_swiglu(fn, n_groups, d_model, d_ffn, rows, x_rows, offsets, row_index, x, dtype,
                        w_gate, w_up, w_down, row_scale, y, nullptr, ws, cap, stream);
}

moe_status moe_grouped_swiglu_train(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                                    const int32_t* offsets, const int32_t* row_index,
                                    const void* x, moe_dtype dtype, const void* w_gate,
                                    const void* w_up, const void* w_down, const float* row_scale,
                                    void* y, void* au, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  const char* fn = "moe_grouped_swiglu_train";
  if (dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 only", fn);
  if (!au) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  return grouped_swiglu(fn, n_groups, d_model, d_ffn, rows, x_rows, offsets, row_index, x, dtype,
                        w_gate, w_up, w_down, row_scale, y, au, workspace, workspace_bytes,
                        stream);
}

moe_status moe_combine(int T, int d_model, int K, int E_s, const void* h, const void* y_shared,
                       const void* y_perm, const int32_t* slot_row, const float* gates,
                       moe_dtype dtype, void* y, void* stream) {
  if (T < 1 || d_model < 1 || K < 1 || E_s < 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: T=%d d_model=%d K=%d E_s=%d", T, d_model, K,
                E_s);
  if (K > MOE_MAX_TOPK) return fail(MOE_ERR_INVALID_ARG, "moe_combine: K=%d > %d", K, MOE_MAX_TOPK);
  if (!valid_dtype(dtype)) return fail(MOE_ERR_INVALID_ARG, "moe_combine: bad dtype");
  if (d_model % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "moe_combine: d_model=%d not a multiple of 8", d_model);
  if (!h || !y_perm || !slot_row || !gates || !y || (E_s > 0 && !y_shared))
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: null pointer");
  if (static_cast<long long>(T) * K > INT32_MAX)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: T*K overflows int32");
  return hip_status(moe::launch_combine(T, d_model, K, E_s, h, y_shared, y_perm, slot_row, gates,
                                        dtype == MOE_BF16, y, as_stream(stream)),
                    "moe_combine");
}

moe_status moe_bias_update(int T, int E_r, int K, float gamma, const int32_t* loads, float* b,
                           moe_bias_stats* stats, void* stream) {
  if (T < 1 || E_r < 1 || K < 1)
    return fail(MOE_ERR_INVALID_ARG, "moe_bias_update: T=%d E_r=%d K=%d must be >= 1", T, E_r, K);
  if (E_r > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "moe_bias_update: E_r=%d > %d", E_r, MOE_MAX_EXPERTS);
  if (!(gamma >= 0.0f) || gamma > 1e30f)
    return fail(MOE_ERR_INVALID_ARG, "moe_bias_update: gamma must be finite and >= 0");
  if (!loads || !b) return fail(MOE_ERR_INVALID_ARG, "moe_bias_update: null pointer");
  return hip_status(moe::launch_bias_update(T, E_r, K, gamma, loads, b,
                                            reinterpret_cast<moe::BiasStats*>(stats),
                                            as_stream(stream)),
                    "moe_bias_update");
}

moe_status moe_calib_mfma_loop(int workgroups, int iters, const void* operands, float* out,
                               double* flops, void* stream) {
  if (workgroups < 1 || iters < 1)
    return fail(MOE_ERR_INVALID_ARG, "moe_calib_mfma_loop: workgroups=%d iters=%d must be >= 1",
                workgroups, iters);
  if (workgroups > (1 << 20))
    return fail(MOE_ERR_INVALID_ARG, "moe_calib_mfma_loop: workgroups=%d > %d", workgroups, 1 << 20);
  if (!operands || !out) return fail(MOE_ERR_INVALID_ARG, "moe_calib_mfma_loop: null pointer");
  if (flops) *flops = moe::mfma_loop_flops(workgroups, iters);
  return hip_status(moe::launch_mfma_loop(workgroups, iters,
                                          static_cast<const uint16_t*>(operands), out,
                                          as_stream(stream)),
                    "moe_calib_mfma_loop");
}

moe_status moe_calib_stream_read(int workgroups, const void* src, size_t bytes, uint32_t* out,
                                 void* stream) {
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(MOE_ERR_INVALID_ARG, "moe_calib_stream_read: workgroups=%d outside 1..%d",
                workgroups, 1 << 20);
  if (!src || !out) return fail(MOE_ERR_INVALID_ARG, "moe_calib_stream_read: null pointer");
  if (bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_calib_stream_read: bytes (%zu) and src must be non-zero multiples of 16",
                bytes);
  return hip_status(moe::launch_stream_read(workgroups, src, bytes, out, as_stream(stream)),
                    "moe_calib_stream_read");
}

}  // extern "C"

// ---------------------------------------------------------------- profiling

namespace {

struct ProfRec {
  std::string name;
  hipEvent_t a, b;
  bool closed;
};

std::mutex g_prof_mu;
bool g_prof_on = false;
std::string g_prof_tag;
std::vector<std::string> g_prof_only;  // record only names containing one of these (empty: all)
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace moe {

int prof_begin(hipStream_t s, const char* name) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return -1;
  const std::string full = g_prof_tag + name;
  if (!g_prof_only.empty()) {
    bool hit = false;
    for (const std::string& f : g_prof_only) hit = hit || full.find(f) != std::string::npos;
    if (!hit) return -1;
  }
  hipEvent_t a = prof_event(), b = prof_event();
  if (!a || !b) return -1;
  if (hipEventRecord(a, s) != hipSuccess) return -1;
  g_prof_recs.push_back(ProfRec{full, a, b, false});
  return static_cast<int>(g_prof_recs.size()) - 1;
}

void prof_end(int token, hipStream_t s) {
  if (token < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (token >= static_cast<int>(g_prof_recs.size())) return;
  ProfRec& r = g_prof_recs[token];
  if (hipEventRecord(r.b, s) == hipSuccess) r.closed = true;
}

}  // namespace moe

extern "C" {

moe_status moe_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return MOE_OK;
}

moe_status moe_profile_only(const char* names) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_only.clear();
  if (names) {
    std::string cur;
    for (const char* c = names;; ++c) {
      if (*c == ',' || *c == '\0') {
        if (!cur.empty()) g_prof_only.push_back(cur);
        cur.clear();
        if (*c == '\0') break;
      } else {
        cur += *c;
      }
    }
  }
  return MOE_OK;
}

moe_status moe_profile_tag(const char* tag) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_tag = tag ? tag : "";
  return MOE_OK;
}

moe_status moe_profile_report(char* buf, size_t buf_bytes) {
  if (!buf || buf_bytes == 0) return fail(MOE_ERR_INVALID_ARG, "moe_profile_report: no buffer");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  struct Agg { int n = 0; double tot = 0, mn = 1e30, mx = 0; };
  std::map<std::string, Agg> agg;
  moe_status st = MOE_OK;
  for (ProfRec& r : g_prof_recs) {
    if (r.closed) {
      float ms = 0.0f;
      if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
        st = fail(MOE_ERR_HIP, "moe_profile_report: event query failed");
      } else {
        Agg& a = agg[r.name];
        a.n += 1;
        a.tot += ms;
        a.mn = std::min(a.mn, static_cast<double>(ms));
        a.mx = std::max(a.mx, static_cast<double>(ms));
      }
    }
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  std::string out;
  char line[256];
  for (auto& kv : agg) {
    snprintf(line, sizeof(line), "%s %d %.6f %.6f %.6f\n", kv.first.c_str(), kv.second.n,
             kv.second.tot, kv.second.mn, kv.second.mx);
    out += line;
  }
  if (out.size() + 1 > buf_bytes) return fail(MOE_ERR_INVALID_ARG, "moe_profile_report: buffer too small");
  memcpy(buf, out.c_str(), out.size() + 1);
  return st;
}

}  // extern "C"

namespace moe {
size_t swiglu_workspace_bytes(int n_groups, int d_model, int d_ffn, int rows, int bf16) {
  (void)d_model;
  return swiglu_layout(nullptr, n_groups, d_ffn, rows, bf16 ? 2 : 4, 32).bytes;
}
}  // namespace moe

// ---------------------------------------------------------------- backward

moe_status moe_transpose_experts(int n, int rows, int cols, const void* src, moe_dtype dtype,
                                 void* dst, int ld_dst, int col_offset, void* stream) {
  if (n < 1 || rows < 1 || cols < 1 || col_offset < 0 || ld_dst < rows + col_offset)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_transpose_experts: n=%d rows=%d cols=%d ld_dst=%d col_offset=%d", n, rows,
                cols, ld_dst, col_offset);
  if (n > 65535) return fail(MOE_ERR_UNSUPPORTED, "moe_transpose_experts: n=%d > 65535", n);
  if (dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "moe_transpose_experts: bf16 only");
  if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "moe_transpose_experts: null pointer");
  return hip_status(moe::launch_transpose_experts(n, rows, cols, static_cast<const uint16_t*>(src),
                                                  static_cast<uint16_t*>(dst), ld_dst, col_offset,
                                                  as_stream(stream)),
                    "moe_transpose_experts");
}

moe_status moe_combine_backward(int T, int d_model, int K, const void* dy, const void* y_perm,
                                const int32_t* slot_row, const float* gates, moe_dtype dtype,
                                void* dy_perm, float* dgates, void* stream) {
  if (T < 1 || d_model < 1 || K < 1 || K > MOE_MAX_TOPK)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine_backward: T=%d d_model=%d K=%d", T, d_model, K);
  if (static_cast<long long>(T) * K > INT32_MAX)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine_backward: T*K overflows int32");
  if (dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "moe_combine_backward: bf16 only");
  if (d_model % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "moe_combine_backward: d_model=%d must be a multiple of 8",
                d_model);
  if (static_cast<long long>(T) * K * d_model * 2 >= (1ll << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_combine_backward: y_perm exceeds 2 GiB");
  if (!dy || !y_perm || !slot_row || !gates || !dy_perm || !dgates)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine_backward: null pointer");
  return hip_status(moe::launch_combine_backward(T, d_model, K, static_cast<const uint16_t*>(dy),
                                                 static_cast<const uint16_t*>(y_perm), slot_row,
                                                 gates, static_cast<uint16_t*>(dy_perm), dgates,
                                                 as_stream(stream)),
                    "moe_combine_backward");
}

size_t moe_grouped_swiglu_backward_workspace_size(int n_groups, int d_model, int d_ffn,
                                                  int rows) {
  if (n_groups < 1 || d_model < 1 || d_ffn < 1 || rows < 0) return 0;
  return moe::bwd_workspace_bytes(n_groups, d_model, d_ffn, rows);
}

moe_status moe_grouped_swiglu_backward(int n_groups, int d_model, int d_ffn, int rows,
                                       int x_rows, const int32_t* offsets,
                                       const int32_t* row_index, const void* x, moe_dtype dtype,
                                       const void* w_gate, const void* w_up, const void* w_gu_t,
                                       const void* w_down_t, const void* dy, const void* au,
                                       void* dx, void* dw_gate, void* dw_up, void* dw_down,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_grouped_swiglu_backward";
  if (n_groups < 1 || d_model < 1 || d_ffn < 1 || rows < 0 || x_rows < 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: n_groups=%d d_model=%d d_ffn=%d rows=%d x_rows=%d", fn,
                n_groups, d_model, d_ffn, rows, x_rows);
  if (n_groups > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "%s: n_groups=%d > %d", fn, n_groups, MOE_MAX_EXPERTS);
  if (dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 only", fn);
  if (d_model % 64 != 0 || d_ffn % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: d_model and d_ffn must be multiples of 64", fn);
  if (!offsets || !x || !w_gate || !w_up || !w_gu_t || !w_down_t || !dy || !dx || !dw_gate ||
      !dw_up || !dw_down || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (row_index == nullptr && x_rows < rows)
    return fail(MOE_ERR_INVALID_ARG, "%s: x_rows=%d < rows=%d without row_index", fn, x_rows,
                rows);
  const size_t need = moe::bwd_workspace_bytes(n_groups, d_model, d_ffn, rows);
  if (workspace_bytes < need)
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  // every operand the kernels address through one buffer descriptor stays under
  // 2 GiB; one expert's transposed block holds at most d_model x (rows + 64)
  const long long two_gib = 1LL << 31;
  const long long mx = std::max(d_model, d_ffn);
  if (static_cast<long long>(rows) * 2 * d_ffn * 2 >= two_gib ||
      static_cast<long long>(rows) * d_model * 2 >= two_gib ||
      static_cast<long long>(x_rows) * d_model * 2 >= two_gib ||
      static_cast<long long>(d_model) * 2 * d_ffn * 2 >= two_gib ||
      mx * (static_cast<long long>(rows) + 64) * 2 >= two_gib)
    return fail(MOE_ERR_UNSUPPORTED, "%s: an operand is 2 GiB or larger", fn);
  if (rows == 0) return MOE_OK;
  return hip_status(
      moe::launch_swiglu_backward(n_groups, d_model, d_ffn, rows, x_rows, offsets, row_index,
                                  static_cast<const uint16_t*>(x),
                                  static_cast<const uint16_t*>(w_gate),
                                  static_cast<const uint16_t*>(w_up),
                                  static_cast<const uint16_t*>(w_gu_t),
                                  static_cast<const uint16_t*>(w_down_t),
                                  static_cast<const uint16_t*>(dy),
                                  static_cast<const uint16_t*>(au), static_cast<uint16_t*>(dx),
                                  static_cast<uint16_t*>(dw_gate), static_cast<uint16_t*>(dw_up),
                                  static_cast<uint16_t*>(dw_down), workspace, as_stream(stream)),
      fn);
}

moe_status moe_route_backward(int T, int d_model, int E_r, int K, moe_score_fn fn, const void* h,
                              moe_dtype h_dtype, const float* e, const int32_t* topk_idx,
                              const float* dgates, const int32_t* offsets,
                              const int32_t* row_token, float* dz, void* dh, float* de,
                              void* stream) {
  const char* nm = "moe_route_backward";
  if (T < 1 || d_model < 1 || E_r < 1 || K < 1 || K > E_r || K > MOE_MAX_TOPK)
    return fail(MOE_ERR_INVALID_ARG, "%s: T=%d d_model=%d E_r=%d K=%d", nm, T, d_model, E_r, K);
  if (E_r > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "%s: E_r=%d", nm, E_r);
  if (fn != MOE_SIGMOID && fn != MOE_SOFTMAX)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown score function %d", nm, (int)fn);
  if (h_dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 tokens only", nm);
  if (d_model % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "%s: d_model=%d must be a multiple of 8", nm, d_model);
  if (!h || !e || !topk_idx || !dgates || !offsets || !row_token || !dz || !dh || !de)
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", nm);
  if (static_cast<long long>(T) * K > INT32_MAX)
    return fail(MOE_ERR_INVALID_ARG, "%s: T*K overflows int32", nm);
  return hip_status(moe::launch_route_backward(T, d_model, E_r, K, (int)fn,
                                               static_cast<const uint16_t*>(h), e, topk_idx,
                                               dgates, offsets, row_token, dz,
                                               static_cast<uint16_t*>(dh), de, as_stream(stream)),
                    nm);
}

