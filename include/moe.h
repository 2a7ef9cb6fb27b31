/*
 * moe.h -- C ABI of the single-GPU sparse Mixture-of-Experts layer forward
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (Sparse MoE routing-math page, arman1o1.github.io, section 0,
 * layer-output equation) is
 *
 *     y_t = h_t + sum_{j<E_s} SwiGLU^S_j(h_t) + sum_{i in I_t} g_{t,i} SwiGLU^R_i(h_t),
 *     SwiGLU(h) = (SiLU(h W_gate) * (h W_up)) W_down,
 *
 * with biased selection I_t = TopK({s_{t,i} + b_i}, K), unbiased gates
 * g_{t,i} = s_{t,i} / sum_{j in I_t} s_{t,j}, and the per-step bias update
 * b_i <- b_i + gamma * sign(cbar - c_i) (same page, section 2).
 *
 * Five entry points, called in this order for one layer forward:
 *   moe_route -> moe_permute -> moe_grouped_swiglu (routed, then shared)
 *   -> moe_combine -> moe_bias_update (training steps only).
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise.  The
 *     caller owns all memory; no entry point allocates or frees.
 *   - Matrices are row-major and densely packed.  Expert weights use the
 *     [out, in] layout of a linear layer: W_gate, W_up [n, d_ffn, d_model] and
 *     W_down [n, d_model, d_ffn], stacked over experts.
 *   - bf16 data is passed as raw 16-bit bfloat16 words; fp32 is IEEE binary32.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on that stream: it neither synchronises
 *     with the host nor copies data back to it.
 *   - Arguments are validated on the host before anything is launched.  A
 *     non-OK status means nothing was enqueued; moe_last_error() then returns
 *     a message for the calling thread.  Device-side contents (expert ids,
 *     offsets, row indices) are bounds-checked in the kernels: out-of-range
 *     entries are skipped, never dereferenced.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums are passed as 32-bit ints.  A C++ translation unit gives them that
 * fixed underlying type, so any int a caller passes is a value of the type and
 * the library's range checks on it are well defined. */
#ifdef __cplusplus
#define MOE_ENUM : int32_t
#else
#define MOE_ENUM
#endif

typedef enum MOE_ENUM {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, bad size, K > E_r, ...            */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but not built: shape alignment, dtype mix  */
  MOE_ERR_HIP = 3           /* the HIP runtime reported an error on launch      */
} moe_status;

typedef enum MOE_ENUM { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum MOE_ENUM {
  MOE_SIGMOID = 0,  /* s = sigmoid(z): DeepSeek-V3 affinity                      */
  MOE_SOFTMAX = 1   /* p = softmax(z) over all E_r experts: Mixtral / GShard     */
} moe_score_fn;

/* Load statistics written by moe_bias_update (device memory). */
typedef struct {
  int32_t max_load;  /* max_i c_i                                                */
  int32_t min_load;  /* min_i c_i                                                */
  float max_vio;     /* (max_i c_i - cbar) / cbar, cbar = K T / E_r              */
  int32_t reserved;
} moe_bias_stats;

/* Router balance diagnostics (forward values), filled by moe_router_diag. */
typedef struct {
  float switch_fP;     /* sum_i f_i P_i (times alpha_aux: the Switch auxiliary loss) */
  float z_loss;        /* (1/T) sum_t logsumexp(z_t)^2 (times c_z: the router z-loss) */
  float load_entropy;  /* -sum_i share_i log(max(share_i, 1e-9)), share = c / sum c  */
  float max_vio;       /* (max_i c_i - cbar) / cbar, cbar = K T / E_r              */
  float dropped;       /* 1 - kept copies / (T K); 0 when no dispatch is given     */
  float reserved[3];
} moe_router_diag_values;

#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16
/* Scratch of moe_grouped_swiglu_noalloc: one array of this size per GPU. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * moe_route -- router scores, biased top-K selection, unbiased gates, loads.
 *
 * Defined by: Sparse MoE routing-math page, section 2 (biased selection and
 * unbiased gate equations; sigmoid affinity s = sigma(h^T e)); section 1 and
 * its classical-router listing (softmax, top-K, renormalise, clamp 1e-12);
 * section 4 item 2 (router matmul and score function in fp32).
 *
 *   h        [T, d_model]   tokens, fp32 or bf16 (h_dtype)
 *   e        [E_r, d_model] fp32 expert centroids
 *   b        [E_r] fp32 selection bias, or NULL for b = 0 (softmax configs)
 *   topk_idx [T, K] int32 out: the K picked experts, ascending expert id
 *   gates    [T, K] fp32 out: g = s_i / max(sum_{j in I_t} s_j, 1e-12), the
 *            denominator summed in ascending expert id; aligned with topk_idx
 *   loads    [E_r] int32 out: c_i = #{t : i in I_t} (zeroed by this call)
 *
 *   workspace device scratch of at least moe_route_workspace_size() bytes
 *            (partial logits; 0 bytes and NULL allowed for fp32 tokens)
 *
 * z = h . e_i has fp32 accuracy (bf16 tokens: e split exactly into three bf16
 * parts on the matrix cores, fp32 accumulation; fp32 tokens: fp32 FMA); the
 * selection ranks v = fl32(s + b); equal v -> the lower expert id is picked.
 * With MOE_SOFTMAX and a non-NULL b, the bias is added to p.  Deterministic.
 * Limits: 1 <= K <= min(E_r, MOE_MAX_TOPK), E_r <= 512, d_model % 8 == 0
 * (bf16 tokens: d_model % 32 == 0 and d_model <= 2^20).
 */
size_t moe_route_workspace_size(int T, int d_model, int E_r, moe_dtype h_dtype);
moe_status moe_route(int T, int d_model, int E_r, int K, moe_score_fn fn,
                     const void* h, moe_dtype h_dtype, const float* e, const float* b,
                     int32_t* topk_idx, float* gates, int32_t* loads, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * moe_route_stats -- moe_route plus the per-batch router statistics the
 * diagnostics need, computed by the same kernels from the same fp32 logits.
 *
 * Defined by: Sparse MoE routing-math page, section 1 (Switch auxiliary loss:
 * P_i = (1/T) sum_t p_{t,i} with p = softmax(z); router z-loss: the mean of
 * logsumexp(z_t)^2).  For a sigmoid router p is still the softmax of z (the
 * Switch definition); the selection itself is unchanged.
 *
 *   p_mean    [E_r] fp32 out: P_i
 *   zsq_mean  [1] fp32 out: (1/T) sum_t logsumexp(z_t)^2
 *   workspace at least moe_route_stats_workspace_size() bytes (the routing
 *             scratch plus T*E_r + T floats of per-token values)
 * Every other argument is that of moe_route, with the same outputs and
 * errors; NULL p_mean or zsq_mean -> MOE_ERR_INVALID_ARG.  The token sums
 * run in a fixed order (deterministic).
 */
size_t moe_route_stats_workspace_size(int T, int d_model, int E_r, moe_dtype h_dtype);
moe_status moe_route_stats(int T, int d_model, int E_r, int K, moe_score_fn fn,
                           const void* h, moe_dtype h_dtype, const float* e, const float* b,
                           int32_t* topk_idx, float* gates, int32_t* loads, float* p_mean,
                           float* zsq_mean, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * moe_router_diag -- the router's balance diagnostics for one batch.
 *
 * Defined by: Sparse MoE routing-math page, section 1 (f_i = E_r/(K T) c_i,
 * the Switch product sum_i f_i P_i, minimised at 1 by uniform load; router
 * z-loss) and section 4 item 1 (MaxVio); the Mixture of Experts designs page,
 * router log (entropy of the load share, share clamped at 1e-9 in the log;
 * dropped-copy rate).
 *
 *   loads     [E_r] int32: c_i from moe_route / moe_route_stats
 *   p_mean, zsq_mean      from moe_route_stats
 *   offsets   [E_r + 1] int32 from moe_permute / moe_permute_capacity, or
 *             NULL (dropped = 0)
 *   f         [E_r] fp32 out f_i, or NULL
 *   diag      device moe_router_diag_values out
 * Errors: T, E_r, K < 1, K > E_r, E_r > MOE_MAX_EXPERTS or a NULL required
 * pointer -> MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED before any launch.
 * Deterministic (fixed-order reductions in one workgroup).
 */
moe_status moe_router_diag(int T, int E_r, int K, const int32_t* loads, const float* p_mean,
                           const float* zsq_mean, const int32_t* offsets, float* f,
                           moe_router_diag_values* diag, void* stream);

/*
 * moe_permute -- dispatch: expert histogram, exclusive scan, stable
 * permutation of the T*K token copies, and (optionally) the row gather.
 *
 * Defined by: Sparse MoE routing-math page, section 3 (sort local tokens by
 * target expert id; per-expert token lists of the layer listing, in token
 * order) and the Routing-and-Load-Balancing page, section 5 (admission in
 * token order).  No capacity limit: every copy is kept.
 *
 *   topk_idx  [T, K] int32 expert ids (entries outside [0, E_r) are skipped)
 *   h         [T, d_model] tokens (only read when x_perm != NULL)
 *   offsets   [E_r + 1] int32 out: exclusive scan of the loads;
 *             offsets[E_r] = number of kept copies (T*K for valid ids)
 *   row_token [T*K] int32 out: source token of permuted row r; rows inside an
 *             expert's segment are in ascending token order; entries past
 *             offsets[E_r] are set to -1
 *   slot_row  [T*K] int32 out: permuted row of copy (t, k) (-1 if skipped)
 *   x_perm    [T*K, d_model] out, or NULL: x_perm[r] = h[row_token[r]]
 *   workspace device scratch of at least moe_permute_workspace_size(T, E_r)
 *             bytes
 * Fully deterministic: no result depends on thread timing.
 */
size_t moe_permute_workspace_size(int T, int E_r);
moe_status moe_permute(int T, int d_model, int E_r, int K, const int32_t* topk_idx,
                       const void* h, moe_dtype dtype, int32_t* offsets, int32_t* row_token,
                       int32_t* slot_row, void* x_perm, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * moe_expert_capacity -- host helper: C = ceil(CF * T * K / E_r), the number
 * of rows one expert's buffer holds (Sparse MoE routing-math page, section 3,
 * expert buffer capacity equation), evaluated as ceil((CF * (T*K)) / E_r) in
 * IEEE double.  Returns -1 for T, K or E_r < 1, a negative or NaN factor, or a
 * result beyond INT32_MAX.  No device work.
 */
int moe_expert_capacity(int T, int K, int E_r, double capacity_factor);

/*
 * moe_permute_capacity -- moe_permute with a per-expert capacity: expert i
 * admits its copies in ascending token order until it holds `capacity` rows;
 * a later copy is dropped (the token keeps its residual, its shared experts
 * and its other routed experts; gates are not renormalised).
 *
 * Defined by: Sparse MoE routing-math page, section 3 (capacity C and token
 * dropping; the layer listing keeps the first C of each expert's token list)
 * and the Routing-and-Load-Balancing page, section 5 (admission in token
 * order, so the result depends on the batch order by design).
 *
 *   capacity  rows per expert, >= 0 (see moe_expert_capacity); otherwise
 *             MOE_ERR_INVALID_ARG
 *   offsets   [E_r + 1] int32 out: exclusive scan of min(c_i, capacity);
 *             offsets[E_r] = number of kept copies
 *   slot_row  [T*K] int32 out: permuted row of copy (t, k), or -1 when the
 *             copy was dropped (or its id is outside [0, E_r))
 * Every other argument, the outputs' layout, ownership and error behaviour
 * are those of moe_permute; the loads from moe_route stay the router's
 * counts (before any drop), which is what the bias update uses.
 */
moe_status moe_permute_capacity(int T, int d_model, int E_r, int K, int capacity,
                                const int32_t* topk_idx, const void* h, moe_dtype dtype,
                                int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                                void* x_perm, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * moe_grouped_swiglu -- one grouped SwiGLU over variable-size row groups:
 * group g runs expert g on rows offsets[g] .. offsets[g+1]-1.
 *
 * Defined by: Sparse MoE routing-math page, section 0 (SwiGLU expert) and
 * section 3 (all local experts in one grouped GEMM over variable-sized token
 * buckets); Expert-Parallelism page (mohakchugh.is-a.dev), inference section
 * (variable token counts per expert without padding).
 *
 *   n_groups   number of experts in this call (E_r for routed, E_s for shared)
 *   rows       size of the grouped row space (T*K routed, E_s*T shared)
 *   offsets    [n_groups + 1] int32 device: non-decreasing, offsets[0] = 0,
 *              offsets[n_groups] <= rows (clamped into [0, rows] on device)
 *   row_index  [rows] int32 device: grouped row r reads x[row_index[r]]
 *              (gather on load; entries outside [0, x_rows) give a zero row),
 *              or NULL: grouped row r reads x[r]
 *   x          [x_rows, d_model] input rows, fp32 or bf16 (dtype)
 *   w_gate, w_up [n_groups, d_ffn, d_model]; w_down [n_groups, d_model, d_ffn]
 *   row_scale  [rows] fp32 per-row output factor (a gate), or NULL (= 1)
 *   y          [rows, d_model] out: SwiGLU_g(x_row) * row_scale; rows past
 *              offsets[n_groups] are not written
 *   workspace  device scratch of at least moe_grouped_swiglu_workspace_size()
 *              bytes (the SiLU(gate)*up activations and the tile list)
 * bf16: fp32 accumulation on the matrix cores; the activation is rounded to
 * bf16 before W_down and y to bf16 (round to nearest even).
 * Limits: bf16 needs d_model % 64 == 0, d_ffn % 64 == 0 and each of x, the
 * activations [rows, d_ffn] and one expert's weight matrix under 2 GiB; fp32
 * needs d_model % 16 == 0 and d_ffn % 16 == 0.
 */
size_t moe_grouped_swiglu_workspace_size(int n_groups, int d_model, int d_ffn, int rows,
                                         moe_dtype dtype);
moe_status moe_grouped_swiglu(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                              const int32_t* offsets, const int32_t* row_index,
                              const void* x, moe_dtype dtype, const void* w_gate,
                              const void* w_up, const void* w_down, const float* row_scale,
                              void* y, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * moe_experts_swiglu -- the routed and the shared experts of one layer in one
 * grouped launch per product (gate/up, then down).
 *
 * Defined by: Sparse MoE routing-math page, section 0 (layer output: the
 * always-active shared experts beside the gated routed experts; SwiGLU
 * expert) and section 3 (all local experts in one grouped GEMM over
 * variable-sized token buckets).  The same per-row results as
 * moe_grouped_swiglu on the routed rows followed by moe_grouped_swiglu on the
 * shared rows; one launch lets the shared experts' matrix-core work run on
 * the CUs beside the routed experts' weight streaming.
 *
 *   E_r, E_s   routed and shared experts (E_s = 0 allowed)
 *   T, K       tokens and picks per token
 *   offsets    [E_r + 1] int32 device, from moe_permute / moe_permute_capacity
 *   row_token  [T*K] int32 device, from the same call
 *   h          [T, d_model] tokens, fp32 or bf16 (dtype)
 *   w_gate, w_up [E_r, d_ffn, d_model]; w_down [E_r, d_model, d_ffn]
 *   ws_gate, ws_up [E_s, d_ffn, d_model]; ws_down [E_s, d_model, d_ffn]
 *              (may be NULL when E_s = 0)
 *   y          [T*K + E_s*T, d_model] out: rows 0 .. T*K-1 are y_perm (routed
 *              row r = expert output for row_token[r]; rows past offsets[E_r]
 *              are not written), then shared expert j's output for token t at
 *              row T*K + j*T + t -- so y + T*K*d_model is moe_combine's
 *              y_shared and y its y_perm
 *   workspace  device scratch of at least moe_experts_swiglu_workspace_size()
 *              bytes (the combined row index, activations, tile list)
 * bf16: fp32 accumulation on the matrix cores, activations and y rounded to
 * bf16; fp32 runs the two sets of experts as two grouped launches.
 * Limits: those of moe_grouped_swiglu with rows = T*K + E_s*T and x = h;
 * E_r, E_s <= MOE_MAX_EXPERTS; bf16 also needs E_r + 8*E_s row groups or
 * fewer, at most 2048 (MOE_ERR_UNSUPPORTED otherwise; separate
 * moe_grouped_swiglu calls then serve).
 */
size_t moe_experts_swiglu_workspace_size(int E_r, int E_s, int T, int K, int d_model, int d_ffn,
                                         moe_dtype dtype);
moe_status moe_experts_swiglu(int E_r, int E_s, int T, int K, int d_model, int d_ffn,
                              const int32_t* offsets, const int32_t* row_token, const void* h,
                              moe_dtype dtype, const void* w_gate, const void* w_up,
                              const void* w_down, const void* ws_gate, const void* ws_up,
                              const void* ws_down, void* y, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * moe_grouped_swiglu_noalloc -- moe_grouped_swiglu that allocates nothing, for
 * callers that cannot allocate device memory or take a workspace: code under
 * HIP graph capture, tight serving loops (decode-sized batches), harnesses
 * that forbid hipMalloc.
 *
 * The same computation, outputs and argument meanings as moe_grouped_swiglu,
 * without the workspace arguments: its scratch (the activations and the tile
 * list) is a device array of MOE_NOALLOC_SCRATCH_BYTES (32 MiB) inside the
 * library, one per GPU, loaded with the library's code on that GPU and held
 * until the process ends.  Its device address is looked up on the first call
 * on each device (hipGetSymbolAddress, which may load the library's code on
 * that device); later calls only launch.  Calls no hipMalloc or hipFree.
 *
 * The current device must be the stream's device.  Every call on one GPU
 * uses that GPU's one array: calls that overlap on one GPU (on different
 * streams, or from several threads) race and give wrong results; calls in
 * order on one stream are safe.  Nothing in the array has to start at zero.
 *
 * Errors: the arguments are checked as for moe_grouped_swiglu, before any
 * launch; a call whose scratch need (moe_grouped_swiglu_workspace_size)
 * exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_UNSUPPORTED with the
 * sizes in moe_last_error() -- e.g. at d_ffn = 2048 (bf16) up to about 8000
 * grouped rows fit.
 */
moe_status moe_grouped_swiglu_noalloc(int n_groups, int d_model, int d_ffn, int rows,
                                      int x_rows, const int32_t* offsets,
                                      const int32_t* row_index, const void* x, moe_dtype dtype,
                                      const void* w_gate, const void* w_up, const void* w_down,
                                      const float* row_scale, void* y, void* stream);

/*
 * moe_grouped_swiglu_train -- moe_grouped_swiglu for a training forward pass:
 * the same outputs, and the gate and up projections of every grouped row
 * (SwiGLU expert, routing-math page section 0) kept for the backward pass.
 *
 *   au   [rows, 2 d_ffn] bf16 out: row r holds a_r = x_r W_gate^T in
 *        columns 0 .. d_ffn-1 and u_r = x_r W_up^T in d_ffn .. 2 d_ffn-1,
 *        each rounded to bf16 from the fp32 accumulator; rows past
 *        offsets[n_groups] are not written.  Caller-owned; pass it to
 *        moe_grouped_swiglu_backward, which then skips recomputing them.
 * Every other argument, the workspace size and the limits are those of
 * moe_grouped_swiglu; bf16 only (else MOE_ERR_UNSUPPORTED); au NULL gives
 * MOE_ERR_INVALID_ARG.  Costs the writes of au (4 rows d_ffn bytes).
 */
moe_status moe_grouped_swiglu_train(int n_groups, int d_model, int d_ffn, int rows, int x_rows,
                                    const int32_t* offsets, const int32_t* row_index,
                                    const void* x, moe_dtype dtype, const void* w_gate,
                                    const void* w_up, const void* w_down, const float* row_scale,
                                    void* y, void* au, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * moe_combine -- gate-weighted sum of the expert outputs plus the residual and
 * the shared experts:
 *     y_t = h_t + sum_{j<E_s} y_shared[j, t] + sum_k gates[t,k] * y_perm[slot_row[t*K+k]]
 *
 * Defined by: Sparse MoE routing-math page, section 0 (layer-output equation)
 * and section 3 (un-permute and accumulate the gate-weighted sum).
 *
 *   h        [T, d_model], y_shared [E_s, T, d_model] (NULL when E_s == 0),
 *   y_perm   [T*K, d_model], all in `dtype`
 *   slot_row [T*K] int32 (entries outside [0, T*K) contribute nothing)
 *   gates    [T, K] fp32
 *   y        [T, d_model] out (dtype), fp32 accumulation in a fixed order,
 *            bf16 output rounded to nearest even.  Deterministic.
 * Limits: d_model % 8 == 0; T*K <= INT32_MAX.  y_perm may be any size (each
 * gathered row is addressed from its own base).
 */
moe_status moe_combine(int T, int d_model, int K, int E_s, const void* h,
                       const void* y_shared, const void* y_perm, const int32_t* slot_row,
                       const float* gates, moe_dtype dtype, void* y, void* stream);

/*
 * moe_bias_update -- auxiliary-loss-free bias step after the loads of the
 * batch are counted:  b_i <- b_i + gamma * sign(cbar - c_i), cbar = K T / E_r.
 *
 * Defined by: Sparse MoE routing-math page, section 2 (bias update equation);
 * Mixture of Experts designs page (raminaeye.github.io), section 1 worked
 * example (sign 0 leaves a bias unchanged); section 4 item 1 of the
 * routing-math page (MaxVio).
 *
 *   loads [E_r] int32 (from moe_route);  b [E_r] fp32, updated in place
 *   stats device moe_bias_stats out, or NULL
 * The sign is decided in integers (K*T vs E_r*c_i); the update is one fp32
 * add of +gamma, -gamma or 0, so it is bit-reproducible.  gamma = 0 freezes b.
 */
moe_status moe_bias_update(int T, int E_r, int K, float gamma, const int32_t* loads, float* b,
                           moe_bias_stats* stats, void* stream);

/*
 * Optional kernel timing (benchmarking aid, not needed for the layer).
 * moe_profile_enable(1): from then on every kernel the library launches is
 * bracketed by a pair of hipEvents recorded on the stream it runs on.
 * moe_profile_report waits for the recorded events, writes one text line per
 * kernel name -- "name launches total_ms min_ms max_ms" -- into the host
 * buffer `buf` (NUL-terminated) and clears the records.  Returns
 * MOE_ERR_INVALID_ARG if the buffer is too small.  Events are created once and
 * reused; no device memory is allocated.
 */
moe_status moe_profile_enable(int on);
/* Prefix for the names of the records that follow (host string, copied;
 * NULL or "" clears it), e.g. to tell the routed and the shared grouped
 * SwiGLU calls apart. */
moe_status moe_profile_tag(const char* tag);
/* Restricts the records to kernels whose name (with its tag prefix) contains
 * one of the comma-separated substrings in `names` (host string, copied), so
 * that a timed run brackets only the launches it reports; NULL or "" records
 * every kernel again.  The other launches then carry no events at all. */
moe_status moe_profile_only(const char* names);
moe_status moe_profile_report(char* buf, size_t buf_bytes);

/*
 * Measurement aid, not part of the layer: the bf16 matrix-core rate with no
 * memory traffic, against which the grouped SwiGLU's matrix-core fraction is
 * read.  `workgroups` workgroups of 256 threads; every wave issues, `iters`
 * times, the MFMA sequence of one wave of the grouped SwiGLU tile over two
 * k-steps (2 x 4 blocks of v_mfma_f32_32x32x16_bf16 each, 8 independent
 * accumulators) on two sets of fragments held in registers.
 *   operands  device, workgroups * 256 * 96 bf16 values (random in practice;
 *             each thread loads its own 192 bytes once)
 *   out       device, workgroups * 256 floats (sums of the accumulators, so the
 *             work cannot be dropped)
 *   flops     host, or NULL: receives the FLOPs the launch performs
 * Asynchronous on `stream`; time it with events on that stream.
 * MOE_ERR_INVALID_ARG for workgroups or iters < 1, workgroups > 2^20 or a
 * null device pointer.
 */
moe_status moe_calib_mfma_loop(int workgroups, int iters, const void* operands, float* out,
                               double* flops, void* stream);

/*
 * Measurement aid, not part of the layer: the HBM read rate a plain streaming
 * kernel reaches, against which the weight-streaming kernels are read.
 * `workgroups` workgroups of 256 threads read the `bytes` at device pointer
 * `src` once in 16-byte vectors (grid-stride, eight loads in flight per thread)
 * and write one folded word per thread to `out` (device, workgroups * 256
 * uint32).  MOE_ERR_INVALID_ARG for workgroups outside 1..2^20, a null
 * pointer, or bytes / src not non-zero multiples of 16.
 */
moe_status moe_calib_stream_read(int workgroups, const void* src, size_t bytes, uint32_t* out,
                                 void* stream);

/* Message for the last non-OK status returned on the calling thread. */
const char* moe_last_error(void);

/* Library version string (host memory, static). */
const char* moe_version(void);

/* ================================================================ backward
 *
 * Gradients of a loss L through the layer output y (dy = dL/dy), with the
 * routing decisions of the forward pass fixed.  Defined by the chain rule on
 * the Sparse MoE routing-math page's layer-output, SwiGLU, gate and score
 * equations (sections 0 and 2); the gate gradient reaches the router only
 * through the unbiased scores s, and the bias b gets none (section 2: it
 * decides the selection only).  bf16 operands, fp32 accumulation; gradients
 * are written in bf16 (weights) or fp32 (centroids, gates, logits).
 *
 * One backward step, after a forward with the same buffers:
 *   moe_combine_backward          dy -> dy_perm (g * dy per copy), dgates
 *   moe_grouped_swiglu_backward   routed experts: dy_perm -> dx_perm, dW
 *   moe_grouped_swiglu_backward   shared experts: dy -> dx_shared, dW_shared
 * (the forward's expert calls may be moe_grouped_swiglu_train, whose a|u
 * output the backward then reads instead of recomputing)
 *   moe_combine (gates = 1)       dh = dy + sum dx_shared + sum_k dx_perm
 *   moe_route_backward            dh += router term; de
 */

/*
 * moe_transpose_experts -- dst[i][c][col_offset + r] = src[i][r][c] for n
 * matrices [rows, cols] (bf16).  Builds the transposed weight copies the
 * backward takes: W_down^T [E, d_ffn, d_model] (rows = d_model, cols = d_ffn,
 * ld_dst = d_model, col_offset 0) and [W_gate^T | W_up^T] [E, d_model,
 * 2 d_ffn] (two calls, ld_dst = 2 d_ffn, col_offset 0 and d_ffn).
 * ld_dst >= rows + col_offset, else MOE_ERR_INVALID_ARG.
 */
moe_status moe_transpose_experts(int n, int rows, int cols, const void* src, moe_dtype dtype,
                                 void* dst, int ld_dst, int col_offset, void* stream);

/*
 * moe_combine_backward -- gradients of y_t = h_t + sum_j y_shared[j, t] +
 * sum_k g_{t,k} y_perm[slot_row[t,k]] (routing-math page, section 0):
 *   dy_perm [T*K, d_model] out: row slot_row[t,k] = g_{t,k} dy_t (rows of
 *           dropped copies are not written)
 *   dgates  [T, K] fp32 out: <dy_t, y_perm[slot_row[t,k]]> (0 when dropped)
 * The residual and the shared experts receive dy itself.  bf16 only, d_model
 * a multiple of 8, y_perm under 2 GiB (else MOE_ERR_UNSUPPORTED).
 */
moe_status moe_combine_backward(int T, int d_model, int K, const void* dy, const void* y_perm,
                                const int32_t* slot_row, const float* gates, moe_dtype dtype,
                                void* dy_perm, float* dgates, void* stream);

/*
 * moe_grouped_swiglu_backward -- backward of moe_grouped_swiglu (without a
 * row scale): with a = x W_gate^T, u = x W_up^T, act = SiLU(a) u per group,
 *   d act = dy W_down;  da = d act * u * SiLU'(a);  du = d act * SiLU(a)
 *   dx = da W_gate + du W_up;  dW_down = dy^T act;  dW_gate = da^T x;
 *   dW_up = du^T x,   SiLU'(a) = sigma(a) (1 + a (1 - sigma(a))).
 *
 *   offsets, row_index, x, w_gate, w_up  as in the forward call
 *   w_gu_t    [n_groups, d_model, 2 d_ffn] [W_gate^T | W_up^T]
 *   w_down_t  [n_groups, d_ffn, d_model] W_down^T
 *   dy        [rows, d_model] gradient of the grouped outputs
 *   au        [rows, 2 d_ffn] bf16 [a | u] as written by
 *             moe_grouped_swiglu_train with the same x, weights and
 *             offsets, or NULL: the backward recomputes them (two more
 *             grouped products) into its workspace
 *   dx        [rows, d_model] out: gradient of each grouped row's input
 *   dw_gate, dw_up [n_groups, d_ffn, d_model] out; dw_down [n_groups,
 *             d_model, d_ffn] out; groups without rows get zeros
 *   workspace at least moe_grouped_swiglu_backward_workspace_size() bytes
 * bf16 only; d_model and d_ffn multiples of 64; every operand addressed
 * through one buffer descriptor under 2 GiB (else MOE_ERR_UNSUPPORTED).
 */
size_t moe_grouped_swiglu_backward_workspace_size(int n_groups, int d_model, int d_ffn,
                                                  int rows);
moe_status moe_grouped_swiglu_backward(int n_groups, int d_model, int d_ffn, int rows,
                                       int x_rows, const int32_t* offsets,
                                       const int32_t* row_index, const void* x, moe_dtype dtype,
                                       const void* w_gate, const void* w_up, const void* w_gu_t,
                                       const void* w_down_t, const void* dy, const void* au,
                                       void* dx, void* dw_gate, void* dw_up, void* dw_down,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route_backward -- gradient of the gates g_{t,k} w.r.t. the router:
 * sigmoid: g_i = s_i / S, S = sum_{j in I_t} s_j: dz_i = (dg_i - sum_j g_j
 * dg_j) / S * s_i (1 - s_i); softmax renormalised over the picks: dz_i =
 * g_i (dg_i - sum_j g_j dg_j).  The logits of the picks are recomputed in fp32.
 *
 *   topk_idx, h, e   as in the forward moe_route call (bf16 tokens)
 *   dgates    [T, K] fp32 from moe_combine_backward
 *   offsets, row_token  the dispatch of every pick (moe_permute, no capacity)
 *   dz        [T, K] fp32 out: dL/dz of the picks
 *   dh        [T, d_model] in/out (bf16): dh_t += sum_k dz_{t,k} e_{idx[t,k]}
 *   de        [E_r, d_model] fp32 out: sum over picks of dz h_t (fixed order)
 * bf16 tokens, d_model a multiple of 8 (else MOE_ERR_UNSUPPORTED).
 */
moe_status moe_route_backward(int T, int d_model, int E_r, int K, moe_score_fn fn, const void* h,
                              moe_dtype h_dtype, const float* e, const int32_t* topk_idx,
                              const float* dgates, const int32_t* offsets,
                              const int32_t* row_token, float* dz, void* dh, float* de,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
