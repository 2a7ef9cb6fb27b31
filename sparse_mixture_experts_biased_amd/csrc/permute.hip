// Dispatch: expert histogram, exclusive scan and the stable permutation of
// the T*K token copies (expert-major, ascending token inside an expert).
//
// Method: Sparse MoE routing-math page (arman1o1.github.io), section 3 (sort
// local tokens by target expert id; the layer listing collects each expert's
// token list in token order) and the Routing-and-Load-Balancing page
// (yiqiao-yin.github.io), section 5 (tokens are admitted in the order they
// appear).
//
// Three small kernels, no global atomics, so every output is deterministic:
//   1. per 256-token chunk, an LDS histogram of expert ids -> counts[chunk][e]
//   2. one workgroup: running sums over chunks per expert, exclusive scan over
//      experts -> offsets, and per-chunk segment bases
//   3. per chunk, an LDS bitmap bits[e][token in chunk]; the rank of token t
//      inside expert e's segment is the popcount of the bits below t.
//
// With a capacity C (routing-math page, section 3: C = ceil(CF*T*K/E_r)
// rows per expert; admission in token order per the routing-and-load-
// balancing page, section 5) the scan sums min(c_e, C) and a copy whose rank
// inside its expert is C or more is dropped (slot -1, no row).
#include "common.h"

namespace moe {
namespace {

constexpr int kChunk = kPermChunk;           // 256 tokens = 8 words per expert
constexpr int kWords = kChunk / 32;

__global__ __launch_bounds__(kChunk) void hist_kernel(int T, int E, int K,
                                                      const int32_t* __restrict__ idx,
                                                      int32_t* __restrict__ counts) {
  extern __shared__ int32_t cnt[];
  // the token's K ids loaded together (before any is used), then counted
  const int t = blockIdx.x * kChunk + threadIdx.x;
  int ex[MOE_MAX_TOPK_DEV];
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
    ex[k] = (t < T && k < K) ? idx[static_cast<size_t>(t) * K + k] : -1;
  for (int i = threadIdx.x; i < E; i += kChunk) cnt[i] = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
    if (ex[k] >= 0 && ex[k] < E) atomicAdd(&cnt[ex[k]], 1);
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += kChunk)
    counts[static_cast<size_t>(blockIdx.x) * E + i] = cnt[i];
}

// One workgroup of 1024 threads (E <= 1024).
// cap < 0: no capacity limit.
__global__ __launch_bounds__(1024) void scan_kernel(int E, int n_chunks, int TK, int cap,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ row_token) {
  __shared__ int32_t part[1024];
  __shared__ int32_t total_s;
  const int e = threadIdx.x;
  // chunk counts in batches of kB loads in flight (one at a time, every load
  // waited for the one before)
  constexpr int kB = 8;
  int tot = 0;
  if (e < E)
    for (int c0 = 0; c0 < n_chunks; c0 += kB) {
      int v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u)
        v[u] = c0 + u < n_chunks ? counts[static_cast<size_t>(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kB; ++u) tot += v[u];
    }
  if (cap >= 0) tot = min(tot, cap);  // kept rows of expert e
  // inclusive Hillis-Steele scan over experts
  part[e] = (e < E) ? tot : 0;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int v = (e >= off) ? part[e - off] : 0;
    __syncthreads();
    part[e] += v;
    __syncthreads();
  }
  const int excl = part[e] - ((e < E) ? tot : 0);
  if (e < E) offsets[e] = excl;
  if (e == 1023) {
    offsets[E] = part[1023];
    total_s = part[1023];
  }
  if (e < E) {
    int run = excl;
    for (int c0 = 0; c0 < n_chunks; c0 += kB) {
      int v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u)
        v[u] = c0 + u < n_chunks ? counts[static_cast<size_t>(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (c0 + u < n_chunks) {
          counts[static_cast<size_t>(c0 + u) * E + e] = run;
          run += v[u];
        }
    }
  }
  __syncthreads();
  for (int r = total_s + e; r < TK; r += 1024) row_token[r] = -1;
}

__global__ __launch_bounds__(kChunk) void assign_kernel(int T, int E, int K, int cap,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ base,
                                                        int32_t* __restrict__ row_token,
                                                        int32_t* __restrict__ slot_row) {
  extern __shared__ uint32_t bits[];  // [E][kWords]
  const int tl = threadIdx.x;
  const int t = blockIdx.x * kChunk + tl;
  const int w = tl / 32;
  const uint32_t bit = 1u << (tl % 32);
  // the token's K ids loaded together (before any is used)
  int exs[MOE_MAX_TOPK_DEV], bs[MOE_MAX_TOPK_DEV], os[MOE_MAX_TOPK_DEV];
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
    exs[k] = (t < T && k < K) ? idx[static_cast<size_t>(t) * K + k] : -1;
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
    if (exs[k] >= E) exs[k] = -1;
  for (int i = threadIdx.x; i < E * kWords; i += kChunk) bits[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k)
    if (exs[k] >= 0) atomicOr(&bits[exs[k] * kWords + w], bit);
  __syncthreads();
  if (t >= T) return;
  // the segment bases (and offsets) loaded before any store, so their loads
  // are in flight together
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) {
    const bool ok = k < K && exs[k] >= 0;
    bs[k] = ok ? base[static_cast<size_t>(blockIdx.x) * E + exs[k]] : 0;
    os[k] = (ok && cap >= 0) ? offsets[exs[k]] : 0;
  }
#pragma unroll
  for (int k = 0; k < MOE_MAX_TOPK_DEV; ++k) {
    if (k >= K) break;
    const size_t q = static_cast<size_t>(t) * K + k;
    const int ex = exs[k];
    if (ex < 0) {
      slot_row[q] = -1;
      continue;
    }
    const uint32_t* row = bits + ex * kWords;
    int rank = __popc(row[w] & (bit - 1u));
    for (int ww = 0; ww < w; ++ww) rank += __popc(row[ww]);
    const int slot = bs[k] + rank;
    if (cap >= 0 && slot - os[k] >= cap) {  // expert full: dropped
      slot_row[q] = -1;
      continue;
    }
    slot_row[q] = slot;
    row_token[slot] = t;
  }
}

// x_perm[r] = h[row_token[r]] for r < offsets[E]; one wave per row, 16-byte
// vectors.
__global__ __launch_bounds__(256) void gather_rows_kernel(int TK, int row_vecs, int T,
                                                          const int32_t* __restrict__ count,
                                                          const int32_t* __restrict__ row_token,
                                                          const uint4* __restrict__ src,
                                                          uint4* __restrict__ dst) {
  const int r = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (r >= TK) return;
  const int n = *count;
  const int t = (r < n) ? row_token[r] : -1;
  uint4* out = dst + static_cast<size_t>(r) * row_vecs;
  if (t < 0 || t >= T) {
    for (int c = lane; c < row_vecs; c += kWave) out[c] = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint4* in = src + static_cast<size_t>(t) * row_vecs;
  for (int c = lane; c < row_vecs; c += kWave) out[c] = in[c];
}

}  // namespace

size_t permute_workspace_bytes(int T, int E) {
  size_t n_chunks = (static_cast<size_t>(T) + kChunk - 1) / kChunk;
  return align_up(n_chunks * E * sizeof(int32_t), 256);
}

hipError_t launch_permute(int T, int d, int E, int K, int cap, const int32_t* idx,
                          const void* h, int elem_bytes, int32_t* offsets, int32_t* row_token,
                          int32_t* slot_row, void* x_perm, void* ws, hipStream_t s) {
  const int n_chunks = (T + kChunk - 1) / kChunk;
  const int TK = T * K;
  int32_t* counts = static_cast<int32_t*>(ws);
  {
    ProfScope prof_(s, "perm_hist");
    hipLaunchKernelGGL(hist_kernel, dim3(n_chunks), dim3(kChunk), E * sizeof(int32_t), s, T, E,
                       K, idx, counts);
  }
  {
    ProfScope prof_(s, "perm_scan");
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, E, n_chunks, TK, cap, counts,
                       offsets, row_token);
  }
  {
    ProfScope prof_(s, "perm_assign");
    hipLaunchKernelGGL(assign_kernel, dim3(n_chunks), dim3(kChunk),
                       static_cast<size_t>(E) * kWords * sizeof(uint32_t), s, T, E, K, cap, idx,
                       offsets, counts, row_token, slot_row);
  }
  if (x_perm != nullptr) {
    const int row_vecs = d * elem_bytes / 16;
    {
      ProfScope prof_(s, "perm_gather");
      hipLaunchKernelGGL(gather_rows_kernel, dim3((TK + 3) / 4), dim3(256), 0, s, TK, row_vecs,
                         T, offsets + E, row_token, static_cast<const uint4*>(h),
                         static_cast<uint4*>(x_perm));
    }
  }
  return hipGetLastError();
}

}  // namespace moe
