"""CPU oracle for the single-GPU sparse MoE layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only the tests, the smoke check and the CPU-baseline leg of the benchmark call
it.  It shares no code with the HIP library.

Plain NumPy, written from the method's definitions, one function per step:

  * Sparse MoE routing-math page (arman1o1.github.io), section 0, layer-output
    equation: y_t = h_t + sum_j SwiGLU^S_j(h_t) + sum_{i in TopK} g_{t,i} SwiGLU^R_i(h_t),
    with SwiGLU(h) = (SiLU(h W_gate) * (h W_up)) W_down.
  * Same page, section 2, biased selection and unbiased gate:
    I_t = TopK({s_{t,i} + b_i}, K), g_{t,i} = s_{t,i} / sum_{j in I_t} s_{t,j};
    bias update b_i <- b_i + gamma * sign(cbar - c_i), c_i = #{t : i in I_t},
    cbar = K T / E_r.
  * Same page, section 1 and its classical-router listing: softmax router,
    top-K of p, renormalised over the picked experts, clamp 1e-12.
  * Same page, section 4, item 2: router matmul and score function in fp32.
  * Same page, section 4, item 1: MaxVio = (max_i c_i - cbar) / cbar.
  * Same page, section 3: sort token copies by expert, run each expert on its
    rows, weight by the gate, add back; with a capacity factor CF, expert
    buffers hold C = ceil(CF * T * K / E_r) rows and a copy routed to a full
    expert is dropped (the token keeps only its residual and other experts).
  * Routing-and-load-balancing page (yiqiao-yin.github.io), section 5: tokens
    are admitted to an expert in the order they appear.
  * Backward pass of the layer (gradients of a loss through y, with the
    routing decisions I_t fixed): the chain rule applied to the layer-output,
    SwiGLU, gate and score equations above.  The gate gradient reaches the
    router only through the unbiased scores s (routing-math page, section 2:
    the bias decides the selection only, so it receives no gradient).
  * Router diagnostics (forward values): routing-math page, section 1 (Switch
    auxiliary loss f_i P_i with f_i = E_r/(K T) * #{t : i in I_t} and
    P_i = mean_t p_{t,i}; router z-loss = mean_t logsumexp(z_t)^2) and the
    designs page (raminaeye.github.io), per-layer log: MaxVio, dropped-copy
    rate and the entropy of the load share (share clamped at 1e-9 in the log).

Precision.  The pages fix the router at fp32: z is the fp64 dot product of
the exact inputs rounded once to fp32, s = sigma(z) is evaluated in fp64 and
rounded to fp32, and the selection compares fp32 values v = fl32(s + b).  The
expert math, the gates and the combine are fp64.  The bias update is one fp32
add of +-gamma or 0, with the sign decided in integers (K*T vs E_r*c_i).

Readings where the pages are silent (each listed in the design notes):
  * ties in v: the lower expert index wins;
  * topk_idx is reported in ascending expert id (a canonical order);
  * the gate denominator is summed in ascending expert id;
  * sign(0) = 0, so an expert exactly at the fair share keeps its bias;
  * inside an expert's segment, rows are in ascending token order;
  * for softmax + bias (no workload uses it) the bias is added to p.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence, Tuple, Union

import numpy as np

GATE_CLAMP = 1e-12


# ---------------------------------------------------------------- inputs

def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact fp64 values of a bf16 (uint16 bit patterns) or fp32 array."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.dtype == np.float32 or x.dtype == np.float64:
        return x.astype(np.float64)
    raise TypeError(f"unsupported input dtype {x.dtype}")


# ---------------------------------------------------------------- router

def router_logits(h: np.ndarray, e: np.ndarray) -> np.ndarray:
    """z_{t,i} = h_t . e_i, fp64 accumulation rounded once to fp32.  [T, E_r]"""
    return (to_f64(h) @ to_f64(e).T).astype(np.float32)


def sigmoid_scores(z: np.ndarray) -> np.ndarray:
    """s = 1 / (1 + exp(-z)), evaluated in fp64, rounded to fp32."""
    z64 = z.astype(np.float64)
    return (1.0 / (1.0 + np.exp(-z64))).astype(np.float32)


def softmax_scores(z: np.ndarray) -> np.ndarray:
    """p = exp(z - max z) / sum exp(z - max z) over all E_r, fp64, rounded to fp32."""
    z64 = z.astype(np.float64)
    ez = np.exp(z64 - z64.max(axis=-1, keepdims=True))
    return (ez / ez.sum(axis=-1, keepdims=True)).astype(np.float32)


def scores(z: np.ndarray, fn: str) -> np.ndarray:
    if fn == "sigmoid":
        return sigmoid_scores(z)
    if fn == "softmax":
        return softmax_scores(z)
    raise ValueError(fn)


def biased_values(s: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """v = fl32(s + b): the values the selection ranks (b absent -> v = s)."""
    if b is None:
        return s.astype(np.float32)
    return (s.astype(np.float32) + b.astype(np.float32)[None, :]).astype(np.float32)


def biased_topk(s: np.ndarray, b: Optional[np.ndarray], K: int) -> np.ndarray:
    """I_t = the K largest v_{t,i}; equal v -> lower i first.

    Returned as int32 [T, K] in ascending expert id.
    """
    v = biased_values(s, b)
    order = np.argsort(-v, axis=-1, kind="stable")  # descending v, ties by lower index
    return np.sort(order[:, :K], axis=-1).astype(np.int32)


def topk_margin(s: np.ndarray, b: Optional[np.ndarray], K: int) -> np.ndarray:
    """v_(K) - v_(K+1) per token (inf when K == E_r): small margins are near-ties."""
    v = biased_values(s, b).astype(np.float64)
    if K >= v.shape[1]:
        return np.full(v.shape[0], np.inf)
    srt = -np.sort(-v, axis=-1)
    return srt[:, K - 1] - srt[:, K]


def gates(s: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g_{t,k} = s_{t,idx[t,k]} / max(sum over the picked experts, 1e-12), fp32 out.

    The denominator is accumulated over the picked experts in ascending id.
    """
    picked = np.take_along_axis(s.astype(np.float64), idx.astype(np.int64), axis=-1)
    den = np.zeros(picked.shape[0], dtype=np.float64)
    for k in range(picked.shape[1]):
        den = den + picked[:, k]
    den = np.maximum(den, GATE_CLAMP)
    return (picked / den[:, None]).astype(np.float32)


def load_count(idx: np.ndarray, E_r: int) -> np.ndarray:
    """c_i = #{t : i in I_t} as int32 [E_r]."""
    return np.bincount(idx.reshape(-1).astype(np.int64), minlength=E_r).astype(np.int32)


def route(h, e, b, K: int, fn: str):
    """Router + biased top-K + unbiased gates + load count (one layer call)."""
    z = router_logits(h, e)
    s = scores(z, fn)
    idx = biased_topk(s, b, K)
    g = gates(s, idx)
    c = load_count(idx, e.shape[0])
    return dict(z=z, s=s, idx=idx, gates=g, loads=c)


# ---------------------------------------------------------------- dispatch

def permute(idx: np.ndarray, E_r: int):
    """Expert-sorted order of the T*K token copies.

    offsets[E_r + 1]: exclusive scan of the loads; inside expert i's segment the
    rows are in ascending token order.  row_token[r] is the source token of
    permuted row r; slot_row[t*K + k] is the permuted row of copy (t, k).
    """
    T, K = idx.shape
    c = load_count(idx, E_r)
    offsets = np.zeros(E_r + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(c)
    flat_e = idx.reshape(-1).astype(np.int64)
    flat_t = np.repeat(np.arange(T, dtype=np.int64), K)
    order = np.lexsort((flat_t, flat_e))          # by expert, then by token
    row_token = flat_t[order]
    slot_row = np.empty(T * K, dtype=np.int64)
    slot_row[order] = np.arange(T * K, dtype=np.int64)
    return offsets.astype(np.int32), row_token.astype(np.int32), slot_row.astype(np.int32)


def expert_capacity(T: int, K: int, E_r: int, cf: float) -> int:
    """C = ceil(CF * T * K / E_r), evaluated as ceil((cf * (T*K)) / E_r) in
    IEEE double."""
    return int(math.ceil(float(cf) * float(T * K) / float(E_r)))


def permute_capacity(idx: np.ndarray, E_r: int, C: int):
    """Capacity-bounded dispatch: expert i admits its copies in ascending token
    order until it holds C rows; later copies are dropped.

    Returns (offsets over the kept rows, row_token of the kept rows, slot_row
    with -1 for a dropped copy, kept count per expert).
    """
    T, K = idx.shape
    kept = np.zeros(E_r, dtype=np.int64)
    lists = [[] for _ in range(E_r)]           # admitted (t, k) per expert
    slot_row = np.full(T * K, -1, dtype=np.int64)
    for t in range(T):                          # arrival order
        for k in range(K):
            i = int(idx[t, k])
            if kept[i] < C:
                lists[i].append(t * K + k)
                kept[i] += 1
    offsets = np.zeros(E_r + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    row_token = np.empty(int(offsets[-1]), dtype=np.int64)
    for i in range(E_r):
        for j, q in enumerate(lists[i]):
            r = offsets[i] + j
            row_token[r] = q // K
            slot_row[q] = r
    return (offsets.astype(np.int32), row_token.astype(np.int32), slot_row.astype(np.int32),
            kept.astype(np.int32))


# ---------------------------------------------------------------- experts

def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x * sigma(x)."""
    return x / (1.0 + np.exp(-x))


def swiglu(x, w_gate, w_up, w_down) -> np.ndarray:
    """(SiLU(x W_gate^T) * (x W_up^T)) W_down^T in fp64; weights in [out, in] layout."""
    x64 = to_f64(x) if x.dtype != np.float64 else x
    a = x64 @ to_f64(w_gate).T
    u = x64 @ to_f64(w_up).T
    return (silu(a) * u) @ to_f64(w_down).T


ExpertSource = Union[Sequence, Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]]


def _expert(weights: ExpertSource, i: int):
    if callable(weights):
        return weights(i)
    wg, wu, wd = weights
    return wg[i], wu[i], wd[i]


def grouped_swiglu(x: np.ndarray, offsets: np.ndarray, row_index: Optional[np.ndarray],
                   weights: ExpertSource, groups: Optional[Sequence[int]] = None) -> np.ndarray:
    """Run expert g on rows offsets[g]:offsets[g+1] of the grouped input.

    Grouped row r reads x[row_index[r]] (or x[r] when row_index is None).
    Returns fp64 [rows, d_model]; rows of groups not listed in `groups` stay 0.
    """
    rows = int(offsets[-1])
    x64 = to_f64(x)
    src = np.arange(rows) if row_index is None else row_index.astype(np.int64)
    out = np.zeros((rows, x64.shape[1]), dtype=np.float64)
    n_groups = len(offsets) - 1
    for gi in (range(n_groups) if groups is None else groups):
        lo, hi = int(offsets[gi]), int(offsets[gi + 1])
        if hi == lo:
            continue
        wg, wu, wd = _expert(weights, gi)
        out[lo:hi] = swiglu(x64[src[lo:hi]], wg, wu, wd)
    return out


def grouped_gate_up(x: np.ndarray, offsets: np.ndarray, row_index: Optional[np.ndarray],
                    weights: ExpertSource) -> np.ndarray:
    """The two input projections of each grouped row's expert (the SwiGLU
    expert of the routing-math page, section 0): fp64 [rows, 2 d_ffn] holding
    a = x W_gate^T in the first d_ffn columns and u = x W_up^T in the rest.
    Rows are gathered as in grouped_swiglu."""
    rows = int(offsets[-1])
    x64 = to_f64(x)
    src = np.arange(rows) if row_index is None else row_index.astype(np.int64)
    f = _expert(weights, 0)[0].shape[0]
    out = np.zeros((rows, 2 * f), dtype=np.float64)
    for gi in range(len(offsets) - 1):
        lo, hi = int(offsets[gi]), int(offsets[gi + 1])
        if hi == lo:
            continue
        wg, wu, _ = _expert(weights, gi)
        xs = x64[src[lo:hi]]
        out[lo:hi, :f] = xs @ to_f64(wg).T
        out[lo:hi, f:] = xs @ to_f64(wu).T
    return out


def shared_experts(h: np.ndarray, weights: Optional[ExpertSource], E_s: int) -> np.ndarray:
    """Sum over the always-active experts (gate 1) on every token, fp64 [T, d]."""
    h64 = to_f64(h)
    out = np.zeros_like(h64)
    for j in range(E_s):
        wg, wu, wd = _expert(weights, j)
        out += swiglu(h64, wg, wu, wd)
    return out


# ---------------------------------------------------------------- combine

def combine(h: np.ndarray, y_shared: Optional[np.ndarray], y_perm: np.ndarray,
            slot_row: np.ndarray, g: np.ndarray) -> np.ndarray:
    """y_t = h_t + y_shared_t + sum_k g_{t,k} * y_perm[slot_row[t,k]], fp64.

    A dropped copy (slot_row < 0, capacity dispatch) contributes nothing."""
    h64 = to_f64(h)
    T = h64.shape[0]
    K = g.shape[1]
    y = h64.copy()
    if y_shared is not None:
        y += y_shared
    sr = slot_row.reshape(T, K).astype(np.int64)
    for k in range(K):
        keep = sr[:, k] >= 0
        y[keep] += g[keep, k:k + 1].astype(np.float64) * y_perm[sr[keep, k]]
    return y


# ---------------------------------------------------------------- bias update

def bias_update(b: np.ndarray, loads: np.ndarray, T: int, K: int, gamma: float) -> np.ndarray:
    """b_i <- fl32(b_i + gamma * sign(cbar - c_i)), cbar = K T / E_r.

    sign(cbar - c_i) = sign(K*T - E_r*c_i) is decided in integers.
    """
    E_r = loads.shape[0]
    diff = np.int64(K) * np.int64(T) - np.int64(E_r) * loads.astype(np.int64)
    sgn = np.sign(diff).astype(np.float32)
    return (b.astype(np.float32) + np.float32(gamma) * sgn).astype(np.float32)


def max_vio(loads: np.ndarray, T: int, K: int) -> float:
    """MaxVio = (max_i c_i - cbar) / cbar."""
    cbar = K * T / loads.shape[0]
    return (float(loads.max()) - cbar) / cbar


def load_stats(loads: np.ndarray, T: int, K: int):
    return dict(max_load=int(loads.max()), min_load=int(loads.min()),
                max_vio=max_vio(loads, T, K))


# ---------------------------------------------------------------- diagnostics

def router_diagnostics(z: np.ndarray, idx: np.ndarray, E_r: int,
                       kept: Optional[np.ndarray] = None) -> dict:
    """Forward values of the router's balance diagnostics, fp64.

    z: [T, E_r] logits; idx: [T, K] picked experts; kept: [T, K] bool mask of
    the copies a capacity dispatch kept (None: all kept).
    """
    z64 = np.asarray(z, dtype=np.float64)
    T, K = idx.shape
    m = z64.max(axis=1, keepdims=True)
    ez = np.exp(z64 - m)
    lse = m[:, 0] + np.log(ez.sum(axis=1))              # logsumexp per token
    p = ez / ez.sum(axis=1, keepdims=True)               # softmax probabilities
    P = p.mean(axis=0)                                   # P_i
    c = load_count(idx, E_r).astype(np.float64)
    f = c * E_r / (K * T)                                # f_i
    share = c / c.sum()
    entropy = float(-(share * np.log(np.maximum(share, 1e-9))).sum())
    cbar = K * T / E_r
    return dict(P=P, f=f, switch_fP=float((f * P).sum()), z_loss=float((lse ** 2).mean()),
                load_entropy=entropy, max_vio=float((c.max() - cbar) / cbar),
                dropped=0.0 if kept is None else float(1.0 - kept.mean()))


# ---------------------------------------------------------------- backward

def combine_backward(dy: np.ndarray, y_perm: np.ndarray, slot_row: np.ndarray,
                     g: np.ndarray):
    """Gradients of y_t = h_t + y_shared_t + sum_k g_{t,k} y_perm[slot_row[t,k]].

    Returns (dy_perm [rows, d]: g_{t,k} dy_t on row slot_row[t,k]; dg [T, K]:
    <dy_t, y_perm[slot_row[t,k]]>, 0 for a dropped copy).  The residual and the
    shared experts receive dy itself.
    """
    dy64 = to_f64(dy)
    T, K = g.shape
    sr = slot_row.reshape(T, K).astype(np.int64)
    dy_perm = np.zeros_like(y_perm, dtype=np.float64)
    dg = np.zeros((T, K), dtype=np.float64)
    for k in range(K):
        keep = sr[:, k] >= 0
        dy_perm[sr[keep, k]] = g[keep, k:k + 1].astype(np.float64) * dy64[keep]
        dg[keep, k] = np.einsum("td,td->t", dy64[keep], y_perm[sr[keep, k]])
    return dy_perm, dg


def swiglu_backward(x, w_gate, w_up, w_down, dy):
    """Gradients of (SiLU(x W_gate^T) * (x W_up^T)) W_down^T, fp64.

    With a = x W_gate^T, u = x W_up^T, act = SiLU(a) u and SiLU'(a) =
    sigma(a) (1 + a (1 - sigma(a))): d act = dy W_down, dW_down = dy^T act,
    da = d act * u * SiLU'(a), du = d act * SiLU(a), dx = da W_gate + du W_up,
    dW_gate = da^T x, dW_up = du^T x.  Returns (dx, dW_gate, dW_up, dW_down).
    """
    x64 = to_f64(x) if x.dtype != np.float64 else x
    wg, wu, wd = to_f64(w_gate), to_f64(w_up), to_f64(w_down)
    dy64 = to_f64(dy) if dy.dtype != np.float64 else dy
    a = x64 @ wg.T
    u = x64 @ wu.T
    sa = 1.0 / (1.0 + np.exp(-a))
    act = a * sa * u
    dact = dy64 @ wd
    dwd = dy64.T @ act
    da = dact * u * sa * (1.0 + a * (1.0 - sa))
    du = dact * a * sa
    dx = da @ wg + du @ wu
    return dx, da.T @ x64, du.T @ x64, dwd


def grouped_swiglu_backward(x: np.ndarray, offsets: np.ndarray, row_index: Optional[np.ndarray],
                            weights: ExpertSource, dy_rows: np.ndarray,
                            groups: Optional[Sequence[int]] = None):
    """Backward of grouped_swiglu: dx_rows [rows, d] (gradient of each grouped
    row's input) and {g: (dW_gate, dW_up, dW_down)} for the groups with rows."""
    x64 = to_f64(x)
    rows = int(offsets[-1])
    src = np.arange(rows) if row_index is None else row_index.astype(np.int64)
    dx = np.zeros((rows, x64.shape[1]), dtype=np.float64)
    dw = {}
    n_groups = len(offsets) - 1
    for gi in (range(n_groups) if groups is None else groups):
        lo, hi = int(offsets[gi]), int(offsets[gi + 1])
        if hi == lo:
            continue
        wg, wu, wd = _expert(weights, gi)
        dx[lo:hi], dwg, dwu, dwd = swiglu_backward(x64[src[lo:hi]], wg, wu, wd, dy_rows[lo:hi])
        dw[gi] = (dwg, dwu, dwd)
    return dx, dw


def router_backward(h: np.ndarray, e: np.ndarray, idx: np.ndarray, fn: str,
                    dg: np.ndarray):
    """Gradient of the gates g_{t,k} (the picks I_t fixed) w.r.t. the logits of
    the picked experts, the tokens and the centroids, fp64.

    sigmoid: g_i = s_i / S, S = sum_{j in I_t} s_j, s = sigma(z): ds_i =
    (dg_i - sum_j g_j dg_j) / S and dz_i = ds_i s_i (1 - s_i).
    softmax renormalised over the picks: g_i = exp(z_i) / sum_{j in I_t}
    exp(z_j) (the full normaliser cancels), so dz_i = g_i (dg_i - sum_j g_j dg_j).
    Returns (dz [T, K], dh [T, d] = sum_k dz_{t,k} e_{idx[t,k]}, de [E_r, d] =
    sum over picks of dz h_t).  The bias gets no gradient.
    """
    h64, e64 = to_f64(h), to_f64(e)
    ii = idx.astype(np.int64)
    z = np.einsum("td,tkd->tk", h64, e64[ii])             # logits of the picks
    dg64 = dg.astype(np.float64)
    if fn == "sigmoid":
        sv = 1.0 / (1.0 + np.exp(-z))
        S = sv.sum(axis=1, keepdims=True)
        g = sv / S
        ds = (dg64 - (g * dg64).sum(axis=1, keepdims=True)) / S
        dz = ds * sv * (1.0 - sv)
    elif fn == "softmax":
        ez = np.exp(z - z.max(axis=1, keepdims=True))
        g = ez / ez.sum(axis=1, keepdims=True)
        dz = g * (dg64 - (g * dg64).sum(axis=1, keepdims=True))
    else:
        raise ValueError(fn)
    dh = np.einsum("tk,tkd->td", dz, e64[ii])
    de = np.zeros_like(e64)
    np.add.at(de, ii.reshape(-1), dz.reshape(-1, 1) * np.repeat(h64, idx.shape[1], axis=0))
    return dz, dh, de


def layer_backward(h, e, b, K: int, fn: str, routed: ExpertSource, dy,
                   shared: Optional[ExpertSource] = None, E_s: int = 0,
                   capacity: Optional[int] = None):
    """Gradients of sum_t <dy_t, y_t> for one layer call (the routing decisions
    of the forward pass held fixed): dh, de and the expert weight gradients."""
    out = layer_forward(h, e, b, K, fn, routed, shared, E_s, capacity=capacity)
    dy_perm, dg = combine_backward(dy, out["y_perm"], out["slot_row"], out["gates"])
    dx_perm, dw = grouped_swiglu_backward(h, out["offsets"], out["row_token"], routed, dy_perm)
    dh = to_f64(dy).copy()
    T = dh.shape[0]
    sr = out["slot_row"].reshape(T, K).astype(np.int64)
    for k in range(K):
        keep = sr[:, k] >= 0
        dh[keep] += dx_perm[sr[keep, k]]
    dw_shared = {}
    for j in range(E_s):
        wg, wu, wd = _expert(shared, j)
        dxs, dwg, dwu, dwd = swiglu_backward(to_f64(h), wg, wu, wd, to_f64(dy))
        dh += dxs
        dw_shared[j] = (dwg, dwu, dwd)
    dz, dh_r, de = router_backward(h, e, out["idx"], fn, dg)
    dh += dh_r
    return dict(out, dy_perm=dy_perm, dg=dg, dx_perm=dx_perm, dz=dz, dh=dh, de=de,
                dw=dw, dw_shared=dw_shared)


# ---------------------------------------------------------------- layer

def layer_forward(h, e, b, K: int, fn: str, routed: ExpertSource,
                  shared: Optional[ExpertSource] = None, E_s: int = 0,
                  gamma: Optional[float] = None, capacity: Optional[int] = None):
    """One full layer call: route, dispatch (capacity-bounded when `capacity`
    is given), routed + shared experts, combine, and (when gamma is given) the
    per-step bias update after counting.  The bias update counts the router's
    choices (before any drop)."""
    E_r = e.shape[0]
    T = h.shape[0]
    r = route(h, e, b, K, fn)
    if capacity is None:
        offsets, row_token, slot_row = permute(r["idx"], E_r)
    else:
        offsets, row_token, slot_row, _ = permute_capacity(r["idx"], E_r, capacity)
    y_perm = grouped_swiglu(h, offsets, row_token, routed)
    y_sh = shared_experts(h, shared, E_s) if E_s else None
    y = combine(h, y_sh, y_perm, slot_row, r["gates"])
    out = dict(r, offsets=offsets, row_token=row_token, slot_row=slot_row,
               y_perm=y_perm, y_shared=y_sh, y=y)
    if gamma is not None:
        b0 = b if b is not None else np.zeros(E_r, dtype=np.float32)
        out["b_new"] = bias_update(b0, r["loads"], T, K, gamma)
        out["stats"] = load_stats(r["loads"], T, K)
    return out
