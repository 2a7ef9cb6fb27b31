"""End-to-end layer check shared by the full-size GPU tests.

The GPU runs the whole layer through the C ABI; the oracle routes every token
from the same inputs, and recomputes the layer output of a sample of tokens
(all tokens when T is small) plus the expert outputs of a sample of experts.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

from gpu_common import NEAR_TIE, check_route, out_tol, rel_err, say, to_host_f64
from oracle import moe_oracle as O
from sparse_mixture_experts_biased_amd import LayerShape, MoELayer
from synthetic import host_array


def runner_for(lay, T=None, capacity_factor=None, diagnostics=False, fuse_shared=False):
    c = lay.cfg
    shape = LayerShape(T or c.T, c.d_model, c.E_r, c.K, c.E_s, c.d_ffn, c.dtype, c.score)
    return MoELayer(shape, lay.e, lay.w_gate, lay.w_up, lay.w_down, lay.ws_gate, lay.ws_up,
                    lay.ws_down, capacity_factor=capacity_factor, diagnostics=diagnostics,
                    fuse_shared=fuse_shared)


def _expert_source(w_gate, w_up, w_down):
    def get(i):
        return host_array(w_gate[i]), host_array(w_up[i]), host_array(w_down[i])
    return get


def check_permutation_valid(idx, offsets, row_token, slot_row, E):
    """Properties any correct dispatch of `idx` has (used when a near-tie flip
    makes the GPU's picks differ from the oracle's)."""
    T, K = idx.shape
    counts = np.bincount(idx.reshape(-1), minlength=E)
    assert np.array_equal(np.diff(offsets), counts) and offsets[0] == 0
    flat_t = np.repeat(np.arange(T), K)
    assert np.array_equal(row_token[slot_row], flat_t)
    for i in range(E):
        seg = row_token[offsets[i]:offsets[i + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all((idx[seg] == i).any(axis=1))


def check_layer(lay, h, b_in, gamma, run, n_tok_sample=16, n_exp_sample=4, seed=0,
                check_all_tokens=False, rows_per_expert=None, label=None):
    """Run one layer forward on the GPU and compare with the oracle.  With a
    capacity (run.capacity), the oracle's capacity dispatch of the whole batch
    decides which copies are kept.

    Returns a dict with near-tie / flip counts and the observed errors."""
    c = lay.cfg
    T, E, K = h.shape[0], c.E_r, c.K
    b_dev = b_in.clone() if b_in is not None else None
    run.forward(h, b_dev, gamma)
    torch.cuda.synchronize()
    idx = run.topk_idx.cpu().numpy()
    off = run.offsets.cpu().numpy()
    rt = run.row_token.cpu().numpy()
    sr = run.slot_row.cpu().numpy()

    n_near, n_flip, r = check_route(h, lay.e, b_in, K, c.score, run.topk_idx, run.gates,
                                    run.loads, E)
    flipped = np.nonzero(~np.all(idx == r["idx"], axis=1))[0]
    cap = run.capacity
    kept = np.ones((T, K), dtype=bool)
    if cap is not None:
        # which copies survive depends on every earlier token: decided on the
        # GPU's own picks (teacher forcing; equal to the oracle's without flips)
        o_off, o_rt, o_sr, o_kept = O.permute_capacity(idx, E, cap)
        assert np.array_equal(off, o_off)
        assert np.array_equal(rt[:int(o_off[-1])], o_rt) and np.array_equal(sr, o_sr)
        assert np.all(rt[int(o_off[-1]):] == -1)
        kept = (o_sr >= 0).reshape(T, K)
        say(f"capacity {cap}: {int((~kept).sum())} of {T * K} copies dropped")
    elif n_flip == 0:
        o_off, o_rt, o_sr = O.permute(r["idx"], E)
        assert np.array_equal(off, o_off)
        assert np.array_equal(rt, o_rt) and np.array_equal(sr, o_sr)
    else:
        check_permutation_valid(idx, off, rt, sr, E)
    res = dict(near_ties=n_near, flipped=n_flip, b_new=b_dev, dropped=int((~kept).sum()))

    # bias update after counting: bit-exact against the oracle's update of the
    # GPU's own loads (teacher forcing), flips or not; without flips those loads
    # equal the oracle's (check_route asserts it)
    if gamma is not None and b_in is not None:
        b_ref = O.bias_update(host_array(b_in), run.loads.cpu().numpy(), T, K, gamma)
        b_gpu = host_array(b_dev)
        assert np.array_equal(b_gpu.view(np.uint32), b_ref.view(np.uint32))
        if n_flip == 0:
            b_free = O.bias_update(host_array(b_in), r["loads"], T, K, gamma)
            assert np.array_equal(b_gpu.view(np.uint32), b_free.view(np.uint32))
        st = run.stats_host()
        ls = O.load_stats(run.loads.cpu().numpy(), T, K)
        assert st["max_load"] == ls["max_load"] and st["min_load"] == ls["min_load"]
        assert abs(st["max_vio"] - ls["max_vio"]) <= 1e-6 * max(1.0, abs(ls["max_vio"]))
        res["stats"] = st

    rng = np.random.default_rng(seed)
    experts = _expert_source(lay.w_gate, lay.w_up, lay.w_down)
    shared = _expert_source(lay.ws_gate, lay.ws_up, lay.ws_down) if c.E_s else None
    h_host = host_array(h)
    tol = out_tol(c.dtype)

    # layer output on a token sample (tokens whose picks flipped are excluded)
    cand = np.setdiff1d(np.arange(T), flipped)
    toks = cand if (check_all_tokens or len(cand) <= n_tok_sample) else np.sort(
        rng.choice(cand, n_tok_sample, replace=False))
    idx_s, g_s = r["idx"][toks], r["gates"][toks]
    off_s, rt_s, sr_s = O.permute(idx_s, E)
    sr_s = np.where(kept[toks].reshape(-1), sr_s, -1).astype(np.int32)   # dropped copies

    # routed expert outputs (y_perm): all rows of a sample of non-empty experts,
    # or (rows_per_expert set) a few rows of every non-empty expert.  The GPU's
    # own dispatch decides the rows (teacher forcing), so flips do not matter:
    # each permuted row is expert i's SwiGLU of the token it came from.
    nonempty = np.nonzero(np.diff(off) > 0)[0]
    if rows_per_expert is not None:
        ex = nonempty
    else:
        ex = nonempty if len(nonempty) <= n_exp_sample else np.sort(
            rng.choice(nonempty, n_exp_sample, replace=False))
    picks = {}
    for i in ex:
        lo, hi = int(off[i]), int(off[i + 1])
        cap_rows = 256 if rows_per_expert is None else rows_per_expert
        picks[int(i)] = np.sort(rng.choice(hi - lo, cap_rows, replace=False)) \
            if hi - lo > cap_rows else np.arange(hi - lo)

    # One oracle SwiGLU call per expert on the union of the rows it is checked
    # on: its sampled y_perm rows and the sampled tokens' copies routed to it
    # (rows are independent, so this is the per-expert step of the oracle's
    # grouped SwiGLU); experts run in threads (numpy releases the GIL).
    x_s = h_host[toks]
    y_perm_s = np.zeros((len(toks) * K, c.d_model), dtype=np.float64)
    sample_experts = set(np.nonzero(np.diff(off_s) > 0)[0].tolist())

    def one(i):
        lo_s, hi_s = int(off_s[i]), int(off_s[i + 1])
        rows_a = x_s[rt_s[lo_s:hi_s]]
        if i in picks:
            lo, hi = int(off[i]), int(off[i + 1])
            rows_b = h_host[rt[lo:hi][picks[i]]]
        else:
            rows_b = h_host[:0]
        out = O.swiglu(np.concatenate([rows_a, rows_b]), *experts(i))
        return i, out[:hi_s - lo_s], out[hi_s - lo_s:]

    # one BLAS thread per call: the pool supplies the parallelism (a
    # multithreaded BLAS called from every pool thread oversubscribes the cores)
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=12) as pool:
        outs = list(pool.map(one, sorted(sample_experts | set(picks))))
    ref_b = {}
    for i, ya, yb in outs:
        y_perm_s[int(off_s[i]):int(off_s[i + 1])] = ya
        if i in picks:
            ref_b[i] = yb
    y_sh_s = O.shared_experts(x_s, shared, c.E_s) if c.E_s else None
    y_ref = O.combine(x_s, y_sh_s, y_perm_s, sr_s, g_s)
    y_gpu = to_host_f64(run.y)[toks]
    err = rel_err(y_gpu, y_ref)
    h64 = O.to_f64(x_s)
    err_delta = rel_err(y_gpu - h64, y_ref - h64)
    say(f"layer y: max|d|/max|y| = {err:.2e}; on y - h: {err_delta:.2e} ({len(toks)} tokens)")
    assert err <= tol
    # the expert part (y - h), with one output rounding of y allowed per element
    assert np.all(np.abs((y_gpu - h64) - (y_ref - h64))
                  <= tol * np.max(np.abs(y_ref - h64)) + 2.0 ** -8 * np.abs(y_ref))
    res["y_rel_err"] = err
    res["y_minus_h_rel_err"] = err_delta

    y_perm = host_array(run.y_perm)
    errs = {}
    for i, ref in ref_b.items():
        lo = int(off[i])
        errs[i] = rel_err(O.to_f64(y_perm[lo + picks[i]]), ref)
    worst = max(errs.values(), default=0.0)
    bad = {i: e for i, e in errs.items() if e > tol}
    assert not bad, f"experts over tolerance: {bad}"
    res["expert_rel_err"] = worst
    res["experts_checked"] = len(errs)
    res["expert_rows_checked"] = int(sum(len(p) for p in picks.values()))
    say(f"expert outputs: worst max|d|/max|ref| = {worst:.2e} over {len(errs)} experts, "
        f"{res['expert_rows_checked']} rows")
    if c.E_s:
        ysh = to_host_f64(run.y_shared).reshape(c.E_s, T, c.d_model)
        for j in range(c.E_s):
            ref = O.swiglu(h_host[toks], *shared(j))
            assert rel_err(ysh[j][toks], ref) <= tol
    record_parity(label or c.name, T, res)
    return res


def record_parity(name, T, res):
    """Append this check's routing counts and errors to the parity record
    under gpurun_out/ (kept with the run's other outputs)."""
    import json
    import os
    rec = {k: v for k, v in res.items() if k != "b_new"}
    rec.update(workload=name, T=int(T))
    out = os.path.join(os.environ.get("GRAFT_REPO_ROOT", "."), "gpurun_out")
    try:
        os.makedirs(out, exist_ok=True)
        with open(os.path.join(out, "parity_counts.jsonl"), "a") as fh:
            fh.write(json.dumps(rec, default=float) + "\n")
    except OSError:
        pass

