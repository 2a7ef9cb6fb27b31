"""Throughput of one sparse MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload dsv3_prefill]

One step = the whole layer on one batch: route (fp32 router, biased top-K,
gates, loads) -> permute -> grouped SwiGLU over the routed experts -> shared
expert -> combine -> bias update (gamma = 0.001).  Inputs are seeded synthetic
tensors already resident in HBM; the token batch rotates over several copies so
the 256 MB Infinity Cache cannot serve them from one step to the next (the
22.6 GB of weights never fit anyway).  Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s at DeepSeek-V3 shape (1 GPU); % bf16 MFMA peak / % HBM BW"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def algorithmic(cfg, n_touched, n_touched_shared, rows=None, fused=False):
    """Algorithmic bytes / flops of the gate/up launch and of the whole layer.

    Per touched routed or shared expert: W_gate + W_up = 2 * d * f bf16 words
    (gate/up launch) and W_down = d * f words (down launch).  Per token: h read
    once (d words) and y written once (d words).  The activation the gate/up
    launch writes for the down launch (f words per assignment row) is a staged
    intermediate, overhead against these bytes, as are x rows re-read per
    column tile.  Expert flops: 6 d f per row (2 d f each for gate, up and
    down), rows = T*K routed (the kept copies under a capacity) + T*E_s shared.
    fused: the gate/up launch also runs the shared experts (moe_experts_swiglu).
    """
    d, f, T, K = cfg.d_model, cfg.d_ffn, cfg.T, cfg.K
    rows = T * K if rows is None else rows
    eb = 2 if cfg.dtype == "bf16" else 4
    gu_experts = n_touched + (n_touched_shared if fused else 0)
    gateup_bytes = gu_experts * 2 * d * f * eb + T * d * eb
    gateup_flops = 4.0 * d * f * (rows + (T * cfg.E_s if fused else 0))
    layer_bytes = (n_touched + n_touched_shared) * 3 * d * f * eb + 2 * T * d * eb
    layer_flops = 6.0 * d * f * (rows + T * cfg.E_s) + 2.0 * T * d * cfg.E_r
    return gateup_bytes, gateup_flops, layer_bytes, layer_flops


def stage_rooflines(cfg, stages, n_touched, rows, fused=False):
    """Achieved rate of the non-GEMM stages and of the down launch against
    their bound, from the library's per-stage event times (ms per call).

    Algorithmic bytes (staged intermediates such as the split-K logit
    partials are overhead):
      route   (logits + top-K): h read, centroids read, bias read, ids and
              gates written; fp32-exact logits are 2 T d E_r flops, run as
              three bf16 products each on the matrix cores
      permute (histogram, scan, assignment): ids read, offsets, row_token
              and slot_row written
      combine: h, the shared outputs, K gathered rows read and y written,
              plus ids and gates
      routed.down: W_down of the touched experts, the activation read and
              y_perm written (fused: experts.down, the shared experts' W_down
              and rows included)
    """
    d, f, T, K, E, Es = cfg.d_model, cfg.d_ffn, cfg.T, cfg.K, cfg.E_r, cfg.E_s
    eb = 2 if cfg.dtype == "bf16" else 4
    out = {}

    def put(name, ms, nbytes, flops=None, mfma_mult=None):
        if not ms:
            return
        rec = dict(ms=round(ms, 5), algorithmic_bytes=int(nbytes),
                   hbm_gbs=round(nbytes / ms / 1e6, 1),
                   hbm_frac=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4))
        if flops is not None:
            rec["flops"] = flops
            if mfma_mult:
                rec["mfma_tflops"] = round(flops * mfma_mult / ms / 1e9, 1)
                rec["mfma_frac"] = round(flops * mfma_mult / ms / 1e9 / BF16_PEAK_TFLOPS, 4)
        out[name] = rec

    route_ms = stages.get("route_logits", 0.0) + stages.get("route_topk", 0.0)
    route_bytes = T * d * eb + E * d * 4 + E * 4 + T * K * 8 + E * 4
    put("route", route_ms, route_bytes, 2.0 * T * d * E, 3 if eb == 2 else None)
    perm_ms = sum(stages.get(k, 0.0) for k in ("perm_hist", "perm_scan", "perm_assign"))
    put("permute", perm_ms, T * K * 4 + (E + 1) * 4 + 2 * T * K * 4)
    put("combine", stages.get("combine"), (K + Es + 2) * T * d * eb + T * K * 8)
    if fused:
        n_touched, rows = n_touched + Es, rows + Es * T
    name = "experts.down" if fused else "routed.down"
    put(name, stages.get(f"{name}_{cfg.dtype}"),
        n_touched * d * f * eb + rows * (f + d) * eb, 2.0 * d * f * rows, 1)
    return out


def recorded_traffic(workload: str, launch: str = "routed.gateup_bf16"):
    """HBM bytes per gate/up launch (`launch`: its stage name) from the
    FETCH_SIZE / WRITE_SIZE counter runs summarised in
    profiles/hbm_traffic_<workload>.md, already scaled by the copy calibration.
    None when no such record exists or the kernel sources changed since the
    counters were taken (their hash differs)."""
    import re
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    digest = kernel_source_hash()
    with open(path) as fh:
        for line in fh:
            m = re.match(r"traffic (\S+) (\S+) bytes=(\d+) .*sources=([0-9a-f]+)", line)
            if (m and m.group(1) == launch and m.group(2) == workload
                    and digest.startswith(m.group(4))):
                return int(m.group(3))
    return None


def kernel_source_hash() -> str:
    """sha256 of the grouped-SwiGLU kernel sources with comments and blank
    lines removed (a comment edit leaves the kernel, and its counters, as they
    were)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("swiglu_bf16.hip", "swiglu_tiles.h", "common.h"):
        with open(os.path.join(ROOT, "sparse_mixture_experts_biased_amd", "csrc", f)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.split("\n"):
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def spread_order(n: int):
    """0..n-1 in bit-reversed order: every prefix is spread over the range."""
    bits = max(1, (n - 1).bit_length())
    out = []
    for i in range(1 << bits):
        r = int(f"{i:0{bits}b}"[::-1], 2)
        if r < n:
            out.append(r)
    return out


def fit_expert_cost(rows, secs):
    """Least-squares fit secs ~ a + b * rows with a, b >= 0 (one sample: b only)."""
    import numpy as np
    from scipy.optimize import nnls
    rows = np.asarray(rows, dtype=np.float64)
    secs = np.asarray(secs, dtype=np.float64)
    if len(rows) < 2 or np.all(rows == rows[0]):
        return 0.0, float(secs.sum() / rows.sum())
    coef, _ = nnls(np.stack([np.ones_like(rows), rows], axis=1), secs)
    return float(coef[0]), float(coef[1])


def cpu_baseline(cfg, lay, b_host, budget_s=12.0, sample_shared=1024, capacity=None,
                 idx_gpu=None):
    """Time the oracle on a bounded sample of the same workload on host cores.

    Sample: routing of all T tokens; routed experts one at a time, on all
    their rows, in an order spread over the experts sorted by row count (so a
    skewed load's few large experts and many small ones are both sampled early),
    until their oracle time reaches budget_s or every expert is done; the shared
    expert on the first sample_shared tokens; the full combine and bias update.
    Unsampled experts are costed by a fit a + b * rows over the sampled ones
    (weight conversion per expert, GEMM work per row); the shared-expert time
    is scaled by T / tokens run.  With idx_gpu (the GPU's picks for the same
    tokens and bias), also counts near-ties and tokens whose picks differ.
    """
    import numpy as np

    from oracle import moe_oracle as O
    from synthetic import host_array

    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
        threads = max([n for _, n in blas if n] or [1])
    except Exception:  # threadpoolctl missing
        blas, threads = [], len(os.sched_getaffinity(0))
    h = host_array(lay.h)
    e = host_array(lay.e)
    ws = (host_array(lay.ws_gate[0]), host_array(lay.ws_up[0]), host_array(lay.ws_down[0])) \
        if cfg.E_s else None

    t0 = time.perf_counter()
    r = O.route(h, e, b_host, cfg.K, cfg.score)
    if capacity is None:
        off, rt, sr = O.permute(r["idx"], cfg.E_r)
    else:
        off, rt, sr, _ = O.permute_capacity(r["idx"], cfg.E_r, capacity)
    t_route = time.perf_counter() - t0

    routing = None
    if idx_gpu is not None:
        near = O.topk_margin(r["s"], b_host, cfg.K) < 1e-5
        same = np.all(idx_gpu == r["idx"], axis=1)
        routing = dict(tokens=int(cfg.T), near_ties=int(near.sum()),
                       flipped=int((~same).sum()), flipped_not_near=int((~same & ~near).sum()))

    rows_e = np.diff(off.astype(np.int64))
    nz = np.nonzero(rows_e > 0)[0]
    by_rows = nz[np.argsort(rows_e[nz], kind="stable")]
    order = [int(by_rows[j]) for j in spread_order(len(by_rows))]
    # Expert weights come to the host one at a time (outside the timed calls),
    # so host memory stays at one expert's weights.
    y_perm = None
    done, secs = [], []
    for i in order:
        if done and sum(secs) >= budget_s:
            break
        w = (host_array(lay.w_gate[i]), host_array(lay.w_up[i]), host_array(lay.w_down[i]))
        t0 = time.perf_counter()
        part = O.grouped_swiglu(h, off, rt, lambda _: w, groups=[i])
        secs.append(time.perf_counter() - t0)
        done.append(i)
        y_perm = part if y_perm is None else y_perm + part   # disjoint rows; the rest stay 0
        del w
    t_exp = sum(secs)
    a, bcoef = fit_expert_cost(rows_e[done], secs)
    if len(done) == len(nz):
        est_exp = t_exp
    else:
        est_exp = t_exp + sum(a + bcoef * rows_e[i] for i in set(nz.tolist()) - set(done))
    rows = int(rows_e[done].sum())

    t_sh, n_sh = 0.0, min(cfg.T, sample_shared)
    if ws is not None:
        t0 = time.perf_counter()
        O.swiglu(h[:n_sh], *ws)
        t_sh = time.perf_counter() - t0

    t0 = time.perf_counter()
    O.combine(h, None, y_perm, sr, r["gates"])
    O.bias_update(b_host if b_host is not None else np.zeros(cfg.E_r, np.float32), r["loads"],
                  cfg.T, cfg.K, 0.001)
    t_comb = time.perf_counter() - t0

    est = t_route + est_exp + t_comb
    if ws is not None:
        est += t_sh * cfg.T / n_sh
    measured = t_route + t_exp + t_sh + t_comb
    log(f"cpu oracle: route {t_route:.2f}s, {len(done)} of {len(nz)} experts ({rows} of "
        f"{int(rows_e.sum())} rows) {t_exp:.2f}s, fit {a:.4f}s + {bcoef * 1e3:.4f}ms/row, "
        f"shared on {n_sh} tokens {t_sh:.2f}s, combine {t_comb:.2f}s -> layer est {est:.1f}s")
    out = dict(
        value=cfg.T / est, unit="tokens/s", cores=int(threads), kind="oracle",
        sample=(f"oracle (NumPy fp64, BLAS {blas}) on: routing of all {cfg.T} tokens; "
                f"{len(done)} of {len(nz)} touched routed experts on all their rows ({rows} of "
                f"{int(rows_e.sum())} rows), taken spread over the experts sorted by rows; "
                f"the others costed by the fit {a:.4f} s + {bcoef * 1e3:.4f} ms per row; "
                f"shared expert on {n_sh if ws is not None else 0} of {cfg.T} tokens "
                f"(time x{(cfg.T / n_sh) if ws is not None else 0:g}); full combine + bias "
                f"update -> whole-layer estimate {est:.2f} s ({measured:.2f} s measured)"),
    )
    return out, routing


def copy_probe(nbytes: int) -> int:
    """A plain device-to-device copy of known size: the reference that scales
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {nbytes} bytes 3 times")
    return 0


def calibrate() -> int:
    """Achievable peaks on this GPU, the references the roofline fractions are
    also read against: a plain device copy of 2 GiB (HBM), the matrix-core
    loop moe_calib_mfma_loop (bf16 MFMA with no memory traffic), and the vendor
    GEMM library (hipBLASLt, through torch.matmul) on dense bf16 products of
    the expert GEMMs' sizes.  Random operands throughout (the core clock
    depends on the data).  Prints one JSON line."""
    import torch
    import sparse_mixture_experts_biased_amd._lib as L
    torch.manual_seed(0)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {}
    n = 1 << 31
    src = torch.randint(-(1 << 30), 1 << 30, (n // 4,), dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src), 10)
    out["copy_2GiB"] = {"ms": round(ms, 4), "GB/s (read + write)": round(2 * n / ms / 1e6, 1)}
    del dst
    log(f"copy: {out['copy_2GiB']}")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(8 * cus * 256, dtype=torch.int32, device="cuda")
    ms = timed(lambda: L.moe_calib_stream_read(8 * cus, src, sink), 10)
    out["read_2GiB"] = {"ms": round(ms, 4), "GB/s": round(n / ms / 1e6, 1)}
    del src, sink
    log(f"streaming read: {out['read_2GiB']}")

    wg, iters = 4 * cus, 512
    ops = torch.randn(wg * 256 * 96, device="cuda").to(torch.bfloat16)
    res = torch.empty(wg * 256, device="cuda")
    fl = [0.0]

    def loop():
        fl[0] = L.moe_calib_mfma_loop(wg, iters, ops, res)

    ms = timed(loop, 10)
    out["mfma_loop"] = {"workgroups": wg, "iters": iters, "ms": round(ms, 4),
                        "TFLOP/s": round(fl[0] / ms / 1e9, 1)}
    log(f"mfma loop: {out['mfma_loop']}")

    # dense equivalents of the expert GEMMs (M rows x N outputs x K), and one
    # DeepSeek-V3 prefill expert as the library would see it without grouping
    shapes = {
        "mixtral gate/up 8192x28672x4096": (8192, 28672, 4096),
        "mixtral down 8192x4096x14336": (8192, 4096, 14336),
        "dsv3 hot expert gate/up 8192x4096x7168": (8192, 4096, 7168),
        "dsv3 hot expert down 8192x7168x2048": (8192, 7168, 2048),
        "dsv3 prefill one expert gate/up 128x4096x7168": (128, 4096, 7168),
    }
    lib = {}
    for name, (M, N, K) in shapes.items():
        # weights [N, K] as the layer stores them (K-contiguous, like the kernels'
        # operands); a 2-D product with the transposed view is one library GEMM
        a = torch.randn(M, K, device="cuda").to(torch.bfloat16)
        w = torch.randn(N, K, device="cuda").to(torch.bfloat16)
        ms = timed(lambda: torch.mm(a, w.t()), 10)
        lib[name] = {"ms": round(ms, 4), "TFLOP/s": round(2.0 * M * N * K / ms / 1e9, 1),
                     "GB/s (operands + output)": round(2.0 * (M * K + K * N + M * N) / ms / 1e6, 1)}
        log(f"hipBLASLt {name}: {lib[name]}")
        del a, w
    out["hipblaslt"] = lib
    print(json.dumps({"calibration": out, "device": torch.cuda.get_device_name(0), "cus": cus}),
          flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_prefill",
                    choices=["dsv3_prefill", "dsv3_decode", "dsv3_skewed", "mixtral_8x7b"])
    ap.add_argument("--rotate", type=int, default=10, help="token batches cycled through")
    ap.add_argument("--tokens", type=int, default=None, metavar="T",
                    help="override the workload's token count T (same layer otherwise)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--capacity-factor", type=float, default=None, metavar="CF",
                    help="cap every expert at ceil(CF*T*K/E_r) rows (token dropping)")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step: the forward pass plus the backward pass of the "
                         "layer (gradients of tokens, centroids and every expert weight)")
    ap.add_argument("--shared-start", default="layer", choices=["layer", "routed"],
                    help="when the side stream starts the shared experts: with the layer "
                         "(default) or once routing and dispatch are done")
    ap.add_argument("--serial-shared", action="store_true",
                    help="run the shared experts after the routed ones on one stream "
                         "(default: on a second stream beside the routing)")
    ap.add_argument("--fused-shared", action="store_true",
                    help="run the shared experts inside the routed experts' grouped launches "
                         "(moe_experts_swiglu) instead of launches of their own")
    ap.add_argument("--diagnostics", action="store_true",
                    help="route with the router statistics and compute the balance diagnostics "
                         "(Switch f.P, z-loss, load entropy, MaxVio, dropped rate) every step")
    ap.add_argument("--stage-events", default="dominant", choices=["dominant", "all"],
                    help="which launches carry hipEvents in the timed steps: only the gate/up "
                         "launch the roofline reports (default; the other stages are timed in "
                         "a few extra steps after the timed region) or every launch")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only copy a BYTES-sized buffer 3 times (calibrates HBM byte counters)")
    ap.add_argument("--calibrate", action="store_true",
                    help="only measure the achievable peaks (device copy, matrix-core loop, "
                         "hipBLASLt on the expert GEMM sizes) and print them as one JSON line")
    args = ap.parse_args(argv)
    if args.copy_probe:
        return copy_probe(args.copy_probe)
    if args.calibrate:
        return calibrate()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        log("bench.py measures the single-GPU layer forward only: this build has no "
            "multi-GPU path (expert parallelism is out of scope). Run with --gpus 1.")
        return 2

    import numpy as np
    import torch

    from sparse_mixture_experts_biased_amd import (LayerShape, MoELayer, load,
                                                   moe_profile_enable, moe_profile_only,
                                                   moe_profile_report)
    from synthetic import CONFIGS, host_array, make_layer, make_tokens

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    load()
    cfg = CONFIGS[args.workload]
    if args.tokens is not None:
        if args.tokens < 1:
            log("--tokens must be >= 1")
            return 2
        cfg = cfg.with_tokens(args.tokens)
    log(f"workload {cfg.name}: T={cfg.T} d_model={cfg.d_model} E_r={cfg.E_r} K={cfg.K} "
        f"E_s={cfg.E_s} d_ffn={cfg.d_ffn} {cfg.dtype} {cfg.score}")
    t0 = time.perf_counter()
    beta = None
    if cfg.hot_experts:
        with open(os.path.join(ROOT, "tests", "golden", "skew_beta.json")) as f:
            beta = json.load(f)["beta"]
    lay = make_layer(cfg, device="cuda", beta=beta)
    # a multi-step training run takes a fresh batch every step
    n_batches = max(args.rotate, cfg.steps)
    hs = [lay.h] + [make_tokens(cfg, step=i, device="cuda") for i in range(1, n_batches)]
    torch.cuda.synchronize()
    log(f"inputs drawn in {time.perf_counter() - t0:.1f}s "
        f"({cfg.weight_bytes() / 1e9:.2f} GB of expert weights)")
    shape = LayerShape(cfg.T, cfg.d_model, cfg.E_r, cfg.K, cfg.E_s, cfg.d_ffn, cfg.dtype,
                       cfg.score)
    run = MoELayer(shape, lay.e, lay.w_gate, lay.w_up, lay.w_down, lay.ws_gate, lay.ws_up,
                   lay.ws_down, capacity_factor=args.capacity_factor,
                   overlap_shared=not args.serial_shared, shared_start=args.shared_start,
                   diagnostics=args.diagnostics, fuse_shared=args.fused_shared)
    b = lay.b.clone() if lay.b is not None else None
    b_host0 = host_array(lay.b) if lay.b is not None else None
    gamma = cfg.gamma if b is not None else None
    stream = torch.cuda.current_stream()
    run.profile_tags = True
    dy = None
    if args.backward:
        run.prepare_backward(stream)     # transposed weight copies: outside the timed steps
        dy = make_tokens(cfg, step=10_000, device="cuda")

    # per-step load statistics of a multi-step training run (the skewed workload):
    # a 16-byte device copy after each step's bias update
    stats_hist = None

    # backward wall time per timed step: events on the caller's stream around
    # run.backward (which returns after joining the side stream's work)
    bw_evs = None

    def step(i):
        run.forward(hs[i % len(hs)], b, gamma, stream)
        if dy is not None:
            if bw_evs is not None:
                bw_evs[i][0].record(stream)
            run.backward(hs[i % len(hs)], dy, stream)
            if bw_evs is not None:
                bw_evs[i][1].record(stream)
        if stats_hist is not None:
            stats_hist[i].copy_(run.stats, non_blocking=True)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    moe_profile_report()  # drop warm-up records
    # the forward's expert launches: fused (routed + shared) unless a training
    # forward or --unfused-shared kept them apart
    fused = run.fuse_shared and dy is None
    pfx = "experts." if fused else "routed."
    # in the timed steps only the launch the roofline reports carries events
    # (each event pair is a queue packet of its own between two launches)
    moe_profile_only(pfx + "gateup" if args.stage_events == "dominant" else "")
    moe_profile_enable(True)
    if cfg.steps > 1 and gamma is not None:
        stats_hist = torch.zeros((args.steps, 4), dtype=torch.int32, device="cuda")
        b.copy_(lay.b)   # the timed steps are steps 0, 1, ... of the run, from b0
    # one event per step boundary (recording does not synchronise): per-step times
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    if dy is not None:
        bw_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    moe_profile_enable(False)
    prof = moe_profile_report()
    ev_ms = evs[0].elapsed_time(evs[-1])
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    loads = run.loads.cpu().numpy()
    n_touched = int((loads > 0).sum())
    kept_rows = int(run.offsets[-1].item())
    layer_stats = run.stats_host()  # the last timed step's load statistics
    if args.stage_events == "dominant":
        # every stage's launch time from a few more steps with all events on
        # (outside the timed region; the timed gate/up figure is kept)
        moe_profile_only("")
        moe_profile_enable(True)
        for i in range(min(5, args.steps)):
            run.forward(hs[i % len(hs)], b, gamma, stream)
            if dy is not None:
                run.backward(hs[i % len(hs)], dy, stream)
        torch.cuda.synchronize()
        moe_profile_enable(False)
        prof = {**moe_profile_report(), **prof}

    ms_per_step = wall * 1000.0 / args.steps
    tokens_per_s = cfg.T / (ms_per_step / 1000.0)
    gu_bytes, gu_flops, layer_bytes, layer_flops = algorithmic(cfg, n_touched, cfg.E_s, kept_rows,
                                                               fused)
    stages = {k: round(v[1] / v[0], 5) for k, v in prof.items()}
    log("per-kernel average ms: " + json.dumps(stages))
    log(f"wall {wall * 1000:.2f} ms, events {ev_ms:.2f} ms over {args.steps} steps")
    routed_ms = stages.get(pfx + "gateup_bf16")
    sec = routed_ms / 1000.0
    gbs = gu_bytes / sec / 1e9
    tfs = gu_flops / sec / 1e12
    # the launch's bound: HBM when its algorithmic intensity is below the bf16 ridge
    mfma_bound = gu_flops / gu_bytes > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roofline = dict(bound="mfma", achieved=round(tfs, 1), peak=BF16_PEAK_TFLOPS,
                        unit="TFLOP/s", frac=round(tfs / BF16_PEAK_TFLOPS, 4), traffic=None)
    else:
        roofline = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None)
    # the counter record covers the dispatch without a capacity limit
    traffic = recorded_traffic(cfg.name, pfx + "gateup_bf16") if run.capacity is None else None
    roofline["traffic"] = traffic
    roofline.update(kernel="gateup_bf16 (routed + shared experts)" if fused
                    else "gateup_bf16 (routed experts)", avg_ms=round(routed_ms, 4),
                    algorithmic_bytes=gu_bytes, algorithmic_flops=gu_flops,
                    hbm_gbs=round(gbs, 1), mfma_tflops=round(tfs, 1),
                    mfma_frac=round(tfs / BF16_PEAK_TFLOPS, 4))
    layer = dict(algorithmic_bytes=layer_bytes, flops=layer_flops,
                 hbm_gbs=round(layer_bytes / (ms_per_step / 1000.0) / 1e9, 1),
                 hbm_frac=round(layer_bytes / (ms_per_step / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
                 mfma_tflops=round(layer_flops / (ms_per_step / 1000.0) / 1e12, 1),
                 mfma_frac=round(layer_flops / (ms_per_step / 1000.0) / 1e12 / BF16_PEAK_TFLOPS, 4),
                 experts_touched=n_touched, stats=layer_stats)
    # the roofline fraction the layer attains: the larger of its MFMA and HBM fractions
    layer["attainable_frac"] = max(layer["hbm_frac"], layer["mfma_frac"])

    cpu = routing = None
    if not args.no_cpu_baseline:
        # the GPU's picks for the first batch from the initial bias (outside the
        # timed steps), compared with the oracle's in the baseline leg
        b0 = lay.b.clone() if lay.b is not None else None
        run.route(lay.h, b0)
        idx_gpu = run.topk_idx.cpu().numpy()
        cpu, routing = cpu_baseline(cfg, lay, b_host0, capacity=run.capacity, idx_gpu=idx_gpu)

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded Gaussian tokens and weights, random-init experts)",
        "config": {"workload": f"{cfg.name}: T={cfg.T} d_model={cfg.d_model} E_r={cfg.E_r} "
                               f"K={cfg.K} E_s={cfg.E_s} d_ffn={cfg.d_ffn} {cfg.score} router, "
                               f"bias update gamma={cfg.gamma}" +
                               ("" if run.capacity is None else
                                f", capacity factor {args.capacity_factor} (C={run.capacity} "
                                f"rows per expert, {cfg.T * cfg.K - kept_rows} of "
                                f"{cfg.T * cfg.K} copies dropped)"),
                   "tokens_per_step": cfg.T, "parallelism": "single GPU"},
        "roofline": roofline, "layer": layer, "stages_ms": stages,
        "stage_rooflines": stage_rooflines(cfg, stages, n_touched, kept_rows, fused),
        "cpu_baseline": cpu,
        "routing_vs_oracle": routing,
        "step_ms": {"median": round(step_ms[len(step_ms) // 2], 4), "min": round(step_ms[0], 4),
                    "max": round(step_ms[-1], 4)},
    }
    if stats_hist is not None:
        h = stats_hist.cpu()
        out["load_stats_per_step"] = [
            {"max_load": int(r[0]), "min_load": int(r[1]),
             "max_vio": round(float(r[2:3].view(torch.float32)[0]), 4)} for r in h]
    if args.diagnostics:
        out["router_diag"] = {k: round(v, 6) for k, v in run.diag_host().items()}
    if args.backward:
        # per touched expert: W_down^T and [W_gate^T | W_up^T] read, three gradients
        # written: 6 d f words; per assignment row dy_perm, dx (2 d words) and the
        # a|u kept by the forward, da|du (4 f words) are overhead
        d, f = cfg.d_model, cfg.d_ffn
        bw_bytes = (n_touched + cfg.E_s) * 6 * d * f * 2
        bw_ms = sum(e0.elapsed_time(e1) for e0, e1 in bw_evs) / args.steps
        out["mode"] = "forward+backward"
        out["backward"] = dict(ms_per_step=round(bw_ms, 4), algorithmic_bytes=bw_bytes,
                               hbm_gbs=round(bw_bytes / (bw_ms / 1000.0) / 1e9, 1),
                               hbm_frac=round(bw_bytes / (bw_ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
                               flops=6.0 * 2 * d * f * (kept_rows + cfg.T * cfg.E_s))
        out["config"]["workload"] += ", training step (forward + backward)"
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
