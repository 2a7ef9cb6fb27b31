"""End-to-end parity at DeepSeek-V3 shape (d_model 7168, 256 routed experts of
d_ffn 2048, K = 8, one shared expert; about 22.6 GB of bf16 weights resident):
prefill (T = 4096), decode (T = 64) and the 20-step skewed-load training run
(T = 16384, gamma = 0.001, b0 = 0)."""
import json
import os

import numpy as np
import pytest
import torch

from gpu_common import check_route, say
from layer_check import check_layer, runner_for
from oracle import moe_oracle as O
from synthetic import CONFIGS, host_array, make_layer, make_tokens
from synthetic.gen import make_centroids

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsv3():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    say("drawing the DeepSeek-V3-shaped layer (22.6 GB)")
    lay = make_layer(CONFIGS["dsv3_prefill"], device="cuda")
    torch.cuda.synchronize()
    yield lay
    del lay
    torch.cuda.empty_cache()


def test_dsv3_prefill_full_size(dsv3):
    cfg = dsv3.cfg
    run = runner_for(dsv3)
    res = check_layer(dsv3, dsv3.h, dsv3.b, cfg.gamma, run, n_tok_sample=8, n_exp_sample=4,
                      seed=3)
    say(str(res))


@pytest.mark.parametrize("cf", [1.0, 1.25])
def test_dsv3_prefill_capacity_factor(dsv3, cf):
    """Capacity-bounded dispatch at full size: C = ceil(CF*T*K/E_r) = 128 / 160
    rows per expert (the loads reach about 167, so copies are dropped)."""
    cfg = dsv3.cfg
    run = runner_for(dsv3, capacity_factor=cf)
    assert run.capacity == O.expert_capacity(cfg.T, cfg.K, cfg.E_r, cf)
    res = check_layer(dsv3, dsv3.h, dsv3.b, cfg.gamma, run, n_tok_sample=12, n_exp_sample=4,
                      seed=5)
    assert res["dropped"] > 0
    say(str(res))


def test_dsv3_prefill_with_router_diagnostics(dsv3):
    """The layer with diagnostics on (moe_route_stats + moe_router_diag after
    a CF = 1.0 dispatch): same outputs as without, diagnostics vs the oracle."""
    cfg = dsv3.cfg
    run = runner_for(dsv3, capacity_factor=1.0)
    run_d = runner_for(dsv3, capacity_factor=1.0, diagnostics=True)
    y0 = run.forward(dsv3.h, dsv3.b.clone()).clone()
    y1 = run_d.forward(dsv3.h, dsv3.b.clone())
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    dv = run_d.diag_host()
    idx = run_d.topk_idx.cpu().numpy()
    kept = (run_d.slot_row.cpu().numpy() >= 0).reshape(cfg.T, cfg.K)
    z = O.router_logits(host_array(dsv3.h), host_array(dsv3.e))
    ref = O.router_diagnostics(z, idx, cfg.E_r, kept=kept)
    say(f"diagnostics {dv} vs oracle { {k: ref[k] for k in dv} }")
    for k, v in dv.items():
        assert abs(v - ref[k]) <= 1e-4 * max(1.0, abs(ref[k])), k


def test_dsv3_decode_full_size(dsv3):
    cfg = CONFIGS["dsv3_decode"]
    h = make_tokens(cfg, device="cuda")
    run = runner_for(dsv3, T=cfg.T)
    res = check_layer(dsv3, h, dsv3.b, cfg.gamma, run, n_tok_sample=16, n_exp_sample=6, seed=4)
    n_exp = int((run.loads > 0).sum())
    say(f"decode: {n_exp} distinct experts touched; {res}")


def test_dsv3_skewed_20_steps(dsv3, golden_dir):
    cfg = CONFIGS["dsv3_skewed"]
    with open(os.path.join(golden_dir, "skew_beta.json")) as f:
        beta = json.load(f)["beta"]
    e = make_centroids(cfg, device="cuda", beta=beta)
    run = runner_for(dsv3, T=cfg.T)
    run.e = e
    b = torch.zeros(cfg.E_r, dtype=torch.float32, device="cuda")
    b_oracle = np.zeros(cfg.E_r, dtype=np.float32)
    lay = dsv3
    flips = 0
    for step in range(cfg.steps):
        h = make_tokens(cfg, step=step, device="cuda")
        b_before = b.clone()
        if step in (0, cfg.steps - 1):
            # full layer check (sampled) on the first and the last step
            view = type(lay)(cfg, h, e, b_before, lay.w_gate, lay.w_up, lay.w_down,
                             lay.ws_gate, lay.ws_up, lay.ws_down)
            res = check_layer(view, h, b_before, cfg.gamma, run, n_tok_sample=8,
                              n_exp_sample=3, seed=10 + step)
            b = res["b_new"]
        else:
            run.forward(h, b, cfg.gamma)
        torch.cuda.synchronize()
        # the GPU ran this step from b_before; the oracle's own trajectory must match it
        assert np.array_equal(host_array(b_before).view(np.uint32), b_oracle.view(np.uint32))
        n_near, n_flip, r = check_route(h, e, b_before, cfg.K, cfg.score, run.topk_idx,
                                        run.gates, run.loads, cfg.E_r)
        flips += n_flip
        b_oracle = O.bias_update(b_oracle, r["loads"], cfg.T, cfg.K, cfg.gamma)
        st = run.stats_host()
        ls = O.load_stats(r["loads"], cfg.T, cfg.K)
        say(f"step {step:2d}: max {st['max_load']} min {st['min_load']} MaxVio "
            f"{st['max_vio']:.3f} (oracle {ls['max_vio']:.3f}); near-ties {n_near} flips {n_flip}")
        if n_flip == 0:
            assert st["max_load"] == ls["max_load"] and st["min_load"] == ls["min_load"]
    assert np.array_equal(host_array(b).view(np.uint32), b_oracle.view(np.uint32))
    say(f"20 steps: total flips {flips}")
