"""End-to-end layer parity on the GPU for the tiny fp32 layer and the
Mixtral-8x7B-shaped layer (full sizes; the oracle recomputes a token sample
and an expert sample at Mixtral size)."""
import numpy as np
import pytest
import torch

from gpu_common import say
from layer_check import check_layer, runner_for
from oracle import moe_oracle as O
from synthetic import CONFIGS, host_array, make_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    yield
    torch.cuda.synchronize()


def test_tiny_fp32_layer_and_one_bias_update():
    cfg = CONFIGS["tiny_fp32"]
    say(f"{cfg.name}: T={cfg.T} d={cfg.d_model} E={cfg.E_r} K={cfg.K}")
    lay = make_layer(cfg, device="cuda")
    run = runner_for(lay)
    b0 = lay.b.clone()
    res = check_layer(lay, lay.h, b0, cfg.gamma, run, check_all_tokens=True)
    say(str(res))
    # one update with gamma = 0.1 against cbar = 16, then re-route with the new b:
    b1 = b0.clone()
    run.forward(lay.h, b1, cfg.gamma)
    torch.cuda.synchronize()
    ref_b1 = O.bias_update(host_array(b0), O.route(host_array(lay.h), host_array(lay.e),
                                                   host_array(b0), cfg.K, cfg.score)["loads"],
                           cfg.T, cfg.K, cfg.gamma)
    assert np.array_equal(host_array(b1).view(np.uint32), ref_b1.view(np.uint32))
    idx0, g0 = run.topk_idx.clone(), run.gates.clone()
    run.route(lay.h, b1)
    torch.cuda.synchronize()
    same = (idx0 == run.topk_idx).all(dim=1)
    assert torch.equal(g0[same].view(torch.int32), run.gates[same].view(torch.int32))
    check_layer(lay, lay.h, b1, None, run, check_all_tokens=True)


def test_mixtral_layer_full_size():
    cfg = CONFIGS["mixtral_8x7b"]
    say(f"{cfg.name}: T={cfg.T} d={cfg.d_model} E={cfg.E_r} K={cfg.K} d_ffn={cfg.d_ffn}")
    lay = make_layer(cfg, device="cuda")
    run = runner_for(lay)
    res = check_layer(lay, lay.h, None, None, run, n_tok_sample=12, n_exp_sample=3, seed=1)
    say(str(res))


def test_mixtral_layer_ragged_tokens():
    cfg = CONFIGS["mixtral_8x7b"].with_tokens(333)
    lay = make_layer(cfg, device="cuda")
    run = runner_for(lay)
    check_layer(lay, lay.h, None, None, run, n_tok_sample=8, n_exp_sample=2, seed=2)


def test_shared_expert_overlap_matches_sequential():
    """The shared experts on the side stream (started with the layer, or once
    the routing is done) give the same bits as run in sequence, forward and
    backward, and again on a second call."""
    from dataclasses import replace
    from sparse_mixture_experts_biased_amd import LayerShape, MoELayer
    cfg = replace(CONFIGS["dsv3_prefill"], T=300, d_model=1024, E_r=32, K=4, d_ffn=512)
    say(f"overlap vs sequential: T={cfg.T} d={cfg.d_model} E={cfg.E_r} K={cfg.K} E_s={cfg.E_s}")
    lay = make_layer(cfg, device="cuda")
    shape = LayerShape(cfg.T, cfg.d_model, cfg.E_r, cfg.K, cfg.E_s, cfg.d_ffn, cfg.dtype,
                       cfg.score)
    dy = torch.randn(cfg.T, cfg.d_model, generator=torch.Generator("cuda").manual_seed(5),
                     device="cuda").to(torch.bfloat16)
    outs = {}
    for name, overlap, start in (("overlap", True, "layer"), ("overlap-routed", True, "routed"),
                                 ("sequential", False, "layer")):
        run = MoELayer(shape, lay.e, lay.w_gate, lay.w_up, lay.w_down, lay.ws_gate, lay.ws_up,
                       lay.ws_down, overlap_shared=overlap, shared_start=start)
        run.prepare_backward()
        ys = []
        for _ in range(2):
            ys.append(run.forward(lay.h, lay.b).clone())
            run.backward(lay.h, dy)
        torch.cuda.synchronize()
        assert torch.equal(ys[0], ys[1]), name
        outs[name] = (ys[0], run.dh.clone(), run.dws_gate.clone(), run.dws_down.clone(),
                      run.de.clone())
    for name in ("overlap", "overlap-routed"):
        for a, b in zip(outs[name], outs["sequential"]):
            assert torch.equal(a, b), name


@pytest.mark.parametrize("T,d,E,K,E_s,f,cf", [
    (300, 1024, 32, 4, 1, 512, None),     # one shared row group
    (2500, 512, 16, 2, 2, 256, None),     # two shared experts, 4 row groups each
    (700, 512, 24, 3, 1, 256, 1.0),       # capacity: dropped copies leave a gap of rows
    (64, 1024, 64, 8, 1, 512, None),      # decode-sized batch
])
def test_fused_shared_matches_separate_launches(T, d, E, K, E_s, f, cf):
    """moe_experts_swiglu (routed + shared experts in one grouped launch per
    product) gives the same bits as the separate launches, in sequence or with
    the shared experts on the side stream, and the layer matches the oracle."""
    from dataclasses import replace
    from sparse_mixture_experts_biased_amd import LayerShape, MoELayer
    cfg = replace(CONFIGS["dsv3_prefill"], T=T, d_model=d, E_r=E, K=K, E_s=E_s, d_ffn=f)
    say(f"fused vs separate: T={T} d={d} E={E} K={K} E_s={E_s} f={f} cf={cf}")
    lay = make_layer(cfg, device="cuda")
    shape = LayerShape(T, d, E, K, E_s, f, cfg.dtype, cfg.score)
    runs = {}
    for name, fuse, overlap in (("fused", True, True), ("side", False, True),
                                ("serial", False, False)):
        runs[name] = MoELayer(shape, lay.e, lay.w_gate, lay.w_up, lay.w_down, lay.ws_gate,
                              lay.ws_up, lay.ws_down, capacity_factor=cf, fuse_shared=fuse,
                              overlap_shared=overlap)
    ys = {n: r.forward(lay.h, lay.b).clone() for n, r in runs.items()}
    y2 = runs["fused"].forward(lay.h, lay.b).clone()
    torch.cuda.synchronize()
    assert torch.equal(ys["fused"], y2)
    for n in ("side", "serial"):
        assert torch.equal(runs["fused"].y_shared, runs[n].y_shared), n
        kept = int(runs[n].offsets[-1].item())
        assert torch.equal(runs["fused"].y_perm[:kept], runs[n].y_perm[:kept]), n
        assert torch.equal(ys["fused"], ys[n]), n
    check_layer(lay, lay.h, None, None, runs["fused"], n_tok_sample=12, n_exp_sample=3, seed=8,
                label=f"fused T={T} E_s={E_s}")


@pytest.mark.parametrize("fuse", [False, True])
def test_single_token_layer(fuse):
    """One token through the whole bf16 layer (router tile of one row, one
    split-K partial per split, one row per touched expert, one shared row)."""
    from dataclasses import replace
    from sparse_mixture_experts_biased_amd import LayerShape, MoELayer
    cfg = replace(CONFIGS["dsv3_prefill"], T=1, d_model=512, E_r=16, K=4, d_ffn=256)
    lay = make_layer(cfg, device="cuda")
    shape = LayerShape(1, cfg.d_model, cfg.E_r, cfg.K, cfg.E_s, cfg.d_ffn, cfg.dtype, cfg.score)
    run = MoELayer(shape, lay.e, lay.w_gate, lay.w_up, lay.w_down, lay.ws_gate, lay.ws_up,
                   lay.ws_down, fuse_shared=fuse)
    res = check_layer(lay, lay.h, lay.b, cfg.gamma, run, check_all_tokens=True, seed=1,
                      label=f"single token fuse={fuse}")
    assert res["experts_checked"] == cfg.K
