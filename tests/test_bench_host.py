"""Host-side logic of bench.py that needs no GPU: the bounded CPU-oracle
sample behind the bench line's cpu_baseline."""
from dataclasses import replace

import numpy as np
import pytest

import bench
from oracle import moe_oracle as O
from synthetic import CONFIGS, host_array, make_layer

# A small bf16 layer with a shared expert, the DeepSeek-V3 routing recipe.
CFG = replace(CONFIGS["dsv3_prefill"], T=96, d_model=64, E_r=12, K=2, d_ffn=32)


@pytest.fixture(scope="module")
def lay():
    return make_layer(CFG, device="cpu")


def test_spread_order_is_a_permutation_with_spread_prefixes():
    for n in (1, 2, 5, 12, 256):
        o = bench.spread_order(n)
        assert sorted(o) == list(range(n))
    o = bench.spread_order(256)
    # the first 8 positions land in 8 different 32-wide bands of the sorted range
    assert len({p // 32 for p in o[:8]}) == 8


def test_fit_expert_cost_recovers_a_linear_cost():
    rows = np.array([10, 200, 35, 8000, 120])
    secs = 0.05 + 2e-4 * rows
    a, b = bench.fit_expert_cost(rows, secs)
    assert a == pytest.approx(0.05, rel=1e-6) and b == pytest.approx(2e-4, rel=1e-6)
    a, b = bench.fit_expert_cost([50], [0.5])
    assert a == 0.0 and b == pytest.approx(0.01)


def test_cpu_baseline_zero_budget_runs_one_expert(lay):
    out, routing = bench.cpu_baseline(CFG, lay, host_array(lay.b), budget_s=0.0,
                                      sample_shared=32)
    assert routing is None
    assert out["kind"] == "oracle" and out["unit"] == "tokens/s" and out["value"] > 0
    assert "1 of 12 touched routed experts" in out["sample"]
    assert "time x3" in out["sample"]


def test_cpu_baseline_large_budget_covers_every_expert(lay):
    r = O.route(host_array(lay.h), host_array(lay.e), host_array(lay.b), CFG.K, CFG.score)
    idx = r["idx"].copy()
    idx[5] = (idx[5] + 1) % CFG.E_r            # one token's picks differ
    idx[5].sort()
    out, routing = bench.cpu_baseline(CFG, lay, host_array(lay.b), budget_s=1e9,
                                      sample_shared=4096, idx_gpu=idx)
    n = int((np.diff(O.permute(r["idx"], CFG.E_r)[0]) > 0).sum())
    assert f"{n} of {n} touched routed experts" in out["sample"]
    assert "time x1)" in out["sample"]
    assert routing["tokens"] == CFG.T and routing["flipped"] == 1


def test_stage_rooflines_bytes_and_fractions():
    cfg = CONFIGS["dsv3_prefill"]
    T, d, K, E, f = cfg.T, cfg.d_model, cfg.K, cfg.E_r, cfg.d_ffn
    stages = {"route_logits": 0.05, "route_topk": 0.02, "perm_hist": 0.01, "perm_scan": 0.01,
              "perm_assign": 0.01, "combine": 0.1, "routed.down_bf16": 1.5}
    r = bench.stage_rooflines(cfg, stages, n_touched=256, rows=T * K)
    # combine: h, one shared output, K gathered rows read, y written (bf16), ids + gates
    assert r["combine"]["algorithmic_bytes"] == (K + 3) * T * d * 2 + T * K * 8 == 646184960
    assert r["combine"]["hbm_frac"] == pytest.approx(646184960 / 0.1e-3 / 8e12, abs=1e-4)
    assert r["route"]["ms"] == pytest.approx(0.07)
    assert r["route"]["algorithmic_bytes"] == T * d * 2 + E * d * 4 + 2 * E * 4 + T * K * 8
    # fp32-exact logits, three bf16 products each on the matrix cores
    assert r["route"]["mfma_tflops"] == pytest.approx(3 * 2 * T * d * E / 0.07e-3 / 1e12, rel=1e-3)
    assert r["permute"]["ms"] == pytest.approx(0.03)
    assert r["routed.down"]["algorithmic_bytes"] == 256 * d * f * 2 + T * K * (f + d) * 2
    # a stage the run did not time is left out
    assert "combine" not in bench.stage_rooflines(cfg, {"route_logits": 0.05}, 256, T * K)
