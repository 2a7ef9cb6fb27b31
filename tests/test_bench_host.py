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
