"""Host-side logic of bench.py that needs no GPU: the bounded CPU-oracle
sample behind the bench line's cpu_baseline."""
from dataclasses import replace

import pytest

import bench
from synthetic import CONFIGS, host_array, make_layer

# A small bf16 layer with a shared expert, the DeepSeek-V3 routing recipe.
CFG = replace(CONFIGS["dsv3_prefill"], T=96, d_model=64, E_r=12, K=2, d_ffn=32)


@pytest.fixture(scope="module")
def lay():
    return make_layer(CFG, device="cpu")


def test_cpu_baseline_zero_budget_runs_one_chunk(lay):
    out = bench.cpu_baseline(CFG, lay, host_array(lay.b), budget_s=0.0, chunk=5, sample_shared=32)
    assert out["kind"] == "oracle" and out["unit"] == "tokens/s" and out["value"] > 0
    assert "experts 0-4 of 12" in out["sample"]
    assert "expert time x2.4" in out["sample"] and "shared time x3" in out["sample"]


def test_cpu_baseline_large_budget_covers_every_expert(lay):
    out = bench.cpu_baseline(CFG, lay, host_array(lay.b), budget_s=1e9, chunk=5, sample_shared=4096)
    assert "experts 0-11 of 12" in out["sample"]
    assert "expert time x1," in out["sample"] and "shared time x1 " in out["sample"]
