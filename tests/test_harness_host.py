"""The GPU parity harness (layer_check.check_layer) run on the CPU against a
stand-in for the layer whose outputs are the oracle's own, rounded as the GPU
rounds them: it must accept them, and it must reject planted mistakes (a wrong
expert row, a wrong bias update, a swapped gate)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import layer_check
from oracle import moe_oracle as O
from synthetic import CONFIGS, host_array, make_layer

CFG = replace(CONFIGS["dsv3_prefill"], T=48, d_model=64, E_r=12, K=3, d_ffn=64)


def _bf16(a64):
    return torch.from_numpy(np.asarray(a64, dtype=np.float32)).to(torch.bfloat16)


class OracleRun:
    """Buffers named as MoELayer's, filled from the oracle."""

    def __init__(self, lay, plant=None):
        self.lay, self.plant, self.capacity = lay, plant, None

    def forward(self, h, b, gamma):
        c = self.lay.cfg
        hh, e = host_array(h), host_array(self.lay.e)
        bb = host_array(b) if b is not None else None
        r = O.route(hh, e, bb, c.K, c.score)
        off, rt, sr = O.permute(r["idx"], c.E_r)

        def src(wg, wu, wd):
            return lambda i: (host_array(wg[i]), host_array(wu[i]), host_array(wd[i]))
        yp = O.grouped_swiglu(hh, off, rt, src(self.lay.w_gate, self.lay.w_up, self.lay.w_down))
        ysh = O.shared_experts(hh, src(self.lay.ws_gate, self.lay.ws_up, self.lay.ws_down),
                               c.E_s)
        g = r["gates"].copy()
        if self.plant == "expert_row":
            yp[int(off[3])] += 0.5 * np.abs(yp).max()
        if self.plant == "gate_swap":
            g[5] = g[5][::-1]
        y = O.combine(hh, ysh, yp, sr, g)
        self.topk_idx = torch.from_numpy(r["idx"])
        self.gates = torch.from_numpy(r["gates"])
        self.loads = torch.from_numpy(r["loads"])
        self.offsets, self.row_token = torch.from_numpy(off), torch.from_numpy(rt)
        self.slot_row = torch.from_numpy(sr)
        self.y_perm, self.y_shared, self.y = _bf16(yp), _bf16(ysh), _bf16(y)
        if gamma is not None and b is not None:
            nb = O.bias_update(bb, r["loads"], c.T, c.K, gamma)
            if self.plant == "bias":
                nb[2] += np.float32(gamma)
            b.copy_(torch.from_numpy(nb))
            st = O.load_stats(r["loads"], c.T, c.K)
            self._stats = dict(max_load=st["max_load"], min_load=st["min_load"],
                               max_vio=float(np.float32(st["max_vio"])))
        return self.y

    def stats_host(self):
        return self._stats


@pytest.fixture(scope="module")
def lay():
    return make_layer(CFG, device="cpu")


@pytest.fixture(autouse=True)
def _no_device_sync(monkeypatch):
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)


@pytest.mark.parametrize("rows_per_expert", [None, 2])
def test_harness_accepts_the_oracle(lay, rows_per_expert):
    res = layer_check.check_layer(lay, lay.h, lay.b, CFG.gamma, OracleRun(lay), n_tok_sample=10,
                                  n_exp_sample=3, rows_per_expert=rows_per_expert)
    assert res["flipped"] == 0
    if rows_per_expert is not None:
        idx = O.route(host_array(lay.h), host_array(lay.e), host_array(lay.b), CFG.K,
                      CFG.score)["idx"]
        assert res["experts_checked"] == int((np.bincount(idx.reshape(-1)) > 0).sum())
    else:
        assert res["experts_checked"] == 3


@pytest.mark.parametrize("plant", ["expert_row", "bias", "gate_swap"])
def test_harness_rejects_planted_mistakes(lay, plant):
    with pytest.raises(AssertionError):
        layer_check.check_layer(lay, lay.h, lay.b, CFG.gamma, OracleRun(lay, plant),
                                check_all_tokens=True, rows_per_expert=CFG.T * CFG.K)
