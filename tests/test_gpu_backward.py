"""Backward pass on the GPU against the oracle's gradients (bf16 operands,
fp32 accumulation): grouped SwiGLU, combine and router backward, the whole
layer at small sizes (sigmoid and softmax routers, with and without a
capacity), and sampled gradients at the DeepSeek-V3 prefill size."""
import math

import numpy as np
import pytest
import torch

from gpu_common import out_tol, rel_err, say, to_host_f64
from layer_check import runner_for
from oracle import moe_oracle as O
from sparse_mixture_experts_biased_amd import LayerShape, MoELayer
from sparse_mixture_experts_biased_amd import _lib as L
from synthetic import CONFIGS, host_array, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = out_tol("bf16")   # max|d| <= 2e-2 max|ref| per gradient tensor


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _bf16(shape, scale, seed):
    return (torch.randn(shape, generator=_gen(seed), device=DEV) * scale).to(torch.bfloat16)


def _prep_t(wg, wu, wd):
    n, f, d = wg.shape
    gu_t = torch.empty((n, d, 2 * f), dtype=torch.bfloat16, device=DEV)
    d_t = torch.empty((n, f, d), dtype=torch.bfloat16, device=DEV)
    L.moe_transpose_experts(n, f, d, wg, L.MOE_BF16, gu_t, 2 * f, 0)
    L.moe_transpose_experts(n, f, d, wu, L.MOE_BF16, gu_t, 2 * f, f)
    L.moe_transpose_experts(n, d, f, wd, L.MOE_BF16, d_t, d, 0)
    return gu_t, d_t


def test_transpose_experts():
    w = _bf16((3, 70, 130), 1.0, 1)
    out = torch.zeros((3, 130, 200), dtype=torch.bfloat16, device=DEV)
    L.moe_transpose_experts(3, 70, 130, w, L.MOE_BF16, out, 200, 50)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, 50:120], w.transpose(1, 2))
    assert torch.all(out[:, :, :50] == 0) and torch.all(out[:, :, 120:] == 0)


@pytest.mark.parametrize("stored", [False, True], ids=["recompute", "stored_au"])
@pytest.mark.parametrize("T,d,f,E,K,identity", [
    (200, 128, 128, 6, 2, False),
    (700, 256, 192, 5, 3, False),     # 192 = one and a half column tiles
    (3, 128, 64, 16, 2, False),       # nearly all groups empty
    (1100, 64, 128, 3, 1, False),     # groups of ~370 rows: several 128-row tiles
    (300, 128, 128, 1, 1, True),      # one group, identity rows (shared-expert form)
    (1300, 512, 512, 4, 1, False)])   # streaming-kernel shapes in the a|u forward
def test_grouped_swiglu_backward_parity(T, d, f, E, K, identity, stored):
    _check_grouped_backward(T, d, f, E, K, identity, stored)


# Groups of at most 128 rows on average with K and N of whole slices and column
# tiles: the activation-gradient products run over the row tiles of the kernel
# that sends both operands by LDS DMA; hot: expert 0 takes most tokens (a group
# of several such row tiles beside small ones).
@pytest.mark.parametrize("stored", [False, True], ids=["recompute", "stored_au"])
@pytest.mark.parametrize("T,d,f,E,K,hot", [
    (1000, 1024, 768, 16, 2, False),
    (900, 768, 1024, 16, 2, True)])
def test_grouped_swiglu_backward_dma_tiles(T, d, f, E, K, hot, stored):
    _check_grouped_backward(T, d, f, E, K, False, stored, hot=hot)


def _check_grouped_backward(T, d, f, E, K, identity, stored, hot=False):
    say(f"moe_grouped_swiglu_backward T={T} d={d} f={f} E={E} K={K} identity={identity} "
        f"stored={stored} hot={hot}")
    rng = np.random.default_rng(T + E)
    x = _bf16((T, d), 1.0, 3 + T)
    wg = _bf16((E, f, d), 1 / math.sqrt(d), 4)
    wu = _bf16((E, f, d), 1 / math.sqrt(d), 5)
    wd = _bf16((E, d, f), 1 / math.sqrt(f), 6)
    if identity:
        off = np.array([0, T], np.int32)
        rt = None
    else:
        scores = rng.random((T, E)).astype(np.float32)
        if hot:
            scores[:, 0] += 0.6
        idx = O.biased_topk(scores, None, K)
        off, rt, _ = O.permute(idx, E)
        if hot:
            assert np.diff(off)[0] > 2 * 168 and off[-1] <= 128 * E
    rows = int(off[-1])
    dy = _bf16((rows, d), 1.0, 7)
    gu_t, d_t = _prep_t(wg, wu, wd)
    dx = torch.zeros((rows, d), dtype=torch.bfloat16, device=DEV)
    dwg, dwu, dwd = torch.full_like(wg, 7.0), torch.full_like(wu, 7.0), torch.full_like(wd, 7.0)
    offs = torch.from_numpy(off).to(DEV)
    ri = None if rt is None else torch.from_numpy(rt).to(DEV)
    au = None
    if stored:   # the training forward's a|u
        fb = L.moe_grouped_swiglu_workspace_size(E, d, f, rows, L.MOE_BF16)
        fws = torch.empty(fb, dtype=torch.uint8, device=DEV)
        au = torch.empty((rows, 2 * f), dtype=torch.bfloat16, device=DEV)
        y = torch.empty((rows, d), dtype=torch.bfloat16, device=DEV)
        L.moe_grouped_swiglu_train(E, d, f, rows, T, offs, ri, x, L.MOE_BF16, wg, wu, wd, None,
                                   y, au, fws, fb)
    wsb = L.moe_grouped_swiglu_backward_workspace_size(E, d, f, rows)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    L.moe_grouped_swiglu_backward(E, d, f, rows, T, offs, ri, x, L.MOE_BF16, wg, wu, gu_t, d_t,
                                  dy, au, dx, dwg, dwu, dwd, ws, wsb)
    torch.cuda.synchronize()
    w_host = (host_array(wg), host_array(wu), host_array(wd))
    rdx, rdw = O.grouped_swiglu_backward(host_array(x), off, rt, w_host, to_host_f64(dy))
    e_dx = rel_err(to_host_f64(dx), rdx)
    say(f"dx {e_dx:.2e}")
    assert e_dx <= TOL
    for i in range(E):
        got = [to_host_f64(t[i]) for t in (dwg, dwu, dwd)]
        if i not in rdw:                       # no rows: zero gradient
            assert all(np.all(g == 0) for g in got)
            continue
        for m in range(3):
            e = rel_err(got[m], rdw[i][m])
            assert e <= TOL, (i, m, e)


def test_combine_backward_parity():
    T, d, E, K = 300, 256, 8, 3
    rng = np.random.default_rng(8)
    idx = O.biased_topk(rng.random((T, E)).astype(np.float32), None, K)
    C = O.expert_capacity(T, K, E, 1.0)
    off, rt, sr, _ = O.permute_capacity(idx, E, C)
    g = torch.rand((T, K), generator=_gen(9), device=DEV)
    yp = _bf16((T * K, d), 1.0, 10)
    dy = _bf16((T, d), 1.0, 11)
    dyp = torch.zeros((T * K, d), dtype=torch.bfloat16, device=DEV)
    dg = torch.full((T, K), 5.0, device=DEV)
    L.moe_combine_backward(T, d, K, dy, yp, torch.from_numpy(sr).to(DEV), g, L.MOE_BF16, dyp, dg)
    torch.cuda.synchronize()
    r_dyp, r_dg = O.combine_backward(host_array(dy), to_host_f64(yp), sr, g.cpu().numpy())
    n = int(off[-1])
    assert rel_err(to_host_f64(dyp)[:n], r_dyp[:n]) <= 2 ** -8
    assert np.all(to_host_f64(dyp)[n:] == 0)           # no row for a dropped copy
    assert np.allclose(dg.cpu().numpy(), r_dg, rtol=1e-4, atol=1e-4 * np.abs(r_dg).max())
    assert np.all(dg.cpu().numpy()[sr.reshape(T, K) < 0] == 0)


@pytest.mark.parametrize("fn", ["sigmoid", "softmax"])
def test_route_backward_parity(fn):
    T, d, E, K = 500, 256, 32, 4
    h = _bf16((T, d), 1.0, 12)
    e = (torch.randn((E, d), generator=_gen(13), device=DEV) / math.sqrt(d)).float()
    rng = np.random.default_rng(14)
    idx = O.biased_topk(rng.random((T, E)).astype(np.float32), None, K)
    dgt = torch.randn((T, K), generator=_gen(15), device=DEV)
    off, rt, _ = O.permute(idx, E)
    dz = torch.empty((T, K), device=DEV)
    dh0 = _bf16((T, d), 1.0, 16)
    dh = dh0.clone()
    de = torch.empty((E, d), device=DEV)
    L.moe_route_backward(T, d, E, K, L.MOE_SIGMOID if fn == "sigmoid" else L.MOE_SOFTMAX, h,
                         L.MOE_BF16, e, torch.from_numpy(idx).to(DEV), dgt,
                         torch.from_numpy(off).to(DEV), torch.from_numpy(rt).to(DEV), dz, dh, de)
    torch.cuda.synchronize()
    r_dz, r_dh, r_de = O.router_backward(host_array(h), host_array(e), idx, fn,
                                         dgt.cpu().numpy())
    assert np.allclose(dz.cpu().numpy(), r_dz, rtol=1e-4, atol=1e-5 * np.abs(r_dz).max())
    # dh is bf16 in and out: one rounding of dh0 + router term per element
    want = to_host_f64(dh0) + r_dh
    assert np.all(np.abs(to_host_f64(dh) - want) <= 2.0 ** -8 * np.abs(want) +
                  1e-3 * np.abs(r_dh).max())
    assert np.allclose(de.cpu().numpy(), r_de, rtol=1e-3, atol=1e-4 * np.abs(r_de).max())


def _small_bf16_layer(T, d, f, E, K, E_s, fn, seed):
    h = _bf16((T, d), 1.0, seed)
    e = (torch.randn((E, d), generator=_gen(seed + 1), device=DEV) / math.sqrt(d)).float()
    w = (_bf16((E, f, d), 1 / math.sqrt(d), seed + 2), _bf16((E, f, d), 1 / math.sqrt(d), seed + 3),
         _bf16((E, d, f), 1 / math.sqrt(f), seed + 4))
    ws = (_bf16((E_s, f, d), 1 / math.sqrt(d), seed + 5), _bf16((E_s, f, d), 1 / math.sqrt(d),
          seed + 6), _bf16((E_s, d, f), 1 / math.sqrt(f), seed + 7)) if E_s else (None,) * 3
    b = (torch.rand(E, generator=_gen(seed + 8), device=DEV) * 0.02 - 0.01).float() \
        if fn == "sigmoid" else None
    return h, e, w, ws, b


@pytest.mark.parametrize("fn,cf,E_s,keep_au", [("sigmoid", None, 1, True),
                                               ("softmax", None, 0, True),
                                               ("sigmoid", 1.0, 1, True),
                                               ("sigmoid", None, 1, False)])
def test_layer_backward_small(fn, cf, E_s, keep_au):
    T, d, f, E, K = 256, 256, 128, 16, 4
    h, e, w, ws, b = _small_bf16_layer(T, d, f, E, K, E_s, fn, 20)
    shape = LayerShape(T, d, E, K, E_s, f, "bf16", fn)
    run = MoELayer(shape, e, *w, *ws, capacity_factor=cf)
    run.prepare_backward(keep_au=keep_au)
    run.forward(h, b)
    dy = _bf16((T, d), 1.0, 30)
    run.backward(h, dy)
    torch.cuda.synchronize()
    wh = tuple(host_array(t) for t in w)
    wsh = tuple(host_array(t) for t in ws) if E_s else None
    cap = None if cf is None else run.capacity
    ref = O.layer_backward(host_array(h), host_array(e), None if b is None else host_array(b), K,
                           fn, wh, to_host_f64(dy), wsh, E_s, capacity=cap)
    assert np.array_equal(run.topk_idx.cpu().numpy(), ref["idx"])   # no near-ties here
    e_dh = rel_err(to_host_f64(run.dh), ref["dh"])
    e_de = rel_err(run.de.cpu().numpy().astype(np.float64), ref["de"])
    say(f"dh {e_dh:.2e} de {e_de:.2e}")
    assert e_dh <= TOL and e_de <= TOL
    worst = 0.0
    for i in range(E):
        got = [to_host_f64(t[i]) for t in (run.dw_gate, run.dw_up, run.dw_down)]
        if i not in ref["dw"]:
            assert all(np.all(x == 0) for x in got)
            continue
        for m in range(3):
            worst = max(worst, rel_err(got[m], ref["dw"][i][m]))
    for m, t in enumerate((run.dws_gate, run.dws_up, run.dws_down) if E_s else ()):
        worst = max(worst, rel_err(to_host_f64(t[0]), ref["dw_shared"][0][m]))
    say(f"weight gradients: worst {worst:.2e}")
    assert worst <= TOL


def test_dsv3_prefill_backward_sampled():
    """Full DeepSeek-V3 prefill size (22.6 GB of weights, their transposes and
    gradients resident): the weight gradients of sampled experts, dh and the
    gate gradients of sampled tokens, and the router gradients (dz, de) of all
    tokens given the GPU's gate gradients."""
    cfg = CONFIGS["dsv3_prefill"]
    lay = make_layer(cfg, device=DEV)
    run = runner_for(lay)
    run.prepare_backward()
    run.forward(lay.h, lay.b.clone())
    dy = _bf16((cfg.T, cfg.d_model), 1.0, 40)
    run.backward(lay.h, dy)
    torch.cuda.synchronize()
    T, K, E = cfg.T, cfg.K, cfg.E_r
    idx = run.topk_idx.cpu().numpy()
    g = run.gates.cpu().numpy()
    off = run.offsets.cpu().numpy()
    rt = run.row_token.cpu().numpy()
    sr = run.slot_row.cpu().numpy()
    h = host_array(lay.h)
    dyh = to_host_f64(dy)
    rng = np.random.default_rng(41)

    def expert(i):
        return host_array(lay.w_gate[i]), host_array(lay.w_up[i]), host_array(lay.w_down[i])

    # weight gradients of sampled experts: dy_perm rows = g * dy (fp64)
    for i in rng.choice(E, 2, replace=False):
        lo, hi = int(off[i]), int(off[i + 1])
        toks = rt[lo:hi]
        kk = np.array([np.nonzero(idx[t] == i)[0][0] for t in toks])
        dyp = g[toks, kk][:, None].astype(np.float64) * dyh[toks]
        _, rdwg, rdwu, rdwd = O.swiglu_backward(h[toks], *expert(i), dyp)
        for got, ref in ((run.dw_gate[i], rdwg), (run.dw_up[i], rdwu), (run.dw_down[i], rdwd)):
            e_w = rel_err(to_host_f64(got), ref)
            say(f"expert {i}: dW {e_w:.2e}")
            assert e_w <= TOL
    # dh and dgates of sampled tokens
    ws = tuple(host_array(t[0]) for t in (lay.ws_gate, lay.ws_up, lay.ws_down))
    for t in rng.choice(T, 3, replace=False):
        x = h[t:t + 1]
        dht = dyh[t].copy()
        dg_ref = np.zeros(K)
        for k in range(K):
            wgi, wui, wdi = expert(int(idx[t, k]))
            dg_ref[k] = float(dyh[t] @ O.swiglu(x, wgi, wui, wdi)[0])
            dx, _, _, _ = O.swiglu_backward(x, wgi, wui, wdi, g[t, k] * dyh[t:t + 1])
            dht += dx[0]
        dxs, _, _, _ = O.swiglu_backward(x, *ws, dyh[t:t + 1])
        dht += dxs[0]
        _, rdh, _ = O.router_backward(x, host_array(lay.e), idx[t:t + 1], cfg.score,
                                      dg_ref[None, :])
        dht += rdh[0]
        e_dh = rel_err(to_host_f64(run.dh[t:t + 1])[0], dht)
        e_dg = rel_err(run.dgates[t].cpu().numpy().astype(np.float64), dg_ref)
        say(f"token {t}: dh {e_dh:.2e} dgates {e_dg:.2e}")
        assert e_dh <= TOL and e_dg <= TOL
    # the shared expert's weight gradients reduce over all T rows: a block of
    # hidden units is an exact sub-problem (each unit's gradients depend only on
    # its own gate, up and down weights), so the oracle runs on those units alone
    units = np.sort(rng.choice(cfg.d_ffn, 128, replace=False))
    wsg, wsu, wsd = ws
    _, rg, ru, rd = O.swiglu_backward(h, wsg[units], wsu[units], wsd[:, units], dyh)
    for name, got, ref in (("dws_gate", run.dws_gate[0][units], rg),
                           ("dws_up", run.dws_up[0][units], ru),
                           ("dws_down", run.dws_down[0][:, units], rd)):
        e_w = rel_err(to_host_f64(got.contiguous()), ref)
        say(f"shared {name} on {len(units)} hidden units x {T} rows: {e_w:.2e}")
        assert e_w <= TOL
    # the shared expert's input gradient on a token sample (rows are independent)
    toks = np.sort(rng.choice(T, 64, replace=False))
    rdx, _, _, _ = O.swiglu_backward(h[toks], *ws, dyh[toks])
    e_dx = rel_err(to_host_f64(run.dx_shared)[toks], rdx)
    say(f"shared dx on {len(toks)} tokens: {e_dx:.2e}")
    assert e_dx <= TOL
    # router gradients of every token from the GPU's gate gradients
    r_dz, _, r_de = O.router_backward(h, host_array(lay.e), idx, cfg.score,
                                      run.dgates.cpu().numpy())
    assert np.allclose(run.dz.cpu().numpy(), r_dz, rtol=1e-3, atol=1e-4 * np.abs(r_dz).max())
    assert rel_err(run.de.cpu().numpy().astype(np.float64), r_de) <= 1e-3
    del run, lay
    torch.cuda.empty_cache()


def test_backward_call_order_is_enforced():
    """backward() reads the a | u a training forward stores: it must come after
    prepare_backward() and a forward, else it raises before launching anything."""
    T, d, f, E, K = 128, 256, 128, 8, 2
    h, e, w, ws, b = _small_bf16_layer(T, d, f, E, K, 1, "sigmoid", 50)
    shape = LayerShape(T, d, E, K, 1, f, "bf16", "sigmoid")
    run = MoELayer(shape, e, *w, *ws)
    dy = _bf16((T, d), 1.0, 51)
    with pytest.raises(RuntimeError):
        run.backward(h, dy)                       # no prepare_backward
    run.forward(h, b)
    run.prepare_backward()
    with pytest.raises(RuntimeError):
        run.backward(h, dy)                       # a | u not written since prepare
    run.forward(h, b)
    run.backward(h, dy)                           # the documented order
    torch.cuda.synchronize()
    dh0 = run.dh.clone()
    run.prepare_backward()                        # e.g. after a weight update
    with pytest.raises(RuntimeError):
        run.backward(h, dy)
    run.forward(h, b)
    run.backward(h, dy)
    torch.cuda.synchronize()
    assert torch.equal(run.dh, dh0)
    with pytest.raises(ValueError):
        run.backward(h, dy[:-1])                  # dy of the wrong shape
