"""Per-entry-point parity on the GPU at sizes the oracle finishes in seconds:
each HIP entry point gets oracle-made (or generator-made) inputs and its output
is compared with the oracle's on the same inputs.  Shapes span several tiles
and ragged tails; edge cases: empty experts, total collapse, K = 1, K = E_r,
invalid expert ids, softmax with a bias."""
import math

import numpy as np
import pytest
import torch

from gpu_common import GATE_TOL, check_route, out_tol, rel_err, say, to_host_f64
from oracle import moe_oracle as O
from sparse_mixture_experts_biased_amd import _lib as L
from synthetic import host_array

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    L.load()
    yield
    torch.cuda.synchronize()


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _tokens(T, d, dtype, seed, scale=1.0):
    x = torch.randn((T, d), generator=_gen(seed), device=DEV) * scale
    return x.to(dtype)


def _centroids(E, d, seed):
    return (torch.randn((E, d), generator=_gen(seed), device=DEV) / math.sqrt(d)).contiguous()


def _route_gpu(h, e, b, K, fn):
    T, d = h.shape
    E = e.shape[0]
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    gates = torch.empty((T, K), dtype=torch.float32, device=DEV)
    loads = torch.empty((E,), dtype=torch.int32, device=DEV)
    dt = L.MOE_BF16 if h.dtype == torch.bfloat16 else L.MOE_F32
    wsb = L.moe_route_workspace_size(T, d, E, dt)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=DEV)
    L.moe_route(T, d, E, K, fn, h, dt, e, b, idx, gates, loads, ws, wsb)
    torch.cuda.synchronize()
    return idx, gates, loads


ROUTE_CASES = [
    # T, d, E, K, fn, dtype, bias
    (64, 128, 8, 2, "sigmoid", torch.float32, "zero"),
    (333, 256, 8, 2, "softmax", torch.bfloat16, None),
    (200, 512, 256, 8, "sigmoid", torch.bfloat16, "uniform"),
    (77, 192, 64, 6, "sigmoid", torch.float32, "uniform"),
    (50, 128, 16, 1, "sigmoid", torch.bfloat16, "uniform"),
    (40, 128, 12, 12, "sigmoid", torch.float32, "uniform"),   # K = E_r
    (129, 256, 512, 16, "sigmoid", torch.bfloat16, "uniform"),
    (90, 128, 32, 4, "softmax", torch.float32, "uniform"),    # softmax + bias on p
    (300, 1792, 256, 8, "sigmoid", torch.bfloat16, "uniform"),  # 3.5 k-slices per split
    (32768, 320, 128, 8, "sigmoid", torch.bfloat16, "uniform"),  # one split, 5 k-slices
]


@pytest.mark.parametrize("T,d,E,K,fn,dtype,bias", ROUTE_CASES)
def test_route_parity(T, d, E, K, fn, dtype, bias):
    say(f"moe_route T={T} d={d} E={E} K={K} {fn} {dtype}")
    h = _tokens(T, d, dtype, 1000 + T)
    e = _centroids(E, d, 2000 + E)
    b = None
    if bias == "zero":
        b = torch.zeros(E, device=DEV)
    elif bias == "uniform":
        b = (torch.rand(E, generator=_gen(3000 + E), device=DEV) * 0.02 - 0.01)
    idx, gates, loads = _route_gpu(h, e, b, K, L.MOE_SIGMOID if fn == "sigmoid" else L.MOE_SOFTMAX)
    n_near, n_flip, _ = check_route(h, e, b, K, fn, idx, gates, loads, E)
    say(f"near-ties {n_near}, flipped {n_flip}")


def test_route_deterministic_and_gates_bias_invariant():
    T, d, E, K = 500, 256, 64, 4
    h = _tokens(T, d, torch.bfloat16, 11)
    e = _centroids(E, d, 12)
    b0 = torch.rand(E, generator=_gen(13), device=DEV) * 0.02 - 0.01
    b1 = b0 + torch.rand(E, generator=_gen(14), device=DEV) * 0.002 - 0.001
    i0, g0, c0 = _route_gpu(h, e, b0, K, L.MOE_SIGMOID)
    i0b, g0b, c0b = _route_gpu(h, e, b0, K, L.MOE_SIGMOID)
    assert torch.equal(i0, i0b) and torch.equal(g0.view(torch.int32), g0b.view(torch.int32))
    assert torch.equal(c0, c0b)
    i1, g1, _ = _route_gpu(h, e, b1, K, L.MOE_SIGMOID)
    same = (i0 == i1).all(dim=1)
    assert same.sum() > 0 and (~same).sum() > 0
    # the bias only picks: identical selections give bit-identical gates
    assert torch.equal(g0[same].view(torch.int32), g1[same].view(torch.int32))


def test_route_worked_example_bias_moves_pick():
    # The "cat" token of the Mixture of Experts designs page, section 1:
    # logits 1.2, 1.0, -0.2, 0.0 (scores 0.77, 0.73, 0.45, 0.50); a bias of
    # (-0.1, +0.1, +0.1, 0) moves its top-1 from E1 to E2 while the gate stays s/s = 1.
    h = torch.tensor([[1.2, 1.0, -0.2, 0.0, 0, 0, 0, 0]], device=DEV, dtype=torch.float32)
    e = torch.zeros((4, 8), device=DEV)
    for i in range(4):
        e[i, i] = 1.0
    i0, g0, c0 = _route_gpu(h, e, torch.zeros(4, device=DEV), 1, L.MOE_SIGMOID)
    i1, g1, c1 = _route_gpu(h, e, torch.tensor([-0.1, 0.1, 0.1, 0.0], device=DEV), 1,
                            L.MOE_SIGMOID)
    assert i0.item() == 0 and i1.item() == 1
    assert g0.item() == 1.0 and g1.item() == 1.0
    assert c0.tolist() == [1, 0, 0, 0] and c1.tolist() == [0, 1, 0, 0]
    i2, g2, _ = _route_gpu(h, e, None, 2, L.MOE_SIGMOID)
    s = 1.0 / (1.0 + np.exp(-np.array([1.2, 1.0])))
    assert i2.tolist() == [[0, 1]]
    assert np.allclose(g2.cpu().numpy()[0], s / s.sum(), atol=GATE_TOL)


DIAG_REL = 1e-4   # fp32 sums over up to T tokens in a fixed chunked order vs fp64


@pytest.mark.parametrize("T,d,E,K,fn,dtype,cf", [
    (64, 128, 8, 2, "sigmoid", torch.float32, None),
    (300, 256, 16, 4, "softmax", torch.bfloat16, None),
    (1000, 512, 64, 6, "sigmoid", torch.bfloat16, 1.0),
    (4096, 7168, 256, 8, "sigmoid", torch.bfloat16, 1.0),
    (2000, 1024, 512, 8, "softmax", torch.float32, 1.25)])
def test_route_stats_and_router_diag(T, d, E, K, fn, dtype, cf):
    say(f"moe_route_stats / moe_router_diag T={T} d={d} E={E} K={K} {fn} {dtype} cf={cf}")
    h = _tokens(T, d, dtype, 90 + T)
    g = _gen(91 + E)
    e = (torch.randn((E, d), generator=g, device=DEV) / math.sqrt(d)).float()
    b = (torch.rand(E, generator=g, device=DEV) * 0.02 - 0.01).float() if fn == "sigmoid" else None
    dt = L.MOE_BF16 if dtype == torch.bfloat16 else L.MOE_F32
    fnc = L.MOE_SIGMOID if fn == "sigmoid" else L.MOE_SOFTMAX
    i32 = dict(dtype=torch.int32, device=DEV)
    idx0, idx1 = torch.empty((T, K), **i32), torch.empty((T, K), **i32)
    g0 = torch.empty((T, K), dtype=torch.float32, device=DEV)
    g1 = torch.empty_like(g0)
    l0, l1 = torch.empty(E, **i32), torch.empty(E, **i32)
    wsb0 = L.moe_route_workspace_size(T, d, E, dt)
    ws0 = torch.empty(max(wsb0, 1), dtype=torch.uint8, device=DEV)
    L.moe_route(T, d, E, K, fnc, h, dt, e, b, idx0, g0, l0, ws0, wsb0)
    wsb = L.moe_route_stats_workspace_size(T, d, E, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    p_mean = torch.empty(E, dtype=torch.float32, device=DEV)
    zsq = torch.empty(1, dtype=torch.float32, device=DEV)
    L.moe_route_stats(T, d, E, K, fnc, h, dt, e, b, idx1, g1, l1, p_mean, zsq, ws, wsb)
    torch.cuda.synchronize()
    # the statistics leave the routing untouched: bit-identical outputs
    assert torch.equal(idx0, idx1) and torch.equal(g0.view(torch.int32), g1.view(torch.int32))
    assert torch.equal(l0, l1)
    idx = idx1.cpu().numpy()
    offsets = None
    kept = None
    if cf is not None:
        C = L.moe_expert_capacity(T, K, E, cf)
        offsets, _, sr, _ = _permute_capacity_gpu(idx1, E, C)
        kept = (sr.cpu().numpy() >= 0).reshape(T, K)
    f = torch.empty(E, dtype=torch.float32, device=DEV)
    diag = torch.zeros(8, dtype=torch.float32, device=DEV)
    L.moe_router_diag(T, E, K, l1, p_mean, zsq, offsets, f, diag)
    torch.cuda.synchronize()
    z = O.router_logits(host_array(h), host_array(e))
    ref = O.router_diagnostics(z, idx, E, kept=kept)   # teacher-forced on the GPU's picks
    pm = p_mean.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(pm - ref["P"]) / ref["P"]) <= DIAG_REL
    assert np.allclose(f.cpu().numpy(), ref["f"], rtol=1e-6, atol=0)
    dv = dict(zip(L.DIAG_FIELDS, diag.cpu().tolist()))
    say(str(dv))
    for k in ("switch_fP", "z_loss", "load_entropy", "max_vio", "dropped"):
        assert abs(dv[k] - ref[k]) <= DIAG_REL * max(1.0, abs(ref[k])), (k, dv[k], ref[k])
    assert (dv["dropped"] > 0) == (cf is not None and kept is not None and not kept.all())


def _permute_gpu(idx, E, h=None):
    T, K = idx.shape
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    row_token = torch.empty(T * K, dtype=torch.int32, device=DEV)
    slot_row = torch.empty(T * K, dtype=torch.int32, device=DEV)
    wsb = L.moe_permute_workspace_size(T, E)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    x_perm = None
    dt = L.MOE_BF16
    if h is not None:
        x_perm = torch.empty((T * K, h.shape[1]), dtype=h.dtype, device=DEV)
        dt = L.MOE_BF16 if h.dtype == torch.bfloat16 else L.MOE_F32
    L.moe_permute(T, h.shape[1] if h is not None else 8, E, K, idx, h, dt, offsets, row_token,
                  slot_row, x_perm, ws, wsb)
    torch.cuda.synchronize()
    return offsets, row_token, slot_row, x_perm


@pytest.mark.parametrize("T,E,K", [(1, 4, 2), (255, 8, 2), (256, 8, 2), (1000, 256, 8),
                                   (3, 64, 2), (4097, 1024, 3), (16384, 256, 8)])
def test_permute_parity(T, E, K):
    say(f"moe_permute T={T} E={E} K={K}")
    rng = np.random.default_rng(T * 7 + E)
    v = rng.random((T, E)).astype(np.float32)
    idx = O.biased_topk(v, None, K)
    off, rt, sr, _ = _permute_gpu(torch.from_numpy(idx).to(DEV), E)
    o_off, o_rt, o_sr = O.permute(idx, E)
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert np.array_equal(rt.cpu().numpy(), o_rt)
    assert np.array_equal(sr.cpu().numpy(), o_sr)


def _permute_capacity_gpu(idx, E, C, h=None):
    T, K = idx.shape
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    row_token = torch.empty(T * K, dtype=torch.int32, device=DEV)
    slot_row = torch.empty(T * K, dtype=torch.int32, device=DEV)
    wsb = L.moe_permute_workspace_size(T, E)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    x_perm = None if h is None else torch.empty((T * K, h.shape[1]), dtype=h.dtype, device=DEV)
    L.moe_permute_capacity(T, h.shape[1] if h is not None else 8, E, K, C, idx, h, L.MOE_BF16,
                           offsets, row_token, slot_row, x_perm, ws, wsb)
    torch.cuda.synchronize()
    return offsets, row_token, slot_row, x_perm


@pytest.mark.parametrize("T,E,K,cf", [(1, 4, 2, 1.0), (300, 8, 2, 1.0), (1000, 64, 4, 0.5),
                                      (4096, 256, 8, 1.0), (4096, 256, 8, 1.25),
                                      (16384, 256, 8, 1.0), (513, 1024, 3, 2.0)])
def test_permute_capacity_parity(T, E, K, cf):
    C = L.moe_expert_capacity(T, K, E, cf)
    assert C == O.expert_capacity(T, K, E, cf)
    say(f"moe_permute_capacity T={T} E={E} K={K} C={C}")
    rng = np.random.default_rng(T + 11 * E)
    # skewed picks so that some experts overflow
    v = rng.random((T, E)).astype(np.float32) * np.linspace(1.0, 2.0, E, dtype=np.float32)
    idx = O.biased_topk(v, None, K)
    off, rt, sr, _ = _permute_capacity_gpu(torch.from_numpy(idx).to(DEV), E, C)
    o_off, o_rt, o_sr, kept = O.permute_capacity(idx, E, C)
    n = int(o_off[-1])
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert np.array_equal(rt.cpu().numpy()[:n], o_rt)
    assert np.all(rt.cpu().numpy()[n:] == -1)
    assert np.array_equal(sr.cpu().numpy(), o_sr)


def test_permute_capacity_edges_and_order_dependence():
    T, E, K, d = 500, 8, 2, 64
    rng = np.random.default_rng(12)
    v = rng.random((T, E)).astype(np.float32)
    v[:, 2] += 0.5                                   # expert 2 over-subscribed
    idx = O.biased_topk(v, None, K)
    h = _tokens(T, d, torch.bfloat16, 13)
    # C = 0: everything dropped; C >= max load: identical to moe_permute
    off, rt, sr, _ = _permute_capacity_gpu(torch.from_numpy(idx).to(DEV), E, 0)
    assert int(off[-1]) == 0 and torch.all(sr == -1) and torch.all(rt == -1)
    c = O.load_count(idx, E)
    a = _permute_gpu(torch.from_numpy(idx).to(DEV), E, h)
    b = _permute_capacity_gpu(torch.from_numpy(idx).to(DEV), E, int(c.max()), h)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # the same copies in another token order: the dropped set changes
    C = O.expert_capacity(T, K, E, 1.0)
    assert c[2] > C
    perm = rng.permutation(T)
    _, _, sr0, _ = _permute_capacity_gpu(torch.from_numpy(idx).to(DEV), E, C)
    _, _, sr1, _ = _permute_capacity_gpu(torch.from_numpy(idx[perm]).to(DEV), E, C)
    k0 = (sr0.cpu().numpy() >= 0).reshape(T, K)
    k1 = (sr1.cpu().numpy() >= 0).reshape(T, K)
    assert not np.array_equal(k1, k0[perm]) and k1.sum() == k0.sum()
    assert np.array_equal(sr1.cpu().numpy(), O.permute_capacity(idx[perm], E, C)[2])


def test_permute_total_collapse_and_gather():
    T, E, K, d = 700, 16, 2, 64
    idx = np.tile(np.array([[3, 9]], dtype=np.int32), (T, 1))
    h = _tokens(T, d, torch.bfloat16, 21)
    off, rt, sr, xp = _permute_gpu(torch.from_numpy(idx).to(DEV), E, h)
    o_off, o_rt, o_sr = O.permute(idx, E)
    assert np.array_equal(off.cpu().numpy(), o_off) and np.array_equal(rt.cpu().numpy(), o_rt)
    assert np.array_equal(sr.cpu().numpy(), o_sr)
    assert torch.equal(xp, h[rt.long()])


def test_permute_skips_invalid_ids():
    T, E, K = 300, 8, 2
    rng = np.random.default_rng(5)
    idx = O.biased_topk(rng.random((T, E)).astype(np.float32), None, K)
    bad = idx.copy()
    bad[7, 1] = -1
    bad[100, 0] = E
    off, rt, sr, _ = _permute_gpu(torch.from_numpy(bad).to(DEV), E)
    keep = (bad >= 0) & (bad < E)
    assert int(off[-1]) == keep.sum() == T * K - 2
    srh = sr.cpu().numpy().reshape(T, K)
    assert srh[7, 1] == -1 and srh[100, 0] == -1
    rth = rt.cpu().numpy()
    assert np.all(rth[T * K - 2:] == -1)
    # the kept copies are a valid stable permutation
    counts = np.bincount(bad[keep], minlength=E)
    assert np.array_equal(np.diff(off.cpu().numpy()), counts)
    for i in range(E):
        seg = rth[off[i]:off[i + 1]]
        assert np.all(np.diff(seg) > 0)


def _swiglu_gpu(x, offsets, row_index, wg, wu, wd, rows, row_scale=None):
    n_groups = wg.shape[0]
    d, f = x.shape[1], wg.shape[1]
    dt = L.MOE_BF16 if x.dtype == torch.bfloat16 else L.MOE_F32
    wsb = L.moe_grouped_swiglu_workspace_size(n_groups, d, f, rows, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    y = torch.zeros((rows, d), dtype=x.dtype, device=DEV)
    L.moe_grouped_swiglu(n_groups, d, f, rows, x.shape[0], offsets, row_index, x, dt, wg, wu, wd,
                         row_scale, y, ws, wsb)
    torch.cuda.synchronize()
    return y


def _weights(E, d, f, dtype, seed):
    g = _gen(seed)
    wg = (torch.randn((E, f, d), generator=g, device=DEV) / math.sqrt(d)).to(dtype)
    wu = (torch.randn((E, f, d), generator=g, device=DEV) / math.sqrt(d)).to(dtype)
    wd = (torch.randn((E, d, f), generator=g, device=DEV) / math.sqrt(f)).to(dtype)
    return wg, wu, wd


SWIGLU_CASES = [
    # T, d, f, E, K, dtype
    (64, 128, 256, 8, 2, torch.float32),
    (333, 256, 192, 5, 2, torch.bfloat16),     # partial column tile (192 = 128 + 64)
    (300, 512, 256, 16, 4, torch.bfloat16),
    (3, 128, 128, 64, 2, torch.bfloat16),      # mostly empty experts
    (1000, 256, 128, 4, 1, torch.bfloat16),    # big groups: many row tiles
    (97, 64, 64, 3, 3, torch.bfloat16),        # K = E_r, smallest aligned sizes
    (150, 96, 80, 6, 2, torch.float32),
    # K spans >= 8 even 64-wide slices and N is a multiple of the column tile
    # in both GEMMs: the one-workgroup-per-CU streaming kernels
    (600, 512, 512, 8, 2, torch.bfloat16),
    (5, 512, 512, 64, 2, torch.bfloat16),      # nearly all experts empty
    (2000, 512, 512, 4, 2, torch.bfloat16),    # 1000-row groups: four row tiles each
    (4000, 1024, 1024, 48, 4, torch.bfloat16),  # several work items per workgroup
    # >= 256 rows per expert on average: the LDS-fed streaming kernel
    (1500, 512, 512, 6, 2, torch.bfloat16),    # ragged groups of ~500 rows
    # longer K (gate/up 1024, down 2048), < 256 rows per expert on average:
    # the register-staged streaming kernel over many slices and items
    (2000, 1024, 2048, 96, 4, torch.bfloat16),  # ~83-row groups, several items per workgroup
    (40, 1024, 1024, 64, 2, torch.bfloat16),    # decode-like: 0-4 rows per group
    (600, 768, 1536, 16, 2, torch.bfloat16),    # 12 and 24 slices: no zero slices padded in
    # weight-DMA kernel, several items per workgroup, items of 12, 13, 16, 20
    # and 24 slices: the three weight stages rotate through the items, so an
    # item ends (and the load side changes item) on every one of them
    (1200, 832, 1024, 96, 4, torch.bfloat16),   # gate/up 13 slices, 3 items per workgroup
    (1200, 768, 1280, 96, 4, torch.bfloat16),   # gate/up 12 slices (the fewest), down 20
    (1000, 1536, 1024, 96, 2, torch.bfloat16),  # down 16 slices, 2-3 items per workgroup
    # K = 512 with four items per workgroup: too few slices for the weight-DMA
    # kernel, the register-staged one takes the gate/up product
    (1000, 512, 2048, 64, 4, torch.bfloat16),
]

# (T, d, f, E, K, hot): the first `hot` experts' scores raised by 0.5, so
# they take most tokens and need several row tiles while the average stays
# below 128 rows (160-row tiles, both operands sent by LDS DMA)
SWIGLU_SKEW_CASES = [
    (1500, 1024, 1024, 64, 4, 4),
    (700, 768, 1280, 80, 2, 2),
]


@pytest.mark.parametrize("T,d,f,E,K,hot", SWIGLU_SKEW_CASES)
def test_grouped_swiglu_skewed_groups(T, d, f, E, K, hot):
    say(f"moe_grouped_swiglu skewed T={T} d={d} f={f} E={E} K={K} hot={hot}")
    rng = np.random.default_rng(T + d + f + hot)
    scores = rng.random((T, E)).astype(np.float32)
    scores[:, :hot] += 0.5
    idx = O.biased_topk(scores, None, K)
    off, rt, _ = O.permute(idx, E)
    loads = np.diff(off)
    assert loads[:hot].min() > 160 and T * K <= 128 * E  # several row tiles, 160-row tiles
    x = _tokens(T, d, torch.bfloat16, 60 + T)
    wg, wu, wd = _weights(E, d, f, torch.bfloat16, 70 + E)
    y = _swiglu_gpu(x, torch.from_numpy(off).to(DEV), torch.from_numpy(rt).to(DEV), wg, wu, wd,
                    T * K)
    ref = O.grouped_swiglu(host_array(x), off, rt, (host_array(wg), host_array(wu), host_array(wd)))
    yh = to_host_f64(y)
    assert rel_err(yh, ref) <= out_tol("bf16")
    for i in range(E):
        lo, hi = off[i], off[i + 1]
        if hi > lo:
            assert rel_err(yh[lo:hi], ref[lo:hi]) <= 4 * out_tol("bf16")


# (T, d, f, E, K, hot, bump): groups of at least 256 rows on average with K and
# N of whole slices and column tiles in both products, so each group's last
# rows, when fewer than 128, run on the second launch over their own tile list
# (both-operands-by-DMA kernel) and the full tiles on the LDS-fed kernel; the
# first `hot` experts' scores raised by `bump` to mix groups of several full
# tiles with small and empty ones
SWIGLU_SPLIT_CASES = [
    (1100, 1024, 768, 4, 1, 0, 0.0),      # every group: full tiles + a small remainder
    (2100, 768, 1024, 16, 2, 4, 0.8),     # small and empty groups beside four large ones
    (2100, 1024, 1024, 16, 2, 4, 0.6),    # small remainders, partial tiles, small groups
    (1300, 768, 1280, 12, 3, 3, 0.45),    # mostly remainders of 128 rows or more (partial)
    (1100, 1024, 768, 1, 1, 0, 0.0),      # one group (a shared expert's form): 4 full tiles + 76 rows
]


@pytest.mark.parametrize("T,d,f,E,K,hot,bump", SWIGLU_SPLIT_CASES)
def test_grouped_swiglu_split_remainders(T, d, f, E, K, hot, bump):
    say(f"moe_grouped_swiglu split T={T} d={d} f={f} E={E} K={K} hot={hot}")
    rng = np.random.default_rng(T + E + hot)
    scores = rng.random((T, E)).astype(np.float32)
    if hot:
        scores[:, :hot] += bump
    idx = O.biased_topk(scores, None, K)
    off, rt, _ = O.permute(idx, E)
    m = np.diff(off)
    assert T * K >= 256 * E and np.any((m % 256 > 0) & (m % 256 < 128))
    x = _tokens(T, d, torch.bfloat16, 80 + T)
    wg, wu, wd = _weights(E, d, f, torch.bfloat16, 90 + E)
    y = _swiglu_gpu(x, torch.from_numpy(off).to(DEV), torch.from_numpy(rt).to(DEV), wg, wu, wd,
                    T * K)
    ref = O.grouped_swiglu(host_array(x), off, rt, (host_array(wg), host_array(wu), host_array(wd)))
    yh = to_host_f64(y)
    assert rel_err(yh, ref) <= out_tol("bf16")
    for i in range(E):
        lo, hi = off[i], off[i + 1]
        if hi > lo:
            assert rel_err(yh[lo:hi], ref[lo:hi]) <= 4 * out_tol("bf16"), i


def _random_swiglu_shapes(n):
    """n seeded shapes over the kernels' selection rules: K of 8 to 28 slices,
    N a multiple of the column tile or not, 2 to 600 rows per expert on
    average, 4 to 128 experts (the oracle's work kept to a few seconds); every
    other one with both products of whole slices and column tiles."""
    out = []
    i = 0
    while len(out) < n:
        rng = np.random.default_rng(1000 + i)
        i += 1
        if i % 2:  # both products of whole slices and column tiles: the streaming kernels
            d = int(rng.choice([768, 1024, 1280, 1536, 1792]))
            f = int(rng.choice([768, 1024, 1280, 1536]))
        else:
            d = int(rng.choice([512, 640, 768, 896, 1024, 1280, 1536]))
            f = int(rng.choice([256, 384, 512, 768, 1024, 1280, 1536, 2048]))
        E = int(rng.choice([4, 8, 16, 32, 64, 128]))
        K = int(rng.integers(1, min(8, E) + 1))
        avg = int(rng.choice([2, 20, 80, 130, 200, 300, 600]))
        T = max(1, avg * E // K)
        if T * K * d * f * 6 <= 6e9:
            out.append((T, d, f, E, K, 1000 + i - 1))
    return out


@pytest.mark.parametrize("T,d,f,E,K,seed", _random_swiglu_shapes(16))
def test_grouped_swiglu_random_shapes(T, d, f, E, K, seed):
    say(f"moe_grouped_swiglu random T={T} d={d} f={f} E={E} K={K} seed={seed}")
    rng = np.random.default_rng(seed)
    idx = O.biased_topk(rng.random((T, E)).astype(np.float32), None, K)
    off, rt, _ = O.permute(idx, E)
    x = _tokens(T, d, torch.bfloat16, seed)
    wg, wu, wd = _weights(E, d, f, torch.bfloat16, seed + 1)
    y = _swiglu_gpu(x, torch.from_numpy(off).to(DEV), torch.from_numpy(rt).to(DEV), wg, wu, wd,
                    T * K)
    ref = O.grouped_swiglu(host_array(x), off, rt, (host_array(wg), host_array(wu), host_array(wd)))
    yh = to_host_f64(y)
    assert rel_err(yh, ref) <= out_tol("bf16")
    for i in range(E):
        lo, hi = off[i], off[i + 1]
        if hi > lo:
            assert rel_err(yh[lo:hi], ref[lo:hi]) <= 4 * out_tol("bf16"), i


@pytest.mark.parametrize("T,d,f,E,K,dtype", SWIGLU_CASES)
def test_grouped_swiglu_parity(T, d, f, E, K, dtype):
    say(f"moe_grouped_swiglu T={T} d={d} f={f} E={E} K={K} {dtype}")
    rng = np.random.default_rng(T + d + f)
    idx = O.biased_topk(rng.random((T, E)).astype(np.float32), None, K)
    off, rt, _ = O.permute(idx, E)
    x = _tokens(T, d, dtype, 40 + T)
    wg, wu, wd = _weights(E, d, f, dtype, 50 + E)
    y = _swiglu_gpu(x, torch.from_numpy(off).to(DEV), torch.from_numpy(rt).to(DEV), wg, wu, wd,
                    T * K)
    w_host = (host_array(wg), host_array(wu), host_array(wd))
    ref = O.grouped_swiglu(host_array(x), off, rt, w_host)
    err = rel_err(to_host_f64(y), ref)
    say(f"max|d|/max|ref| = {err:.3e}")
    assert err <= out_tol("bf16" if dtype == torch.bfloat16 else "f32")
    # per expert too, so a wrong or missing expert cannot hide behind the others
    for i in range(E):
        lo, hi = off[i], off[i + 1]
        if hi > lo:
            assert rel_err(to_host_f64(y)[lo:hi], ref[lo:hi]) <= 4 * out_tol(
                "bf16" if dtype == torch.bfloat16 else "f32")


@pytest.mark.parametrize("T,d,f,E,K", [
    (333, 256, 192, 5, 2),     # one-tile-per-workgroup kernel, partial column tile
    (3, 128, 128, 64, 2),      # mostly empty experts
    (300, 512, 256, 16, 4),    # register-staged streaming kernel
    (1500, 512, 512, 6, 2),    # LDS-fed streaming kernel
    (2000, 1024, 1024, 40, 2),  # register-staged streaming kernel, K = 1024
])
def test_grouped_swiglu_train_outputs(T, d, f, E, K):
    """The training form: the same y as the inference form (bit for bit: the
    same kernels, with extra output passes), and a|u against the oracle's
    projections; rows past the last group are left alone."""
    say(f"moe_grouped_swiglu_train T={T} d={d} f={f} E={E} K={K}")
    rng = np.random.default_rng(T + d + f + 1)
    idx = O.biased_topk(rng.random((T, E)).astype(np.float32), None, K)
    off, rt, _ = O.permute(idx, E)
    rows = T * K + 3                                   # three rows outside every group
    rt_pad = np.concatenate([rt, np.full(3, -1, np.int32)])
    x = _tokens(T, d, torch.bfloat16, 90 + T)
    wg, wu, wd = _weights(E, d, f, torch.bfloat16, 91 + E)
    offs, ri = torch.from_numpy(off).to(DEV), torch.from_numpy(rt_pad).to(DEV)
    y_inf = _swiglu_gpu(x, offs, ri, wg, wu, wd, rows)
    wsb = L.moe_grouped_swiglu_workspace_size(E, d, f, rows, L.MOE_BF16)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    y = torch.zeros((rows, d), dtype=torch.bfloat16, device=DEV)
    au = torch.full((rows, 2 * f), 7.0, dtype=torch.bfloat16, device=DEV)
    L.moe_grouped_swiglu_train(E, d, f, rows, T, offs, ri, x, L.MOE_BF16, wg, wu, wd, None, y,
                               au, ws, wsb)
    torch.cuda.synchronize()
    assert torch.equal(y, y_inf)
    auh = to_host_f64(au)
    assert np.all(auh[T * K:] == 7.0)
    w_host = (host_array(wg), host_array(wu), host_array(wd))
    ref = O.grouped_gate_up(host_array(x), off, rt, w_host)
    for half in (slice(0, f), slice(f, 2 * f)):       # a and u separately
        err = rel_err(auh[:T * K, half], ref[:, half])
        say(f"a|u half {half.start}: max|d|/max|ref| = {err:.3e}")
        assert err <= out_tol("bf16")


@pytest.mark.parametrize("d,f,extra_empty", [(512, 512, 0), (512, 512, 16), (256, 192, 0),
                                              (1024, 1024, 16)])
def test_grouped_swiglu_many_row_tiles_per_group(d, f, extra_empty):
    """Groups of 5, 6 and 9 row tiles (256 rows each), walked in blocks of
    four row tiles by all column tiles with a partial last block; an empty
    group between them.  (512, 512): the LDS-fed streaming kernel, or with 16
    more empty groups (under 256 rows per group on average) the
    register-staged one; (256, 192): the one-tile-per-workgroup kernel;
    (1024, 1024) with 16 empty groups: the register-staged one at K = 1024."""
    sizes = [1100, 0, 1500, 2200] + [0] * extra_empty
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = int(off[-1])
    say(f"many row tiles per group: d={d} f={f} groups {sizes}")
    x = _tokens(T, d, torch.bfloat16, 95)
    wg, wu, wd = _weights(len(sizes), d, f, torch.bfloat16, 96)
    ri = np.random.default_rng(97).permutation(T).astype(np.int32)
    y = _swiglu_gpu(x, torch.from_numpy(off).to(DEV), torch.from_numpy(ri).to(DEV), wg, wu, wd, T)
    w_host = (host_array(wg), host_array(wu), host_array(wd))
    ref = O.grouped_swiglu(host_array(x), off, ri, w_host)
    yh = to_host_f64(y)
    for i in range(len(sizes)):
        lo, hi = off[i], off[i + 1]
        if hi > lo:
            assert rel_err(yh[lo:hi], ref[lo:hi]) <= out_tol("bf16"), i


def test_grouped_swiglu_row_scale_and_direct_rows():
    T, d, f, E = 257, 128, 128, 3
    x = _tokens(T, d, torch.bfloat16, 61)
    wg, wu, wd = _weights(E, d, f, torch.bfloat16, 62)
    off = np.array([0, 100, 100, 257], dtype=np.int32)    # one empty group
    scale = torch.rand(T, generator=_gen(63), device=DEV)
    y = _swiglu_gpu(x, torch.from_numpy(off).to(DEV), None, wg, wu, wd, T, scale)
    ref = O.grouped_swiglu(host_array(x), off, None,
                           (host_array(wg), host_array(wu), host_array(wd)))
    ref = ref * scale.cpu().numpy().astype(np.float64)[:, None]
    assert rel_err(to_host_f64(y), ref) <= out_tol("bf16")


@pytest.mark.parametrize("T,off,d", [
    # < 256 rows per group on average: the register-staged streaming kernel
    (700, [0, 300, 300, 301, 590, 700], 512),
    # >= 256 rows per group on average: the LDS-fed one (a 589-row group spans three row tiles)
    (1300, [0, 600, 600, 601, 1190, 1300], 512),
    # the register-staged kernel at K = 1024
    (700, [0, 300, 300, 301, 590, 700], 1024),
])
def test_grouped_swiglu_streaming_row_scale_direct_rows_and_bad_rows(T, off, d):
    """The streaming kernels (d, f >= 512) with a per-row scale, identity rows
    (row_index NULL) and gathered rows with out-of-range entries; empty and
    1-row groups."""
    say(f"streaming swiglu T={T} groups={off} d=f={d}")
    f, E = d, 5
    x = _tokens(T, d, torch.bfloat16, 81)
    wg, wu, wd = _weights(E, d, f, torch.bfloat16, 82)
    w_host = (host_array(wg), host_array(wu), host_array(wd))
    off = np.array(off, dtype=np.int32)
    scale = torch.rand(T, generator=_gen(83), device=DEV)
    y = _swiglu_gpu(x, torch.from_numpy(off).to(DEV), None, wg, wu, wd, T, scale)
    ref = O.grouped_swiglu(host_array(x), off, None, w_host)
    ref = ref * scale.cpu().numpy().astype(np.float64)[:, None]
    assert rel_err(to_host_f64(y), ref) <= out_tol("bf16")
    ri = (np.arange(T, dtype=np.int32) * 7) % T
    ri[[0, 299, 450]] = [-1, T, 1 << 30]
    y = _swiglu_gpu(x, torch.from_numpy(off).to(DEV), torch.from_numpy(ri).to(DEV), wg, wu, wd,
                    T)
    yh = to_host_f64(y)
    assert np.all(yh[[0, 299, 450]] == 0)
    ok = np.ones(T, bool)
    ok[[0, 299, 450]] = False
    ref = O.grouped_swiglu(host_array(x), off, np.where(ok, ri, 0).astype(np.int32), w_host)
    assert rel_err(yh[ok], ref[ok]) <= out_tol("bf16")


def test_grouped_swiglu_bad_row_index_reads_zero_row():
    T, d, f, E = 40, 64, 64, 2
    x = _tokens(T, d, torch.bfloat16, 71)
    wg, wu, wd = _weights(E, d, f, torch.bfloat16, 72)
    off = np.array([0, 20, 40], dtype=np.int32)
    ri = np.arange(40, dtype=np.int32) % T
    ri[5] = -3
    ri[30] = 10_000
    y = _swiglu_gpu(x, torch.from_numpy(off).to(DEV), torch.from_numpy(ri).to(DEV), wg, wu, wd, 40)
    yh = to_host_f64(y)
    assert np.all(yh[5] == 0) and np.all(yh[30] == 0)   # SwiGLU(0) = 0


def _combine_gpu(h, y_shared, y_perm, slot_row, gates, E_s):
    T, d = h.shape
    K = gates.shape[1]
    dt = L.MOE_BF16 if h.dtype == torch.bfloat16 else L.MOE_F32
    y = torch.empty_like(h)
    L.moe_combine(T, d, K, E_s, h, y_shared, y_perm, slot_row, gates, dt, y)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("T,d,K,E_s,dtype,drop", [
    (64, 128, 2, 0, torch.float32, False),
    (333, 256, 8, 1, torch.bfloat16, False),
    (100, 7168, 8, 2, torch.bfloat16, False),
    (31, 64, 1, 0, torch.bfloat16, False),
    # rows of 125 and 65 16-byte chunks: a ragged tail per wave; row strides
    # that are not powers of two
    (150, 1000, 4, 1, torch.bfloat16, False),
    (77, 520, 3, 0, torch.bfloat16, True),
    (500, 7168, 8, 1, torch.bfloat16, True),
    # small batches split each row over several waves: 129 chunks in two
    # shares of 65 and 64; the decode shape in eight shares of 112
    (40, 1032, 5, 1, torch.bfloat16, False),
    (64, 7168, 8, 1, torch.bfloat16, False),
])
def test_combine_parity(T, d, K, E_s, dtype, drop):
    say(f"moe_combine T={T} d={d} K={K} E_s={E_s} {dtype} dropped slots={drop}")
    rng = np.random.default_rng(T + K)
    h = _tokens(T, d, dtype, 81)
    yp = _tokens(T * K, d, dtype, 82, 0.3)
    ys = _tokens(E_s * T, d, dtype, 83, 0.5) if E_s else None
    perm = rng.permutation(T * K).astype(np.int32)
    if drop:   # copies dropped by a capacity limit carry slot -1 and add nothing
        perm[rng.random(T * K) < 0.2] = -1
    g = rng.random((T, K)).astype(np.float32)
    g /= g.sum(1, keepdims=True)
    y = _combine_gpu(h, ys, yp, torch.from_numpy(perm).to(DEV), torch.from_numpy(g).to(DEV), E_s)
    ysh = to_host_f64(ys).reshape(E_s, T, d).sum(0) if E_s else None
    ref = O.combine(host_array(h), ysh, to_host_f64(yp), perm, g)
    yh = to_host_f64(y)
    # fp32 accumulation then one rounding of the output
    tol = (2.0 ** -7) * np.abs(ref) + 1e-6 if dtype == torch.bfloat16 else 1e-5 * np.abs(ref) + 1e-6
    assert np.all(np.abs(yh - ref) <= tol)


def _bias_gpu(T, K, gamma, loads, b):
    E = loads.shape[0]
    lt = torch.from_numpy(loads.astype(np.int32)).to(DEV)
    bt = torch.from_numpy(b.astype(np.float32)).to(DEV)
    st = torch.zeros(4, dtype=torch.int32, device=DEV)
    L.moe_bias_update(T, E, K, gamma, lt, bt, st)
    torch.cuda.synchronize()
    sth = st.cpu()
    return bt.cpu().numpy(), (int(sth[0]), int(sth[1]), float(sth[2:3].view(torch.float32)[0]))


def test_bias_update_worked_example(golden_dir):
    import json
    import os
    with open(os.path.join(golden_dir, "bias_update_example.json")) as f:
        ex = json.load(f)
    b1, st = _bias_gpu(ex["T"], ex["K"], ex["gamma"], np.array(ex["loads"]), np.array(ex["b0"]))
    assert np.array_equal(b1, np.array(ex["b1"], dtype=np.float32))
    assert st[0] == 3 and st[1] == 0 and st[2] == pytest.approx(ex["max_vio"], rel=1e-7)


@pytest.mark.parametrize("T,E,K,gamma", [(64, 8, 2, 0.1), (4096, 256, 8, 0.001),
                                         (5, 4, 3, 0.5), (16384, 256, 8, 0.0),
                                         (1000, 1024, 7, 0.01)])
def test_bias_update_parity(T, E, K, gamma):
    rng = np.random.default_rng(E + K)
    loads = rng.multinomial(T * K, np.ones(E) / E).astype(np.int32)
    if K * T % E == 0:
        loads[0] = K * T // E  # one expert exactly at the fair share: bias unchanged
    b = (rng.random(E) * 0.02 - 0.01).astype(np.float32)
    b1, st = _bias_gpu(T, K, gamma, loads, b)
    ref = O.bias_update(b, loads, T, K, gamma)
    assert np.array_equal(b1.view(np.uint32), ref.view(np.uint32))
    ls = O.load_stats(loads, T, K)
    assert st[0] == ls["max_load"] and st[1] == ls["min_load"]
    assert st[2] == pytest.approx(ls["max_vio"], rel=1e-6, abs=1e-7)


@pytest.mark.parametrize("T,d,f,E,K,E_s,dtype", [
    (333, 256, 192, 5, 2, 1, torch.bfloat16),    # tile kernel (N not a multiple of the column tile)
    (300, 512, 256, 16, 4, 2, torch.bfloat16),   # streaming kernels, two shared experts
    (100, 512, 256, 8, 2, 0, torch.bfloat16),    # no shared experts
    (64, 128, 256, 8, 2, 1, torch.float32),      # fp32: two grouped launches inside
    (90, 64, 32, 6, 3, 2, torch.float32),
])
def test_experts_swiglu_parity(T, d, f, E, K, E_s, dtype):
    """moe_experts_swiglu: routed rows first (y_perm), then the shared experts'
    rows (token order, expert by expert), each against the oracle's grouped
    SwiGLU of the same rows."""
    say(f"moe_experts_swiglu T={T} d={d} f={f} E={E} K={K} E_s={E_s} {dtype}")
    rng = np.random.default_rng(T + E + E_s)
    idx = O.biased_topk(rng.random((T, E)).astype(np.float32), None, K)
    off, rt, _ = O.permute(idx, E)
    x = _tokens(T, d, dtype, 60 + T)
    wg, wu, wd = _weights(E, d, f, dtype, 61 + E)
    sw = _weights(max(E_s, 1), d, f, dtype, 62 + E)
    dt = L.MOE_BF16 if dtype == torch.bfloat16 else L.MOE_F32
    wsb = L.moe_experts_swiglu_workspace_size(E, E_s, T, K, d, f, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    y = torch.zeros((T * K + E_s * T, d), dtype=dtype, device=DEV)
    L.moe_experts_swiglu(E, E_s, T, K, d, f, torch.from_numpy(off).to(DEV),
                         torch.from_numpy(rt).to(DEV), x, dt, wg, wu, wd,
                         *(sw if E_s else (None, None, None)), y, ws, wsb)
    torch.cuda.synchronize()
    kind = "bf16" if dtype == torch.bfloat16 else "f32"
    yh = to_host_f64(y)
    ref = O.grouped_swiglu(host_array(x), off, rt, (host_array(wg), host_array(wu), host_array(wd)))
    assert rel_err(yh[:T * K], ref) <= out_tol(kind)
    if E_s:
        sh_off = (np.arange(E_s + 1) * T).astype(np.int32)
        sh_rows = np.tile(np.arange(T, dtype=np.int32), E_s)
        ref_s = O.grouped_swiglu(host_array(x), sh_off, sh_rows, tuple(host_array(w) for w in sw))
        assert rel_err(yh[T * K:], ref_s) <= out_tol(kind)
