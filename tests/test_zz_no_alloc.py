"""The entry point that allocates nothing, moe_grouped_swiglu_noalloc, through
the C ABI: the same bits as moe_grouped_swiglu with a caller workspace, and
within tolerance of the oracle, on two calls in a row -- the second smaller,
so it runs over what the first left in the library's scratch array."""
import math

import numpy as np
import pytest
import torch

from gpu_common import out_tol, rel_err, say, to_host_f64
from oracle import moe_oracle as O
from sparse_mixture_experts_biased_amd import _lib as L
from synthetic import host_array

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _case(T, d, f, E, K, dtype, seed):
    rng = np.random.default_rng(seed)
    idx = O.biased_topk(rng.random((T, E)).astype(np.float32), None, K)
    off, rt, sr = O.permute(idx, E)
    g = _gen(seed)
    x = torch.randn((T, d), generator=g, device=DEV).to(dtype)
    wg = (torch.randn((E, f, d), generator=g, device=DEV) / math.sqrt(d)).to(dtype)
    wu = (torch.randn((E, f, d), generator=g, device=DEV) / math.sqrt(d)).to(dtype)
    wd = (torch.randn((E, d, f), generator=g, device=DEV) / math.sqrt(f)).to(dtype)
    # gates as row scales, in permuted-row order
    gates = torch.rand((T * K,), generator=g, device=DEV)
    return dict(T=T, d=d, f=f, E=E, K=K, dtype=dtype, off=off, rt=rt, x=x, w=(wg, wu, wd),
                offs=torch.from_numpy(off).to(DEV), ri=torch.from_numpy(rt).to(DEV),
                scale=gates)


def _with_workspace(c, dt):
    rows = c["T"] * c["K"]
    wsb = L.moe_grouped_swiglu_workspace_size(c["E"], c["d"], c["f"], rows, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    y = torch.zeros((rows, c["d"]), dtype=c["dtype"], device=DEV)
    L.moe_grouped_swiglu(c["E"], c["d"], c["f"], rows, c["T"], c["offs"], c["ri"], c["x"], dt,
                         *c["w"], c["scale"], y, ws, wsb)
    return y


def _noalloc(c, dt):
    rows = c["T"] * c["K"]
    y = torch.zeros((rows, c["d"]), dtype=c["dtype"], device=DEV)
    L.moe_grouped_swiglu_noalloc(c["E"], c["d"], c["f"], rows, c["T"], c["offs"], c["ri"],
                                 c["x"], dt, *c["w"], c["scale"], y)
    return y


def _check(c, y_na, y_ws, dt):
    assert torch.equal(y_na, y_ws), "no-alloc form differs from the workspace form"
    w_host = tuple(host_array(t) for t in c["w"])
    ref = O.grouped_swiglu(host_array(c["x"]), c["off"], c["rt"], w_host)
    ref = ref * c["scale"].cpu().numpy().astype(np.float64)[:, None]
    err = rel_err(to_host_f64(y_na), ref)
    tol = out_tol("bf16" if dt == L.MOE_BF16 else "f32")
    say(f"  max|d|/max|ref| = {err:.3e} (tol {tol})")
    assert err <= tol


@pytest.mark.parametrize("first,second,dtype", [
    # (T, d, f, E, K): decode-like DeepSeek-V3 routing on a narrower layer, then smaller
    ((64, 1024, 1024, 64, 8), (16, 1024, 1024, 64, 8), torch.bfloat16),
    # streaming kernels (K >= 8 slices, whole column tiles), then a ragged small call
    ((600, 512, 512, 8, 2), (97, 512, 512, 8, 2), torch.bfloat16),
    # fp32 tiles
    ((150, 96, 80, 6, 2), (33, 96, 80, 6, 2), torch.float32),
])
def test_noalloc_matches_workspace_form_twice(first, second, dtype):
    dt = L.MOE_BF16 if dtype == torch.bfloat16 else L.MOE_F32
    for n, shape in enumerate((first, second)):
        say(f"call {n + 1}: T={shape[0]} d={shape[1]} f={shape[2]} E={shape[3]} K={shape[4]} "
            f"{dtype}")
        c = _case(*shape, dtype, seed=100 + 10 * n + shape[0])
        y_na = _noalloc(c, dt)
        y_ws = _with_workspace(c, dt)
        torch.cuda.synchronize()
        _check(c, y_na, y_ws, dt)


def test_noalloc_rejects_oversize_before_launch():
    # DeepSeek-V3 prefill routed rows need ~128 MiB of activations: refused
    rows, d, f, E = 32768, 7168, 2048, 256
    need = L.moe_grouped_swiglu_workspace_size(E, d, f, rows, L.MOE_BF16)
    assert need > (32 << 20)
    P = 256
    lib = L.load()
    rc = lib.moe_grouped_swiglu_noalloc(E, d, f, rows, 4096, P, P, P, L.MOE_BF16, P, P, P, None,
                                        P, None)
    assert rc == L.MOE_ERR_UNSUPPORTED
    assert "moe_grouped_swiglu with a workspace" in L.moe_last_error()
