"""The C-ABI library: it loads, exports every function include/moe.h declares,
and rejects invalid arguments on the host without launching anything (CPU
only: none of these calls reaches the GPU)."""
import ctypes
import os
import re

import pytest

from sparse_mixture_experts_biased_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_entry_points():
    names = _declared()
    for n in ("moe_route", "moe_permute", "moe_grouped_swiglu", "moe_combine",
              "moe_bias_update"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = L.load()
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(_declared()) == sorted(L.EXPORTED)


def test_version():
    assert "gfx950" in L.moe_version()


def _st(rc):
    return rc, L.moe_last_error()


def test_route_rejects_bad_arguments():
    lib = L.load()
    P = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    assert _st(lib.moe_route(0, 128, 8, 2, 0, P, 1, P, None, P, P, P, P, 1 << 30, None))[0] == L.MOE_ERR_INVALID_ARG
    rc, msg = _st(lib.moe_route(64, 128, 8, 9, 0, P, 1, P, None, P, P, P, P, 1 << 30, None))
    assert rc == L.MOE_ERR_INVALID_ARG and "K=9 > E_r=8" in msg
    assert lib.moe_route(64, 128, 32, 17, 0, P, 1, P, None, P, P, P, P, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route(64, 128, 8, 2, 0, None, 1, P, None, P, P, P, P, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route(64, 100, 8, 2, 0, P, 1, P, None, P, P, P, P, 1 << 30, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_route(64, 128, 1024, 2, 0, P, 1, P, None, P, P, P, P, 1 << 30, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_route(64, 128, 8, 2, 7, P, 1, P, None, P, P, P, P, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route(64, 128, 8, 2, 0, P, 5, P, None, P, P, P, P, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    # bf16 tokens run the matrix-core logits: d_model % 32 and a workspace are required
    assert lib.moe_route(64, 136, 8, 2, 0, P, 1, P, None, P, P, P, P, 1 << 30, None) == L.MOE_ERR_UNSUPPORTED
    rc, msg = _st(lib.moe_route(64, (1 << 20) + 32, 8, 2, 0, P, 1, P, None, P, P, P, P, 1 << 40, None))
    assert rc == L.MOE_ERR_UNSUPPORTED and "1048576" in msg
    need = L.moe_route_workspace_size(4096, 7168, 256, L.MOE_BF16)
    assert need >= 4096 * 256 * 4
    rc, msg = _st(lib.moe_route(4096, 7168, 256, 8, 0, P, 1, P, None, P, P, P, P, need - 1, None))
    assert rc == L.MOE_ERR_INVALID_ARG and "workspace" in msg
    assert lib.moe_route(4096, 7168, 256, 8, 0, P, 1, P, None, P, P, P, None, need, None) == L.MOE_ERR_INVALID_ARG
    assert L.moe_route_workspace_size(64, 128, 8, L.MOE_F32) == 0


def test_permute_rejects_bad_arguments():
    lib = L.load()
    P = ctypes.c_void_p(16)
    need = L.moe_permute_workspace_size(100, 8)
    assert need > 0
    rc, msg = _st(lib.moe_permute(100, 64, 8, 2, P, None, 1, P, P, P, None, P, need - 1, None))
    assert rc == L.MOE_ERR_INVALID_ARG and "workspace" in msg
    assert lib.moe_permute(100, 64, 8, 2, P, None, 1, P, P, P, P, P, need, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(100, 64, 2000, 2, P, None, 1, P, P, P, None, P, 1 << 30, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_permute(100, 64, 8, 0, P, None, 1, P, P, P, None, P, need, None) == L.MOE_ERR_INVALID_ARG


def test_expert_capacity_and_capacity_permute_arguments():
    # C = ceil(CF*T*K/E_r) on the host, no device work
    assert L.moe_expert_capacity(4096, 8, 256, 1.0) == 128
    assert L.moe_expert_capacity(4096, 8, 256, 1.25) == 160
    assert L.moe_expert_capacity(10, 1, 4, 1.0) == 3
    assert L.moe_expert_capacity(10, 1, 4, 0.0) == 0
    assert L.moe_expert_capacity(10, 1, 4, -0.5) == -1
    assert L.moe_expert_capacity(10, 1, 4, float("nan")) == -1
    assert L.moe_expert_capacity(0, 1, 4, 1.0) == -1
    lib = L.load()
    P = ctypes.c_void_p(16)
    need = L.moe_permute_workspace_size(100, 8)
    rc, msg = _st(lib.moe_permute_capacity(100, 64, 8, 2, -1, P, None, 1, P, P, P, None, P, need,
                                           None))
    assert rc == L.MOE_ERR_INVALID_ARG and "capacity" in msg
    rc, msg = _st(lib.moe_permute_capacity(100, 64, 8, 2, 5, P, None, 1, P, P, P, None, P,
                                           need - 1, None))
    assert rc == L.MOE_ERR_INVALID_ARG and "workspace" in msg
    assert lib.moe_permute_capacity(100, 64, 8, 9, 5, P, None, 1, P, P, P, None, P, need,
                                    None) == L.MOE_ERR_INVALID_ARG


def test_route_stats_and_router_diag_arguments():
    lib = L.load()
    P = ctypes.c_void_p(16)
    base = L.moe_route_workspace_size(4096, 7168, 256, L.MOE_BF16)
    need = L.moe_route_stats_workspace_size(4096, 7168, 256, L.MOE_BF16)
    assert need >= base + 4096 * 256 * 4 + 4096 * 4
    assert L.moe_route_stats_workspace_size(64, 128, 8, L.MOE_F32) >= 64 * 8 * 4 + 64 * 4
    rc, msg = _st(lib.moe_route_stats(4096, 7168, 256, 8, 0, P, 1, P, None, P, P, P, P, P, P,
                                      need - 1, None))
    assert rc == L.MOE_ERR_INVALID_ARG and "workspace" in msg
    rc, msg = _st(lib.moe_route_stats(4096, 7168, 256, 8, 0, P, 1, P, None, P, P, P, None, P, P,
                                      need, None))
    assert rc == L.MOE_ERR_INVALID_ARG and "null" in msg
    assert lib.moe_route_stats(64, 128, 8, 9, 0, P, 0, P, None, P, P, P, P, P, P, 1 << 20,
                               None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_router_diag(64, 8, 9, P, P, P, None, None, P, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_router_diag(64, 8, 2, P, None, P, None, None, P, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_router_diag(64, 8, 2, P, P, P, None, None, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_router_diag(64, 2048, 2, P, P, P, None, None, P, None) == L.MOE_ERR_UNSUPPORTED
    assert ctypes.sizeof(L.MoeRouterDiag) == 32


def test_backward_entry_points_reject_bad_arguments():
    lib = L.load()
    P = ctypes.c_void_p(16)
    need = L.moe_grouped_swiglu_backward_workspace_size(8, 256, 512, 1000)
    assert need >= 1000 * 4 * 512 * 2            # a|u and da|du at least
    args = [8, 256, 512, 1000, 500, P, P, P, 1, P, P, P, P, P, None, P, P, P, P, P]
    rc, msg = _st(lib.moe_grouped_swiglu_backward(*args, need - 1, None))
    assert rc == L.MOE_ERR_INVALID_ARG and "workspace" in msg
    bad = list(args); bad[8] = 0                   # fp32
    assert lib.moe_grouped_swiglu_backward(*bad, need, None) == L.MOE_ERR_UNSUPPORTED
    bad = list(args); bad[1] = 200                 # d_model % 64
    assert lib.moe_grouped_swiglu_backward(*bad, need, None) == L.MOE_ERR_UNSUPPORTED
    bad = list(args); bad[11] = None               # w_gu_t
    assert lib.moe_grouped_swiglu_backward(*bad, need, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_backward(10, 64, 2, P, P, P, P, 0, P, P, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine_backward(10, 64, 2, P, P, P, P, 1, None, P, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_backward(10, 60, 2, P, P, P, P, 1, P, P, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine_backward(1 << 17, 8192, 8, P, P, P, P, 1, P, P, None) == \
        L.MOE_ERR_UNSUPPORTED   # y_perm of 2^17 * 8 rows x 8192 bf16 = 16 GiB
    assert lib.moe_route_backward(10, 64, 8, 9, 0, P, 1, P, P, P, P, P, P, P, P, None) == \
        L.MOE_ERR_INVALID_ARG
    assert lib.moe_route_backward(10, 64, 8, 2, 0, P, 0, P, P, P, P, P, P, P, P, None) == \
        L.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_backward(10, 60, 8, 2, 0, P, 1, P, P, P, P, P, P, P, P, None) == \
        L.MOE_ERR_UNSUPPORTED   # d_model not a multiple of 8
    assert lib.moe_transpose_experts(2, 10, 20, P, 1, P, 9, 0, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_transpose_experts(2, 10, 20, P, 0, P, 10, 0, None) == L.MOE_ERR_UNSUPPORTED


def test_grouped_swiglu_rejects_bad_arguments():
    lib = L.load()
    P = ctypes.c_void_p(16)
    need = L.moe_grouped_swiglu_workspace_size(8, 256, 512, 1000, L.MOE_BF16)
    assert need >= 1000 * 512 * 2
    assert L.moe_grouped_swiglu_workspace_size(8, 256, 512, 1000, L.MOE_F32) >= 1000 * 512 * 4
    rc, msg = _st(lib.moe_grouped_swiglu(8, 256, 512, 1000, 500, P, P, P, 1, P, P, P, None, P, P,
                                         need - 1, None))
    assert rc == L.MOE_ERR_INVALID_ARG and "workspace" in msg
    rc, msg = _st(lib.moe_grouped_swiglu(8, 200, 512, 1000, 500, P, P, P, 1, P, P, P, None, P, P,
                                         need, None))
    assert rc == L.MOE_ERR_UNSUPPORTED and "multiples of 64" in msg
    assert lib.moe_grouped_swiglu(8, 256, 512, 1000, 500, P, None, P, 1, P, P, P, None, P, P,
                                  need, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_grouped_swiglu(8, 256, 512, 1000, 500, None, P, P, 1, P, P, P, None, P, P,
                                  need, None) == L.MOE_ERR_INVALID_ARG
    # the matrix-core path needs every bf16 operand under 2 GiB
    big = L.moe_grouped_swiglu_workspace_size(8, 7168, 2048, 1 << 19, L.MOE_BF16)
    rc, msg = _st(lib.moe_grouped_swiglu(8, 7168, 2048, 1 << 19, 1 << 18, P, P, P, 1, P, P, P,
                                         None, P, P, big, None))
    assert rc == L.MOE_ERR_UNSUPPORTED and "2 GiB" in msg
    # zero rows is a valid no-op
    assert lib.moe_grouped_swiglu(8, 256, 512, 0, 500, P, P, P, 1, P, P, P, None, P, P,
                                  need, None) == L.MOE_OK
    # the training form: bf16 only, a|u required, otherwise the same checks
    rc, msg = _st(lib.moe_grouped_swiglu_train(8, 256, 512, 1000, 500, P, P, P, 0, P, P, P,
                                               None, P, P, P, need, None))
    assert rc == L.MOE_ERR_UNSUPPORTED and "bf16" in msg
    rc, msg = _st(lib.moe_grouped_swiglu_train(8, 256, 512, 1000, 500, P, P, P, 1, P, P, P,
                                               None, P, None, P, need, None))
    assert rc == L.MOE_ERR_INVALID_ARG and "null" in msg
    rc, msg = _st(lib.moe_grouped_swiglu_train(8, 256, 512, 1000, 500, P, P, P, 1, P, P, P,
                                               None, P, P, P, need - 1, None))
    assert rc == L.MOE_ERR_INVALID_ARG and "moe_grouped_swiglu_train: workspace" in msg
    assert lib.moe_grouped_swiglu_train(8, 256, 512, 0, 500, P, P, P, 1, P, P, P, None, P, P, P,
                                        need, None) == L.MOE_OK


def test_experts_swiglu_rejects_bad_arguments():
    lib = L.load()
    P = ctypes.c_void_p(16)
    T, K, E, Es, d, f = 4096, 8, 256, 1, 7168, 2048
    need = L.moe_experts_swiglu_workspace_size(E, Es, T, K, d, f, L.MOE_BF16)
    # activations of every routed and shared row, their row index, the tile list
    assert need >= (T * K + Es * T) * (2 * f + 4)
    assert L.moe_experts_swiglu_workspace_size(E, Es, T, K, d, f, L.MOE_F32) >= T * K * f * 4
    assert L.moe_experts_swiglu_workspace_size(E, Es, T, E + 1, d, f, L.MOE_BF16) == 0

    def call(*a, ws=need, shared=P):
        return _st(lib.moe_experts_swiglu(*a, P, P, P, L.MOE_BF16, P, P, P, shared, shared, shared,
                                          P, P, ws, None))
    rc, msg = call(E, Es, T, K, d, f, ws=need - 1)
    assert rc == L.MOE_ERR_INVALID_ARG and "workspace" in msg
    rc, msg = call(E, Es, T, K, d, f, shared=None)
    assert rc == L.MOE_ERR_INVALID_ARG and "shared" in msg
    rc, msg = call(E, Es, T, E + 1, d, f)
    assert rc == L.MOE_ERR_INVALID_ARG and "K <= E_r" in msg
    rc, msg = call(E, Es, T, K, 7000, f)
    assert rc == L.MOE_ERR_UNSUPPORTED and "multiples of 64" in msg
    # more row groups than the tile builder takes: E_r + 8 E_s > 2048
    rc, msg = call(1024, 200, T, K, 256, 256, ws=1 << 40)
    assert rc == L.MOE_ERR_UNSUPPORTED and "row groups" in msg
    # every bf16 operand under 2 GiB: activations of (K + E_s) T rows
    rc, msg = call(E, Es, 65536, K, d, f, ws=1 << 42)
    assert rc == L.MOE_ERR_UNSUPPORTED and "2 GiB" in msg
    assert lib.moe_experts_swiglu(E, Es, T, K, d, f, None, P, P, L.MOE_BF16, P, P, P, P, P, P,
                                  P, P, need, None) == L.MOE_ERR_INVALID_ARG


def test_combine_and_bias_update_reject_bad_arguments():
    lib = L.load()
    P = ctypes.c_void_p(16)
    assert lib.moe_combine(10, 64, 2, 1, P, None, P, P, P, 1, P, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(10, 60, 2, 0, P, None, P, P, P, 1, P, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine(10, 64, 17, 0, P, None, P, P, P, 1, P, None) == L.MOE_ERR_INVALID_ARG
    # T*K past int32 is refused; a large y_perm alone is not (rows have their own bases)
    assert lib.moe_combine(1 << 28, 64, 16, 0, P, None, P, P, P, 1, P, None) == \
        L.MOE_ERR_INVALID_ARG
    assert lib.moe_bias_update(10, 8, 2, -0.1, P, P, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_bias_update(10, 8, 2, float("nan"), P, P, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_bias_update(10, 8, 2, 0.1, None, P, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_bias_update(10, 4096, 2, 0.1, P, P, None, None) == L.MOE_ERR_UNSUPPORTED


def test_calibration_aids_reject_bad_arguments():
    lib = L.load()
    P = ctypes.c_void_p(16)
    fl = ctypes.c_double(-1.0)
    assert lib.moe_calib_mfma_loop(0, 10, P, P, ctypes.byref(fl), None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_mfma_loop(4, 0, P, P, ctypes.byref(fl), None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_mfma_loop(4, 10, None, P, ctypes.byref(fl), None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_mfma_loop(4, 10, P, None, ctypes.byref(fl), None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_mfma_loop((1 << 20) + 1, 10, P, P, None, None) == L.MOE_ERR_INVALID_ARG
    assert fl.value == -1.0  # nothing written on a rejected call
    assert lib.moe_calib_stream_read(0, P, 1024, P, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_stream_read(8, None, 1024, P, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_stream_read(8, P, 1000, P, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_stream_read(8, ctypes.c_void_p(24), 1024, P, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_calib_stream_read(8, P, 0, P, None) == L.MOE_ERR_INVALID_ARG


def test_python_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    t = torch.zeros(4)
    with pytest.raises(ValueError):
        L._ptr(t)
