"""ctypes binding of libmoe_mi355x.so: one Python function per C entry point,
same names and argument order.  Argument marshalling only -- every step of
the layer runs in the HIP library.  Tensors are passed by device pointer.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB may name another build of the same library (the host-sanitized one)
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(PKG, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = 0, 1, 2, 3
MOE_F32, MOE_BF16 = 0, 1
MOE_SIGMOID, MOE_SOFTMAX = 0, 1

EXPORTED = ["moe_route_workspace_size", "moe_route", "moe_permute_workspace_size", "moe_permute",
            "moe_expert_capacity", "moe_permute_capacity", "moe_route_stats_workspace_size",
            "moe_route_stats", "moe_router_diag", "moe_transpose_experts",
            "moe_combine_backward", "moe_grouped_swiglu_backward_workspace_size",
            "moe_grouped_swiglu_backward", "moe_route_backward",
            "moe_grouped_swiglu_workspace_size", "moe_grouped_swiglu",
            "moe_grouped_swiglu_train", "moe_grouped_swiglu_noalloc",
            "moe_experts_swiglu_workspace_size", "moe_experts_swiglu", "moe_combine",
            "moe_bias_update", "moe_calib_mfma_loop", "moe_calib_stream_read",
            "moe_profile_enable", "moe_profile_tag", "moe_profile_only", "moe_profile_report",
            "moe_last_error",
            "moe_version"]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


class MoeRouterDiag(ctypes.Structure):
    _fields_ = [("switch_fP", ctypes.c_float), ("z_loss", ctypes.c_float),
                ("load_entropy", ctypes.c_float), ("max_vio", ctypes.c_float),
                ("dropped", ctypes.c_float), ("reserved", ctypes.c_float * 3)]


class MoeBiasStats(ctypes.Structure):
    _fields_ = [("max_load", ctypes.c_int32), ("min_load", ctypes.c_int32),
                ("max_vio", ctypes.c_float), ("reserved", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None

_i, _p, _f, _sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t


def load() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_mixture_experts_biased_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "moe_route_workspace_size": ([_i, _i, _i, _i], _sz),
        "moe_route": ([_i, _i, _i, _i, _i, _p, _i, _p, _p, _p, _p, _p, _p, _sz, _p], _i),
        "moe_permute_workspace_size": ([_i, _i], _sz),
        "moe_permute": ([_i, _i, _i, _i, _p, _p, _i, _p, _p, _p, _p, _p, _sz, _p], _i),
        "moe_expert_capacity": ([_i, _i, _i, ctypes.c_double], _i),
        "moe_route_stats_workspace_size": ([_i, _i, _i, _i], _sz),
        "moe_route_stats": ([_i, _i, _i, _i, _i, _p, _i, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p],
                            _i),
        "moe_router_diag": ([_i, _i, _i, _p, _p, _p, _p, _p, _p, _p], _i),
        "moe_transpose_experts": ([_i, _i, _i, _p, _i, _p, _i, _i, _p], _i),
        "moe_combine_backward": ([_i, _i, _i, _p, _p, _p, _p, _i, _p, _p, _p], _i),
        "moe_grouped_swiglu_backward_workspace_size": ([_i, _i, _i, _i], _sz),
        "moe_grouped_swiglu_backward": ([_i, _i, _i, _i, _i, _p, _p, _p, _i, _p, _p, _p, _p, _p,
                                         _p, _p, _p, _p, _p, _p, _sz, _p], _i),
        "moe_route_backward": ([_i, _i, _i, _i, _i, _p, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p],
                               _i),
        "moe_permute_capacity": ([_i, _i, _i, _i, _i, _p, _p, _i, _p, _p, _p, _p, _p, _sz, _p],
                                 _i),
        "moe_grouped_swiglu_workspace_size": ([_i, _i, _i, _i, _i], _sz),
        "moe_grouped_swiglu": ([_i, _i, _i, _i, _i, _p, _p, _p, _i, _p, _p, _p, _p, _p, _p,
                                _sz, _p], _i),
        "moe_experts_swiglu_workspace_size": ([_i, _i, _i, _i, _i, _i, _i], _sz),
        "moe_experts_swiglu": ([_i, _i, _i, _i, _i, _i, _p, _p, _p, _i, _p, _p, _p, _p, _p, _p,
                                _p, _p, _sz, _p], _i),
        "moe_grouped_swiglu_train": ([_i, _i, _i, _i, _i, _p, _p, _p, _i, _p, _p, _p, _p, _p,
                                      _p, _p, _sz, _p], _i),
        "moe_grouped_swiglu_noalloc": ([_i, _i, _i, _i, _i, _p, _p, _p, _i, _p, _p, _p, _p,
                                        _p, _p], _i),
        "moe_combine": ([_i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _p], _i),
        "moe_bias_update": ([_i, _i, _i, _f, _p, _p, _p, _p], _i),
        "moe_calib_mfma_loop": ([_i, _i, _p, _p, ctypes.POINTER(ctypes.c_double), _p], _i),
        "moe_calib_stream_read": ([_i, _p, _sz, _p, _p], _i),
        "moe_profile_enable": ([_i], _i),
        "moe_profile_tag": ([ctypes.c_char_p], _i),
        "moe_profile_only": ([ctypes.c_char_p], _i),
        "moe_profile_report": ([ctypes.c_char_p, _sz], _i),
        "moe_last_error": ([], ctypes.c_char_p),
        "moe_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (None -> NULL); plain ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    if t.device.type != "cuda":
        raise ValueError("tensor arguments must live on the GPU")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != MOE_OK:
        msg = load().moe_last_error().decode(errors="replace")
        raise MoeError(status, msg)


def moe_version() -> str:
    return load().moe_version().decode()


def moe_last_error() -> str:
    return load().moe_last_error().decode(errors="replace")


def moe_route_workspace_size(T, d_model, E_r, h_dtype) -> int:
    return int(load().moe_route_workspace_size(T, d_model, E_r, h_dtype))


def moe_route(T, d_model, E_r, K, fn, h, h_dtype, e, b, topk_idx, gates, loads, workspace,
              workspace_bytes, stream=None):
    _check(load().moe_route(T, d_model, E_r, K, fn, _ptr(h), h_dtype, _ptr(e), _ptr(b),
                            _ptr(topk_idx), _ptr(gates), _ptr(loads), _ptr(workspace),
                            workspace_bytes, _stream(stream)))


def moe_route_stats_workspace_size(T, d_model, E_r, h_dtype) -> int:
    return int(load().moe_route_stats_workspace_size(T, d_model, E_r, h_dtype))


def moe_route_stats(T, d_model, E_r, K, fn, h, h_dtype, e, b, topk_idx, gates, loads, p_mean,
                    zsq_mean, workspace, workspace_bytes, stream=None):
    _check(load().moe_route_stats(T, d_model, E_r, K, fn, _ptr(h), h_dtype, _ptr(e), _ptr(b),
                                  _ptr(topk_idx), _ptr(gates), _ptr(loads), _ptr(p_mean),
                                  _ptr(zsq_mean), _ptr(workspace), workspace_bytes,
                                  _stream(stream)))


def moe_router_diag(T, E_r, K, loads, p_mean, zsq_mean, offsets, f, diag, stream=None):
    """diag: a device tensor of at least 8 float32 (the moe_router_diag_values layout)."""
    _check(load().moe_router_diag(T, E_r, K, _ptr(loads), _ptr(p_mean), _ptr(zsq_mean),
                                  _ptr(offsets), _ptr(f), _ptr(diag), _stream(stream)))


DIAG_FIELDS = ("switch_fP", "z_loss", "load_entropy", "max_vio", "dropped")


def moe_permute_workspace_size(T, E_r) -> int:
    return int(load().moe_permute_workspace_size(T, E_r))


def moe_permute(T, d_model, E_r, K, topk_idx, h, dtype, offsets, row_token, slot_row, x_perm,
                workspace, workspace_bytes, stream=None):
    _check(load().moe_permute(T, d_model, E_r, K, _ptr(topk_idx), _ptr(h), dtype, _ptr(offsets),
                              _ptr(row_token), _ptr(slot_row), _ptr(x_perm), _ptr(workspace),
                              workspace_bytes, _stream(stream)))


def moe_expert_capacity(T, K, E_r, capacity_factor) -> int:
    return int(load().moe_expert_capacity(T, K, E_r, float(capacity_factor)))


def moe_permute_capacity(T, d_model, E_r, K, capacity, topk_idx, h, dtype, offsets, row_token,
                         slot_row, x_perm, workspace, workspace_bytes, stream=None):
    _check(load().moe_permute_capacity(T, d_model, E_r, K, capacity, _ptr(topk_idx), _ptr(h),
                                       dtype, _ptr(offsets), _ptr(row_token), _ptr(slot_row),
                                       _ptr(x_perm), _ptr(workspace), workspace_bytes,
                                       _stream(stream)))


def moe_grouped_swiglu_workspace_size(n_groups, d_model, d_ffn, rows, dtype) -> int:
    return int(load().moe_grouped_swiglu_workspace_size(n_groups, d_model, d_ffn, rows, dtype))


def moe_grouped_swiglu(n_groups, d_model, d_ffn, rows, x_rows, offsets, row_index, x, dtype,
                       w_gate, w_up, w_down, row_scale, y, workspace, workspace_bytes,
                       stream=None):
    _check(load().moe_grouped_swiglu(n_groups, d_model, d_ffn, rows, x_rows, _ptr(offsets),
                                     _ptr(row_index), _ptr(x), dtype, _ptr(w_gate), _ptr(w_up),
                                     _ptr(w_down), _ptr(row_scale), _ptr(y), _ptr(workspace),
                                     workspace_bytes, _stream(stream)))


def moe_experts_swiglu_workspace_size(E_r, E_s, T, K, d_model, d_ffn, dtype) -> int:
    return int(load().moe_experts_swiglu_workspace_size(E_r, E_s, T, K, d_model, d_ffn, dtype))


def moe_experts_swiglu(E_r, E_s, T, K, d_model, d_ffn, offsets, row_token, h, dtype, w_gate,
                       w_up, w_down, ws_gate, ws_up, ws_down, y, workspace, workspace_bytes,
                       stream=None):
    _check(load().moe_experts_swiglu(E_r, E_s, T, K, d_model, d_ffn, _ptr(offsets),
                                     _ptr(row_token), _ptr(h), dtype, _ptr(w_gate), _ptr(w_up),
                                     _ptr(w_down), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down),
                                     _ptr(y), _ptr(workspace), workspace_bytes, _stream(stream)))


def moe_grouped_swiglu_train(n_groups, d_model, d_ffn, rows, x_rows, offsets, row_index, x,
                             dtype, w_gate, w_up, w_down, row_scale, y, au, workspace,
                             workspace_bytes, stream=None):
    _check(load().moe_grouped_swiglu_train(n_groups, d_model, d_ffn, rows, x_rows, _ptr(offsets),
                                           _ptr(row_index), _ptr(x), dtype, _ptr(w_gate),
                                           _ptr(w_up), _ptr(w_down), _ptr(row_scale), _ptr(y),
                                           _ptr(au), _ptr(workspace), workspace_bytes,
                                           _stream(stream)))


def moe_grouped_swiglu_noalloc(n_groups, d_model, d_ffn, rows, x_rows, offsets, row_index, x,
                               dtype, w_gate, w_up, w_down, row_scale, y, stream=None):
    _check(load().moe_grouped_swiglu_noalloc(n_groups, d_model, d_ffn, rows, x_rows,
                                             _ptr(offsets), _ptr(row_index), _ptr(x), dtype,
                                             _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                             _ptr(row_scale), _ptr(y), _stream(stream)))


def moe_combine(T, d_model, K, E_s, h, y_shared, y_perm, slot_row, gates, dtype, y,
                stream=None):
    _check(load().moe_combine(T, d_model, K, E_s, _ptr(h), _ptr(y_shared), _ptr(y_perm),
                              _ptr(slot_row), _ptr(gates), dtype, _ptr(y), _stream(stream)))


def moe_bias_update(T, E_r, K, gamma, loads, b, stats, stream=None):
    _check(load().moe_bias_update(T, E_r, K, float(gamma), _ptr(loads), _ptr(b), _ptr(stats),
                                  _stream(stream)))


def moe_calib_mfma_loop(workgroups: int, iters: int, operands, out, stream=None) -> float:
    """Launch the pure matrix-core loop (a measurement aid) on `stream`
    (default: torch's current stream); returns the FLOPs it performs."""
    fl = ctypes.c_double(0.0)
    _check(load().moe_calib_mfma_loop(workgroups, iters, _ptr(operands), _ptr(out),
                                      ctypes.byref(fl), _stream(stream)))
    return fl.value


def moe_calib_stream_read(workgroups: int, src, out, stream=None):
    """Launch the streaming-read kernel (a measurement aid) over all of `src`."""
    _check(load().moe_calib_stream_read(workgroups, _ptr(src), src.numel() * src.element_size(),
                                        _ptr(out), _stream(stream)))


def moe_profile_enable(on: bool = True):
    _check(load().moe_profile_enable(1 if on else 0))


def moe_profile_tag(tag: str = ""):
    _check(load().moe_profile_tag(tag.encode()))


def moe_profile_only(names: str = ""):
    """Record only kernels whose tagged name contains one of the
    comma-separated substrings ("" records all)."""
    _check(load().moe_profile_only(names.encode()))


def moe_profile_report() -> dict:
    """{kernel name: (launches, total_ms, min_ms, max_ms)} since the last report."""
    buf = ctypes.create_string_buffer(1 << 16)
    _check(load().moe_profile_report(buf, len(buf)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, tot, mn, mx = line.split()
        out[name] = (int(n), float(tot), float(mn), float(mx))
    return out


def moe_transpose_experts(n, rows, cols, src, dtype, dst, ld_dst, col_offset, stream=None):
    _check(load().moe_transpose_experts(n, rows, cols, _ptr(src), dtype, _ptr(dst), ld_dst,
                                        col_offset, _stream(stream)))


def moe_combine_backward(T, d_model, K, dy, y_perm, slot_row, gates, dtype, dy_perm, dgates,
                         stream=None):
    _check(load().moe_combine_backward(T, d_model, K, _ptr(dy), _ptr(y_perm), _ptr(slot_row),
                                       _ptr(gates), dtype, _ptr(dy_perm), _ptr(dgates),
                                       _stream(stream)))


def moe_grouped_swiglu_backward_workspace_size(n_groups, d_model, d_ffn, rows) -> int:
    return int(load().moe_grouped_swiglu_backward_workspace_size(n_groups, d_model, d_ffn, rows))


def moe_grouped_swiglu_backward(n_groups, d_model, d_ffn, rows, x_rows, offsets, row_index, x,
                                dtype, w_gate, w_up, w_gu_t, w_down_t, dy, au, dx, dw_gate,
                                dw_up, dw_down, workspace, workspace_bytes, stream=None):
    _check(load().moe_grouped_swiglu_backward(
        n_groups, d_model, d_ffn, rows, x_rows, _ptr(offsets), _ptr(row_index), _ptr(x), dtype,
        _ptr(w_gate), _ptr(w_up), _ptr(w_gu_t), _ptr(w_down_t), _ptr(dy), _ptr(au), _ptr(dx),
        _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down), _ptr(workspace), workspace_bytes,
        _stream(stream)))


def moe_route_backward(T, d_model, E_r, K, fn, h, h_dtype, e, topk_idx, dgates, offsets,
                       row_token, dz, dh, de, stream=None):
    _check(load().moe_route_backward(T, d_model, E_r, K, fn, _ptr(h), h_dtype, _ptr(e),
                                     _ptr(topk_idx), _ptr(dgates), _ptr(offsets),
                                     _ptr(row_token), _ptr(dz), _ptr(dh), _ptr(de),
                                     _stream(stream)))

