"""One MoE layer forward driven through the C ABI.

MoELayer owns the intermediate device buffers (allocated once, with torch, at
construction) and calls the five entry points in order on one stream:

    moe_route -> moe_permute (or moe_permute_capacity) -> moe_grouped_swiglu (routed experts)
    -> moe_grouped_swiglu (shared experts) -> moe_combine -> moe_bias_update

Layer output (Sparse MoE routing-math page, section 0):
    y_t = h_t + sum_j SwiGLU^S_j(h_t) + sum_{i in I_t} g_{t,i} SwiGLU^R_i(h_t)
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L


@dataclass
class LayerShape:
    T: int
    d_model: int
    E_r: int
    K: int
    E_s: int
    d_ffn: int
    dtype: str    # "bf16" or "f32"
    score: str    # "sigmoid" or "softmax"


class MoELayer:
    def __init__(self, shape: LayerShape, e, w_gate, w_up, w_down, ws_gate=None, ws_up=None,
                 ws_down=None, device="cuda", capacity_factor: Optional[float] = None,
                 diagnostics: bool = False, overlap_shared: bool = True,
                 shared_start: str = "layer", fuse_shared: bool = False):
        """capacity_factor: None dispatches every copy; a factor CF caps each
        expert at C = ceil(CF*T*K/E_r) rows, admitted in token order.
        diagnostics: route with moe_route_stats and fill the router's balance
        diagnostics (moe_router_diag) after the dispatch of every forward.
        overlap_shared: run the shared experts (which need no routing) on a
        second stream, side by side with the routing and the routed experts,
        joined before the combine; False runs them in sequence.
        shared_start: with overlap_shared, when the side stream starts them:
        "layer" (as soon as h is ready) or "routed" (once the router and the
        dispatch are done, so those small kernels have every CU to themselves
        and the shared experts overlap the routed experts instead).
        fuse_shared: an inference forward runs the routed and the shared
        experts in one grouped launch per product (moe_experts_swiglu): one
        stream, no events (e.g. for a caller that captures the layer on a
        single stream).  Same bits; at the DeepSeek-V3 shapes 1-2 % slower
        than the shared experts on a side stream.  overlap_shared and
        shared_start then only apply to training forwards."""
        if shared_start not in ("layer", "routed"):
            raise ValueError(f"shared_start must be 'layer' or 'routed', not {shared_start!r}")
        self.shared_start = shared_start
        s = self.shape = shape
        self.capacity = (None if capacity_factor is None else
                         L.moe_expert_capacity(s.T, s.K, s.E_r, capacity_factor))
        if self.capacity is not None and self.capacity < 0:
            raise ValueError(f"bad capacity factor {capacity_factor}")
        self.profile_tags = False   # label routed / shared launches in the kernel timing
        self.dt = L.MOE_BF16 if s.dtype == "bf16" else L.MOE_F32
        self.tdt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
        self.fn = L.MOE_SIGMOID if s.score == "sigmoid" else L.MOE_SOFTMAX
        self.e, self.w_gate, self.w_up, self.w_down = e, w_gate, w_up, w_down
        self.ws_gate, self.ws_up, self.ws_down = ws_gate, ws_up, ws_down
        T, K, E, d = s.T, s.K, s.E_r, s.d_model
        TK = T * K
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_idx = torch.empty((T, K), **i32)
        self.gates = torch.empty((T, K), dtype=torch.float32, device=device)
        self.loads = torch.empty((E,), **i32)
        self.diagnostics = diagnostics
        if diagnostics:
            f32 = dict(dtype=torch.float32, device=device)
            self.p_mean = torch.empty((E,), **f32)
            self.zsq_mean = torch.empty((1,), **f32)
            self.f = torch.empty((E,), **f32)
            self.diag = torch.zeros((8,), **f32)
            self.route_ws_bytes = L.moe_route_stats_workspace_size(T, d, E, self.dt)
        else:
            self.route_ws_bytes = L.moe_route_workspace_size(T, d, E, self.dt)
        self.route_ws = torch.empty((max(self.route_ws_bytes, 1),), dtype=torch.uint8,
                                    device=device)
        self.offsets = torch.empty((E + 1,), **i32)
        self.row_token = torch.empty((TK,), **i32)
        self.slot_row = torch.empty((TK,), **i32)
        self.perm_ws_bytes = L.moe_permute_workspace_size(T, E)
        self.perm_ws = torch.empty((self.perm_ws_bytes,), dtype=torch.uint8, device=device)
        # y_perm and the shared outputs are the two parts of one buffer, the
        # layout moe_experts_swiglu writes
        self.y_all = torch.empty((TK + s.E_s * T, d), dtype=self.tdt, device=device)
        self.y_perm = self.y_all[:TK]
        ws_bytes = L.moe_grouped_swiglu_workspace_size(E, d, s.d_ffn, TK, self.dt)
        self.fuse_shared = bool(fuse_shared and s.E_s)
        if self.fuse_shared:
            ws_bytes = max(ws_bytes, L.moe_experts_swiglu_workspace_size(
                E, s.E_s, T, s.K, d, s.d_ffn, self.dt))
        self.side = None
        if s.E_s:
            sh_bytes = L.moe_grouped_swiglu_workspace_size(s.E_s, d, s.d_ffn, s.E_s * T, self.dt)
            ws_bytes = max(ws_bytes, sh_bytes)
            if overlap_shared:
                # the shared experts get their own workspace, stream and events
                # (default priority, like every stream here)
                self.sh_ws_bytes = sh_bytes
                self.sh_ws = torch.empty((sh_bytes,), dtype=torch.uint8, device=device)
                self.side = torch.cuda.Stream(device=device)
                self.ev_in = torch.cuda.Event()
                self.ev_sh = torch.cuda.Event()
            self.sh_offsets = (torch.arange(s.E_s + 1, **i32) * T).contiguous()
            self.sh_rows = torch.arange(T, **i32).repeat(s.E_s).contiguous()
            self.y_shared = self.y_all[TK:]
        else:
            self.sh_offsets = self.sh_rows = self.y_shared = None
        self.sw_ws_bytes = ws_bytes
        self.sw_ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=device)
        if self.side is None:
            self.sh_ws, self.sh_ws_bytes = self.sw_ws, self.sw_ws_bytes
        self.y = torch.empty((T, d), dtype=self.tdt, device=device)
        self.stats = torch.zeros((4,), dtype=torch.int32, device=device)
        # [a | u] of the routed and shared experts, kept by a training forward;
        # au_valid is set by such a forward and cleared by prepare_backward
        self.au_perm = self.au_shared = None
        self.au_valid = False

    def _check(self, name, t, shape, dtype):
        """Raise ValueError unless t is a contiguous tensor of this shape and
        dtype on this layer's device (the C ABI gets bare pointers)."""
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
        if t.device != self.y.device:
            raise ValueError(f"{name}: on {t.device}, the layer is on {self.y.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")

    def _check_inputs(self, h, b=None):
        s = self.shape
        self._check("h", h, (s.T, s.d_model), self.tdt)
        if b is not None:
            self._check("b", b, (s.E_r,), torch.float32)

    # individual stages -------------------------------------------------
    def route(self, h, b, stream=None):
        s = self.shape
        if self.diagnostics:
            L.moe_route_stats(s.T, s.d_model, s.E_r, s.K, self.fn, h, self.dt, self.e, b,
                              self.topk_idx, self.gates, self.loads, self.p_mean, self.zsq_mean,
                              self.route_ws, self.route_ws_bytes, stream)
        else:
            L.moe_route(s.T, s.d_model, s.E_r, s.K, self.fn, h, self.dt, self.e, b,
                        self.topk_idx, self.gates, self.loads, self.route_ws,
                        self.route_ws_bytes, stream)

    def router_diag(self, stream=None):
        s = self.shape
        L.moe_router_diag(s.T, s.E_r, s.K, self.loads, self.p_mean, self.zsq_mean, self.offsets,
                          self.f, self.diag, stream)

    def diag_host(self):
        v = self.diag.cpu().tolist()
        return dict(zip(L.DIAG_FIELDS, v[:len(L.DIAG_FIELDS)]))

    def permute(self, h=None, x_perm=None, stream=None):
        s = self.shape
        if self.capacity is None:
            L.moe_permute(s.T, s.d_model, s.E_r, s.K, self.topk_idx, h, self.dt, self.offsets,
                          self.row_token, self.slot_row, x_perm, self.perm_ws,
                          self.perm_ws_bytes, stream)
        else:
            L.moe_permute_capacity(s.T, s.d_model, s.E_r, s.K, self.capacity, self.topk_idx, h,
                                   self.dt, self.offsets, self.row_token, self.slot_row, x_perm,
                                   self.perm_ws, self.perm_ws_bytes, stream)

    def routed_experts(self, h, stream=None):
        s = self.shape
        if self.profile_tags:
            L.moe_profile_tag("routed.")
        if self.au_perm is None:
            L.moe_grouped_swiglu(s.E_r, s.d_model, s.d_ffn, s.T * s.K, s.T, self.offsets,
                                 self.row_token, h, self.dt, self.w_gate, self.w_up, self.w_down,
                                 None, self.y_perm, self.sw_ws, self.sw_ws_bytes, stream)
        else:
            L.moe_grouped_swiglu_train(s.E_r, s.d_model, s.d_ffn, s.T * s.K, s.T, self.offsets,
                                       self.row_token, h, self.dt, self.w_gate, self.w_up,
                                       self.w_down, None, self.y_perm, self.au_perm, self.sw_ws,
                                       self.sw_ws_bytes, stream)
        if self.profile_tags:
            L.moe_profile_tag("")

    def shared_experts(self, h, stream=None):
        s = self.shape
        if not s.E_s:
            return
        if self.profile_tags:
            L.moe_profile_tag("shared.")
        if self.au_shared is None:
            L.moe_grouped_swiglu(s.E_s, s.d_model, s.d_ffn, s.E_s * s.T, s.T, self.sh_offsets,
                                 self.sh_rows, h, self.dt, self.ws_gate, self.ws_up,
                                 self.ws_down, None, self.y_shared, self.sh_ws, self.sh_ws_bytes,
                                 stream)
        else:
            L.moe_grouped_swiglu_train(s.E_s, s.d_model, s.d_ffn, s.E_s * s.T, s.T,
                                       self.sh_offsets, self.sh_rows, h, self.dt, self.ws_gate,
                                       self.ws_up, self.ws_down, None, self.y_shared,
                                       self.au_shared, self.sh_ws, self.sh_ws_bytes, stream)
        if self.profile_tags:
            L.moe_profile_tag("")

    def experts_fused(self, h, stream=None):
        """Routed and shared experts in one grouped launch per product."""
        s = self.shape
        if self.profile_tags:
            L.moe_profile_tag("experts.")
        L.moe_experts_swiglu(s.E_r, s.E_s, s.T, s.K, s.d_model, s.d_ffn, self.offsets,
                             self.row_token, h, self.dt, self.w_gate, self.w_up, self.w_down,
                             self.ws_gate, self.ws_up, self.ws_down, self.y_all, self.sw_ws,
                             self.sw_ws_bytes, stream)
        if self.profile_tags:
            L.moe_profile_tag("")

    def combine(self, h, stream=None):
        s = self.shape
        L.moe_combine(s.T, s.d_model, s.K, s.E_s, h, self.y_shared, self.y_perm, self.slot_row,
                      self.gates, self.dt, self.y, stream)

    def bias_update(self, b, gamma, stream=None):
        s = self.shape
        L.moe_bias_update(s.T, s.E_r, s.K, gamma, self.loads, b, self.stats, stream)

    # whole layer --------------------------------------------------------
    def forward(self, h, b: Optional[torch.Tensor] = None, gamma: Optional[float] = None,
                stream=None):
        """One layer forward; when gamma is given, b is updated in place after
        the loads are counted (the update affects the next call)."""
        self._check_inputs(h, b)
        if self.fuse_shared and self.au_perm is None:
            self.route(h, b, stream)
            self.permute(stream=stream)
            if self.diagnostics:
                self.router_diag(stream)
            self.experts_fused(h, stream)
            self.combine(h, stream)
            if gamma is not None and b is not None:
                self.bias_update(b, gamma, stream)
            self.au_valid = False
            return self.y
        # the shared experts on the side stream once h is ready on this one
        # (a raw stream handle cannot carry events: then in sequence)
        overlap = self.side is not None and not isinstance(stream, int)
        main = None
        if overlap:
            main = stream if stream is not None else torch.cuda.current_stream()

        def start_shared():
            self.ev_in.record(main)
            self.side.wait_event(self.ev_in)
            self.shared_experts(h, self.side)
            self.ev_sh.record(self.side)

        if overlap and self.shared_start == "layer":
            start_shared()
        self.route(h, b, stream)
        self.permute(stream=stream)
        if self.diagnostics:
            self.router_diag(stream)
        if overlap and self.shared_start == "routed":
            start_shared()
        self.routed_experts(h, stream)
        if overlap:
            main.wait_event(self.ev_sh)
        else:
            self.shared_experts(h, stream)
        self.combine(h, stream)
        if gamma is not None and b is not None:
            self.bias_update(b, gamma, stream)
        # a training forward has now written a | u for the backward
        self.au_valid = self.au_perm is not None
        return self.y

    # backward -----------------------------------------------------------
    def prepare_backward(self, stream=None, keep_au: bool = True):
        """Allocate the backward buffers and build the transposed weight copies
        ([W_gate^T | W_up^T] and W_down^T); call again after the weights change.
        With keep_au, later forwards also store the experts' gate and up
        projections ([rows, 2 d_ffn] bf16 each for the routed and shared
        experts), which the backward reads instead of recomputing."""
        s = self.shape
        if s.dtype != "bf16":
            raise NotImplementedError("the backward pass runs on bf16 layers")
        if s.E_s > 1:
            raise NotImplementedError("the backward pass takes at most one shared expert")
        dev = self.y.device
        T, K, E, d, f = s.T, s.K, s.E_r, s.d_model, s.d_ffn
        bf = dict(dtype=torch.bfloat16, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)

        def transposed(wg, wu, wd, n):
            gu_t = torch.empty((n, d, 2 * f), **bf)
            d_t = torch.empty((n, f, d), **bf)
            L.moe_transpose_experts(n, f, d, wg, self.dt, gu_t, 2 * f, 0, stream)
            L.moe_transpose_experts(n, f, d, wu, self.dt, gu_t, 2 * f, f, stream)
            L.moe_transpose_experts(n, d, f, wd, self.dt, d_t, d, 0, stream)
            return gu_t, d_t

        self.w_gu_t, self.w_down_t = transposed(self.w_gate, self.w_up, self.w_down, E)
        self.dy_perm = torch.zeros((T * K, d), **bf)
        self.dx_perm = torch.zeros((T * K, d), **bf)
        self.dgates = torch.empty((T, K), **f32)
        self.dz = torch.empty((T, K), **f32)
        self.dh = torch.empty((T, d), **bf)
        self.de = torch.empty((E, d), **f32)
        self.ones = torch.ones((T, K), **f32)
        self.dw_gate = torch.empty_like(self.w_gate)
        self.dw_up = torch.empty_like(self.w_up)
        self.dw_down = torch.empty_like(self.w_down)
        bw = L.moe_grouped_swiglu_backward_workspace_size(E, d, f, T * K)
        if s.E_s:
            self.ws_gu_t, self.ws_down_t = transposed(self.ws_gate, self.ws_up, self.ws_down,
                                                      s.E_s)
            self.dx_shared = torch.empty((T, d), **bf)
            self.dws_gate = torch.empty_like(self.ws_gate)
            self.dws_up = torch.empty_like(self.ws_up)
            self.dws_down = torch.empty_like(self.ws_down)
            bw = max(bw, L.moe_grouped_swiglu_backward_workspace_size(s.E_s, d, f, T))
        else:
            self.dx_shared = None
        self.bw_ws_bytes = bw
        self.bw_ws = torch.empty((bw,), dtype=torch.uint8, device=dev)
        self.sh_bw_ws, self.sh_bw_ws_bytes = self.bw_ws, self.bw_ws_bytes
        if s.E_s and self.side is not None:  # the shared experts' backward on the side stream
            self.sh_bw_ws_bytes = L.moe_grouped_swiglu_backward_workspace_size(s.E_s, d, f, T)
            self.sh_bw_ws = torch.empty((self.sh_bw_ws_bytes,), dtype=torch.uint8, device=dev)
        if keep_au:
            self.au_perm = torch.empty((T * K, 2 * f), **bf)
            self.au_shared = torch.empty((T, 2 * f), **bf) if s.E_s else None
        else:
            self.au_perm = self.au_shared = None
        # the new a | u buffers hold nothing until a forward fills them
        self.au_valid = False
        self.bw_ready = True
        if self.capacity is not None:   # the router's gradient covers every pick
            self.all_offsets = torch.empty((E + 1,), **i32)
            self.all_row_token = torch.empty((T * K,), **i32)
            self.all_slot_row = torch.empty((T * K,), **i32)

    def backward(self, h, dy, stream=None):
        """Gradients of sum_t <dy_t, y_t> after forward(h): dh, de and the
        expert weight gradients (routed: dw_*, shared: dws_*), with the
        forward's routing decisions fixed.  Requires prepare_backward() before
        that forward."""
        s = self.shape
        T, K, E, d, f = s.T, s.K, s.E_r, s.d_model, s.d_ffn
        if not getattr(self, "bw_ready", False):
            raise RuntimeError("backward() needs prepare_backward() and then a forward()")
        if self.au_perm is not None and not self.au_valid:
            raise RuntimeError("backward() reads the a | u of the last forward: call forward() "
                               "after prepare_backward() and before backward()")
        self._check_inputs(h)
        self._check("dy", dy, (T, d), self.tdt)

        def shared_backward(st):  # needs only dy, h and the forward's a | u
            L.moe_grouped_swiglu_backward(s.E_s, d, f, T, T, self.sh_offsets, self.sh_rows, h,
                                          self.dt, self.ws_gate, self.ws_up, self.ws_gu_t,
                                          self.ws_down_t, dy, self.au_shared, self.dx_shared,
                                          self.dws_gate, self.dws_up, self.dws_down,
                                          self.sh_bw_ws, self.sh_bw_ws_bytes, st)

        # the shared experts' backward on the side stream, beside the routed one
        overlap = bool(s.E_s) and self.side is not None and not isinstance(stream, int)
        if overlap:
            main = stream if stream is not None else torch.cuda.current_stream()
            self.ev_in.record(main)
            self.side.wait_event(self.ev_in)
            shared_backward(self.side)
            self.ev_sh.record(self.side)
        L.moe_combine_backward(T, d, K, dy, self.y_perm, self.slot_row, self.gates, self.dt,
                               self.dy_perm, self.dgates, stream)
        L.moe_grouped_swiglu_backward(E, d, f, T * K, T, self.offsets, self.row_token, h, self.dt,
                                      self.w_gate, self.w_up, self.w_gu_t, self.w_down_t,
                                      self.dy_perm, self.au_perm, self.dx_perm, self.dw_gate,
                                      self.dw_up, self.dw_down, self.bw_ws, self.bw_ws_bytes,
                                      stream)
        if overlap:
            main.wait_event(self.ev_sh)
        elif s.E_s:
            shared_backward(stream)
        # dh = dy + dx_shared + sum_k dx_perm[slot] (the combine with unit gates)
        L.moe_combine(T, d, K, s.E_s, dy, self.dx_shared, self.dx_perm, self.slot_row,
                      self.ones, self.dt, self.dh, stream)
        if self.capacity is None:
            offs, rtok = self.offsets, self.row_token
        else:
            L.moe_permute(T, d, E, K, self.topk_idx, None, self.dt, self.all_offsets,
                          self.all_row_token, self.all_slot_row, None, self.perm_ws,
                          self.perm_ws_bytes, stream)
            offs, rtok = self.all_offsets, self.all_row_token
        L.moe_route_backward(T, d, E, K, self.fn, h, self.dt, self.e, self.topk_idx,
                             self.dgates, offs, rtok, self.dz, self.dh, self.de, stream)
        return self.dh

    def stats_host(self):
        st = self.stats.cpu()
        return dict(max_load=int(st[0]), min_load=int(st[1]),
                    max_vio=float(st[2:3].view(torch.float32)[0]))
