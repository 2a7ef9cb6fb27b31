"""Seeded input generators.

Every tensor is a pure function of (base seed, config index, tensor tag,
index): each gets its own torch.Generator on the target device, seeded from a
BLAKE2b digest of that key.  Per-expert weights are drawn expert by expert, so
any single expert can be redrawn on its own.

Distributions (the layer workloads' recipe):
  tokens h            N(0, 1)                (fp32 or bf16, RNE cast)
  centroids e         N(0, 1/d_model)        fp32 (the router is fp32)
  W_gate, W_up        N(0, 1/d_model)        [E, d_ffn, d_model], nn.Linear layout
  W_down              N(0, 1/d_ffn)          [E, d_model, d_ffn]
  bias b              0, absent, or U(-r, r) fp32
Skewed workload: tokens h = a * u_c + N(0, I) with c ~ U{0..M-1} and unit
vectors u_c of disjoint support (coordinate j belongs to component j mod M,
random sign, magnitude 1/sqrt(d/M)); hot experts j < 8 get
e_j += beta * (u_p + u_q) / sqrt(2) for a fixed list of component pairs, so
every component has exactly four aligned hot experts.

GPU tests copy these tensors to the host for the oracle: the values come from
this module on both sides.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import LayerConfig

# Component pairs for the hot experts of the skewed workload (four components).
HOT_PAIRS = [(0, 1), (2, 3), (0, 2), (1, 3), (0, 3), (1, 2), (0, 1), (2, 3)]

_TAGS = {"h": 1, "e": 2, "b": 3, "w_gate": 4, "w_up": 5, "w_down": 6,
         "ws_gate": 7, "ws_up": 8, "ws_down": 9, "labels": 10, "u_sign": 11}


def seed_of(base: int, cfg_index: int, tag: str, index: int = 0) -> int:
    key = f"{base}/{cfg_index}/{_TAGS[tag]}/{index}".encode()
    return int.from_bytes(hashlib.blake2b(key, digest_size=8).digest(), "little") >> 1


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std: float, seed: int, device, out_dtype) -> torch.Tensor:
    x = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(np.float32(std).item())
    return x.to(out_dtype)


def _tdtype(cfg: LayerConfig):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


@dataclass
class LayerInputs:
    cfg: LayerConfig
    h: torch.Tensor                 # [T, d_model]
    e: torch.Tensor                 # [E_r, d_model] fp32
    b: Optional[torch.Tensor]       # [E_r] fp32 or None
    w_gate: torch.Tensor            # [E_r, d_ffn, d_model]
    w_up: torch.Tensor              # [E_r, d_ffn, d_model]
    w_down: torch.Tensor            # [E_r, d_model, d_ffn]
    ws_gate: Optional[torch.Tensor]  # [E_s, d_ffn, d_model] or None
    ws_up: Optional[torch.Tensor]
    ws_down: Optional[torch.Tensor]


def _mixture_dirs(cfg: LayerConfig, base: int, device) -> torch.Tensor:
    """Unit vectors u_c [M, d] with disjoint supports and random signs."""
    M, d = cfg.mixture, cfg.d_model
    sign = torch.randint(0, 2, (d,), generator=_gen(seed_of(base, cfg.index, "u_sign"), device),
                         device=device).to(torch.float32).mul_(2.0).sub_(1.0)
    mag = np.float32(1.0 / math.sqrt(d / M)).item()
    comp = torch.arange(d, device=device) % M
    u = torch.zeros(M, d, dtype=torch.float32, device=device)
    for c in range(M):
        u[c] = torch.where(comp == c, sign * mag, torch.zeros_like(sign))
    return u


def make_tokens(cfg: LayerConfig, step: int = 0, device="cpu", base: int = 0) -> torch.Tensor:
    """Token rows h [T, d_model] for one step of the workload."""
    dt = _tdtype(cfg)
    if cfg.mixture == 0:
        return _normal((cfg.T, cfg.d_model), 1.0, seed_of(base, cfg.index, "h", step), device, dt)
    u = _mixture_dirs(cfg, base, device)
    labels = torch.randint(0, cfg.mixture, (cfg.T,),
                           generator=_gen(seed_of(base, cfg.index, "labels", step), device),
                           device=device)
    noise = _normal((cfg.T, cfg.d_model), 1.0, seed_of(base, cfg.index, "h", step), device,
                    torch.float32)
    shift = u[labels].mul_(np.float32(cfg.mixture_scale).item())
    return (shift + noise).to(dt)


def make_centroids(cfg: LayerConfig, device="cpu", base: int = 0,
                   beta: Optional[float] = None) -> torch.Tensor:
    e = _normal((cfg.E_r, cfg.d_model), 1.0 / math.sqrt(cfg.d_model),
                seed_of(base, cfg.param_index, "e"), device, torch.float32)
    if cfg.hot_experts:
        if beta is None:
            raise ValueError("the skewed workload needs its alignment strength beta")
        u = _mixture_dirs(cfg, base, device)
        inv_sqrt2 = np.float32(1.0 / math.sqrt(2.0)).item()
        bf = np.float32(beta).item()
        for j in range(cfg.hot_experts):
            p, q = HOT_PAIRS[j % len(HOT_PAIRS)]
            w = (u[p] + u[q]).mul_(inv_sqrt2)
            e[j] = e[j] + w.mul_(bf)
    return e


def make_bias(cfg: LayerConfig, device="cpu", base: int = 0) -> Optional[torch.Tensor]:
    if cfg.bias == "none":
        return None
    if cfg.bias == "zero":
        return torch.zeros(cfg.E_r, dtype=torch.float32, device=device)
    r = np.float32(cfg.bias_range).item()
    u = torch.rand(cfg.E_r, generator=_gen(seed_of(base, cfg.param_index, "b"), device),
                   device=device, dtype=torch.float32)
    return u.mul_(2.0 * r).sub_(r)


def _expert_stack(cfg, tag, n, rows, cols, std, device, base):
    dt = _tdtype(cfg)
    out = torch.empty((n, rows, cols), dtype=dt, device=device)
    for i in range(n):
        out[i] = _normal((rows, cols), std, seed_of(base, cfg.param_index, tag, i), device, dt)
    return out


def make_expert(cfg: LayerConfig, i: int, shared: bool = False, device="cpu", base: int = 0):
    """(W_gate, W_up, W_down) of one routed (or shared) expert, drawn on its own."""
    dt = _tdtype(cfg)
    d, f = cfg.d_model, cfg.d_ffn
    pre = "ws_" if shared else "w_"
    pi = cfg.param_index
    wg = _normal((f, d), 1.0 / math.sqrt(d), seed_of(base, pi, pre + "gate", i), device, dt)
    wu = _normal((f, d), 1.0 / math.sqrt(d), seed_of(base, pi, pre + "up", i), device, dt)
    wd = _normal((d, f), 1.0 / math.sqrt(f), seed_of(base, pi, pre + "down", i), device, dt)
    return wg, wu, wd


def make_layer(cfg: LayerConfig, device="cpu", base: int = 0, beta: Optional[float] = None,
               step: int = 0) -> LayerInputs:
    d, f = cfg.d_model, cfg.d_ffn
    sd, sf = 1.0 / math.sqrt(d), 1.0 / math.sqrt(f)
    h = make_tokens(cfg, step, device, base)
    e = make_centroids(cfg, device, base, beta)
    b = make_bias(cfg, device, base)
    wg = _expert_stack(cfg, "w_gate", cfg.E_r, f, d, sd, device, base)
    wu = _expert_stack(cfg, "w_up", cfg.E_r, f, d, sd, device, base)
    wd = _expert_stack(cfg, "w_down", cfg.E_r, d, f, sf, device, base)
    if cfg.E_s:
        sg = _expert_stack(cfg, "ws_gate", cfg.E_s, f, d, sd, device, base)
        su = _expert_stack(cfg, "ws_up", cfg.E_s, f, d, sd, device, base)
        sdn = _expert_stack(cfg, "ws_down", cfg.E_s, d, f, sf, device, base)
    else:
        sg = su = sdn = None
    return LayerInputs(cfg, h, e, b, wg, wu, wd, sg, su, sdn)


# ---- host views for the oracle side (plain copies, no arithmetic) ----

def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a bfloat16 tensor as uint16."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_array(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.float32
    return t.detach().contiguous().cpu().numpy()


def host_array(t: Optional[torch.Tensor]):
    """bf16 tensors -> uint16 bit patterns; fp32 -> float32; int -> int array."""
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    if t.dtype == torch.float32:
        return f32_array(t)
    return t.detach().cpu().numpy()
