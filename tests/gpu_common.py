"""Helpers for the GPU parity tests: run the HIP entry points on seeded inputs
and compare with the CPU oracle run on host copies of the very same inputs.

Acceptance (written once here, used by every parity test):
  * expert ids, loads, offsets, row maps, bias updates: bit-exact, except
    tokens whose oracle top-K margin v_(K) - v_(K+1) is below NEAR_TIE; on
    those the GPU's set must still be a valid top-K within NEAR_TIE;
  * gates: |g_gpu - g_oracle| <= GATE_TOL;
  * layer / expert outputs: max|d| <= 2e-2 * max|y_ref| with bf16 data and
    fp32 accumulation, <= 1e-4 * max|y_ref| for fp32 data.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import moe_oracle as O
from synthetic import host_array

NEAR_TIE = 1e-5
GATE_TOL = 1e-5
BF16_REL = 2e-2
F32_REL = 1e-4


def say(msg: str):
    sys.stderr.write(f"   .. {msg}\n")
    sys.stderr.flush()


def out_tol(dtype: str) -> float:
    return BF16_REL if dtype == "bf16" else F32_REL


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return O.to_f64(host_array(t))


def check_route(h, e, b, K, fn, idx_gpu, gates_gpu, loads_gpu, E):
    """Compare one routing call with the oracle. Returns (n_near, n_flipped, oracle dict)."""
    hh, ee = host_array(h), host_array(e)
    bb = host_array(b) if b is not None else None
    r = O.route(hh, ee, bb, K, fn)
    margin = O.topk_margin(r["s"], bb, K)
    near = margin < NEAR_TIE
    gi = idx_gpu.cpu().numpy()
    gg = gates_gpu.cpu().numpy()
    gl = loads_gpu.cpu().numpy()
    same = np.all(gi == r["idx"], axis=1)
    # every differing token must be a near-tie, and the GPU's set a valid top-K
    bad = ~same & ~near
    assert not bad.any(), f"{bad.sum()} tokens differ with margin >= {NEAR_TIE}"
    v = O.biased_values(r["s"], bb).astype(np.float64)
    flipped = np.nonzero(~same)[0]
    for t in flipped:
        kth = -np.sort(-v[t])[K - 1]
        assert np.all(v[t, gi[t]] >= kth - NEAR_TIE)
        assert len(set(gi[t].tolist())) == K and np.all(np.diff(gi[t]) > 0)
    # ids ascending and distinct everywhere
    assert np.all(np.diff(gi, axis=1) > 0)
    # gates where the set matches
    assert np.max(np.abs(gg[same] - r["gates"][same]), initial=0.0) <= GATE_TOL
    # loads are the histogram of the GPU's own picks; equal to the oracle's when nothing flipped
    assert np.array_equal(gl, np.bincount(gi.reshape(-1), minlength=E))
    if len(flipped) == 0:
        assert np.array_equal(gl, r["loads"])
    return int(near.sum()), int(len(flipped)), r


def rel_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    scale = np.max(np.abs(y_ref))
    return float(np.max(np.abs(y_gpu - y_ref)) / (scale if scale > 0 else 1.0))
