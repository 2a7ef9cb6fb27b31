"""Host-side argument checks of the Python layer (CPU only: every call below
raises before any library call reaches the GPU)."""
import pytest
import torch

from sparse_mixture_experts_biased_amd import LayerShape, MoELayer


def _layer(dtype="bf16"):
    T, d, E, K, f = 16, 64, 8, 2, 32
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    shape = LayerShape(T, d, E, K, 0, f, dtype, "sigmoid")
    e = torch.zeros((E, d))
    w = (torch.zeros((E, f, d), dtype=tdt), torch.zeros((E, f, d), dtype=tdt),
         torch.zeros((E, d, f), dtype=tdt))
    return MoELayer(shape, e, *w, device="cpu", overlap_shared=False), shape, tdt


def test_forward_rejects_mismatched_tokens():
    run, s, tdt = _layer()
    with pytest.raises(ValueError, match="shape"):
        run.forward(torch.zeros((s.T - 1, s.d_model), dtype=tdt))
    with pytest.raises(ValueError, match="shape"):
        run.forward(torch.zeros((s.T, s.d_model + 8), dtype=tdt))
    with pytest.raises(ValueError, match="dtype"):
        run.forward(torch.zeros((s.T, s.d_model), dtype=torch.float32))
    with pytest.raises(ValueError, match="contiguous"):
        run.forward(torch.zeros((s.d_model, s.T), dtype=tdt).t())
    with pytest.raises(ValueError):
        run.forward(None)


def test_forward_rejects_mismatched_bias():
    run, s, tdt = _layer()
    h = torch.zeros((s.T, s.d_model), dtype=tdt)
    with pytest.raises(ValueError, match="shape"):
        run.forward(h, torch.zeros(s.E_r + 1), 0.001)
    with pytest.raises(ValueError, match="dtype"):
        run.forward(h, torch.zeros(s.E_r, dtype=torch.float64), 0.001)


def test_backward_needs_prepare_and_forward():
    run, s, tdt = _layer()
    h = torch.zeros((s.T, s.d_model), dtype=tdt)
    with pytest.raises(RuntimeError, match="prepare_backward"):
        run.backward(h, h)
