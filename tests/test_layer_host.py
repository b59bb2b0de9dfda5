"""Host-side checks of the layer object (no kernel runs)."""
import pytest

import workloads as W
from sparse_mixture_experts_atomic_amd import MoELayer
from sparse_mixture_experts_atomic_amd import _lib as L
from workloads.device import layer_kwargs


def test_backward_refuses_a_gathered_layer():
    cfg = W.shrink(W.MIXTRAL, T=16, d=64, d_ff=64, E=4, k=2)
    arr = W.generate(cfg)
    C = L.capacity(cfg.T, cfg.k, cfg.E, cfg.cf, cfg.cap_round)
    layer = MoELayer(**layer_kwargs(cfg, arr, C, "cpu"), gather_rows=True)
    with pytest.raises(ValueError, match="packed rows"):
        layer.enable_backward()
