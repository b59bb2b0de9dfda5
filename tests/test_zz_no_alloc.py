"""GPU check of moe_router_topk_noalloc, the router entry point that takes no
workspace (for callers that cannot allocate): its outputs must equal those
of moe_router_topk, which takes a caller workspace, bit for bit, on two calls
in a row where the second is smaller (so the fixed scratch still holds the
first call's values), for each router kernel family: at most 8 experts with
bf16 x (one launch), more than 8 experts (tiled logits and finishing
kernels, partial logits in the scratch) and fp32 x.  The outputs are also
held to the oracle's router protocol.  A call that would need more than the
fixed scratch is refused before any launch.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_harness import compare_router, say
import oracle as O
from sparse_mixture_experts_atomic_amd import _lib as L
from workloads.device import to_tensor

pytestmark = pytest.mark.gpu


def _inputs(cfg):
    arr = W.generate(cfg, with_experts=False)
    x = to_tensor(arr["x"], "cuda")
    w_g = to_tensor(arr["w_g"], "cuda")
    b_g = to_tensor(arr["b_g"], "cuda")
    return arr, x, w_g, b_g


def _outputs(T, k, E):
    return (torch.full((T, k), -1, dtype=torch.int32, device="cuda"),
            torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((E,), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda"))


def _both(cfg):
    arr, x, w_g, b_g = _inputs(cfg)
    T, E, k = cfg.T, cfg.E, cfg.k
    gate = L.GATE_MODES[cfg.gate]
    ref = _outputs(T, k, E)
    ws = torch.zeros(max(L.router_workspace_size(T, cfg.d, E, L.dtype_code(x)), 256), dtype=torch.uint8,
                     device="cuda")
    L.router_topk(x, w_g, b_g, k, gate, *ref, workspace=ws)
    got = _outputs(T, k, E)
    L.router_topk_noalloc(x, w_g, b_g, k, gate, *got)
    torch.cuda.synchronize()
    for name, a, b in zip(("topk_idx", "topk_gate", "prob_colsum", "logits"), got, ref):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{cfg.name}: {name} differs"
    # the oracle's router protocol on the allocation-free outputs
    z = O.router_logits(O.to_f64(arr["x"], cfg.act_dtype), arr["w_g"].astype(np.float64),
                        None if arr["b_g"] is None else arr["b_g"].astype(np.float64))
    compare_router(cfg.name, z, k, cfg.gate, got[0].cpu().numpy(), got[1].cpu().numpy().astype(np.float64),
                   got[2].cpu().numpy().astype(np.float64))
    say(f"noalloc {cfg.name}: T={T} d={cfg.d} E={E} k={k} {cfg.act_dtype}: bit-identical to the workspace call "
        f"(scratch {L.router_workspace_size(T, cfg.d, E, L.dtype_code(x))} bytes)")


# (first call, smaller second call) per router kernel family
PAIRS = {
    "mf8": (W.MIXTRAL, W.shrink(W.MIXTRAL, T=1000, d=1024, E=8, k=2)),
    "tiled": (W.DEEPSEEK, W.shrink(W.DEEPSEEK, T=777, d=2048, E=64, k=6)),
    "f32": (W.P1_GELU, W.TINY),
}


@pytest.mark.parametrize("family", list(PAIRS))
def test_noalloc_router_equals_the_workspace_router_on_two_calls(family):
    first, second = PAIRS[family]
    say(f"[case] noalloc router {family}: {first.name} then {second.name}")
    _both(first)
    _both(second)


def test_noalloc_router_refuses_a_call_beyond_its_scratch():
    say("[case] noalloc router beyond the fixed scratch")
    cfg = W.STRESS                                   # 32768 tokens x 256 experts: tens of MB of partial logits
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    assert L.router_workspace_size(T, d, E, L.BF16) > L.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, d), dtype=torch.bfloat16, device="cuda")
    w_g = torch.zeros((E, d), dtype=torch.float32, device="cuda")
    idx, gate, colsum, _ = _outputs(T, k, E)
    with pytest.raises(L.MoEError) as ei:
        L.router_topk_noalloc(x, w_g, None, k, L.GATE_PROB, idx, gate, colsum)
    assert ei.value.status == L.ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert torch.all(idx == -1)                     # nothing was written
