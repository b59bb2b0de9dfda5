"""GPU parity of dispatch and combine at the edges of their launch shapes.

Each case calls the C entry points through the binding with seeded inputs
and compares every output with the oracle (P1 §2.4 gather per expert and
scatter back; P5 专家容量 capacity drops):
  * rows wider than the one-launch dispatch kernel holds (fp32 d = 16392,
    bf16 d = 32776): they take the count/rank/permute kernels;
  * more than 256 slots per token (E = 512, k = 300);
  * more tokens than one launch has block rows in grid y (combine, T = 70000).
Integer outputs and packed rows are compared bit for bit, combine within the
fp32 / bf16 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_harness import act_to_f64, rownorm_err, say
from sparse_mixture_experts_atomic_amd import _lib as L

pytestmark = pytest.mark.gpu


def _distinct_ids(rng, T, k, E):
    """k distinct expert ids per token, in random order."""
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


def _dispatch(idx, E, C, x):
    T, k = idx.shape
    dev = "cuda"
    t_idx = torch.from_numpy(idx).to(dev)
    out = {n: torch.full(s, -7, dtype=torch.int32, device=dev)
           for n, s in (("counts_routed", (E,)), ("counts_kept", (E,)), ("offsets", (E + 1,)),
                        ("dest_pos", (T, k)), ("perm_token", (max(T * k, 1),)))}
    xp = torch.zeros((T * k, x.shape[1]), dtype=x.dtype, device=dev)
    ws = torch.zeros(max(L.dispatch_workspace_size(T, k, E), 256), dtype=torch.uint8, device=dev)
    L.dispatch_permute(t_idx, E, C, x, xp, out["counts_routed"], out["counts_kept"], out["offsets"],
                       out["dest_pos"], out["perm_token"], ws)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in out.items()}, xp


def _check_dispatch(name, idx, E, C, x):
    got, xp = _dispatch(idx, E, C, x)
    ref = O.dispatch(idx, E, C)
    for n in ("counts_routed", "counts_kept", "offsets", "dest_pos"):
        assert np.array_equal(got[n], ref[n]), f"{name}: {n} differs"
    A = int(ref["offsets"][-1])
    assert np.array_equal(got["perm_token"][:A], ref["perm_token"]), f"{name}: perm_token differs"
    # packed rows, byte for byte, against the oracle's permute of x
    view = torch.int16 if x.dtype == torch.bfloat16 else torch.int32
    want = O.permute(x.cpu().view(view).numpy(), ref["perm_token"])
    assert np.array_equal(xp[:A].cpu().view(view).numpy(), want), f"{name}: packed rows differ"
    say(f"{name}: T={idx.shape[0]} k={idx.shape[1]} E={E} C={C} kept {A} dropped {int((ref['dest_pos'] < 0).sum())}")


@pytest.mark.parametrize("dtype,d", [(torch.float32, 16392), (torch.bfloat16, 32776)])
def test_dispatch_rows_wider_than_the_one_launch_kernel(dtype, d):
    say(f"[case] dispatch wide rows {dtype} d={d}")
    rng = np.random.default_rng(61)
    T, k, E = 37, 2, 5
    idx = _distinct_ids(rng, T, k, E)
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to("cuda").to(dtype)
    _check_dispatch(f"wide {dtype} d={d}", idx, E, -1, x)
    _check_dispatch(f"wide {dtype} d={d} cap", idx, E, 9, x)


def test_dispatch_more_than_256_slots_per_token():
    say("[case] dispatch k = 300")
    rng = np.random.default_rng(62)
    T, k, E = 8, 300, 512
    idx = _distinct_ids(rng, T, k, E)
    x = torch.from_numpy(rng.standard_normal((T, 64)).astype(np.float32)).to("cuda").to(torch.bfloat16)
    _check_dispatch("k300", idx, E, -1, x)
    _check_dispatch("k300 cap", idx, E, 3, x)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_combine_beyond_the_grid_y_limit(dtype):
    say(f"[case] combine T = 70000 {dtype}")
    rng = np.random.default_rng(63)
    T, k, E, d = 70000, 2, 4, 16
    idx = _distinct_ids(rng, T, k, E)
    disp = O.dispatch(idx, E, int(T * k * 0.9 / E))          # some slots dropped
    A = int(disp["offsets"][-1])
    ye = torch.from_numpy(rng.standard_normal((A, d)).astype(np.float32)).to("cuda").to(dtype)
    gate = torch.from_numpy(rng.random((T, k)).astype(np.float32)).cuda()
    dest = torch.from_numpy(disp["dest_pos"]).cuda()
    res = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to("cuda").to(dtype)
    y = torch.full((T, d), float("nan"), dtype=dtype, device="cuda")
    L.combine(ye, dest, gate, d, None, 0, res, y)
    torch.cuda.synchronize()
    ref = O.combine(act_to_f64(ye), disp["dest_pos"], gate.cpu().numpy().astype(np.float64), None,
                    act_to_f64(res))
    err = rownorm_err(act_to_f64(y), ref)
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    assert err <= tol, f"combine T={T}: err {err:.3e}"
    say(f"combine T={T} {dtype}: err {err:.2e}, dropped slots {int((disp['dest_pos'] < 0).sum())}")


@pytest.mark.parametrize("T,k,E,C,skew", [(1000, 6, 16, -1, False), (777, 6, 100, 40, True),
                                          (4096, 6, 64, -1, True), (3000, 2, 9, 500, True)])
def test_dispatch_with_precounted_blocks(T, k, E, C, skew):
    """More than 8 experts and more than 4096 ids: the one-launch kernel takes
    its counts from the per-256-token-block counts of a launch before it;
    token ranges that straddle those blocks, capacity drops, skewed loads."""
    name = f"dispatch precount T={T} k={k} E={E} C={C}"
    say(f"[case] {name}")
    rng = np.random.default_rng(T + E)
    if skew:
        # a few experts take most of the assignments
        p = rng.random(E) ** 6
        p /= p.sum()
        idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    else:
        idx = _distinct_ids(rng, T, k, E)
    x = torch.from_numpy(rng.standard_normal((T, 256)).astype(np.float32)).to(torch.bfloat16).to("cuda")
    _check_dispatch(name, idx, E, C, x)
