"""Pins of the backward-pass oracle (oracle/moe_backward.py).

Each gradient is tied to something other than the oracle itself:
  * torch.autograd in float64 on the CPU, differentiating an independent
    dense formulation of the layer (P4 完整代码: every expert runs on every
    token and the outputs are weighted; here the weights are the gates of the
    selected, kept slots), with the selection and the drop decisions held
    fixed, as the oracle's reading takes them;
  * central finite differences of the oracle's own forward pass;
  * closed forms: no router gradient from the balance loss when the hard
    loads are uniform, none at all with one expert, the linear expert's
    weight gradient as an explicit sum, and nothing reaching the experts
    when every slot is dropped.
Planted mistakes (the renormalisation term dropped, the sign of the
softmax backward's correction flipped, SiLU's derivative taken as the
sigmoid, the gate left out of the expert-row gradient) each fail both the
autograd and the finite-difference pins.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle import moe_backward as B

F = torch.nn.functional


def _weights(rng, kind, E, d, d_ff, d_out, bias):
    n1 = d_out if kind == "linear" else d_ff
    w = {"w1": rng.standard_normal((E, n1, d)) / math.sqrt(d)}
    if kind == "swiglu":
        w["w3"] = rng.standard_normal((E, d_ff, d)) / math.sqrt(d)
    if kind != "linear":
        w["w2"] = rng.standard_normal((E, d_out, d_ff)) / math.sqrt(d_ff)
    if bias and kind != "swiglu":
        w["b1"] = rng.standard_normal((E, n1)) * 0.3
        if kind != "linear":
            w["b2"] = rng.standard_normal((E, d_out)) * 0.3
    return w


def _case(seed, kind, gate, C, n_shared, T=24, d=8, d_ff=12, E=5, k=2, bias=True, bg=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    w_g = rng.standard_normal((E, d)) * 0.7
    b_g = rng.standard_normal(E) * 0.5 if bg else None
    w = _weights(rng, kind, E, d, d_ff, d, bias)
    sh = _weights(rng, kind, n_shared, d, d_ff, d, bias) if n_shared else None
    dy = rng.standard_normal((T, d))
    return x, w_g, b_g, w, sh, dy


def _torch_ffn(kind, xt, w, e):
    def g(n):
        return None if w.get(n) is None else w[n][e]
    h = F.linear(xt, w["w1"][e], g("b1"))
    if kind == "linear":
        return h
    if kind == "relu":
        a = F.relu(h)
    elif kind == "gelu":
        a = F.gelu(h)
    else:
        a = F.silu(h) * F.linear(xt, w["w3"][e])
    return F.linear(a, w["w2"][e], g("b2"))


def _autograd(x, w_g, b_g, w, sh, dy, kind, gate, fwd, k, alpha, daux, residual):
    """Gradients of <dy, y> + daux * aux by torch.autograd on a dense layer
    with the oracle forward's selection (topk_idx) and drops (dest_pos < 0)
    as constants."""
    T, E = fwd["probs"].shape
    tt = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)  # noqa: E731
    xt, wgt = tt(x), tt(w_g)
    bgt = tt(b_g) if b_g is not None else None
    wt = {n: tt(v) for n, v in w.items()}
    sht = {n: tt(v) for n, v in sh.items()} if sh else None
    idx = torch.tensor(fwd["topk_idx"].astype(np.int64))
    keep = torch.tensor(fwd["dest_pos"] >= 0)
    p = torch.softmax(F.linear(xt, wgt, bgt), dim=-1)
    sel = torch.gather(p, 1, idx)
    g = sel / sel.sum(dim=1, keepdim=True) if gate == "renorm" else sel
    y = torch.zeros((T, dy.shape[1]), dtype=torch.float64)
    for e in range(E):
        we = (g * ((idx == e) & keep)).sum(dim=1)
        y = y + we[:, None] * _torch_ffn(kind, xt, wt, e)
    if sht:
        for s in range(sh["w1"].shape[0]):
            y = y + _torch_ffn(kind, xt, sht, s)
    if residual:
        y = y + xt
    f = torch.tensor(fwd["counts_routed"], dtype=torch.float64) / (T * k)
    aux = alpha * E * torch.sum(f * p.mean(dim=0))
    loss = torch.sum(torch.tensor(dy) * y) + daux * aux
    loss.backward()
    out = {"dx": xt.grad.numpy(), "dw_g": wgt.grad.numpy(), "db_g": None if bgt is None else bgt.grad.numpy(),
           "experts": {"d" + n: v.grad.numpy() for n, v in wt.items()},
           "shared": {"d" + n: v.grad.numpy() for n, v in sht.items()} if sht else {}}
    return out, float(aux.detach())


def _run(x, w_g, b_g, w, sh, dy, kind, gate, C, k, alpha=0.01, daux=1.0, residual=False):
    fwd = O.forward(x, w_g, b_g, k, gate, C, kind, w, sh, alpha, residual=x if residual else None)
    grad = B.backward(fwd, dy, x, w_g, k, gate, kind, w, sh, alpha, daux, residual)
    return fwd, grad


CASES = [(kind, gate, C, ns) for kind in ("linear", "relu", "gelu", "swiglu") for gate in ("prob", "renorm")
         for C, ns in ((-1, 0), (5, 1))]


@pytest.mark.parametrize("kind,gate,C,n_shared", CASES)
def test_backward_matches_torch_autograd(kind, gate, C, n_shared):
    x, w_g, b_g, w, sh, dy = _case(100 + CASES.index((kind, gate, C, n_shared)), kind, gate, C, n_shared)
    fwd, got = _run(x, w_g, b_g, w, sh, dy, kind, gate, C, 2, residual=n_shared > 0)
    if C >= 0:
        assert (fwd["dest_pos"] < 0).any()          # the drop path is exercised
    ref, _ = _autograd(x, w_g, b_g, w, sh, dy, kind, gate, fwd, 2, 0.01, 1.0, n_shared > 0)
    np.testing.assert_allclose(got["dx"], ref["dx"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["dw_g"], ref["dw_g"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["db_g"], ref["db_g"], rtol=1e-10, atol=1e-12)
    assert sorted(got["experts"]) == sorted(ref["experts"])
    for n in ref["experts"]:
        np.testing.assert_allclose(got["experts"][n], ref["experts"][n], rtol=1e-10, atol=1e-12, err_msg=n)
    for n in ref["shared"]:
        np.testing.assert_allclose(got["shared"][n], ref["shared"][n], rtol=1e-10, atol=1e-12, err_msg=n)


def _loss(x, w_g, b_g, w, sh, dy, kind, gate, C, k, alpha, daux):
    fwd = O.forward(x, w_g, b_g, k, gate, C, kind, w, sh, alpha)
    return float(np.sum(dy * fwd["y"]) + daux * fwd["aux_loss"]), fwd


@pytest.mark.parametrize("kind,gate", [("swiglu", "renorm"), ("gelu", "prob"), ("relu", "renorm")])
def test_backward_matches_central_differences(kind, gate):
    x, w_g, b_g, w, sh, dy = _case(7, kind, gate, 4, 1, T=16, d=6, d_ff=10, E=4, k=2)
    C, k, alpha, daux = 4, 2, 0.05, 0.7
    fwd, grad = _run(x, w_g, b_g, w, sh, dy, kind, gate, C, k, alpha, daux)
    rng = np.random.default_rng(8)
    h = 1e-5
    params = {"x": x, "w_g": w_g, "b_g": b_g, **{"e_" + n: v for n, v in w.items()},
              **{"s_" + n: v for n, v in sh.items()}}
    grads = {"x": grad["dx"], "w_g": grad["dw_g"], "b_g": grad["db_g"],
             **{"e_" + n: grad["experts"]["d" + n] for n in w}, **{"s_" + n: grad["shared"]["d" + n] for n in sh}}
    for name, v in params.items():
        dirn = rng.standard_normal(v.shape)

        def at(sign):
            pv = {n: (a + sign * h * dirn if n == name else a) for n, a in params.items()}
            ww = {n[2:]: a for n, a in pv.items() if n.startswith("e_")}
            ss = {n[2:]: a for n, a in pv.items() if n.startswith("s_")}
            val, f2 = _loss(pv["x"], pv["w_g"], pv["b_g"], ww, ss, dy, kind, gate, C, k, alpha, daux)
            # the selection and the drops must not move inside the step
            assert np.array_equal(f2["topk_idx"], fwd["topk_idx"])
            assert np.array_equal(f2["dest_pos"], fwd["dest_pos"])
            return val

        fd = (at(1.0) - at(-1.0)) / (2 * h)
        an = float(np.sum(grads[name] * dirn))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_balance_loss_gives_no_router_gradient_when_loads_are_uniform():
    # P5 负载均衡损失函数: the loss reaches the router only through P_i; with
    # uniform hard loads f_i = 1/E the gradient on p is the same for every
    # expert, and the softmax turns a constant into zero
    E, k, d = 4, 1, 4
    T = 4 * E
    x = np.tile(np.eye(d), (T // d, 1)) * 3.0               # token t prefers expert t mod E
    w_g = np.eye(E, d)
    w = _weights(np.random.default_rng(1), "linear", E, d, 0, d, True)
    fwd, grad = _run(x, w_g, None, w, None, np.zeros((T, d)), "linear", "prob", -1, k, alpha=0.3, daux=1.0)
    assert np.all(fwd["counts_routed"] == T * k // E)
    np.testing.assert_allclose(grad["dz"], 0.0, atol=1e-15)
    np.testing.assert_allclose(grad["dw_g"], 0.0, atol=1e-14)
    # with unequal loads the same loss does push the router
    w_g2 = w_g.copy()
    w_g2[0] += 2.0
    fwd2, grad2 = _run(x, w_g2, None, w, None, np.zeros((T, d)), "linear", "prob", -1, k, alpha=0.3, daux=1.0)
    assert fwd2["counts_routed"][0] > T // E
    assert np.abs(grad2["dz"]).max() > 1e-3
    # the overloaded expert's logits are pushed down: dL/dz_0 > 0 summed over tokens
    assert grad2["dz"][:, 0].sum() > 0


def test_one_expert_gives_no_router_gradient():
    x, w_g, b_g, w, sh, dy = _case(3, "swiglu", "renorm", -1, 0, E=1)
    _, grad = _run(x, w_g, b_g, w, sh, dy, "swiglu", "renorm", -1, 1)
    assert np.all(grad["dz"] == 0.0) and np.all(grad["dw_g"] == 0.0) and np.all(grad["db_g"] == 0.0)


def test_linear_expert_weight_gradient_is_the_gated_outer_product_sum():
    x, w_g, b_g, w, sh, dy = _case(4, "linear", "renorm", 3, 0, T=20, E=3, k=2)
    fwd, grad = _run(x, w_g, b_g, w, sh, dy, "linear", "renorm", 3, 2)
    E = w_g.shape[0]
    want_w = np.zeros_like(w["w1"])
    want_b = np.zeros_like(w["b1"])
    for t in range(x.shape[0]):
        for j in range(2):
            if fwd["dest_pos"][t, j] >= 0:
                e = fwd["topk_idx"][t, j]
                gj = fwd["topk_gate"][t, j]
                for r in range(want_w.shape[1]):
                    want_b[e, r] += gj * dy[t, r]
                    for c in range(want_w.shape[2]):
                        want_w[e, r, c] += gj * dy[t, r] * x[t, c]
    np.testing.assert_allclose(grad["experts"]["dw1"], want_w, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(grad["experts"]["db1"], want_b, rtol=1e-12, atol=1e-13)
    assert E == 3


def test_every_slot_dropped_leaves_the_experts_without_gradient():
    x, w_g, b_g, w, sh, dy = _case(5, "gelu", "renorm", 0, 0)
    fwd, grad = _run(x, w_g, b_g, w, sh, dy, "gelu", "renorm", 0, 2, alpha=0.1, daux=1.0, residual=True)
    assert np.all(fwd["dest_pos"] < 0)
    for v in grad["experts"].values():
        assert np.all(v == 0.0)
    assert np.all(grad["dg"] == 0.0)
    # only the residual and the balance loss reach x
    np.testing.assert_allclose(grad["dx"], dy + grad["dx_router"], rtol=0, atol=0)


def test_renormalisation_term_is_in_the_graph():
    # P1 §4.3: a detach in the top-k weight normalisation cuts part of the
    # router's gradient; the oracle keeps it, and autograd agrees
    x, w_g, b_g, w, sh, dy = _case(6, "relu", "renorm", -1, 0)
    fwd, grad = _run(x, w_g, b_g, w, sh, dy, "relu", "renorm", -1, 2, daux=0.0)
    idx, g, p = fwd["topk_idx"], fwd["topk_gate"], fwd["probs"]
    detached = np.zeros_like(p)
    for t in range(p.shape[0]):
        s = p[t, idx[t]].sum()
        for j in range(2):
            detached[t, idx[t, j]] += grad["dg"][t, j] / s
    assert np.abs(grad["dp"] - detached).max() > 1e-3
    ref, _ = _autograd(x, w_g, b_g, w, sh, dy, "relu", "renorm", fwd, 2, 0.01, 0.0, False)
    np.testing.assert_allclose(grad["dw_g"], ref["dw_g"], rtol=1e-10, atol=1e-12)


def test_activation_derivatives_closed_forms():
    # silu'(0) = 1/2, gelu'(0) = 1/2, gelu'(u) -> 1 and 0 in the tails;
    # against central differences of the forward forms elsewhere
    assert B.silu_grad(np.array(0.0)) == 0.5
    assert B.gelu_grad(np.array(0.0)) == 0.5
    assert B.gelu_grad(np.array(12.0)) == pytest.approx(1.0, abs=1e-15)
    assert B.gelu_grad(np.array(-12.0)) == pytest.approx(0.0, abs=1e-15)
    u = np.linspace(-6, 6, 241)
    h = 1e-6
    np.testing.assert_allclose(B.silu_grad(u), (O.silu(u + h) - O.silu(u - h)) / (2 * h), rtol=1e-8, atol=1e-9)
    np.testing.assert_allclose(B.gelu_grad(u), (O.gelu(u + h) - O.gelu(u - h)) / (2 * h), rtol=1e-8, atol=1e-9)
