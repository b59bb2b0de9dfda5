"""CPU oracle for the backward pass of the sparse MoE layer (float64).

TEST INFRASTRUCTURE ONLY, like the forward oracle next to it: only the
tests, the smoke check and the CPU-baseline leg of the benchmark may import
it; the product library never does and shares no code with it.

Sources (the same five pages as the forward oracle, cited by page and
section):
  P1 §2.4 and §4.3: the expert inputs are gathered and the outputs scattered
      back with index_add_ into a zero tensor; written that way the gradient
      of every token reaches exactly the expert rows it came from.  The
      top-k weight renormalisation must stay inside the graph (a detach there
      cuts the router's gradient).
  P1 §3.5: the training step differentiates task loss + coef * aux loss.
  P3 §2.2: the router's gradient comes back through the experts, and only the
      k selected experts of a token receive any.
  P5 负载均衡损失函数: in the balance loss f_i (hard assignment share) is
      discrete and carries no gradient; P_i (mean router probability) does.

Readings taken (the pages fix the forward only):
  * The top-k selection and the capacity drop decisions are piecewise
    constant in the inputs, so no gradient flows through them (a dropped
    slot's expert receives nothing and its gate weight has gradient 0).
  * The upstream gradient of the layer is dy [T, d_out] for y and daux for
    the aux loss value; the gradient of a residual input is dy itself.
  * ReLU'(0) = 0 (the value torch's relu takes).

Every step is written out in float64 with numpy matmul as the only library
primitive (and scipy's erf for GELU), in the reverse order of the forward
steps: combine, experts, permute, shared experts, gates, aux loss, softmax,
router matmul.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import scipy.special

from .moe_oracle import gelu, silu


def _sigmoid(u: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-u))


def gelu_grad(u: np.ndarray) -> np.ndarray:
    """d/du of u * Phi(u) = Phi(u) + u * phi(u) (phi the normal density)."""
    u = np.asarray(u, np.float64)
    Phi = 0.5 * (1.0 + scipy.special.erf(u / math.sqrt(2.0)))
    phi = np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)
    return Phi + u * phi


def silu_grad(u: np.ndarray) -> np.ndarray:
    """d/du of u * sigmoid(u) = sigmoid(u) * (1 + u * (1 - sigmoid(u)))."""
    s = _sigmoid(np.asarray(u, np.float64))
    return s * (1.0 + u * (1.0 - s))


def expert_ffn_backward(kind: str, rows: np.ndarray, dout: np.ndarray, w1: np.ndarray,
                        w3: Optional[np.ndarray] = None, w2: Optional[np.ndarray] = None,
                        b1: Optional[np.ndarray] = None, b2: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradients of one expert (the forms of the forward oracle's expert_ffn)
    for the batch `rows` [n, d] given the output gradient `dout` [n, d_out].

    Returns drows [n, d] and the weight gradients dw1 (and dw3, dw2, db1, db2
    where the expert has them), each summed over the n rows.
    """
    rows = np.asarray(rows, np.float64)
    dout = np.asarray(dout, np.float64)
    h = rows @ w1.T
    if b1 is not None:
        h = h + b1[None, :]
    out: Dict[str, np.ndarray] = {}
    if kind == "linear":
        dh = dout
    else:
        if kind == "relu":
            a = np.maximum(h, 0.0)
        elif kind == "gelu":
            a = gelu(h)
        elif kind == "swiglu":
            h3 = rows @ w3.T
            a = silu(h) * h3
        else:
            raise ValueError(kind)
        # second matrix: y = a W2^T + b2
        out["dw2"] = dout.T @ a
        if b2 is not None:
            out["db2"] = dout.sum(axis=0)
        da = dout @ w2
        if kind == "relu":
            dh = da * (h > 0.0)
        elif kind == "gelu":
            dh = da * gelu_grad(h)
        else:
            dh = da * h3 * silu_grad(h)
            dh3 = da * silu(h)
            out["dw3"] = dh3.T @ rows
    out["dw1"] = dh.T @ rows
    if b1 is not None:
        out["db1"] = dh.sum(axis=0)
    drows = dh @ w1
    if kind == "swiglu":
        drows = drows + dh3 @ w3
    out["drows"] = drows
    return out


def combine_backward(dy: np.ndarray, ye: np.ndarray, dest_pos: np.ndarray, g: np.ndarray):
    """Gradient of y[t] = sum_j (kept) g[t,j] Ye[dest[t,j]] with respect to
    the expert rows and the gate weights.

    The forward accumulates into a zero output (P1 §4.3, index_add_), so each
    kept slot's expert row receives g[t,j] * dy[t] and its gate weight the
    dot product dy[t] . Ye[dest[t,j]]; dropped slots receive nothing.
    """
    T, k = dest_pos.shape
    dye = np.zeros((ye.shape[0], dy.shape[1]), np.float64)
    dg = np.zeros((T, k), np.float64)
    for t in range(T):
        for j in range(k):
            p = int(dest_pos[t, j])
            if p >= 0:
                dye[p] = g[t, j] * dy[t]
                dg[t, j] = float(np.dot(dy[t], ye[p]))
    return dye, dg


def permute_backward(dxp: np.ndarray, dest_pos: np.ndarray, T: int) -> np.ndarray:
    """Gradient of Xp[dest[t,j]] = x[t]: every kept slot's row gradient goes
    back to its token (P1 §2.4 gather; the transposed operation is a sum)."""
    dx = np.zeros((T, dxp.shape[1]), np.float64)
    for t in range(T):
        for j in range(dest_pos.shape[1]):
            p = int(dest_pos[t, j])
            if p >= 0:
                dx[t] += dxp[p]
    return dx


def gates_backward(dg: np.ndarray, p: np.ndarray, idx: np.ndarray, g: np.ndarray, mode: str) -> np.ndarray:
    """Gradient of the gate weights with respect to the softmax
    probabilities p [T, E].

    'prob' (g = p of the selected expert): dp[t, S_j] += dg[t, j].
    'renorm' (g_j = p_{S_j} / s with s the sum over the selected experts;
    P1 §4.3: the normalisation stays in the graph):
        dp[t, S_j] += (dg[t, j] - sum_i dg[t, i] g[t, i]) / s.
    """
    T, k = idx.shape
    dp = np.zeros_like(np.asarray(p, np.float64))
    for t in range(T):
        if mode == "prob":
            for j in range(k):
                dp[t, idx[t, j]] += dg[t, j]
        elif mode == "renorm":
            s = float(np.sum(p[t, idx[t]]))
            c = float(np.dot(dg[t], g[t]))
            for j in range(k):
                dp[t, idx[t, j]] += (dg[t, j] - c) / s
        else:
            raise ValueError(mode)
    return dp


def aux_loss_grad_probs(counts_routed: np.ndarray, T: int, k: int, E: int, alpha: float,
                        daux: float) -> np.ndarray:
    """Gradient of L = alpha E sum_e f_e P_e with respect to p[t, e].

    P5 负载均衡损失函数: f_e is a count of hard assignments (no gradient);
    P_e = (1/T) sum_t p[t, e], so dL/dp[t, e] = alpha E f_e / T for every t.
    Returned as one row [E] (the same for every token).
    """
    f = np.asarray(counts_routed, np.float64) / float(T * k)
    return daux * alpha * E * f / float(T)


def softmax_backward(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """dz[t, e] = p[t, e] (dp[t, e] - sum_e' p[t, e'] dp[t, e'])."""
    p = np.asarray(p, np.float64)
    return p * (dp - np.sum(p * dp, axis=1, keepdims=True))


def router_backward(x: np.ndarray, w_g: np.ndarray, dz: np.ndarray):
    """z = x W_g^T + b_g: dW_g = dz^T x, db_g = sum_t dz[t], dx = dz W_g."""
    x = np.asarray(x, np.float64)
    return dz.T @ x, dz.sum(axis=0), dz @ np.asarray(w_g, np.float64)


def backward(fwd: Dict[str, np.ndarray], dy: np.ndarray, x: np.ndarray, w_g: np.ndarray, k: int,
             gate_mode: str, kind: str, weights: Dict[str, np.ndarray],
             shared: Optional[Dict[str, np.ndarray]] = None, alpha: float = 1.0, daux: float = 1.0,
             residual: bool = False) -> Dict[str, object]:
    """Gradients of <dy, y> + daux * aux for the layer run by the forward
    oracle (`fwd` is what moe_oracle.forward returned on the same inputs).

    Steps, in reverse order of the forward: combine, experts, permute,
    shared experts, residual, gates, aux loss, softmax, router.
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    T = x.shape[0]
    E = w_g.shape[0]
    dest = fwd["dest_pos"]
    dye, dg = combine_backward(dy, fwd["ye"], dest, fwd["topk_gate"])
    offsets = np.asarray(fwd["offsets"], np.int64)
    dxp = np.zeros((int(offsets[E]), x.shape[1]), np.float64)
    ex_grads: Dict[str, np.ndarray] = {}
    for name in ("w1", "w3", "w2", "b1", "b2"):
        if weights.get(name) is not None:
            ex_grads["d" + name] = np.zeros_like(weights[name], dtype=np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b <= a:
            continue
        r = expert_ffn_backward(kind, fwd["xp"][a:b], dye[a:b], weights["w1"][e],
                                None if weights.get("w3") is None else weights["w3"][e],
                                None if weights.get("w2") is None else weights["w2"][e],
                                None if weights.get("b1") is None else weights["b1"][e],
                                None if weights.get("b2") is None else weights["b2"][e])
        dxp[a:b] = r["drows"]
        for name, v in r.items():
            if name != "drows":
                ex_grads[name][e] = v
    dx = permute_backward(dxp, dest, T)
    sh_grads: Dict[str, np.ndarray] = {}
    if shared:
        for name in ("w1", "w3", "w2", "b1", "b2"):
            if shared.get(name) is not None:
                sh_grads["d" + name] = np.zeros_like(shared[name], dtype=np.float64)
        dxs = np.zeros_like(x)
        for s in range(shared["w1"].shape[0]):
            r = expert_ffn_backward(kind, x, dy, shared["w1"][s],
                                    None if shared.get("w3") is None else shared["w3"][s],
                                    None if shared.get("w2") is None else shared["w2"][s],
                                    None if shared.get("b1") is None else shared["b1"][s],
                                    None if shared.get("b2") is None else shared["b2"][s])
            dxs += r["drows"]
            for name, v in r.items():
                if name != "drows":
                    sh_grads[name][s] = v
        dx = dx + dxs
    else:
        dxs = None
    if residual:
        dx = dx + dy
    p = fwd["probs"]
    dp = gates_backward(dg, p, fwd["topk_idx"], fwd["topk_gate"], gate_mode)
    dp = dp + aux_loss_grad_probs(fwd["counts_routed"], T, k, E, alpha, daux)[None, :]
    dz = softmax_backward(p, dp)
    dw_g, db_g, dx_router = router_backward(x, w_g, dz)
    dx = dx + dx_router
    return {"dx": dx, "dw_g": dw_g, "db_g": db_g, "dye": dye, "dg": dg, "dxp": dxp, "dxs": dxs, "dp": dp,
            "dz": dz, "dx_router": dx_router, "experts": ex_grads, "shared": sh_grads}
