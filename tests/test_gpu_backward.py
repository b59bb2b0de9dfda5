"""GPU parity of the backward pass (moe_combine_backward,
moe_expert_ffn_grouped_backward, moe_router_backward, moe_permute_backward)
against the float64 backward oracle (oracle/moe_backward.py).

Stage-wise, as for the forward: each stage is checked against the oracle fed
the GPU's own upstream values (the forward's packed rows, expert outputs,
logits, ids and gates; the backward's dYe, dgate, dXp), so that rounding in
one stage is never charged to the next.  Then the whole backward against
the oracle run from scratch on shapes without near-tied tokens.

Tolerances:
  * bf16 outputs (dYe, dXp, dx) and the weight gradients of the bf16 FFN
    (fp32, but from bf16 operands and bf16 intermediates h, dh, a): 2e-2 in
    the row-normwise form (max over rows of the inf-norm of the difference
    over the inf-norm of the reference row, floor 1e-6 of the largest row);
  * fp32 sums (dgate = dy . Ye, dW_g = dz^T x, db_g, and dz = p (dp -
    sum p dp), which cancels where a token's dp are nearly equal): the error
    of a sum of n terms is bounded by n eps |terms|, so the bound is 1e-5
    times the sum of the absolute values of the terms, element by element;
  * end to end from scratch: 3e-2 (the forward's bf16 expert outputs feed
    dgate, which feeds every router gradient), row-normwise for dx and dW_g,
    and normwise over each expert's whole matrix for the expert weight
    gradients: a weight-gradient row of an expert with one or two rows is a
    single product, whose relative error is that of one element of dYe W2,
    and the bf16 rounding of dYe (the forward stores Ye in bf16, and
    moe_combine_backward writes dYe in bf16) leaves that unbounded where the
    element nearly cancels.  The stage-wise check, fed the GPU's own dYe,
    keeps the per-row form for them.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_harness import act_to_f64, rownorm_err, say
from oracle import moe_backward as B
from sparse_mixture_experts_atomic_amd import MoELayer
from sparse_mixture_experts_atomic_amd import _lib as L
from workloads.device import layer_kwargs, to_tensor

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-5
E2E_TOL = 3e-2


def _cfg(name, **kw):
    base = dict(d_out=0, cf=None, act_dtype="bf16", w_dtype="bf16", alpha=1e-2)
    base.update(kw)
    if not base["d_out"]:
        base["d_out"] = base["d"]
    return W.MoEConfig(name=name, **base)


CASES = {
    "mixtral_s": W.shrink(W.MIXTRAL, T=600, d=256, d_ff=448, E=8, k=2),
    "deepseek_s": W.shrink(W.DEEPSEEK, T=500, d=256, d_ff=192, E=64, k=6),
    "switch_drop_s": W.shrink(W.SWITCH_DROP, T=700, d=256, d_ff=384, E=8, k=1),
    "cap_hit_k4": _cfg("cap_hit_k4", T=513, d=128, E=8, k=4, ffn="swiglu", d_ff=136, gate="renorm", cf=0.6,
                       wg_dist=("normal", 1 / 128), bg_var=1.0, w1_var=1 / 128, w3_var=1 / 128, w2_var=1 / 136,
                       seed=25),
    "gelu_bias": W.P1_GELU.scaled(name="p1_gelu_bf16", act_dtype="bf16", w_dtype="bf16", seed=42),
    "linear_bias": _cfg("linear_bias", T=333, d=72, d_out=40, E=5, k=2, ffn="linear", d_ff=0, gate="prob",
                        wg_dist=("normal", 1 / 72), w1_var=1 / 72, b1_var=0.1, seed=23),
    "empty_experts": _cfg("empty_experts", T=40, d=64, E=64, k=1, ffn="swiglu", d_ff=64, gate="prob",
                          wg_dist=("normal", 1 / 64), w1_var=1 / 64, w3_var=1 / 64, w2_var=1 / 64, seed=24),
}


def _sum_bound_err(got, ref, absterms):
    """max |got - ref| / (1e-5 * sum |terms|), elementwise (<= 1 passes)."""
    den = np.maximum(F32_TOL * absterms, 1e-30)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref) / den)) if ref.size else 0.0


class BwdRun:
    def __init__(self, cfg, seed=77, residual=False, keep_pre=True, arr=None):
        self.cfg = cfg
        self.arr = W.generate(cfg) if arr is None else arr
        self.C = L.capacity(cfg.T, cfg.k, cfg.E, cfg.cf, cfg.cap_round)
        assert self.C == O.capacity(cfg.T, cfg.k, cfg.E, cfg.cf, cfg.cap_round)
        self.layer = MoELayer(**layer_kwargs(cfg, self.arr, self.C, "cuda"))
        self.layer.enable_backward(keep_pre=keep_pre)
        self.x = to_tensor(self.arr["x"], "cuda")
        self.x64 = O.to_f64(self.arr["x"], cfg.act_dtype)
        rng = np.random.default_rng(seed)
        dy32 = rng.standard_normal((cfg.T, cfg.d_out)).astype(np.float32)
        self.dy = torch.from_numpy(dy32).to("cuda").to(torch.bfloat16)
        self.dy64 = act_to_f64(self.dy)
        self.residual = residual
        self.daux = 0.75
        self.w = O.decode_weights(self.arr, cfg.w_dtype)
        self.sh = O.decode_weights(self.arr, cfg.w_dtype, prefix="sh_") if cfg.n_shared else None
        self.w_g = self.arr["w_g"].astype(np.float64)
        self.b_g = None if self.arr["b_g"] is None else self.arr["b_g"].astype(np.float64)

    def run(self):
        ly = self.layer
        ly.forward(self.x, self.x if self.residual else None)
        ly.backward(self.x, self.dy, self.daux, self.residual)
        torch.cuda.synchronize()
        g = lambda t: t.cpu().numpy()  # noqa: E731
        self.dest = g(ly.dest_pos)
        self.idx = g(ly.topk_idx)
        self.gate = g(ly.topk_gate).astype(np.float64)
        self.offsets = g(ly.offsets).astype(np.int64)
        self.counts = g(ly.counts_routed)
        self.A = int(self.offsets[-1])

    # -- stages ---------------------------------------------------------------
    def check_combine(self):
        ly, cfg = self.layer, self.cfg
        ye = act_to_f64(ly.y_rows[:max(self.A, 1)])[:self.A]
        dye_ref, dg_ref = B.combine_backward(self.dy64, ye, self.dest, self.gate)
        dye = act_to_f64(ly.dy_rows[:max(self.A, 1)])[:self.A]
        e1 = rownorm_err(dye, dye_ref)
        absdot = np.zeros_like(dg_ref)
        for t in range(cfg.T):
            for j in range(cfg.k):
                if self.dest[t, j] >= 0:
                    absdot[t, j] = np.sum(np.abs(self.dy64[t] * ye[self.dest[t, j]]))
        dg = ly.dgate.cpu().numpy()
        e2 = _sum_bound_err(dg, dg_ref, absdot)
        assert np.all(dg[self.dest < 0] == 0.0)
        assert e1 <= BF16_TOL and e2 <= 1.0, (e1, e2)
        self.dye, self.dg = dye, dg.astype(np.float64)
        say(f"combine bwd {cfg.name}: dYe rows {self.A} err {e1:.2e}; dgate {cfg.T}x{cfg.k} err/bound {e2:.2e}")

    def _ffn_stage(self, name, rows_in, dy_rows, w, offsets, dx_rows_gpu, grads_gpu, experts=None):
        cfg = self.cfg
        worst = {}
        E = len(offsets) - 1
        for e in (range(E) if experts is None else experts):
            a, b = int(offsets[e]), int(offsets[e + 1])
            pick = lambda n: None if w.get(n) is None else w[n][e]  # noqa: E731
            if b <= a:
                # no rows: zero gradients
                for n, t in grads_gpu.items():
                    assert np.all(t[e] == 0.0), (name, n, e)
                continue
            r = B.expert_ffn_backward(cfg.ffn, rows_in(a, b), dy_rows(a, b), pick("w1"), pick("w3"), pick("w2"),
                                      pick("b1"), pick("b2"))
            worst["dx"] = max(worst.get("dx", 0.0), rownorm_err(dx_rows_gpu(a, b), r["drows"]))
            for n, t in grads_gpu.items():
                ref = r[n]
                got = t[e].astype(np.float64)
                err = rownorm_err(got.reshape(ref.shape[0], -1), ref.reshape(ref.shape[0], -1)) if ref.ndim == 2 \
                    else rownorm_err(got[None, :], ref[None, :])
                worst[n] = max(worst.get(n, 0.0), err)
        for n, v in worst.items():
            assert v <= BF16_TOL, (name, n, v)
        say(f"ffn bwd {name} {cfg.name}: " + " ".join(f"{n} {v:.2e}" for n, v in sorted(worst.items())))

    def check_experts(self, experts=None):
        ly = self.layer
        xp = lambda a, b: act_to_f64(ly.x_perm[a:b])  # noqa: E731
        dyr = lambda a, b: act_to_f64(ly.dy_rows[a:b])  # noqa: E731
        dxr = lambda a, b: act_to_f64(ly.dx_rows[a:b])  # noqa: E731
        grads = {"d" + n: ly.grad[n].cpu().numpy() for n in ("w1", "w3", "w2", "b1", "b2") if n in ly.grad}
        self._ffn_stage("routed", xp, dyr, self.w, self.offsets, dxr, grads, experts)
        if self.cfg.n_shared:
            T = self.cfg.T
            sh_off = np.arange(0, (self.cfg.n_shared + 1) * T, T)
            grads = {"d" + n: ly.grad["sh_" + n].cpu().numpy() for n in ("w1", "w3", "w2", "b1", "b2")
                     if "sh_" + n in ly.grad}
            dxs = ly.dx_shared.reshape(-1, self.cfg.d)
            self._ffn_stage("shared", lambda a, b: self.x64, lambda a, b: self.dy64, self.sh, sh_off,
                            lambda a, b: act_to_f64(dxs[a:b]), grads)

    def check_router(self):
        ly, cfg = self.layer, self.cfg
        z = ly.logits.cpu().numpy().astype(np.float64)
        p = O.softmax(z)
        dp = B.gates_backward(self.dg, p, self.idx, self.gate, cfg.gate)
        dp = dp + B.aux_loss_grad_probs(self.counts, cfg.T, cfg.k, cfg.E, cfg.alpha, self.daux)[None, :]
        dz_ref = B.softmax_backward(p, dp)
        dz = ly.dz.cpu().numpy()
        # dz = p (dp - sum p dp) cancels where a token's dp are nearly equal,
        # and dp (renorm: (dg_j - sum_i dg_i g_i) / s) cancels too: bound the
        # fp32 error by the size of the terms both are formed from
        absdp = np.broadcast_to(B.aux_loss_grad_probs(self.counts, cfg.T, cfg.k, cfg.E, cfg.alpha, self.daux),
                                p.shape).copy()
        for t in range(cfg.T):
            if cfg.gate == "renorm":
                s_t = np.sum(p[t, self.idx[t]])
                c_t = np.sum(np.abs(self.dg[t]) * self.gate[t])
                for j in range(cfg.k):
                    absdp[t, self.idx[t, j]] += (abs(self.dg[t, j]) + c_t) / s_t
            else:
                for j in range(cfg.k):
                    absdp[t, self.idx[t, j]] += abs(self.dg[t, j])
        e1 = _sum_bound_err(dz, dz_ref, p * (absdp + np.sum(p * absdp, axis=1, keepdims=True)))
        dwg_ref, dbg_ref, _ = B.router_backward(self.x64, self.w_g, dz.astype(np.float64))
        e2 = _sum_bound_err(ly.grad["w_g"].cpu().numpy(), dwg_ref, np.abs(dz).T.astype(np.float64) @ np.abs(self.x64))
        e3 = _sum_bound_err(ly.grad["b_g"].cpu().numpy(), dbg_ref, np.sum(np.abs(dz), axis=0).astype(np.float64))
        assert e1 <= 1.0 and e2 <= 1.0 and e3 <= 1.0, (e1, e2, e3)
        self.dz = dz.astype(np.float64)
        say(f"router bwd {cfg.name}: dz err/bound {e1:.2e}; dW_g err/bound {e2:.2e}; db_g err/bound {e3:.2e}")

    def check_permute(self):
        ly, cfg = self.layer, self.cfg
        dxp = act_to_f64(ly.dx_rows[:max(self.A, 1)])[:self.A]
        ref = B.permute_backward(dxp, self.dest, cfg.T)
        if cfg.n_shared:
            ref = ref + act_to_f64(ly.dx_shared).sum(axis=0)
        if self.residual:
            ref = ref + self.dy64
        ref = ref + self.dz @ self.w_g
        err = rownorm_err(act_to_f64(ly.dx), ref)
        assert err <= BF16_TOL, err
        say(f"permute bwd {cfg.name}: dx {cfg.T} rows err {err:.2e}")

    def check_e2e(self):
        cfg = self.cfg
        fwd = O.forward(self.x64, self.w_g, self.b_g, cfg.k, cfg.gate, self.C, cfg.ffn, self.w, self.sh, cfg.alpha,
                        residual=self.x64 if self.residual else None)
        if fwd["near_tie"].any() or not np.array_equal(fwd["topk_idx"], self.idx):
            say(f"e2e bwd {cfg.name}: skipped ({int(fwd['near_tie'].sum())} near-tied tokens)")
            return
        ref = B.backward(fwd, self.dy64, self.x64, self.w_g, cfg.k, cfg.gate, cfg.ffn, self.w, self.sh, cfg.alpha,
                         self.daux, self.residual)
        ly = self.layer
        errs = {"dx": rownorm_err(act_to_f64(ly.dx), ref["dx"]),
                "dw_g": rownorm_err(ly.grad["w_g"].cpu().numpy(), ref["dw_g"])}
        if self.b_g is not None:
            errs["db_g"] = rownorm_err(ly.grad["b_g"].cpu().numpy()[None, :], ref["db_g"][None, :])
        # weight gradients from scratch: normwise over each expert's whole
        # matrix (see the module docstring)
        for n, v in ref["experts"].items():
            got = ly.grad[n[1:]].cpu().numpy().astype(np.float64)
            errs["routed " + n] = rownorm_err(got.reshape(v.shape[0], -1), v.reshape(v.shape[0], -1))
        for n, v in ref["shared"].items():
            got = ly.grad["sh_" + n[1:]].cpu().numpy().astype(np.float64)
            errs["shared " + n] = rownorm_err(got.reshape(v.shape[0], -1), v.reshape(v.shape[0], -1))
        for n, v in errs.items():
            assert v <= E2E_TOL, (n, v)
        say(f"e2e bwd {cfg.name}: " + " ".join(f"{n} {v:.2e}" for n, v in errs.items()))

    def run_all(self, e2e=True):
        self.run()
        self.check_combine()
        self.check_experts()
        self.check_router()
        self.check_permute()
        if e2e:
            self.check_e2e()


@pytest.mark.parametrize("name", list(CASES))
def test_backward_stages_and_end_to_end(name):
    say(f"[case] backward {name}")
    BwdRun(CASES[name], residual=name == "deepseek_s").run_all()


def test_backward_is_deterministic():
    say("[case] backward determinism")
    r = BwdRun(CASES["deepseek_s"])
    outs = []
    for _ in range(2):
        r.run()
        outs.append([r.layer.dx.clone(), r.layer.dz.clone()] + [t.clone() for t in r.layer.grad.values()])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.timeout(600)
def test_backward_mixtral_full():
    """The Mixtral-shaped layer at full size: every stage, the FFN backward on
    three whole experts (first, middle, last)."""
    say("[case] backward full mixtral")
    r = BwdRun(W.MIXTRAL)
    r.run()
    r.check_combine()
    r.check_experts(experts=[0, 3, 7])
    r.check_router()
    r.check_permute()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["mixtral_s", "deepseek_s", "switch_drop_s", "gelu_bias", "cap_hit_k4",
                                  "empty_experts", "mixtral_full"])
def test_kept_pre_activations_match_recompute(name):
    """Training forward keeping the first product's fp32 pre-activations
    (moe_expert_ffn_grouped_train) and the backward reading them
    (moe_expert_ffn_grouped_backward_kept).  The backward's gradients are
    the recomputing backward's, bit for bit, on the same rows (the kept and
    the recomputed pre-activations are the same GEMM, unsplit).  The
    forward's output: bit for bit where the plain forward does not split
    tail tiles over K (the full Mixtral shape), else within the bf16
    tolerance (the split sums in another order).  Shapes the kept path does
    not take (d = 64) fall back to the recomputing path."""
    cfg = W.MIXTRAL if name == "mixtral_full" else CASES[name]
    say(f"[case] kept pre-activations {name}: T={cfg.T} d={cfg.d} E={cfg.E} {cfg.ffn}")
    r = BwdRun(cfg, residual=name == "deepseek_s")
    r.run()
    ly = r.layer
    flags = dict(ly._kept)
    expect = cfg.d % 128 == 0
    assert flags["routed"] == expect, flags
    if cfg.n_shared:
        assert flags["shared"] == expect, flags
    w = ly.w
    A = cfg.T * cfg.k
    # the plain forward of the routed experts on the same rows
    y_plain = torch.empty_like(ly.y_rows)
    L.expert_ffn_grouped(ly.kind, ly.x_perm, A, L.ROWS_PACKED, ly.offsets, cfg.E, cfg.d, cfg.d_ff, cfg.d_out,
                         w["w1"], w.get("w3"), w.get("w2"), None, None, None, w.get("b1"), w.get("b2"), y_plain,
                         ly.ws_ffn)
    # the recomputing backward on the same rows and output gradients
    ws = torch.empty(L.ffn_backward_workspace_size(ly.kind, A, cfg.E, cfg.d, cfg.d_ff, cfg.d_out),
                     dtype=torch.uint8, device="cuda")
    names = [n for n in ("w1", "w3", "w2", "b1", "b2") if n in ly.grad]
    g = {n: torch.full_like(ly.grad[n], -7.0) for n in names}
    dx_rows = torch.full_like(ly.dx_rows, -7.0)
    L.expert_ffn_grouped_backward(ly.kind, ly.x_perm, A, L.ROWS_PACKED, ly.offsets, cfg.E, cfg.d, cfg.d_ff,
                                  cfg.d_out, w["w1"], w.get("w3"), w.get("w2"), w.get("b1"), w.get("b2"), ly.dy_rows,
                                  dx_rows, g["w1"], g.get("w3"), g.get("w2"), g.get("b1"), g.get("b2"), ws)
    torch.cuda.synchronize()
    n_rows = r.A
    for n in names:
        assert torch.equal(_bits(ly.grad[n]), _bits(g[n])), n
    assert torch.equal(_bits(ly.dx_rows[:n_rows]), _bits(dx_rows[:n_rows])), "dx_rows"
    got, ref = ly.y_rows[:n_rows], y_plain[:n_rows]
    if name == "mixtral_full":
        assert torch.equal(_bits(got), _bits(ref)), "y_rows"
    else:
        err = rownorm_err(act_to_f64(got), act_to_f64(ref))
        assert err <= BF16_TOL, err
    differ = int((_bits(got) != _bits(ref)).sum())
    say(f"  kept {flags}: gradients and dx_rows bit-identical to the recomputing backward; "
        f"forward y_rows: {differ} of {got.numel()} elements differ from the plain forward")
