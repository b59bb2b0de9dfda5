"""One MoE layer forward on the GPU: owns its device buffers and runs the
five library calls in order on the current stream.

router -> dispatch/permute -> grouped FFN (routed, then shared) -> combine
-> aux loss.  Every step runs in libmoe.so; this class only allocates the
buffers once and passes pointers.
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import _lib as L


class MoELayer:
    def __init__(self, *, T: int, d: int, d_out: int, E: int, k: int, kind: str, d_ff: int, gate: str,
                 capacity: int, n_shared: int, alpha: float, act_dtype: torch.dtype,
                 weights: Dict[str, Optional[torch.Tensor]], device="cuda", gather_rows: bool = False,
                 fp8_act: bool = False):
        self.T, self.d, self.d_out, self.E, self.k = T, d, d_out, E, k
        self.kind = L.FFN_KINDS[kind]
        self.d_ff = d_ff
        self.gate = L.GATE_MODES[gate]
        self.capacity = capacity
        self.n_shared = n_shared
        self.alpha = alpha
        self.act_dtype = act_dtype
        self.w = weights
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        A = T * k
        self.topk_idx = torch.empty((T, k), **i32)
        self.topk_gate = torch.empty((T, k), **f32)
        self.prob_colsum = torch.empty((E,), **f32)
        self.counts_routed = torch.empty((E,), **i32)
        self.counts_kept = torch.empty((E,), **i32)
        self.offsets = torch.empty((E + 1,), **i32)
        self.dest_pos = torch.empty((T, k), **i32)
        self.perm_token = torch.empty((max(A, 1),), **i32)
        # gather_rows: the routed FFN reads x through perm_token (no packed copy)
        # fp8_act: the experts run on e4m3 activations (x quantised per row,
        # read through perm_token; e4m3 weights required)
        self.fp8_act = fp8_act
        if fp8_act:
            if weights.get("s1") is None or act_dtype != torch.bfloat16:
                raise ValueError("fp8 activations need e4m3 expert weights and bf16 x")
            gather_rows = True
            self.xq = torch.empty((T, d), dtype=torch.uint8, device=dev)
            self.xs = torch.empty((max(T, 1),), dtype=torch.float32, device=dev)
            self.ws_f8 = self._ws(L.ffn_fp8_workspace_size(self.kind, A, E, d_ff), dev)
        self.gather_rows = gather_rows
        self._x_src = None
        self.x_perm = None if gather_rows else torch.empty((max(A, 1), d), dtype=act_dtype, device=dev)
        self.y_rows = torch.empty((max(A, 1), d_out), dtype=act_dtype, device=dev)
        self.y = torch.empty((T, d_out), dtype=act_dtype, device=dev)
        self.loss = torch.empty((1,), **f32)
        # training: the router keeps its fp32 logits for the backward pass
        self.logits = None
        # training with the expert FFNs' pre-activations kept: buffers, and
        # whether the last forward filled them (routed, shared)
        self._keep = None
        self._kept = None
        act = L.F32 if act_dtype == torch.float32 else L.BF16
        self.ws_router = self._ws(L.router_workspace_size(T, d, E, act), dev)
        self._router_ws = (self.ws_router, False)   # the workspace aux() reads (noisy or not)
        self.ws_disp = self._ws(L.dispatch_workspace_size(T, k, E), dev)
        self.ws_ffn = self._ws(L.ffn_workspace_size(self.kind, act, A, E, d, d_ff, d_out), dev)
        if n_shared:
            self.shared_y = torch.empty((n_shared, T, d_out), dtype=act_dtype, device=dev)
            self.sh_offsets = torch.arange(0, (n_shared + 1) * T, T, **i32)
            self.ws_sh = self._ws(L.ffn_workspace_size(self.kind, act, n_shared * T, n_shared, d, d_ff, d_out), dev)
            if fp8_act:
                self.ws_sh_f8 = self._ws(L.ffn_fp8_workspace_size(self.kind, n_shared * T, n_shared, d_ff), dev)
        else:
            self.shared_y = None

    @staticmethod
    def _ws(n: int, dev) -> torch.Tensor:
        return torch.zeros((max(int(n), 256),), dtype=torch.uint8, device=dev)

    # individual stages (the tests drive them one at a time) ----------------
    def router(self, x, with_colsum=False):
        """Router; its per-block probability column sums stay in the workspace
        for aux() (one launch fewer), unless with_colsum asks the router to
        reduce them into prob_colsum itself."""
        L.router_topk(x, self.w["w_g"], self.w.get("b_g"), self.k, self.gate, self.topk_idx, self.topk_gate,
                      self.prob_colsum if with_colsum else None, self.logits, self.ws_router)
        self._router_ws = (self.ws_router, False)

    def router_noisy(self, x, w_n, b_n, noise, eps=1e-2, with_colsum=False, seed=None, offset=0):
        """Training-mode router with noisy gating: the same outputs as router(),
        from logits with noise[t, e] * (softplus(x W_n^T + b_n) + eps) added.
        noise: the [T, E] normal draws, or None with ``seed`` given: draw
        t E + e of the counter-based stream (seed, offset), drawn in the
        router's kernels."""
        if getattr(self, "ws_router_noisy", None) is None:
            act = L.F32 if self.act_dtype == torch.float32 else L.BF16
            self.ws_router_noisy = self._ws(L.router_noisy_workspace_size(self.T, self.d, self.E, act), x.device)
        colsum = self.prob_colsum if with_colsum else None
        if noise is None:
            if seed is None:
                raise ValueError("router_noisy needs the draws (noise) or a seed for the counter-based stream")
            L.router_topk_noisy_philox(x, self.w["w_g"], self.w.get("b_g"), w_n, b_n, seed, offset, eps, self.k,
                                       self.gate, self.topk_idx, self.topk_gate, colsum, None, self.ws_router_noisy)
        else:
            L.router_topk_noisy(x, self.w["w_g"], self.w.get("b_g"), w_n, b_n, noise, eps, self.k, self.gate,
                                self.topk_idx, self.topk_gate, colsum, None, self.ws_router_noisy)
        self._router_ws = (self.ws_router_noisy, True)

    def dispatch(self, x, topk_idx=None):
        if self.gather_rows:
            self._x_src = x
        L.dispatch_permute(self.topk_idx if topk_idx is None else topk_idx, self.E, self.capacity,
                           None if self.gather_rows else x, self.x_perm,
                           self.counts_routed, self.counts_kept, self.offsets, self.dest_pos, self.perm_token,
                           self.ws_disp)

    def quantize(self, x):
        """fp8 activations: x quantised per row (codes and scales)."""
        if self.fp8_act:
            L.quantize_rows_e4m3(x, self.xq, self.xs)

    def experts(self, x_perm=None, offsets=None):
        w = self.w
        if self._keep is not None:
            self._kept["routed"] = False
        if self.fp8_act:
            L.expert_ffn_fp8(self.kind, self.xq, self.xs, self.perm_token, L.ROWS_PACKED, self.T * self.k,
                             self.offsets if offsets is None else offsets, self.E, self.d, self.d_ff, self.d_out,
                             w["w1"], w.get("w3"), w.get("w2"), w.get("s1"), w.get("s3"), w.get("s2"), self.y_rows,
                             self.ws_f8)
            return
        if self.gather_rows and x_perm is None:
            L.expert_ffn_gathered(self.kind, self._x_src, self.perm_token, self.T * self.k,
                                  self.offsets if offsets is None else offsets, self.E, self.d, self.d_ff, self.d_out,
                                  w["w1"], w.get("w3"), w.get("w2"), w.get("s1"), w.get("s3"), w.get("s2"),
                                  w.get("b1"), w.get("b2"), self.y_rows, self.ws_ffn)
            return
        xr = self.x_perm if x_perm is None else x_perm
        offs = self.offsets if offsets is None else offsets
        if self._keep is not None:
            # training: the first product's fp32 pre-activations are kept for
            # the backward pass where the library takes the shape
            h1, h3 = self._keep["routed"]
            self._kept["routed"] = L.expert_ffn_grouped_train(
                self.kind, xr, self.T * self.k, L.ROWS_PACKED, offs, self.E, self.d, self.d_ff, self.d_out, w["w1"],
                w.get("w3"), w.get("w2"), w.get("b1"), w.get("b2"), self.y_rows, h1, h3, self.ws_ffn)
            if self._kept["routed"]:
                return
        L.expert_ffn_grouped(self.kind, xr, self.T * self.k, L.ROWS_PACKED, offs, self.E, self.d, self.d_ff,
                             self.d_out, w["w1"], w.get("w3"), w.get("w2"), w.get("s1"), w.get("s3"), w.get("s2"),
                             w.get("b1"), w.get("b2"), self.y_rows, self.ws_ffn)

    def shared(self, x):
        if not self.n_shared:
            return
        w = self.w
        if self._keep is not None:
            self._kept["shared"] = False
        if self.fp8_act:
            L.expert_ffn_fp8(self.kind, self.xq, self.xs, None, L.ROWS_SHARED, self.n_shared * self.T, self.sh_offsets,
                             self.n_shared, self.d, self.d_ff, self.d_out, w["sh_w1"], w.get("sh_w3"), w.get("sh_w2"),
                             w.get("sh_s1"), w.get("sh_s3"), w.get("sh_s2"), self.shared_y, self.ws_sh_f8)
            return
        if self._keep is not None:
            h1, h3 = self._keep["shared"]
            self._kept["shared"] = L.expert_ffn_grouped_train(
                self.kind, x, self.n_shared * self.T, L.ROWS_SHARED, self.sh_offsets, self.n_shared, self.d,
                self.d_ff, self.d_out, w["sh_w1"], w.get("sh_w3"), w.get("sh_w2"), w.get("sh_b1"), w.get("sh_b2"),
                self.shared_y, h1, h3, self.ws_sh)
            if self._kept["shared"]:
                return
        L.expert_ffn_grouped(self.kind, x, self.n_shared * self.T, L.ROWS_SHARED, self.sh_offsets, self.n_shared,
                             self.d, self.d_ff, self.d_out, w["sh_w1"], w.get("sh_w3"), w.get("sh_w2"),
                             w.get("sh_s1"), w.get("sh_s3"), w.get("sh_s2"), w.get("sh_b1"), w.get("sh_b2"),
                             self.shared_y, self.ws_sh)

    def combine(self, residual=None, y_rows=None, dest_pos=None, topk_gate=None, shared_y=None):
        L.combine(self.y_rows if y_rows is None else y_rows, self.dest_pos if dest_pos is None else dest_pos,
                  self.topk_gate if topk_gate is None else topk_gate, self.d_out,
                  self.shared_y if shared_y is None else shared_y, self.n_shared, residual, self.y)

    def aux(self):
        """Balance loss and prob_colsum from the last router call's workspace
        (moe_aux_loss_from_router: one launch for both)."""
        ws, noisy = self._router_ws
        act = L.F32 if self.act_dtype == torch.float32 else L.BF16
        L.aux_loss_from_router(self.counts_routed, ws, self.T, self.d, self.E, act, noisy, self.k, self.alpha,
                               self.loss, self.prob_colsum)

    # ---------------------------------------------------------------- training
    def enable_backward(self, keep_pre=True):
        """Allocate what the backward pass needs (the forward then also keeps
        the router logits and, with keep_pre, the expert FFNs' fp32
        pre-activations, so that the backward does not recompute the first
        product); gradients land in self.grad after backward()."""
        if self.logits is not None:
            return
        if self.gather_rows:
            # the backward reads the packed rows the dispatch copied
            raise ValueError("the backward pass needs the packed rows: build the layer with gather_rows=False "
                             "and bf16 (not e4m3) expert weights")
        dev = self.topk_idx.device
        T, d, E, k, A = self.T, self.d, self.E, self.k, self.T * self.k
        f32 = dict(dtype=torch.float32, device=dev)
        act = self.act_dtype
        self.logits = torch.empty((T, E), **f32)
        self.dgate = torch.empty((T, k), **f32)
        self.dz = torch.empty((T, E), **f32)
        self.dy_rows = torch.empty((max(A, 1), self.d_out), dtype=act, device=dev)
        self.dx_rows = torch.empty((max(A, 1), d), dtype=act, device=dev)
        self.dx = torch.empty((T, d), dtype=act, device=dev)
        self.ws_rbwd = self._ws(L.router_backward_workspace_size(T, d, E), dev)
        keep = (keep_pre and self.kind != L.FFN_LINEAR and act == torch.bfloat16 and not self.fp8_act
                and self.w["w1"].dtype == torch.bfloat16)
        if keep:
            def pre(rows):
                h1 = torch.empty((max(rows, 1), self.d_ff), **f32)
                return h1, (torch.empty_like(h1) if self.kind == L.FFN_SWIGLU else None)
            self._keep = {"routed": pre(A), "shared": pre(self.n_shared * T) if self.n_shared else None}
            self._kept = {"routed": False, "shared": False}
            wsz = L.ffn_backward_kept_workspace_size
        else:
            wsz = L.ffn_backward_workspace_size
        # the recomputing backward's larger workspace is made only if a
        # forward could not keep the pre-activations
        self.ws_fbwd = self._ws(wsz(self.kind, A, E, d, self.d_ff, self.d_out), dev)
        g = {"w_g": torch.empty((E, d), **f32), "b_g": torch.empty((E,), **f32)}
        for pre in ("", "sh_"):
            for n in ("w1", "w3", "w2", "b1", "b2"):
                t = self.w.get(pre + n)
                if t is not None:
                    g[pre + n] = torch.empty(t.shape, **f32)
        self.grad = g
        if self.n_shared:
            self.dx_shared = torch.empty((self.n_shared, T, d), dtype=act, device=dev)
            self.ws_sbwd = self._ws(wsz(self.kind, self.n_shared * T, self.n_shared, d, self.d_ff, self.d_out), dev)

    def backward_combine(self, dy):
        L.combine_backward(dy, self.y_rows, self.dest_pos, self.topk_gate, self.dy_rows, self.dgate)

    def _bwd_ws(self, name, rows, E):
        """The workspace of the recomputing FFN backward (made on first use
        when the layer was set up to keep the pre-activations)."""
        ws = getattr(self, name)
        need = L.ffn_backward_workspace_size(self.kind, rows, E, self.d, self.d_ff, self.d_out)
        if ws.numel() < need:
            ws = self._ws(need, ws.device)
            setattr(self, name, ws)
        return ws

    def backward_experts(self):
        w, g = self.w, self.grad
        A = self.T * self.k
        if self._keep is not None and self._kept["routed"]:
            h1, h3 = self._keep["routed"]
            L.expert_ffn_grouped_backward_kept(self.kind, self.x_perm, A, L.ROWS_PACKED, self.offsets, self.E, self.d,
                                               self.d_ff, self.d_out, w["w1"], w.get("w3"), w.get("w2"), w.get("b1"),
                                               w.get("b2"), h1, h3, self.dy_rows, self.dx_rows, g["w1"], g.get("w3"),
                                               g.get("w2"), g.get("b1"), g.get("b2"), self.ws_fbwd)
            return
        L.expert_ffn_grouped_backward(self.kind, self.x_perm, A, L.ROWS_PACKED, self.offsets, self.E,
                                      self.d, self.d_ff, self.d_out, w["w1"], w.get("w3"), w.get("w2"), w.get("b1"),
                                      w.get("b2"), self.dy_rows, self.dx_rows, g["w1"], g.get("w3"), g.get("w2"),
                                      g.get("b1"), g.get("b2"), self._bwd_ws("ws_fbwd", A, self.E))

    def backward_shared(self, x, dy):
        if not self.n_shared:
            return
        w, g = self.w, self.grad
        R = self.n_shared * self.T
        if self._keep is not None and self._kept["shared"]:
            h1, h3 = self._keep["shared"]
            L.expert_ffn_grouped_backward_kept(self.kind, x, R, L.ROWS_SHARED, self.sh_offsets, self.n_shared, self.d,
                                               self.d_ff, self.d_out, w["sh_w1"], w.get("sh_w3"), w.get("sh_w2"),
                                               w.get("sh_b1"), w.get("sh_b2"), h1, h3, dy, self.dx_shared,
                                               g["sh_w1"], g.get("sh_w3"), g.get("sh_w2"), g.get("sh_b1"),
                                               g.get("sh_b2"), self.ws_sbwd)
            return
        L.expert_ffn_grouped_backward(self.kind, x, R, L.ROWS_SHARED, self.sh_offsets,
                                      self.n_shared, self.d, self.d_ff, self.d_out, w["sh_w1"], w.get("sh_w3"),
                                      w.get("sh_w2"), w.get("sh_b1"), w.get("sh_b2"), dy, self.dx_shared, g["sh_w1"],
                                      g.get("sh_w3"), g.get("sh_w2"), g.get("sh_b1"), g.get("sh_b2"),
                                      self._bwd_ws("ws_sbwd", R, self.n_shared))

    def backward_router(self, x, daux=1.0):
        L.router_backward(x, self.logits, self.topk_idx, self.topk_gate, self.dgate, self.counts_routed, self.gate,
                          self.alpha, daux, self.dz, self.grad["w_g"], self.grad["b_g"], self.ws_rbwd)

    def backward_permute(self, dy=None, residual=False):
        L.permute_backward(self.dx_rows, self.dest_pos, self.d, self.dx_shared if self.n_shared else None,
                           self.n_shared, dy if residual else None, self.dz, self.w["w_g"], self.dx)

    def backward(self, x, dy, daux=1.0, residual=False):
        """Gradients of <dy, y> + daux * aux for the last forward(x) (which
        must have run after enable_backward()); returns dx, fills self.grad.
        The gradient of b_g is kept whether or not the router has a bias."""
        self.backward_combine(dy)
        self.backward_experts()
        self.backward_shared(x, dy)
        self.backward_router(x, daux)
        self.backward_permute(dy, residual)
        return self.dx

    def forward(self, x, residual=None):
        """Whole layer; returns (y, aux loss tensor).  Asynchronous."""
        self.router(x)
        self.dispatch(x)
        self.quantize(x)
        self.experts()
        self.shared(x)
        self.combine(residual)
        self.aux()
        return self.y, self.loss
