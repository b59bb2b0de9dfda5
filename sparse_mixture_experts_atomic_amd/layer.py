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
                 weights: Dict[str, Optional[torch.Tensor]], device="cuda", gather_rows: bool = False):
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
        self.gather_rows = gather_rows
        self._x_src = None
        self.x_perm = None if gather_rows else torch.empty((max(A, 1), d), dtype=act_dtype, device=dev)
        self.y_rows = torch.empty((max(A, 1), d_out), dtype=act_dtype, device=dev)
        self.y = torch.empty((T, d_out), dtype=act_dtype, device=dev)
        self.loss = torch.empty((1,), **f32)
        act = L.F32 if act_dtype == torch.float32 else L.BF16
        self.ws_router = self._ws(L.router_workspace_size(T, d, E, act), dev)
        self.ws_disp = self._ws(L.dispatch_workspace_size(T, k, E), dev)
        self.ws_ffn = self._ws(L.ffn_workspace_size(self.kind, act, A, E, d, d_ff, d_out), dev)
        if n_shared:
            self.shared_y = torch.empty((n_shared, T, d_out), dtype=act_dtype, device=dev)
            self.sh_offsets = torch.arange(0, (n_shared + 1) * T, T, **i32)
            self.ws_sh = self._ws(L.ffn_workspace_size(self.kind, act, n_shared * T, n_shared, d, d_ff, d_out), dev)
        else:
            self.shared_y = None

    @staticmethod
    def _ws(n: int, dev) -> torch.Tensor:
        return torch.zeros((max(int(n), 256),), dtype=torch.uint8, device=dev)

    # individual stages (the tests drive them one at a time) ----------------
    def router(self, x):
        L.router_topk(x, self.w["w_g"], self.w.get("b_g"), self.k, self.gate, self.topk_idx, self.topk_gate,
                      self.prob_colsum, None, self.ws_router)

    def router_noisy(self, x, w_n, b_n, noise, eps=1e-2):
        """Training-mode router with noisy gating: the same outputs as router(),
        from logits with noise[t, e] * (softplus(x W_n^T + b_n) + eps) added."""
        if getattr(self, "ws_router_noisy", None) is None:
            act = L.F32 if self.act_dtype == torch.float32 else L.BF16
            self.ws_router_noisy = self._ws(L.router_noisy_workspace_size(self.T, self.d, self.E, act), x.device)
        L.router_topk_noisy(x, self.w["w_g"], self.w.get("b_g"), w_n, b_n, noise, eps, self.k, self.gate,
                            self.topk_idx, self.topk_gate, self.prob_colsum, None, self.ws_router_noisy)

    def dispatch(self, x, topk_idx=None):
        if self.gather_rows:
            self._x_src = x
        L.dispatch_permute(self.topk_idx if topk_idx is None else topk_idx, self.E, self.capacity,
                           None if self.gather_rows else x, self.x_perm,
                           self.counts_routed, self.counts_kept, self.offsets, self.dest_pos, self.perm_token,
                           self.ws_disp)

    def experts(self, x_perm=None, offsets=None):
        w = self.w
        if self.gather_rows and x_perm is None:
            L.expert_ffn_gathered(self.kind, self._x_src, self.perm_token, self.T * self.k,
                                  self.offsets if offsets is None else offsets, self.E, self.d, self.d_ff, self.d_out,
                                  w["w1"], w.get("w3"), w.get("w2"), w.get("s1"), w.get("s3"), w.get("s2"),
                                  w.get("b1"), w.get("b2"), self.y_rows, self.ws_ffn)
            return
        L.expert_ffn_grouped(self.kind, self.x_perm if x_perm is None else x_perm, self.T * self.k, L.ROWS_PACKED,
                             self.offsets if offsets is None else offsets, self.E, self.d, self.d_ff, self.d_out,
                             w["w1"], w.get("w3"), w.get("w2"), w.get("s1"), w.get("s3"), w.get("s2"),
                             w.get("b1"), w.get("b2"), self.y_rows, self.ws_ffn)

    def shared(self, x):
        if not self.n_shared:
            return
        w = self.w
        L.expert_ffn_grouped(self.kind, x, self.n_shared * self.T, L.ROWS_SHARED, self.sh_offsets, self.n_shared,
                             self.d, self.d_ff, self.d_out, w["sh_w1"], w.get("sh_w3"), w.get("sh_w2"),
                             w.get("sh_s1"), w.get("sh_s3"), w.get("sh_s2"), w.get("sh_b1"), w.get("sh_b2"),
                             self.shared_y, self.ws_sh)

    def combine(self, residual=None, y_rows=None, dest_pos=None, topk_gate=None, shared_y=None):
        L.combine(self.y_rows if y_rows is None else y_rows, self.dest_pos if dest_pos is None else dest_pos,
                  self.topk_gate if topk_gate is None else topk_gate, self.d_out,
                  self.shared_y if shared_y is None else shared_y, self.n_shared, residual, self.y)

    def aux(self):
        L.aux_loss(self.counts_routed, self.prob_colsum, self.T, self.k, self.E, self.alpha, self.loss)

    def forward(self, x, residual=None):
        """Whole layer; returns (y, aux loss tensor).  Asynchronous."""
        self.router(x)
        self.dispatch(x)
        self.experts()
        self.shared(x)
        self.combine(residual)
        self.aux()
        return self.y, self.loss
