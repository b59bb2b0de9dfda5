"""Stage-by-stage parity of the GPU layer against the CPU oracle.

Protocol (each stage is fed the GPU's own upstream outputs, so a near-tie in
the router cannot cascade):
  router   top-k ids bit-exact on tokens whose top-(k+1) logits have no gap
           below 1e-5 (elsewhere the GPU's choice must be a valid top-k);
           gates and probability column sums within 1e-5 relative.
  dispatch every integer output bit-exact, recomputed by the oracle from the
           GPU's top-k ids; packed rows byte-identical to x[perm_token].
  ffn      packed outputs vs the oracle FFN of the GPU's packed rows.
  combine  vs the oracle combine of the GPU's expert outputs and gates.
  e2e      vs the oracle run from scratch, on tokens without near-ties.
  aux      vs the oracle aux loss of the GPU's counts and column sums.
Float tolerance: row-normwise relative error (max over rows of the inf-norm
of the difference over the inf-norm of the reference, with a floor of 1e-6
times the largest reference row norm): 1e-5 for fp32 outputs, 2e-2 for bf16.
"""
from __future__ import annotations

import sys
from typing import Dict, Optional

import numpy as np
import torch

import oracle as O
import workloads as W
from sparse_mixture_experts_atomic_amd import MoELayer
from sparse_mixture_experts_atomic_amd import _lib as L
from workloads.device import layer_kwargs, to_tensor

GAP = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rownorm_err(y: np.ndarray, r: np.ndarray) -> float:
    if y.size == 0:
        return 0.0
    y = np.asarray(y, np.float64).reshape(r.shape)
    num = np.max(np.abs(y - r), axis=1)
    den = np.max(np.abs(r), axis=1)
    floor = 1e-6 * max(float(den.max()), 1e-300)
    return float(np.max(num / np.maximum(den, floor)))


def rel_err(a, b, floor_frac=1e-6) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if b.size == 0:
        return 0.0
    floor = max(floor_frac * float(np.max(np.abs(b))), 1e-300)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), floor)))


def tol_for(cfg) -> float:
    return 1e-5 if cfg.act_dtype == "f32" else 2e-2


def act_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare_router(name, z, k, gate_mode, idx_g, gate_g, colsum_g):
    """GPU router outputs against the oracle's logits z (float64 [T, E]).

    Top-k ids bit-exact on tokens without a near-tie; everywhere a valid
    top-k set in descending order; gates and column sums within 1e-5
    relative.  Returns the near-tie mask and the two errors."""
    T, E = z.shape
    p = O.softmax(z)
    idx_o = O.topk_select(z, k)
    tie = O.near_tie_mask(z, k, GAP)
    ok = ~tie
    mism = int(np.sum(np.any(idx_g[ok] != idx_o[ok], axis=1)))
    assert mism == 0, f"{name}: {mism} untied tokens differ in top-k ids"
    # validity everywhere (near-tied tokens may pick another valid set)
    assert np.all((idx_g >= 0) & (idx_g < E))
    srt = np.sort(idx_g, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1]) if k > 1 else True
    if T:
        sel = np.take_along_axis(z, idx_g.astype(np.int64), axis=1)
        kth = -np.sort(-z, axis=1)[:, k - 1]
        assert np.all(sel >= kth[:, None] - GAP)
        assert np.all(np.diff(sel, axis=1) <= GAP)
    g_ref = O.gates(p, idx_g, gate_mode)
    eg = rel_err(gate_g, g_ref, floor_frac=1e-30)
    assert eg <= 1e-5, f"{name}: gate rel err {eg:.3e}"
    ec = rel_err(colsum_g, p.sum(axis=0))
    assert ec <= 1e-5, f"{name}: prob_colsum rel err {ec:.3e}"
    return tie, eg, ec


class Run:
    """One workload uploaded to the GPU with its oracle-side float64 views."""

    def __init__(self, cfg: W.MoEConfig, arrays: Optional[Dict] = None, device: str = "cuda"):
        self.cfg = cfg
        self.arr = arrays if arrays is not None else W.generate(cfg)
        # the layer runs with the library's own capacity; the oracle's must agree
        self.C = L.capacity(cfg.T, cfg.k, cfg.E, cfg.cf, cfg.cap_round)
        assert self.C == O.capacity(cfg.T, cfg.k, cfg.E, cfg.cf, cfg.cap_round), cfg.name
        self.layer = MoELayer(**layer_kwargs(cfg, self.arr, self.C, device))
        self.x = to_tensor(self.arr["x"], device)
        self.x64 = O.to_f64(self.arr["x"], cfg.act_dtype)
        self.w_g = self.arr["w_g"].astype(np.float64)
        self.b_g = None if self.arr["b_g"] is None else self.arr["b_g"].astype(np.float64)
        self._z = None
        self._wcache = {}
        self._wbytes = 0

    # -- oracle pieces --------------------------------------------------------
    @property
    def z(self):
        if self._z is None:
            self._z = O.router_logits(self.x64, self.w_g, self.b_g)
        return self._z

    # float64 weights of the experts decoded so far, up to this many bytes
    # (one Mixtral-shaped expert is 1.4 GB in float64)
    WCACHE_BYTES = 3 << 30

    def expert_w(self, e: int, shared: bool = False):
        key = (e, shared)
        if key not in self._wcache:
            pre = "sh_" if shared else ""
            sub = {}
            for n in ("w1", "s1", "w3", "s3", "w2", "s2", "b1", "b2"):
                a = self.arr.get(pre + n)
                sub[n] = None if a is None else a[e:e + 1]
            w = {k: v[0] for k, v in O.decode_weights(sub, self.cfg.w_dtype).items()}
            nbytes = sum(v.nbytes for v in w.values())
            while self._wcache and self._wbytes + nbytes > self.WCACHE_BYTES:
                old = next(iter(self._wcache))
                self._wbytes -= sum(v.nbytes for v in self._wcache.pop(old).values())
            self._wcache[key] = w
            self._wbytes += nbytes
        return self._wcache[key]

    def ffn64(self, e: int, rows: np.ndarray, shared: bool = False) -> np.ndarray:
        w = self.expert_w(e, shared)
        return O.expert_ffn(self.cfg.ffn, rows, w["w1"], w.get("w3"), w.get("w2"), w.get("b1"), w.get("b2"))

    # -- stages ---------------------------------------------------------------
    def check_router(self):
        cfg = self.cfg
        self.layer.router(self.x, with_colsum=True)
        torch.cuda.synchronize()
        idx_g = self.layer.topk_idx.cpu().numpy()
        gate_g = self.layer.topk_gate.cpu().numpy().astype(np.float64)
        colsum_g = self.layer.prob_colsum.cpu().numpy().astype(np.float64)
        tie, eg, ec = compare_router(cfg.name, self.z, cfg.k, cfg.gate, idx_g, gate_g, colsum_g)
        self.idx_g, self.gate_g, self.colsum_g, self.tie = idx_g, gate_g, colsum_g, tie
        say(f"router {cfg.name}: T={cfg.T} E={cfg.E} k={cfg.k} near-tied {int(tie.sum())} "
            f"gate err {eg:.2e} colsum err {ec:.2e}")
        return idx_g

    def check_dispatch(self, row_sample: Optional[int] = None, seed: int = 0):
        cfg = self.cfg
        self.layer.dispatch(self.x)
        torch.cuda.synchronize()
        ref = O.dispatch(self.idx_g, cfg.E, self.C)
        ly = self.layer
        got = {"counts_routed": ly.counts_routed, "counts_kept": ly.counts_kept, "offsets": ly.offsets,
               "dest_pos": ly.dest_pos}
        for k, t in got.items():
            a = t.cpu().numpy()
            assert np.array_equal(a, ref[k]), f"{cfg.name}: dispatch {k} differs"
        A = int(ref["offsets"][-1])
        perm = ly.perm_token[:A].cpu().numpy()
        assert np.array_equal(perm, ref["perm_token"]), f"{cfg.name}: perm_token differs"
        # packed rows are exact copies: every row (or a sample), compared as
        # bytes on the host in chunks of about 256 MB
        rows = np.arange(A) if row_sample is None or row_sample >= A else \
            np.unique(np.concatenate([np.random.default_rng(seed).choice(A, row_sample, replace=False),
                                      ref["offsets"][:-1][ref["counts_kept"] > 0], [A - 1]]))
        x_host = self.x.cpu()
        x_host = x_host.view(torch.int16) if x_host.dtype == torch.bfloat16 else x_host.view(torch.int32)
        step = max(1, (256 << 20) // max(1, x_host.shape[1] * x_host.element_size()))
        for c0 in range(0, len(rows), step):
            rc = rows[c0:c0 + step]
            xp = ly.x_perm[torch.from_numpy(rc).to(ly.x_perm.device)].cpu()
            xp = xp.view(torch.int16) if xp.dtype == torch.bfloat16 else xp.view(torch.int32)
            src = x_host[torch.from_numpy(perm[rc].astype(np.int64))]
            assert torch.equal(xp, src), f"{cfg.name}: x_perm bytes differ in rows {rc[0]}..{rc[-1]}"
        self.xp_rows_checked = len(rows)
        self.disp = ref
        dropped = int((ref["dest_pos"] < 0).sum())
        say(f"dispatch {cfg.name}: kept {A} dropped {dropped} C={self.C} loads "
            f"{int(ref['counts_routed'].min())}..{int(ref['counts_routed'].max())}; "
            f"{len(rows)} packed rows byte-compared")
        return ref

    def _segment_rows(self, max_experts: Optional[int], rows_per_expert: Optional[int], seed: int):
        off = self.disp["offsets"]
        E = self.cfg.E
        nonempty = [e for e in range(E) if off[e + 1] > off[e]]
        rng = np.random.default_rng(seed)
        if max_experts is not None and len(nonempty) > max_experts:
            pick = set([nonempty[0], nonempty[-1]])
            pick.update(rng.choice(nonempty, max_experts - 2, replace=False).tolist())
            experts = sorted(pick)
        else:
            experts = nonempty
        out = {}
        for e in experts:
            a, b = int(off[e]), int(off[e + 1])
            if rows_per_expert is None or b - a <= rows_per_expert:
                out[e] = np.arange(a, b)
            else:
                r = set([a, a + 1, b - 2, b - 1])
                # the start of the last (possibly partial) 128-row tile
                r.add(a + ((b - a - 1) // 128) * 128)
                r.update(rng.integers(a, b, rows_per_expert - len(r)).tolist())
                out[e] = np.array(sorted(r))
        return out

    def check_ffn(self, max_experts=None, rows_per_expert=None, seed=1):
        cfg = self.cfg
        self.layer.experts()
        torch.cuda.synchronize()
        segs = self._segment_rows(max_experts, rows_per_expert, seed)
        worst = 0.0
        n = 0
        for i, (e, rows) in enumerate(segs.items()):
            ridx = torch.from_numpy(rows).to(self.layer.y_rows.device)
            xp = act_to_f64(self.layer.x_perm[ridx])
            yg = act_to_f64(self.layer.y_rows[ridx])
            ref = self.ffn64(e, xp)
            worst = max(worst, rownorm_err(yg, ref))
            n += len(rows)
            if i % 16 == 15:
                say(f"  ffn {cfg.name}: {i + 1}/{len(segs)} experts, {n} rows so far, err {worst:.2e}")
        assert worst <= tol_for(cfg), f"{cfg.name}: expert FFN err {worst:.3e}"
        whole = sum(1 for e, r in segs.items() if len(r) == self.disp["offsets"][e + 1] - self.disp["offsets"][e])
        say(f"ffn {cfg.name}: {len(segs)} experts ({whole} whole segments) {n} of "
            f"{int(self.disp['offsets'][-1])} rows err {worst:.2e}")
        return worst

    def check_shared(self, rows: Optional[np.ndarray] = None):
        cfg = self.cfg
        if not cfg.n_shared:
            return 0.0
        self.layer.shared(self.x)
        torch.cuda.synchronize()
        rows = np.arange(cfg.T) if rows is None else rows
        worst = 0.0
        for s in range(cfg.n_shared):
            ridx = torch.from_numpy(rows).to(self.x.device)
            yg = act_to_f64(self.layer.shared_y[s][ridx])
            ref = self.ffn64(s, self.x64[rows], shared=True)
            worst = max(worst, rownorm_err(yg, ref))
        assert worst <= tol_for(cfg), f"{cfg.name}: shared FFN err {worst:.3e}"
        say(f"shared {cfg.name}: {cfg.n_shared} experts {len(rows)} rows err {worst:.2e}")
        return worst

    def check_combine(self, tokens: Optional[np.ndarray] = None, residual: bool = False, chunk: int = 4096):
        cfg = self.cfg
        res = self.x if residual else None
        self.layer.combine(res)
        torch.cuda.synchronize()
        tokens = np.arange(cfg.T) if tokens is None else tokens
        worst, alldrop = 0.0, 0
        for c0 in range(0, max(len(tokens), 1), chunk):
            e, a = self._combine_chunk(tokens[c0:c0 + chunk], residual)
            worst, alldrop = max(worst, e), alldrop + a
        assert worst <= tol_for(cfg), f"{cfg.name}: combine err {worst:.3e}"
        say(f"combine {cfg.name}: {len(tokens)} of {cfg.T} tokens err {worst:.2e} all-dropped {alldrop}")
        return worst

    def _combine_chunk(self, tokens: np.ndarray, residual: bool):
        cfg = self.cfg
        dest = self.disp["dest_pos"][tokens]
        used = np.unique(dest[dest >= 0])
        remap = np.full(max(int(self.disp["offsets"][-1]), 1), -1, dtype=np.int64)
        remap[used] = np.arange(len(used))
        dest_sub = np.where(dest >= 0, remap[np.maximum(dest, 0)], -1)
        dev = self.layer.y_rows.device
        ye = act_to_f64(self.layer.y_rows[torch.from_numpy(used).to(dev)]) if len(used) else \
            np.zeros((0, cfg.d_out))
        tk = torch.from_numpy(tokens).to(dev)
        ys = None
        if cfg.n_shared:
            ys = sum(act_to_f64(self.layer.shared_y[s][tk]) for s in range(cfg.n_shared))
        r = self.x64[tokens] if residual else None
        ref = O.combine(ye, dest_sub, self.gate_g[tokens], ys, r)
        yg = act_to_f64(self.layer.y[tk])
        err = rownorm_err(yg, ref)
        # a token with every slot dropped and no shared expert is exactly 0 (or x)
        alldrop = np.all(dest < 0, axis=1)
        if not cfg.n_shared and alldrop.any():
            want = self.x64[tokens][alldrop] if residual else 0.0
            assert np.all(yg[alldrop] == want), f"{cfg.name}: dropped tokens not exact"
        return err, int(alldrop.sum())

    def check_aux(self):
        cfg = self.cfg
        self.layer.aux()
        torch.cuda.synchronize()
        got = float(self.layer.loss.item())
        # the column sums the fused aux call forms from the router's workspace
        # are the router's own, bit for bit
        assert np.array_equal(self.layer.prob_colsum.cpu().numpy().astype(np.float64), self.colsum_g), \
            f"{cfg.name}: prob_colsum from moe_aux_loss_from_router differs from the router's"
        ref = O.aux_loss(self.disp["counts_routed"], self.colsum_g, cfg.T, cfg.k, cfg.E, cfg.alpha)
        assert abs(got - ref) <= 1e-5 * max(abs(ref), 1e-30), f"{cfg.name}: aux {got} vs {ref}"
        # and from scratch (counts from the oracle's own routing)
        p = O.softmax(self.z)
        ref2 = O.aux_loss(O.dispatch(O.topk_select(self.z, cfg.k), cfg.E, self.C)["counts_routed"],
                          p.sum(axis=0), cfg.T, cfg.k, cfg.E, cfg.alpha)
        if not self.tie.any():
            assert abs(got - ref2) <= 1e-5 * max(abs(ref2), 1e-30)
        say(f"aux {cfg.name}: {got:.7f} (oracle {ref:.7f})")
        return got

    def check_e2e(self, tokens: Optional[np.ndarray] = None):
        """y vs the oracle from scratch (its own routing and dispatch)."""
        cfg = self.cfg
        z = self.z
        p = O.softmax(z)
        idx = O.topk_select(z, cfg.k)
        g = O.gates(p, idx, cfg.gate)
        disp = O.dispatch(idx, cfg.E, self.C)
        T = cfg.T
        tokens = np.arange(T) if tokens is None else tokens
        keep_o = disp["dest_pos"][tokens] >= 0
        keep_g = self.disp["dest_pos"][tokens] >= 0
        good = ~self.tie[tokens] & np.all(keep_o == keep_g, axis=1)
        toks = tokens[good]
        ref = np.zeros((len(toks), cfg.d_out))
        by_e = {}
        for i, t in enumerate(toks):
            for j in range(cfg.k):
                if disp["dest_pos"][t, j] >= 0:
                    by_e.setdefault(int(idx[t, j]), []).append((i, t, j))
        for n_done, (e, lst) in enumerate(sorted(by_e.items())):
            ii = np.array([i for i, _, _ in lst], dtype=np.int64)
            tt = np.array([t for _, t, _ in lst], dtype=np.int64)
            jj = np.array([j for _, _, j in lst], dtype=np.int64)
            out = self.ffn64(e, self.x64[tt])
            np.add.at(ref, ii, g[tt, jj][:, None] * out)
            if n_done % 32 == 31:
                say(f"  e2e {cfg.name}: {n_done + 1}/{len(by_e)} experts")
        for s in range(cfg.n_shared):
            ref += self.ffn64(s, self.x64[toks], shared=True)
        yg = act_to_f64(self.layer.y[torch.from_numpy(toks).to(self.layer.y.device)])
        err = rownorm_err(yg, ref)
        assert err <= tol_for(cfg), f"{cfg.name}: end-to-end err {err:.3e}"
        assert good.mean() >= 0.98, f"{cfg.name}: too many tokens excluded ({(~good).sum()})"
        say(f"e2e {cfg.name}: {len(toks)} of {len(tokens)} tokens err {err:.2e} excluded {int((~good).sum())} "
            f"(near-tied or dropped differently)")
        return err

    def run_all(self, ffn_experts=None, ffn_rows=None, tokens=None, e2e_tokens=None, row_sample=None,
                residual=False):
        self.check_router()
        self.check_dispatch(row_sample=row_sample)
        self.check_ffn(ffn_experts, ffn_rows)
        self.check_shared(None if tokens is None else tokens)
        self.check_combine(tokens, residual=residual)
        self.check_aux()
        self.check_e2e(e2e_tokens if e2e_tokens is not None else tokens)
