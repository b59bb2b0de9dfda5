"""GPU parity of the fp8-activation expert path (moe_quantize_rows_e4m3,
moe_expert_ffn_fp8, MoELayer(fp8_act=True)) against the oracle's per-row
e4m3 quantisation and fp8 expert (oracle.quantize_rows_e4m3,
oracle.expert_ffn_fp8).

  * quantiser: codes and scales bit for bit (the rounding decision is taken
    in fp32 on both sides, from the same bf16 or fp32 values);
  * FFN, stage by stage, each stage fed the GPU's own upstream values (the
    workspace layout is documented in moe.h), element by element within a
    rigorous bound: the matrix cores cut each product toward zero to 13 bits
    below the largest product of its aligned group of 8 k (7 2^-13 max|a|
    max|w| per group at most) and add the groups with fp32 precision ((K + 5)
    2^-24 sum|terms| in any order), the activations' hardware exp2/rcp and
    the erfc polynomial add a relative 2^-20 (and 2^-21 |u| for GELU), and
    the bf16 store adds half a bf16 step of the value (the group cut is
    pinned by test_e4m3_products_cut_per_group_of_8 on exact probes).  Each
    stage is also held to 2e-2 row-normwise.  Stages: the first product and the
    activation (the bf16 hidden layer H) on the GPU's x codes and scales; the
    hidden layer's codes and scales bit for bit against the oracle's quantiser
    of the GPU's H; the second product on the GPU's hidden codes and scales;
  * FFN end to end against the oracle's fp8 expert on the GPU's x codes: the
    GPU's H and the oracle's (float64, rounded to bf16) differ within the
    bound above, and where that difference straddles an e4m3 rounding
    midpoint the two hidden codes differ, both correct for their H (as for
    near-tied router logits).  Every row is held to the second product's
    bound plus what the hidden-code differences carry through the second
    matrix (|dequant difference| @ |w2|^T); rows whose hidden codes agree are
    also held to 2e-2 row-normwise;
  * combine on the GPU's routing and expert rows (2e-2).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_harness import act_to_f64, rownorm_err, say
from sparse_mixture_experts_atomic_amd import MoELayer
from sparse_mixture_experts_atomic_amd import _lib as L
from workloads.device import layer_kwargs, to_tensor

pytestmark = pytest.mark.gpu
TOL = 2e-2
U = 2.0 ** -24


def _sum_bound(a, w):
    """bound on the error of the e4m3 product a @ w^T as the matrix cores form
    it.  Inside each aligned group of 8 consecutive k the products are cut
    toward zero to a multiple of 2^(E - 13), E the exponent of the group's
    largest |product| (measured on gfx950 with exactly representable probes:
    a product 2^-12 beside +-2^2 vanishes, beside +-2^1 it stays; (1 + m/8)
    2^-3 beside 2^8 becomes a multiple of 2^-5, either sign), so a group is
    off by less than 7 2^-13 max|a_k| max|w_k|; the group sums are then added
    with fp32 precision, (K + 5) 2^-24 sum|terms| for any order (the 5 covers
    the two scale multiplies and the 16-wide pairing of groups)."""
    K = a.shape[1]
    assert K % 8 == 0
    ga = np.abs(a).reshape(a.shape[0], K // 8, 8).max(axis=2)
    gw = np.abs(w).reshape(w.shape[0], K // 8, 8).max(axis=2)
    return 7 * 2.0 ** -13 * (ga @ gw.T) + (K + 5) * U * (np.abs(a) @ np.abs(w).T)


def _ratio(got, exact, bound):
    """max over elements of |got - exact| / (bound + half a bf16 step of a
    value of magnitude |exact| + bound)"""
    got = np.asarray(got, np.float64).reshape(exact.shape)
    if got.size == 0:
        return 0.0
    mag = np.maximum(np.abs(exact) + bound, np.finfo(np.float32).tiny)
    half = np.ldexp(1.0, np.floor(np.log2(mag)).astype(np.int64) - 8)
    return float(np.max(np.abs(got - exact) / (bound + half)))


def _quant_gpu(x):
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((max(rows, 1),), dtype=torch.float32, device="cuda")
    L.quantize_rows_e4m3(x, q, s)
    torch.cuda.synchronize()
    return q, s[:rows]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("cols", [264, 4104, 16392])
def test_row_quantiser_is_bit_exact(dtype, cols):
    """the row held in registers (up to 4096 or 16384 values per row for
    fp32 or bf16) and the two-pass kernel beyond"""
    say(f"[case] e4m3 row quantiser {dtype} cols={cols}")
    rng = np.random.default_rng(71)
    rows = 333 if cols < 1000 else 40
    x = rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-12, 12, (rows, 1)))
    x[5] = 0.0                                   # an all-zero row: scale 1, codes 0
    x[6] = -0.0
    x[7] = 3.25                                  # a constant row: every code 448
    x[8, ::2] = -x[8, ::2]
    x[9] = np.ldexp(1.0, -130)                   # fp32 subnormal input
    xt = torch.from_numpy(x.astype(np.float32)).to("cuda").to(dtype)
    q, s = _quant_gpu(xt)
    vals = act_to_f64(xt)
    q_ref, s_ref = O.quantize_rows_e4m3(vals)
    assert np.array_equal(s.cpu().numpy(), s_ref), "scales differ"
    got = q.cpu().numpy()
    bad = np.argwhere(got != q_ref)
    assert len(bad) == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}: " \
                          f"{[(int(got[r, c]), int(q_ref[r, c]), vals[r, c]) for r, c in bad[:5]]}"
    say(f"quantiser {dtype}: {rows} x {cols} codes and scales bit-exact")


def _e4m3(a, m=0, neg=False):
    """the e4m3 code of (1 + m/8) 2^a, a in [-6, 8]"""
    assert -6 <= a <= 8 and 0 <= m < 8 and not (a == 8 and m == 7)
    return ((a + 7) << 3) | m | (0x80 if neg else 0)


def _cut_model(x, w):
    """x @ w^T with each product cut toward zero to a multiple of 2^(E - 13),
    E = floor(log2) of the largest |product| of its aligned group of 8, and
    exact sums (the probes below keep every sum exact in fp32)"""
    P = x[:, None, :] * w[None, :, :]
    R, N, K = P.shape
    G = P.reshape(R, N, K // 8, 8)
    mx = np.abs(G).max(axis=3, keepdims=True)
    E = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
    unit = np.ldexp(1.0, (E - 13).astype(np.int64))
    return (np.trunc(G / unit) * unit).sum(axis=(2, 3))


def test_e4m3_products_cut_per_group_of_8():
    """The e4m3 matrix-core product on exactly representable probes (linear
    kind, one expert, unit scales): a cancelling pair +-2^j beside small
    products in the same group of 8 k, beside them in other groups, across
    instructions, and a product (1 + m/8) 2^e beside +-2^8 with either sign.
    The GPU must match the group-cut model bit for bit; plain fp32 sums
    would differ from it in the first two families."""
    say("[case] e4m3 product group cut")
    K, N = 256, 64
    rows_x, rows_w = [], np.zeros((N, K), np.uint8)
    # weights: column c has +-2^(c-6) at k = 0, 1 (c < 15), 2^-6 at k = 2..7
    # and 8..15, 2^0 at k = 20, +2^4 at k = 64 / -2^4 at k = 65 (col 15..16)
    for c in range(15):
        rows_w[c, 0], rows_w[c, 1] = _e4m3(c - 6), _e4m3(c - 6, neg=True)
    rows_w[:15, 2:16] = _e4m3(-6)
    rows_w[15, 16], rows_w[15, 64], rows_w[15, 20] = _e4m3(4), _e4m3(4, neg=True), _e4m3(0)
    rows_w[16, 16], rows_w[16, 64], rows_w[16, 20] = _e4m3(4, neg=True), _e4m3(4), _e4m3(0, neg=True)
    for a in range(-6, 9):                       # pair +-2^(a + c - 6) beside 2^-12 products
        r = np.zeros(K, np.uint8)
        r[0] = r[1] = _e4m3(a)
        r[2:8] = _e4m3(-6)
        r[8:16] = _e4m3(-6) if a % 2 else 0
        rows_x.append(r)
    for e in (-5, -4, -3, -2):                   # 2^8 at k=16, (1+m/8)2^e at k=20, -2^8 at k=64
        for m in range(0, 8, 3):
            r = np.zeros(K, np.uint8)
            r[16] = r[64] = _e4m3(4)
            r[20] = _e4m3(e, m)
            rows_x.append(r)
    X = np.stack(rows_x)
    R = X.shape[0]
    assert X.shape == (R, K) and rows_w.shape == (N, K) and R <= 64
    dev = "cuda"
    xq = torch.from_numpy(X).to(dev)
    xs = torch.ones(R, dtype=torch.float32, device=dev)
    w1 = torch.from_numpy(rows_w).to(dev)
    s1 = torch.ones(N, dtype=torch.float32, device=dev)
    off = torch.tensor([0, R], dtype=torch.int32, device=dev)
    y = torch.zeros((R, N), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(L.ffn_fp8_workspace_size(L.FFN_LINEAR, R, 1, 0), 256), dtype=torch.uint8, device=dev)
    L.expert_ffn_fp8(L.FFN_LINEAR, xq, xs, None, 0, R, off, 1, K, 0, N, w1, None, None, s1, None, None, y, ws)
    torch.cuda.synchronize()
    got = act_to_f64(y)
    xv = O.dequantize_rows_e4m3(X, np.ones(R))
    wv = O.dequantize_rows_e4m3(rows_w, np.ones(N))
    model = _cut_model(xv, wv)
    assert np.array_equal(O.bf16_round(model), model), "probe sums must be exact in bf16"
    exact = xv @ wv.T
    bad = np.argwhere(got != model)
    assert len(bad) == 0, f"{len(bad)} outputs differ from the group-cut model, first " \
                          f"{[(int(r), int(c), got[r, c], model[r, c], exact[r, c]) for r, c in bad[:5]]}"
    say(f"group cut: {R} x {N} probe outputs match the model bit for bit; "
        f"{int((model != exact).sum())} of them differ from the exact sum")


def _cfg(name, **kw):
    base = dict(d_out=0, cf=None, act_dtype="bf16", w_dtype="fp8", alpha=1e-2)
    base.update(kw)
    if not base["d_out"]:
        base["d_out"] = base["d"]
    return W.MoEConfig(name=name, **base)


CASES = {
    # stress-shaped: many experts, top-8, a shared expert, capacity drops
    "stress_s": W.shrink(W.STRESS, T=1000, d=256, d_ff=256, E=32, k=8),
    # ragged segments of a few hundred rows, ReLU / GELU / linear experts
    "relu": _cfg("f8_relu", T=700, d=384, E=6, k=2, ffn="relu", d_ff=256, gate="renorm",
                 wg_dist=("normal", 1 / 384), w1_var=1 / 384, w2_var=1 / 256, seed=72),
    "gelu_shared": _cfg("f8_gelu", T=500, d=256, E=5, k=2, ffn="gelu", d_ff=384, gate="prob", n_shared=2,
                        wg_dist=("normal", 1 / 256), w1_var=1 / 256, w2_var=1 / 384, seed=73),
    "linear": _cfg("f8_linear", T=300, d=256, d_out=200, E=4, k=2, ffn="linear", d_ff=0, gate="prob",
                   wg_dist=("normal", 1 / 256), w1_var=1 / 256, seed=74),
    # empty experts and one-row segments
    "sparse": _cfg("f8_sparse", T=40, d=128, E=64, k=1, ffn="swiglu", d_ff=128, gate="prob",
                   wg_dist=("normal", 1 / 128), w1_var=1 / 128, w3_var=1 / 128, w2_var=1 / 128, seed=75),
}


class F8Run:
    def __init__(self, cfg):
        self.cfg = cfg
        self.arr = W.generate(cfg)
        self.C = L.capacity(cfg.T, cfg.k, cfg.E, cfg.cf, cfg.cap_round)
        self.layer = MoELayer(**layer_kwargs(cfg, self.arr, self.C, "cuda"), fp8_act=True)
        self.x = to_tensor(self.arr["x"], "cuda")
        self.w = {}

    def expert(self, e, shared=False):
        key = (e, shared)
        if key not in self.w:
            if len(self.w) > 8:
                self.w.clear()
            pre = "sh_" if shared else ""
            sub = {n: (None if self.arr.get(pre + n) is None else self.arr[pre + n][e:e + 1])
                   for n in ("w1", "s1", "w3", "s3", "w2", "s2")}
            self.w[key] = {k: v[0] for k, v in O.decode_weights(sub, "fp8").items()}
        return self.w[key]

    def ffn_ref(self, e, codes, scales, shared=False):
        w = self.expert(e, shared)
        return O.expert_ffn_fp8(self.cfg.ffn, codes, scales, w["w1"], w.get("w3"), w.get("w2"))

    def run(self):
        ly = self.layer
        ly.forward(self.x)
        torch.cuda.synchronize()
        self.xq = ly.xq.cpu().numpy()
        self.xs = ly.xs[:self.cfg.T].cpu().numpy()
        self.off = ly.offsets.cpu().numpy().astype(np.int64)
        self.perm = ly.perm_token[:max(int(self.off[-1]), 1)].cpu().numpy().astype(np.int64)
        q_ref, s_ref = O.quantize_rows_e4m3(act_to_f64(self.x))
        assert np.array_equal(self.xq, q_ref) and np.array_equal(self.xs, s_ref), "layer x codes differ"

    def _hidden(self, ws, max_rows):
        """The hidden layer the GPU formed: H (bf16), its codes and row
        scales, at the workspace offsets moe.h documents."""
        cfg = self.cfg
        al = lambda n: (n + 255) // 256 * 256  # noqa: E731
        o_h = al((cfg.E if ws is self.layer.ws_f8 else cfg.n_shared) * 4 + 4)
        ff = max_rows * cfg.d_ff
        H = ws[o_h:o_h + 2 * ff].view(torch.bfloat16).view(max_rows, cfg.d_ff)
        o_q = o_h + al(2 * ff)
        Hq = ws[o_q:o_q + ff].view(max_rows, cfg.d_ff)
        o_s = o_q + al(ff)
        sh = ws[o_s:o_s + 4 * max_rows].view(torch.float32)
        return H, Hq, sh

    def _segment(self, e, rows_src, y_gpu, H, Hq, sh, shared=False):
        """bound ratios (err / bound, must stay <= 1) of one segment's stages
        and end to end, its 2e-2 row-normwise error on rows whose hidden codes
        agree with the oracle's; returns (ratios, errs, n_rows, n_rows_differing)"""
        cfg = self.cfg
        w = self.expert(e, shared)
        xh = O.dequantize_rows_e4m3(self.xq[rows_src], self.xs[rows_src])
        g = xh @ w["w1"].T
        dg = _sum_bound(xh, w["w1"])
        if cfg.ffn == "linear":
            return {"y": _ratio(y_gpu, g, dg)}, {"y": rownorm_err(y_gpu, g)}, len(rows_src), 0
        if cfg.ffn == "relu":
            h, dh = np.maximum(g, 0.0), dg
        elif cfg.ffn == "gelu":
            h = O.gelu(g)
            dh = 1.13 * dg + 2.0 ** -21 * (np.abs(g) + dg) + 2.0 ** -20 * np.abs(h)
        else:
            u = xh @ w["w3"].T
            du = _sum_bound(xh, w["w3"])
            sg = O.silu(g)
            ds = 1.1 * dg + 2.0 ** -20 * (np.abs(sg) + 1.1 * dg)
            h = sg * u
            dh = ds * (np.abs(u) + du) + np.abs(sg) * du + 2.0 ** -20 * np.abs(h)
        Hg = act_to_f64(H)
        ratios = {"H": _ratio(Hg, h, dh)}
        errs = {"H": rownorm_err(Hg, h)}
        q_ref, s_ref = O.quantize_rows_e4m3(Hg)
        Hqg, shg = Hq.cpu().numpy(), sh.cpu().numpy()
        assert np.array_equal(q_ref, Hqg) and np.array_equal(s_ref, shg), f"{cfg.name}: hidden codes differ ({e})"
        hg = O.dequantize_rows_e4m3(Hqg, shg)
        y_down = hg @ w["w2"].T
        dy = _sum_bound(hg, w["w2"])
        ratios["down"] = _ratio(y_gpu, y_down, dy)
        errs["down"] = rownorm_err(y_gpu, y_down)
        qo, so = O.quantize_rows_e4m3(O.bf16_round(h))
        ref = O.expert_ffn_fp8(cfg.ffn, self.xq[rows_src], self.xs[rows_src], w["w1"], w.get("w3"), w.get("w2"))
        carried = np.abs(hg - O.dequantize_rows_e4m3(qo, so)) @ np.abs(w["w2"]).T
        ratios["e2e"] = _ratio(y_gpu, ref, dy + carried)
        differ = np.any(qo != Hqg, axis=1) | (so != shg)
        errs["e2e"] = rownorm_err(y_gpu[~differ], ref[~differ]) if (~differ).any() else 0.0
        return ratios, errs, len(rows_src), int(differ.sum())

    def check_ffn(self, experts=None, shared_rows=None):
        cfg, ly = self.cfg, self.layer
        worst_r, worst_e, rows, differ = {}, {}, 0, 0

        def fold(ratios, errs, n, d):
            nonlocal rows, differ
            for k_, v in ratios.items():
                worst_r[k_] = max(worst_r.get(k_, 0.0), v)
            for k_, v in errs.items():
                worst_e[k_] = max(worst_e.get(k_, 0.0), v)
            rows += n
            differ += d

        H, Hq, sh = self._hidden(ly.ws_f8, cfg.T * cfg.k)
        for e in (range(cfg.E) if experts is None else experts):
            a, b = int(self.off[e]), int(self.off[e + 1])
            if b > a:
                fold(*self._segment(e, self.perm[a:b], act_to_f64(ly.y_rows[a:b]), H[a:b], Hq[a:b], sh[a:b]))
        if cfg.n_shared:
            Hs, Hqs, shs = self._hidden(ly.ws_sh_f8, cfg.n_shared * cfg.T)
            rr = np.arange(cfg.T) if shared_rows is None else shared_rows
            for s_ in range(cfg.n_shared):
                o = s_ * cfg.T + rr
                fold(*self._segment(s_, rr, act_to_f64(ly.shared_y[s_][rr]), Hs[o], Hqs[o], shs[o], shared=True))
        for k_, v in worst_r.items():
            assert v <= 1.0, f"{cfg.name}: fp8 FFN {k_} outside its bound (ratio {v:.3f})"
        for k_, v in worst_e.items():
            assert v <= TOL, f"{cfg.name}: fp8 FFN {k_} err {v:.3e}"
        say(f"fp8 ffn {cfg.name}: {rows} rows; error/bound " + " ".join(f"{k_} {v:.3f}" for k_, v in worst_r.items())
            + "; " + " ".join(f"{k_} {v:.2e}" for k_, v in worst_e.items()) +
            f" (rows with agreeing hidden codes); hidden codes bit-exact; {differ} rows whose hidden codes differ "
            "from the oracle's within the H bound")

    def check_layer(self):
        """combine on the GPU's routing, gates and expert rows"""
        cfg, ly = self.cfg, self.layer
        dest = ly.dest_pos.cpu().numpy()
        g = ly.topk_gate.cpu().numpy().astype(np.float64)
        A = int(self.off[-1])
        ye = act_to_f64(ly.y_rows[:max(A, 1)])[:A]
        ys = sum(act_to_f64(ly.shared_y[s_]) for s_ in range(cfg.n_shared)) if cfg.n_shared else None
        ref = O.combine(ye, dest, g, ys)
        err = rownorm_err(act_to_f64(ly.y), ref)
        assert err <= TOL, f"{cfg.name}: fp8 layer err {err:.3e}"
        say(f"fp8 layer {cfg.name}: {cfg.T} tokens err {err:.2e} (dropped slots {int((dest < 0).sum())})")


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_activation_layer(name):
    say(f"[case] fp8 activations {name}")
    r = F8Run(CASES[name])
    r.run()
    r.check_ffn()
    r.check_layer()


@pytest.mark.timeout(900)
def test_fp8_activation_stress_full():
    """The stress shape (32768 tokens, 256 + 1 experts, top-8, e4m3 weights,
    drops) with fp8 activations: 16 whole routed segments and the shared
    expert's first 2048 rows."""
    say("[case] fp8 activations full stress")
    r = F8Run(W.STRESS)
    r.run()
    rng = np.random.default_rng(76)
    nonempty = [e for e in range(r.cfg.E) if r.off[e + 1] > r.off[e]]
    experts = sorted(set([nonempty[0], nonempty[-1]] + rng.choice(nonempty, 14, replace=False).tolist()))
    r.check_ffn(experts=experts, shared_rows=np.arange(2048))
    r.check_layer()
