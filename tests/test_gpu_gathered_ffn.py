"""GPU parity of the grouped FFN that reads its rows through the dispatch
permutation (moe_expert_ffn_gathered): no packed copy of x.

P1 §2.4 gathers an expert's tokens into one batch before running it; here
the gather is the first matrix product's row addressing.  The same kernels
compute in the same order, so the gathered layer must equal the packed one
bit for bit (expert rows and layer output); sampled expert rows are also
compared with the oracle's FFN of x[perm_token] at the bf16/fp32 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_harness import act_to_f64, rownorm_err, say, tol_for
from sparse_mixture_experts_atomic_amd import MoELayer
from sparse_mixture_experts_atomic_amd import _lib as L
from workloads.device import layer_kwargs, to_tensor

pytestmark = pytest.mark.gpu


def _cfg(name, **kw):
    base = dict(d_out=0, cf=None, act_dtype="bf16", w_dtype="bf16", alpha=1e-2)
    base.update(kw)
    if not base["d_out"]:
        base["d_out"] = base["d"]
    return W.MoEConfig(name=name, **base)


CASES = {
    # LDS-DMA GEMM (K % 128 == 0), SwiGLU, ragged segments
    "mixtral_s": W.shrink(W.MIXTRAL, T=600, d=256, d_ff=448, E=8, k=2),
    # 64 experts with shared experts (those read x directly, not gathered)
    "deepseek_s": W.shrink(W.DEEPSEEK, T=500, d=256, d_ff=192, E=64, k=6),
    # register-staged GEMM (K off the 128-column grid), e4m3 weights, shared
    "fp8_shared": _cfg("fp8_shared", T=300, d=160, E=12, k=3, ffn="swiglu", d_ff=208, gate="prob", cf=1.0,
                       n_shared=2, w_dtype="fp8", wg_dist=("uniform", 1 / np.sqrt(160)),
                       w1_var=1 / 160, w3_var=1 / 160, w2_var=1 / 208, seed=26),
    # capacity drops: only kept rows are gathered
    "cap_hit_k4": _cfg("cap_hit_k4", T=513, d=128, E=8, k=4, ffn="swiglu", d_ff=136, gate="renorm", cf=0.6,
                       wg_dist=("normal", 1 / 128), bg_var=1.0, w1_var=1 / 128, w3_var=1 / 128,
                       w2_var=1 / 136, seed=25),
    # GELU with biases on the DMA GEMM (the from-scratch page's model, bf16)
    "p1_gelu_bf16": W.P1_GELU.scaled(name="p1_gelu_bf16", act_dtype="bf16", w_dtype="bf16", seed=42),
    # fp32 path
    "p1_gelu_f32": W.P1_GELU,
    # one token; one expert (every row in one segment)
    "t1": _cfg("t1", T=1, d=128, E=4, k=2, ffn="swiglu", d_ff=128, gate="renorm", wg_dist=("normal", 1 / 128),
               w1_var=1 / 128, w3_var=1 / 128, w2_var=1 / 128, seed=44),
    "e1": _cfg("e1", T=300, d=256, E=1, k=1, ffn="gelu", d_ff=256, gate="renorm", wg_dist=("normal", 1 / 256),
               w1_var=1 / 256, w2_var=1 / 256, b1_var=0.1, b2_var=0.1, seed=45),
    # Mixtral shape at full size
    "mixtral": W.MIXTRAL,
}


def _layers(cfg):
    arr = W.generate(cfg)
    C = L.capacity(cfg.T, cfg.k, cfg.E, cfg.cf, cfg.cap_round)
    assert C == O.capacity(cfg.T, cfg.k, cfg.E, cfg.cf, cfg.cap_round)
    kw = layer_kwargs(cfg, arr, C, "cuda")
    packed = MoELayer(**kw)
    gathered = MoELayer(**kw, gather_rows=True)
    return arr, packed, gathered


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", list(CASES))
def test_gathered_ffn_equals_packed_and_oracle(name):
    cfg = CASES[name]
    say(f"gathered ffn {name}: T={cfg.T} d={cfg.d} E={cfg.E}+{cfg.n_shared} k={cfg.k} {cfg.ffn} "
        f"x {cfg.act_dtype} w {cfg.w_dtype}")
    arr, packed, gathered = _layers(cfg)
    x = to_tensor(arr["x"], "cuda")
    y_p, loss_p = packed.forward(x)
    y_p, loss_p = y_p.clone(), loss_p.clone()
    y_g, loss_g = gathered.forward(x)
    torch.cuda.synchronize()
    assert gathered.x_perm is None
    n = int(packed.offsets[-1].item())
    assert torch.equal(packed.perm_token[:n], gathered.perm_token[:n])
    rows_p, rows_g = packed.y_rows[:n], gathered.y_rows[:n]
    if cfg.act_dtype == "bf16":
        assert torch.equal(rows_p.view(torch.int16), rows_g.view(torch.int16)), f"{name}: expert rows differ"
        assert torch.equal(y_p.view(torch.int16), y_g.view(torch.int16)), f"{name}: layer output differs"
    else:
        assert torch.equal(rows_p, rows_g) and torch.equal(y_p, y_g), f"{name}: outputs differ"
    assert torch.equal(loss_p, loss_g)

    # sampled packed rows against the oracle FFN of x[perm_token]
    offs = gathered.offsets.cpu().numpy().astype(np.int64)
    perm = gathered.perm_token[:n].cpu().numpy().astype(np.int64)
    rng = np.random.default_rng(0)
    x64 = O.to_f64(arr["x"], cfg.act_dtype)
    worst = 0.0
    for e in range(cfg.E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi <= lo:
            continue
        rows = np.unique(np.concatenate([rng.integers(lo, hi, size=min(8, hi - lo)), [lo, hi - 1]]))
        sub = {k_: (None if arr.get(k_) is None else arr[k_][e:e + 1]) for k_ in ("w1", "s1", "w3", "s3", "w2", "s2", "b1", "b2")}
        w = {k_: v[0] for k_, v in O.decode_weights(sub, cfg.w_dtype).items()}
        ref = O.expert_ffn(cfg.ffn, x64[perm[rows]], w["w1"], w.get("w3"), w.get("w2"), w.get("b1"), w.get("b2"))
        got = act_to_f64(gathered.y_rows[torch.from_numpy(rows).cuda()])
        worst = max(worst, rownorm_err(got, ref))
    assert worst <= tol_for(cfg), f"{name}: expert rows vs oracle {worst:.3e}"
    say(f"  {n} rows bit-identical to the packed path; sampled rows vs oracle {worst:.2e}")


@pytest.mark.timeout(300)
def test_gathered_ffn_beyond_32bit_row_offsets():
    """x of 2^30 + 8192 bf16 elements (> 2^31 bytes): the LDS-DMA kernel's
    32-bit row offsets cannot reach every source row, so the register-staged
    kernel gathers; rows near the end of x must come out right."""
    cfg = _cfg("gather_2g", T=131073, d=8192, d_out=16, E=2, k=1, ffn="linear", d_ff=0, gate="prob",
               wg_dist=("normal", 1 / 8192), w1_var=1 / 8192, seed=43)
    say(f"gathered ffn {cfg.name}: T={cfg.T} d={cfg.d} ({cfg.T * cfg.d * 2 / 2**30:.3f} GiB of x)")
    arr = W.generate(cfg)
    C = L.capacity(cfg.T, cfg.k, cfg.E, cfg.cf, cfg.cap_round)
    assert C == O.capacity(cfg.T, cfg.k, cfg.E, cfg.cf, cfg.cap_round)
    kw = layer_kwargs(cfg, arr, C, "cuda")
    g = MoELayer(**kw, gather_rows=True)
    x = to_tensor(arr["x"], "cuda")
    g.router(x)
    g.dispatch(x)
    g.experts()
    torch.cuda.synchronize()
    offs = g.offsets.cpu().numpy().astype(np.int64)
    perm = g.perm_token[:int(offs[-1])].cpu().numpy().astype(np.int64)
    x64 = None
    worst = 0.0
    for e in range(cfg.E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi <= lo:
            continue
        # the last packed rows of each segment come from the end of x
        rows = np.arange(max(lo, hi - 16), hi)
        src = perm[rows]
        xs = O.to_f64(arr["x"][src], cfg.act_dtype)
        w = O.decode_weights({"w1": arr["w1"][e:e + 1], "s1": None, "b1": None}, cfg.w_dtype)
        ref = O.expert_ffn("linear", xs, w["w1"][0])
        got = act_to_f64(g.y_rows[torch.from_numpy(rows).cuda()])
        worst = max(worst, rownorm_err(got, ref))
        assert src.max() > cfg.T - 4096
    assert worst <= tol_for(cfg), f"rows vs oracle {worst:.3e}"
    say(f"  last rows of each segment vs oracle {worst:.2e}")


def test_gathered_ffn_with_capacity_zero_reads_no_rows():
    """Capacity 0: no packed row exists, perm_token is never written, and the
    gathered FFN must not read it; the layer output is 0."""
    cfg = _cfg("cap0", T=200, d=128, E=4, k=2, ffn="swiglu", d_ff=128, gate="renorm", cf=1e-9,
               wg_dist=("normal", 1 / 128), w1_var=1 / 128, w3_var=1 / 128, w2_var=1 / 128, seed=46)
    say("gathered ffn cap0: capacity 0, every assignment dropped")
    arr = W.generate(cfg)
    kw = layer_kwargs(cfg, arr, 0, "cuda")
    g = MoELayer(**kw, gather_rows=True)
    g.perm_token.fill_(0)                # a valid row: a wrong read would show as written rows
    g.y_rows.fill_(7.0)
    x = to_tensor(arr["x"], "cuda")
    y, _ = g.forward(x)
    torch.cuda.synchronize()
    assert int(g.offsets[-1].item()) == 0
    assert torch.all(g.y_rows.float() == 7.0)       # untouched
    assert torch.all(y.float() == 0.0)
