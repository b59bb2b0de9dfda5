"""GPU parity: every stage of the HIP path against the CPU oracle.

Small shapes run the full oracle on every row (several tiles and ragged
tails); the five workloads run at their full sizes with the oracle on
sampled rows/tokens where the full float64 computation would take minutes.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_harness import Run, act_to_f64, rownorm_err, say
from sparse_mixture_experts_atomic_amd import MoELayer
from sparse_mixture_experts_atomic_amd import _lib as L
from workloads.device import to_tensor

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")

# small versions of the five workloads (same structure and distributions)
SMALL = {
    "tiny": W.TINY,
    "switch_s": W.shrink(W.SWITCH, T=700, d=256, d_ff=384, E=8, k=1),
    "switch_drop_s": W.shrink(W.SWITCH_DROP, T=700, d=256, d_ff=384, E=8, k=1),
    "mixtral_s": W.shrink(W.MIXTRAL, T=600, d=256, d_ff=448, E=8, k=2),
    "deepseek_s": W.shrink(W.DEEPSEEK, T=500, d=256, d_ff=192, E=64, k=6),
    "stress_s": W.shrink(W.STRESS, T=1000, d=256, d_ff=128, E=32, k=8),
}

_base = dict(d_out=0, cf=None, act_dtype="bf16", w_dtype="bf16", alpha=1e-2)


def _cfg(name, **kw):
    d = dict(_base)
    d.update(kw)
    if not d["d_out"]:
        d["d_out"] = d["d"]
    return W.MoEConfig(name=name, **d)


EDGE = {
    # one expert, top-1: a plain FFN on every token
    "e1_k1": _cfg("e1_k1", T=130, d=64, E=1, k=1, ffn="swiglu", d_ff=96, gate="renorm",
                  wg_dist=("normal", 1 / 64), w1_var=1 / 64, w3_var=1 / 64, w2_var=1 / 96, seed=21),
    # three experts (not a power of two), k = E, ReLU with biases
    "e3_k3_relu_bias": _cfg("e3_k3_relu_bias", T=257, d=128, E=3, k=3, ffn="relu", d_ff=200, gate="renorm",
                            wg_dist=("normal", 1 / 128), w1_var=1 / 128, w2_var=1 / 200, b1_var=0.1,
                            b2_var=0.1, seed=22),
    # linear experts, widths off the 64/128 tile grid (K and N tails)
    "linear_tails": _cfg("linear_tails", T=333, d=72, d_out=40, E=5, k=2, ffn="linear", d_ff=0,
                         gate="prob", wg_dist=("normal", 1 / 72), w1_var=1 / 72, b1_var=0.1, seed=23),
    # many experts, few tokens: empty segments
    "empty_experts": _cfg("empty_experts", T=40, d=64, E=64, k=1, ffn="swiglu", d_ff=64, gate="prob",
                          wg_dist=("normal", 1 / 64), w1_var=1 / 64, w3_var=1 / 64, w2_var=1 / 64, seed=24),
    # capacity hit hard, k=4
    "cap_hit_k4": _cfg("cap_hit_k4", T=513, d=128, E=8, k=4, ffn="swiglu", d_ff=136, gate="renorm", cf=0.6,
                       wg_dist=("normal", 1 / 128), bg_var=1.0, w1_var=1 / 128, w3_var=1 / 128,
                       w2_var=1 / 136, seed=25),
    # fp8 weights with shared experts and an off-tile hidden width
    "fp8_shared": _cfg("fp8_shared", T=300, d=160, E=12, k=3, ffn="swiglu", d_ff=208, gate="prob", cf=1.0,
                       n_shared=2, w_dtype="fp8", wg_dist=("uniform", 1 / np.sqrt(160)),
                       w1_var=1 / 160, w3_var=1 / 160, w2_var=1 / 208, seed=26),
    "fp8_relu": _cfg("fp8_relu", T=200, d=96, E=4, k=2, ffn="relu", d_ff=160, gate="renorm", w_dtype="fp8",
                     wg_dist=("normal", 1 / 96), w1_var=1 / 96, w2_var=1 / 160, seed=27),
    # fp32 end to end with a SwiGLU and shared experts
    "f32_swiglu_shared": _cfg("f32_swiglu_shared", T=90, d=24, E=6, k=2, ffn="swiglu", d_ff=40, gate="renorm",
                              n_shared=1, act_dtype="f32", w_dtype="f32", wg_dist=("normal", 1 / 24),
                              w1_var=1 / 24, w3_var=1 / 24, w2_var=1 / 40, seed=28),
    # tiled router GEMM: expert count off the 64-expert blocks, a partial
    # last 64-column chunk, a token count off the 64-token blocks, router bias
    "router_mfma_tails": _cfg("router_mfma_tails", T=77, d=72, E=20, k=3, ffn="swiglu", d_ff=64, gate="prob",
                              wg_dist=("normal", 1 / 72), bg_var=0.5, w1_var=1 / 72, w3_var=1 / 72,
                              w2_var=1 / 64, seed=33),
    # tiled router GEMM split over four K slices (the last one ends in a
    # partial chunk), two expert blocks (the second of 6 experts), bias
    "router_kslices": _cfg("router_kslices", T=300, d=1544, d_out=16, E=70, k=5, ffn="linear", d_ff=0,
                           gate="prob", wg_dist=("normal", 1 / 1544), bg_var=0.5, w1_var=1 / 1544, seed=39),
    # router at the largest expert count (four experts per lane slot)
    "router_e256": _cfg("router_e256", T=1100, d=256, E=256, k=8, ffn="linear", d_ff=0, gate="renorm",
                        wg_dist=("normal", 1 / 256), w1_var=1 / 256, seed=34),
    # e4m3 weights on the LDS-DMA GEMM (K % 128 == 0): ReLU with biases, and a
    # Linear layer whose output width is off the 256-column tiles
    "fp8_dma_relu_bias": _cfg("fp8_dma_relu_bias", T=300, d=256, E=6, k=2, ffn="relu", d_ff=384, gate="renorm",
                              w_dtype="fp8", wg_dist=("normal", 1 / 256), w1_var=1 / 256, w2_var=1 / 384,
                              b1_var=0.1, b2_var=0.1, seed=35),
    "fp8_dma_linear": _cfg("fp8_dma_linear", T=260, d=384, d_out=200, E=5, k=2, ffn="linear", d_ff=0, gate="prob",
                           w_dtype="fp8", wg_dist=("normal", 1 / 384), w1_var=1 / 384, seed=36),
    # GELU experts with biases: on the register-staged GEMM (K off the
    # 128-column grid, N off the tiles), on the LDS-DMA GEMM with e4m3
    # weights, and the from-scratch page's own model shape in bf16 (DMA GEMM)
    "gelu_bias_tails": _cfg("gelu_bias_tails", T=257, d=136, d_out=72, E=5, k=2, ffn="gelu", d_ff=200,
                            gate="renorm", wg_dist=("normal", 1 / 136), w1_var=1 / 136, w2_var=1 / 200,
                            b1_var=0.1, b2_var=0.1, seed=40),
    "fp8_dma_gelu_bias": _cfg("fp8_dma_gelu_bias", T=300, d=256, E=6, k=2, ffn="gelu", d_ff=384, gate="prob",
                              w_dtype="fp8", wg_dist=("normal", 1 / 256), w1_var=1 / 256, w2_var=1 / 384,
                              b1_var=0.1, b2_var=0.1, seed=41),
    "p1_gelu_bf16": W.P1_GELU.scaled(name="p1_gelu_bf16", act_dtype="bf16", w_dtype="bf16", seed=42),
    # E <= 8 MFMA router: rows wider than one round of chunks, with a last
    # chunk of 8 columns; seven experts, router bias
    "router_e8_wide": _cfg("router_e8_wide", T=300, d=4360, d_out=16, E=7, k=3, ffn="linear", d_ff=0,
                           gate="renorm", wg_dist=("normal", 1 / 4360), bg_var=0.5, w1_var=1 / 4360, seed=37),
    # E <= 8 MFMA router with several token groups per block (narrow rows,
    # long batch) and a ragged last block
    "router_e8_groups": _cfg("router_e8_groups", T=8200, d=64, d_out=16, E=8, k=2, ffn="linear", d_ff=0,
                             gate="prob", wg_dist=("normal", 1 / 64), w1_var=1 / 64, seed=38),
    "t1": _cfg("t1", T=1, d=64, E=4, k=2, ffn="swiglu", d_ff=64, gate="renorm", wg_dist=("normal", 1 / 64),
               w1_var=1 / 64, w3_var=1 / 64, w2_var=1 / 64, seed=29),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workloads_all_stages(name):
    say(f"[case] small workload {name}")
    Run(SMALL[name]).run_all()


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases_all_stages(name):
    say(f"[case] edge {name}")
    Run(EDGE[name]).run_all()


def test_residual_and_all_dropped_tokens():
    """Capacity 0 (rounding down a tiny factor): every slot drops, so y is
    exactly 0, and exactly x with the residual."""
    say("[case] capacity zero")
    cfg = _cfg("cap_zero", T=100, d=64, E=4, k=2, ffn="swiglu", d_ff=64, gate="renorm", cf=0.01,
               cap_round="floor", wg_dist=("normal", 1 / 64), w1_var=1 / 64, w3_var=1 / 64, w2_var=1 / 64, seed=30)
    r = Run(cfg)
    assert r.C == 0
    r.check_router()
    r.check_dispatch()
    r.check_ffn()
    r.check_combine(residual=False)
    r.check_combine(residual=True)
    r.check_aux()


def test_all_tokens_to_one_expert():
    say("[case] one hot expert")
    cfg = _cfg("one_hot", T=400, d=64, E=8, k=2, ffn="swiglu", d_ff=64, gate="prob",
               wg_dist=("normal", 1 / 64), w1_var=1 / 64, w3_var=1 / 64, w2_var=1 / 64, seed=31)
    arr = W.generate(cfg)
    arr["b_g"] = np.zeros(8, np.float32)
    arr["b_g"][5] = 40.0                       # expert 5 wins every token
    r = Run(cfg, arr)
    r.run_all()
    assert r.disp["counts_routed"][5] == cfg.T


def test_page_worked_example_on_gpu():
    """P4 一个小算例 through the HIP path: 3 linear experts with A=0 and
    b = 10, 20, 30, router logits [1, 2, 3], k = 3, renormalised gates."""
    say("[case] page worked example")
    ex = json.load(open(os.path.join(GOLD, "p4_worked_example.json"), encoding="utf-8"))
    cfg = _cfg("page_example", T=1, d=1, E=3, k=3, ffn="linear", d_ff=0, gate="renorm",
               act_dtype="f32", w_dtype="f32")
    arr = {"x": np.ones((1, 1), np.float32), "w_g": np.array(ex["logits"], np.float32).reshape(3, 1),
           "b_g": None, "w1": np.zeros((3, 1, 1), np.float32), "b1": np.array(ex["expert_outputs"], np.float32).reshape(3, 1)}
    r = Run(cfg, arr)
    y, loss = r.layer.forward(r.x)
    torch.cuda.synchronize()
    g = r.layer.topk_gate.cpu().numpy()[0].astype(np.float64)
    idx = r.layer.topk_idx.cpu().numpy()[0]
    assert idx.tolist() == [2, 1, 0]
    assert np.round(g[np.argsort(idx)], 2).tolist() == ex["gates_printed"]
    assert abs(float(y.item()) - ex["y_printed"]) < 0.05
    r.run_all()


def test_fp8_decode_every_code_exactly():
    """A linear fp8 expert applied to identity rows returns its decoded
    weights: every finite e4m3 code must decode exactly (bf16 holds them)."""
    say("[case] fp8 decode table")
    codes = np.arange(256, dtype=np.uint8).reshape(16, 16)        # W[n, c]
    codes = np.where((codes & 0x7F) == 0x7F, 0, codes).astype(np.uint8)   # drop the two NaN codes
    Kd = 16
    x = torch.eye(Kd, dtype=torch.bfloat16, device="cuda")          # 16 rows
    w1 = torch.from_numpy(codes.reshape(1, 16, 16)).cuda()
    s1 = torch.ones((1, 16), dtype=torch.float32, device="cuda")
    off = torch.tensor([0, Kd], dtype=torch.int32, device="cuda")
    y = torch.empty((Kd, 16), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(L.ffn_workspace_size(L.FFN_LINEAR, L.BF16, Kd, 1, Kd, 0, 16), dtype=torch.uint8, device="cuda")
    L.expert_ffn_grouped(L.FFN_LINEAR, x, Kd, L.ROWS_PACKED, off, 1, Kd, 0, 16, w1, None, None, s1, None, None,
                         None, None, y, ws)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy()            # got[a, n] = decode(codes[n, a])
    ref = O.e4m3_to_f64(codes).T
    assert np.array_equal(got.astype(np.float64), ref)


def test_zero_tokens_is_a_no_op():
    say("[case] T = 0")
    cfg = _cfg("t0", T=0, d=64, E=4, k=2, ffn="swiglu", d_ff=64, gate="renorm", wg_dist=("normal", 1 / 64),
               w1_var=1 / 64, w3_var=1 / 64, w2_var=1 / 64, seed=32)
    arr = W.generate(cfg)
    from workloads.device import layer_kwargs
    layer = MoELayer(**layer_kwargs(cfg, arr, -1))
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    y, loss = layer.forward(x)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)
    assert layer.offsets.cpu().tolist() == [0] * 5
    assert layer.prob_colsum.cpu().tolist() == [0.0] * 4
    assert float(loss.item()) == 0.0


def test_layer_is_deterministic():
    say("[case] determinism")
    cfg = SMALL["deepseek_s"]
    r = Run(cfg)
    outs = []
    for _ in range(2):
        y, loss = r.layer.forward(r.x)
        torch.cuda.synchronize()
        outs.append((y.clone(), r.layer.dest_pos.clone(), r.layer.prob_colsum.clone(), loss.clone()))
    a, b = outs
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2]) and torch.equal(a[3], b[3])


# ---------------------------------------------------------------- full sizes
# Switch, Mixtral and DeepSeekMoE: every packed row, every FFN row, every
# shared-expert row, every token through combine and end to end (the float64
# oracle takes seconds per expert).  Stress: every packed row and every token
# through combine, 16 whole routed segments, 4096 shared-expert rows and 512
# tokens end to end (decoding all 256 fp8 experts to float64 for the rest
# would take minutes).

@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["switch", "switch_drop"])
def test_switch_full(name):
    say(f"[case] full {name}")
    Run(W.CONFIGS[name]).run_all()


@pytest.mark.timeout(300)
def test_p1_gelu_full():
    """The from-scratch page's GELU model at its own size, fp32, full oracle."""
    say("[case] full p1_gelu")
    Run(W.P1_GELU).run_all()


@pytest.mark.timeout(300)
def test_switch_gelu_full():
    say("[case] full switch_gelu")
    Run(W.SWITCH_GELU).run_all()


@pytest.mark.timeout(400)
def test_mixtral_full():
    say("[case] full mixtral")
    Run(W.MIXTRAL).run_all()


@pytest.mark.timeout(400)
def test_deepseek_full():
    say("[case] full deepseek")
    r = Run(W.DEEPSEEK)
    r.run_all()
    share = np.isin(np.argmax(r.z, axis=1), np.argsort(-r.disp["counts_routed"])[:3]).mean()
    say(f"deepseek: share of tokens whose top-1 expert is among the 3 most loaded: {share:.3f}")


@pytest.mark.timeout(900)
def test_stress_full():
    say("[case] full stress (fp8)")
    r = Run(W.STRESS)
    rng = np.random.default_rng(5)
    toks = np.unique(np.concatenate([rng.choice(W.STRESS.T, 4094, replace=False), [0, W.STRESS.T - 1]]))
    r.check_router()
    r.check_dispatch()
    r.check_ffn(max_experts=16)
    r.check_shared(toks)
    r.check_combine()
    r.check_aux()
    e2e = np.unique(np.concatenate([rng.choice(W.STRESS.T, 510, replace=False), [0, W.STRESS.T - 1]]))
    r.check_e2e(e2e)
