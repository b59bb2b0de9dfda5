"""GPU parity of the noisy-gating router (moe_router_topk_noisy) against the
oracle's noisy_router on the same seeded inputs and normal draws.

Noisy logits: P2 §2.1 (Noisy Top-k 门控; no floor) and P5 代码实战
(NoisyTop1Gate in training mode: bias on the noise projection, floor 1e-2,
top-1 with the probability as its gate).  The comparison protocol is the
clean router's: ids bit-exact on tokens without a near-tie (gap 1e-5),
gates and probability column sums within 1e-5 relative; the returned noisy
logits within 1e-5 of the oracle's, relative to max(1, |z|) of the row.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_harness import compare_router, say
from sparse_mixture_experts_atomic_amd import _lib as L
from workloads.device import to_tensor

pytestmark = pytest.mark.gpu

# name -> (workload, noise floor eps, bias on the noise projection)
CASES = {
    # Mixtral-shaped router with P2's noisy top-2 (no floor, no bias)
    "mixtral_p2": (W.MIXTRAL, 0.0, False),
    # Switch-shaped top-1 router with P5's gate (bias, floor 1e-2)
    "switch_p5_top1": (W.SWITCH, 1e-2, True),
    # DeepSeekMoE-shaped router: 64 experts, top-6, router bias
    "deepseek": (W.DEEPSEEK, 1e-2, True),
    # stress-shaped router at full size: 256 experts, top-8, d = 7168 (the
    # tiled GEMM over 512 stacked rows, 128-token blocks)
    "stress": (W.STRESS, 1e-2, True),
    # fp32 activations (the generic kernel), the small workload
    "tiny_f32": (W.TINY, 1e-2, True),
    # fp32, two 64-expert groups with a ragged second one, ragged tokens
    "f32_ragged": (W.TINY.scaled(name="f32_ragged", T=333, d=40, d_out=40, E=70, k=5, seed=21), 0.0, True),
    # bf16: partial 64-column chunk, 2 E = 40 rows in one expert block
    "bf16_tails": (W.MIXTRAL.scaled(name="bf16_tails", T=77, d=72, d_out=72, E=20, k=3, gate="prob",
                                    wg_dist=("normal", 1.0 / 72), bg_var=0.5, seed=22), 1e-2, True),
    # bf16 at the largest expert count: 2 E = 512 rows in 8 expert blocks
    "bf16_e256": (W.MIXTRAL.scaled(name="bf16_e256", T=300, d=256, d_out=256, E=256, k=8, gate="renorm",
                                   wg_dist=("normal", 1.0 / 256), seed=23), 0.0, True),
    # bf16 split over K slices with a partial last chunk
    "bf16_kslices": (W.MIXTRAL.scaled(name="bf16_kslices", T=300, d=1544, d_out=1544, E=70, k=5, gate="prob",
                                      wg_dist=("normal", 1.0 / 1544), seed=24), 1e-2, False),
    # bf16, at most 8 experts (the single-launch MFMA router with a second
    # accumulator): seven experts, rows over several rounds of chunks with a
    # last chunk of 8 columns, router bias
    "bf16_e7_wide": (W.MIXTRAL.scaled(name="bf16_e7_wide", T=300, d=4360, d_out=16, E=7, k=3, gate="prob",
                                      wg_dist=("normal", 1.0 / 4360), bg_var=0.5, seed=26), 1e-2, True),
    # degenerate shapes: one token, one expert (the gate is 1 whatever the
    # noise); fp32 with k = E (every expert chosen, ids ordered by noisy logit)
    "bf16_t1_e1": (W.MIXTRAL.scaled(name="bf16_t1_e1", T=1, d=64, d_out=64, E=1, k=1, gate="renorm",
                                    wg_dist=("normal", 1.0 / 64), seed=27), 1e-2, True),
    "f32_k_eq_e": (W.TINY.scaled(name="f32_k_eq_e", T=50, d=24, d_out=24, E=5, k=5, gate="prob", seed=28), 0.0, True),
    # bf16, at most 8 experts, several token groups per block (narrow rows)
    "bf16_bm128": (W.MIXTRAL.scaled(name="bf16_bm128", T=8200, d=64, d_out=64, E=8, k=2,
                                    wg_dist=("normal", 1.0 / 64), seed=25), 1e-2, True),
}


def _run(x, w_g, b_g, w_n, b_n, noise, eps, k, gate, T, d, E, dt):
    dev = "cuda"
    t = lambda a: to_tensor(a, dev)
    idx = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    gte = torch.full((T, k), -7.0, dtype=torch.float32, device=dev)
    colsum = torch.full((E,), -7.0, dtype=torch.float32, device=dev)
    lg = torch.full((T, E), -7.0, dtype=torch.float32, device=dev)
    ws_bytes = max(L.router_noisy_workspace_size(T, d, E, dt), 256)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    L.router_topk_noisy(t(x), t(w_g), t(b_g), t(w_n), t(b_n), t(noise), eps, k, L.GATE_MODES[gate],
                        idx, gte, colsum, lg, ws)
    torch.cuda.synchronize()
    return (idx.cpu().numpy(), gte.cpu().numpy().astype(np.float64), colsum.cpu().numpy().astype(np.float64),
            lg.cpu().numpy().astype(np.float64))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", list(CASES))
def test_noisy_router_matches_oracle(name):
    cfg, eps, bias = CASES[name]
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    say(f"noisy router {name}: T={T} d={d} E={E} k={k} x {cfg.act_dtype} gate {cfg.gate} eps={eps} bias_n={bias}")
    x = W.gen_x(cfg)
    w_g, b_g = W.gen_router(cfg)
    w_n, b_n, noise = W.gen_noisy_gate(cfg, bias)
    dt = L.F32 if cfg.act_dtype == "f32" else L.BF16
    idx_g, gate_g, colsum_g, lg_g = _run(x, w_g, b_g, w_n, b_n, noise, eps, k, cfg.gate, T, d, E, dt)

    f64 = lambda a: None if a is None else a.astype(np.float64)
    z = O.noisy_router_logits(O.to_f64(x, cfg.act_dtype), f64(w_g), f64(b_g), f64(w_n), f64(b_n), f64(noise), eps)
    tie, eg, ec = compare_router(name, z, k, cfg.gate, idx_g, gate_g, colsum_g)
    zerr = float(np.max(np.abs(lg_g - z) / np.maximum(1.0, np.max(np.abs(z), axis=1, keepdims=True))))
    assert zerr <= 1e-5, f"{name}: noisy logit err {zerr:.3e}"
    # the noise decides: the clean router picks another set for many tokens
    clean = O.topk_select(O.router_logits(O.to_f64(x, cfg.act_dtype), f64(w_g), f64(b_g)), k)
    changed = int(np.sum(np.any(np.sort(clean, axis=1) != np.sort(idx_g, axis=1), axis=1)))
    if k < E and T > 1:
        assert changed > 0
    # same inputs, same draws: the same bits
    again = _run(x, w_g, b_g, w_n, b_n, noise, eps, k, cfg.gate, T, d, E, dt)
    for a, b in zip((idx_g, gate_g, colsum_g, lg_g), again):
        np.testing.assert_array_equal(a, b)
    say(f"  near-tied {int(tie.sum())}, tokens whose set the noise changed {changed}, "
        f"gate err {eg:.2e}, colsum err {ec:.2e}, logit err {zerr:.2e}")


def test_noisy_router_zero_tokens_writes_zero_column_sums():
    cfg = W.MIXTRAL.scaled(name="t0", T=0, d=64, d_out=64, E=8, k=2)
    say("noisy router T=0: only the column sums are written")
    dev = "cuda"
    w_g = torch.zeros((8, 64), dtype=torch.float32, device=dev)
    colsum = torch.full((8,), -7.0, dtype=torch.float32, device=dev)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    idx = torch.zeros((0, 2), dtype=torch.int32, device=dev)
    g = torch.zeros((0, 2), dtype=torch.float32, device=dev)
    noise = torch.zeros((0, 8), dtype=torch.float32, device=dev)
    L.router_topk_noisy(x, w_g, None, w_g, None, noise, 1e-2, cfg.k, L.GATE_RENORM, idx, g, colsum, None, ws)
    torch.cuda.synchronize()
    assert torch.all(colsum.cpu() == 0)


# ---- draws from the counter-based generator (moe_gate_noise_philox and
# moe_router_topk_noisy_philox) --------------------------------------------

from oracle import philox as OP    # noqa: E402


@pytest.mark.parametrize("seed,offset,n", [(0, 0, 1000003), (0x0123456789ABCDEF, 0xFEDCBA9876543210, 65537),
                                           (2 ** 64 - 1, 2 ** 64 - 1, 4099)])
def test_philox_draws_match_oracle(seed, offset, n):
    say(f"philox draws: seed {seed:#x} offset {offset:#x} n {n}")
    out = torch.full((n,), -7.0, dtype=torch.float32, device="cuda")
    L.gate_noise_philox(seed, offset, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = OP.philox_normals(seed, offset, n)
    # fp64 on both sides, rounded once to fp32 on the GPU: within one fp32
    # ulp of the oracle, and the same fp32 value unless the fp64 results sit
    # on either side of a rounding boundary
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= ulp), f"max err {np.max(err / ulp):.2f} ulp"
    differ = int(np.sum(got != ref.astype(np.float32).astype(np.float64)))
    assert differ <= max(2, n // 100000), differ
    say(f"  {differ} of {n} draws differ from the oracle's fp32 rounding (by one ulp)")


PHILOX_CASES = ["mixtral_p2", "switch_p5_top1", "deepseek", "stress", "tiny_f32", "f32_ragged", "bf16_e7_wide",
                "bf16_kslices", "bf16_t1_e1"]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", PHILOX_CASES)
def test_noisy_router_philox_matches_oracle(name):
    cfg, eps, bias = CASES[name]
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    seed, offset = 0x5EED0000 + cfg.seed, 3 * cfg.seed + 1
    say(f"noisy router, drawn on the device {name}: T={T} d={d} E={E} k={k} seed {seed:#x} offset {offset}")
    dev = "cuda"
    x = W.gen_x(cfg)
    w_g, b_g = W.gen_router(cfg)
    w_n, b_n, _ = W.gen_noisy_gate(cfg, bias)
    dt = L.F32 if cfg.act_dtype == "f32" else L.BF16
    t = lambda a: to_tensor(a, dev)
    idx = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    gte = torch.full((T, k), -7.0, dtype=torch.float32, device=dev)
    colsum = torch.full((E,), -7.0, dtype=torch.float32, device=dev)
    lg = torch.full((T, E), -7.0, dtype=torch.float32, device=dev)
    ws = torch.empty(max(L.router_noisy_workspace_size(T, d, E, dt), 256), dtype=torch.uint8, device=dev)
    L.router_topk_noisy_philox(t(x), t(w_g), t(b_g), t(w_n), t(b_n), seed, offset, eps, k, L.GATE_MODES[cfg.gate],
                               idx, gte, colsum, lg, ws)
    torch.cuda.synchronize()
    got = (idx.cpu().numpy(), gte.cpu().numpy().astype(np.float64), colsum.cpu().numpy().astype(np.float64),
           lg.cpu().numpy().astype(np.float64))

    # against the oracle, with the oracle's draws of the same stream (fp32, as
    # the layer holds them)
    noise = OP.gate_noise(seed, offset, T, E).astype(np.float32)
    f64 = lambda a: None if a is None else a.astype(np.float64)
    z = O.noisy_router_logits(O.to_f64(x, cfg.act_dtype), f64(w_g), f64(b_g), f64(w_n), f64(b_n), f64(noise), eps)
    tie, eg, ec = compare_router(name, z, k, cfg.gate, got[0], got[1], got[2])
    zerr = float(np.max(np.abs(got[3] - z) / np.maximum(1.0, np.max(np.abs(z), axis=1, keepdims=True))))
    assert zerr <= 1e-5, f"{name}: noisy logit err {zerr:.3e}"

    # the same bits as moe_router_topk_noisy fed the generator's [T, E] draws
    drawn = torch.empty((T, E), dtype=torch.float32, device=dev)
    L.gate_noise_philox(seed, offset, drawn)
    ref = _run(x, w_g, b_g, w_n, b_n, drawn.cpu().numpy(), eps, k, cfg.gate, T, d, E, dt)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)
    # another offset draws another sample
    if T * E >= 64:
        L.router_topk_noisy_philox(t(x), t(w_g), t(b_g), t(w_n), t(b_n), seed, offset + 1, eps, k,
                                   L.GATE_MODES[cfg.gate], idx, gte, colsum, lg, ws)
        torch.cuda.synchronize()
        assert not np.array_equal(lg.cpu().numpy().astype(np.float64), got[3])
    say(f"  near-tied {int(tie.sum())}, gate err {eg:.2e}, colsum err {ec:.2e}, logit err {zerr:.2e}")
