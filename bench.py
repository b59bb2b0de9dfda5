"""Benchmark: MoE-layer forward on one MI355X.

A step is one pass of the whole layer (router -> dispatch/permute -> routed
expert FFN -> shared expert FFN -> combine -> aux loss) over one batch of the
workload, with inputs already resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload mixtral]

The roofline object describes the grouped expert FFN (the only dense
contraction, and the dominant cost): algorithmic FLOPs of one call over its
median duration, measured with HIP events on the stream the kernels run on.
A third pass repeats the steps after a 512 MB scratch write each ("cold":
no input left in the last-level cache); a last one times whole steps of the
same layer with the routed FFN gathering its rows through the dispatch
permutation ("gathered"); then training steps (forward + backward) and, on
the same shapes with e4m3 expert weights, steps of the layer with the expert
products on e4m3 activations ("fp8", reported apart: another precision).
The CPU baseline times the float64
oracle on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/s + grouped-GEMM TFLOP/s (% MFMA peak), 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_traffic_mixtral.json")


def ffn_flops_per_row(cfg) -> float:
    if cfg.ffn == "linear":
        return 2.0 * cfg.d * cfg.d_out
    if cfg.ffn in ("relu", "gelu"):
        return 2.0 * cfg.d * cfg.d_ff + 2.0 * cfg.d_ff * cfg.d_out
    return 4.0 * cfg.d * cfg.d_ff + 2.0 * cfg.d_ff * cfg.d_out


def stage_bytes(cfg, a_kept: int) -> dict:
    """Minimum HBM bytes each memory-bound stage must move."""
    sx = 4 if cfg.act_dtype == "f32" else 2
    T, d, E, k, do = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_out
    router = T * d * sx + E * d * 4 + T * k * 8 + E * 4
    # noisy gating adds the noise projection, its bias and the draws
    router_noisy = router + E * d * 4 + E * 4 + T * E * 4
    # draws from the counter-based generator inside the kernels: no [T, E] read
    router_noisy_philox = router + E * d * 4 + E * 4
    dispatch = T * k * 4 + T * d * sx + a_kept * d * sx + T * k * 4 * 2
    combine = a_kept * do * sx + T * k * 8 + T * do * sx + (cfg.n_shared * T * do * sx)
    return {"router": router, "dispatch": dispatch, "combine": combine, "router_noisy": router_noisy,
            "router_noisy_philox": router_noisy_philox}


FFN_SOURCES = ("ffn.hip", "grouped_gemm.hip", "moe_internal.hpp")


def kernel_source_hash() -> str:
    """Hash of the sources the grouped FFN kernels are built from."""
    h = hashlib.sha256()
    for name in FFN_SOURCES:
        with open(os.path.join(ROOT, "sparse_mixture_experts_atomic_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per FFN call from committed rocprofv3 counter runs, if they
    were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("ffn_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("bytes_per_call")


def cpu_baseline(cfg, arr, C, n_tokens: int, min_seconds: float = 10.0, max_reps: int = 8):
    """The oracle, as it stands, on the first n_tokens tokens (all experts),
    repeated until at least min_seconds of CPU work have been timed."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    cap = O.capacity(n_tokens, cfg.k, cfg.E, cfg.cf, cfg.cap_round)
    reps, dt = 0, 0.0
    while reps < max_reps and (reps == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        w = O.decode_weights(arr, cfg.w_dtype)
        sh = O.decode_weights(arr, cfg.w_dtype, prefix="sh_") if cfg.n_shared else None
        x = O.to_f64(arr["x"][:n_tokens], cfg.act_dtype)
        b_g = None if arr["b_g"] is None else arr["b_g"].astype(np.float64)
        O.forward(x, arr["w_g"].astype(np.float64), b_g, cfg.k, cfg.gate, cap, cfg.ffn, w, sh, cfg.alpha)
        dt += time.perf_counter() - t0
        reps += 1
        del w, sh
    return {"value": reps * n_tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n_tokens} of {cfg.T} tokens of the {cfg.name} workload, {reps} repetition(s); "
                      f"float64 numpy oracle incl. decoding all expert weights to float64 each time; {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first steps after a cold start run a few % slower while clocks and
    # power settle (30 warm-up steps: whole steps 2.4% faster than after 5)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the training-step (forward + backward) leg")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8-activation leg")
    ap.add_argument("--no-gathered", action="store_true",
                    help="skip the gathered-FFN leg (its GEMMs share kernel names with the layer's own)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a 1 GiB device copy (for counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU path is not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calib:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "launches": 3}))
        return

    import workloads as W
    from sparse_mixture_experts_atomic_amd import MoELayer
    from sparse_mixture_experts_atomic_amd import _lib as L
    from workloads.device import layer_kwargs, to_tensor

    cfg = W.CONFIGS[args.workload]
    t0 = time.perf_counter()
    arr = W.generate(cfg)
    C = L.capacity(cfg.T, cfg.k, cfg.E, cfg.cf, cfg.cap_round)
    print(f"[bench] generated {cfg.name} inputs in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    lkw = layer_kwargs(cfg, arr, C, device="cuda")
    layer = MoELayer(**lkw)
    x = to_tensor(arr["x"], "cuda")
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        layer.forward(x)
    torch.cuda.synchronize()

    # timed region 1: whole steps back to back (this is `value`)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        layer.forward(x)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps

    # timed region 2: the same steps with HIP events between the stages, on
    # the stream the kernels are launched on (per-stage medians, roofline)
    stages = ["router", "dispatch", "experts", "shared", "combine", "aux"]
    ev = {s: [] for s in stages}
    torch.cuda.synchronize()
    for _ in range(args.steps):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
        marks[0].record()
        layer.router(x)
        marks[1].record()
        layer.dispatch(x)
        marks[2].record()
        layer.experts()
        marks[3].record()
        layer.shared(x)
        marks[4].record()
        layer.combine()
        marks[5].record()
        layer.aux()
        marks[6].record()
        for i, s in enumerate(stages):
            ev[s].append((marks[i], marks[i + 1]))
    torch.cuda.synchronize()
    st_ms = {s: float(np.median([a.elapsed_time(b) for a, b in ev[s]])) for s in stages}

    # timed region 2b: each stage alone, `steps` back-to-back calls between
    # one event pair (the stages are idempotent: each rewrites the same
    # outputs from the same inputs).  An event recorded between two kernels
    # costs a 6-11 us bubble before the next one, which region 2 charges to
    # the short stages; here it is paid once per loop.  Inputs a stage re-reads
    # stay in the last-level cache, as in the layer for all but the router.
    def loop_ms(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps
    loop_st_ms = {"router": loop_ms(lambda: layer.router(x)), "dispatch": loop_ms(lambda: layer.dispatch(x)),
                  "combine": loop_ms(layer.combine), "aux": loop_ms(layer.aux)}
    # the training-mode router with noisy gating (normal draws and the noise
    # projection resident like the other inputs; floor 1e-2), timed the same
    # way; it rewrites the router outputs, so the layer router runs again after
    w_n, b_n, noise = W.gen_noisy_gate(cfg)
    w_n, b_n, noise = to_tensor(w_n, "cuda"), to_tensor(b_n, "cuda"), to_tensor(noise, "cuda")
    loop_st_ms["router_noisy"] = loop_ms(lambda: layer.router_noisy(x, w_n, b_n, noise, 1e-2))
    loop_st_ms["router_noisy_philox"] = loop_ms(lambda: layer.router_noisy(x, w_n, b_n, None, 1e-2, seed=1234,
                                                                           offset=5))
    layer.router(x)
    torch.cuda.synchronize()

    # timed region 3 (reported apart, labelled cold): every step after a
    # 512 MB scratch write, so that no input is left in the 256 MB
    # last-level cache; the scratch write itself is outside the events
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold_step, cold_st = [], {s: [] for s in stages}
    for _ in range(args.steps):
        scratch.fill_(1)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
        marks[0].record()
        layer.router(x)
        marks[1].record()
        layer.dispatch(x)
        marks[2].record()
        layer.experts()
        marks[3].record()
        layer.shared(x)
        marks[4].record()
        layer.combine()
        marks[5].record()
        layer.aux()
        marks[6].record()
        torch.cuda.synchronize()
        cold_step.append(marks[0].elapsed_time(marks[-1]))
        for i, s in enumerate(stages):
            cold_st[s].append(marks[i].elapsed_time(marks[i + 1]))
    del scratch
    cold_ms = float(np.median(cold_step))
    cold_st_ms = {s: float(np.median(v)) for s, v in cold_st.items()}

    # timed region 4 (last, so that the regions above keep their kernel
    # order for the profiles): whole steps of the same layer with the routed FFN
    # reading x through the dispatch permutation (no packed copy of x; the
    # same weight tensors, bit-identical output)
    gathered = None
    glayer = None if args.no_gathered else MoELayer(**lkw, gather_rows=True)
    for _ in range(args.warmup if glayer is not None else 0):
        glayer.forward(x)
    if glayer is not None:
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            glayer.forward(x)
        stop.record()
        torch.cuda.synchronize()
        ms_step_gather = start.elapsed_time(stop) / args.steps
        gd, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gf = torch.cuda.Event(enable_timing=True)
        g_disp, g_exp = [], []
        for _ in range(args.steps):
            glayer.router(x)
            gd.record()
            glayer.dispatch(x)
            ge.record()
            glayer.experts()
            gf.record()
            torch.cuda.synchronize()
            g_disp.append(gd.elapsed_time(ge))
            g_exp.append(ge.elapsed_time(gf))
        gathered = {"ms_per_step": ms_step_gather, "value": cfg.T / (ms_step_gather * 1e-3),
                    "dispatch_ms": float(np.median(g_disp)), "experts_ms": float(np.median(g_exp)),
                    "note": "routed FFN reads x through perm_token (moe_expert_ffn_gathered); dispatch copies no rows"}
        del glayer

    # timed region 5 (last): training steps, forward + backward of a layer
    # instance that keeps the router logits; dy is a fixed seeded draw.  The
    # FFN backward's algorithmic FLOPs are twice the forward's per kept row
    # (dgrad and wgrad of every matrix); the fp32 recompute of the first
    # layer's pre-activations is not counted.
    backward = None
    if not args.no_backward and cfg.act_dtype == "bf16" and cfg.w_dtype == "bf16":
        blayer = MoELayer(**lkw)
        blayer.enable_backward()
        gen = torch.Generator(device="cpu").manual_seed(1234)
        dy = torch.randn((cfg.T, cfg.d_out), generator=gen).to(torch.bfloat16).to("cuda")
        for _ in range(min(args.warmup, 5)):
            blayer.forward(x)
            blayer.backward(x, dy)
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            blayer.forward(x)
            blayer.backward(x, dy)
        stop.record()
        torch.cuda.synchronize()
        ms_train = start.elapsed_time(stop) / args.steps
        bst = ["combine", "experts", "shared", "router", "permute"]
        bev = {s_: [] for s_ in bst}
        for _ in range(args.steps):
            blayer.forward(x)
            m = [torch.cuda.Event(enable_timing=True) for _ in range(len(bst) + 1)]
            m[0].record()
            blayer.backward_combine(dy)
            m[1].record()
            blayer.backward_experts()
            m[2].record()
            blayer.backward_shared(x, dy)
            m[3].record()
            blayer.backward_router(x)
            m[4].record()
            blayer.backward_permute(dy)
            m[5].record()
            for i, s_ in enumerate(bst):
                bev[s_].append((m[i], m[i + 1]))
        torch.cuda.synchronize()
        bms = {s_: float(np.median([a_.elapsed_time(b_) for a_, b_ in bev[s_]])) for s_ in bst}
        kept = int(blayer.offsets[-1].item())
        bwd_flops = 2.0 * ffn_flops_per_row(cfg) * kept
        backward = {"ms_per_train_step": ms_train, "train_tokens_per_s": cfg.T / (ms_train * 1e-3),
                    "stages_ms": bms, "ffn_bwd_flops": bwd_flops,
                    "ffn_bwd_tflops": bwd_flops / (bms["experts"] * 1e-3) / 1e12,
                    "kept_pre_activations": bool(blayer._kept and blayer._kept["routed"]),
                    "note": "training forward (moe_expert_ffn_grouped_train: the first product's fp32 "
                            "pre-activations kept) + backward (moe_combine_backward, "
                            "moe_expert_ffn_grouped_backward_kept, moe_router_backward, moe_permute_backward); "
                            "stage medians with HIP events between them"}
        del blayer

    # timed region 6 (last): the same shapes with e4m3 expert weights and the
    # expert products on e4m3 activations (per-row codes and scales for x and
    # the hidden layer); another precision, so reported apart from `value`
    fp8 = None
    if not args.no_fp8 and cfg.act_dtype == "bf16" and cfg.ffn != "linear" and cfg.d % 128 == 0 \
            and cfg.d_ff % 128 == 0:
        import dataclasses
        cfg8 = dataclasses.replace(cfg, w_dtype="fp8", name=cfg.name + "_e4m3")
        arr8 = W.generate(cfg8)
        flayer = MoELayer(**layer_kwargs(cfg8, arr8, C, device="cuda"), fp8_act=True)
        del arr8
        for _ in range(args.warmup):
            flayer.forward(x)
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            flayer.forward(x)
        stop.record()
        torch.cuda.synchronize()
        ms_f8 = start.elapsed_time(stop) / args.steps
        fst = ["router", "dispatch", "quantize", "experts", "shared", "combine"]
        fev = {s_: [] for s_ in fst}
        for _ in range(args.steps):
            m = [torch.cuda.Event(enable_timing=True) for _ in range(len(fst) + 1)]
            m[0].record()
            flayer.router(x)
            m[1].record()
            flayer.dispatch(x)
            m[2].record()
            flayer.quantize(x)
            m[3].record()
            flayer.experts()
            m[4].record()
            flayer.shared(x)
            m[5].record()
            flayer.combine()
            m[6].record()
            for i, s_ in enumerate(fst):
                fev[s_].append((m[i], m[i + 1]))
        torch.cuda.synchronize()
        fms = {s_: float(np.median([a_.elapsed_time(b_) for a_, b_ in fev[s_]])) for s_ in fst}
        f_kept = int(flayer.offsets[-1].item())
        f_flops = ffn_flops_per_row(cfg) * f_kept
        f_tf = f_flops / (fms["experts"] * 1e-3) / 1e12
        fp8 = {"ms_per_step": ms_f8, "value": cfg.T / (ms_f8 * 1e-3), "unit": "tokens/s", "stages_ms": fms,
               "ffn_tflops": f_tf, "peak": PEAK_FP8_TFLOPS, "frac": f_tf / PEAK_FP8_TFLOPS,
               "ffn_flops_per_launch": f_flops,
               "note": "e4m3 expert weights (per-row scales) and e4m3 activations (per-row scales, hidden layer "
                       "requantised); moe_quantize_rows_e4m3 + moe_expert_ffn_fp8 (rows gathered through "
                       "perm_token); router fp32"}
        del flayer

    a_kept = int(layer.offsets[-1].item())
    ffn_flops = ffn_flops_per_row(cfg) * a_kept
    sh_flops = ffn_flops_per_row(cfg) * cfg.T * cfg.n_shared
    ffn_tflops = ffn_flops / (st_ms["experts"] * 1e-3) / 1e12
    byts = stage_bytes(cfg, a_kept)
    traffic = stored_traffic()

    out = {
        "metric": METRIC,
        "value": cfg.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d, "E": cfg.E, "k": cfg.k,
                   "n_shared": cfg.n_shared, "d_ff": cfg.d_ff, "ffn": cfg.ffn, "gate": cfg.gate,
                   "capacity": C, "activations": cfg.act_dtype, "expert_weights": cfg.w_dtype,
                   "router": "fp32"},
        "roofline": {"bound": "mfma", "achieved": ffn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": ffn_tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": "moe_expert_ffn_grouped (routed experts): gate/up GEMM + down GEMM",
                     "flops_per_launch": ffn_flops, "median_ms": st_ms["experts"]},
        "stages_ms": st_ms,
        "gathered": gathered,
        "stages_hbm_frac": {
            "router": byts["router"] / (st_ms["router"] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "dispatch": byts["dispatch"] / (st_ms["dispatch"] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "combine": byts["combine"] / (st_ms["combine"] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        },
        "stages_ms_loop": loop_st_ms,
        "stages_hbm_frac_loop": {k_: byts[k_] / (loop_st_ms[k_] * 1e-3) / 1e9 / PEAK_HBM_GBPS
                                 for k_ in ("router", "dispatch", "combine", "router_noisy", "router_noisy_philox")},
        "shared_tflops": (sh_flops / (st_ms["shared"] * 1e-3) / 1e12) if cfg.n_shared else None,
        "backward": backward,
        "fp8": fp8,
        "kept_rows": a_kept,
        "cold": {
            "note": "median step with a 512 MB scratch write before each step (no input in the last-level cache)",
            "ms_per_step": cold_ms, "value": cfg.T / (cold_ms * 1e-3), "stages_ms": cold_st_ms,
            "stages_hbm_frac": {k_: byts[k_] / (cold_st_ms[k_] * 1e-3) / 1e9 / PEAK_HBM_GBPS
                                for k_ in ("router", "dispatch", "combine")},
            "ffn_tflops": ffn_flops / (cold_st_ms["experts"] * 1e-3) / 1e12,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, arr, C, min(args.cpu_tokens, cfg.T))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
