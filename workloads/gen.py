"""Seeded synthetic inputs for the MoE layer workloads.

Every tensor (and, for expert weights, every expert) draws from its own
numpy PCG64 stream keyed by ``(seed, tensor tag, expert index)``, so any one
expert can be regenerated alone and the draws can run on several threads
without changing a single value.  Draws are float32 standard normals (or
uniforms) scaled by the configured standard deviation, then stored as the
workload's dtype: fp32 as is, bf16 by round-to-nearest-even, fp8 e4m3 as
codes with one fp32 scale per output row (scale = row max / 448).

Layouts are row-major: x [T, d]; W_g [E, d]; b_g [E]; W1, W3 [E, d_ff, d]
(W1 is [E, d_out, d] for linear experts); W2 [E, d_out, d_ff]; expert biases
b1 [E, rows of W1], b2 [E, d_out]; shared experts use the same layouts with
a leading K_s axis.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

from .configs import MoEConfig
from .encode import f32_to_bf16_bits, quantize_rows_e4m3

_TAGS = {"x": 1, "w_g": 2, "b_g": 3, "w1": 4, "w3": 5, "w2": 6, "b1": 7,
         "b2": 8, "sw1": 9, "sw3": 10, "sw2": 11, "sb1": 12, "sb2": 13,
         "w_n": 14, "b_n": 15, "noise": 16}


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, tag: str, idx: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, _TAGS[tag], idx]))


def _draw(rng: np.random.Generator, shape, dist) -> np.ndarray:
    kind, v = dist
    if kind == "normal":
        out = rng.standard_normal(shape, dtype=np.float32)
        out *= np.float32(math.sqrt(v))
        return out
    if kind == "uniform":
        return rng.uniform(-v, v, size=shape).astype(np.float32)
    raise ValueError(kind)


def _store(w32: np.ndarray, dtype: str):
    if dtype == "f32":
        return w32, None
    if dtype == "bf16":
        return f32_to_bf16_bits(w32), None
    if dtype == "fp8":
        return quantize_rows_e4m3(w32)
    raise ValueError(dtype)


def gen_x(cfg: MoEConfig, rows: Optional[slice] = None) -> np.ndarray:
    """x [T, d] in the activation dtype (float32 or bf16 bit patterns)."""
    # x is drawn in row chunks of 1024 tokens so a slice can be regenerated.
    chunk = 1024
    T = cfg.T
    start, stop = (0, T) if rows is None else (rows.start or 0, rows.stop if rows.stop is not None else T)
    if stop <= start:
        return _store(np.zeros((0, cfg.d), np.float32), cfg.act_dtype)[0]
    c0, c1 = start // chunk, (stop + chunk - 1) // chunk

    def one(ci):
        n = min(chunk, T - ci * chunk)
        return _draw(_rng(cfg.seed, "x", ci), (n, cfg.d), cfg.x_dist)

    if c1 - c0 > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            parts = list(ex.map(one, range(c0, c1)))
    else:
        parts = [one(ci) for ci in range(c0, c1)]
    x32 = np.concatenate(parts, axis=0)[start - c0 * chunk: stop - c0 * chunk]
    return _store(np.ascontiguousarray(x32), cfg.act_dtype)[0]


def gen_expert(cfg: MoEConfig, e: int, shared: bool = False) -> Dict[str, np.ndarray]:
    """Weights (and scales / biases) of one routed expert, or of shared expert ``e``."""
    p = "s" if shared else ""
    out = {}
    wdt = cfg.w_dtype
    n1 = cfg.n1
    w1 = _draw(_rng(cfg.seed, p + "w1", e), (n1, cfg.d), ("normal", cfg.w1_var))
    out["w1"], out["s1"] = _store(w1, wdt)
    if cfg.has_w3:
        w3 = _draw(_rng(cfg.seed, p + "w3", e), (cfg.d_ff, cfg.d), ("normal", cfg.w3_var))
        out["w3"], out["s3"] = _store(w3, wdt)
    if cfg.has_w2:
        w2 = _draw(_rng(cfg.seed, p + "w2", e), (cfg.d_out, cfg.d_ff), ("normal", cfg.w2_var))
        out["w2"], out["s2"] = _store(w2, wdt)
    if cfg.b1_var is not None:
        out["b1"] = _draw(_rng(cfg.seed, p + "b1", e), (n1,), ("normal", cfg.b1_var))
    if cfg.b2_var is not None and cfg.has_w2:
        out["b2"] = _draw(_rng(cfg.seed, p + "b2", e), (cfg.d_out,), ("normal", cfg.b2_var))
    return out


def _stack(parts, key):
    if parts[0].get(key) is None:
        return None
    return np.ascontiguousarray(np.stack([p[key] for p in parts]))


def gen_experts(cfg: MoEConfig, shared: bool = False) -> Dict[str, Optional[np.ndarray]]:
    n = cfg.n_shared if shared else cfg.E
    if n == 0:
        return {}
    if n > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            parts = list(ex.map(lambda e: gen_expert(cfg, e, shared), range(n)))
    else:
        parts = [gen_expert(cfg, 0, shared)]
    keys = ("w1", "s1", "w3", "s3", "w2", "s2", "b1", "b2")
    return {k: _stack(parts, k) for k in keys}


def gen_router(cfg: MoEConfig):
    w_g = _draw(_rng(cfg.seed, "w_g"), (cfg.E, cfg.d), cfg.wg_dist)
    b_g = None
    if cfg.bg_var is not None:
        b_g = _draw(_rng(cfg.seed, "b_g"), (cfg.E,), ("normal", cfg.bg_var))
    return w_g, b_g


def gen_noisy_gate(cfg: MoEConfig, bias: bool = True):
    """Inputs of the noisy gate in training mode: the noise projection W_n
    [E, d] and its bias b_n [E] (or None), both uniform in +-1/sqrt(d) as a
    freshly initialised linear layer draws them, and the standard normal
    draws noise [T, E], all float32."""
    h = 1.0 / math.sqrt(cfg.d)
    w_n = _draw(_rng(cfg.seed, "w_n"), (cfg.E, cfg.d), ("uniform", h))
    b_n = _draw(_rng(cfg.seed, "b_n"), (cfg.E,), ("uniform", h)) if bias else None
    noise = _draw(_rng(cfg.seed, "noise"), (cfg.T, cfg.E), ("normal", 1.0))
    return w_n, b_n, noise


def generate(cfg: MoEConfig, with_experts: bool = True) -> Dict[str, Optional[np.ndarray]]:
    """All inputs of one workload as numpy arrays in their stored dtypes.

    Keys: x, w_g, b_g, and when ``with_experts``: w1, s1, w3, s3, w2, s2, b1,
    b2 for routed experts and the same keys prefixed ``sh_`` for shared ones.
    Missing tensors are None.
    """
    out: Dict[str, Optional[np.ndarray]] = {}
    out["x"] = gen_x(cfg)
    out["w_g"], out["b_g"] = gen_router(cfg)
    if with_experts:
        r = gen_experts(cfg)
        for k in ("w1", "s1", "w3", "s3", "w2", "s2", "b1", "b2"):
            out[k] = r.get(k)
        s = gen_experts(cfg, shared=True)
        for k in ("w1", "s1", "w3", "s3", "w2", "s2", "b1", "b2"):
            out["sh_" + k] = s.get(k) if s else None
    return out
