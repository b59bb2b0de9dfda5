"""Workload definitions for the sparse MoE layer forward pass.

Each configuration fixes shapes, dtypes, gate mode, capacity and the value
distributions of its synthetic inputs.  Variances are written as variances:
``N(0, v)`` means mean 0 and variance ``v`` (the Switch Transformer
walkthrough, "缩小的初始化方差", describes its s=0.1 as an initialisation
*variance* scale, and 1/d_in is the usual fan-in variance).

Nothing here computes any part of the layer; the capacity integer is left to
the oracle and to the library.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                      # tokens
    d: int                      # d_model (input width)
    d_out: int                  # output width
    E: int                      # routed experts
    k: int                      # experts per token
    ffn: str                    # 'linear' | 'relu' | 'swiglu' | 'gelu'
    d_ff: int                   # hidden width (ignored for 'linear')
    gate: str                   # 'renorm' | 'prob'
    cf: Optional[float]         # capacity factor, None = no capacity limit
    cap_round: str = "ceil"     # 'ceil' | 'floor'
    n_shared: int = 0           # always-on shared experts
    act_dtype: str = "bf16"     # 'f32' | 'bf16'
    w_dtype: str = "bf16"       # 'f32' | 'bf16' | 'fp8'
    alpha: float = 1e-2         # aux-loss coefficient
    seed: int = 0
    # value distributions: ('normal', variance) or ('uniform', half_width)
    x_dist: Tuple[str, float] = ("normal", 1.0)
    wg_dist: Tuple[str, float] = ("normal", 1.0)
    bg_var: Optional[float] = None     # router bias variance (None = no bias)
    w1_var: float = 1.0
    w3_var: float = 1.0
    w2_var: float = 1.0
    b1_var: Optional[float] = None     # expert biases (None = none)
    b2_var: Optional[float] = None

    @property
    def n1(self) -> int:
        """Rows of the first expert matrix (d_out for linear experts)."""
        return self.d_out if self.ffn == "linear" else self.d_ff

    @property
    def has_w3(self) -> bool:
        return self.ffn == "swiglu"

    @property
    def has_w2(self) -> bool:
        return self.ffn in ("relu", "swiglu", "gelu")

    def scaled(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


TINY = MoEConfig(
    name="tiny", T=64, d=32, d_out=32, E=4, k=2, ffn="linear", d_ff=0,
    gate="renorm", cf=None, act_dtype="f32", w_dtype="f32", alpha=1.0, seed=0,
    x_dist=("normal", 1.0), wg_dist=("normal", 1.0 / 32),
    w1_var=1.0 / 32, b1_var=0.1)

SWITCH = MoEConfig(
    name="switch", T=8192, d=768, d_out=768, E=8, k=1, ffn="relu", d_ff=3072,
    gate="prob", cf=1.25, act_dtype="bf16", w_dtype="bf16", alpha=1e-2, seed=1,
    x_dist=("normal", 1.0), wg_dist=("normal", 0.1 / 768),
    w1_var=0.1 / 768, w2_var=0.1 / 3072)

# same shape with capacity factor 1.0, so that the drop path is exercised
SWITCH_DROP = SWITCH.scaled(name="switch_drop", cf=1.0, seed=11)

MIXTRAL = MoEConfig(
    name="mixtral", T=4096, d=4096, d_out=4096, E=8, k=2, ffn="swiglu",
    d_ff=14336, gate="renorm", cf=None, act_dtype="bf16", w_dtype="bf16",
    alpha=1e-2, seed=2, x_dist=("normal", 1.0), wg_dist=("normal", 1.0 / 4096),
    w1_var=1.0 / 4096, w3_var=1.0 / 4096, w2_var=1.0 / 14336)

DEEPSEEK = MoEConfig(
    name="deepseek", T=4096, d=2048, d_out=2048, E=64, k=6, ffn="swiglu",
    d_ff=1408, gate="prob", cf=None, n_shared=2, act_dtype="bf16",
    w_dtype="bf16", alpha=1e-2, seed=3, x_dist=("normal", 1.0),
    wg_dist=("normal", 1.0 / 2048), bg_var=2.0,
    w1_var=1.0 / 2048, w3_var=1.0 / 2048, w2_var=1.0 / 1408)

STRESS = MoEConfig(
    name="stress", T=32768, d=7168, d_out=7168, E=256, k=8, ffn="swiglu",
    d_ff=2048, gate="prob", cf=1.0, n_shared=1, act_dtype="bf16",
    w_dtype="fp8", alpha=1e-2, seed=4, x_dist=("normal", 1.0),
    wg_dist=("uniform", 1.0 / math.sqrt(7168)),
    w1_var=1.0 / 7168, w3_var=1.0 / 7168, w2_var=1.0 / 2048)

# GELU experts (the two-layer nn.GELU experts of the from-scratch MoE page,
# section 3): that page's own model (input 128, hidden 256, output 128, 8
# experts, top-2 renormalised, biases everywhere, batch 32 x sequence 64,
# fp32, linear layers at their default uniform init, given here as the
# matching variances), and the Switch-shaped layer with GELU experts
P1_GELU = MoEConfig(
    name="p1_gelu", T=2048, d=128, d_out=128, E=8, k=2, ffn="gelu", d_ff=256,
    gate="renorm", cf=None, act_dtype="f32", w_dtype="f32", alpha=1e-2, seed=5,
    x_dist=("normal", 1.0), wg_dist=("uniform", 1.0 / math.sqrt(128)), bg_var=1.0 / 384,
    w1_var=1.0 / 384, w2_var=1.0 / 768, b1_var=1.0 / 384, b2_var=1.0 / 768)

SWITCH_GELU = SWITCH.scaled(name="switch_gelu", ffn="gelu", seed=6, b1_var=1e-2, b2_var=1e-2)

CONFIGS = {c.name: c for c in (TINY, SWITCH, SWITCH_DROP, MIXTRAL, DEEPSEEK, STRESS, P1_GELU, SWITCH_GELU)}

# The five workloads in their canonical order (tiny, Switch, Mixtral,
# DeepSeekMoE, stress).
CANONICAL = ("tiny", "switch", "mixtral", "deepseek", "stress")


def get_config(name: str) -> MoEConfig:
    return CONFIGS[name]


def shrink(cfg: MoEConfig, T: int, d: Optional[int] = None,
           d_ff: Optional[int] = None, E: Optional[int] = None,
           k: Optional[int] = None, **kw) -> MoEConfig:
    """Same structure and distributions at a size the oracle finishes fast.

    Variances that are written as 1/d_in in the workload are rescaled to the
    new widths so logits and activations keep their magnitudes.
    """
    d2 = d if d is not None else cfg.d
    f2 = d_ff if d_ff is not None else cfg.d_ff
    rep = dict(T=T, d=d2, d_out=d2, d_ff=f2, name=cfg.name + "_small")
    if E is not None:
        rep["E"] = E
    if k is not None:
        rep["k"] = k
    kind, v = cfg.wg_dist
    if kind == "normal":
        rep["wg_dist"] = ("normal", v * cfg.d / d2)
    else:
        rep["wg_dist"] = ("uniform", v * math.sqrt(cfg.d / d2))
    rep["w1_var"] = cfg.w1_var * cfg.d / d2
    rep["w3_var"] = cfg.w3_var * cfg.d / d2
    if cfg.d_ff:
        rep["w2_var"] = cfg.w2_var * cfg.d_ff / f2
    rep.update(kw)
    return dataclasses.replace(cfg, **rep)
