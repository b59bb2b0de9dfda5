"""CPU oracle for the sparsely gated MoE FFN layer forward pass (float64).

TEST INFRASTRUCTURE ONLY.  This module is the independent reference that the
GPU path is checked against.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import it; the product library never does
and shares no code with it.

Sources (web pages on the method; cited by page and section):
  P1  "混合专家模型MoE入门实战：从零搭建可运行的小型MoE模型" (0539edu.com)
  P2  "MoE架构解析：混合专家模型原理与工程实践" (jsqmd.com)
  P3  "MoE混合专家模型原理与实战：稀疏激活如何实现万亿参数高效推理" (framerc.cn)
  P4  "混合专家 MOE 是什么" (dgblog.top)
  P5  "MoE 混合专家模型串讲：从 Switch Transformer 到 DeepSeekMoE" (uestc.de5.net)

Every step is written the plain way, in float64, with numpy matmul (and
scipy's erf for GELU) as the only library primitives.  Readings taken where the pages are silent or
disagree are listed next to the function that takes them.

Parity status: every function here is pinned by a CPU test (worked example,
closed forms, brute force, invariants or a library routine); large-shape FFN
values have no printed anchor beyond those structural pins.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import scipy.special

# ---------------------------------------------------------------------------
# stored-value decoding
# ---------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> float64: the pattern is the top half of an fp32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    """Value of one OCP E4M3FN code, from the format definition.

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
    holds subnormals m * 2**-9; S.1111.111 is NaN; there is no infinity.
    """
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def to_f64(a: np.ndarray, dtype: str, scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Stored tensor -> float64.  fp8 rows are multiplied by their row scale."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(a)
    if dtype == "fp8":
        v = e4m3_to_f64(a)
        return v * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# router, softmax, top-k, gates
# ---------------------------------------------------------------------------


def router_logits(x: np.ndarray, w_g: np.ndarray, b_g: Optional[np.ndarray] = None) -> np.ndarray:
    """z[t, e] = sum_c x[t, c] * W_g[e, c] (+ b_g[e]).

    P4, 公式：三步走 step one: the router score is W_g x with W_g shaped
    (experts x input width).  P1 §3.3 and P3 §3.1 use a Linear layer (P1
    with a bias, P3 without); the bias is optional here.
    """
    z = np.asarray(x, np.float64) @ np.asarray(w_g, np.float64).T
    if b_g is not None:
        z = z + np.asarray(b_g, np.float64)[None, :]
    return z


def softmax(z: np.ndarray) -> np.ndarray:
    """Row softmax exp(z_i) / sum_j exp(z_j) (P4, 一个小算例).

    The row maximum is subtracted first; this changes nothing mathematically.
    """
    z = np.asarray(z, np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def topk_select(z: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest router logits per token, largest first.

    Selection is on the logits, rounded to fp32 first: Switch keeps the
    router in float32 (P5, 选择性精度), so the selection decision is taken in
    that precision.  Selecting on logits equals selecting on softmax
    probabilities (softmax is monotone; P1 §3.3 selects on probabilities,
    P2 §2.1 and P3 §3.1 on logits).  Equal values: the lower expert index
    comes first (the pages fix no tie order; this is the reading taken).
    """
    z32 = np.asarray(z, np.float64).astype(np.float32).astype(np.float64)
    T, E = z32.shape
    if not 1 <= k <= E:
        raise ValueError("k must satisfy 1 <= k <= E")
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        # stable sort of -z keeps lower indices first among equal values
        order = np.argsort(-z32[t], kind="stable")
        out[t] = order[:k]
    return out


def near_tie_mask(z: np.ndarray, k: int, gap: float = 1e-5) -> np.ndarray:
    """True for tokens whose top-(k+1) sorted logits have a consecutive gap < gap.

    For such tokens more than one top-k answer is correct within fp32
    rounding, so index parity is not required there (only validity).
    """
    z = np.asarray(z, np.float64)
    T, E = z.shape
    kk = min(k + 1, E)
    s = -np.sort(-z, axis=-1)[:, :kk]
    if kk < 2:
        return np.zeros(T, dtype=bool)
    return np.any((s[:, :-1] - s[:, 1:]) < gap, axis=-1)


def gates(p: np.ndarray, idx: np.ndarray, mode: str) -> np.ndarray:
    """Gate weight of each selected expert.

    'renorm': the selected probabilities divided by their sum (P1 §3.3), which
    equals a softmax over the selected logits (P2 §2.1 top_k_gating, P3 §3.1).
    'prob': the softmax probability itself, zero elsewhere (P5 DeepSeekMoE
    数学定义, conventional top-K routing; P5 代码实战 top-1 gate: probs times
    a one-hot mask).
    """
    sel = np.take_along_axis(np.asarray(p, np.float64), idx.astype(np.int64), axis=-1)
    if mode == "renorm":
        return sel / np.sum(sel, axis=-1, keepdims=True)
    if mode == "prob":
        return sel
    raise ValueError(mode)


def softplus(u: np.ndarray) -> np.ndarray:
    """softplus(u) = ln(1 + e^u), written as max(u, 0) + ln(1 + e^-|u|) so
    that large |u| neither overflows nor loses the small term."""
    u = np.asarray(u, np.float64)
    return np.maximum(u, 0.0) + np.log1p(np.exp(-np.abs(u)))


def noisy_router_logits(x: np.ndarray, w_g: np.ndarray, b_g: Optional[np.ndarray],
                        w_n: np.ndarray, b_n: Optional[np.ndarray], noise: np.ndarray,
                        eps: float = 0.0) -> np.ndarray:
    """Noisy router logits: clean logits plus a standard normal draw times a
    learned, input-dependent noise scale.

    P2 §2.1 (Noisy Top-k 门控): the noise scale is softplus of a second
    projection x W_noise of the input, multiplied by a standard normal
    sample and added to the clean logits x W_gate; the top-k gating then
    runs on these noisy logits.  P5 代码实战 (NoisyTop1Gate, training mode):
    the second projection is a Linear layer with a bias, and the scale gets a
    floor of 1e-2 added after the softplus.  Both are this function, with
    eps = 0 (P2) or 1e-2 (P5).  The normal samples are an input
    (noise[t, e], one per token and expert), so the GPU and this function see
    the same draws.
    """
    z = router_logits(x, w_g, b_g)
    zn = router_logits(x, w_n, b_n)
    return z + np.asarray(noise, np.float64) * (softplus(zn) + float(eps))


def noisy_router(x: np.ndarray, w_g: np.ndarray, b_g: Optional[np.ndarray],
                 w_n: np.ndarray, b_n: Optional[np.ndarray], noise: np.ndarray, eps: float,
                 k: int, gate_mode: str) -> Dict[str, np.ndarray]:
    """Router in training mode with noisy gating: softmax, top-k and gates of
    the noisy logits, as the clean router does for its logits.

    P2 §2.1 passes the noisy logits to the same top-k gating (softmax over the
    k selected logits: gate mode 'renorm').  P5 代码实战 takes the softmax of
    the noisy logits, the arg-max as the top-1 expert, the probability as its
    weight (gate mode 'prob') and those probabilities in its balance loss, so
    the column sums here are of the noisy softmax.
    """
    z = noisy_router_logits(x, w_g, b_g, w_n, b_n, noise, eps)
    p = softmax(z)
    idx = topk_select(z, k)
    return {"logits": z, "probs": p, "topk_idx": idx, "topk_gate": gates(p, idx, gate_mode),
            "prob_colsum": np.sum(p, axis=0), "near_tie": near_tie_mask(z, k)}


# ---------------------------------------------------------------------------
# capacity and dispatch
# ---------------------------------------------------------------------------


def capacity(T: int, k: int, E: int, cf: Optional[float], round_mode: str = "ceil") -> int:
    """Expert capacity; -1 means no limit (cf None or <= 0).

    P1 §4.2 gives capacity = factor * tokens / experts (1000 tokens, 8
    experts, factor 1.25 -> 156, i.e. rounded down); P5 专家容量 states that
    top-1 routing needs half the factor of top-2, so capacity scales with k.
    Reading taken: C = round(T * k * cf / E), rounded up by default, with a
    rounding-down mode that reproduces P1's example.
    """
    if cf is None or cf <= 0:
        return -1
    v = T * k * cf / E
    if round_mode == "ceil":
        return int(math.ceil(v))
    if round_mode == "floor":
        return int(math.floor(v))
    raise ValueError(round_mode)


def dispatch(idx: np.ndarray, E: int, C: int) -> Dict[str, np.ndarray]:
    """Capacity-limited dispatch in token order.

    Assignment (t, j) goes to expert e = idx[t, j].  Its rank is the number
    of assignments to e from tokens before t (a token never picks the same
    expert twice, so the slot j never breaks a tie).  It is kept iff rank < C
    (P5 专家容量: tokens beyond capacity skip the expert; which ones drop is
    read as "the later tokens").  Kept rows are packed expert by expert, in
    token order inside each expert (P1 §2.4: gather the tokens of one expert
    together, run them, scatter back).

    Returns counts_routed[E], counts_kept[E], offsets[E+1], dest_pos[T,k]
    (-1 = dropped) and perm_token[A_kept] (source token of each packed row).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    counts_routed = np.zeros(E, dtype=np.int64)
    rank = np.zeros((T, k), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            rank[t, j] = counts_routed[e]
            counts_routed[e] += 1
    if C < 0:
        counts_kept = counts_routed.copy()
    else:
        counts_kept = np.minimum(counts_routed, C)
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts_kept[e]
    dest_pos = np.full((T, k), -1, dtype=np.int64)
    perm_token = np.zeros(int(offsets[E]), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if C < 0 or rank[t, j] < C:
                p = offsets[e] + rank[t, j]
                dest_pos[t, j] = p
                perm_token[p] = t
    return {
        "counts_routed": counts_routed.astype(np.int32),
        "counts_kept": counts_kept.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "dest_pos": dest_pos.astype(np.int32),
        "perm_token": perm_token.astype(np.int32),
        "rank": rank.astype(np.int32),
    }


def permute(x: np.ndarray, perm_token: np.ndarray) -> np.ndarray:
    """Packed expert input rows: Xp[p] = x[perm_token[p]]."""
    return np.asarray(x)[np.asarray(perm_token, dtype=np.int64)]


# ---------------------------------------------------------------------------
# experts
# ---------------------------------------------------------------------------


def silu(u: np.ndarray) -> np.ndarray:
    return u / (1.0 + np.exp(-u))


def gelu(u: np.ndarray) -> np.ndarray:
    """GELU in its exact form u * Phi(u) = u/2 * (1 + erf(u / sqrt 2)): the
    experts of P1 §3.2 and P3 §3.1 use torch's nn.GELU, whose default is this
    form (not the tanh approximation)."""
    u = np.asarray(u, np.float64)
    return 0.5 * u * (1.0 + scipy.special.erf(u / math.sqrt(2.0)))


def expert_ffn(kind: str, rows: np.ndarray, w1: np.ndarray, w3: Optional[np.ndarray] = None,
               w2: Optional[np.ndarray] = None, b1: Optional[np.ndarray] = None,
               b2: Optional[np.ndarray] = None) -> np.ndarray:
    """One expert applied to a batch of rows, all operands float64.

    'linear': A x + b (P4, 公式：三步走 step two, the simplest expert).
    'relu'  : W2 relu(W1 x + b1) + b2 (the two-layer FFN of P1 §3.2 and
              P3 §3.1, with the activation read as ReLU for the Switch-style
              workload).
    'swiglu': W2 (silu(W1 x) * (W3 x)) (not on the pages; the standard
              gated-linear form is the reading taken).
    'gelu'  : W2 gelu(W1 x + b1) + b2, the two-layer FFN of P1 §3.2 and
              P3 §3.1 with their GELU activation.
    Weights are [out, in]; rows are [n, in].
    """
    rows = np.asarray(rows, np.float64)
    h = rows @ w1.T
    if b1 is not None:
        h = h + b1[None, :]
    if kind == "linear":
        return h
    if kind == "relu":
        h = np.maximum(h, 0.0)
    elif kind == "gelu":
        h = gelu(h)
    elif kind == "swiglu":
        h = silu(h) * (rows @ w3.T)
    else:
        raise ValueError(kind)
    y = h @ w2.T
    if b2 is not None:
        y = y + b2[None, :]
    return y


def experts_packed(kind: str, xp: np.ndarray, offsets: np.ndarray, weights: Dict[str, np.ndarray]) -> np.ndarray:
    """Ye[p] = FFN_e(Xp[p]) for each packed segment e (float64 weights)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    E = len(offsets) - 1
    n_out = weights["w2"].shape[1] if kind != "linear" else weights["w1"].shape[1]
    ye = np.zeros((int(offsets[E]), n_out), dtype=np.float64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            ye[a:b] = expert_ffn(kind, xp[a:b], weights["w1"][e],
                                 None if weights.get("w3") is None else weights["w3"][e],
                                 None if weights.get("w2") is None else weights["w2"][e],
                                 None if weights.get("b1") is None else weights["b1"][e],
                                 None if weights.get("b2") is None else weights["b2"][e])
    return ye


def shared_experts(kind: str, x: np.ndarray, weights: Dict[str, np.ndarray]) -> np.ndarray:
    """Sum of the always-on shared experts over every token, weight 1.

    P5 共享专家隔离: K_s experts are active for every token whatever the
    router does; P1 §5.2 describes the same split.  Their outputs are added
    with weight one and never dropped (reading taken).
    """
    n = weights["w1"].shape[0]
    acc = None
    for s in range(n):
        y = expert_ffn(kind, x, weights["w1"][s],
                       None if weights.get("w3") is None else weights["w3"][s],
                       None if weights.get("w2") is None else weights["w2"][s],
                       None if weights.get("b1") is None else weights["b1"][s],
                       None if weights.get("b2") is None else weights["b2"][s])
        acc = y if acc is None else acc + y
    return acc


# ---------------------------------------------------------------------------
# combine and aux loss
# ---------------------------------------------------------------------------


def combine(ye: np.ndarray, dest_pos: np.ndarray, g: np.ndarray, ys: Optional[np.ndarray] = None,
            residual: Optional[np.ndarray] = None) -> np.ndarray:
    """y[t] = sum over kept slots g[t,j] * Ye[dest[t,j]] (+ shared) (+ residual).

    P1 §3.4 accumulates weight * expert output into a zero-initialised output
    per (slot, expert) mask; P3 §3.1 and P4 完整代码 form the same weighted
    sum.  A dropped slot adds nothing (P5 专家容量: the expert output of a
    dropped token is 0) and the remaining gates are left as they are.
    """
    T, k = dest_pos.shape
    y = np.zeros((T, ye.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            p = int(dest_pos[t, j])
            if p >= 0:
                y[t] += g[t, j] * ye[p]
    if ys is not None:
        y = y + ys
    if residual is not None:
        y = y + residual
    return y


def aux_loss(counts_routed: np.ndarray, prob_colsum: np.ndarray, T: int, k: int, E: int,
             alpha: float) -> float:
    """Switch load-balancing loss alpha * E * sum_e f_e * P_e.

    f_e: fraction of the T*k assignments that chose e, counted before any
    capacity drop (P1 §3.4 divides the selection counts by tokens * k);
    P_e: mean router probability of e over the T tokens (P5 负载均衡损失函数).
    With uniform routing both are 1/E and the sum times E is 1.
    """
    f = np.asarray(counts_routed, np.float64) / float(T * k)
    P = np.asarray(prob_colsum, np.float64) / float(T)
    return float(alpha * E * np.sum(f * P))


def dense_moe(x: np.ndarray, w_g: np.ndarray, b_g: Optional[np.ndarray], kind: str,
              weights: Dict[str, np.ndarray]) -> np.ndarray:
    """Dense MoE: every expert runs and is weighted by the full softmax.

    P4, 公式：三步走: g = softmax(W_g x), y = sum_i g_i e_i(x); P4 完整代码
    (BasicMOE) computes all experts and the weighted sum.  P4 稠密 vs 稀疏:
    the sparse layer only adds a top-k step, so at k = E with no capacity
    limit the sparse result must equal this one.
    """
    p = softmax(router_logits(x, w_g, b_g))
    E = p.shape[1]
    y = None
    for e in range(E):
        ye = expert_ffn(kind, x, weights["w1"][e],
                        None if weights.get("w3") is None else weights["w3"][e],
                        None if weights.get("w2") is None else weights["w2"][e],
                        None if weights.get("b1") is None else weights["b1"][e],
                        None if weights.get("b2") is None else weights["b2"][e])
        term = p[:, e:e + 1] * ye
        y = term if y is None else y + term
    return y


# ---------------------------------------------------------------------------
# fp8 activations (expert inputs and hidden layer quantised per row)
# ---------------------------------------------------------------------------
# P2's deployment paragraph quantises the expert weights to int8; P3 §4.2
# runs the experts in INT4 and keeps the router in FP16.  The pages fix the
# principle (quantise the experts, keep the router precise), not a format.
# Readings taken: the e4m3 format of the stored weights (OCP E4M3FN) for the
# expert inputs too, one fp32 scale per row (per token) set so that the row's
# largest magnitude maps to 448, the format's largest finite value, exactly
# as the weights are scaled per output row; the hidden layer of a two-layer
# expert is rounded to bf16 (the kernel's precision for that value) and then
# quantised per row the same way before the second matrix.


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Values rounded to fp32, then to bf16 (nearest, ties to the even
    pattern), returned as float64."""
    u = np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float32)).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


_E4M3_POS = E4M3_TABLE[:127]          # codes 0x00..0x7E: 0 .. 448, increasing


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """fp32 values -> OCP E4M3FN codes: the nearest finite value, ties to the
    code with an even mantissa, magnitudes past 448 to 448; the sign bit is
    that of the input (so -0.0 and negatives that round to 0 give 0x80)."""
    v = np.asarray(v, np.float32).astype(np.float64)
    mag = np.minimum(np.abs(v), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, mag, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - mag
    code = np.where(d_hi < d_lo, hi, np.where(d_lo < d_hi, lo, np.where(hi % 2 == 0, hi, lo)))
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def quantize_rows_e4m3(x: np.ndarray):
    """Per-row quantisation of fp32-representable values: scale s = amax / 448
    in fp32 (1 for an all-zero row), codes = e4m3_round(x / s) with the
    division in fp32.  Returns (codes [rows, cols] uint8, s [rows] fp32)."""
    x32 = np.asarray(x, np.float64).astype(np.float32)
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return e4m3_round(x32 / s[:, None]), s


def dequantize_rows_e4m3(codes: np.ndarray, s: np.ndarray) -> np.ndarray:
    return e4m3_to_f64(codes) * np.asarray(s, np.float32).astype(np.float64)[:, None]


def expert_ffn_fp8(kind: str, codes: np.ndarray, s: np.ndarray, w1: np.ndarray, w3: Optional[np.ndarray] = None,
                   w2: Optional[np.ndarray] = None) -> np.ndarray:
    """One expert on per-row e4m3 inputs (codes, scales), float64 weights:
    the first matrix on the dequantised rows, the activation, the hidden
    layer rounded to bf16 and quantised per row, the second matrix on the
    dequantised hidden rows.  No biases."""
    xh = dequantize_rows_e4m3(codes, s)
    h = xh @ w1.T
    if kind == "linear":
        return h
    if kind == "relu":
        h = np.maximum(h, 0.0)
    elif kind == "gelu":
        h = gelu(h)
    elif kind == "swiglu":
        h = silu(h) * (xh @ w3.T)
    else:
        raise ValueError(kind)
    hq, hs = quantize_rows_e4m3(bf16_round(h))
    return dequantize_rows_e4m3(hq, hs) @ w2.T


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------


def decode_weights(raw: Dict[str, Optional[np.ndarray]], w_dtype: str, prefix: str = "") -> Dict[str, np.ndarray]:
    """Stored expert tensors -> float64 (fp8 codes times their row scales)."""
    out = {}
    for w, s in (("w1", "s1"), ("w3", "s3"), ("w2", "s2")):
        a = raw.get(prefix + w)
        if a is not None:
            out[w] = to_f64(a, w_dtype, raw.get(prefix + s))
    for b in ("b1", "b2"):
        a = raw.get(prefix + b)
        if a is not None:
            out[b] = np.asarray(a, np.float32).astype(np.float64)
    return out


def forward(x: np.ndarray, w_g: np.ndarray, b_g: Optional[np.ndarray], k: int, gate_mode: str,
            C: int, kind: str, weights: Dict[str, np.ndarray],
            shared: Optional[Dict[str, np.ndarray]] = None, alpha: float = 1.0,
            residual: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The whole layer on float64 inputs, every stage's output returned.

    Steps, in order: router logits, softmax, top-k, gates, capacity-limited
    dispatch, permute, per-expert FFN, shared experts, combine, aux loss.
    """
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    E = w_g.shape[0]
    z = router_logits(x, w_g, b_g)
    p = softmax(z)
    idx = topk_select(z, k)
    g = gates(p, idx, gate_mode)
    disp = dispatch(idx, E, C)
    xp = permute(x, disp["perm_token"])
    ye = experts_packed(kind, xp, disp["offsets"], weights)
    ys = shared_experts(kind, x, shared) if shared else None
    y = combine(ye, disp["dest_pos"], g, ys, residual)
    prob_colsum = np.sum(p, axis=0)
    loss = aux_loss(disp["counts_routed"], prob_colsum, T, k, E, alpha)
    out = {"logits": z, "probs": p, "topk_idx": idx, "topk_gate": g,
           "prob_colsum": prob_colsum, "xp": xp, "ye": ye, "ys": ys, "y": y,
           "aux_loss": loss, "near_tie": near_tie_mask(z, k)}
    out.update(disp)
    return out
