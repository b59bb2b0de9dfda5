"""ctypes binding of libmoe.so: one Python function per C entry point.

Argument marshalling only: tensors are passed as device pointers, the
stream is torch's current stream, and a negative status raises MoEError.
The library must have been built (``python -m
sparse_mixture_experts_atomic_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

# moe_dtype
F32, BF16, FP8_E4M3 = 0, 1, 2
# moe_gate_mode
GATE_PROB, GATE_RENORM = 0, 1
# moe_ffn_kind
FFN_LINEAR, FFN_RELU, FFN_SWIGLU, FFN_GELU = 0, 1, 2, 3
# moe_cap_round
CAP_CEIL, CAP_FLOOR = 0, 1
# moe_row_mode
ROWS_PACKED, ROWS_SHARED = 0, 1
# moe_status
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE, ERR_SCRATCH_LIMIT = 0, -1, -2, -3, -4, -5
# fixed scratch of the allocation-free router (MOE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 16 << 20

GATE_MODES = {"prob": GATE_PROB, "renorm": GATE_RENORM}
CAP_ROUNDS = {"ceil": CAP_CEIL, "floor": CAP_FLOOR}
FFN_KINDS = {"linear": FFN_LINEAR, "relu": FFN_RELU, "swiglu": FFN_SWIGLU, "gelu": FFN_GELU}

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_f = ctypes.c_float
_u64 = ctypes.c_uint64

_SIGS = {
    "moe_abi_version": (_i, []),
    "moe_status_string": (ctypes.c_char_p, [_i]),
    "moe_last_hip_error": (_i, []),
    "moe_capacity": (_i, [_i, _i, _i, ctypes.c_double, _i]),
    "moe_router_workspace_size": (_sz, [_i, _i, _i, _i]),
    "moe_router_topk": (_i, [_vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_router_topk_noalloc": (_i, [_vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "moe_router_noisy_workspace_size": (_sz, [_i, _i, _i, _i]),
    "moe_router_topk_noisy": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _vp, _f, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp,
                                   _vp, _sz, _vp]),
    "moe_router_topk_noisy_philox": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _u64, _u64, _f, _i, _i, _i, _i, _i, _vp,
                                          _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_gate_noise_philox": (_i, [_u64, _u64, _sz, _vp, _vp]),
    "moe_dispatch_workspace_size": (_sz, [_i, _i, _i]),
    "moe_dispatch_permute": (_i, [_vp, _i, _i, _i, _i, _vp, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_ffn_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "moe_expert_ffn_grouped": (_i, [_i, _vp, _i, _i, _i, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _i,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_expert_ffn_gathered": (_i, [_i, _vp, _i, _i, _vp, _i, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _i,
                                     _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_combine": (_i, [_vp, _i, _vp, _vp, _i, _i, _i, _vp, _i, _vp, _vp, _vp]),
    "moe_aux_loss": (_i, [_vp, _vp, _i, _i, _i, _f, _vp, _vp]),
    "moe_aux_loss_from_router": (_i, [_vp, _vp, _sz, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp]),
    "moe_quantize_rows_e4m3": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp]),
    "moe_ffn_fp8_workspace_size": (_sz, [_i, _i, _i, _i]),
    "moe_expert_ffn_fp8": (_i, [_i, _vp, _vp, _i, _vp, _i, _i, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp, _sz, _vp]),
    "moe_combine_backward": (_i, [_vp, _i, _vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp]),
    "moe_ffn_backward_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "moe_expert_ffn_grouped_backward": (_i, [_i, _vp, _i, _i, _i, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _i,
                                             _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_expert_ffn_grouped_train": (_i, [_i, _vp, _i, _i, _i, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _i, _vp, _vp,
                                          _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_ffn_backward_kept_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "moe_expert_ffn_grouped_backward_kept": (_i, [_i, _vp, _i, _i, _i, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _i,
                                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                                  _vp]),
    "moe_router_backward_workspace_size": (_sz, [_i, _i, _i]),
    "moe_router_backward": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _f, _vp, _vp, _vp,
                                 _vp, _sz, _vp]),
    "moe_permute_backward": (_i, [_vp, _i, _vp, _i, _i, _i, _vp, _i, _vp, _vp, _vp, _i, _vp, _vp]),
}

_lib = None


class MoEError(RuntimeError):
    def __init__(self, name: str, status: int):
        msg = lib().moe_status_string(status).decode()
        if status == ERR_HIP:
            msg += f" (hipError {lib().moe_last_hip_error()})"
        super().__init__(f"{name}: {msg}")
        self.status = status


def lib():
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_mixture_experts_atomic_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(name: str, st: int):
    if st != OK:
        raise MoEError(name, st)


def capacity(T: int, k: int, E: int, cf: Optional[float], round_mode=CAP_CEIL) -> int:
    """moe_capacity: C >= 0, or -1 (no limit) when cf is None or <= 0.
    round_mode is CAP_CEIL / CAP_FLOOR or their names 'ceil' / 'floor'."""
    if isinstance(round_mode, str):
        round_mode = CAP_ROUNDS[round_mode]
    if T < 0 or k < 1 or E < 1:
        raise ValueError("moe_capacity needs T >= 0, k >= 1 and E >= 1")
    return lib().moe_capacity(T, k, E, 0.0 if cf is None else float(cf), round_mode)


def router_workspace_size(T, d, E, x_dt) -> int:
    return lib().moe_router_workspace_size(T, d, E, x_dt)


def dispatch_workspace_size(T, k, E) -> int:
    return lib().moe_dispatch_workspace_size(T, k, E)


def ffn_workspace_size(kind, act_dt, max_rows, E, d, d_ff, d_out) -> int:
    return lib().moe_ffn_workspace_size(kind, act_dt, max_rows, E, d, d_ff, d_out)


def router_topk(x, w_g, b_g, k, gate_mode, topk_idx, topk_gate, prob_colsum=None, logits_dbg=None,
                workspace=None, stream=None):
    T, d = x.shape
    E = w_g.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().moe_router_topk(_p(x), dtype_code(x), _p(w_g), _p(b_g), T, d, E, k, gate_mode,
                               _p(topk_idx), _p(topk_gate), _p(prob_colsum), _p(logits_dbg),
                               _p(workspace), ws_bytes, _stream(stream))
    _check("moe_router_topk", st)


def router_topk_noalloc(x, w_g, b_g, k, gate_mode, topk_idx, topk_gate, prob_colsum=None, logits_dbg=None,
                        stream=None):
    """moe_router_topk_noalloc: moe_router_topk with the library's fixed scratch."""
    T, d = x.shape
    E = w_g.shape[0]
    st = lib().moe_router_topk_noalloc(_p(x), dtype_code(x), _p(w_g), _p(b_g), T, d, E, k, gate_mode,
                                       _p(topk_idx), _p(topk_gate), _p(prob_colsum), _p(logits_dbg),
                                       _stream(stream))
    _check("moe_router_topk_noalloc", st)


def router_noisy_workspace_size(T, d, E, x_dt) -> int:
    return lib().moe_router_noisy_workspace_size(T, d, E, x_dt)


def router_topk_noisy(x, w_g, b_g, w_n, b_n, noise, noise_eps, k, gate_mode, topk_idx, topk_gate,
                      prob_colsum=None, logits_dbg=None, workspace=None, stream=None):
    T, d = x.shape
    E = w_g.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().moe_router_topk_noisy(_p(x), dtype_code(x), _p(w_g), _p(b_g), _p(w_n), _p(b_n), _p(noise),
                                     float(noise_eps), T, d, E, k, gate_mode, _p(topk_idx), _p(topk_gate),
                                     _p(prob_colsum), _p(logits_dbg), _p(workspace), ws_bytes, _stream(stream))
    _check("moe_router_topk_noisy", st)


def router_topk_noisy_philox(x, w_g, b_g, w_n, b_n, seed, offset, noise_eps, k, gate_mode, topk_idx, topk_gate,
                             prob_colsum=None, logits_dbg=None, workspace=None, stream=None):
    T, d = x.shape
    E = w_g.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().moe_router_topk_noisy_philox(_p(x), dtype_code(x), _p(w_g), _p(b_g), _p(w_n), _p(b_n), int(seed),
                                            int(offset), float(noise_eps), T, d, E, k, gate_mode, _p(topk_idx),
                                            _p(topk_gate), _p(prob_colsum), _p(logits_dbg), _p(workspace), ws_bytes,
                                            _stream(stream))
    _check("moe_router_topk_noisy_philox", st)


def gate_noise_philox(seed, offset, out, stream=None):
    st = lib().moe_gate_noise_philox(int(seed), int(offset), out.numel(), _p(out), _stream(stream))
    _check("moe_gate_noise_philox", st)


def dispatch_permute(topk_idx, E, capacity_, x, x_perm, counts_routed, counts_kept, offsets, dest_pos,
                     perm_token, workspace, stream=None):
    T, k = topk_idx.shape
    d = x.shape[1] if x is not None else 0
    x_dt = dtype_code(x) if x is not None else BF16
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().moe_dispatch_permute(_p(topk_idx), T, k, E, capacity_, _p(x), x_dt, d, _p(x_perm),
                                    _p(counts_routed), _p(counts_kept), _p(offsets), _p(dest_pos),
                                    _p(perm_token), _p(workspace), ws_bytes, _stream(stream))
    _check("moe_dispatch_permute", st)


def expert_ffn_grouped(kind, x_rows, max_rows, row_mode, offsets, E, d, d_ff, d_out, w1, w3, w2,
                       s1, s3, s2, b1, b2, y_rows, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().moe_expert_ffn_grouped(kind, _p(x_rows), dtype_code(x_rows), max_rows, row_mode, _p(offsets),
                                      E, d, d_ff, d_out, _p(w1), _p(w3), _p(w2), dtype_code(w1),
                                      _p(s1), _p(s3), _p(s2), _p(b1), _p(b2), _p(y_rows), _p(workspace),
                                      ws_bytes, _stream(stream))
    _check("moe_expert_ffn_grouped", st)


def expert_ffn_gathered(kind, x, perm_token, max_rows, offsets, E, d, d_ff, d_out, w1, w3, w2,
                        s1, s3, s2, b1, b2, y_rows, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().moe_expert_ffn_gathered(kind, _p(x), dtype_code(x), x.shape[0], _p(perm_token), max_rows, _p(offsets),
                                       E, d, d_ff, d_out, _p(w1), _p(w3), _p(w2), dtype_code(w1),
                                       _p(s1), _p(s3), _p(s2), _p(b1), _p(b2), _p(y_rows), _p(workspace),
                                       ws_bytes, _stream(stream))
    _check("moe_expert_ffn_gathered", st)


def combine(y_rows, dest_pos, topk_gate, d_out, shared_y, n_shared, residual, y, stream=None):
    T, k = dest_pos.shape
    st = lib().moe_combine(_p(y_rows), dtype_code(y_rows), _p(dest_pos), _p(topk_gate), T, k, d_out,
                           _p(shared_y), n_shared, _p(residual), _p(y), _stream(stream))
    _check("moe_combine", st)


def aux_loss(counts_routed, prob_colsum, T, k, E, alpha, loss, stream=None):
    st = lib().moe_aux_loss(_p(counts_routed), _p(prob_colsum), T, k, E, float(alpha), _p(loss),
                            _stream(stream))
    _check("moe_aux_loss", st)


def aux_loss_from_router(counts_routed, router_workspace, T, d, E, x_dt, noisy, k, alpha, loss, prob_colsum,
                         stream=None):
    ws_bytes = router_workspace.numel() * router_workspace.element_size()
    st = lib().moe_aux_loss_from_router(_p(counts_routed), _p(router_workspace), ws_bytes, T, d, E, x_dt,
                                        1 if noisy else 0, k, float(alpha), _p(prob_colsum), _p(loss),
                                        _stream(stream))
    _check("moe_aux_loss_from_router", st)


# ---------------------------------------------------------------- backward


def combine_backward(dy, y_rows, dest_pos, topk_gate, dy_rows, dgate, stream=None):
    T, k = dest_pos.shape
    st = lib().moe_combine_backward(_p(dy), dtype_code(dy), _p(y_rows), _p(dest_pos), _p(topk_gate), T, k,
                                    dy.shape[1], _p(dy_rows), _p(dgate), _stream(stream))
    _check("moe_combine_backward", st)


def ffn_backward_workspace_size(kind, max_rows, E, d, d_ff, d_out) -> int:
    return lib().moe_ffn_backward_workspace_size(kind, max_rows, E, d, d_ff, d_out)


def expert_ffn_grouped_backward(kind, x_rows, max_rows, row_mode, offsets, E, d, d_ff, d_out, w1, w3, w2, b1, b2,
                                dy_rows, dx_rows, dw1, dw3, dw2, db1, db2, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().moe_expert_ffn_grouped_backward(kind, _p(x_rows), dtype_code(x_rows), max_rows, row_mode, _p(offsets),
                                               E, d, d_ff, d_out, _p(w1), _p(w3), _p(w2), dtype_code(w1), _p(b1),
                                               _p(b2), _p(dy_rows), _p(dx_rows), _p(dw1), _p(dw3), _p(dw2), _p(db1),
                                               _p(db2), _p(workspace), ws_bytes, _stream(stream))
    _check("moe_expert_ffn_grouped_backward", st)


def expert_ffn_grouped_train(kind, x_rows, max_rows, row_mode, offsets, E, d, d_ff, d_out, w1, w3, w2, b1, b2,
                             y_rows, h1, h3, workspace, stream=None) -> bool:
    """Training forward keeping the first product's fp32 pre-activations in
    h1 (h3); False (nothing written) where the library does not take the
    shape, and moe_expert_ffn_grouped must run instead."""
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().moe_expert_ffn_grouped_train(kind, _p(x_rows), dtype_code(x_rows), max_rows, row_mode, _p(offsets), E,
                                            d, d_ff, d_out, _p(w1), _p(w3), _p(w2), dtype_code(w1), _p(b1), _p(b2),
                                            _p(y_rows), _p(h1), _p(h3), _p(workspace), ws_bytes, _stream(stream))
    if st == ERR_UNSUPPORTED:
        return False
    _check("moe_expert_ffn_grouped_train", st)
    return True


def ffn_backward_kept_workspace_size(kind, max_rows, E, d, d_ff, d_out) -> int:
    return lib().moe_ffn_backward_kept_workspace_size(kind, max_rows, E, d, d_ff, d_out)


def expert_ffn_grouped_backward_kept(kind, x_rows, max_rows, row_mode, offsets, E, d, d_ff, d_out, w1, w3, w2, b1,
                                     b2, h1, h3, dy_rows, dx_rows, dw1, dw3, dw2, db1, db2, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().moe_expert_ffn_grouped_backward_kept(kind, _p(x_rows), dtype_code(x_rows), max_rows, row_mode,
                                                    _p(offsets), E, d, d_ff, d_out, _p(w1), _p(w3), _p(w2),
                                                    dtype_code(w1), _p(b1), _p(b2), _p(h1), _p(h3), _p(dy_rows),
                                                    _p(dx_rows), _p(dw1), _p(dw3), _p(dw2), _p(db1), _p(db2),
                                                    _p(workspace), ws_bytes, _stream(stream))
    _check("moe_expert_ffn_grouped_backward_kept", st)


def router_backward_workspace_size(T, d, E) -> int:
    return lib().moe_router_backward_workspace_size(T, d, E)


def router_backward(x, logits, topk_idx, topk_gate, dgate, counts_routed, gate_mode, alpha, daux, dz, dw_g, db_g,
                    workspace, stream=None):
    T, d = x.shape
    E = logits.shape[1]
    k = topk_idx.shape[1]
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().moe_router_backward(_p(x), dtype_code(x), _p(logits), _p(topk_idx), _p(topk_gate), _p(dgate),
                                   _p(counts_routed), T, d, E, k, gate_mode, float(alpha), float(daux), _p(dz),
                                   _p(dw_g), _p(db_g), _p(workspace), ws_bytes, _stream(stream))
    _check("moe_router_backward", st)


def permute_backward(dx_rows, dest_pos, d, dx_shared, n_shared, dres, dz, w_g, dx, stream=None):
    T, k = dest_pos.shape
    E = w_g.shape[0] if w_g is not None else 0
    st = lib().moe_permute_backward(_p(dx_rows), dtype_code(dx_rows), _p(dest_pos), T, k, d, _p(dx_shared), n_shared,
                                    _p(dres), _p(dz), _p(w_g), E, _p(dx), _stream(stream))
    _check("moe_permute_backward", st)


# ---------------------------------------------------------------- fp8 activations


def quantize_rows_e4m3(x, q, scale, stream=None):
    rows, cols = x.shape
    st = lib().moe_quantize_rows_e4m3(_p(x), dtype_code(x), rows, cols, _p(q), _p(scale), _stream(stream))
    _check("moe_quantize_rows_e4m3", st)


def ffn_fp8_workspace_size(kind, max_rows, E, d_ff) -> int:
    return lib().moe_ffn_fp8_workspace_size(kind, max_rows, E, d_ff)


def expert_ffn_fp8(kind, xq, x_scale, gather, row_mode, max_rows, offsets, E, d, d_ff, d_out, w1, w3, w2, s1, s3, s2,
                   y_rows, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().moe_expert_ffn_fp8(kind, _p(xq), _p(x_scale), xq.shape[0], _p(gather), row_mode, max_rows, _p(offsets),
                                  E, d, d_ff, d_out, _p(w1), _p(w3), _p(w2), _p(s1), _p(s3), _p(s2), _p(y_rows),
                                  _p(workspace), ws_bytes, _stream(stream))
    _check("moe_expert_ffn_fp8", st)
