"""Host-side pieces of bench.py: the algorithmic FLOP and byte counts its
roofline numbers divide by, and its refusal of more than one GPU.  No GPU
work runs here."""
import os
import subprocess
import sys

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_ffn_flops_per_kept_row():
    # two FLOPs per multiply-add: Linear d x d_out; ReLU/GELU d x d_ff then
    # d_ff x d_out; SwiGLU adds the up projection (another d x d_ff)
    m = W.MIXTRAL
    assert bench.ffn_flops_per_row(m) == 2 * (2 * 4096 * 14336) + 2 * 14336 * 4096
    s = W.SWITCH
    assert bench.ffn_flops_per_row(s) == 2 * 768 * 3072 + 2 * 3072 * 768
    assert bench.ffn_flops_per_row(W.SWITCH_GELU) == bench.ffn_flops_per_row(s)
    assert bench.ffn_flops_per_row(W.TINY) == 2 * 32 * 32
    # the Mixtral-shaped layer's 8192 kept rows: 2.886 TFLOP per grouped FFN call
    assert bench.ffn_flops_per_row(m) * 8192 == 2886218022912


def test_stage_bytes_at_the_mixtral_shape():
    b = bench.stage_bytes(W.MIXTRAL, 8192)
    T, d, E, k = 4096, 4096, 8, 2
    # router: x once, W_g once, top-k ids and gates out, column sums out
    assert b["router"] == T * d * 2 + E * d * 4 + T * k * 8 + E * 4
    # dispatch: ids in, x once, every kept row written, dest_pos and perm_token out
    assert b["dispatch"] == T * k * 4 + T * d * 2 + 8192 * d * 2 + T * k * 8
    # combine: every kept expert row read, gates and dest_pos in, y written
    assert b["combine"] == 8192 * d * 2 + T * k * 8 + T * d * 2
    # noisy gating adds the noise projection, its bias and the draws
    assert b["router_noisy"] == b["router"] + E * d * 4 + E * 4 + T * E * 4
    assert abs(b["dispatch"] - 100.8e6) < 0.1e6 and abs(b["router"] - 33.7e6) < 0.1e6


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
