"""Input generators: stored formats against library conversions, determinism."""
import numpy as np
import torch

import workloads as W


def test_bf16_encoder_matches_torch_rne():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # exact ties (lower 16 bits = 0x8000) with both parities of the kept lsb
    u = rng.integers(0, 2 ** 31, size=2000, dtype=np.uint32) & np.uint32(0x7F7F0000)
    ties = (u | np.uint32(0x8000)).view(np.float32)
    a = np.concatenate([a, ties, -ties, np.array([0.0, -0.0, 1.0, 3.0e38], np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bf16_bits(a), ref)
    assert np.array_equal(W.bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_e4m3_encoder_matches_torch_in_range():
    rng = np.random.default_rng(1)
    a = (rng.standard_normal(300000) * np.exp(rng.uniform(-12, 6, 300000))).astype(np.float32)
    a = np.clip(a, -448, 448)
    # midpoints between neighbouring finite codes (ties) and the codes themselves
    vals = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    pos = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    a = np.concatenate([a, pos, -pos, mids, -mids])
    ref = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = W.f32_to_e4m3(a)
    # torch keeps the sign of zero; so do we
    assert np.array_equal(got, ref)


def test_e4m3_roundtrip_all_finite_codes_and_saturation():
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    fin = np.isfinite(vals)
    assert fin.sum() == 254
    assert np.array_equal(W.f32_to_e4m3(vals[fin]), codes[fin])
    assert W.f32_to_e4m3(np.array([1000.0, -1000.0, 470.0], np.float32)).tolist() == [0x7E, 0xFE, 0x7E]


def test_row_quantisation_scale_and_error_bound():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((64, 300)).astype(np.float32) * 0.01
    w[3] = 0.0
    q, s = W.quantize_rows_e4m3(w)
    assert s[3] == 1.0 and np.all(q[3] == 0)
    deq = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy() * s[:, None]
    rel = np.abs(deq - w) / np.max(np.abs(w), axis=1, keepdims=True).clip(1e-30)
    assert rel.max() <= 2.0 ** -4 + 1e-6            # half an e4m3 ulp at the top binade


def test_generation_is_deterministic_and_sliceable():
    cfg = W.shrink(W.DEEPSEEK, T=300, d=64, d_ff=48, E=6, k=2)
    a = W.generate(cfg)
    b = W.generate(cfg)
    for key, v in a.items():
        if v is None:
            assert b[key] is None
        else:
            assert np.array_equal(v, b[key]), key
    one = W.gen_expert(cfg, 4)
    assert np.array_equal(one["w1"], a["w1"][4])
    assert np.array_equal(W.gen_x(cfg, slice(100, 250)), a["x"][100:250])
    assert a["x"].dtype == np.uint16 and a["x"].shape == (300, 64)
    assert a["w1"].shape == (6, 48, 64) and a["w2"].shape == (6, 64, 48)
    assert a["sh_w1"].shape == (2, 48, 64)
    assert a["b_g"].shape == (6,)


def test_fp8_workload_layout():
    cfg = W.shrink(W.STRESS, T=64, d=128, d_ff=64, E=4, k=2)
    a = W.generate(cfg)
    assert a["w1"].dtype == np.uint8 and a["s1"].shape == (4, 64)
    assert a["w2"].dtype == np.uint8 and a["s2"].shape == (4, 128)
    assert a["sh_w3"].shape == (1, 64, 128)


def test_workload_table():
    assert W.CANONICAL == ("tiny", "switch", "mixtral", "deepseek", "stress")
    m = W.MIXTRAL
    assert (m.T, m.d, m.E, m.k, m.d_ff, m.ffn, m.gate) == (4096, 4096, 8, 2, 14336, "swiglu", "renorm")
    s = W.STRESS
    assert (s.T, s.d, s.E, s.k, s.n_shared, s.w_dtype, s.cf) == (32768, 7168, 256, 8, 1, "fp8", 1.0)
