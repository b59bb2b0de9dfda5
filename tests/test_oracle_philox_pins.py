"""Pins of the oracle's counter-based normal draws (oracle/philox.py).

The generator is pinned by the known-answer vectors published with it
(tests/golden/philox4x32_kat.json: three counters and keys at 7 and at 10
rounds, so a wrong multiplier, Weyl constant, word permutation or key
schedule fails); the stream layout by the KAT block at seed 0, offset 0,
index 0; the Box-Muller normals by their distribution (a dropped factor,
a swapped u1/u2 or a wrong pairing of words fails one of them).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.stats

from oracle import philox as P


_HERE = os.path.dirname(os.path.abspath(__file__))


def _kat():
    with open(os.path.join(_HERE, "golden", "philox4x32_kat.json")) as f:
        return json.load(f)["vectors"]


@pytest.mark.parametrize("v", _kat(), ids=lambda v: f"r{v['rounds']}_{v['ctr'][0]}")
def test_known_answer_vectors(v):
    ctr = [int(h, 16) for h in v["ctr"]]
    key = [int(h, 16) for h in v["key"]]
    out = P.philox4x32(ctr, key, rounds=v["rounds"])
    assert [int(o) for o in out] == [int(h, 16) for h in v["out"]]


def test_vectorised_matches_one_at_a_time():
    # a batch of counters gives what each counter gives alone (no mixing
    # across array elements, 32-bit wrap-around of the key schedule)
    rng = np.random.default_rng(5)
    ctr = [rng.integers(0, 2 ** 32, 7, dtype=np.uint64) for _ in range(4)]
    key = (0xFFFFFFF0, 0xFFFFFFFF)
    batch = P.philox4x32(ctr, key)
    for i in range(7):
        one = P.philox4x32([c[i] for c in ctr], key)
        assert [int(b[i]) for b in batch] == [int(o) for o in one]


def test_stream_layout_at_the_first_block():
    # seed 0, offset 0: block 0 is the all-zero counter under the zero key,
    # whose words the first KAT vector gives; draws 0, 1 use words 0, 1 and
    # draws 2, 3 words 2, 3
    w = [int(h, 16) for h in _kat()[0]["out"]]
    n = P.philox_normals(0, 0, 4)
    for p in range(2):
        u1 = (w[2 * p] + 0.5) / 2 ** 32
        u2 = (w[2 * p + 1] + 0.5) / 2 ** 32
        r = math.sqrt(-2.0 * math.log(u1))
        assert n[2 * p] == pytest.approx(r * math.cos(2 * math.pi * u2), rel=1e-14, abs=1e-14)
        assert n[2 * p + 1] == pytest.approx(r * math.sin(2 * math.pi * u2), rel=1e-14, abs=1e-14)


def test_seed_and_offset_select_key_and_counter_words():
    # seed (hi, lo) is the key (lo, hi); offset (hi, lo) is counter words 2, 3
    seed = (0x299F31D0 << 32) | 0xA4093822
    offset = (0x03707344 << 32) | 0x13198A2E
    j = (0x85A308D3 << 32) | 0x243F6A88
    w = P.philox_words(seed, offset, np.array([j], np.uint64))
    assert [int(x[0]) for x in w] == [int(h, 16) for h in _kat()[2]["out"]]
    # draws start .. start + n - 1 do not depend on where the call starts
    a = P.philox_normals(seed, 7, 40)
    b = P.philox_normals(seed, 7, 13, start=27)
    np.testing.assert_array_equal(a[27:], b)


def test_normals_are_standard_normal():
    n = 1 << 20
    z = P.philox_normals(0x1234, 99, n)
    assert abs(z.mean()) < 5.0 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5.0 * math.sqrt(2.0 / n)
    assert abs(scipy.stats.kurtosis(z)) < 5.0 * math.sqrt(24.0 / n)
    assert scipy.stats.kstest(z, "norm").pvalue > 1e-4
    # even and odd draws separately (cos and sin branches)
    assert scipy.stats.kstest(z[0::2], "norm").pvalue > 1e-4
    assert scipy.stats.kstest(z[1::2], "norm").pvalue > 1e-4


def test_pairs_have_exponential_radius_and_uniform_angle():
    # Box-Muller pairs (2m, 2m + 1): squared radius -2 ln u1 ~ Exp(mean 2),
    # angle 2 pi u2 uniform, independent of each other
    z = P.philox_normals(77, 3, 1 << 18).reshape(-1, 2)
    r2 = z[:, 0] ** 2 + z[:, 1] ** 2
    ang = np.arctan2(z[:, 1], z[:, 0])
    assert scipy.stats.kstest(r2, "expon", args=(0, 2.0)).pvalue > 1e-4
    assert scipy.stats.kstest(ang, "uniform", args=(-math.pi, 2 * math.pi)).pvalue > 1e-4
    assert abs(np.corrcoef(r2, ang)[0, 1]) < 5.0 / math.sqrt(len(r2))
    # neighbouring pairs and streams are uncorrelated
    assert abs(np.corrcoef(z[:-1, 0], z[1:, 0])[0, 1]) < 5.0 / math.sqrt(len(r2))
    other = P.philox_normals(77, 4, 1 << 18)
    assert abs(np.corrcoef(z.ravel(), other)[0, 1]) < 5.0 / math.sqrt(len(other))


def test_gate_noise_is_row_major_over_tokens_and_experts():
    T, E = 5, 7
    g = P.gate_noise(11, 2, T, E)
    flat = P.philox_normals(11, 2, T * E)
    np.testing.assert_array_equal(g, flat.reshape(T, E))
