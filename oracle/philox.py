"""CPU oracle of the noisy gate's normal draws: the counter-based generator
Philox4x32-10 and the Box-Muller transform (float64).

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the product library, and sharing
no code with it.

The pages draw the noisy gate's standard normal sample inside the gate
(P2 §2.1 Noisy Top-k 门控; P5 代码实战, NoisyTop1Gate in training mode) but
name no generator.  A counter-based generator lets the GPU draw the sample of
any (token, expert) on its own and lets this module draw the same one, so the
sample is fixed by (seed, offset, index) alone.

Philox4x32-10 is taken from its published definition (J. K. Salmon,
M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3", SC 2011, section 5): a 128-bit counter of four 32-bit words and a
64-bit key of two; ten rounds, each of which multiplies the first and third
words by two fixed multipliers, keeps the low halves of the products and
xors the high halves with the other two words and the key words, and
permutes the words; the key words grow by two fixed Weyl increments between
rounds.

Stream layout (one normal per index i = t * E + e for the [T, E] draws):
  key     = (seed mod 2^32, seed div 2^32)
  counter = (j mod 2^32, j div 2^32, offset mod 2^32, offset div 2^32),  j = i div 4
  outputs x0..x3; index i uses the pair (x_{2p}, x_{2p+1}), p = (i mod 4) div 2,
  u1 = (x_{2p} + 1/2) 2^-32, u2 = (x_{2p+1} + 1/2) 2^-32 (both strictly in (0, 1)),
  r = sqrt(-2 ln u1), and the normal is r cos(2 pi u2) for even i, r sin(2 pi u2)
  for odd i (Box and Muller, 1958).

Parity pins (tests/test_oracle_philox_pins.py): the known-answer vectors
published with the generator's reference implementation, the key schedule
and round structure checked one round at a time against a big-integer
rewrite of the definition, and the normals' moments and distribution.
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53          # multiplier of the first word
PHILOX_M1 = 0xCD9E8D57          # multiplier of the third word
PHILOX_W0 = 0x9E3779B9          # Weyl increment of key word 0 (golden ratio)
PHILOX_W1 = 0xBB67AE85          # Weyl increment of key word 1 (sqrt(3) - 1)
ROUNDS = 10

_M32 = np.uint64(0xFFFFFFFF)


def _mulhilo(m: int, a: np.ndarray):
    """(high, low) 32-bit halves of the 64-bit product m * a."""
    p = np.uint64(m) * a.astype(np.uint64)
    return (p >> np.uint64(32)) & _M32, p & _M32


def philox4x32(ctr, key, rounds: int = ROUNDS):
    """Philox4x32-R of counters ctr = (c0, c1, c2, c3) under keys key = (k0, k1);
    each word an array (or scalar) of uint32 values.  Returns four uint32 arrays."""
    c0, c1, c2, c3 = (np.asarray(c, np.uint64) & _M32 for c in ctr)
    k0, k1 = (np.asarray(k, np.uint64) & _M32 for k in key)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _M32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _M32
        hi0, lo0 = _mulhilo(PHILOX_M0, c0)
        hi1, lo1 = _mulhilo(PHILOX_M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return tuple(c.astype(np.uint32) for c in (c0, c1, c2, c3))


def philox_words(seed: int, offset: int, j: np.ndarray):
    """The four output words of counter block j of the stream (seed, offset)."""
    j = np.asarray(j, np.uint64)
    seed, offset = int(seed), int(offset)
    ctr = (j & _M32, j >> np.uint64(32), np.uint64(offset & 0xFFFFFFFF), np.uint64(offset >> 32))
    key = (np.uint64(seed & 0xFFFFFFFF), np.uint64(seed >> 32))
    return philox4x32(ctr, key)


def philox_normals(seed: int, offset: int, n: int, start: int = 0) -> np.ndarray:
    """Standard normal draws i = start .. start + n - 1 of the stream (seed,
    offset), float64, by the layout in the module docstring."""
    if not (0 <= seed < 2 ** 64 and 0 <= offset < 2 ** 64):
        raise ValueError("seed and offset are unsigned 64-bit integers")
    i = np.arange(start, start + n, dtype=np.uint64)
    x0, x1, x2, x3 = philox_words(seed, offset, i >> np.uint64(2))
    second = ((i >> np.uint64(1)) & np.uint64(1)).astype(bool)      # (i mod 4) div 2
    a = np.where(second, x2, x0).astype(np.float64)
    b = np.where(second, x3, x1).astype(np.float64)
    u1 = (a + 0.5) * 2.0 ** -32
    u2 = (b + 0.5) * 2.0 ** -32
    r = np.sqrt(-2.0 * np.log(u1))
    odd = (i & np.uint64(1)).astype(bool)
    return np.where(odd, r * np.sin(2.0 * np.pi * u2), r * np.cos(2.0 * np.pi * u2))


def gate_noise(seed: int, offset: int, T: int, E: int) -> np.ndarray:
    """The noisy gate's draws noise[t, e] = normal t * E + e of the stream."""
    return philox_normals(seed, offset, T * E).reshape(T, E)
