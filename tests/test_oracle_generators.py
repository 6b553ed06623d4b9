"""Pins of the oracle's on-the-fly step angles (CPU only).

* Philox4x64-10 against numpy's Philox bit generator, an independent
  implementation of the same published generator (numpy advances its 256-bit
  counter by one before each block), across keys, counters and carries.
* The random variant's angles: the counter layout (a block per two positions
  of four pairs, 32 bits per element) checked with numpy's generator as the
  source of the words, and the draws are uniform on (-f_b, f_b): bounds,
  first two moments, no correlation between neighbours or between steps, zero
  bound.
* The token-table and constant sources against explicit loops.
"""
import numpy as np
import pytest

import oracle
from accumulated_rotation_positional_amd import workloads as wl

M64 = (1 << 64) - 1


def _numpy_block(counter: int, key) -> np.ndarray:
    """Philox block at the 256-bit counter value `counter` from numpy (which
    adds one to its state before producing a block)."""
    c = (counter - 1) % (1 << 256)
    words = np.array([(c >> (64 * i)) & M64 for i in range(4)], dtype=np.uint64)
    g = np.random.Philox(key=np.asarray(key, dtype=np.uint64), counter=words)
    return g.random_raw(4)


@pytest.mark.parametrize("key", [(0, 0), (5, 7), (M64, 1), (0x0123456789ABCDEF, M64)])
@pytest.mark.parametrize("counter", [0, 1, 12345, M64, (7 << 64) | 3, (1 << 255) + 99])
def test_philox_matches_numpy(counter, key):
    words = [(counter >> (64 * i)) & M64 for i in range(4)]
    got = oracle.philox4x64_10(words, key)
    assert np.array_equal(got, _numpy_block(counter, key))


@pytest.mark.parametrize("L", [5, 6])
def test_random_phi_layout_matches_numpy_words(L):
    B, G, P = 2, 3, 8
    seed, step = 0xC0FFEE, 11
    bound = np.abs(np.random.default_rng(0).standard_normal((G, P))).astype(np.float32) + 0.1
    got = oracle.random_phi(B, G, L, P, seed, step, bound)
    want = np.empty_like(got)
    half = (L + 1) // 2
    for b, g, t, p in np.ndindex(B, G, L, P):
        c = ((b * G + g) * half + t // 2) * (P // 4) + p // 4
        w = int(_numpy_block((step << 64) | c, (seed, 0))[p % 4])
        bits = (w & 0xFFFFFFFF) if t % 2 == 0 else (w >> 32)
        want[b, g, t, p] = np.float32(float(bound[g, p]) * (2.0 * bits * 2.0 ** -32 - 1.0))
    assert np.array_equal(got, want)


def test_random_phi_is_uniform_on_the_band():
    L, P = 8192, 32
    bound = wl.rope_frequencies(2 * P)[None, :]
    phi = oracle.random_phi(1, 1, L, P, 3, 0, bound)[0, 0].astype(np.float64)
    x = phi / bound[0].astype(np.float64)   # uniform on [-1, 1) per pair
    assert np.all(x >= -1.0) and np.all(x < 1.0)
    # mean 0 (sd 1/sqrt(3L)), second moment 1/3 (sd sqrt(4/45/L)), per pair
    assert np.all(np.abs(x.mean(axis=0)) < 5.0 / np.sqrt(3 * L))
    assert np.all(np.abs((x ** 2).mean(axis=0) - 1.0 / 3.0) < 5.0 * np.sqrt(4.0 / 45.0 / L))
    # neighbours in position and in pair are uncorrelated (sd of a correlation ~ 1/sqrt(n))
    for a, b in ((x[1:], x[:-1]), (x[:, 1:], x[:, :-1])):
        r = np.corrcoef(a.ravel(), b.ravel())[0, 1]
        assert abs(r) < 5.0 / np.sqrt(a.size)
    # each forward pass draws afresh
    y = oracle.random_phi(1, 1, L, P, 3, 1, bound)[0, 0] / bound[0]
    r = np.corrcoef(x.ravel(), y.ravel())[0, 1]
    assert abs(r) < 5.0 / np.sqrt(x.size)
    assert not np.array_equal(oracle.random_phi(1, 1, 64, P, 4, 0, bound),
                              oracle.random_phi(1, 1, 64, P, 3, 0, bound))


def test_random_phi_zero_bound_and_reproducible():
    z = oracle.random_phi(2, 1, 100, 16, 9, 2, np.zeros((1, 16), np.float32))
    assert np.all(z == 0.0)
    bound = np.ones((2, 16), np.float32)
    assert np.array_equal(oracle.random_phi(1, 2, 77, 16, 9, 2, bound),
                          oracle.random_phi(1, 2, 77, 16, 9, 2, bound))


def test_token_and_constant_sources():
    rng = np.random.default_rng(5)
    B, G, L, P, V = 2, 3, 7, 4, 11
    tokens = rng.integers(0, V, size=(B, L))
    table = rng.standard_normal((V, G, P)).astype(np.float32)
    got = oracle.token_phi(tokens, table)
    freq = rng.standard_normal((G, P)).astype(np.float32)
    const = oracle.constant_phi(B, L, freq)
    for b in range(B):
        for g in range(G):
            for t in range(L):
                for p in range(P):
                    assert got[b, g, t, p] == table[tokens[b, t], g, p]
                    assert const[b, g, t, p] == freq[g, p]
