"""Seeded input generators: determinism, shapes, and the angle statistics the
method paper's mixing-window result predicts for them.

"Why Do Accumulated Transformations Extrapolate?", Sec. 3, Theorem 1 and
Example 1: for i.i.d. step angles, E cos(sum of n steps) = beta^n with
beta = E cos(phi); beta = sin(a)/a for angles uniform on [-a, a] (so beta = 0
at a = pi), and beta = exp(-sigma^2/2) for N(0, sigma^2) angles.
"""
import math

import numpy as np
import pytest

from accumulated_rotation_positional_amd import workloads as wl


def test_bf16_packing_round_trip_and_rounding():
    x = np.array([1.0, -2.5, 3.14159265, 1e-3, 65504.0, -0.0], dtype=np.float32)
    b = wl.to_bf16_bits(x)
    y = wl.from_bf16_bits(b)
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)
    # round-to-nearest-even on exact ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    tie = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)
    np.testing.assert_array_equal(wl.from_bf16_bits(wl.to_bf16_bits(tie)),
                                  np.array([1.0, 1.0 + 2.0 ** -6], dtype=np.float32))
    np.testing.assert_array_equal(wl.to_bf16_bits(y), b)


def test_alibi_slopes_geometric():
    m = wl.alibi_slopes(16)
    assert m.dtype == np.float32 and m.shape == (16,)
    assert m[0] == pytest.approx(2 ** -0.5) and m[-1] == pytest.approx(2 ** -8)
    np.testing.assert_allclose(m[1:] / m[:-1], 2 ** -0.5, rtol=1e-6)


@pytest.mark.parametrize("name", list(wl.SPECS))
def test_shapes_dtypes_and_determinism(name):
    a = wl.make(name, seqlen=64, batch=1, heads=2)
    b = wl.make(name, seqlen=64, batch=1, heads=2)
    d = wl.SPECS[name].head_dim
    assert a.q.shape == (1, 2, 64, d)
    assert a.phi.shape[2:] == (64, d // 2) and a.phi.dtype == np.float32
    assert a.q.dtype == (np.float32 if wl.SPECS[name].dtype == "f32" else np.uint16)
    for f in ("q", "k", "v", "phi"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.q, a.k)


def test_learned_angles_mixing_rate():
    """phi = W x with x ~ N(0, I_512), W ~ N(0, 0.02^2): given W, each pair's
    angle is N(0, sigma_p^2) with sigma_p^2 = sum_c W_cp^2 (about 0.2048), so
    E cos(sum of n consecutive steps) = exp(-n sigma_p^2 / 2)."""
    w = wl.make("train_1k", batch=2, heads=2, seqlen=4096)
    phi = w.phi.astype(np.float64)
    var = phi.var(axis=2).mean()
    assert var == pytest.approx(512 * 0.02 ** 2, rel=0.1)
    sig2 = phi.var(axis=2)                                   # [B, H, P] per-pair variance
    for n in (1, 4, 16):
        c = np.cumsum(phi, axis=2)
        route = c[:, :, n:, :] - c[:, :, :-n, :]             # sums of n consecutive steps
        emp = np.cos(route).mean()
        pred = np.exp(-n * sig2 / 2).mean()
        se = np.cos(route).std() / math.sqrt(route.size / n)
        assert abs(emp - pred) < 5 * se + 1e-3


def test_uniform_angles_have_zero_first_moment():
    """Example 1 at a = pi: beta = sin(pi)/pi = 0."""
    w = wl.make("farmass_32k", seqlen=4096, heads=4)
    c = np.cos(w.phi.astype(np.float64))
    assert abs(c.mean()) < 5 * c.std() / math.sqrt(c.size)
    assert w.phi.min() >= -math.pi - 1e-6 and w.phi.max() <= math.pi + 1e-6


def test_rope_angles_and_shared_table():
    w = wl.make("rope_8k_d128", batch=1, heads=2, seqlen=16)
    theta = np.power(10000.0, -2.0 * np.arange(64) / 128).astype(np.float32)
    assert np.array_equal(w.phi[0, 1, 5], theta)
    t = wl.make("tiny_f32")
    assert t.phi.shape == (1, 1, 256, 32)   # one angle stream shared by both heads
    assert t.q.dtype == np.float32 and abs(t.q.std() - 1.0) < 0.05


def test_flops_formula():
    assert wl.attn_flops(2, 8, 16384, 64) == 4 * 64 * (16384 * 16385 // 2) * 16


def test_bench_parity_row_sampling():
    """The benchmark's per-workload parity rows: valid flat row indices, each
    head present with its last (longest) row, about the requested count."""
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "bench_mod", os.path.join(os.path.dirname(os.path.dirname(__file__)), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for name in ("tiny_f32", "train_1k", "farmass_32k", "rope_8k_d128"):
        s = wl.SPECS[name]
        w = wl.make(name, batch=s.batch, heads=min(s.heads, 4), seqlen=min(s.seqlen, 4096))
        rows = bench._parity_rows(w, total=256)
        L, bh = w.seqlen, w.batch * w.heads
        assert rows.dtype == np.int64 and np.all(np.diff(rows) > 0)
        assert rows.min() >= 0 and rows.max() < bh * L
        heads = rows // L
        assert set(heads.tolist()) == set(range(bh))
        for h in range(bh):
            assert h * L + L - 1 in rows
        assert rows.size <= 256 + bh
