"""GPU parity of the whole forward pass (scan + rotation + attention) against
the fp64 oracle on identical seeded inputs.

Bars: bf16 I/O max |error| <= 2e-2 (and rms error <= 1% of the output's rms);
fp32 I/O max |error| <= 1e-4.  Small problems are compared element by element
on every output; the five full-size workloads are compared on sampled rows
(tile edges, the first and last rows, random rows of every head), in the same
launch configuration the benchmark times."""
import dataclasses

import numpy as np
import pytest
import torch

from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import (assert_close, circular_err, oracle_flags, oracle_problem, run_forward,
                      sample_rows, say, to_dev, to_host)
import oracle

pytestmark = pytest.mark.gpu

FLAG_SETS = [
    dict(rotate_qk=True, rotate_v=False, alibi=False),
    dict(rotate_qk=True, rotate_v=True, alibi=False),
    dict(rotate_qk=True, rotate_v=True, alibi=True),
    dict(rotate_qk=True, rotate_v=False, alibi=True),
    dict(rotate_qk=False, rotate_v=False, alibi=False),
    dict(rotate_qk=False, rotate_v=True, alibi=False),
    dict(rotate_qk=True, rotate_v=True, alibi=False, exclusive=True),
]


def _dt(w):
    return "f32" if w.q.dtype == np.float32 else "bf16"


def _as_f32(w):
    """The same workload with fp32 q/k/v (the exact values of the bf16 draws)."""
    for n in ("q", "k", "v"):
        setattr(w, n, w.values(n).copy())
    return w


def _ids(fs):
    return "-".join(k for k, v in fs.items() if v) or "nope"


@pytest.mark.parametrize("flags", FLAG_SETS, ids=[_ids(f) for f in FLAG_SETS])
@pytest.mark.parametrize("name,L", [("train_1k", 333), ("rope_8k_d128", 200), ("tiny_f32", 256),
                                    ("tiny_f32", 97)])
def test_small_all_flags(name, L, flags):
    w = wl.make(name, batch=2, heads=3, seqlen=L)
    got, theta = run_forward(w, **flags)
    want = oracle_problem(w, **flags).output()
    assert_close(got, want, _dt(w), f"{name} L={L} {flags}")
    th_ref = oracle.angle_scan(w.phi, exclusive=flags.get("exclusive", False))
    assert circular_err(theta, th_ref) <= 1e-4


@pytest.mark.parametrize("L", [1, 2, 3, 33, 65, 130])
def test_fp32_ragged_lengths(L):
    """fp32 I/O at lengths that leave some of a query's key lanes
    without keys (query 0 has one key) and tiles part-filled."""
    w = wl.make("tiny_f32", batch=1, heads=2, seqlen=L)
    flags = dict(rotate_qk=True, rotate_v=True, alibi=True)
    got, _ = run_forward(w, **flags)
    assert_close(got, oracle_problem(w, **flags).output(), "f32", f"fp32 L={L}")


@pytest.mark.parametrize("heads,L", [(8, 1100), (2, 1100)])
def test_fp32_lane_splits(heads, L):
    """The fp32 kernel splits each query's keys over 4 lanes on grids of at
    least one 64-query workgroup per compute unit (2 x 8 heads x 18 tiles =
    288 here) and over 32 lanes below that (2 x 2 x 18 = 72): both against the
    oracle, ragged length, every flag that changes the kernel."""
    w = wl.make("tiny_f32", batch=2, heads=heads, seqlen=L)
    flags = dict(rotate_qk=True, rotate_v=True, alibi=True)
    got, _ = run_forward(w, **flags)
    rows = sample_rows(w, per_head=24)
    want = oracle_problem(w, **flags).rows(rows)
    assert_close(got.reshape(-1, w.head_dim)[rows], want, "f32", f"fp32 lane split H={heads} L={L}")


@pytest.mark.parametrize("flags", FLAG_SETS[:3], ids=[_ids(f) for f in FLAG_SETS[:3]])
def test_fp32_head_dim_128(flags):
    w = _as_f32(wl.make("rope_8k_d128", batch=1, heads=2, seqlen=150))
    w.phi = wl.make("train_1k", batch=1, heads=2, seqlen=150).phi.repeat(2, axis=3)
    got, _ = run_forward(w, **flags)
    want = oracle_problem(w, **flags).output()
    assert_close(got, want, "f32", f"fp32 d=128 {flags}")


@pytest.mark.parametrize("L", [1, 2, 31, 64, 65, 255, 256, 257, 511, 700])
@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_ragged_lengths(name, L):
    w = wl.make(name, batch=1, heads=2, seqlen=L)
    got, _ = run_forward(w, rotate_v=True, alibi=True)
    want = oracle_problem(w, rotate_v=True, alibi=True).output()
    assert_close(got, want, _dt(w), f"{name} L={L}")


def test_shared_angle_heads_bf16():
    w = wl.make("train_1k", batch=2, heads=4, seqlen=300)
    w.phi = np.ascontiguousarray(w.phi[:, :1])
    got, _ = run_forward(w, rotate_v=True)
    want = oracle_problem(w, rotate_v=True).output()
    assert_close(got, want, "bf16", "shared phi")


def test_large_logits_bf16():
    """Peaked softmax: inputs scaled so logits reach tens of units (the lazy
    rescale of the running maximum is exercised)."""
    w = wl.make("train_1k", batch=1, heads=2, seqlen=1000)
    x = wl.from_bf16_bits(w.q) * np.float32(16.0)
    w.q = wl.to_bf16_bits(x)
    x = wl.from_bf16_bits(w.k) * np.float32(16.0)
    w.k = wl.to_bf16_bits(x)
    got, _ = run_forward(w, rotate_v=True)
    want = oracle_problem(w, rotate_v=True).output()
    max_abs = float(np.abs(got - want).max())
    say(f"[gpu] large logits max_abs={max_abs:.3e}")
    assert max_abs <= 2e-2 * max(1.0, float(np.abs(want).max()))


@pytest.mark.parametrize("heads,L", [(2, 2000), (16, 16384)])
def test_growing_key_norms_rescale_on_late_tiles(heads, L):
    """Keys whose norm grows along the sequence (x1 at key 0 to x12 at the
    end) and queries scaled by 16: each row's largest logits sit near its own
    position, so the running maximum must be raised on late key tiles, and a
    bound from the largest key norm never clears the rescale threshold after
    the first tile -- the per-tile bound has to keep running.  2 heads at 2000
    tokens take the 128-query workgroups; 16 heads at 16384 the 512-query ones
    (sampled rows)."""
    w = wl.make("train_1k", batch=1, heads=heads, seqlen=L)
    grow = (1.0 + 11.0 * np.arange(L, dtype=np.float32) / L)[None, None, :, None]
    w.k = wl.to_bf16_bits(wl.from_bf16_bits(w.k) * grow)
    w.q = wl.to_bf16_bits(wl.from_bf16_bits(w.q) * np.float32(16.0))
    got, _ = run_forward(w, rotate_v=True)
    prob = oracle_problem(w, rotate_v=True)
    if heads * L > 100_000:
        rows = sample_rows(w, per_head=8)
        got, want = got.reshape(-1, w.head_dim)[rows], prob.rows(rows)
    else:
        want = prob.output()
    max_abs = float(np.abs(got - want).max())
    say(f"[gpu] growing key norms H={heads} L={L}: max_abs={max_abs:.3e}")
    assert np.all(np.isfinite(got))
    assert max_abs <= 2e-2 * max(1.0, float(np.abs(want).max()))


@pytest.mark.parametrize("name", list(wl.SPECS))
def test_full_size_workload_sampled_rows(name):
    w = wl.make(name)
    got, theta = run_forward(w)
    assert np.all(np.isfinite(got))
    rows = sample_rows(w)
    prob = oracle_problem(w)
    want = prob.rows(rows)
    sel = got.reshape(-1, w.head_dim)[rows]
    assert_close(sel, want, _dt(w), f"{name} full size, {rows.size} sampled rows")
    assert circular_err(theta, oracle.angle_scan(w.phi)) <= 1e-4


def test_rope_workload_matches_closed_form_rope():
    """RoPE special case: constant angles theta_p; the attention output equals
    the one computed with the closed-form position angles t * theta_p
    (AdaRoPE eq. (8): only position differences matter)."""
    w = wl.make("rope_8k_d128", batch=1, heads=2, seqlen=512)
    got, _ = run_forward(w)
    # oracle with position angles t*theta_p fed as an exclusive scan of constant steps
    want = oracle_problem(w, exclusive=True).output()
    assert_close(got, want, "bf16", "rope vs closed form")


# ---- rotation fused into the attention kernel's staging (ARP_FUSED_ROTATION) ----

@pytest.mark.parametrize("flags", FLAG_SETS, ids=[_ids(f) for f in FLAG_SETS])
@pytest.mark.parametrize("name,L", [("train_1k", 333), ("rope_8k_d128", 200), ("train_1k", 64)])
def test_fused_rotation_all_flags(name, L, flags):
    w = wl.make(name, batch=2, heads=3, seqlen=L)
    got, theta = run_forward(w, fused=True, **flags)
    want = oracle_problem(w, **flags).output()
    assert_close(got, want, "bf16", f"fused {name} L={L} {flags}")


@pytest.mark.parametrize("L", [1, 31, 65, 257, 700])
@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_fused_rotation_ragged(name, L):
    w = wl.make(name, batch=1, heads=2, seqlen=L)
    got, _ = run_forward(w, rotate_v=True, alibi=True, fused=True)
    want = oracle_problem(w, rotate_v=True, alibi=True).output()
    assert_close(got, want, "bf16", f"fused {name} L={L}")


@pytest.mark.parametrize("name", ["extrap_16k", "farmass_32k", "rope_8k_d128"])
def test_fused_rotation_full_size_sampled_rows(name):
    """The fused variant at full size, compared with the oracle on sampled rows
    and with the pre-rotation path on every output."""
    w = wl.make(name)
    got, _ = run_forward(w, fused=True)
    rows = sample_rows(w, per_head=12)
    want = oracle_problem(w).rows(rows)
    assert_close(got.reshape(-1, w.head_dim)[rows], want, "bf16", f"fused {name} sampled rows")
    ref, _ = run_forward(w)
    d = float(np.abs(got - ref).max())
    say(f"[gpu] fused vs pre-rotated {name}: max |diff| = {d:.3e}")
    assert d <= 2e-2


@pytest.mark.parametrize("alibi", [False, True])
def test_million_token_sequence_sampled_rows(alibi):
    """2^20 tokens in one head (64x the longest workload): every index product
    the kernels form past 2^31 elements-times-bytes is exercised; sampled rows
    (tile edges, the last rows) against the oracle.  The distance bias takes
    one gentle slope so the walk is long."""
    w = wl.make("farmass_32k", batch=1, heads=1, seqlen=1 << 20)
    w.alibi = np.array([2.0 ** -12], dtype=np.float32)
    got, _ = run_forward(w, rotate_v=True, alibi=alibi)
    rows = sample_rows(w, per_head=16)
    want = oracle_problem(w, rotate_v=True, alibi=alibi).rows(rows)
    assert_close(got.reshape(-1, w.head_dim)[rows], want, "bf16", f"2^20 tokens alibi={alibi}")


@pytest.mark.parametrize("name,heads,L,rotate_v", [("train_1k", 32, 2000, False),
                                                   ("train_1k", 32, 2000, True),
                                                   ("rope_8k_d128", 32, 2000, False)])
def test_paired_small_shape_matches_unpaired(name, heads, L, rotate_v):
    """The 4 waves x 32 queries shape pairs the c-th longest and c-th
    shortest query tiles in one workgroup when the pairs still fill every CU
    (tiles / 2 >= 256 on an MI355X), the walks are at most 8192 keys and the
    tile count is a multiple of 16: 32 heads at 2000 tokens make 32 x 16 = 512
    tiles of 128 queries (ragged: the last tile holds 80).  Three of those
    heads alone (48 tiles) take the unpaired launch.  Every row is computed
    the same way in both, so they must agree bit for bit, log-sum-exp too;
    the paired run is also checked against the oracle on sampled rows."""
    w = wl.make(name, batch=1, heads=heads, seqlen=L)

    def run(x):
        say(f"[gpu] paired small shape {name} H={x.heads} L={x.seqlen} v={rotate_v}")
        o, _, lse = binding.forward_ex(to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.phi),
                                       rotate_v=rotate_v, with_lse=True)
        torch.cuda.synchronize()
        return to_host(o), lse.cpu().numpy()

    got, lse = run(w)
    rows = sample_rows(w, per_head=6)
    want = oracle.Problem(w.q, w.k, w.v, w.phi, oracle_flags(True, rotate_v, False)).rows(rows)
    assert_close(got.reshape(-1, w.head_dim)[rows], want, "bf16", f"paired 4x32, {name} L={L}")
    part = dataclasses.replace(w, heads=3, **{n: np.ascontiguousarray(getattr(w, n)[:, :3])
                                              for n in ("q", "k", "v", "phi")})
    small, lse_small = run(part)
    assert np.array_equal(small, got[:, :3]), float(np.abs(small - got[:, :3]).max())
    assert np.array_equal(lse_small, lse[:, :3])


@pytest.mark.parametrize("rotate_v", [False, True])
def test_fused_paired_small_shape_matches_unpaired(rotate_v):
    """With the rotation fused into the staging, d=64 grids that miss the
    512-query rule take 4 waves x 32 queries, paired by the same rule as the
    pre-rotation path: 32 heads at 2000 tokens (512 tiles) pair, three of
    those heads alone do not.  Rows are computed the same way in both: bit for
    bit, and the paired run against the oracle on sampled rows."""
    w = wl.make("train_1k", batch=1, heads=32, seqlen=2000)
    got, _ = run_forward(w, rotate_v=rotate_v, fused=True)
    rows = sample_rows(w, per_head=6)
    want = oracle_problem(w, rotate_v=rotate_v).rows(rows)
    assert_close(got.reshape(-1, w.head_dim)[rows], want, "bf16", "fused paired 4x32")
    part = dataclasses.replace(w, heads=3, **{n: np.ascontiguousarray(getattr(w, n)[:, :3])
                                              for n in ("q", "k", "v", "phi")})
    small, _ = run_forward(part, rotate_v=rotate_v, fused=True)
    assert np.array_equal(small, got[:, :3]), float(np.abs(small - got[:, :3]).max())


@pytest.mark.parametrize("name,heads,L,rotate_v", [("train_1k", 16, 16400, False),
                                                   ("train_1k", 16, 16400, True),
                                                   ("train_1k", 17, 16896, True),
                                                   ("rope_8k_d128", 32, 8200, False)])
def test_workgroup_shapes_agree_on_a_ragged_length(name, heads, L, rotate_v):
    """The d=64 attention takes 512-query workgroups (8 waves x 64 queries)
    for unbiased walks over at least 4096 tokens whose 512-query grid fills
    every CU twice, and 128-query workgroups (4 waves x 32 queries, two per
    CU) otherwise.  16 heads at 16400 tokens (16400 = 256*64 + 16, a ragged
    16-key tail; 528 workgroups of 512) take the first; three of those heads
    alone take the second.  Every row is computed the same way in both, so
    the three heads must agree bit for bit, log-sum-exp too; the big run is
    also checked against the oracle on sampled rows.  The 512-query shape
    pairs the c-th longest and c-th shortest query tiles in one workgroup
    when the tile count is a multiple of 16 (16 x 33 = 528 tiles); 17 heads
    at 16896 tokens make 561 tiles, the unpaired launch.  At d=128 the shapes are
    8 waves x 32 queries (unbiased grids of at least four 256-query
    workgroups per CU: 32 heads at 8200 tokens make 1056) and 4 waves x 32."""
    w = wl.make(name, batch=1, heads=heads, seqlen=L)

    def run(x):
        say(f"[gpu] shapes H={x.heads} L={x.seqlen} v={rotate_v}")
        o, _, lse = binding.forward_ex(to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.phi),
                                       rotate_v=rotate_v, with_lse=True)
        torch.cuda.synchronize()
        return to_host(o), lse.cpu().numpy()

    got, lse = run(w)
    rows = sample_rows(w, per_head=6)
    want = oracle.Problem(w.q, w.k, w.v, w.phi, oracle_flags(True, rotate_v, False)).rows(rows)
    assert_close(got.reshape(-1, w.head_dim)[rows], want, "bf16", f"8-wave shape, {name} L={L}")
    part = dataclasses.replace(w, heads=3, **{n: np.ascontiguousarray(getattr(w, n)[:, :3])
                                              for n in ("q", "k", "v", "phi")})
    small, lse_small = run(part)
    assert np.array_equal(small, got[:, :3]), float(np.abs(small - got[:, :3]).max())
    assert np.array_equal(lse_small, lse[:, :3])
