"""Seeded random shapes and flag combinations against the fp64 oracle, on
sampled rows (tile edges, the ends, random rows of every head).  The shapes
straddle the attention kernel's workgroup-shape rule (512-query workgroups
for unbiased walks over at least 4096 tokens on deep grids, 128-query
workgroups otherwise, paired where they fill the CUs, at d=64; the d=128
rule on 256-query grids), ragged
lengths, both head dims, shared angle heads, the exclusive scan, ALiBi and
forget gates.  Bar: the forward's bf16 bar on the sampled rows."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import assert_close, oracle_flags, sample_rows, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _cases():
    rng = np.random.Generator(np.random.PCG64(2024))
    cases = []
    # (B, H, L) chosen around the shape rule's edges, then random ones
    fixed = [(1, 16, 16384), (2, 8, 16385), (1, 32, 16383), (1, 8, 16400), (4, 8, 4097),
             (1, 40, 8200), (2, 2, 513), (3, 5, 777), (8, 8, 4096), (4, 16, 4100), (8, 8, 4000), (2, 3, 300), (1, 16, 8192)]
    for i, (B, H, L) in enumerate(fixed):
        cases.append(dict(B=B, H=H, L=L, d=64 if i % 3 else 128, rotate_v=bool(i % 2),
                          alibi=i % 4 == 3, gate=i % 5 == 4, exclusive=i % 6 == 5,
                          shared=i % 7 == 6, seed=100 + i))
    for i in range(10):
        L = int(rng.integers(1, 20000))
        cases.append(dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 12)), L=L,
                          d=int(rng.choice([64, 128])), rotate_v=bool(rng.integers(0, 2)),
                          alibi=bool(rng.integers(0, 2)), gate=bool(rng.integers(0, 3) == 0),
                          exclusive=bool(rng.integers(0, 4) == 0),
                          shared=bool(rng.integers(0, 4) == 0), seed=200 + i))
    return cases


CASES = _cases()


def _id(c):
    flags = "".join(f for f, on in (("v", c["rotate_v"]), ("a", c["alibi"]), ("g", c["gate"]),
                                    ("x", c["exclusive"]), ("s", c["shared"])) if on)
    return f"B{c['B']}H{c['H']}L{c['L']}d{c['d']}{('-' + flags) if flags else ''}"


@pytest.mark.parametrize("c", CASES, ids=[_id(c) for c in CASES])
def test_random_shape_sampled_rows(c):
    name = "train_1k" if c["d"] == 64 else "rope_8k_d128"
    w = wl.make(name, batch=c["B"], heads=c["H"], seqlen=c["L"], seed=c["seed"])
    if c["d"] == 128:  # token-dependent angles at d=128 too (not the constant RoPE steps)
        rng = np.random.Generator(np.random.PCG64(c["seed"]))
        w = dataclasses.replace(w, phi=rng.uniform(-0.5, 0.5, size=w.phi.shape).astype(np.float32))
    if c["shared"]:
        w = dataclasses.replace(w, phi=np.ascontiguousarray(w.phi[:, :1]))
    slopes = wl.alibi_slopes(w.heads) if c["alibi"] else None
    logf = None
    if c["gate"]:
        z = np.random.default_rng(c["seed"]).normal(2.0, 1.0, size=(w.batch, w.heads, w.seqlen))
        logf = (-np.logaddexp(0.0, -z)).astype(np.float32)
    say(f"[gpu] random case {_id(c)}")
    o, theta, _ = binding.forward_ex(to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi),
                                     rotate_v=c["rotate_v"],
                                     alibi=None if slopes is None else to_dev(slopes),
                                     logf=None if logf is None else to_dev(logf),
                                     exclusive=c["exclusive"])
    torch.cuda.synchronize()
    got = to_host(o)
    assert np.all(np.isfinite(got))
    rows = sample_rows(w, per_head=6, seed=c["seed"])
    flags = oracle_flags(True, c["rotate_v"], c["alibi"], c["exclusive"]) | \
        (oracle.FORGET if c["gate"] else 0)
    want = oracle.Problem(w.q, w.k, w.v, w.phi, flags, alibi=slopes, logf=logf).rows(rows)
    assert_close(got.reshape(-1, w.head_dim)[rows], want, "bf16", _id(c))
