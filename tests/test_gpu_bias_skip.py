"""GPU parity where the biases leave most of a row's keys with probability
exactly zero (below fp32's smallest subnormal), so the biased kernels walk
the key tiles from the diagonal backwards and stop once a bound on every
remaining score is far enough below the running maximum.  All rows against
the fp64 oracle at 2048 tokens (32 key tiles): steep ALiBi slopes, strong
forget gates, both together, a negative slope (the bias then rises with the
distance, which turns the stopping rule off), and head dimension 128."""
import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import assert_close, oracle_flags, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _gates(w, seed, mean):
    z = np.random.default_rng(seed).normal(mean, 1.0, size=(w.batch, w.heads, w.seqlen))
    return (-np.logaddexp(0.0, -z)).astype(np.float32)  # log sigmoid(z)


def _check(w, slopes, logf, rotate_v, what):
    say(f"[gpu] bias walk {what}: {w.name} B={w.batch} H={w.heads} L={w.seqlen} d={w.head_dim}")
    al = None if slopes is None else to_dev(np.asarray(slopes, dtype=np.float32))
    lg = None if logf is None else to_dev(logf)
    o, _, _ = binding.forward_ex(to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi),
                                 rotate_qk=True, rotate_v=rotate_v, alibi=al, logf=lg)
    torch.cuda.synchronize()
    flags = oracle_flags(True, rotate_v, slopes is not None) | (oracle.FORGET if logf is not None else 0)
    want = oracle.Problem(w.q, w.k, w.v, w.phi, flags,
                          alibi=None if slopes is None else np.asarray(slopes, dtype=np.float32),
                          logf=logf).output()
    assert_close(to_host(o), want, "bf16", what)


@pytest.mark.parametrize("name,L", [("train_1k", 2048), ("rope_8k_d128", 1024)])
def test_steep_alibi_slopes(name, L):
    w = wl.make(name, batch=1, heads=4, seqlen=L)
    _check(w, [2.0, 1.0, 0.25, 1.0 / 64], None, True, f"steep alibi {name}")


@pytest.mark.parametrize("name,L", [("train_1k", 2048), ("rope_8k_d128", 1024)])
def test_strong_gates(name, L):
    w = wl.make(name, batch=1, heads=2, seqlen=L)
    _check(w, None, _gates(w, 31, 0.0), True, f"strong gates {name}")


def test_gates_with_alibi_ragged():
    w = wl.make("train_1k", batch=2, heads=2, seqlen=1500)
    _check(w, [0.5, 1.0 / 32], _gates(w, 32, 1.0), False, "gates + alibi L=1500")


def test_negative_slope():
    w = wl.make("train_1k", batch=1, heads=2, seqlen=700)
    _check(w, [-0.01, 0.5], None, True, "negative slope")
