"""Seeded random shapes and flag combinations for the backward (arp_backward_ex,
with and without forget gates) against the fp64 oracle's gradients, every
element.  Lengths up to 1500 tokens (ragged against the 64-token tiles and the
256- and 128-token workgroups), both head dims, shared angle heads, the
exclusive scan, ALiBi, value transport and gates.

Bars: dq, dk, dv and dTheta as in the backward tests (2e-2 of their own
maximum, rms 1e-2); dlogf to 2e-2 of its own scale (maximum and rms); dphi is
the suffix sum of the computed dTheta (summed over the heads of a shared
stream; t > s for the exclusive scan) up to fp32 accumulation, and within the
summed dTheta error of the oracle's dphi."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import oracle_flags, say, to_dev, to_host
from test_gpu_backward import assert_dphi_close, assert_grad_close

pytestmark = pytest.mark.gpu


def _cases():
    rng = np.random.Generator(np.random.PCG64(77))
    cases = []
    for i in range(12):
        cases.append(dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)),
                          L=int(rng.integers(2, 1500)), d=int(rng.choice([64, 128])),
                          rotate_v=bool(rng.integers(0, 2)), alibi=bool(rng.integers(0, 2)),
                          gate=bool(i % 2), exclusive=bool(rng.integers(0, 4) == 0),
                          shared=bool(rng.integers(0, 4) == 0), seed=300 + i))
    return cases


CASES = _cases()


def _id(c):
    flags = "".join(f for f, on in (("v", c["rotate_v"]), ("a", c["alibi"]), ("g", c["gate"]),
                                    ("x", c["exclusive"]), ("s", c["shared"])) if on)
    return f"B{c['B']}H{c['H']}L{c['L']}d{c['d']}{('-' + flags) if flags else ''}"


def _suffix(dth, hphi, exclusive):
    """dphi from dTheta [B, H, L, P]: suffix sums over positions, summed over the
    heads of a stream; the exclusive scan leaves t = s out."""
    x = dth.sum(axis=1, keepdims=True) if hphi == 1 else dth
    suf = np.cumsum(x[:, :, ::-1], axis=2)[:, :, ::-1]
    if exclusive:
        suf = np.concatenate([suf[:, :, 1:], np.zeros_like(suf[:, :, :1])], axis=2)
    return suf


@pytest.mark.parametrize("c", CASES, ids=[_id(c) for c in CASES])
def test_random_shape_backward(c):
    name = "train_1k" if c["d"] == 64 else "rope_8k_d128"
    w = wl.make(name, batch=c["B"], heads=c["H"], seqlen=c["L"], seed=c["seed"])
    rng = np.random.Generator(np.random.PCG64(c["seed"]))
    if c["d"] == 128:  # token-dependent angles at d=128 too
        w = dataclasses.replace(w, phi=rng.uniform(-0.5, 0.5, size=w.phi.shape).astype(np.float32))
    if c["shared"]:
        w = dataclasses.replace(w, phi=np.ascontiguousarray(w.phi[:, :1]))
    B, H, L, d = w.q.shape
    hphi = w.phi.shape[1]
    slopes = wl.alibi_slopes(H) if c["alibi"] else None
    logf = None
    if c["gate"]:
        z = rng.normal(1.0, 1.0, size=(B, H, L))
        logf = (-np.logaddexp(0.0, -z)).astype(np.float32)
    dout = wl.to_bf16_bits(rng.standard_normal((B, H, L, d)).astype(np.float32))
    say(f"[gpu] random backward {_id(c)}")

    q, k, v, phi = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi)
    al = to_dev(slopes) if slopes is not None else None
    lf = to_dev(logf) if logf is not None else None
    o, theta, lse = binding.forward_ex(q, k, v, phi, rotate_qk=True, rotate_v=c["rotate_v"],
                                       alibi=al, logf=lf, exclusive=c["exclusive"], with_lse=True)
    flags = binding.flags_for(rotate_qk=True, rotate_v=c["rotate_v"], alibi=c["alibi"],
                              shared_phi=hphi == 1 and H != 1, exclusive=c["exclusive"],
                              forget=c["gate"])
    dq, dk, dv, dphi, dtheta, dlogf = binding.backward_ex(binding.desc_for(q, flags), q, k, v, phi,
                                                          theta, o, lse, to_dev(dout), alibi=al,
                                                          logf=lf)
    torch.cuda.synchronize()
    got = dict(dq=to_host(dq), dk=to_host(dk), dv=to_host(dv), dtheta=dtheta.cpu().numpy(),
               dphi=dphi.cpu().numpy())

    of = oracle_flags(True, c["rotate_v"], c["alibi"]) | (oracle.FORGET if c["gate"] else 0)
    if c["exclusive"]:
        of |= oracle.SCAN_EXCLUSIVE
    want = oracle.Problem(w.q, w.k, w.v, w.phi, of, alibi=slopes, logf=logf).backward(dout)
    tag = f"random {_id(c)}"
    for n in ("dq", "dk", "dv", "dtheta"):
        assert_grad_close(got[n], want[n], f"{tag} {n}")
    dth = got["dtheta"].astype(np.float64)
    suf = _suffix(dth, hphi, c["exclusive"])
    absum = _suffix(np.abs(dth), hphi, c["exclusive"])
    assert np.all(np.abs(got["dphi"] - suf) <= 1e-5 * absum + 1e-30), f"{tag}: dphi not the suffix sum"
    walk = _suffix(np.abs(dth - want["dtheta"]), hphi, c["exclusive"])
    err = np.abs(got["dphi"].astype(np.float64) - want["dphi"])
    say(f"[gpu] {tag} dphi: max err {err.max():.3e} (ref max {np.abs(want['dphi']).max():.3e})")
    assert np.all(err <= walk + 1e-5 * absum + 1e-12), f"{tag}: dphi beyond the summed dTheta error"
    if c["gate"]:
        assert_dphi_close(dlogf.cpu().numpy(), want["dlogf"], f"{tag} dlogf")
    else:
        assert dlogf is None
