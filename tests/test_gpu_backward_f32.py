"""GPU parity of the fp32 I/O backward (arp_forward_train / arp_backward with
fp32 tensors: plain-FMA gradient kernels) against the fp64 oracle's gradients.

Every product and sum is fp32, so the gradients are held to fp32-level bars:
max |err| <= 1e-4 of each gradient's own maximum (dq, dk, dv, dTheta, dphi),
and the forward's log-sum-exp to 1e-5 (base-2 units)."""
import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import oracle_flags, say, to_dev

pytestmark = pytest.mark.gpu

REL = 1e-4
FLAG_SETS = [
    dict(rotate_qk=True, rotate_v=False, alibi=False),
    dict(rotate_qk=True, rotate_v=True, alibi=False),
    dict(rotate_qk=True, rotate_v=True, alibi=True),
    dict(rotate_qk=False, rotate_v=False, alibi=False),
    dict(rotate_qk=False, rotate_v=True, alibi=True),
    dict(rotate_qk=True, rotate_v=True, alibi=False, exclusive=True),
]


def _ids(fs):
    return "-".join(k for k, v in fs.items() if v) or "nope"


def _f32(name, **kw):
    w = wl.make(name, **kw)
    for n in ("q", "k", "v"):
        setattr(w, n, w.values(n).astype(np.float32).copy())
    if w.head_dim == 128:  # token-dependent angles
        rng = np.random.Generator(np.random.PCG64(5))
        w.phi = rng.uniform(-0.5, 0.5, size=w.phi.shape).astype(np.float32)
    return w


def run(w, dout, rotate_qk=True, rotate_v=False, alibi=False, exclusive=False):
    say(f"[gpu] fp32 backward {w.name} B={w.batch} H={w.heads} L={w.seqlen} d={w.head_dim} "
        f"qk={rotate_qk} v={rotate_v} alibi={alibi} excl={exclusive}")
    q, k, v, phi = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi)
    al = to_dev(wl.alibi_slopes(w.heads)) if alibi else None
    o, theta, lse, desc = binding.forward_train(q, k, v, phi, rotate_qk=rotate_qk,
                                                rotate_v=rotate_v, alibi=al, exclusive=exclusive)
    dq, dk, dv, dphi, dtheta = binding.backward(desc, q, k, v, phi, theta, o, lse, to_dev(dout),
                                                alibi=al)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dphi", dphi),
                                             ("dtheta", dtheta), ("lse", lse), ("o", o))}


def _want(w, dout, rotate_qk=True, rotate_v=False, alibi=False, exclusive=False):
    prob = oracle.Problem(w.q, w.k, w.v, w.phi, oracle_flags(rotate_qk, rotate_v, alibi, exclusive),
                          alibi=wl.alibi_slopes(w.heads) if alibi else None)
    return prob, prob.backward(dout)


def _close(got, want, what):
    scale = max(float(np.abs(want).max()), 1e-30)
    err = float(np.abs(got.astype(np.float64) - want).max())
    say(f"[gpu] {what}: max err {err:.3e} (ref max {scale:.3e})")
    assert np.all(np.isfinite(got)), what
    assert err <= REL * scale, f"{what}: max err {err:.3e} > {REL} * {scale:.3e}"


def compare(w, flags, got, tag):
    dout = _dout(w)
    prob, want = _want(w, dout, **flags)
    for n in ("dq", "dk", "dv"):
        _close(got[n], want[n], f"{tag} {n}")
    if flags.get("rotate_qk", True) or flags.get("rotate_v", False):
        _close(got["dtheta"], want["dtheta"], f"{tag} dtheta")
        _close(got["dphi"], want["dphi"], f"{tag} dphi")
    else:
        assert np.abs(got["dphi"]).max() == 0.0 and np.abs(got["dtheta"]).max() == 0.0
    B, H, L, _ = w.q.shape
    for b in range(B):
        for h in range(H):
            for i in sorted({0, L // 2, L - 1}):
                s = prob.scores_row(b, h, i)
                m = s.max()
                ref = (m + np.log(np.exp(s - m).sum())) / np.log(2.0)
                assert abs(got["lse"][b, h, i] - ref) <= 1e-5 * max(1.0, abs(ref)), (b, h, i)


def _dout(w, seed=102):
    g = np.random.default_rng(seed).standard_normal((w.batch, w.heads, w.seqlen, w.head_dim))
    return g.astype(np.float32)


@pytest.mark.parametrize("flags", FLAG_SETS, ids=[_ids(f) for f in FLAG_SETS])
@pytest.mark.parametrize("name,L", [("tiny_f32", 256), ("rope_8k_d128", 150)])
def test_f32_backward_all_flags(name, L, flags):
    w = _f32(name, batch=1, heads=2, seqlen=L)
    compare(w, flags, run(w, _dout(w), **flags), f"fp32 {name} L={L} {_ids(flags)}")


@pytest.mark.parametrize("L", [2, 3, 33, 64, 65, 130, 300])
def test_f32_backward_ragged_lengths(L):
    w = _f32("tiny_f32", batch=2, heads=2, seqlen=L)
    flags = dict(rotate_qk=True, rotate_v=True, alibi=True)
    compare(w, flags, run(w, _dout(w), **flags), f"fp32 L={L}")


def test_f32_backward_single_token():
    """L = 1: o = v exactly, so dv = dO and every other gradient is zero up to
    fp32 rounding of D = <dO, o>."""
    w = _f32("tiny_f32", batch=1, heads=2, seqlen=1)
    dout = _dout(w)
    got = run(w, dout, rotate_v=True, alibi=True)
    assert np.abs(got["dv"] - dout).max() <= 1e-5 * np.abs(dout).max()
    for n in ("dq", "dk", "dphi"):
        assert np.abs(got[n]).max() <= 1e-5, (n, np.abs(got[n]).max())


def test_f32_backward_shared_angle_heads():
    w = _f32("tiny_f32", batch=2, heads=3, seqlen=200)
    w.phi = np.ascontiguousarray(w.phi[:, :1]) if w.phi.shape[1] != 1 else w.phi
    flags = dict(rotate_qk=True, rotate_v=True)
    compare(w, flags, run(w, _dout(w), **flags), "fp32 shared phi")
