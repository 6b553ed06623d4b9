"""GPU parity of AdaScale's per-head query multiplier ("AdaRoPE: Not All
Attention Heads Should Rotate and Scale Equally", Sec. 3.3, AdaScale; applied
to the query only, Sec. 3.4) on every path that takes it, against the fp64
oracle given the same fp32 multipliers:
  * forward: the pre-rotation path (both workgroup shapes), the fused
    rotation, fp32 I/O, and the gated forward;
  * training: lse and the backward's dq, dk, dv, dTheta, dphi (bf16 and fp32);
  * decode: every decoded row against the oracle's whole-sequence rows.
The multipliers come from the library's schedule routine (arp_adascale_lambda)
with per-head tau and gamma spread around the page's reported values (tau near
1, gamma mostly positive).  Bars: those of the forward, backward and decode
tests (bf16 max |err| <= 2e-2 and rms <= 1% of the output's rms; fp32 1e-4;
gradients 2e-2 of their own scale)."""
import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import (DEV, assert_close, oracle_flags, sample_rows, say, to_dev, to_host)
from test_gpu_backward import _dout, assert_dphi_close, assert_grad_close

pytestmark = pytest.mark.gpu


def _lambda(heads, L, L_ref=1024, seed=0):
    rng = np.random.default_rng(seed)
    tau = rng.uniform(0.6, 1.6, heads).astype(np.float32)
    gamma = rng.uniform(-0.5, 2.0, heads).astype(np.float32)
    return binding.adascale_lambda(tau, gamma, L, L_ref).numpy()


def _oracle(w, lam, *, rotate_qk=True, rotate_v=False, alibi=False, exclusive=False, logf=None):
    slopes = wl.alibi_slopes(w.heads) if alibi else None
    flags = oracle_flags(rotate_qk, rotate_v, alibi, exclusive) | (oracle.FORGET if logf is not None else 0)
    return oracle.Problem(w.q, w.k, w.v, w.phi, flags, alibi=slopes, logf=logf, head_scale=lam)


def _forward(w, lam, *, fused=False, **flags):
    say(f"[gpu] adascale forward {w.name} B={w.batch} H={w.heads} L={w.seqlen} d={w.head_dim} "
        f"fused={fused} {flags}")
    al = to_dev(wl.alibi_slopes(w.heads)) if flags.get("alibi") else None
    o, _ = binding.forward(to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi),
                           rotate_qk=flags.get("rotate_qk", True),
                           rotate_v=flags.get("rotate_v", False), alibi=al,
                           exclusive=flags.get("exclusive", False), fused=fused,
                           head_scale=to_dev(lam))
    torch.cuda.synchronize()
    return to_host(o)


FLAG_SETS = [dict(rotate_v=False), dict(rotate_v=True), dict(rotate_v=True, alibi=True),
             dict(rotate_qk=False), dict(exclusive=True)]


@pytest.mark.parametrize("flags", FLAG_SETS, ids=lambda f: "-".join(f) or "qk")
@pytest.mark.parametrize("name,L", [("train_1k", 333), ("rope_8k_d128", 200), ("tiny_f32", 97)])
def test_forward_with_head_scale(name, L, flags):
    w = wl.make(name, batch=2, heads=3, seqlen=L)
    lam = _lambda(3, 4 * L)
    got = _forward(w, lam, **flags)
    want = _oracle(w, lam, **flags).output()
    assert_close(got, want, "f32" if w.q.dtype == np.float32 else "bf16",
                 f"adascale {name} L={L} {flags}")


@pytest.mark.parametrize("name,L", [("train_1k", 333), ("rope_8k_d128", 200)])
def test_fused_rotation_with_head_scale(name, L):
    w = wl.make(name, batch=2, heads=3, seqlen=L)
    lam = _lambda(3, 4 * L, seed=1)
    got = _forward(w, lam, fused=True, rotate_v=True, alibi=True)
    want = _oracle(w, lam, rotate_v=True, alibi=True).output()
    assert_close(got, want, "bf16", f"adascale fused {name} L={L}")


def test_head_scale_is_per_head():
    """Head h alone with multiplier lambda_h gives the same output as head h in
    the full run (the multiplier follows the head, not the position in the
    grid), and a unit multiplier changes nothing bit for bit."""
    w = wl.make("train_1k", batch=1, heads=4, seqlen=300)
    lam = np.array([0.5, 1.0, 2.0, 3.0], dtype=np.float32)
    full = _forward(w, lam, rotate_v=True)
    plain = binding.forward(to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi), rotate_v=True)[0]
    torch.cuda.synchronize()
    assert np.array_equal(full[:, 1], to_host(plain)[:, 1])
    want = _oracle(w, lam, rotate_v=True).output()
    assert_close(full, want, "bf16", "adascale per head")


def test_full_size_shape_with_head_scale_sampled_rows():
    """The 16x-extrapolation workload (512-query workgroups) with multipliers
    for its 16384-token context against a 1024-token reference length."""
    w = wl.make("extrap_16k")
    lam = _lambda(w.heads, w.seqlen, 1024, seed=2)
    got = _forward(w, lam, rotate_v=True)
    rows = sample_rows(w, per_head=10)
    want = _oracle(w, lam, rotate_v=True).rows(rows)
    assert_close(got.reshape(-1, w.head_dim)[rows], want, "bf16", "adascale extrap_16k sampled rows")


def test_gated_forward_with_head_scale():
    w = wl.make("train_1k", batch=2, heads=3, seqlen=700)
    lam = _lambda(3, 2800, seed=3)
    z = np.random.default_rng(8).standard_normal((2, 3, 700)).astype(np.float32) + 2.0
    logf = (-np.log1p(np.exp(-z))).astype(np.float32)
    o, _, _ = binding.forward_ex(to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi),
                                 rotate_v=True, logf=to_dev(logf), head_scale=to_dev(lam))
    torch.cuda.synchronize()
    want = _oracle(w, lam, rotate_v=True, logf=logf).output()
    assert_close(to_host(o), want, "bf16", "adascale gated forward")


@pytest.mark.parametrize("name,L,flags", [("train_1k", 300, dict(rotate_v=True, alibi=True)),
                                          ("train_1k", 257, dict(exclusive=True)),
                                          ("rope_8k_d128", 200, dict(rotate_v=True)),
                                          ("tiny_f32", 150, dict(rotate_v=True, alibi=True))])
def test_training_with_head_scale(name, L, flags):
    w = wl.make(name, batch=1, heads=3, seqlen=L)
    if w.q.dtype == np.float32:
        dout = np.random.default_rng(100).standard_normal(w.q.shape).astype(np.float32)
    else:
        dout = _dout(w)
    lam = _lambda(3, 4 * L, seed=4)
    say(f"[gpu] adascale backward {name} L={L} {flags}")
    q, k, v, phi = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi)
    al = to_dev(wl.alibi_slopes(3)) if flags.get("alibi") else None
    o, theta, lse, desc = binding.forward_train(q, k, v, phi, rotate_v=flags.get("rotate_v", False),
                                                alibi=al, exclusive=flags.get("exclusive", False),
                                                head_scale=to_dev(lam))
    dq, dk, dv, dphi, dtheta = binding.backward(desc, q, k, v, phi, theta, o, lse, to_dev(dout),
                                                alibi=al)
    torch.cuda.synchronize()
    prob = _oracle(w, lam, **flags)
    # lse: base-2 log-sum-exp of the scaled logits, from the oracle's scores.
    # Bar: q~ scale lambda_h log2 e and k~ are each rounded to bf16 (2^-9
    # relative) before the product, so a base-2 logit -- and the log-sum-exp,
    # a smooth maximum of them -- can be off by 2^-8 of the largest logit.
    rows = [(0, h, i) for h in range(3) for i in (0, 1, L // 2, L - 1)]
    lse_h = lse.cpu().numpy()
    for (b_, h, i) in rows:
        s = prob.scores_row(b_, h, i) / np.log(2.0)
        ref = s.max() + np.log2(np.exp2(s - s.max()).sum())
        bar = 2.0 ** -8 * max(1.0, float(np.abs(s).max()))
        assert abs(lse_h[b_, h, i] - ref) <= bar, (h, i, lse_h[b_, h, i], ref, bar)
    want = prob.backward(dout)
    f32 = w.q.dtype == np.float32
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dtheta", dtheta)):
        got = to_host(t) if n != "dtheta" else t.cpu().numpy()
        if f32:
            scale = max(float(np.abs(want[n]).max()), 1e-6)
            err = float(np.abs(got - want[n]).max())
            say(f"[gpu] adascale f32 {n}: max err {err:.3e} of {scale:.3e}")
            assert err <= 1e-4 * scale, (n, err, scale)
        else:
            assert_grad_close(got, want[n], f"adascale {name} {n}")
    if f32:
        err = float(np.abs(dphi.cpu().numpy() - want["dphi"]).max())
        assert err <= 1e-4 * max(float(np.abs(want["dphi"]).max()), 1e-6), err
    else:
        assert_dphi_close(dphi.cpu().numpy(), want["dphi"], f"adascale {name} dphi")


@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_decode_with_head_scale(name):
    """Prefill 100 tokens, decode 40 more with the multipliers: each decoded
    row against the oracle's row of the whole sequence."""
    w = wl.make(name, batch=2, heads=3, seqlen=140)
    lam = _lambda(3, 560, seed=5)
    q, k, v, phi = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi)
    B, H, L, d = q.shape
    flags = binding.flags_for(rotate_v=True)
    cache = binding.DecodeCache(B, H, L, d, rotate_v=True, head_scale=to_dev(lam), device=DEV)
    t0 = 100
    th0 = binding.angle_scan(phi[:, :, :t0].contiguous(), binding.make_desc(B, H, t0, d, "bf16", flags))
    cache.prefill(k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous(),
                  phi[:, :, :t0].contiguous(), th0)
    outs = []
    for t in range(t0, L):
        outs.append(cache.step(t, q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                               v[:, :, t].contiguous(), phi[:, :, t].contiguous()).clone())
    torch.cuda.synchronize()
    got = to_host(torch.stack(outs, dim=2))
    want = _oracle(w, lam, rotate_v=True).output()[:, :, t0:]
    assert_close(got, want, "bf16", f"adascale decode {name}")
