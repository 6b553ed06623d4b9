"""Forget gates over 2^20 tokens with strong gates (log f = log sigmoid(z),
z ~ N(0, 0.5): about -0.7 per token), where the gate prefix reaches ~1e6 in
base-2 logit units and an fp32 prefix would lose 0.06 units of every logit
(fp32's spacing at 1e6).  The library keeps the prefix per 64-token tile with
an fp64 base (forward, backward) and in fp64 (decode); these tests hold it to
the forward's and the backward's bars at that length.

  * forward: sampled rows of the whole sequence against the oracle, which
    sums the route's log gates in fp64 directly;
  * backward: a wall gate (log f = -200 at S = L - 2048) makes every route
    from a key before S into the last 2048 queries carry a factor 2^-288, so
    those probabilities are exactly zero in fp32 (the kernels skip them) and
    below 1e-86 in the oracle: the last 2048 tokens form a problem of their
    own, whose gradients the oracle computes whole (scores and transported
    values only see angle differences, so the window's angles may start from
    zero);
  * decode: a 2^20 - 12 token prompt, then 12 steps, each against the
    oracle's row.
Bars: the forward's (bf16 max |err| <= 2e-2, rms <= 1% of the output's) and
the backward's (2e-2 of each gradient's own scale; dlogf 2e-2 of its own
scale for the maximum and the rms; dphi, the suffix sum of dTheta, within the
summed dTheta error, as in the gated backward tests)."""
import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import (DEV, assert_close, oracle_flags, sample_rows, say, to_dev, to_host)
from test_gpu_backward import _dout, assert_dphi_close, assert_grad_close
from test_gpu_forget_backward import assert_dphi_bars

pytestmark = pytest.mark.gpu

L = 1 << 20
S = L - 2048


def _strong_gates(B, H, n, seed):
    z = np.random.default_rng(seed).standard_normal((B, H, n)) * 0.5
    return (-np.log1p(np.exp(-z))).astype(np.float32)


@pytest.fixture(scope="module")
def problem():
    w = wl.make("farmass_32k", batch=1, heads=1, seqlen=L)
    logf = _strong_gates(1, 1, L, 41)
    return w, logf


def test_long_gated_forward_sampled_rows(problem):
    w, logf = problem
    say(f"[gpu] long gated forward L={L}")
    o, _, _ = binding.forward_ex(to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi),
                                 rotate_v=True, logf=to_dev(logf))
    torch.cuda.synchronize()
    got = to_host(o)
    rows = sample_rows(w, per_head=24, seed=5)
    prob = oracle.Problem(w.q, w.k, w.v, w.phi, oracle_flags(True, True) | oracle.FORGET, logf=logf)
    assert_close(got.reshape(-1, w.head_dim)[rows], prob.rows(rows), "bf16",
                 f"gated forward at {L} tokens, sampled rows")


def test_long_gated_backward_last_window(problem):
    w, logf = problem
    logf = logf.copy()
    logf[:, :, S] = -200.0  # the wall
    dout = _dout(w, seed=43)
    say(f"[gpu] long gated backward L={L}, window [{S}, {L})")
    q, k, v, phi = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi)
    lf = to_dev(logf)
    o, theta, lse = binding.forward_ex(q, k, v, phi, rotate_v=True, logf=lf, with_lse=True)
    desc = binding.desc_for(q, binding.flags_for(rotate_v=True, forget=True))
    dq, dk, dv, dphi, dtheta, dlogf = binding.backward_ex(desc, q, k, v, phi, theta, o, lse,
                                                          to_dev(dout), logf=lf)
    torch.cuda.synchronize()
    win = slice(S, L)
    sub = oracle.Problem(np.ascontiguousarray(w.q[:, :, win]), np.ascontiguousarray(w.k[:, :, win]),
                         np.ascontiguousarray(w.v[:, :, win]), np.ascontiguousarray(w.phi[:, :, win]),
                         oracle_flags(True, True) | oracle.FORGET,
                         logf=np.ascontiguousarray(logf[:, :, win]))
    assert_close(to_host(o)[:, :, win], sub.output(), "bf16", "long gated forward, last window")
    want = sub.backward(np.ascontiguousarray(dout[:, :, win]))
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_grad_close(to_host(t)[:, :, win], want[n], f"long gated {n}")
    got_th = dtheta.cpu().numpy()[:, :, win]
    assert_grad_close(got_th, want["dtheta"], "long gated dtheta")
    # dphi: the suffix sum of the computed dTheta, within the summed dTheta
    # error of the oracle's (the gated backward tests' bar: under strong
    # forgetting the exact dphi is a small difference of many dTheta terms)
    assert_dphi_bars({"dphi": dphi.cpu().numpy()[:, :, win], "dtheta": got_th}, want,
                     "long gated dphi")
    assert_dphi_close(dlogf.cpu().numpy()[:, :, win], want["dlogf"], "long gated dlogf")


def test_long_gated_decode(problem):
    w, logf = problem
    t0 = L - 12
    say(f"[gpu] long gated decode: prefill {t0}, 12 steps")
    q, k, v, phi = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi)
    lf = to_dev(logf)
    flags = binding.flags_for(rotate_v=True)
    cache = binding.DecodeCache(1, 1, L, 64, rotate_v=True, forget=True, device=DEV)
    th0 = binding.angle_scan(phi[:, :, :t0].contiguous(), binding.make_desc(1, 1, t0, 64, "bf16", flags))
    cache.prefill(k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous(), phi[:, :, :t0].contiguous(),
                  th0, logf=lf[:, :, :t0].contiguous())
    outs = []
    for t in range(t0, L):
        outs.append(cache.step(t, q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                               v[:, :, t].contiguous(), phi[:, :, t].contiguous(),
                               logf=lf[:, :, t].clone()).clone())
    torch.cuda.synchronize()
    got = to_host(torch.stack(outs, dim=2))
    prob = oracle.Problem(w.q, w.k, w.v, w.phi, oracle_flags(True, True) | oracle.FORGET, logf=logf)
    want = prob.rows(np.arange(t0, L, dtype=np.int64)).reshape(1, 1, L - t0, 64)
    assert_close(got, want, "bf16", f"gated decode at {L} tokens")
