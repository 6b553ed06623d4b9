"""GPU parity of the scans whose step angles are generated inside the kernel.

* Random variant: the written-out draws (arp_random_phi) equal the oracle's
  generator bit for bit (Philox4x64-10 and the counter layout); the fused scan
  (arp_angle_scan_random) equals, bit for bit, arp_angle_scan of those draws,
  and the oracle's scan within the scan bar (circular 1e-4 rad).
* Token table and constant steps: bit-identical to arp_angle_scan of the
  gathered / broadcast steps; ids outside [0, vocab) clamp; constant steps
  match the closed form (t + 1) freq.
* End to end: the forward over randomly drawn angles against the oracle's
  attention over the oracle's draws (bf16 bar)."""
import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import DEV, F32_TOL, assert_close, circular_err, oracle_flags, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _desc(B, H, L, P, shared, exclusive=False):
    return binding.make_desc(B, H, L, 2 * P, "bf16",
                             binding.flags_for(shared_phi=shared, exclusive=exclusive))


def _bound(G, P, seed=0):
    rng = np.random.default_rng(seed)
    return (wl.rope_frequencies(2 * P)[None, :] * rng.uniform(0.5, 2.0, size=(G, 1))).astype(np.float32)


CASES = [(2, 3, 1, 32, False), (2, 3, 2, 64, True), (1, 4, 7, 32, False), (2, 2, 1000, 64, False),
         (1, 3, 4097, 32, True), (2, 2, 33333, 64, False)]


@pytest.mark.parametrize("B,H,L,P,shared", CASES)
def test_random_draws_match_oracle_and_scan(B, H, L, P, shared):
    G = 1 if shared else H
    seed, step = 0xFEEDFACECAFEBEEF, (1 << 63) + 5
    bound = _bound(G, P)
    desc = _desc(B, H, L, P, shared)
    say(f"[gpu] random angles B={B} H={H} L={L} P={P} shared={shared}")
    b = to_dev(bound)
    phi = binding.random_phi(desc, seed, step, b)
    theta = binding.angle_scan_random(desc, seed, step, b)
    ref_theta = binding.angle_scan(phi, desc)
    torch.cuda.synchronize()
    want_phi = oracle.random_phi(B, G, L, P, seed, step, bound)
    assert np.array_equal(phi.cpu().numpy(), want_phi)
    got = theta.cpu().numpy()
    assert np.array_equal(got, ref_theta.cpu().numpy())
    assert circular_err(got, oracle.angle_scan(want_phi)) <= F32_TOL


def test_random_exclusive_and_fresh_draws():
    B, H, L, P = 1, 2, 3000, 32
    bound = _bound(H, P, 1)
    b = to_dev(bound)
    d = _desc(B, H, L, P, False, exclusive=True)
    say("[gpu] random angles exclusive")
    t0 = binding.angle_scan_random(d, 7, 0, b).cpu().numpy()
    t0b = binding.angle_scan_random(d, 7, 0, b).cpu().numpy()
    t1 = binding.angle_scan_random(d, 7, 1, b).cpu().numpy()
    assert np.array_equal(t0, t0b) and not np.array_equal(t0, t1)
    phi = oracle.random_phi(B, H, L, P, 7, 0, bound)
    assert circular_err(t0, oracle.angle_scan(phi, exclusive=True)) <= F32_TOL
    assert np.all(t0[:, :, 0] == 0.0)


def test_random_full_size():
    """rope_8k_d128's angle shape (B=4, 32 angle heads, 8192 tokens, 64 pairs)."""
    B, H, L, P = 4, 32, 8192, 64
    bound = np.broadcast_to(wl.rope_frequencies(2 * P), (H, P)).astype(np.float32)
    desc = _desc(B, H, L, P, False)
    b = to_dev(bound)
    say("[gpu] random angles full size")
    phi = binding.random_phi(desc, 99, 3, b)
    theta = binding.angle_scan_random(desc, 99, 3, b)
    ref = binding.angle_scan(phi, desc)
    torch.cuda.synchronize()
    assert torch.equal(theta, ref)
    want = oracle.random_phi(B, H, L, P, 99, 3, bound)
    assert np.array_equal(phi.cpu().numpy(), want)


@pytest.mark.parametrize("L,P,shared", [(1, 32, False), (777, 64, True), (5000, 32, False)])
def test_token_table_scan(L, P, shared):
    B, H, V = 2, 3, 300
    G = 1 if shared else H
    rng = np.random.default_rng(L + P)
    tokens = rng.integers(-20, V + 20, size=(B, L)).astype(np.int32)  # some out of range
    table = rng.uniform(-np.pi, np.pi, size=(V, G, P)).astype(np.float32)
    desc = _desc(B, H, L, P, shared)
    say(f"[gpu] token-table angles L={L} P={P} shared={shared}")
    theta = binding.angle_scan_tokens(desc, to_dev(tokens), to_dev(table))
    phi = oracle.token_phi(np.clip(tokens, 0, V - 1), table)
    ref = binding.angle_scan(to_dev(phi), desc)
    torch.cuda.synchronize()
    got = theta.cpu().numpy()
    assert np.array_equal(got, ref.cpu().numpy())
    assert circular_err(got, oracle.angle_scan(phi)) <= F32_TOL


@pytest.mark.parametrize("L,P,shared,excl", [(1, 64, False, False), (1500, 32, False, False),
                                              (9000, 64, True, False), (777, 32, False, True)])
def test_constant_steps_closed_form(L, P, shared, excl):
    B, H = 2, 4
    G = 1 if shared else H
    rng = np.random.default_rng(L)
    freq = (wl.rope_frequencies(2 * P)[None, :] * rng.uniform(0.5, 3.0, size=(G, P))).astype(np.float32)
    freq[0, :3] = (5.5, -2.0, 0.0)  # a step above pi, a negative one, none
    desc = _desc(B, H, L, P, shared, exclusive=excl)
    say(f"[gpu] constant angles L={L} P={P} shared={shared} excl={excl}")
    theta = binding.angle_scan_const(desc, to_dev(freq))
    phi = oracle.constant_phi(B, L, freq)
    ref = binding.angle_scan(to_dev(phi), desc)
    torch.cuda.synchronize()
    got = theta.cpu().numpy()
    assert np.array_equal(got, ref.cpu().numpy())
    t = np.arange(0 if excl else 1, L + (0 if excl else 1), dtype=np.float64)[None, None, :, None]
    closed = np.broadcast_to(t * freq.astype(np.float64)[None, :, None, :], got.shape)
    assert circular_err(got, closed) <= F32_TOL


def test_forward_over_random_angles():
    w = wl.make("train_1k", batch=1, heads=4, seqlen=700)
    P = w.head_dim // 2
    bound = wl.rope_frequencies(w.head_dim)[None, :]
    flags = binding.flags_for(rotate_v=True, shared_phi=True)
    desc = binding.make_desc(1, 4, 700, w.head_dim, "bf16", flags)
    say("[gpu] forward over random angles")
    theta = binding.angle_scan_random(desc, 5, 0, to_dev(bound))
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    o = binding.attn_fwd(q, k, v, theta, desc)
    torch.cuda.synchronize()
    phi = oracle.random_phi(1, 1, 700, P, 5, 0, bound)
    want = oracle.Problem(w.q, w.k, w.v, phi, oracle_flags(True, True, False)).output()
    assert_close(to_host(o), want, "bf16", "forward over random angles")
