"""GPU parity of the angle scan and the rotation against the fp64 oracle.

Scan: circular error <= 1e-4 rad on every workload's angles (full size), the
exclusive variant, ragged lengths, shared angle heads; an impulse input is
bit-exact; repeated calls on one workspace give bit-identical results (the
scan leaves its look-back state zeroed).  Rotation: the fp32 diagnostic
rotation matches the oracle's to 1e-4 (fp32 rounding only)."""
import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import DEV, F32_TOL, circular_err, say, to_dev

pytestmark = pytest.mark.gpu


def _scan(phi_np: np.ndarray, heads: int, head_dim: int, exclusive=False, shared=None):
    B, Hphi, L, P = phi_np.shape
    shared = (Hphi == 1 and heads != 1) if shared is None else shared
    flags = binding.flags_for(shared_phi=shared, exclusive=exclusive)
    desc = binding.make_desc(B, heads, L, head_dim, "bf16", flags)
    say(f"[gpu] angle_scan B={B} Hphi={Hphi} L={L} P={P} excl={exclusive}")
    theta = binding.angle_scan(to_dev(phi_np), desc)
    torch.cuda.synchronize()
    return theta.cpu().numpy()


@pytest.mark.parametrize("name", list(wl.SPECS))
def test_scan_full_size_workloads(name):
    w = wl.make(name)
    ref = oracle.angle_scan(w.phi)
    got = _scan(w.phi, w.heads, w.head_dim)
    assert got.dtype == np.float32
    assert np.all(got >= -np.float32(np.pi)) and np.all(got <= np.float32(np.pi))
    err = circular_err(got, ref)
    say(f"[gpu] scan {name}: circular max err {err:.3e}")
    assert err <= F32_TOL


@pytest.mark.parametrize("L", [1, 5, 63, 64, 65, 127, 1000, 4097, 33333])
@pytest.mark.parametrize("P", [32, 64])
def test_scan_ragged_lengths_and_exclusive(L, P):
    rng = np.random.Generator(np.random.PCG64(L * 7 + P))
    phi = rng.uniform(-4, 4, size=(2, 3, L, P)).astype(np.float32)
    for excl in (False, True):
        got = _scan(phi, 3, 2 * P, exclusive=excl)
        assert circular_err(got, oracle.angle_scan(phi, exclusive=excl)) <= F32_TOL


def test_scan_shared_angle_heads():
    w = wl.make("tiny_f32")
    got = _scan(w.phi, w.heads, w.head_dim)
    assert got.shape == (1, 1, 256, 32)
    assert circular_err(got, oracle.angle_scan(w.phi)) <= F32_TOL


def test_scan_impulse_is_exact():
    L, P = 3000, 32
    phi = np.zeros((1, 2, L, P), dtype=np.float32)
    phi[0, 1, 1234, 7] = 0.5
    phi[0, 0, 0, 0] = -1.25
    got = _scan(phi, 2, 64)
    want = np.zeros_like(phi)
    want[0, 1, 1234:, 7] = 0.5
    want[0, 0, :, 0] = -1.25
    assert np.array_equal(got, want)


def test_scan_repeated_calls_reuse_workspace_bit_identically():
    """One state buffer, zero-filled once, serves repeated calls and calls of
    other shapes in between (larger and smaller, P = 32 and 64): every result
    is bit-identical to the first call's and within tolerance of the oracle."""
    w = wl.make("farmass_32k", heads=4, seqlen=20000)
    flags = binding.flags_for()
    desc = binding.make_desc(1, 4, 20000, 64, "bf16", flags)
    big = binding.make_desc(2, 4, 30000, 128, "bf16", flags)
    small = binding.make_desc(1, 2, 300, 64, "bf16", flags)
    st = torch.zeros(max(binding.scan_state_bytes(desc), binding.scan_state_bytes(big)),
                     dtype=torch.uint8, device=DEV)
    phi = to_dev(w.phi)
    rng = np.random.Generator(np.random.PCG64(9))
    phi_big = rng.uniform(-3, 3, size=(2, 4, 30000, 64)).astype(np.float32)
    phi_small = rng.uniform(-3, 3, size=(1, 2, 300, 32)).astype(np.float32)
    outs, others = [], []
    for i in range(5):
        outs.append(binding.angle_scan(phi, desc, state=st).cpu().numpy())
        if i == 1:
            others.append((binding.angle_scan(to_dev(phi_big), big, state=st).cpu().numpy(),
                           phi_big))
        if i == 2:
            others.append((binding.angle_scan(to_dev(phi_small), small, state=st).cpu().numpy(),
                           phi_small))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert circular_err(outs[0], oracle.angle_scan(w.phi)) <= F32_TOL
    for got, ph in others:
        assert circular_err(got, oracle.angle_scan(ph)) <= F32_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("inverse", [False, True])
def test_rotation_diagnostic_matches_oracle(dtype, inverse):
    rng = np.random.Generator(np.random.PCG64(5))
    B, H, L, d = 2, 3, 77, 64
    x32 = rng.standard_normal((B, H, L, d)).astype(np.float32)
    x = x32 if dtype == "f32" else wl.to_bf16_bits(x32)
    theta = rng.uniform(-np.pi, np.pi, size=(B, H, L, d // 2)).astype(np.float32)
    desc = binding.make_desc(B, H, L, d, dtype, binding.ROTATE_QK)
    say(f"[gpu] rotate dtype={dtype} inverse={inverse}")
    got = binding.rotate(to_dev(x), to_dev(theta), desc, inverse=inverse)
    torch.cuda.synchronize()
    want = oracle.rotate_rows(x, theta.astype(np.float64), inverse=inverse)
    err = float(np.abs(got.cpu().numpy() - want).max())
    say(f"[gpu] rotate err {err:.3e}")
    assert err <= F32_TOL
    # norm of every pair preserved
    g = got.cpu().numpy()
    xv = wl.from_bf16_bits(x) if dtype == "bf16" else x
    np.testing.assert_allclose(np.hypot(g[..., 0::2], g[..., 1::2]),
                               np.hypot(xv[..., 0::2], xv[..., 1::2]), rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("B,H,L,d,rotv,rotqk,shared", [
    (2, 3, 333, 64, True, True, False),
    (1, 4, 1000, 128, False, True, False),
    (2, 4, 5000, 64, True, True, True),
    (1, 2, 65, 128, True, False, False),
    (1, 3, 1, 64, True, True, False),
    (2, 8, 16384, 64, True, True, False),
    (2, 8, 8191, 128, False, True, True),
])
def test_scan_with_fused_key_rotation_equals_scan_then_pass(B, H, L, d, rotv, rotqk, shared):
    """arp_angle_scan_rotate_kv (the pass in the scan's epilogue) leaves theta
    and the workspace (k~, v~, per-tile key norms) bit-identical to
    arp_angle_scan followed by arp_rotate_kv, on ragged lengths, both head
    dims, shared angle streams, with and without value transport."""
    G = 1 if shared else H
    rng = np.random.default_rng(L + d)
    phi = to_dev((rng.standard_normal((B, G, L, d // 2)) * 0.5).astype(np.float32))
    k, v = (to_dev(wl.to_bf16_bits(rng.standard_normal((B, H, L, d)).astype(np.float32) * 0.4))
            for _ in range(2))
    flags = binding.flags_for(rotate_qk=rotqk, rotate_v=rotv, shared_phi=shared)
    desc = binding.make_desc(B, H, L, d, "bf16", flags)
    say(f"[gpu] scan+rotation B={B} H={H} L={L} d={d} rotv={rotv} rotqk={rotqk} shared={shared}")
    nbytes = binding.workspace_bytes(desc)
    ws_a = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    ws_b = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    th_a = binding.angle_scan(phi, desc)
    binding.rotate_kv(k, v, th_a, desc, ws=ws_a)
    th_b, _ = binding.angle_scan_rotate_kv(phi, k, v, desc, ws=ws_b)
    torch.cuda.synchronize()
    assert torch.equal(th_a.view(torch.int32), th_b.view(torch.int32))
    assert torch.equal(ws_a, ws_b)
