"""The angle scan's fallback path, deterministically.

In the normal build a chunk's look-back reduces a predecessor chunk from its
source only when that predecessor has published nothing for 256 polls, which
depends on scheduling.  The test variant libarp_scan_from_source.so (the same
sources, angle scan compiled with ARP_SCAN_FALLBACK_POLLS=0) ignores every
published prefix and reduces each predecessor from its source, so that the
fallback's reduction (reduce_pair, the half-wave combine of two lanes per pair
at head_dim 64) produces every chunk's prefix.  Fixed-point sums are exact, so
its angles must equal the normal build's bit for bit, for every source (phi,
Philox draws, token table), both pair counts, shared and per-head angles, and
the exclusive scan; and both must equal the oracle's within the scan bar."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import build as hip_build
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import DEV, F32_TOL, circular_err, say, to_dev

pytestmark = pytest.mark.gpu

_VARIANT = None


def variant():
    global _VARIANT
    if _VARIANT is None:
        _VARIANT = binding.open_library(hip_build.SCAN_TEST_TARGET)
    return _VARIANT


def _scan(lib, fn, desc, *args):
    theta = torch.empty(binding._phi_shape(desc), dtype=torch.float32, device=DEV)
    state = torch.zeros(max(binding.scan_state_bytes(desc), 256), dtype=torch.uint8, device=DEV)
    binding._check(fn, getattr(lib, fn)(ctypes.byref(desc), *args, theta.data_ptr(),
                                        state.data_ptr(), state.numel(), binding._stream(DEV)))
    torch.cuda.synchronize()
    return theta.cpu().numpy()


CASES = [  # B, H, L, P, shared, exclusive
    (2, 3, 20000, 32, False, False),
    (1, 2, 9001, 64, False, True),
    (2, 4, 12345, 32, True, False),
    (1, 3, 5000, 64, True, False),
    (1, 2, 100, 32, False, False),
]


@pytest.mark.parametrize("B,H,L,P,shared,excl", CASES)
def test_scan_from_source_matches_normal_build(B, H, L, P, shared, excl):
    G = 1 if shared else H
    desc = binding.make_desc(B, H, L, 2 * P, "bf16",
                             binding.flags_for(shared_phi=shared, exclusive=excl))
    say(f"[gpu] scan from source B={B} H={H} L={L} P={P} shared={shared} exclusive={excl}")
    rng = np.random.default_rng(L)
    # phi source: learned-style steps of mixed sign and size
    phi = (rng.standard_normal((B, G, L, P)) * 0.7).astype(np.float32)
    phi_d = to_dev(phi)  # held: a temporary's memory could be handed to theta
    a = _scan(binding.lib(), "arp_angle_scan", desc, phi_d.data_ptr())
    b = _scan(variant(), "arp_angle_scan", desc, phi_d.data_ptr())
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert circular_err(a, oracle.angle_scan(phi, exclusive=excl)) <= F32_TOL

    # Philox draws generated inside the scan
    bound = to_dev((wl.rope_frequencies(2 * P)[None, :] *
                    rng.uniform(0.5, 2.0, size=(G, 1))).astype(np.float32))
    seed, step = ctypes.c_uint64(0x1234567887654321), ctypes.c_uint64(99)
    a = _scan(binding.lib(), "arp_angle_scan_random", desc, seed, step, bound.data_ptr())
    b = _scan(variant(), "arp_angle_scan_random", desc, seed, step, bound.data_ptr())
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))

    # token table
    vocab = 77
    tokens = rng.integers(0, vocab, size=(B, L)).astype(np.int32)
    table = (rng.standard_normal((vocab, G, P)) * 0.5).astype(np.float32)
    td, tt = to_dev(tokens), to_dev(table)
    a = _scan(binding.lib(), "arp_angle_scan_tokens", desc, td.data_ptr(), tt.data_ptr(),
              ctypes.c_int64(vocab))
    b = _scan(variant(), "arp_angle_scan_tokens", desc, td.data_ptr(), tt.data_ptr(),
              ctypes.c_int64(vocab))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert circular_err(a, oracle.angle_scan(oracle.token_phi(tokens, table), exclusive=excl)) \
        <= F32_TOL


def test_variant_is_a_separate_build():
    assert os.path.exists(hip_build.SCAN_TEST_TARGET)
    assert os.path.realpath(hip_build.SCAN_TEST_TARGET) != os.path.realpath(binding.LIB_PATH)
    assert variant().arp_abi_version() == binding.ABI_VERSION
