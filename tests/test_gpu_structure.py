"""Structural properties of the GPU path that must hold bit for bit:
causality (outputs of rows <= i ignore keys, values and angles after i),
index layout (each (batch, head) reads its own slice), the first row, and
run-to-run determinism."""
import numpy as np
import pytest
import torch

from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import DEV, run_forward, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128", "tiny_f32"])
@pytest.mark.parametrize("cut", [1, 100, 256, 300])
def test_causal_mask_is_exact(name, cut):
    w = wl.make(name, batch=1, heads=2, seqlen=600)
    base, _ = run_forward(w, rotate_v=True, alibi=True)
    rng = np.random.Generator(np.random.PCG64(cut))
    for f in ("k", "v"):
        a = getattr(w, f).copy()
        if a.dtype == np.uint16:
            a[:, :, cut:] = wl.to_bf16_bits(rng.standard_normal(a[:, :, cut:].shape).astype(np.float32))
        else:
            a[:, :, cut:] = rng.standard_normal(a[:, :, cut:].shape).astype(np.float32)
        setattr(w, f, a)
    w.phi = w.phi.copy()
    w.phi[:, :, cut:] += np.float32(0.7)
    other, _ = run_forward(w, rotate_v=True, alibi=True)
    assert np.array_equal(other[:, :, :cut], base[:, :, :cut])
    assert not np.array_equal(other[:, :, cut:], base[:, :, cut:])


@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128", "tiny_f32"])
def test_index_layout_per_head_tags(name):
    """v[b, h, :, :] = tag(b, h) with distinct small integers and no value
    rotation: every output row of (b, h) is its tag (up to rounding), so any
    mix-up of batch, head or position indexing shows."""
    w = wl.make(name, batch=3, heads=5, seqlen=260)
    tags = np.arange(1, 16, dtype=np.float32).reshape(3, 5, 1, 1) * np.float32(0.25)
    v = np.broadcast_to(tags, w.v.shape).astype(np.float32)
    w.v = wl.to_bf16_bits(v) if w.v.dtype == np.uint16 else v
    got, _ = run_forward(w, rotate_v=False)
    assert np.array_equal(np.round(got * 4), np.broadcast_to(tags * 4, got.shape))
    assert float(np.abs(got - tags).max()) < 1e-5


@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128", "tiny_f32"])
def test_first_row_is_first_value(name):
    w = wl.make(name, batch=2, heads=2, seqlen=130)
    got, _ = run_forward(w, rotate_v=False)
    v0 = w.values("v")[:, :, 0]
    assert np.array_equal(got[:, :, 0], v0)
    got_v, _ = run_forward(w, rotate_v=True)
    assert float(np.abs(got_v[:, :, 0] - v0).max()) < 1e-2 * max(1e-3, float(np.abs(v0).max()))


@pytest.mark.parametrize("name", ["extrap_16k", "tiny_f32"])
def test_deterministic(name):
    w = wl.make(name, seqlen=4096 if name == "extrap_16k" else 256)
    a, ta = run_forward(w)
    b, tb = run_forward(w)
    assert np.array_equal(a, b) and np.array_equal(ta, tb)


def test_step_entry_points_compose_to_forward():
    """arp_angle_scan -> arp_rotate_kv -> arp_attn_rotated gives exactly
    arp_forward's output (the benchmark times the steps separately), with
    value transport (v~ from the pass) and without (the caller's v read by the
    attention kernel)."""
    w = wl.make("extrap_16k", seqlen=2048)
    q, k, v, phi = (to_dev(getattr(w, n)) for n in ("q", "k", "v", "phi"))
    for rv in (True, False):
        say(f"[gpu] step entry points rotate_v={rv}")
        o_fwd, th_fwd = binding.forward(q, k, v, phi, rotate_v=rv)
        desc = binding.desc_for(q, binding.flags_for(rotate_v=rv))
        ws = binding.workspace(desc, DEV)
        theta = binding.angle_scan(phi, desc)
        binding.rotate_kv(k, v, theta, desc, ws=ws)
        o = torch.empty_like(q)
        binding.attn_rotated(q, v, theta, None, o, desc, ws)
        torch.cuda.synchronize()
        assert torch.equal(theta, th_fwd)
        assert torch.equal(o, o_fwd)
