"""arp_forward_noalloc (the forward whose scan state and operand workspace live
in the library's own device array) against arp_forward with caller buffers,
called through the C ABI.  Both run the same kernels on the same inputs, so the
outputs and angles must agree bit for bit (stricter than the bf16 bar).  Calls
in a row of different sizes share the array: a smaller problem after a larger
one must still be exact (the scan state is reused, not re-cleared)."""
import numpy as np
import pytest
import torch

from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _pair(w, **kw):
    q, k, v, phi = (to_dev(getattr(w, n)) for n in ("q", "k", "v", "phi"))
    al = to_dev(wl.alibi_slopes(w.heads)) if kw.pop("alibi", False) else None
    say(f"[gpu] noalloc {w.name} B={w.batch} H={w.heads} L={w.seqlen} d={w.head_dim} {kw} "
        f"alibi={al is not None}")
    o1, th1 = binding.forward_noalloc(q, k, v, phi, alibi=al, **kw)
    o2, th2 = binding.forward(q, k, v, phi, alibi=al, **kw)
    torch.cuda.synchronize()
    return to_host(o1), th1.cpu().numpy(), to_host(o2), th2.cpu().numpy()


def _assert_same(w, **kw):
    o1, th1, o2, th2 = _pair(w, **kw)
    assert np.all(np.isfinite(o1))
    assert np.array_equal(th1.view(np.uint32), th2.view(np.uint32))
    assert np.array_equal(o1, o2), float(np.abs(o1 - o2).max())


def test_noalloc_matches_forward_on_calls_of_shrinking_size():
    # a larger problem first, then a smaller one on the same scratch
    _assert_same(wl.make("train_1k", batch=2, heads=4, seqlen=1000), rotate_v=True, alibi=True)
    _assert_same(wl.make("rope_8k_d128", batch=1, heads=2, seqlen=300), rotate_v=True)
    _assert_same(wl.make("train_1k", batch=1, heads=1, seqlen=65), exclusive=True)


def test_noalloc_fused_and_fp32_paths():
    # the fused rotation needs no operand workspace: a long sequence fits
    _assert_same(wl.make("extrap_16k", batch=1, heads=4, seqlen=8192), rotate_v=True, fused=True)
    _assert_same(wl.make("tiny_f32", batch=1, heads=2, seqlen=256), rotate_v=True)
    _assert_same(wl.make("train_1k", batch=8, heads=8, seqlen=1024))  # the training shape


def test_noalloc_rejects_problems_beyond_its_scratch():
    w = wl.make("extrap_16k", batch=2, heads=8, seqlen=16384)
    q, k, v, phi = (to_dev(getattr(w, n)) for n in ("q", "k", "v", "phi"))
    with pytest.raises(binding.ArpError) as e:
        binding.forward_noalloc(q, k, v, phi, rotate_v=True)  # 96 MiB of operands
    assert e.value.status == binding.ERR_SCRATCH
    o, _ = binding.forward_noalloc(q, k, v, phi, rotate_v=True, fused=True)  # no operands
    ref, _ = binding.forward(q, k, v, phi, rotate_v=True, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
