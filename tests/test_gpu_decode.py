"""GPU parity of decoding with a streaming angle state against the fp64
oracle: decoding token t must give row t of the whole-sequence forward
("Why Do Accumulated Transformations Extrapolate?" eq. (2)-(4), causal), and
its angles must equal the full-sequence scan's bit for bit (both sum the same
48-bit fixed-point turns).

Bars: bf16 outputs max |err| <= 2e-2 (the forward's bar); angles bit-exact
against the library's own full scan and within 1e-4 (circular) of the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import DEV, assert_close, circular_err, oracle_problem, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _decode(w, t0, t1, *, rotate_qk=True, rotate_v=False, alibi=False, exclusive=False):
    """Prefill tokens [0, t0) through the library's scan, then decode t0..t1-1.
    Returns (outputs [B, H, t1-t0, d], decoded angles [B, Hphi, t1-t0, P], full-scan angles)."""
    say(f"[gpu] decode {w.name} B={w.batch} H={w.heads} L={w.seqlen} d={w.head_dim} "
        f"prefill={t0} steps={t1 - t0} qk={rotate_qk} v={rotate_v} alibi={alibi} excl={exclusive}")
    q, k, v, phi = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi)
    B, H, L, d = q.shape
    hphi = phi.shape[1]
    al = to_dev(wl.alibi_slopes(H)) if alibi else None
    flags = binding.flags_for(rotate_qk=rotate_qk, rotate_v=rotate_v, alibi=alibi,
                              shared_phi=hphi == 1 and H != 1, exclusive=exclusive)
    full_theta = binding.angle_scan(phi, binding.make_desc(B, H, L, d, "bf16", flags))
    cache = binding.DecodeCache(B, H, L, d, phi_heads=hphi, rotate_qk=rotate_qk, rotate_v=rotate_v,
                                alibi=alibi, exclusive=exclusive, device=DEV)
    if t0 > 0:
        pd = binding.make_desc(B, H, t0, d, "bf16", flags)
        th0 = binding.angle_scan(phi[:, :, :t0].contiguous(), pd)
        cache.prefill(k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous(),
                      phi[:, :, :t0].contiguous(), th0)
    else:
        cache.prefill()
    outs, thetas = [], []
    for t in range(t0, t1):
        o = cache.step(t, q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                       phi[:, :, t].contiguous(), alibi=al)
        outs.append(o.clone())
        thetas.append(cache.theta.clone())
    torch.cuda.synchronize()
    return (to_host(torch.stack(outs, dim=2)), torch.stack(thetas, dim=2).cpu().numpy(),
            full_theta.cpu().numpy())


def _check(w, t0, t1, **flags):
    got, th, full = _decode(w, t0, t1, **flags)
    assert np.array_equal(th.view(np.uint32), full[:, :, t0:t1].view(np.uint32)), \
        "decoded angles differ from the full scan's"
    ref_th = oracle.angle_scan(w.phi, exclusive=flags.get("exclusive", False))[:, :, t0:t1]
    assert circular_err(th, ref_th) <= 1e-4
    prob = oracle_problem(w, rotate_qk=flags.get("rotate_qk", True),
                          rotate_v=flags.get("rotate_v", False), alibi=flags.get("alibi", False),
                          exclusive=flags.get("exclusive", False))
    B, H, L, d = w.q.shape
    rows = np.array([(b * H + h) * L + t for b in range(B) for h in range(H) for t in range(t0, t1)])
    want = prob.rows(rows).reshape(B, H, t1 - t0, d)
    assert_close(got, want, "bf16", f"decode {w.name} [{t0}, {t1}) {flags}")


@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_decode_from_empty_cache(name):
    w = wl.make(name, batch=2, heads=3, seqlen=70)
    _check(w, 0, 70, rotate_qk=True, rotate_v=True)


FLAG_SETS = [
    dict(rotate_qk=True),
    dict(rotate_qk=True, rotate_v=True),
    dict(rotate_qk=True, rotate_v=True, alibi=True),
    dict(rotate_qk=False, rotate_v=False),
    dict(rotate_qk=True, rotate_v=True, exclusive=True),
]


@pytest.mark.parametrize("flags", FLAG_SETS, ids=lambda f: "-".join(k for k, v in f.items() if v) or "nope")
@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_prefill_then_decode(name, flags):
    w = wl.make(name, batch=2, heads=2, seqlen=620)
    _check(w, 600, 620, **flags)


def test_decode_shared_angle_heads():
    w = wl.make("train_1k", batch=2, heads=4, seqlen=300)
    w.phi = np.ascontiguousarray(w.phi[:, :1])
    _check(w, 257, 300, rotate_qk=True, rotate_v=True)


def test_decode_long_context():
    """extrap_16k's shape (B=2, H=8, d=64): a 16380-token prompt, then the last
    four tokens decoded one by one (rows checked against the oracle)."""
    w = wl.make("extrap_16k")
    _check(w, 16380, 16384, rotate_qk=True, rotate_v=True)
