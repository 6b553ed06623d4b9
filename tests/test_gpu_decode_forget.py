"""GPU parity of decoding with forget gates (arp_decode_prefill_ex /
arp_decode_step_ex) against the fp64 oracle: decoding token t with the gates
of tokens 0..t must give row t of the whole-sequence gated forward (score
(i, j) plus sum_{s=j+1}^{i} log f_s, the PaTH reading notes' Sec. 2.5).

Gates: log f_t = log sigmoid(z), z ~ N(2, 1) (mostly open) or N(0, 1)
(strong forgetting), seeded.  Bar: the forward's bf16 bar, max |err| <= 2e-2;
the gate cache against the fp64 prefix of the gates within fp32 rounding."""
import numpy as np
import pytest
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import DEV, assert_close, oracle_flags, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _gates(w, seed=31, mean=2.0):
    z = np.random.default_rng(seed).normal(mean, 1.0, size=(w.batch, w.heads, w.seqlen))
    return (-np.logaddexp(0.0, -z)).astype(np.float32)  # log sigmoid(z)


def _decode(w, logf, t0, t1, *, rotate_v=False, alibi=False):
    """Prefill tokens [0, t0), decode t0..t1-1.  Returns (outputs [B, H, t1-t0, d],
    the gate cache [B, H, t1], the gate state [B, H])."""
    say(f"[gpu] gated decode {w.name} B={w.batch} H={w.heads} L={w.seqlen} d={w.head_dim} "
        f"prefill={t0} steps={t1 - t0} v={rotate_v} alibi={alibi}")
    q, k, v, phi = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi)
    lf = to_dev(logf)
    B, H, L, d = q.shape
    al = to_dev(wl.alibi_slopes(H)) if alibi else None
    flags = binding.flags_for(rotate_qk=True, rotate_v=rotate_v, alibi=alibi)
    cache = binding.DecodeCache(B, H, L, d, rotate_v=rotate_v, alibi=alibi, forget=True, device=DEV)
    if t0 > 0:
        th0 = binding.angle_scan(phi[:, :, :t0].contiguous(), binding.make_desc(B, H, t0, d, "bf16",
                                                                              flags))
        cache.prefill(k[:, :, :t0].contiguous(), v[:, :, :t0].contiguous(),
                      phi[:, :, :t0].contiguous(), th0, logf=lf[:, :, :t0].contiguous())
    else:
        cache.prefill()
    outs = []
    for t in range(t0, t1):
        o = cache.step(t, q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                       phi[:, :, t].contiguous(), alibi=al, logf=lf[:, :, t].contiguous())
        outs.append(o.clone())
    torch.cuda.synchronize()
    return (to_host(torch.stack(outs, dim=2)), cache.gcache[:, :, :t1].cpu().numpy(),
            cache.gstate.cpu().numpy())


def _check(w, logf, t0, t1, **flags):
    got, gc, gs = _decode(w, logf, t0, t1, **flags)
    # the gate cache (fp64) and state against the fp64 prefix sums of min(log f, 0)
    pre = np.cumsum(np.minimum(logf.astype(np.float64), 0.0), axis=2)[:, :, :t1]
    assert gc.dtype == np.float64
    assert np.all(np.abs(gc - pre * np.log2(np.e)) <= 1e-12 * np.maximum(1.0, np.abs(pre) * 1.45))
    assert np.all(np.abs(gs - pre[:, :, -1]) <= 1e-9 * np.maximum(1.0, np.abs(pre[:, :, -1])))
    rv, al = flags.get("rotate_v", False), flags.get("alibi", False)
    prob = oracle.Problem(w.q, w.k, w.v, w.phi, oracle_flags(True, rv, al) | oracle.FORGET,
                          alibi=wl.alibi_slopes(w.heads) if al else None, logf=logf)
    B, H, L, d = w.q.shape
    rows = np.array([(b * H + h) * L + t for b in range(B) for h in range(H) for t in range(t0, t1)])
    want = prob.rows(rows).reshape(B, H, t1 - t0, d)
    assert_close(got, want, "bf16", f"gated decode {w.name} [{t0}, {t1}) {flags}")


@pytest.mark.parametrize("alibi", [False, True])
@pytest.mark.parametrize("rotate_v", [False, True])
@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_gated_decode_from_empty_cache(name, rotate_v, alibi):
    w = wl.make(name, batch=2, heads=3, seqlen=70)
    _check(w, _gates(w), 0, 70, rotate_v=rotate_v, alibi=alibi)


@pytest.mark.parametrize("name", ["train_1k", "rope_8k_d128"])
def test_gated_decode_after_long_prompt(name):
    """A 600-token prompt (three chunks of the split-key pass, the prefill's
    gate scan over one 1024-token chunk) with strong forgetting, then 40
    steps."""
    w = wl.make(name, batch=1, heads=2, seqlen=640)
    _check(w, _gates(w, seed=32, mean=0.0), 600, 640, rotate_v=True)


def test_gated_decode_prompt_over_several_gate_chunks():
    """A 2100-token prompt: the prefill's gate scan carries over three chunks."""
    w = wl.make("train_1k", batch=1, heads=2, seqlen=2110)
    _check(w, _gates(w, seed=33), 2100, 2110, rotate_v=True, alibi=True)


def test_open_gates_decode_like_plain_decode():
    """log f = 0: the gate terms add exact zeros; outputs equal the ungated
    decode's bit for bit."""
    w = wl.make("train_1k", batch=1, heads=2, seqlen=80)
    logf = np.zeros((1, 2, 80), dtype=np.float32)
    got, _, _ = _decode(w, logf, 30, 80, rotate_v=True)
    q, k, v, phi = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.phi)
    flags = binding.flags_for(rotate_qk=True, rotate_v=True)
    cache = binding.DecodeCache(1, 2, 80, 64, rotate_v=True, device=DEV)
    th0 = binding.angle_scan(phi[:, :, :30].contiguous(), binding.make_desc(1, 2, 30, 64, "bf16", flags))
    cache.prefill(k[:, :, :30].contiguous(), v[:, :, :30].contiguous(), phi[:, :, :30].contiguous(), th0)
    outs = [cache.step(t, q[:, :, t].contiguous(), k[:, :, t].contiguous(), v[:, :, t].contiguous(),
                       phi[:, :, t].contiguous()).clone() for t in range(30, 80)]
    torch.cuda.synchronize()
    assert np.array_equal(got, to_host(torch.stack(outs, dim=2)))


def test_plain_decode_rejects_gates():
    d = binding.make_desc(1, 1, 64, 64, "bf16", binding.flags_for(forget=True))
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device=DEV)
    st = torch.zeros(1, 1, 32, dtype=torch.int64, device=DEV)
    with pytest.raises(binding.ArpError) as e:
        binding._check("arp_decode_prefill", binding.lib().arp_decode_prefill(
            __import__("ctypes").byref(d), 0, None, None, None, None, binding._ptr(x),
            binding._ptr(x), binding._ptr(st), binding._stream(DEV)))
    assert e.value.status == binding.ERR_INVALID_ARG
