"""Out-of-bounds writes: every buffer a kernel writes (outputs, angles, lse,
gradients, scan state, workspaces, decode caches and state) is placed between
two 4 KiB guard bands of a known byte pattern, the entry point is called
through the C ABI on ragged shapes (lengths that are not a multiple of any
tile, so padded and partial tiles are written), and after the copy back both
bands must still hold the pattern.  The guarded results must also equal the
same calls on plain buffers bit for bit (the guards change nothing else).

The path is the one the other GPU tests check against the oracle; this file
checks only where the kernels write."""
import ctypes

import numpy as np
import pytest
import torch

from accumulated_rotation_positional_amd import binding as b
from accumulated_rotation_positional_amd import workloads as wl
from gpu_util import DEV, say, to_dev

pytestmark = pytest.mark.gpu

G = 4096          # guard band bytes on each side (a multiple of 256: alignment is kept)
PATTERN = 0xA5


class Guarded:
    """A tensor of `shape` and `dtype` in the middle of a byte buffer whose
    first and last G bytes hold PATTERN (the tensor itself starts as `fill`)."""

    def __init__(self, name, shape, dtype, fill=None):
        self.name = name
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.raw = torch.full((n + 2 * G,), PATTERN, dtype=torch.uint8, device=DEV)
        self.t = self.raw[G:G + n].view(dtype).view(shape)
        if fill is not None:
            self.t.fill_(fill)

    @property
    def ptr(self):
        return self.t.data_ptr()

    def check(self):
        lo = self.raw[:G].cpu().numpy()
        hi = self.raw[G + self.n:].cpu().numpy()
        bad_lo = np.flatnonzero(lo != PATTERN)
        bad_hi = np.flatnonzero(hi != PATTERN)
        assert bad_lo.size == 0, f"{self.name}: {bad_lo.size} bytes written below the buffer " \
                                 f"(first at -{G - bad_lo[0]})"
        assert bad_hi.size == 0, f"{self.name}: {bad_hi.size} bytes written past the end " \
                                 f"(first at +{bad_hi[0]})"


def _bytes_buffer(name, nbytes, zero=False):
    return Guarded(name, (max(int(nbytes), 256),), torch.uint8, 0 if zero else None)


def _inputs(name, B, H, L, seed=0):
    w = wl.make(name, batch=B, heads=H, seqlen=L)
    q, k, v, phi = (to_dev(getattr(w, n)) for n in ("q", "k", "v", "phi"))
    return w, q, k, v, phi


def _check_all(bufs):
    torch.cuda.synchronize()
    for g in bufs:
        g.check()


@pytest.mark.parametrize("name,L,flags", [
    ("train_1k", 333, dict(rotate_v=True, alibi=True, forget=True)),
    ("rope_8k_d128", 201, dict(rotate_v=False, alibi=False, forget=True)),
    ("train_1k", 97, dict(rotate_v=True, alibi=False, forget=False)),
])
def test_forward_and_backward_write_inside_their_buffers(name, L, flags):
    B, H = 2, 3
    w, q, k, v, phi = _inputs(name, B, H, L)
    d = w.head_dim
    say(f"[gpu] guard bands forward/backward {name} L={L} {flags}")
    al = to_dev(wl.alibi_slopes(H)) if flags["alibi"] else None
    logf = None
    if flags["forget"]:
        z = np.random.default_rng(3).standard_normal((B, H, L)).astype(np.float32) + 1.0
        logf = to_dev((-np.log1p(np.exp(-z))).astype(np.float32))
    fl = b.flags_for(rotate_v=flags["rotate_v"], alibi=flags["alibi"], forget=flags["forget"])
    desc = b.desc_for(q, fl)
    L_ = b.lib()
    theta = Guarded("theta", phi.shape, torch.float32)
    o = Guarded("o", q.shape, torch.bfloat16)
    lse = Guarded("lse", (B, H, L), torch.float32)
    state = _bytes_buffer("scan state", b.scan_state_bytes(desc), zero=True)
    ws = _bytes_buffer("workspace", b.workspace_bytes(desc))
    st = b._stream(DEV)
    b._check("arp_forward_ex", L_.arp_forward_ex(
        ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), phi.data_ptr(), b._ptr(al),
        b._ptr(logf), theta.ptr, o.ptr, lse.ptr, state.ptr, state.n, ws.ptr, ws.n, st))
    _check_all([theta, o, lse, state, ws])
    # the same call on plain buffers
    o_ref, th_ref, lse_ref = b.forward_ex(q, k, v, phi, rotate_v=flags["rotate_v"], alibi=al,
                                          logf=logf, with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o.t, o_ref) and torch.equal(theta.t, th_ref) and torch.equal(lse.t, lse_ref)

    dout = to_dev(wl.to_bf16_bits(np.random.default_rng(5).standard_normal(q.shape)
                                  .astype(np.float32) * 0.1))
    dq = Guarded("dq", q.shape, torch.bfloat16)
    dk = Guarded("dk", q.shape, torch.bfloat16)
    dv = Guarded("dv", q.shape, torch.bfloat16)
    dtheta = Guarded("dtheta", (B, H, L, d // 2), torch.float32)
    dphi = Guarded("dphi", phi.shape, torch.float32)
    dlogf = Guarded("dlogf", (B, H, L), torch.float32) if logf is not None else None
    bws = _bytes_buffer("backward workspace", b.backward_workspace_bytes(desc))
    b._check("arp_backward_ex", L_.arp_backward_ex(
        ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), theta.ptr, b._ptr(al),
        b._ptr(logf), o.ptr, lse.ptr, dout.data_ptr(), dq.ptr, dk.ptr, dv.ptr, dtheta.ptr,
        dphi.ptr, dlogf.ptr if dlogf is not None else None, bws.ptr, bws.n, st))
    outs = [dq, dk, dv, dtheta, dphi, bws] + ([dlogf] if dlogf is not None else [])
    _check_all(outs)
    ref = b.backward_ex(desc, q, k, v, phi, th_ref, o_ref, lse_ref, dout, alibi=al, logf=logf)
    torch.cuda.synchronize()
    for g, r in zip([dq, dk, dv, dphi, dtheta], ref[:5]):
        assert torch.equal(g.t, r), g.name
    if dlogf is not None:
        assert torch.equal(dlogf.t, ref[5])


@pytest.mark.parametrize("L", [97, 333])
def test_fp32_and_fused_paths_write_inside_their_buffers(L):
    B, H = 1, 3
    st = b._stream(DEV)
    L_ = b.lib()
    # fp32 I/O: forward and backward
    w, q, k, v, phi = _inputs("tiny_f32", B, H, L)
    phi = to_dev(wl.make("train_1k", batch=B, heads=H, seqlen=L).phi)
    say(f"[gpu] guard bands fp32 L={L}")
    desc = b.desc_for(q, b.flags_for(rotate_v=True, alibi=False))
    theta = Guarded("theta", phi.shape, torch.float32)
    o = Guarded("o", q.shape, torch.float32)
    lse = Guarded("lse", (B, H, L), torch.float32)
    state = _bytes_buffer("scan state", b.scan_state_bytes(desc), zero=True)
    ws = _bytes_buffer("workspace", b.workspace_bytes(desc))
    b._check("arp_forward_train", L_.arp_forward_train(
        ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), phi.data_ptr(), None,
        theta.ptr, o.ptr, lse.ptr, state.ptr, state.n, ws.ptr, ws.n, st))
    _check_all([theta, o, lse, state, ws])
    dout = torch.randn(q.shape, device=DEV, generator=torch.Generator(device=DEV).manual_seed(1))
    grads = [Guarded(n, q.shape, torch.float32) for n in ("dq", "dk", "dv")]
    dtheta = Guarded("dtheta", phi.shape, torch.float32)
    dphi = Guarded("dphi", phi.shape, torch.float32)
    bws = _bytes_buffer("backward workspace", b.backward_workspace_bytes(desc))
    b._check("arp_backward", L_.arp_backward(
        ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), theta.ptr, None, o.ptr,
        lse.ptr, dout.data_ptr(), grads[0].ptr, grads[1].ptr, grads[2].ptr, dtheta.ptr, dphi.ptr,
        bws.ptr, bws.n, st))
    _check_all(grads + [dtheta, dphi, bws])

    # bf16 with the rotation fused into the attention kernel's staging
    w, q, k, v, phi = _inputs("train_1k", B, H, L)
    desc = b.desc_for(q, b.flags_for(rotate_v=True, alibi=True, fused=True))
    al = to_dev(wl.alibi_slopes(H))
    theta = Guarded("theta", phi.shape, torch.float32)
    o = Guarded("o", q.shape, torch.bfloat16)
    state = _bytes_buffer("scan state", b.scan_state_bytes(desc), zero=True)
    ws = _bytes_buffer("workspace", b.workspace_bytes(desc))
    b._check("arp_forward", L_.arp_forward(
        ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), phi.data_ptr(), al.data_ptr(),
        theta.ptr, o.ptr, state.ptr, state.n, ws.ptr, ws.n, st))
    _check_all([theta, o, state, ws])
    o_ref, _ = b.forward(q, k, v, phi, rotate_v=True, alibi=al, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(o.t, o_ref)


def test_angle_generators_write_inside_their_buffers():
    B, H, L, d = 2, 3, 301, 64
    P = d // 2
    st = b._stream(DEV)
    L_ = b.lib()
    desc = b.make_desc(B, H, L, d, torch.bfloat16, b.flags_for())
    say("[gpu] guard bands angle generators")
    bound = torch.full((H, P), 0.3, dtype=torch.float32, device=DEV)
    theta = Guarded("theta (random)", (B, H, L, P), torch.float32)
    state = _bytes_buffer("scan state", b.scan_state_bytes(desc), zero=True)
    b._check("arp_angle_scan_random", L_.arp_angle_scan_random(
        ctypes.byref(desc), ctypes.c_uint64(7), ctypes.c_uint64(3), bound.data_ptr(), theta.ptr,
        state.ptr, state.n, st))
    phi = Guarded("phi (random)", (B, H, L, P), torch.float32)
    b._check("arp_random_phi", L_.arp_random_phi(
        ctypes.byref(desc), ctypes.c_uint64(7), ctypes.c_uint64(3), bound.data_ptr(), phi.ptr, st))
    _check_all([theta, state, phi])
    vocab = 50
    tokens = torch.randint(0, vocab, (B, L), dtype=torch.int32, device=DEV,
                           generator=torch.Generator(device=DEV).manual_seed(2))
    table = torch.rand(vocab, H, P, dtype=torch.float32, device=DEV,
                       generator=torch.Generator(device=DEV).manual_seed(3))
    theta2 = Guarded("theta (tokens)", (B, H, L, P), torch.float32)
    b._check("arp_angle_scan_tokens", L_.arp_angle_scan_tokens(
        ctypes.byref(desc), tokens.data_ptr(), table.data_ptr(), ctypes.c_int64(vocab), theta2.ptr,
        state.ptr, state.n, st))
    freq = torch.rand(H, P, dtype=torch.float32, device=DEV,
                      generator=torch.Generator(device=DEV).manual_seed(4))
    theta3 = Guarded("theta (constant)", (B, H, L, P), torch.float32)
    b._check("arp_angle_scan_const", L_.arp_angle_scan_const(
        ctypes.byref(desc), freq.data_ptr(), theta3.ptr, st))
    _check_all([theta2, theta3, state])


@pytest.mark.parametrize("forget", [False, True])
def test_decode_writes_inside_its_cache(forget):
    B, H, cap, d = 2, 3, 141, 64
    t0 = 70
    w, q, k, v, phi = _inputs("train_1k", B, H, cap)
    say(f"[gpu] guard bands decode forget={forget}")
    fl = b.flags_for(rotate_v=True, alibi=True, forget=forget)
    desc = b.make_desc(B, H, cap, d, torch.bfloat16, fl)
    st = b._stream(DEV)
    L_ = b.lib()
    al = to_dev(wl.alibi_slopes(H))
    kc = Guarded("kcache", (B, H, cap, d), torch.bfloat16, 0)
    vc = Guarded("vcache", (B, H, cap, d), torch.bfloat16, 0)
    state = Guarded("angle state", (B, H, d // 2), torch.int64, 0)
    theta = Guarded("token theta", (B, H, d // 2), torch.float32, 0)
    gc = Guarded("gate cache", (B, H, cap), torch.float64, 0) if forget else None
    gs = Guarded("gate state", (B, H), torch.float64, 0) if forget else None
    ws = _bytes_buffer("decode workspace", L_.arp_decode_workspace_bytes(ctypes.byref(desc)))
    out = Guarded("o", (B, H, d), torch.bfloat16)
    z = np.random.default_rng(4).standard_normal((B, H, cap)).astype(np.float32) + 1.5
    logf = to_dev((-np.log1p(np.exp(-z))).astype(np.float32))
    pdesc = b.make_desc(B, H, t0, d, torch.bfloat16, fl)
    th0 = b.angle_scan(phi[:, :, :t0].contiguous(), pdesc)
    kp, vp, pp = (x[:, :, :t0].contiguous() for x in (k, v, phi))
    lp = logf[:, :, :t0].contiguous()
    if forget:
        b._check("arp_decode_prefill_ex", L_.arp_decode_prefill_ex(
            ctypes.byref(desc), t0, kp.data_ptr(), vp.data_ptr(), pp.data_ptr(), th0.data_ptr(),
            lp.data_ptr(), kc.ptr, vc.ptr, state.ptr, gc.ptr, gs.ptr, st))
    else:
        b._check("arp_decode_prefill", L_.arp_decode_prefill(
            ctypes.byref(desc), t0, kp.data_ptr(), vp.data_ptr(), pp.data_ptr(), th0.data_ptr(),
            kc.ptr, vc.ptr, state.ptr, st))
    torch.cuda.synchronize()
    for t in range(t0, cap):
        qt, kt, vt, pt = (x[:, :, t].contiguous() for x in (q, k, v, phi))
        if forget:
            lt = logf[:, :, t].clone()
            b._check("arp_decode_step_ex", L_.arp_decode_step_ex(
                ctypes.byref(desc), t, qt.data_ptr(), kt.data_ptr(), vt.data_ptr(), pt.data_ptr(),
                al.data_ptr(), lt.data_ptr(), state.ptr, theta.ptr, kc.ptr, vc.ptr, gc.ptr, gs.ptr,
                out.ptr, ws.ptr, ws.n, st))
        else:
            b._check("arp_decode_step", L_.arp_decode_step(
                ctypes.byref(desc), t, qt.data_ptr(), kt.data_ptr(), vt.data_ptr(), pt.data_ptr(),
                al.data_ptr(), state.ptr, theta.ptr, kc.ptr, vc.ptr, out.ptr, ws.ptr, ws.n, st))
        torch.cuda.synchronize()
    _check_all([kc, vc, state, theta, ws, out] + ([gc, gs] if forget else []))
