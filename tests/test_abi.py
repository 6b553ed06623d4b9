"""The C ABI of libarp.so, on the CPU: the library loads, exports every
function include/arp.h declares, and rejects bad arguments on the host before
anything is enqueued (every call below fails validation, so no kernel is ever
launched and no GPU is needed)."""
import ctypes
import os
import re

import pytest

from accumulated_rotation_positional_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "arp.h")


def _declared():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(arp_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared()
    assert set(names) == set(b.EXPORTS), names
    lib = ctypes.CDLL(b.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    L = b.lib()
    assert L.arp_abi_version() == 2
    for s in range(7):
        assert L.arp_status_string(s) != b"unknown status"
    assert L.arp_status_string(99) == b"unknown status"


def _desc(**kw):
    base = dict(batch=2, heads=8, seqlen=1024, head_dim=64, dtype="bf16", flags=b.ROTATE_QK)
    base.update(kw)
    return b.make_desc(base["batch"], base["heads"], base["seqlen"], base["head_dim"],
                       base["dtype"], base["flags"])


@pytest.mark.parametrize("kw,status", [
    (dict(), b.OK),
    (dict(dtype="f32"), b.OK),
    (dict(head_dim=128), b.OK),
    (dict(batch=0), b.ERR_INVALID_ARG),
    (dict(heads=-1), b.ERR_INVALID_ARG),
    (dict(seqlen=0), b.ERR_INVALID_ARG),
    (dict(head_dim=63), b.ERR_INVALID_ARG),
    (dict(head_dim=96), b.ERR_UNSUPPORTED),
    (dict(head_dim=32), b.ERR_UNSUPPORTED),
    (dict(flags=0x80), b.ERR_INVALID_ARG),
    (dict(seqlen=(1 << 24) + 1), b.ERR_INVALID_ARG),
])
def test_check_descriptor(kw, status):
    d = _desc(**kw)
    assert b.lib().arp_check(ctypes.byref(d)) == status


def test_check_rejects_bad_dtype_reserved_scale_and_null():
    L = b.lib()
    d = _desc()
    d.dtype = 7
    assert L.arp_check(ctypes.byref(d)) == b.ERR_INVALID_ARG
    d = _desc()
    d.reserved = 1
    assert L.arp_check(ctypes.byref(d)) == b.ERR_INVALID_ARG
    d = _desc()
    d.scale = float("nan")
    assert L.arp_check(ctypes.byref(d)) == b.ERR_INVALID_ARG
    d.scale = float("inf")
    assert L.arp_check(ctypes.byref(d)) == b.ERR_INVALID_ARG
    assert L.arp_check(None) == b.ERR_INVALID_ARG


def test_workspace_and_scan_state_bytes():
    L = b.lib()
    d = _desc(batch=2, heads=8, seqlen=16384)
    ws = L.arp_workspace_bytes(ctypes.byref(d))
    operands = 2 * 8 * 16384 * 64 * 2   # k~ only: q is rotated by the attention kernel, v read there
    kmax = 2 * 8 * (16384 // 64) * 4  # max |k~| per 64-key tile, fp32
    assert operands + kmax <= ws < operands + kmax + 4096 and ws % 256 == 0
    transported = _desc(batch=2, heads=8, seqlen=16384, flags=b.ROTATE_QK | b.ROTATE_V)
    assert L.arp_workspace_bytes(ctypes.byref(transported)) == ws + operands  # + v~
    st = L.arp_scan_state_bytes(ctypes.byref(d))
    assert 0 < st < (16 << 20) and st % 256 == 0
    fused = _desc(batch=2, heads=8, seqlen=16384, flags=b.ROTATE_QK | b.FUSED_ROTATION)
    assert L.arp_workspace_bytes(ctypes.byref(fused)) == 0
    assert L.arp_workspace_bytes(ctypes.byref(_desc(dtype="f32"))) == 0
    bad = _desc(head_dim=63)
    assert L.arp_workspace_bytes(ctypes.byref(bad)) == 0
    assert L.arp_scan_state_bytes(ctypes.byref(bad)) == 0
    # shared angle heads need state for one angle head per batch only
    shared = _desc(batch=2, heads=8, seqlen=16384, flags=b.ROTATE_QK | b.PHI_SHARED_HEADS)
    assert L.arp_scan_state_bytes(ctypes.byref(shared)) < st


# Fake device addresses: never dereferenced, because every call fails validation.
A = 0x10000          # 16-byte aligned
M = 0x10004          # misaligned


def test_entry_points_reject_null_and_misaligned_pointers():
    L = b.lib()
    d = _desc()
    big = L.arp_workspace_bytes(ctypes.byref(d))
    st = L.arp_scan_state_bytes(ctypes.byref(d))
    by = ctypes.byref(d)
    assert L.arp_angle_scan(by, None, A, A, st, None) == b.ERR_INVALID_ARG
    assert L.arp_angle_scan(by, M, A, A, st, None) == b.ERR_ALIGNMENT
    assert L.arp_angle_scan(by, A, A, None, st, None) == b.ERR_WORKSPACE
    assert L.arp_angle_scan(by, A, A, A, 16, None) == b.ERR_WORKSPACE
    assert L.arp_angle_scan(by, A, A, A + 16, st, None) == b.ERR_ALIGNMENT
    assert L.arp_rotate_kv(by, None, A, A, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_rotate_kv(by, A, M, A, A, big, None) == b.ERR_ALIGNMENT
    assert L.arp_rotate_kv(by, A, A, None, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_attn_rotated(by, A, A, A, None, None, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_attn_rotated(by, A, A, A, None, A, A, 8, None) == b.ERR_WORKSPACE
    # without value transport the attention reads the caller's v: required
    assert L.arp_attn_rotated(by, A, None, A, None, A, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_attn_rotated(by, None, A, A, None, A, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_attn_fwd(by, A, A, A, A, None, None, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_attn_fwd(by, A, A, A, A, None, M, A, big, None) == b.ERR_ALIGNMENT
    assert L.arp_forward(by, A, A, A, None, None, A, A, A, st, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_forward(by, A, A, A, A, None, None, A, A, st, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_forward(by, A, A, A, A, None, A, A, A, st, A, 0, None) == b.ERR_WORKSPACE
    assert L.arp_forward(by, A, A, A, A, None, A, A, A, 0, A, big, None) == b.ERR_WORKSPACE
    assert L.arp_rotate(by, A, None, A, 0, None) == b.ERR_INVALID_ARG
    assert L.arp_rotate(by, A, A, M, 0, None) == b.ERR_ALIGNMENT


def test_alibi_requires_slopes_and_rotation_requires_theta():
    L = b.lib()
    d = _desc(flags=b.ROTATE_QK | b.ALIBI)
    big = L.arp_workspace_bytes(ctypes.byref(d))
    st = L.arp_scan_state_bytes(ctypes.byref(d))
    by = ctypes.byref(d)
    assert L.arp_forward(by, A, A, A, A, None, A, A, A, st, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_attn_fwd(by, A, A, A, A, None, A, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_attn_rotated(by, A, A, A, None, A, A, big, None) == b.ERR_INVALID_ARG
    dv = _desc(flags=b.ROTATE_V)
    assert L.arp_attn_rotated(ctypes.byref(dv), A, None, None, None, A, A, big, None) == b.ERR_INVALID_ARG
    # with value transport the pass needs v
    assert L.arp_rotate_kv(ctypes.byref(dv), A, None, A, A, big, None) == b.ERR_INVALID_ARG
    df32 = _desc(dtype="f32")
    # the pre-rotation pass and its attention kernel exist for bf16 only
    assert L.arp_rotate_kv(ctypes.byref(df32), A, A, A, A, big, None) == b.ERR_UNSUPPORTED
    assert L.arp_attn_rotated(ctypes.byref(df32), A, A, A, None, A, A, big, None) == b.ERR_UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    phi = torch.zeros(1, 1, 8, 32)
    with pytest.raises(ValueError):
        b.forward(q, q, q, phi)


def test_generated_angle_entry_points_validate_arguments():
    L = b.lib()
    d = _desc()
    by = ctypes.byref(d)
    st = L.arp_scan_state_bytes(by)
    # random draws: bound and theta required and 16-byte aligned, state checked
    assert L.arp_angle_scan_random(by, 1, 0, None, A, A, st, None) == b.ERR_INVALID_ARG
    assert L.arp_angle_scan_random(by, 1, 0, A, None, A, st, None) == b.ERR_INVALID_ARG
    assert L.arp_angle_scan_random(by, 1, 0, M, A, A, st, None) == b.ERR_ALIGNMENT
    assert L.arp_angle_scan_random(by, 1, 0, A, A, None, st, None) == b.ERR_WORKSPACE
    assert L.arp_angle_scan_random(by, 1, 0, A, A, A, 16, None) == b.ERR_WORKSPACE
    assert L.arp_random_phi(by, 1, 0, None, A, None) == b.ERR_INVALID_ARG
    assert L.arp_random_phi(by, 1, 0, A, M, None) == b.ERR_ALIGNMENT
    # token table: ids 4-byte aligned, table 16-byte aligned, vocab in [1, 2^31)
    assert L.arp_angle_scan_tokens(by, A, A, 0, A, A, st, None) == b.ERR_INVALID_ARG
    assert L.arp_angle_scan_tokens(by, A, A, 1 << 31, A, A, st, None) == b.ERR_INVALID_ARG
    assert L.arp_angle_scan_tokens(by, None, A, 10, A, A, st, None) == b.ERR_INVALID_ARG
    assert L.arp_angle_scan_tokens(by, A + 2, A, 10, A, A, st, None) == b.ERR_ALIGNMENT
    assert L.arp_angle_scan_tokens(by, A + 4, M, 10, A, A, st, None) == b.ERR_ALIGNMENT
    assert L.arp_angle_scan_tokens(by, A + 4, A, 10, A, A, 8, None) == b.ERR_WORKSPACE
    # constant steps take no scan state
    assert L.arp_angle_scan_const(by, None, A, None) == b.ERR_INVALID_ARG
    assert L.arp_angle_scan_const(by, A, M, None) == b.ERR_ALIGNMENT
    bad = _desc(head_dim=63)
    assert L.arp_angle_scan_const(ctypes.byref(bad), A, A, None) == b.ERR_INVALID_ARG
    assert L.arp_random_phi(ctypes.byref(bad), 1, 0, A, A, None) == b.ERR_INVALID_ARG


def test_forget_gate_flag_is_refused_outside_the_gated_forward():
    L = b.lib()
    d = _desc(flags=b.ROTATE_QK | b.FORGET_GATE)
    by = ctypes.byref(d)
    big = L.arp_workspace_bytes(by)
    st = L.arp_scan_state_bytes(by)
    assert L.arp_forward(by, A, A, A, A, None, A, A, A, st, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_attn_fwd(by, A, A, A, A, None, A, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_rotate_kv(by, A, A, A, A, big, None) == b.ERR_INVALID_ARG
    assert L.arp_attn_rotated(by, A, A, A, None, A, A, big, None) == b.ERR_INVALID_ARG
    # the gated forward needs the gates
    assert L.arp_forward_ex(by, A, A, A, A, None, None, A, A, None, A, st, A, big,
                            None) == b.ERR_INVALID_ARG
    # fp32 I/O has no gated path
    df = _desc(dtype="f32", flags=b.ROTATE_QK | b.FORGET_GATE)
    assert L.arp_forward_ex(ctypes.byref(df), A, A, A, A, None, A, A, A, None, A, st, A, big,
                            None) == b.ERR_UNSUPPORTED


def test_gated_backward_validates_gates_and_workspace():
    """arp_backward refuses the gate flag (arp_backward_ex takes it); the gated
    backward needs logf and dlogf, and a workspace that also holds the gate
    prefix, its chunk totals and the two dS sums."""
    L = b.lib()
    d = _desc(batch=2, heads=8, seqlen=16384, flags=b.ROTATE_QK | b.FORGET_GATE)
    plain = _desc(batch=2, heads=8, seqlen=16384, flags=b.ROTATE_QK)
    by = ctypes.byref(d)
    ws, ws0 = L.arp_backward_workspace_bytes(by), L.arp_backward_workspace_bytes(ctypes.byref(plain))
    # G offsets, colsum, rowsum (fp32 per token); fp64 base per 64-token tile; fp64 chunk totals
    extra = 3 * 2 * 8 * 16384 * 4 + 2 * 8 * (16384 // 64) * 8 + 2 * 8 * (16384 // 1024) * 8
    assert ws0 + extra <= ws < ws0 + extra + 4 * 256 and ws % 256 == 0
    p14 = [A] * 14
    assert L.arp_backward(by, *p14, ws, None) == b.ERR_INVALID_ARG
    # q k v theta alibi logf o lse dout dq dk dv dtheta dphi dlogf workspace
    args = [A, A, A, A, None, A, A, A, A, A, A, A, A, A, A, A]
    no_logf = list(args)
    no_logf[5] = None
    assert L.arp_backward_ex(by, *no_logf, ws, None) == b.ERR_INVALID_ARG
    no_dlogf = list(args)
    no_dlogf[14] = None
    assert L.arp_backward_ex(by, *no_dlogf, ws, None) == b.ERR_INVALID_ARG
    bad_logf = list(args)
    bad_logf[5] = M
    assert L.arp_backward_ex(by, *bad_logf, ws, None) == b.ERR_ALIGNMENT
    assert L.arp_backward_ex(by, *args, ws - 256, None) == b.ERR_WORKSPACE
    # without the flag the gate arguments are ignored
    assert L.arp_backward_ex(ctypes.byref(plain), *no_logf[:14], None, A, ws0 - 256,
                             None) == b.ERR_WORKSPACE


def test_gated_decode_validates_gate_buffers():
    """The plain decode calls refuse the gate flag; the _ex calls need the
    gates, the gate cache and the gate state (every call here fails
    validation: nothing is launched)."""
    L = b.lib()
    d = _desc(seqlen=512, flags=b.ROTATE_QK | b.FORGET_GATE)
    by = ctypes.byref(d)
    ws = L.arp_decode_workspace_bytes(by)
    # prefill: len k v phi theta [logf] kcache vcache state [gcache gstate]
    assert L.arp_decode_prefill(by, 0, None, None, None, None, A, A, A, None) == b.ERR_INVALID_ARG
    assert L.arp_decode_prefill_ex(by, 0, None, None, None, None, None, A, A, A, None, A,
                                   None) == b.ERR_INVALID_ARG
    assert L.arp_decode_prefill_ex(by, 0, None, None, None, None, None, A, A, A, A, None,
                                   None) == b.ERR_INVALID_ARG
    assert L.arp_decode_prefill_ex(by, 4, A, A, A, A, None, A, A, A, A, A,
                                   None) == b.ERR_INVALID_ARG  # gates of the prompt missing
    assert L.arp_decode_prefill_ex(by, 0, None, None, None, None, None, A, A, A, M, A,
                                   None) == b.ERR_ALIGNMENT
    # step: pos q k v phi alibi [logf] state theta kcache vcache [gcache gstate] o workspace
    assert L.arp_decode_step(by, 0, A, A, A, A, None, A, A, A, A, A, A, ws, None) == b.ERR_INVALID_ARG
    assert L.arp_decode_step_ex(by, 0, A, A, A, A, None, None, A, A, A, A, A, A, A, A, ws,
                                None) == b.ERR_INVALID_ARG
    assert L.arp_decode_step_ex(by, 0, A, A, A, A, None, A, A, A, A, A, None, A, A, A, ws,
                                None) == b.ERR_INVALID_ARG
    assert L.arp_decode_step_ex(by, 0, A, A, A, A, None, M, A, A, A, A, A, A, A, A, ws,
                                None) == b.ERR_ALIGNMENT
    assert L.arp_decode_step_ex(by, 0, A, A, A, A, None, A, A, A, A, A, A, A, A, A, ws - 256,
                                None) == b.ERR_WORKSPACE


def test_scan_state_and_workspace_need_256_byte_alignment():
    """Tensor pointers need 16 bytes; the scan state and the workspaces 256
    (A + 16 is 16-byte aligned, not 256-byte aligned)."""
    L = b.lib()
    d = _desc()
    by = ctypes.byref(d)
    big = L.arp_workspace_bytes(by)
    st = L.arp_scan_state_bytes(by)
    assert A % 256 == 0
    assert L.arp_angle_scan(by, A, A, A + 16, st, None) == b.ERR_ALIGNMENT
    assert L.arp_attn_rotated(by, A, A, A, None, A, A + 16, big, None) == b.ERR_ALIGNMENT
    assert L.arp_rotate_kv(by, A, A, A, A + 16, big, None) == b.ERR_ALIGNMENT
    assert L.arp_forward(by, A, A, A, A, None, A, A, A + 16, st, A, big, None) == b.ERR_ALIGNMENT
    assert L.arp_forward(by, A, A, A, A, None, A, A, A, st, A + 16, big, None) == b.ERR_ALIGNMENT
    bw = L.arp_backward_workspace_bytes(by)
    assert L.arp_backward(by, *([A] * 13), A + 16, bw, None) == b.ERR_ALIGNMENT
    msg = L.arp_status_string(b.ERR_ALIGNMENT).decode()
    assert "16" in msg and "256" in msg


# ---- the Python binding checks shapes, dtypes and buffer sizes before any call ----

def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16)


def test_binding_rejects_mismatched_forward_arguments():
    import torch
    B, H, L, d = 1, 4, 16, 64
    q = _cpu(B, H, L, d)
    phi = _cpu(B, H, L, d // 2, dtype=torch.float32)
    with pytest.raises(ValueError, match="k has shape"):
        b.forward(q, _cpu(B, H, L + 1, d), q, phi)
    with pytest.raises(TypeError, match="v has dtype"):
        b.forward(q, q, _cpu(B, H, L, d, dtype=torch.float32), phi)
    with pytest.raises(ValueError, match="angle heads"):
        b.forward(q, q, q, _cpu(B, 3, L, d // 2, dtype=torch.float32))
    with pytest.raises(ValueError, match="phi has shape"):
        b.forward(q, q, q, _cpu(B, H, L, d // 4, dtype=torch.float32))
    with pytest.raises(TypeError, match="phi has dtype"):
        b.forward(q, q, q, _cpu(B, H, L, d // 2))
    with pytest.raises(ValueError, match="alibi has shape"):
        b.forward(q, q, q, phi, alibi=_cpu(H + 1, dtype=torch.float32))
    with pytest.raises(TypeError, match="alibi has dtype"):
        b.forward(q, q, q, phi, alibi=_cpu(H, dtype=torch.float64))
    with pytest.raises(ValueError, match="out has shape"):
        b.forward(q, q, q, phi, out=_cpu(B, H, L, d + 2))
    with pytest.raises(ValueError, match="theta has shape"):
        b.forward(q, q, q, phi, theta=_cpu(B, 1, L, d // 2, dtype=torch.float32))
    with pytest.raises(ValueError, match="ws holds"):
        b.forward(q, q, q, phi, ws=_cpu(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="state holds"):
        b.forward(q, q, q, phi, state=_cpu(8, dtype=torch.uint8))
    # a buffer of another dtype is sized by its bytes, not its element count
    need = b.workspace_bytes(b.desc_for(q, b.flags_for()))
    with pytest.raises(ValueError, match="ws holds"):
        b.forward(q, q, q, phi, ws=_cpu(need // 8, dtype=torch.float32))
    # well-formed CPU tensors pass validation and then fail the device check
    with pytest.raises(ValueError, match="GPU"):
        b.forward(q, q, q, phi)


def test_binding_rejects_mismatched_gates_angles_and_gradients():
    import torch
    B, H, L, d = 2, 2, 8, 64
    q = _cpu(B, H, L, d)
    phi = _cpu(B, 1, L, d // 2, dtype=torch.float32)
    with pytest.raises(ValueError, match="logf has shape"):
        b.forward_ex(q, q, q, phi, logf=_cpu(B, H, L + 1, dtype=torch.float32))
    with pytest.raises(TypeError, match="logf has dtype"):
        b.forward_ex(q, q, q, phi, logf=_cpu(B, H, L))
    desc = b.desc_for(q, b.flags_for(shared_phi=True))
    with pytest.raises(ValueError, match="theta has shape"):
        b.angle_scan(phi, desc, theta=_cpu(B, H, L, d // 2, dtype=torch.float32))
    with pytest.raises(TypeError, match="tokens has dtype"):
        b.angle_scan_tokens(desc, _cpu(B, L, dtype=torch.int64), _cpu(7, 1, d // 2, dtype=torch.float32))
    with pytest.raises(ValueError, match="table has shape"):
        b.angle_scan_tokens(desc, _cpu(B, L, dtype=torch.int32), _cpu(7, 2, d // 2, dtype=torch.float32))
    with pytest.raises(ValueError, match="bound has shape"):
        b.angle_scan_random(desc, 1, 0, _cpu(2, d // 2, dtype=torch.float32))
    with pytest.raises(ValueError, match="freq has shape"):
        b.angle_scan_const(desc, _cpu(1, d, dtype=torch.float32))
    lse = _cpu(B, H, L, dtype=torch.float32)
    with pytest.raises(ValueError, match="lse has shape"):
        b.backward(desc, q, q, q, phi, phi, q, _cpu(B, H, L - 1, dtype=torch.float32), q)
    with pytest.raises(ValueError, match="dout has shape"):
        b.backward(desc, q, q, q, phi, phi, q, lse, _cpu(B, H, L, d // 2))
    with pytest.raises(ValueError, match="ws holds"):
        b.backward(desc, q, q, q, phi, phi, q, lse, q, ws=_cpu(256, dtype=torch.uint8))


def test_decode_cache_checks_token_and_prompt_shapes():
    import torch
    cache = b.DecodeCache(1, 2, 64, 64, device=torch.device("cpu"))
    tok = _cpu(1, 2, 64)
    phi = _cpu(1, 2, 32, dtype=torch.float32)
    with pytest.raises(ValueError, match="position"):
        cache.step(64, tok, tok, tok, phi)
    with pytest.raises(ValueError, match="q has shape"):
        cache.step(0, _cpu(1, 2, 32), tok, tok, phi)
    with pytest.raises(TypeError, match="phi has dtype"):
        cache.step(0, tok, tok, tok, _cpu(1, 2, 32))
    with pytest.raises(ValueError, match="does not fit"):
        cache.prefill(_cpu(1, 2, 65, 64), _cpu(1, 2, 65, 64), _cpu(1, 2, 65, 32, dtype=torch.float32),
                      _cpu(1, 2, 65, 32, dtype=torch.float32))
    with pytest.raises(ValueError, match="theta has shape"):
        cache.prefill(_cpu(1, 2, 4, 64), _cpu(1, 2, 4, 64), _cpu(1, 2, 4, 32, dtype=torch.float32),
                      _cpu(1, 2, 5, 32, dtype=torch.float32))
    gated = b.DecodeCache(1, 2, 64, 64, forget=True, device=torch.device("cpu"))
    with pytest.raises(ValueError, match="logf"):
        gated.step(0, tok, tok, tok, phi)


def test_head_scale_flag_and_pointer_must_agree():
    L = b.lib()
    d = _desc()
    d.flags |= b.HEAD_SCALE
    assert L.arp_check(ctypes.byref(d)) == b.ERR_INVALID_ARG      # flag without the array
    d.head_scale = A
    assert L.arp_check(ctypes.byref(d)) == b.OK
    d.head_scale = M
    assert L.arp_check(ctypes.byref(d)) == b.ERR_ALIGNMENT
    d = _desc()
    d.head_scale = A
    assert L.arp_check(ctypes.byref(d)) == b.ERR_INVALID_ARG      # array without the flag
    assert ctypes.sizeof(b.Desc) == 40 and b.ABI_VERSION == L.arp_abi_version() == 2


def test_adascale_lambda_host_routine_matches_the_oracle():
    """The library's host routine for AdaScale's schedule against the oracle's
    fp64 evaluation (both written from AdaRoPE Sec. 3.3), rounded once to fp32."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(3)
    tau = rng.uniform(0.5, 2.0, 16).astype(np.float32)
    gamma = rng.uniform(-1.0, 3.0, 16).astype(np.float32)
    for L_, ref in ((1024, 4096), (16384, 1024), (1 << 20, 2048), (4096, 4096)):
        got = b.adascale_lambda(tau, gamma, L_, ref).numpy()
        want = oracle.adascale_lambda(tau.astype(np.float64), gamma.astype(np.float64), L_, ref)
        np.testing.assert_array_equal(got, want.astype(np.float32))
    lib = b.lib()
    f = (ctypes.c_float * 2)(1.0, 1.0)
    out = (ctypes.c_float * 2)()
    assert lib.arp_adascale_lambda(0, f, f, 10, 10, out) == b.ERR_INVALID_ARG
    assert lib.arp_adascale_lambda(2, f, f, 0, 10, out) == b.ERR_INVALID_ARG
    assert lib.arp_adascale_lambda(2, f, f, 10, 0, out) == b.ERR_INVALID_ARG
    assert lib.arp_adascale_lambda(2, None, f, 10, 10, out) == b.ERR_INVALID_ARG
    bad = (ctypes.c_float * 2)(1.0, 0.0)
    assert lib.arp_adascale_lambda(2, bad, f, 10, 10, out) == b.ERR_INVALID_ARG   # tau = 0
    bad = (ctypes.c_float * 2)(1.0, float("nan"))
    assert lib.arp_adascale_lambda(2, f, bad, 10, 10, out) == b.ERR_INVALID_ARG   # gamma NaN
    assert lib.arp_adascale_lambda(2, f, f, 10, 10, out) == b.OK
    assert abs(out[0] - 0.6931472) < 1e-6


def test_scan_rotate_kv_validates_on_the_host():
    L = b.lib()
    d = _desc(flags=b.ROTATE_QK | b.ROTATE_V)
    by = ctypes.byref(d)
    st, ws = L.arp_scan_state_bytes(by), L.arp_workspace_bytes(by)
    f = L.arp_angle_scan_rotate_kv
    assert f(by, None, A, A, A, A, st, A, ws, None) == b.ERR_INVALID_ARG      # phi
    assert f(by, A, None, A, A, A, st, A, ws, None) == b.ERR_INVALID_ARG      # k
    assert f(by, A, A, None, A, A, st, A, ws, None) == b.ERR_INVALID_ARG      # v (transported)
    assert f(by, A, A, A, None, A, st, A, ws, None) == b.ERR_INVALID_ARG      # theta
    assert f(by, M, A, A, A, A, st, A, ws, None) == b.ERR_ALIGNMENT
    assert f(by, A, A, A, A, A + 16, st, A, ws, None) == b.ERR_ALIGNMENT      # state: 256 bytes
    assert f(by, A, A, A, A, A, st, A, ws - 1, None) == b.ERR_WORKSPACE
    for flags in (b.ROTATE_QK | b.FUSED_ROTATION,):
        x = _desc(flags=flags)
        assert f(ctypes.byref(x), A, A, A, A, A, st, A, ws, None) == b.ERR_UNSUPPORTED
    x = _desc(dtype="f32")
    assert f(ctypes.byref(x), A, A, A, A, A, st, A, ws, None) == b.ERR_UNSUPPORTED
    x = _desc(flags=b.ROTATE_QK | b.FORGET_GATE)
    assert f(ctypes.byref(x), A, A, A, A, A, st, A, ws, None) == b.ERR_INVALID_ARG


def test_noalloc_forward_validates_before_touching_the_device():
    """arp_forward_noalloc checks its arguments and its scratch limits on the
    host (fake addresses: nothing is launched, no device is touched)."""
    L = b.lib()
    d = _desc(batch=2, heads=8, seqlen=16384, flags=b.ROTATE_QK | b.ROTATE_V)
    by = ctypes.byref(d)
    assert L.arp_forward_noalloc(by, A, A, A, None, None, A, A, None) == b.ERR_INVALID_ARG
    assert L.arp_forward_noalloc(by, A, A, A, A, None, A, M, None) == b.ERR_ALIGNMENT
    # 64 MiB of pre-rotated operands (k~ and v~) exceed the 40 MiB operand scratch
    assert L.arp_forward_noalloc(by, A, A, A, A, None, A, A, None) == b.ERR_SCRATCH
    # 4 x 32 heads at 32768 tokens (d = 128): a scan state beyond 24 MiB, even fused
    big = _desc(batch=4, heads=32, seqlen=32768, head_dim=128, flags=b.ROTATE_QK | b.FUSED_ROTATION)
    assert L.arp_scan_state_bytes(ctypes.byref(big)) > (24 << 20)
    assert L.arp_forward_noalloc(ctypes.byref(big), A, A, A, A, None, A, A, None) == b.ERR_SCRATCH
    gated = _desc(flags=b.ROTATE_QK | b.FORGET_GATE)
    assert L.arp_forward_noalloc(ctypes.byref(gated), A, A, A, A, None, A, A, None) == b.ERR_INVALID_ARG
