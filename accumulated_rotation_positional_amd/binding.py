"""ctypes binding of libarp.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (``include/arp.h``).  torch is used for device memory
and the current stream, nothing else.  There is no CPU fallback: if the
library is missing, or a tensor is not on a GPU, the call raises.

Tensor conventions (C-contiguous, on the GPU):
  q, k, v, o   [B, H, L, d]   float32 or bfloat16 (all the same dtype)
  phi, theta   [B, Hphi, L, d/2] float32, Hphi in {1, H}
  alibi        [H] float32 slopes
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libarp.so")

# Status codes and flags of include/arp.h.
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_ALIGNMENT, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH = range(7)
DTYPE_F32, DTYPE_BF16 = 0, 1
ROTATE_QK = 0x1
ROTATE_V = 0x2
ALIBI = 0x4
PHI_SHARED_HEADS = 0x8
SCAN_EXCLUSIVE = 0x10
FUSED_ROTATION = 0x20
FORGET_GATE = 0x40
HEAD_SCALE = 0x80
ABI_VERSION = 2

# Every function the header declares (tests check the library exports them all).
EXPORTS = ("arp_abi_version", "arp_status_string", "arp_check", "arp_scan_state_bytes",
           "arp_workspace_bytes",
           "arp_angle_scan", "arp_rotate_kv", "arp_angle_scan_rotate_kv", "arp_attn_rotated", "arp_attn_fwd",
           "arp_forward", "arp_rotate", "arp_forward_train", "arp_backward_workspace_bytes",
           "arp_backward", "arp_decode_workspace_bytes", "arp_decode_prefill", "arp_decode_step",
           "arp_forward_ex", "arp_angle_scan_random", "arp_angle_scan_tokens",
           "arp_angle_scan_const", "arp_random_phi", "arp_backward_ex", "arp_decode_prefill_ex",
           "arp_decode_step_ex", "arp_adascale_lambda", "arp_forward_noalloc")


class ArpError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("scale", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("head_scale", ctypes.c_void_p)]


_LIB = None
_LOCK = threading.Lock()


def lib() -> ctypes.CDLL:
    """Load libarp.so once; raise if it has not been built."""
    global _LIB
    with _LOCK:
        if _LIB is None:
            _LIB = open_library(LIB_PATH)
    return _LIB


def open_library(path: str) -> ctypes.CDLL:
    """Load a build of the library at path with every entry point's prototype
    (lib() uses it for libarp.so; tests use it for the scan test variant)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(path)
    P, S, D = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(Desc)
    U64 = ctypes.c_uint64
    sig = {
        "arp_abi_version": ([], ctypes.c_int),
        "arp_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "arp_check": ([D], ctypes.c_int),
        "arp_scan_state_bytes": ([D], S),
        "arp_workspace_bytes": ([D], S),
        "arp_angle_scan": ([D, P, P, P, S, P], ctypes.c_int),
        "arp_rotate_kv": ([D, P, P, P, P, S, P], ctypes.c_int),
        "arp_angle_scan_rotate_kv": ([D, P, P, P, P, P, S, P, S, P], ctypes.c_int),
        "arp_attn_rotated": ([D, P, P, P, P, P, P, S, P], ctypes.c_int),
        "arp_attn_fwd": ([D, P, P, P, P, P, P, P, S, P], ctypes.c_int),
        "arp_forward": ([D, P, P, P, P, P, P, P, P, S, P, S, P], ctypes.c_int),
        "arp_rotate": ([D, P, P, P, ctypes.c_int, P], ctypes.c_int),
        "arp_forward_train": ([D, P, P, P, P, P, P, P, P, P, S, P, S, P], ctypes.c_int),
        "arp_backward_workspace_bytes": ([D], S),
        "arp_backward": ([D] + [P] * 14 + [S, P], ctypes.c_int),
        "arp_backward_ex": ([D] + [P] * 16 + [S, P], ctypes.c_int),
        "arp_decode_prefill_ex": ([D, ctypes.c_int32] + [P] * 10 + [P], ctypes.c_int),
        "arp_decode_step_ex": ([D, ctypes.c_int32] + [P] * 14 + [S, P], ctypes.c_int),
        "arp_decode_workspace_bytes": ([D], S),
        "arp_decode_prefill": ([D, ctypes.c_int32] + [P] * 7 + [P], ctypes.c_int),
        "arp_decode_step": ([D, ctypes.c_int32] + [P] * 11 + [S, P], ctypes.c_int),
        "arp_forward_ex": ([D] + [P] * 10 + [S, P, S, P], ctypes.c_int),
        "arp_angle_scan_random": ([D, U64, U64, P, P, P, S, P], ctypes.c_int),
        "arp_angle_scan_tokens": ([D, P, P, ctypes.c_int64, P, P, S, P], ctypes.c_int),
        "arp_angle_scan_const": ([D, P, P, P], ctypes.c_int),
        "arp_random_phi": ([D, U64, U64, P, P, P], ctypes.c_int),
        "arp_adascale_lambda": ([ctypes.c_int32, P, P, ctypes.c_int64, ctypes.c_int64, P],
                                ctypes.c_int),
        "arp_forward_noalloc": ([D, P, P, P, P, P, P, P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes, f.restype = args, res
    return L


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise ArpError(fn, status, lib().arp_status_string(status).decode())


def make_desc(batch: int, heads: int, seqlen: int, head_dim: int, dtype, flags: int,
              scale: float | None = None, head_scale: torch.Tensor | None = None) -> Desc:
    """A descriptor; head_scale (float32 [heads] on the GPU: AdaScale's per-head
    query multipliers) sets HEAD_SCALE and is kept alive with the descriptor."""
    if dtype in (torch.float32, "f32", DTYPE_F32):
        code = DTYPE_F32
    elif dtype in (torch.bfloat16, "bf16", DTYPE_BF16):
        code = DTYPE_BF16
    else:
        raise TypeError(f"unsupported dtype {dtype}")
    ptr = None
    if head_scale is not None:
        _expect(head_scale, "head_scale", (heads,), torch.float32)
        ptr = _ptr(head_scale)
        flags |= HEAD_SCALE
    d = Desc(batch, heads, seqlen, head_dim, code, flags, 0.0 if scale is None else scale, 0, ptr)
    d._head_scale = head_scale  # the device array the pointer refers to
    return d


def adascale_lambda(tau, gamma, L: int, L_ref: int) -> torch.Tensor:
    """AdaScale's inverse temperatures lambda_h(L) = (1/tau_h) [ln(1 + max(L, L_ref)/L_ref)]^gamma_h
    computed by the library's host routine (fp64, rounded to fp32); returns a
    CPU float32 tensor [heads] (move it to the GPU for head_scale)."""
    tau = torch.as_tensor(tau, dtype=torch.float32).contiguous().cpu()
    gamma = torch.as_tensor(gamma, dtype=torch.float32).contiguous().cpu()
    if tau.dim() != 1 or tau.shape != gamma.shape:
        raise ValueError("tau and gamma must be [heads]")
    out = torch.empty_like(tau)
    _check("arp_adascale_lambda", lib().arp_adascale_lambda(tau.numel(), tau.data_ptr(),
                                                            gamma.data_ptr(), int(L), int(L_ref),
                                                            out.data_ptr()))
    return out


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _require_gpu(*ts) -> None:
    for t in ts:
        if t is not None:
            _ptr(t)


# ---- argument validation --------------------------------------------------
# The C ABI sees plain pointers and cannot tell a buffer's size, so a tensor of
# the wrong shape or dtype would become an out-of-bounds device access.  Every
# call below checks its tensors against the descriptor first and raises
# ValueError (shape, size) or TypeError (dtype) before anything is launched.

def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _expect(t: torch.Tensor | None, name: str, shape, dtype) -> None:
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _io_dtype(desc: Desc):
    return torch.float32 if desc.dtype == DTYPE_F32 else torch.bfloat16


def _angle_heads(desc: Desc) -> int:
    return 1 if desc.flags & PHI_SHARED_HEADS else desc.heads


def _check_qkv(desc: Desc, **ts) -> None:
    shape = (desc.batch, desc.heads, desc.seqlen, desc.head_dim)
    for name, t in ts.items():
        _expect(t, name, shape, _io_dtype(desc))


def _check_angles(desc: Desc, **ts) -> None:
    shape = (desc.batch, _angle_heads(desc), desc.seqlen, desc.head_dim // 2)
    for name, t in ts.items():
        _expect(t, name, shape, torch.float32)


def _check_rows(desc: Desc, **ts) -> None:
    """Per-row fp32 tensors [B, H, L] (lse, log gates and their gradient)."""
    for name, t in ts.items():
        _expect(t, name, (desc.batch, desc.heads, desc.seqlen), torch.float32)


def _check_alibi(desc: Desc, alibi) -> None:
    if alibi is not None:
        _expect(alibi, "alibi", (desc.heads,), torch.float32)


def _check_buffer(t: torch.Tensor | None, name: str, need: int) -> None:
    if t is not None and _nbytes(t) < need:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, the call needs {need}")


def _check_phi_heads(q: torch.Tensor, phi: torch.Tensor) -> None:
    if q.dim() != 4 or phi.dim() != 4:
        raise ValueError("q must be [B, H, L, d] and phi [B, Hphi, L, d/2]")
    if phi.shape[1] not in (1, q.shape[1]):
        raise ValueError(f"phi has {phi.shape[1]} angle heads; expected 1 (shared) or "
                         f"{q.shape[1]} (one per head)")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def flags_for(*, rotate_qk: bool = True, rotate_v: bool = False, alibi: bool = False,
              shared_phi: bool = False, exclusive: bool = False, fused: bool = False,
              forget: bool = False) -> int:
    return ((ROTATE_QK if rotate_qk else 0) | (ROTATE_V if rotate_v else 0) |
            (ALIBI if alibi else 0) | (PHI_SHARED_HEADS if shared_phi else 0) |
            (SCAN_EXCLUSIVE if exclusive else 0) | (FUSED_ROTATION if fused else 0) |
            (FORGET_GATE if forget else 0))


def desc_for(q: torch.Tensor, flags: int, scale: float | None = None,
             head_scale: torch.Tensor | None = None) -> Desc:
    if q.dim() != 4:
        raise ValueError("q must be [B, H, L, d]")
    B, H, L, d = q.shape
    return make_desc(B, H, L, d, q.dtype, flags, scale, head_scale)


def workspace_bytes(desc: Desc) -> int:
    return int(lib().arp_workspace_bytes(ctypes.byref(desc)))


def scan_state_bytes(desc: Desc) -> int:
    return int(lib().arp_scan_state_bytes(ctypes.byref(desc)))


_STATE: dict = {}
_WS: dict = {}


def scan_state(desc: Desc, device: torch.device) -> torch.Tensor:
    """The angle scan's look-back state, zero-filled once and cached per
    (device, stream); each scan leaves it ready for the next, so one buffer
    serves every later call on that stream that fits in it."""
    need = max(scan_state_bytes(desc), 256)
    key = (device.index, _stream(device))
    st = _STATE.get(key)
    if st is None or st.numel() < need:
        st = torch.zeros(need, dtype=torch.uint8, device=device)
        _STATE[key] = st
    return st


def workspace(desc: Desc, device: torch.device) -> torch.Tensor:
    """Operand workspace (rotated bf16 q/k/v of the pre-rotation path), cached
    per (device, stream); needs no initialisation."""
    need = max(workspace_bytes(desc), 256)
    key = (device.index, _stream(device))
    ws = _WS.get(key)
    if ws is None or ws.numel() < need:
        ws = None
        _WS.pop(key, None)
        ws = torch.empty(need, dtype=torch.uint8, device=device)
        _WS[key] = ws
    return ws


def angle_scan(phi: torch.Tensor, desc: Desc, theta: torch.Tensor | None = None,
               state: torch.Tensor | None = None) -> torch.Tensor:
    _check_angles(desc, phi=phi, theta=theta)
    _check_buffer(state, "state", scan_state_bytes(desc))
    _require_gpu(phi, theta, state)
    theta = torch.empty_like(phi) if theta is None else theta
    state = scan_state(desc, phi.device) if state is None else state
    _check("arp_angle_scan", lib().arp_angle_scan(ctypes.byref(desc), _ptr(phi), _ptr(theta),
                                                  _ptr(state), _nbytes(state), _stream(phi.device)))
    return theta


def _phi_shape(desc: Desc):
    hphi = 1 if desc.flags & PHI_SHARED_HEADS else desc.heads
    return (desc.batch, hphi, desc.seqlen, desc.head_dim // 2)


def angle_scan_random(desc: Desc, seed: int, step: int, bound: torch.Tensor,
                      theta: torch.Tensor | None = None,
                      state: torch.Tensor | None = None) -> torch.Tensor:
    """Accumulated angles of the random variant, drawn inside the scan; bound is
    float32 [angle heads, d/2] on the device."""
    _expect(bound, "bound", (_angle_heads(desc), desc.head_dim // 2), torch.float32)
    _check_angles(desc, theta=theta)
    _check_buffer(state, "state", scan_state_bytes(desc))
    _require_gpu(bound, theta, state)
    dev = bound.device
    theta = torch.empty(_phi_shape(desc), dtype=torch.float32, device=dev) if theta is None else theta
    state = scan_state(desc, dev) if state is None else state
    _check("arp_angle_scan_random",
           lib().arp_angle_scan_random(ctypes.byref(desc), seed, step, _ptr(bound), _ptr(theta),
                                       _ptr(state), _nbytes(state), _stream(dev)))
    return theta


def angle_scan_tokens(desc: Desc, tokens: torch.Tensor, table: torch.Tensor,
                      theta: torch.Tensor | None = None,
                      state: torch.Tensor | None = None) -> torch.Tensor:
    """Accumulated angles of a per-token angle table; tokens int32 [B, L], table
    float32 [vocab, angle heads, d/2], both on the device."""
    _expect(tokens, "tokens", (desc.batch, desc.seqlen), torch.int32)
    if table.dim() != 3 or table.shape[0] < 1:
        raise ValueError("table must be [vocab, angle heads, d/2] with vocab >= 1")
    _expect(table, "table", (table.shape[0], _angle_heads(desc), desc.head_dim // 2), torch.float32)
    _check_angles(desc, theta=theta)
    _check_buffer(state, "state", scan_state_bytes(desc))
    _require_gpu(tokens, table, theta, state)
    dev = table.device
    theta = torch.empty(_phi_shape(desc), dtype=torch.float32, device=dev) if theta is None else theta
    state = scan_state(desc, dev) if state is None else state
    _check("arp_angle_scan_tokens",
           lib().arp_angle_scan_tokens(ctypes.byref(desc), _ptr(tokens), _ptr(table),
                                       table.shape[0], _ptr(theta), _ptr(state), _nbytes(state),
                                       _stream(dev)))
    return theta


def angle_scan_const(desc: Desc, freq: torch.Tensor, theta: torch.Tensor | None = None) -> torch.Tensor:
    """Accumulated angles of constant per-pair steps (closed form); freq float32
    [angle heads, d/2]."""
    _expect(freq, "freq", (_angle_heads(desc), desc.head_dim // 2), torch.float32)
    _check_angles(desc, theta=theta)
    _require_gpu(freq, theta)
    dev = freq.device
    theta = torch.empty(_phi_shape(desc), dtype=torch.float32, device=dev) if theta is None else theta
    _check("arp_angle_scan_const",
           lib().arp_angle_scan_const(ctypes.byref(desc), _ptr(freq), _ptr(theta), _stream(dev)))
    return theta


def random_phi(desc: Desc, seed: int, step: int, bound: torch.Tensor,
               phi: torch.Tensor | None = None) -> torch.Tensor:
    """The random variant's step angles written out (float32 [B, angle heads, L, d/2])."""
    _expect(bound, "bound", (_angle_heads(desc), desc.head_dim // 2), torch.float32)
    _check_angles(desc, phi=phi)
    _require_gpu(bound, phi)
    dev = bound.device
    phi = torch.empty(_phi_shape(desc), dtype=torch.float32, device=dev) if phi is None else phi
    _check("arp_random_phi", lib().arp_random_phi(ctypes.byref(desc), seed, step, _ptr(bound),
                                                  _ptr(phi), _stream(dev)))
    return phi


def rotate_kv(k, v, theta, desc: Desc, ws: torch.Tensor | None = None) -> torch.Tensor:
    """The pre-rotation pass: k~ (and v~ with value transport) into the
    workspace, which it returns."""
    _check_qkv(desc, k=k, v=v)
    _check_angles(desc, theta=theta)
    _check_buffer(ws, "ws", workspace_bytes(desc))
    _require_gpu(k, v, theta, ws)
    ws = workspace(desc, k.device) if ws is None else ws
    _check("arp_rotate_kv", lib().arp_rotate_kv(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(theta),
                                                _ptr(ws), _nbytes(ws), _stream(k.device)))
    return ws


def angle_scan_rotate_kv(phi, k, v, desc: Desc, theta: torch.Tensor | None = None,
                         state: torch.Tensor | None = None,
                         ws: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """The angle scan with the key (and value) pre-rotation in its epilogue:
    returns (theta, ws) as angle_scan then rotate_kv would leave them."""
    _check_qkv(desc, k=k, v=v)
    _check_angles(desc, phi=phi, theta=theta)
    _check_buffer(state, "state", scan_state_bytes(desc))
    _check_buffer(ws, "ws", workspace_bytes(desc))
    _require_gpu(phi, k, v, theta, state, ws)
    theta = torch.empty_like(phi) if theta is None else theta
    state = scan_state(desc, phi.device) if state is None else state
    ws = workspace(desc, phi.device) if ws is None else ws
    _check("arp_angle_scan_rotate_kv", lib().arp_angle_scan_rotate_kv(
        ctypes.byref(desc), _ptr(phi), _ptr(k), _ptr(v), _ptr(theta), _ptr(state), _nbytes(state),
        _ptr(ws), _nbytes(ws), _stream(phi.device)))
    return theta, ws


def attn_rotated(q, v, theta, alibi, out, desc: Desc, ws: torch.Tensor) -> torch.Tensor:
    """Attention over the pass's keys (and values): q is rotated inside the
    kernel; v is the caller's values (read without value transport)."""
    _check_qkv(desc, q=q, v=v, out=out)
    _check_angles(desc, theta=theta)
    _check_alibi(desc, alibi)
    _check_buffer(ws, "ws", workspace_bytes(desc))
    _require_gpu(q, v, theta, alibi, out, ws)
    _check("arp_attn_rotated", lib().arp_attn_rotated(ctypes.byref(desc), _ptr(q), _ptr(v),
                                                      _ptr(theta), _ptr(alibi), _ptr(out),
                                                      _ptr(ws), _nbytes(ws), _stream(out.device)))
    return out


def attn_fwd(q, k, v, theta, desc: Desc, alibi=None, out=None, ws=None) -> torch.Tensor:
    _check_qkv(desc, q=q, k=k, v=v, out=out)
    _check_angles(desc, theta=theta)
    _check_alibi(desc, alibi)
    _check_buffer(ws, "ws", workspace_bytes(desc))
    _require_gpu(q, k, v, theta, alibi, out, ws)
    out = torch.empty_like(q) if out is None else out
    ws = workspace(desc, q.device) if ws is None else ws
    _check("arp_attn_fwd", lib().arp_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(theta), _ptr(alibi), _ptr(out), _ptr(ws),
                                              _nbytes(ws), _stream(q.device)))
    return out


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, phi: torch.Tensor, *,
            rotate_qk: bool = True, rotate_v: bool = False, alibi: torch.Tensor | None = None,
            scale: float | None = None, exclusive: bool = False, fused: bool = False,
            out: torch.Tensor | None = None, theta: torch.Tensor | None = None,
            state: torch.Tensor | None = None, ws: torch.Tensor | None = None,
            head_scale: torch.Tensor | None = None):
    """(q, k, v, phi, flags) -> (o, theta): the whole forward pass on the GPU.
    head_scale: float32 [H] per-head query multipliers (AdaScale), or None."""
    _check_phi_heads(q, phi)
    flags = flags_for(rotate_qk=rotate_qk, rotate_v=rotate_v, alibi=alibi is not None,
                      shared_phi=phi.shape[1] == 1 and q.shape[1] != 1, exclusive=exclusive,
                      fused=fused)
    desc = desc_for(q, flags, scale, head_scale)
    _check_qkv(desc, q=q, k=k, v=v, out=out)
    _check_angles(desc, phi=phi, theta=theta)
    _check_alibi(desc, alibi)
    _check_buffer(state, "state", scan_state_bytes(desc))
    _check_buffer(ws, "ws", workspace_bytes(desc))
    _require_gpu(q, k, v, phi, alibi, out, theta, state, ws)
    out = torch.empty_like(q) if out is None else out
    theta = torch.empty_like(phi) if theta is None else theta
    state = scan_state(desc, q.device) if state is None else state
    ws = workspace(desc, q.device) if ws is None else ws
    _check("arp_forward", lib().arp_forward(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(phi), _ptr(alibi), _ptr(theta), _ptr(out),
                                            _ptr(state), _nbytes(state), _ptr(ws), _nbytes(ws),
                                            _stream(q.device)))
    return out, theta


def forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, phi: torch.Tensor, *,
                    rotate_qk: bool = True, rotate_v: bool = False,
                    alibi: torch.Tensor | None = None, scale: float | None = None,
                    exclusive: bool = False, fused: bool = False, out: torch.Tensor | None = None,
                    theta: torch.Tensor | None = None, head_scale: torch.Tensor | None = None):
    """forward() through arp_forward_noalloc: no scan state or workspace from
    the caller (the library's own device scratch).  Allocates only the outputs
    it is not given; pass out and theta to allocate nothing."""
    _check_phi_heads(q, phi)
    flags = flags_for(rotate_qk=rotate_qk, rotate_v=rotate_v, alibi=alibi is not None,
                      shared_phi=phi.shape[1] == 1 and q.shape[1] != 1, exclusive=exclusive,
                      fused=fused)
    desc = desc_for(q, flags, scale, head_scale)
    _check_qkv(desc, q=q, k=k, v=v, out=out)
    _check_angles(desc, phi=phi, theta=theta)
    _check_alibi(desc, alibi)
    _require_gpu(q, k, v, phi, alibi, out, theta)
    out = torch.empty_like(q) if out is None else out
    theta = torch.empty_like(phi) if theta is None else theta
    _check("arp_forward_noalloc", lib().arp_forward_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(phi), _ptr(alibi), _ptr(theta),
        _ptr(out), _stream(q.device)))
    return out, theta


def rotate(x: torch.Tensor, theta: torch.Tensor, desc: Desc, inverse: bool = False) -> torch.Tensor:
    _check_qkv(desc, x=x)
    _check_angles(desc, theta=theta)
    _require_gpu(x, theta)
    out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _check("arp_rotate", lib().arp_rotate(ctypes.byref(desc), _ptr(x), _ptr(theta), _ptr(out),
                                          int(inverse), _stream(x.device)))
    return out


def forward_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, phi: torch.Tensor, *,
                  rotate_qk: bool = True, rotate_v: bool = False,
                  alibi: torch.Tensor | None = None, scale: float | None = None,
                  exclusive: bool = False, head_scale: torch.Tensor | None = None):
    """Forward pass that also returns the per-row base-2 log-sum-exp (bf16,
    pre-rotation path): (o, theta, lse, desc), everything the backward needs
    (desc carries the head scale, if any, into the backward)."""
    _check_phi_heads(q, phi)
    flags = flags_for(rotate_qk=rotate_qk, rotate_v=rotate_v, alibi=alibi is not None,
                      shared_phi=phi.shape[1] == 1 and q.shape[1] != 1, exclusive=exclusive)
    desc = desc_for(q, flags, scale, head_scale)
    _check_qkv(desc, q=q, k=k, v=v)
    _check_angles(desc, phi=phi)
    _check_alibi(desc, alibi)
    _require_gpu(q, k, v, phi, alibi)
    out = torch.empty_like(q)
    theta = torch.empty_like(phi)
    B, H, L, _ = q.shape
    lse = torch.empty(B, H, L, dtype=torch.float32, device=q.device)
    state = scan_state(desc, q.device)
    ws = workspace(desc, q.device)
    _check("arp_forward_train", lib().arp_forward_train(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(phi), _ptr(alibi), _ptr(theta),
        _ptr(out), _ptr(lse), _ptr(state), _nbytes(state), _ptr(ws), _nbytes(ws),
        _stream(q.device)))
    return out, theta, lse, desc


def backward_workspace_bytes(desc: Desc) -> int:
    return int(lib().arp_backward_workspace_bytes(ctypes.byref(desc)))


_BWS: dict = {}


def backward_workspace(desc: Desc, device: torch.device) -> torch.Tensor:
    """The backward's operand workspace, cached per (device, stream)."""
    need = max(backward_workspace_bytes(desc), 256)
    key = (device.index, _stream(device))
    ws = _BWS.get(key)
    if ws is None or ws.numel() < need:
        _BWS.pop(key, None)
        ws = torch.empty(need, dtype=torch.uint8, device=device)
        _BWS[key] = ws
    return ws


def _check_backward_args(desc: Desc, q, k, v, phi, theta, o, lse, dout, alibi, logf, ws) -> None:
    _check_qkv(desc, q=q, k=k, v=v, o=o, dout=dout)
    _check_angles(desc, phi=phi, theta=theta)
    _check_rows(desc, lse=lse, logf=logf)
    _check_alibi(desc, alibi)
    _check_buffer(ws, "ws", backward_workspace_bytes(desc))


def backward(desc: Desc, q, k, v, phi, theta, o, lse, dout, alibi=None, ws=None):
    """Gradients for dout = dL/do: (dq, dk, dv, dphi, dtheta), with dtheta the
    per-head dL/dTheta ([B, H, L, d/2])."""
    _check_backward_args(desc, q, k, v, phi, theta, o, lse, dout, alibi, None, ws)
    _require_gpu(q, k, v, phi, theta, o, lse, dout, alibi, ws)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, H, L, d = q.shape
    dtheta = torch.empty(B, H, L, d // 2, dtype=torch.float32, device=q.device)
    dphi = torch.empty_like(phi)
    ws = backward_workspace(desc, q.device) if ws is None else ws
    _check("arp_backward", lib().arp_backward(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(theta), _ptr(alibi), _ptr(o),
        _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dtheta), _ptr(dphi),
        _ptr(ws), _nbytes(ws), _stream(q.device)))
    return dq, dk, dv, dphi, dtheta


def backward_ex(desc: Desc, q, k, v, phi, theta, o, lse, dout, alibi=None, logf=None, ws=None):
    """arp_backward_ex: backward() plus, with the forget gates (desc has
    FORGET_GATE; logf [B, H, L] as given to forward_ex), dlogf = dL/d(log f)
    [B, H, L].  Returns (dq, dk, dv, dphi, dtheta, dlogf or None)."""
    _check_backward_args(desc, q, k, v, phi, theta, o, lse, dout, alibi, logf, ws)
    _require_gpu(q, k, v, phi, theta, o, lse, dout, alibi, logf, ws)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, H, L, d = q.shape
    dtheta = torch.empty(B, H, L, d // 2, dtype=torch.float32, device=q.device)
    dphi = torch.empty_like(phi)
    dlogf = torch.empty(B, H, L, dtype=torch.float32, device=q.device) if logf is not None else None
    ws = backward_workspace(desc, q.device) if ws is None else ws
    _check("arp_backward_ex", lib().arp_backward_ex(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(theta), _ptr(alibi), _ptr(logf),
        _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dtheta), _ptr(dphi),
        _ptr(dlogf), _ptr(ws), _nbytes(ws), _stream(q.device)))
    return dq, dk, dv, dphi, dtheta, dlogf


class DecodeCache:
    """Key/value cache (pre-rotated bf16 [B, H, capacity, d]), the angle state
    (uint64 [B, Hphi, d/2]) and the step workspace of one decoding stream;
    with forget=True also the gate-prefix cache (fp64 [B, H, capacity]) and the
    gate state (fp64 [B, H])."""

    def __init__(self, batch: int, heads: int, capacity: int, head_dim: int, *, phi_heads=None,
                 rotate_qk: bool = True, rotate_v: bool = False, alibi: bool = False,
                 exclusive: bool = False, forget: bool = False, scale: float | None = None,
                 head_scale: torch.Tensor | None = None,
                 device: torch.device = torch.device("cuda:0")):
        hphi = heads if phi_heads is None else phi_heads
        flags = flags_for(rotate_qk=rotate_qk, rotate_v=rotate_v, alibi=alibi,
                          shared_phi=hphi == 1 and heads != 1, exclusive=exclusive, forget=forget)
        self.forget = forget
        self.gcache = (torch.zeros(batch, heads, capacity, dtype=torch.float64, device=device)
                       if forget else None)
        self.gstate = torch.zeros(batch, heads, dtype=torch.float64, device=device) if forget else None
        self.desc = make_desc(batch, heads, capacity, head_dim, torch.bfloat16, flags, scale,
                              head_scale)
        self.device = device
        self.kcache = torch.zeros(batch, heads, capacity, head_dim, dtype=torch.bfloat16, device=device)
        self.vcache = torch.zeros_like(self.kcache)
        self.state = torch.zeros(batch, hphi, head_dim // 2, dtype=torch.int64, device=device)
        self.theta = torch.zeros(batch, hphi, head_dim // 2, dtype=torch.float32, device=device)
        nbytes = max(int(lib().arp_decode_workspace_bytes(ctypes.byref(self.desc))), 256)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def prefill(self, k=None, v=None, phi=None, theta=None, logf=None) -> None:
        """Cache rows [0, len) and the state after the len prompt tokens
        (k, v [B, H, len, d]; phi, theta [B, Hphi, len, d/2]; with gates logf
        [B, H, len]); no arguments: an empty prompt (state reset)."""
        n = 0 if k is None else int(k.shape[2])
        d = self.desc
        if n > d.seqlen:
            raise ValueError(f"a prompt of {n} tokens does not fit a cache of {d.seqlen}")
        if n > 0:
            io = (d.batch, d.heads, n, d.head_dim)
            _expect(k, "k", io, torch.bfloat16)
            _expect(v, "v", io, torch.bfloat16)
            ang = (d.batch, _angle_heads(d), n, d.head_dim // 2)
            _expect(phi, "phi", ang, torch.float32)
            _expect(theta, "theta", ang, torch.float32)
            if self.forget:
                if logf is None:
                    raise ValueError("a gated cache needs the prompt's logf")
                _expect(logf, "logf", (d.batch, d.heads, n), torch.float32)
        _require_gpu(k, v, phi, theta, logf)
        if self.forget:
            _check("arp_decode_prefill_ex", lib().arp_decode_prefill_ex(
                ctypes.byref(self.desc), n, _ptr(k), _ptr(v), _ptr(phi), _ptr(theta), _ptr(logf),
                _ptr(self.kcache), _ptr(self.vcache), _ptr(self.state), _ptr(self.gcache),
                _ptr(self.gstate), _stream(self.device)))
            return
        _check("arp_decode_prefill", lib().arp_decode_prefill(
            ctypes.byref(self.desc), n, _ptr(k), _ptr(v), _ptr(phi), _ptr(theta),
            _ptr(self.kcache), _ptr(self.vcache), _ptr(self.state), _stream(self.device)))

    def step(self, pos: int, q, k, v, phi, alibi=None, out=None, logf=None) -> torch.Tensor:
        """One token at position pos: q, k, v [B, H, d]; phi [B, Hphi, d/2];
        with gates logf [B, H].  Returns o [B, H, d]; self.theta holds the
        token's angles."""
        d = self.desc
        if not 0 <= int(pos) < d.seqlen:
            raise ValueError(f"position {pos} outside the cache of {d.seqlen} tokens")
        tok = (d.batch, d.heads, d.head_dim)
        for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
            _expect(t, name, tok, torch.bfloat16)
        _expect(phi, "phi", (d.batch, _angle_heads(d), d.head_dim // 2), torch.float32)
        _check_alibi(d, alibi)
        if self.forget:
            if logf is None:
                raise ValueError("a gated cache needs the token's logf")
            _expect(logf, "logf", (d.batch, d.heads), torch.float32)
        _require_gpu(q, k, v, phi, alibi, out, logf)
        out = torch.empty_like(q) if out is None else out
        if self.forget:
            _check("arp_decode_step_ex", lib().arp_decode_step_ex(
                ctypes.byref(self.desc), int(pos), _ptr(q), _ptr(k), _ptr(v), _ptr(phi),
                _ptr(alibi), _ptr(logf), _ptr(self.state), _ptr(self.theta), _ptr(self.kcache),
                _ptr(self.vcache), _ptr(self.gcache), _ptr(self.gstate), _ptr(out), _ptr(self.ws),
                _nbytes(self.ws), _stream(self.device)))
            return out
        _check("arp_decode_step", lib().arp_decode_step(
            ctypes.byref(self.desc), int(pos), _ptr(q), _ptr(k), _ptr(v), _ptr(phi), _ptr(alibi),
            _ptr(self.state), _ptr(self.theta), _ptr(self.kcache), _ptr(self.vcache), _ptr(out),
            _ptr(self.ws), _nbytes(self.ws), _stream(self.device)))
        return out


def forward_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, phi: torch.Tensor, *,
               rotate_qk: bool = True, rotate_v: bool = False, alibi: torch.Tensor | None = None,
               logf: torch.Tensor | None = None, scale: float | None = None,
               exclusive: bool = False, with_lse: bool = False,
               head_scale: torch.Tensor | None = None):
    """The forward with every option (arp_forward_ex): logf [B, H, L] log forget
    gates (the gate bias is on when given), with_lse also returns the per-row
    base-2 log-sum-exp.  Returns (o, theta, lse or None)."""
    _check_phi_heads(q, phi)
    flags = flags_for(rotate_qk=rotate_qk, rotate_v=rotate_v, alibi=alibi is not None,
                      shared_phi=phi.shape[1] == 1 and q.shape[1] != 1, exclusive=exclusive,
                      forget=logf is not None)
    desc = desc_for(q, flags, scale, head_scale)
    _check_qkv(desc, q=q, k=k, v=v)
    _check_angles(desc, phi=phi)
    _check_alibi(desc, alibi)
    _check_rows(desc, logf=logf)
    _require_gpu(q, k, v, phi, alibi, logf)
    out = torch.empty_like(q)
    theta = torch.empty_like(phi)
    B, H, L, _ = q.shape
    lse = torch.empty(B, H, L, dtype=torch.float32, device=q.device) if with_lse else None
    state = scan_state(desc, q.device)
    ws = workspace(desc, q.device)
    _check("arp_forward_ex", lib().arp_forward_ex(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(phi), _ptr(alibi), _ptr(logf),
        _ptr(theta), _ptr(out), _ptr(lse), _ptr(state), _nbytes(state), _ptr(ws), _nbytes(ws),
        _stream(q.device)))
    return out, theta, lse
