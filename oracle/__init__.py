"""fp64 CPU oracle for causal attention with accumulated SO(2) rotations.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the GPU library never does, and the two
share no code.  The arithmetic lives in ``arp_oracle.c`` (plain C, fp64,
OpenMP over rows); this module only marshals numpy arrays into it.

Array conventions (numpy, C-contiguous):
  q, k, v   [B, H, L, d]   float32, or uint16 holding bf16 bit patterns
  phi       [B, Hphi, L, d/2] float32, Hphi in {1, H}
  alibi     [H] float32 slopes (used only with the ALIBI flag)
Outputs are float64.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(brute-force route products, closed-form RoPE, shift invariance,
orthogonality, textbook attention, closed-form softmax weights, the matched
score of the method paper's App. B.6, and the RoPE post's worked numbers);
the gradients by ``tests/test_oracle_backward.py`` (central differences of
the forward, the one-token closed form, invariance under a common angle
shift, the column-sum identities of softmax attention, and the textbook
attention gradient of a library autodiff); the forget-gate bias by
``tests/test_oracle_forget.py``; the on-the-fly step angles by
``tests/test_oracle_generators.py`` (Philox4x64-10 against numpy's independent
Philox generator, the counter layout with numpy's words, uniformity, the token
and constant sources against explicit loops).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
# A test of the pins themselves may point this package at a deliberately
# broken build of the same source (see tests/test_oracle_mutants.py).
_LIB_OVERRIDE = os.environ.get("ARP_ORACLE_LIB")

ROTATE_QK = 1
ROTATE_V = 2
ALIBI = 4
SCAN_EXCLUSIVE = 16
FORGET = 64

DTYPE_F32 = 0
DTYPE_BF16 = 1


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("phi_heads", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("scale", ctypes.c_double),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("phi", ctypes.c_void_p),
        ("alibi_slopes", ctypes.c_void_p),
        ("logf", ctypes.c_void_p),
        ("head_scale", ctypes.c_void_p),
    ]


_LIB = None


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        path = _LIB_OVERRIDE or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"oracle library missing: {path}; run `python oracle/build.py`")
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_angle_scan.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int, dp]
        lib.oracle_angle_scan.restype = None
        lib.oracle_wrap.argtypes = [ctypes.c_double]
        lib.oracle_wrap.restype = ctypes.c_double
        lib.oracle_wrap_array.argtypes = [dp, ctypes.c_int64, dp]
        lib.oracle_wrap_array.restype = None
        lib.oracle_rotate_rows.argtypes = [ctypes.c_void_p, ctypes.c_int32, dp, ctypes.c_int64,
                                           ctypes.c_int64, ctypes.c_int, dp]
        lib.oracle_rotate_rows.restype = None
        lib.oracle_theta.argtypes = [ctypes.POINTER(_Problem), dp]
        lib.oracle_theta.restype = ctypes.c_int
        lib.oracle_scores_row.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, dp]
        lib.oracle_scores_row.restype = ctypes.c_int
        lib.oracle_attention_rows.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p,
                                              ctypes.c_int64, ctypes.c_int, dp]
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_backward.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_int,
                                        dp, dp, dp, dp, dp, dp]
        lib.oracle_backward.restype = ctypes.c_int
        u64p = ctypes.POINTER(ctypes.c_uint64)
        lib.oracle_philox4x64_10.argtypes = [u64p, u64p, u64p]
        lib.oracle_philox4x64_10.restype = None
        lib.oracle_random_phi.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_random_phi.restype = None
        lib.oracle_adascale_lambda.argtypes = [dp, dp, ctypes.c_int64, ctypes.c_double,
                                               ctypes.c_double, dp]
        lib.oracle_adascale_lambda.restype = None
        _LIB = lib
    return _LIB


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _io_dtype(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DTYPE_F32
    if a.dtype == np.uint16:
        return DTYPE_BF16
    raise TypeError(f"q/k/v must be float32 or uint16 (bf16 bits), got {a.dtype}")


def angle_scan(phi: np.ndarray, exclusive: bool = False) -> np.ndarray:
    """Unwrapped fp64 prefix sums of phi along axis -2 (phi is [..., L, P] float32)."""
    phi = np.ascontiguousarray(phi, dtype=np.float32)
    L, P = phi.shape[-2], phi.shape[-1]
    nseg = int(np.prod(phi.shape[:-2], dtype=np.int64)) if phi.ndim > 2 else 1
    out = np.empty(phi.shape, dtype=np.float64)
    _lib().oracle_angle_scan(phi.ctypes.data, nseg, L, P, int(exclusive), _dptr(out))
    return out


def wrap(x) -> np.ndarray:
    """Angles reduced into [-pi, pi)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    _lib().oracle_wrap_array(_dptr(x), x.size, _dptr(out))
    return out


def rotate_rows(x: np.ndarray, angle: np.ndarray, inverse: bool = False) -> np.ndarray:
    """R(angle) x per pair for rows of x ([..., d]); angle is [..., d/2] (any float dtype)."""
    x = np.ascontiguousarray(x)
    d = x.shape[-1]
    nrows = x.size // d
    ang = np.ascontiguousarray(angle, dtype=np.float64)
    assert ang.size == nrows * (d // 2)
    out = np.empty(x.shape, dtype=np.float64)
    _lib().oracle_rotate_rows(x.ctypes.data, _io_dtype(x), _dptr(ang), nrows, d, int(inverse),
                              _dptr(out))
    return out


def philox4x64_10(counter, key) -> np.ndarray:
    """The four 64-bit words of the Philox4x64-10 block for a 4-word counter and
    a 2-word key (Salmon et al., SC 2011)."""
    c = np.ascontiguousarray(counter, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    assert c.shape == (4,) and k.shape == (2,)
    out = np.empty(4, dtype=np.uint64)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    _lib().oracle_philox4x64_10(c.ctypes.data_as(u64p), k.ctypes.data_as(u64p),
                                out.ctypes.data_as(u64p))
    return out


def random_phi(batch: int, phi_heads: int, seqlen: int, npairs: int, seed: int, step: int,
               bound) -> np.ndarray:
    """Random step angles [B, Hphi, L, P] (fp32) of the method paper's random
    variant: uniform on (-bound[g, p], bound[g, p]), 32 Philox bits per element,
    one block per two positions of four pairs (arp_oracle.c gives the layout)."""
    bound = np.ascontiguousarray(bound, dtype=np.float32)
    assert bound.shape == (phi_heads, npairs)
    out = np.empty((batch, phi_heads, seqlen, npairs), dtype=np.float32)
    _lib().oracle_random_phi(batch, phi_heads, seqlen, npairs, int(seed), int(step),
                             bound.ctypes.data, out.ctypes.data)
    return out


def token_phi(tokens, table) -> np.ndarray:
    """Step angles of the learned token-rotation variant: phi[b, g, t, p] =
    table[tokens[b, t], g, p] (tokens [B, L] integers in [0, V), table
    [V, Hphi, P] fp32)."""
    tokens = np.asarray(tokens)
    table = np.asarray(table, dtype=np.float32)
    return np.ascontiguousarray(table[tokens].transpose(0, 2, 1, 3))


def constant_phi(batch: int, seqlen: int, freq) -> np.ndarray:
    """Position-independent step angles (RoPE, or per-head learned frequencies):
    phi[b, g, t, p] = freq[g, p]."""
    freq = np.asarray(freq, dtype=np.float32)
    return np.ascontiguousarray(np.broadcast_to(freq[None, :, None, :],
                                                (batch, freq.shape[0], seqlen, freq.shape[1])))


class Problem:
    """Holds the arrays of one attention problem and the C descriptor pointing at them."""

    def __init__(self, q, k, v, phi, flags: int, scale: float | None = None, alibi=None,
                 logf=None, head_scale=None):
        self.q = np.ascontiguousarray(q)
        self.k = np.ascontiguousarray(k)
        self.v = np.ascontiguousarray(v)
        self.phi = np.ascontiguousarray(phi, dtype=np.float32)
        if self.q.shape != self.k.shape or self.q.shape != self.v.shape or self.q.ndim != 4:
            raise ValueError("q, k, v must share one [B, H, L, d] shape")
        if not (self.q.dtype == self.k.dtype == self.v.dtype):
            raise ValueError("q, k, v must share one dtype")
        B, H, L, d = self.q.shape
        if self.phi.shape[0] != B or self.phi.shape[2:] != (L, d // 2) or self.phi.shape[1] not in (1, H):
            raise ValueError(f"phi shape {self.phi.shape} does not match q {self.q.shape}")
        self.alibi = None if alibi is None else np.ascontiguousarray(alibi, dtype=np.float32)
        if flags & ALIBI and (self.alibi is None or self.alibi.shape != (H,)):
            raise ValueError("ALIBI needs one slope per head")
        self.logf = None if logf is None else np.ascontiguousarray(logf, dtype=np.float32)
        if flags & FORGET and (self.logf is None or self.logf.shape != (B, H, L)):
            raise ValueError("FORGET needs log forget gates [B, H, L]")
        self.head_scale = (None if head_scale is None
                           else np.ascontiguousarray(head_scale, dtype=np.float32))
        if self.head_scale is not None and self.head_scale.shape != (H,):
            raise ValueError("head_scale needs one multiplier per head")
        self.shape = (B, H, L, d)
        self.flags = int(flags)
        self.scale = float(1.0 / np.sqrt(d) if scale is None else scale)
        self.c = _Problem(B, H, L, d, self.phi.shape[1], _io_dtype(self.q), self.flags, self.scale,
                          self.q.ctypes.data, self.k.ctypes.data, self.v.ctypes.data,
                          self.phi.ctypes.data,
                          None if self.alibi is None else self.alibi.ctypes.data,
                          None if self.logf is None else self.logf.ctypes.data,
                          None if self.head_scale is None else self.head_scale.ctypes.data)

    def theta(self) -> np.ndarray:
        B, H, L, d = self.shape
        out = np.empty((B, self.phi.shape[1], L, d // 2), dtype=np.float64)
        rc = _lib().oracle_theta(ctypes.byref(self.c), _dptr(out))
        if rc:
            raise RuntimeError(f"oracle_theta failed: {rc}")
        return out

    def scores_row(self, b: int, h: int, i: int) -> np.ndarray:
        out = np.empty(i + 1, dtype=np.float64)
        rc = _lib().oracle_scores_row(ctypes.byref(self.c), b, h, i, _dptr(out))
        if rc:
            raise RuntimeError(f"oracle_scores_row failed: {rc}")
        return out

    def rows(self, rows, nthreads: int = 0) -> np.ndarray:
        """Output rows; rows holds flat indices (b*H + h)*L + i."""
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((rows.size, self.shape[3]), dtype=np.float64)
        rc = _lib().oracle_attention_rows(ctypes.byref(self.c), rows.ctypes.data, rows.size,
                                          int(nthreads), _dptr(out))
        if rc:
            raise RuntimeError(f"oracle_attention_rows failed: {rc}")
        return out

    def backward(self, dout, nthreads: int = 0) -> dict:
        """Gradients for the upstream gradient dout ([B, H, L, d], the dtype of q):
        dict of fp64 arrays dq, dk, dv [B, H, L, d], dtheta [B, H, L, d/2]
        (per head), dphi (the shape of phi) and, with the forget gate, dlogf
        [B, H, L].  O(L^2 d) per head."""
        dout = np.ascontiguousarray(dout)
        if dout.shape != self.q.shape or dout.dtype != self.q.dtype:
            raise ValueError("dout must match q in shape and dtype")
        B, H, L, d = self.shape
        out = {n: np.empty(self.shape, dtype=np.float64) for n in ("dq", "dk", "dv")}
        out["dtheta"] = np.empty((B, H, L, d // 2), dtype=np.float64)
        out["dphi"] = np.empty(self.phi.shape, dtype=np.float64)
        gated = (self.flags & FORGET) != 0
        if gated:
            out["dlogf"] = np.empty((B, H, L), dtype=np.float64)
        rc = _lib().oracle_backward(ctypes.byref(self.c), dout.ctypes.data, int(nthreads),
                                    _dptr(out["dq"]), _dptr(out["dk"]), _dptr(out["dv"]),
                                    _dptr(out["dtheta"]), _dptr(out["dphi"]),
                                    _dptr(out["dlogf"]) if gated else None)
        if rc:
            raise RuntimeError(f"oracle_backward failed: {rc}")
        return out

    def output(self, nthreads: int = 0) -> np.ndarray:
        """The full output [B, H, L, d] (small problems only: O(L^2 d) per head)."""
        B, H, L, d = self.shape
        return self.rows(np.arange(B * H * L, dtype=np.int64), nthreads).reshape(B, H, L, d)


def attention(q, k, v, phi, flags: int, scale=None, alibi=None, nthreads: int = 0,
              logf=None, head_scale=None) -> np.ndarray:
    return Problem(q, k, v, phi, flags, scale, alibi, logf, head_scale).output(nthreads)


def adascale_lambda(tau, gamma, L: float, L_ref: float) -> np.ndarray:
    """AdaScale's inverse temperatures lambda_h(L) = (1/tau_h) [ln(1 + max(L, L_ref)/L_ref)]^gamma_h
    (AdaRoPE Sec. 3.3), fp64, one per head."""
    tau = np.ascontiguousarray(tau, dtype=np.float64)
    gamma = np.ascontiguousarray(gamma, dtype=np.float64)
    if tau.shape != gamma.shape or tau.ndim != 1:
        raise ValueError("tau and gamma must be [heads]")
    out = np.empty_like(tau)
    _lib().oracle_adascale_lambda(_dptr(tau), _dptr(gamma), tau.size, ctypes.c_double(L),
                                  ctypes.c_double(L_ref), _dptr(out))
    return out
