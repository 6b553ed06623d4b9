"""Helpers for the GPU parity tests: move a seeded workload to the device, run
the library through its C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from accumulated_rotation_positional_amd import binding
from accumulated_rotation_positional_amd import workloads as wl

DEV = torch.device("cuda:0")
BF16_TOL = 2e-2      # max |o_gpu - o_oracle| for bf16 I/O
F32_TOL = 1e-4       # fp32 I/O, scan and rotation
BF16_REL_RMS = 1e-2  # rms(o_gpu - o_oracle) / rms(o_oracle), a tighter diagnostic bound


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def oracle_flags(rotate_qk=True, rotate_v=False, alibi=False, exclusive=False) -> int:
    return ((oracle.ROTATE_QK if rotate_qk else 0) | (oracle.ROTATE_V if rotate_v else 0) |
            (oracle.ALIBI if alibi else 0) | (oracle.SCAN_EXCLUSIVE if exclusive else 0))


def run_forward(w: wl.Workload, *, rotate_qk=True, rotate_v=None, alibi=None, exclusive=False,
                fused=False):
    """The library's forward pass on workload w; returns (o [B,H,L,d] fp32, theta)."""
    rotate_v = w.rotate_v if rotate_v is None else rotate_v
    use_alibi = w.use_alibi if alibi is None else alibi
    say(f"[gpu] forward {w.name} B={w.batch} H={w.heads} L={w.seqlen} d={w.head_dim} "
        f"qk={rotate_qk} v={rotate_v} alibi={use_alibi} excl={exclusive} fused={fused}")
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    phi = to_dev(w.phi)
    al = to_dev(w.alibi if w.alibi is not None else wl.alibi_slopes(w.heads)) if use_alibi else None
    o, theta = binding.forward(q, k, v, phi, rotate_qk=rotate_qk, rotate_v=rotate_v, alibi=al,
                               exclusive=exclusive, fused=fused)
    torch.cuda.synchronize()
    return to_host(o), theta.cpu().numpy()


def oracle_problem(w: wl.Workload, *, rotate_qk=True, rotate_v=None, alibi=None, exclusive=False):
    rotate_v = w.rotate_v if rotate_v is None else rotate_v
    use_alibi = w.use_alibi if alibi is None else alibi
    slopes = (w.alibi if w.alibi is not None else wl.alibi_slopes(w.heads)) if use_alibi else None
    return oracle.Problem(w.q, w.k, w.v, w.phi,
                          oracle_flags(rotate_qk, rotate_v, use_alibi, exclusive), alibi=slopes)


def errors(got: np.ndarray, want: np.ndarray):
    d = got.astype(np.float64) - want
    max_abs = float(np.abs(d).max())
    rel_rms = float(np.sqrt((d ** 2).mean()) / max(np.sqrt((want ** 2).mean()), 1e-30))
    return max_abs, rel_rms


def assert_close(got, want, dtype: str, what: str = ""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs, rel_rms = errors(got, want)
    say(f"[gpu] {what}: max_abs={max_abs:.3e} rel_rms={rel_rms:.3e}")
    if dtype == "f32":
        assert max_abs <= F32_TOL, (what, max_abs)
    else:
        assert max_abs <= BF16_TOL, (what, max_abs)
        assert rel_rms <= BF16_REL_RMS, (what, rel_rms)


def circular_err(theta_gpu: np.ndarray, theta_ref_unwrapped: np.ndarray) -> float:
    return float(np.abs(oracle.wrap(theta_gpu.astype(np.float64) - theta_ref_unwrapped)).max())


def sample_rows(w: wl.Workload, per_head: int = 24, seed: int = 0) -> np.ndarray:
    """Flat row indices (b*H + h)*L + i: tile edges, the ends, and random rows."""
    L = w.seqlen
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = [i for i in (0, 1, 31, 32, 63, 64, 255, 256, 257, L // 2, L - 257, L - 2, L - 1)
             if 0 <= i < L]
    rows = []
    for bh in range(w.batch * w.heads):
        extra = rng.integers(0, L, size=max(per_head - len(fixed), 0))
        for i in sorted(set(fixed) | set(int(x) for x in extra)):
            rows.append(bh * L + i)
    return np.array(rows, dtype=np.int64)
