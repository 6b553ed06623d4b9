"""Seeded synthetic inputs for accumulated-rotation causal attention.

This module holds random draws and dtype packing only -- none of the method's
arithmetic (no prefix sum, rotation, score or softmax).  Both the GPU path and
the CPU oracle consume its arrays, bit for bit.

The five workloads stand in for the small decoder experiments of "Why Do
Accumulated Transformations Extrapolate?" (Sec. 7 and its "Model variants"
paragraph): a 1024-token training shape, evaluation at 16x that length, a
random-angle far-mass configuration with a distance bias, and the RoPE special
case.  Their angle generators follow that paragraph:

* token-table angles: one learned angle per (token id, pair), shared by all
  heads of a layer -> a table indexed by token id;
* learned token-dependent angles phi_t = W x_t, one projection per head;
* random angles drawn i.i.d. per position and pair (here uniform on [-pi, pi),
  the a = pi case of the paper's Example 1, for which E cos(phi) = 0);
* RoPE: a constant angle theta_p = base^(-2p/d) per pair (AdaRoPE Sec. 2.1).

Randomness: one ``numpy.random.Generator(PCG64(seed))`` per workload, drawn in a
fixed order (q, k, v, then the angle tensors).  Never one seed per vector: the
RoPE decay-curve post shows how nearby seeds give correlated streams.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "SPECS", "make", "to_bf16_bits", "from_bf16_bits", "alibi_slopes",
           "causal_pairs", "attn_flops"]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def alibi_slopes(heads: int) -> np.ndarray:
    """Geometric head slopes m_h = 2^(-8h/H), h = 1..H, as fp32."""
    h = np.arange(1, heads + 1, dtype=np.float64)
    return np.power(2.0, -8.0 * h / heads).astype(np.float32)


def rope_frequencies(head_dim: int, base: float = None) -> np.ndarray:
    """RoPE's log-spaced per-pair frequencies base^(-2p/d), p = 0..d/2-1, as fp32
    (also the bounds f_b of the random-angle variant)."""
    base = ROPE_BASE if base is None else base
    p = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(base, -2.0 * p / head_dim).astype(np.float32)


def causal_pairs(seqlen: int) -> int:
    """(query, key) pairs with key <= query in one head."""
    return seqlen * (seqlen + 1) // 2


def attn_flops(batch: int, heads: int, seqlen: int, head_dim: int) -> float:
    """Algorithmic flops of the two contractions over the causal pairs: 4 d per pair."""
    return 4.0 * head_dim * causal_pairs(seqlen) * batch * heads


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    batch: int
    heads: int
    seqlen: int
    head_dim: int
    dtype: str          # "f32" or "bf16"
    angles: str         # "token_table" | "learned" | "uniform" | "rope"
    rotate_v: bool
    alibi: bool
    seed: int
    description: str


SPECS = {
    s.name: s
    for s in [
        Spec("tiny_f32", 1, 2, 256, 64, "f32", "token_table", False, False, 0,
             "tiny fp32 reference: token-table angles shared by both heads, q/k rotation"),
        Spec("train_1k", 8, 8, 1024, 64, "bf16", "learned", False, False, 1,
             "training shape: learned angles phi = W x, q/k rotation"),
        Spec("extrap_16k", 2, 8, 16384, 64, "bf16", "learned", True, False, 2,
             "16x extrapolation: learned angles, q/k/v rotation"),
        Spec("farmass_32k", 1, 16, 32768, 64, "bf16", "uniform", True, True, 3,
             "far-mass control: uniform random angles, q/k/v rotation, distance bias"),
        Spec("rope_8k_d128", 4, 32, 8192, 128, "bf16", "rope", False, False, 4,
             "RoPE special case: constant angles base^(-2p/d), q/k rotation"),
    ]
}

# Width of the token representation x_t fed to the learned angle map, the
# token vocabulary of the token-table generator, and the RoPE base.
LEARNED_WIDTH = 512
LEARNED_STD = 0.02
VOCAB = 256
ROPE_BASE = 10000.0


@dataclasses.dataclass
class Workload:
    spec: Spec
    batch: int
    heads: int
    seqlen: int
    head_dim: int
    q: np.ndarray       # [B, H, L, d] float32, or uint16 bf16 bits
    k: np.ndarray
    v: np.ndarray
    phi: np.ndarray     # [B, Hphi, L, d/2] float32
    alibi: np.ndarray | None  # [H] float32

    @property
    def name(self) -> str:
        return self.spec.name

    @property
    def dtype(self) -> str:
        return self.spec.dtype

    @property
    def phi_heads(self) -> int:
        return self.phi.shape[1]

    @property
    def rotate_v(self) -> bool:
        return self.spec.rotate_v

    @property
    def use_alibi(self) -> bool:
        return self.spec.alibi

    @property
    def flops(self) -> float:
        return attn_flops(self.batch, self.heads, self.seqlen, self.head_dim)

    def values(self, which: str) -> np.ndarray:
        """q/k/v as fp32 values (decoding bf16 bits where needed)."""
        a = getattr(self, which)
        return from_bf16_bits(a) if a.dtype == np.uint16 else a


def _qkv(rng: np.random.Generator, shape, dtype: str):
    d = shape[-1]
    out = []
    for _ in range(3):
        if dtype == "f32":
            out.append(rng.standard_normal(shape, dtype=np.float32))
        else:
            x = rng.standard_normal(shape, dtype=np.float32) * np.float32(1.0 / math.sqrt(d))
            out.append(to_bf16_bits(x))
    return out


def make(name: str, *, batch: int | None = None, heads: int | None = None,
         seqlen: int | None = None, seed: int | None = None) -> Workload:
    """Build a workload; batch/heads/seqlen/seed override the spec (for small test cases)."""
    spec = SPECS[name]
    B = spec.batch if batch is None else batch
    H = spec.heads if heads is None else heads
    L = spec.seqlen if seqlen is None else seqlen
    d = spec.head_dim
    P = d // 2
    rng = np.random.Generator(np.random.PCG64(spec.seed if seed is None else seed))
    q, k, v = _qkv(rng, (B, H, L, d), spec.dtype)

    if spec.angles == "token_table":
        ids = rng.integers(0, VOCAB, size=(B, L))
        table = rng.uniform(-math.pi, math.pi, size=(VOCAB, P)).astype(np.float32)
        phi = table[ids][:, None, :, :]                       # [B, 1, L, P], shared by heads
    elif spec.angles == "learned":
        x = rng.standard_normal((B, L, LEARNED_WIDTH))
        W = rng.standard_normal((LEARNED_WIDTH, H * P)) * LEARNED_STD
        phi = (x @ W).reshape(B, L, H, P).transpose(0, 2, 1, 3)   # [B, H, L, P]
    elif spec.angles == "uniform":
        phi = rng.uniform(-math.pi, math.pi, size=(B, H, L, P))
    elif spec.angles == "rope":
        p = np.arange(P, dtype=np.float64)
        theta = np.power(ROPE_BASE, -2.0 * p / d)
        phi = np.broadcast_to(theta, (B, H, L, P))
    else:  # pragma: no cover
        raise ValueError(spec.angles)
    phi = np.ascontiguousarray(phi, dtype=np.float32)
    alibi = alibi_slopes(H) if spec.alibi else None
    return Workload(spec, B, H, L, d, q, k, v, phi, alibi)
