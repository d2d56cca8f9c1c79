"""Seeded synthetic inputs for the spacetime-attention workloads.

This module is the only code that both the CPU oracle side (``oracle/``,
``tests/``) and the HIP side (``bench.py``, the GPU tests) draw on. It holds
the workload shapes, the seeded random draws and the round-to-nearest-even
conversion of the drawn values to bfloat16, and none of the arithmetic of
patchify, RoPE or attention.

Recipe (every workload): ``numpy.random.Generator(PCG64(seed))``; tensors are
drawn in the order listed for the workload with ``standard_normal`` in
float32, scaled by the stated standard deviation in float32, and, for bf16
workloads, rounded to bfloat16 with round-to-nearest-even. Both sides then
consume those identical values: the GPU as bf16 (or fp32) bits, the oracle as
float32 copies of the same values, which it widens to fp64 exactly.

Shapes follow the pages:
- the tiny video DiT of the "Video and 3D Generation" cheatsheet (section
  "Tiny video DiT": input (1,4,8,16,16), Conv3d with stride equal to kernel
  (2,2,2), grid (4,8,8), width 64, 2 heads);
- the Wan2.1 480p and 720p token grids of "Video Diffusion Models, in depth"
  (Step 2: 21 x 30 x 52 = 32,760 and 21 x 45 x 80 = 75,600 tokens) and of
  "How AI Generates Video: Inside Sora and Wan2.1 on a Real GPU" (section 4:
  latent [1,16,21,60,104], 1x2x2 tubes, width 1,536 = 12 heads x 128);
- the 40-head, width-5,120 14B shape of "Video Diffusion Models, in depth"
  (Step 2 and Step 3).
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# bfloat16 round-to-nearest-even on the host
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bits, round-to-nearest-even (NaN kept NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bits -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 value, returned as float32."""
    return bf16_to_f32(bf16_bits(x))


# ----------------------------------------------------------------------------
# Draws
# ----------------------------------------------------------------------------

_CHUNK = 1 << 24


def _normal_f32(gen: np.random.Generator, shape, std: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        gen.standard_normal(e - s, dtype=np.float32, out=out[s:e])
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


@dataclasses.dataclass
class Drawn:
    """One drawn tensor: float32 values (already bf16-exact for bf16) and,
    for bf16 workloads, the uint16 bits the GPU consumes."""
    name: str
    f32: np.ndarray
    bits: Optional[np.ndarray]


def draw(seed: int, specs: List[Tuple[str, tuple, float]], dtype: str) -> Dict[str, Drawn]:
    """Draw tensors in order from PCG64(seed). ``specs``: (name, shape, std)."""
    gen = np.random.Generator(np.random.PCG64(seed))
    out: Dict[str, Drawn] = {}
    for name, shape, std in specs:
        v = _normal_f32(gen, shape, std)
        if dtype == "bf16":
            bits = bf16_bits(v)
            out[name] = Drawn(name, bf16_to_f32(bits).reshape(shape), bits.reshape(shape))
        elif dtype == "f32":
            out[name] = Drawn(name, v, None)
        else:
            raise ValueError(f"unknown dtype {dtype!r}")
    return out


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    """A token grid (T, Hp, Wp) with heads x head_dim, batch B and a dtype.

    Q/K/V are token-major ``[B, N, heads, head_dim]`` with
    ``N = T*Hp*Wp`` and token ``n = (t*Hp + h)*Wp + w``.
    A workload with a ``latent`` also describes the patchify input
    ``[B, C, T*pt, Hp*ph, Wp*pw]`` and its Conv3d weight.
    """
    name: str
    B: int
    T: int
    Hp: int
    Wp: int
    heads: int
    head_dim: int
    dtype: str
    seed: int
    C: int = 0
    patch: Tuple[int, int, int] = (1, 1, 1)
    latent_std: float = 1.0
    weight_std: float = 0.02
    rope_split: Optional[Tuple[int, int, int]] = None
    window: Optional[Tuple[int, int, int]] = None

    @property
    def N(self) -> int:
        return self.T * self.Hp * self.Wp

    @property
    def dim(self) -> int:
        return self.heads * self.head_dim

    @property
    def latent_shape(self) -> Tuple[int, int, int, int, int]:
        pt, ph, pw = self.patch
        return (self.B, self.C, self.T * pt, self.Hp * ph, self.Wp * pw)

    @property
    def weight_shape(self) -> Tuple[int, int, int, int, int]:
        pt, ph, pw = self.patch
        return (self.dim, self.C, pt, ph, pw)

    def qkv_shape(self) -> Tuple[int, int, int, int]:
        return (self.B, self.N, self.heads, self.head_dim)

    def draw_qkv(self, q_scale: float = 1.0) -> Dict[str, Drawn]:
        """Independent N(0,1) Q, K, V drawn in that order (``q_scale``
        multiplies the Q and K standard deviation, for peaky-softmax cases)."""
        s = self.qkv_shape()
        return draw(self.seed, [("q", s, q_scale), ("k", s, q_scale), ("v", s, 1.0)], self.dtype)

    def draw_latent(self) -> Dict[str, Drawn]:
        """The patchify input drawn first, then the Conv3d weight (no bias)."""
        return draw(self.seed, [("x", self.latent_shape, self.latent_std),
                                ("w", self.weight_shape, self.weight_std)], self.dtype)


WORKLOADS: Dict[str, Workload] = {
    # Tiny video DiT: latent (1,4,8,16,16) fp32 N(0,1), patch (2,2,2),
    # grid (4,8,8) = 256 tokens, width 64 = 2 heads x 32, weights N(0, 0.02^2).
    "tiny": Workload("tiny", B=1, T=4, Hp=8, Wp=8, heads=2, head_dim=32, dtype="f32",
                     seed=0, C=4, patch=(2, 2, 2)),
    # Wan 1.3B-shaped 480p full 3D attention: 21 x 30 x 52 tokens, 12 x 128.
    "480p_full": Workload("480p_full", B=1, T=21, Hp=30, Wp=52, heads=12, head_dim=128,
                          dtype="bf16", seed=1),
    # Same shape, divided attention, batch 2 (the CFG pair).
    "480p_divided": Workload("480p_divided", B=2, T=21, Hp=30, Wp=52, heads=12, head_dim=128,
                             dtype="bf16", seed=2),
    # 14B-shaped 720p full 3D attention: 21 x 45 x 80 tokens, 40 x 128.
    "720p_full": Workload("720p_full", B=1, T=21, Hp=45, Wp=80, heads=40, head_dim=128,
                          dtype="bf16", seed=3),
    # Block input path: latent (1,16,21,60,104) bf16 -> 1x2x2 patchify to 1536
    # -> 3D RoPE [44,42,42] -> divided attention, 12 x 128.
    "block_input": Workload("block_input", B=1, T=21, Hp=30, Wp=52, heads=12, head_dim=128,
                            dtype="bf16", seed=4, C=16, patch=(1, 2, 2),
                            rope_split=(44, 42, 42)),
    # Windowed attention on the 480p grid: windows of 3 latent frames x half
    # the frame height x half its width, 3 x 15 x 26 = 1,170 tokens, 28 windows.
    "480p_window": Workload("480p_window", B=1, T=21, Hp=30, Wp=52, heads=12, head_dim=128,
                            dtype="bf16", seed=6, window=(3, 15, 26)),
}


@dataclasses.dataclass(frozen=True)
class CrossWorkload:
    """Video queries ``[B, Nq, heads, head_dim]`` against text keys and values
    ``[B, Nk, heads, head_dim]``, drawn N(0,1) in the order q, k, v."""
    name: str
    B: int
    Nq: int
    Nk: int
    heads: int
    head_dim: int
    dtype: str
    seed: int

    def draw(self, q_scale: float = 1.0) -> Dict[str, Drawn]:
        qs = (self.B, self.Nq, self.heads, self.head_dim)
        ks = (self.B, self.Nk, self.heads, self.head_dim)
        return draw(self.seed, [("q", qs, q_scale), ("k", ks, q_scale), ("v", ks, 1.0)], self.dtype)


CROSS_WORKLOADS: Dict[str, CrossWorkload] = {
    # Wan 1.3B attn2 at 480p / 81 frames: 32,760 video queries against the 512
    # UMT5 text embeddings projected to 12 heads x 128.
    "cross_480p": CrossWorkload("cross_480p", B=1, Nq=32760, Nk=512, heads=12, head_dim=128,
                                dtype="bf16", seed=5),
}


@dataclasses.dataclass(frozen=True)
class QkvWorkload:
    """The projection in front of self-attention: tokens x [B, N, dim] drawn
    N(0,1), then the fused weight [3*dim, dim] and bias [3*dim] drawn
    N(0, weight_std^2), then the Q and K RMSNorm gains [dim] drawn as
    1 + N(0, weight_std^2), in that order."""
    name: str
    B: int
    T: int
    Hp: int
    Wp: int
    heads: int
    head_dim: int
    dtype: str
    seed: int
    weight_std: float = 0.02
    rope_split: Optional[Tuple[int, int, int]] = None

    @property
    def N(self) -> int:
        return self.T * self.Hp * self.Wp

    @property
    def dim(self) -> int:
        return self.heads * self.head_dim

    def draw(self) -> Dict[str, Drawn]:
        dim, s = self.dim, self.weight_std
        d = draw(self.seed, [("x", (self.B, self.N, dim), 1.0), ("w", (3 * dim, dim), s), ("bias", (3 * dim,), s),
                             ("gq", (dim,), s), ("gk", (dim,), s)], "f32")
        out: Dict[str, Drawn] = {}
        for name, t in d.items():
            v = t.f32 + np.float32(1.0) if name in ("gq", "gk") else t.f32
            if self.dtype == "bf16":
                bits = bf16_bits(v)
                out[name] = Drawn(name, bf16_to_f32(bits).reshape(v.shape), bits.reshape(v.shape))
            else:
                out[name] = Drawn(name, v, None)
        return out


QKV_WORKLOADS: Dict[str, QkvWorkload] = {
    # Wan 1.3B-shaped attn1 input at 480p: 32,760 tokens of width 1,536 ->
    # Q, K, V of 12 heads x 128, per-head RMSNorm on Q and K, RoPE [44,42,42].
    "qkv_480p": QkvWorkload("qkv_480p", B=1, T=21, Hp=30, Wp=52, heads=12, head_dim=128, dtype="bf16", seed=7,
                            rope_split=(44, 42, 42)),
}


def small_grid(name: str, B: int, T: int, Hp: int, Wp: int, heads: int, head_dim: int,
               dtype: str, seed: int, **kw) -> Workload:
    """An ad-hoc workload for parity and edge cases."""
    return Workload(name, B=B, T=T, Hp=Hp, Wp=Wp, heads=heads, head_dim=head_dim,
                    dtype=dtype, seed=seed, **kw)


def sample_rows(N: int, stride: int, offset: int = 0) -> np.ndarray:
    """Every ``stride``-th query token from ``offset``, plus the last token,
    so a sample always touches the ragged tail."""
    r = np.arange(offset, N, stride, dtype=np.int64)
    if r.size == 0 or r[-1] != N - 1:
        r = np.append(r, np.int64(N - 1))
    return r
