"""Closed-form counts the pages state: token grids, pair counts and FLOPs.

TEST INFRASTRUCTURE (part of the oracle): used by the tests and by the
benchmark for its algorithmic FLOP and byte counts' cross-checks only.

Each function states, in its own terms, the rule of the passage it cites.
"""

from __future__ import annotations

from typing import Sequence, Tuple

# Wan2.1's causal VAE compresses time by 4 and each spatial axis by 8
# ("Video Diffusion Models, in depth", Step 1); its DiT cuts the latent
# into bricks of 1 latent frame by 2 x 2 latent pixels (same page, Step 2).
WAN_COMPRESSION = (4, 8, 8)
WAN_PATCH = (1, 2, 2)


def count_tokens(T: int, H: int, W: int, p_t: int = 2, p_h: int = 8, p_w: int = 8) -> int:
    """(T/P_t)*(H/P_h)*(W/P_w) video tokens, with the cheatsheet defaults
    p_t = 2, p_h = p_w = 8 ("Video and 3D Generation", "Formulas and numbers"
    and "Defaults in the code")."""
    return (T // p_t) * (H // p_h) * (W // p_w)


def latent_frames(frames: int, t_stride: int = 4) -> int:
    """Causal VAE frame rule: frame 0 becomes a latent frame of its own and
    every further run of t_stride frames becomes one more ("Video Diffusion
    Models, in depth", Step 1: 81 frames give 1 + 80/4 = 21)."""
    rest = frames - 1
    return 1 + rest // t_stride


def latent_frames_ceil(frames: int, t_comp: int = 4) -> int:
    """ceil(F / t_comp) latent frames ("Video as a 3D signal", cheat sheet)."""
    return -(-frames // t_comp)


def spacetime_grid(frames: int, height: int, width: int,
                   compression: Sequence[int] = WAN_COMPRESSION,
                   patch: Sequence[int] = WAN_PATCH) -> Tuple[int, int, int]:
    """Token grid (T, Hp, Wp) of a clip: the VAE's latent extents (time by
    the causal rule, each spatial axis divided by its stride), each then
    divided by the brick along that axis; remainders are dropped ("Video
    Diffusion Models, in depth", Steps 1 and 2)."""
    latent = (latent_frames(frames, compression[0]),
              height // compression[1],
              width // compression[2])
    return tuple(extent // brick for extent, brick in zip(latent, patch))


def spacetime_tokens(frames: int, height: int, width: int,
                     compression: Sequence[int] = WAN_COMPRESSION,
                     patch: Sequence[int] = WAN_PATCH) -> int:
    """Number of spacetime tokens: the product of the grid's extents."""
    T, Hp, Wp = spacetime_grid(frames, height, width, compression, patch)
    return T * Hp * Wp


def dense_flop(params: float, tokens: int) -> float:
    """Every weight takes part in one multiply-add per token: 2*P*N FLOP per
    forward ("Video Diffusion Models, in depth", Step 2)."""
    return 2.0 * params * tokens


def attention_flop(tokens: int, width: int, layers: int) -> float:
    """The score product and the value product, over every layer: 4*N^2*dim
    FLOP per forward ("Video Diffusion Models, in depth", Step 2)."""
    per_layer = 2 * (2 * tokens * tokens * width)  # two N x N x width products, 2 FLOP per multiply-add
    return float(per_layer * layers)


def attention_flops_full(B: int, heads: int, N: int, D: int) -> int:
    """QK^T and PV, 2 FLOP per multiply-add each: 4*N^2*D per (b, head)."""
    return 4 * B * heads * N * N * D


def attention_flops_spatial(B: int, heads: int, T: int, HW: int, D: int) -> int:
    """T frames of HW tokens each: the T*(HW)^2 term of the divided cost."""
    return 4 * B * heads * T * HW * HW * D


def attention_flops_temporal(B: int, heads: int, T: int, HW: int, D: int) -> int:
    """HW positions of T tokens each: the (HW)*T^2 term of the divided cost."""
    return 4 * B * heads * HW * T * T * D


def divided_pairs(T: int, HW: int) -> int:
    """(HW)*T^2 + T*(HW)^2 query-key pairs ("Video and 3D Generation",
    "Formulas and numbers", divided attention)."""
    return HW * T * T + T * HW * HW


def full_pairs(N: int) -> int:
    return N * N


def fp16_bytes(pairs: int) -> int:
    """One fp16 score per pair, 2 bytes ("How AI Generates Video ...", section 2)."""
    return 2 * pairs


def temporal_bytes(B: int, heads: int, N: int, D: int, elem: int = 2) -> int:
    """Algorithmic HBM traffic of one attention pass that reads Q, K, V once
    and writes O once: 4 tensors of B*N*heads*D elements."""
    return 4 * B * N * heads * D * elem
