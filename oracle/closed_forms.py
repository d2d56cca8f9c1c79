"""Closed-form counts the pages state: token grids, pair counts and FLOPs.

TEST INFRASTRUCTURE (part of the oracle): used by the tests and by the
benchmark for its algorithmic FLOP and byte counts' cross-checks only.

Each function is the plain formula of the passage it cites.
"""

from __future__ import annotations

from typing import Tuple


def count_tokens(T: int, H: int, W: int, p_t: int = 2, p_h: int = 8, p_w: int = 8) -> int:
    """(T/P_t)*(H/P_h)*(W/P_w) video tokens, with the cheatsheet defaults
    p_t = 2, p_h = p_w = 8 ("Video and 3D Generation", "Formulas and numbers"
    and "Defaults in the code")."""
    return (T // p_t) * (H // p_h) * (W // p_w)


def latent_frames(frames: int, t_stride: int = 4) -> int:
    """Causal VAE frame rule: the first frame alone, then every t_stride frames
    make one latent frame ("Video Diffusion Models, in depth", Step 1 and the
    video_tokens function of Step 2)."""
    return 1 + (frames - 1) // t_stride


def latent_frames_ceil(frames: int, t_comp: int = 4) -> int:
    """ceil(F / t_comp) latent frames ("Video as a 3D signal", cheat sheet)."""
    return -(-frames // t_comp)


def token_grid(frames: int, height: int, width: int, vae_stride=(4, 8, 8),
               patch=(1, 2, 2)) -> Tuple[int, int, int]:
    """(T, Hp, Wp) after the causal VAE and the patch ("Video Diffusion Models,
    in depth", Step 2, video_tokens)."""
    t_lat = latent_frames(frames, vae_stride[0])
    h_lat, w_lat = height // vae_stride[1], width // vae_stride[2]
    return (t_lat // patch[0], h_lat // patch[1], w_lat // patch[2])


def video_tokens(frames: int, height: int, width: int, vae_stride=(4, 8, 8),
                 patch=(1, 2, 2)) -> int:
    T, Hp, Wp = token_grid(frames, height, width, vae_stride, patch)
    return T * Hp * Wp


def forward_flops(tokens: int, params: float = 14e9, layers: int = 40,
                  dim: int = 5120) -> Tuple[float, float]:
    """Dense FLOPs 2*params*N and attention FLOPs 4*N^2*dim*layers
    ("Video Diffusion Models, in depth", Step 2, forward_flops)."""
    dense = 2 * params * tokens
    attn = 4 * tokens * tokens * dim * layers
    return dense, attn


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
