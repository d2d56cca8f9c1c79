"""spacetime_attention_amd: spacetime attention for video DiTs on MI355X (gfx950).

A thin ctypes binding over ``libvdit.so`` (C ABI in ``include/vdit.h``). Every
function here only checks that the torch tensors it is given are contiguous
device tensors of the right dtype and size, then passes their pointers, the
sizes and torch's current HIP stream to the library; all arithmetic runs in
the library's HIP kernels. Output tensors are allocated with torch when the
caller does not pass one. The library is never replaced by any other code
path: if it is not built, every call raises.

Functions (names as in the C ABI, without the ``vdit_`` prefix):
  patchify(latent, weight, bias=None, *, heads, head_dim, patch)
  rope3d(x, grid, split=(44, 42, 42), theta=10000.0, out=None)
  attn_full(q, k, v, grid, scale=0.0, out=None)
  attn_spatial(q, k, v, grid, scale=0.0, out=None)
  attn_full_rope(q, k, v, grid, split=(44, 42, 42), theta=10000.0, scale=0.0, out=None)
  attn_spatial_rope(q, k, v, grid, split=(44, 42, 42), theta=10000.0, scale=0.0, out=None)
  attn_temporal_rope(q, k, v, grid, split=(44, 42, 42), theta=10000.0, scale=0.0, out=None)
  attn_temporal(q, k, v, grid, scale=0.0, out=None)
  attn_cross(q, k, v, scale=0.0, out=None)
  attn_window(q, k, v, grid, window, scale=0.0, out=None)
  qkv_proj(x, w, bias=None, gamma_q=None, gamma_k=None, *, grid, heads, head_dim, ...)
Token tensors are ``[B, N, heads, head_dim]`` with ``N = T*Hp*Wp`` and token
``(t, h, w)`` at ``n = (t*Hp + h)*Wp + w``; ``grid = (T, Hp, Wp)``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvdit.so")

BF16, F32 = 0, 1
STATUS = ["VDIT_OK", "VDIT_E_NULL", "VDIT_E_SHAPE", "VDIT_E_HEAD_DIM", "VDIT_E_ROPE_SPLIT",
          "VDIT_E_ALIGN", "VDIT_E_ALIAS", "VDIT_E_DTYPE", "VDIT_E_LAUNCH"]
EXPORTS = ("vdit_status_str", "vdit_patchify", "vdit_rope3d", "vdit_attn_full",
           "vdit_attn_spatial", "vdit_attn_full_rope", "vdit_attn_spatial_rope", "vdit_attn_temporal_rope",
           "vdit_attn_temporal",
           "vdit_attn_cross", "vdit_attn_window", "vdit_qkv_proj")


class VditError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code
        self.status = STATUS[code] if 0 <= code < len(STATUS) else str(code)


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libvdit.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m spacetime_attention_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.vdit_status_str.argtypes = [i]
    lib.vdit_status_str.restype = ctypes.c_char_p
    lib.vdit_patchify.argtypes = [vp, vp, vp, vp] + [i] * 14 + [vp]
    lib.vdit_patchify.restype = i
    lib.vdit_rope3d.argtypes = [vp, vp] + [i] * 9 + [f, i, vp]
    lib.vdit_rope3d.restype = i
    for name in ("vdit_attn_full", "vdit_attn_spatial", "vdit_attn_temporal"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp] + [i] * 6 + [f, i, vp]
        fn.restype = i
    for name in ("vdit_attn_full_rope", "vdit_attn_spatial_rope", "vdit_attn_temporal_rope"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp] + [i] * 9 + [f, f, i, vp]
        fn.restype = i
    lib.vdit_attn_cross.argtypes = [vp, vp, vp, vp] + [i] * 5 + [f, i, vp]
    lib.vdit_attn_cross.restype = i
    lib.vdit_attn_window.argtypes = [vp, vp, vp, vp] + [i] * 9 + [f, i, vp]
    lib.vdit_attn_window.restype = i
    lib.vdit_qkv_proj.argtypes = [vp] * 8 + [i] * 9 + [f, f, i, vp]
    lib.vdit_qkv_proj.restype = i
    _lib = lib
    return lib


def status_str(code: int) -> str:
    return load_library().vdit_status_str(code).decode()


def _check(code: int):
    if code != 0:
        raise VditError(code, status_str(code))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _dev(t: Optional[torch.Tensor], name: str, dtype=None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def patchify(latent: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None, *,
             heads: int, head_dim: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Conv3d with stride = kernel as token-major tokens ``[B, N, heads*head_dim]``.

    latent ``[B, C, Tl, Hl, Wl]``; weight ``[heads*head_dim, C, pt, ph, pw]``.
    """
    B, C, Tl, Hl, Wl = latent.shape
    Dout, Cw, pt, ph, pw = weight.shape
    if Cw != C or Dout != heads * head_dim:
        raise ValueError("weight shape does not match latent channels / heads*head_dim")
    T, Hp, Wp = Tl // pt, Hl // ph, Wl // pw
    dt = latent.dtype
    if out is None:
        out = torch.empty((B, T * Hp * Wp, Dout), dtype=dt, device=latent.device)
    elif out.shape != (B, T * Hp * Wp, Dout):
        raise ValueError("out has the wrong shape")
    lib = load_library()
    _check(lib.vdit_patchify(_dev(latent, "latent"), _dev(weight, "weight", dt), _dev(bias, "bias", dt),
                             _dev(out, "out", dt), B, C, pt, ph, pw, Tl, Hl, Wl, heads, T, Hp, Wp,
                             head_dim, _dtype_code(latent), _stream(latent)))
    return out


def rope3d(x: torch.Tensor, grid: Tuple[int, int, int], split: Sequence[int] = (44, 42, 42),
           theta: float = 10000.0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """3D factorised RoPE on ``x [B, N, heads, head_dim]``; ``out`` may be ``x``."""
    B, N, heads, D = x.shape
    T, Hp, Wp = grid
    if N != T * Hp * Wp:
        raise ValueError("token count does not match the grid")
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape:
        raise ValueError("out has the wrong shape")
    lib = load_library()
    _check(lib.vdit_rope3d(_dev(x, "x"), _dev(out, "out", x.dtype), B, heads, T, Hp, Wp, D,
                           int(split[0]), int(split[1]), int(split[2]), float(theta),
                           _dtype_code(x), _stream(x)))
    return out


def _attn(fn_name: str, q, k, v, grid, scale, out):
    B, N, heads, D = q.shape
    T, Hp, Wp = grid
    if N != T * Hp * Wp:
        raise ValueError("token count does not match the grid")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out has the wrong shape")
    lib = load_library()
    dt = q.dtype
    _check(getattr(lib, fn_name)(_dev(q, "q"), _dev(k, "k", dt), _dev(v, "v", dt), _dev(out, "out", dt),
                                 B, heads, T, Hp, Wp, D, float(scale), _dtype_code(q), _stream(q)))
    return out


def attn_full(q, k, v, grid, scale: float = 0.0, out=None) -> torch.Tensor:
    """Full 3D attention over all tokens of each clip."""
    return _attn("vdit_attn_full", q, k, v, grid, scale, out)


def attn_spatial(q, k, v, grid, scale: float = 0.0, out=None) -> torch.Tensor:
    """Attention within each latent frame."""
    return _attn("vdit_attn_spatial", q, k, v, grid, scale, out)


def _attn_rope(fn_name: str, q, k, v, grid, split, theta, scale, out):
    B, N, heads, D = q.shape
    T, Hp, Wp = grid
    if N != T * Hp * Wp:
        raise ValueError("token count does not match the grid")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out has the wrong shape")
    d_t, d_h, d_w = (int(a) for a in split)
    lib = load_library()
    dt = q.dtype
    _check(getattr(lib, fn_name)(_dev(q, "q"), _dev(k, "k", dt), _dev(v, "v", dt), _dev(out, "out", dt),
                                 B, heads, T, Hp, Wp, D, d_t, d_h, d_w, float(theta), float(scale),
                                 _dtype_code(q), _stream(q)))
    return out


def attn_full_rope(q, k, v, grid, split: Sequence[int] = (44, 42, 42), theta: float = 10000.0,
                   scale: float = 0.0, out=None) -> torch.Tensor:
    """Full attention of RoPE(q) against RoPE(k), rotated inside the kernel
    (q and k stay unrotated in memory)."""
    return _attn_rope("vdit_attn_full_rope", q, k, v, grid, split, theta, scale, out)


def attn_spatial_rope(q, k, v, grid, split: Sequence[int] = (44, 42, 42), theta: float = 10000.0,
                      scale: float = 0.0, out=None) -> torch.Tensor:
    """Spatial attention of RoPE(q) against RoPE(k), rotated inside the kernel."""
    return _attn_rope("vdit_attn_spatial_rope", q, k, v, grid, split, theta, scale, out)


def attn_temporal_rope(q, k, v, grid, split: Sequence[int] = (44, 42, 42), theta: float = 10000.0,
                       scale: float = 0.0, out=None) -> torch.Tensor:
    """Temporal attention of RoPE(q) against RoPE(k), rotated inside the kernel."""
    return _attn_rope("vdit_attn_temporal_rope", q, k, v, grid, split, theta, scale, out)


def attn_temporal(q, k, v, grid, scale: float = 0.0, out=None) -> torch.Tensor:
    """Attention across frames at each patch position."""
    return _attn("vdit_attn_temporal", q, k, v, grid, scale, out)


def attn_cross(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float = 0.0,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Cross-attention: q ``[B, Nq, heads, D]`` against k/v ``[B, Nk, heads, D]``."""
    B, Nq, heads, D = q.shape
    Bk, Nk, hk, Dk = k.shape
    if (Bk, hk, Dk) != (B, heads, D) or v.shape != k.shape:
        raise ValueError("q and k/v shapes do not match")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out has the wrong shape")
    lib = load_library()
    dt = q.dtype
    _check(lib.vdit_attn_cross(_dev(q, "q"), _dev(k, "k", dt), _dev(v, "v", dt), _dev(out, "out", dt),
                               B, heads, Nq, Nk, D, float(scale), _dtype_code(q), _stream(q)))
    return out


def attn_window(q, k, v, grid, window, scale: float = 0.0, out=None) -> torch.Tensor:
    """Attention within non-overlapping ``window = (wt, wh, ww)`` spacetime
    windows of the token grid (edge windows clipped by the grid)."""
    B, N, heads, D = q.shape
    T, Hp, Wp = grid
    if N != T * Hp * Wp:
        raise ValueError("token count does not match the grid")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape:
        raise ValueError("out has the wrong shape")
    wt, wh, ww = (int(x) for x in window)
    lib = load_library()
    dt = q.dtype
    _check(lib.vdit_attn_window(_dev(q, "q"), _dev(k, "k", dt), _dev(v, "v", dt), _dev(out, "out", dt),
                                B, heads, T, Hp, Wp, D, wt, wh, ww, float(scale), _dtype_code(q), _stream(q)))
    return out


def qkv_proj(x, w, bias=None, gamma_q=None, gamma_k=None, *, grid, heads: int, head_dim: int,
             split: Optional[Sequence[int]] = None, theta: float = 10000.0, eps: float = 1e-6, out=None):
    """Tokens ``x [B, N, dim]`` -> (q, k, v) ``[B, N, heads, head_dim]``: the
    fused projection ``w [3*dim, dim]`` (+ ``bias``), per-head RMSNorm of Q
    and K with gains ``gamma_q`` / ``gamma_k`` (None: not normalised), and 3D
    RoPE on Q and K when ``split`` is given."""
    B, N, dim = x.shape
    T, Hp, Wp = grid
    if N != T * Hp * Wp or dim != heads * head_dim or tuple(w.shape) != (3 * dim, dim):
        raise ValueError("shapes do not match")
    shape = (B, N, heads, head_dim)
    if out is None:
        out = tuple(torch.empty(shape, dtype=x.dtype, device=x.device) for _ in range(3))
    q, k, v = out
    d_t, d_h, d_w = (int(a) for a in split) if split is not None else (0, 0, 0)
    lib = load_library()
    dt = x.dtype
    opt = lambda t, n: None if t is None else _dev(t, n, dt)
    _check(lib.vdit_qkv_proj(_dev(x, "x"), _dev(w, "w", dt), opt(bias, "bias"), opt(gamma_q, "gamma_q"),
                             opt(gamma_k, "gamma_k"), _dev(q, "q", dt), _dev(k, "k", dt), _dev(v, "v", dt),
                             B, T, Hp, Wp, heads, head_dim, d_t, d_h, d_w, float(theta), float(eps),
                             _dtype_code(x), _stream(x)))
    return q, k, v


def divided(x: torch.Tensor, grid, order=("spatial", "temporal"), split: Optional[Sequence[int]] = None,
            theta: float = 10000.0) -> torch.Tensor:
    """A chain of passes over tokens ``x [B, N, heads, D]``: each pass takes
    q = k = RoPE(x) (or x when ``split`` is None) and v = x.

    With a split, a bf16 temporal pass runs the kernel that rotates q and k
    itself (faster than a separate RoPE pass there, as that pass is bound
    by memory traffic); the full and spatial passes keep the separate RoPE
    pass, which is faster for them."""
    fns = {"spatial": attn_spatial, "temporal": attn_temporal, "full": attn_full}
    cur = x
    for mode in order:
        if split is not None and mode == "temporal" and cur.dtype == torch.bfloat16:
            cur = attn_temporal_rope(cur, cur, cur, grid, split, theta)
            continue
        qk = rope3d(cur, grid, split, theta) if split is not None else cur
        cur = fns[mode](qk, qk, cur, grid)
    return cur
