"""fp64 CPU oracle for spacetime attention, patchify and 3D RoPE.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package; the product path (the HIP library
and its Python binding) never does. It shares no code with the HIP side.

The arithmetic lives in ``oracle.c`` (plain nested loops in double precision,
built with gcc into ``liboracle.so``); this module loads it with ctypes,
passes numpy float64 arrays and adds the closed-form counts of the pages
(``closed_forms``) and the composition of passes.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

from . import closed_forms  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FULL, SPATIAL, TEMPORAL = 0, 1, 2
_MODES = {"full": FULL, "spatial": SPATIAL, "temporal": TEMPORAL}

OK, E_ARG, E_ROPE_SPLIT, E_MODE, E_NOMEM = 0, 1, 2, 3, 4


class OracleError(RuntimeError):
    pass


class RopeSplitError(ValueError):
    """The axis split does not sum to the head width, or a part is odd."""


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.oracle_patchify.argtypes = [dp, dp, dp, dp] + [i] * 9
        lib.oracle_patchify.restype = i
        lib.oracle_rope3d.argtypes = [dp, dp] + [i] * 9 + [ctypes.c_double]
        lib.oracle_rope3d.restype = i
        lib.oracle_rope3d_rows.argtypes = [dp, dp, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64] + [i] * 9 + [
            ctypes.c_double]
        lib.oracle_rope3d_rows.restype = i
        lib.oracle_attention.argtypes = [dp, dp, dp, dp] + [i] * 6 + [ctypes.c_double, i,
                                                                      ctypes.POINTER(ctypes.c_int64),
                                                                      ctypes.c_int64]
        lib.oracle_attention.restype = i
        lib.oracle_cross_attention.argtypes = [dp, dp, dp, dp] + [i] * 5 + [ctypes.c_double,
                                                                            ctypes.POINTER(ctypes.c_int64),
                                                                            ctypes.c_int64]
        lib.oracle_cross_attention.restype = i
        lib.oracle_window_attention.argtypes = [dp, dp, dp, dp] + [i] * 9 + [ctypes.c_double,
                                                                             ctypes.POINTER(ctypes.c_int64),
                                                                             ctypes.c_int64]
        lib.oracle_window_attention.restype = i
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _check(rc: int):
    if rc == E_ROPE_SPLIT:
        raise RopeSplitError("rope split must sum to the head width, with even parts")
    if rc != OK:
        raise OracleError(f"oracle returned {rc}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


# ----------------------------------------------------------------------------
# The three routines
# ----------------------------------------------------------------------------

def patchify(x, w, bias=None) -> np.ndarray:
    """Conv3d with stride = kernel. x: (B,C,Tl,Hl,Wl); w: (Dout,C,pt,ph,pw).

    Returns tokens (B, N, Dout), N = (Tl//pt)*(Hl//ph)*(Wl//pw), token-major.
    """
    x, w = _f64(x), _f64(w)
    B, C, Tl, Hl, Wl = x.shape
    Dout, Cw, pt, ph, pw = w.shape
    if Cw != C:
        raise OracleError("weight channels do not match the latent")
    b = None if bias is None else _f64(bias)
    N = (Tl // pt) * (Hl // ph) * (Wl // pw)
    out = np.empty((B, N, Dout), dtype=np.float64)
    _check(_load().oracle_patchify(_ptr(x), _ptr(w), _ptr(b), _ptr(out),
                                   B, C, Tl, Hl, Wl, pt, ph, pw, Dout))
    return out


def rope3d(x, grid: Tuple[int, int, int], split: Sequence[int], theta: float = 10000.0) -> np.ndarray:
    """3D factorised RoPE on x: (B, N, heads, D) with N = T*Hp*Wp."""
    x = _f64(x)
    B, N, heads, D = x.shape
    T, Hp, Wp = grid
    if N != T * Hp * Wp:
        raise OracleError("token count does not match the grid")
    y = np.empty_like(x)
    _check(_load().oracle_rope3d(_ptr(x), _ptr(y), B, T, Hp, Wp, heads, D,
                                 int(split[0]), int(split[1]), int(split[2]), float(theta)))
    return y


def rope3d_rows(x, grid: Tuple[int, int, int], rows, split: Sequence[int], theta: float = 10000.0) -> np.ndarray:
    """3D RoPE on x: (B, R, heads, D) whose row r is grid token rows[r]."""
    x = _f64(x)
    B, R, heads, D = x.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if rows.shape != (R,):
        raise OracleError("one token index per row")
    T, Hp, Wp = grid
    y = np.empty_like(x)
    _check(_load().oracle_rope3d_rows(_ptr(x), _ptr(y), rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), R,
                                      B, T, Hp, Wp, heads, D, int(split[0]), int(split[1]), int(split[2]),
                                      float(theta)))
    return y


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gamma."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * _f64(gamma)


def qkv_proj(x, w, bias, gamma_q, gamma_k, grid: Tuple[int, int, int], heads: int, head_dim: int,
             split: Optional[Sequence[int]] = None, theta: float = 10000.0, eps: float = 1e-6,
             rows: Optional[np.ndarray] = None):
    """The attention input of a DiT block ("How AI Generates Video ...",
    section 5, attn1): tokens x (B, N, dim) projected by the fused weight
    w (3*dim, dim) (+ bias (3*dim,)) into Q, K and V of heads x head_dim;
    Q and K each RMS-normalised over every head's head_dim values with
    gains gamma_q / gamma_k (dim,) (None: no normalisation), then rotated
    by 3D RoPE when a split is given. Returns q, k, v (B, R, heads, D) for
    the token rows ``rows`` (default: all N)."""
    x, w = _f64(x), _f64(w)
    B, N, dim = x.shape
    T, Hp, Wp = grid
    if N != T * Hp * Wp or dim != heads * head_dim or w.shape != (3 * dim, dim):
        raise OracleError("shapes do not match")
    if rows is None:
        rows = np.arange(N, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    y = x[:, rows] @ w.T
    if bias is not None:
        y = y + _f64(bias)
    R = rows.size
    q, k, v = (y[..., i * dim:(i + 1) * dim].reshape(B, R, heads, head_dim) for i in range(3))
    out = []
    for t, g in ((q, gamma_q), (k, gamma_k)):
        if g is not None:
            t = rmsnorm(t, _f64(g).reshape(heads, head_dim), eps)
        if split is not None:
            t = rope3d_rows(t, grid, rows, split, theta)
        out.append(t)
    return out[0], out[1], np.ascontiguousarray(v)


def attention(q, k, v, grid: Tuple[int, int, int], mode: str = "full",
              scale: float = 0.0, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Softmax attention, q/k/v: (B, N, heads, D); mode full|spatial|temporal.

    With ``rows`` (query tokens), returns (B, len(rows), heads, D).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, heads, D = q.shape
    T, Hp, Wp = grid
    if N != T * Hp * Wp or k.shape != q.shape or v.shape != q.shape:
        raise OracleError("q/k/v shapes do not match the grid")
    if rows is None:
        rp, nrows = None, N
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        rp, nrows = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(rows.size)
    out = np.empty((B, nrows, heads, D), dtype=np.float64)
    _check(_load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, T, Hp, Wp,
                                    heads, D, float(scale), _MODES[mode], rp, nrows))
    return out


def cross_attention(q, k, v, scale: float = 0.0, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Cross-attention, q: (B, Nq, heads, D), k/v: (B, Nk, heads, D).

    With ``rows`` (query tokens), returns (B, len(rows), heads, D).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Nq, heads, D = q.shape
    Bk, Nk, hk, Dk = k.shape
    if (Bk, hk, Dk) != (B, heads, D) or v.shape != k.shape:
        raise OracleError("q and k/v shapes do not match")
    if rows is None:
        rp, nrows = None, Nq
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        rp, nrows = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(rows.size)
    out = np.empty((B, nrows, heads, D), dtype=np.float64)
    _check(_load().oracle_cross_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Nq, Nk, heads, D,
                                          float(scale), rp, nrows))
    return out


def window_attention(q, k, v, grid: Tuple[int, int, int], window: Tuple[int, int, int],
                     scale: float = 0.0, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Attention within non-overlapping (wt, wh, ww) spacetime windows."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, heads, D = q.shape
    T, Hp, Wp = grid
    if N != T * Hp * Wp or k.shape != q.shape or v.shape != q.shape:
        raise OracleError("q/k/v shapes do not match the grid")
    if rows is None:
        rp, nrows = None, N
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        rp, nrows = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(rows.size)
    out = np.empty((B, nrows, heads, D), dtype=np.float64)
    wt, wh, ww = window
    _check(_load().oracle_window_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, T, Hp, Wp, heads, D,
                                           int(wt), int(wh), int(ww), float(scale), rp, nrows))
    return out


# ----------------------------------------------------------------------------
# Composition of passes
# ----------------------------------------------------------------------------

def store(x: np.ndarray, storage: Optional[str]) -> np.ndarray:
    """Round an intermediate to a storage type: None keeps fp64, "f32" and
    "bf16" round to nearest even."""
    if storage is None:
        return x
    if storage == "f32":
        return x.astype(np.float32).astype(np.float64)
    if storage == "bf16":
        from synthetic_inputs import round_bf16
        return round_bf16(x.astype(np.float32)).astype(np.float64)
    raise OracleError(f"unknown storage {storage!r}")


def divided(x, grid, order: Sequence[str], rope_split: Optional[Sequence[int]] = None,
            theta: float = 10000.0, storage: Optional[str] = None) -> np.ndarray:
    """Divided attention as a plain chain of passes over tokens x (B,N,heads,D).

    Each pass takes q = k = (RoPE(x) if a split is given, else x) and v = x,
    and its output is the next pass's x. ``order`` is e.g. ("temporal",
    "spatial") for the tiny DiT's time-then-space block, or ("spatial",
    "temporal") for the block-input path. ``storage`` optionally rounds each
    pass's output (and the rotated q/k) to the type the GPU path stores.
    """
    cur = _f64(x)
    for mode in order:
        qk = rope3d(cur, grid, rope_split, theta) if rope_split is not None else cur
        qk = store(qk, storage)
        cur = store(attention(qk, qk, cur, grid, mode), storage)
    return cur


def block_input(x_latent, w, grid, heads: int, head_dim: int, rope_split,
                order=("spatial", "temporal"), theta: float = 10000.0,
                storage: Optional[str] = None, bias=None) -> np.ndarray:
    """Latent -> patchify -> (RoPE on q, k) -> divided attention, as a chain."""
    tok = store(patchify(x_latent, w, bias), storage)
    B, N, dim = tok.shape
    if dim != heads * head_dim:
        raise OracleError("patchify width must equal heads * head_dim")
    return divided(tok.reshape(B, N, heads, head_dim), grid, order, rope_split, theta, storage)
