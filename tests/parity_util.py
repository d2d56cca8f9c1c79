"""Helpers for GPU-vs-oracle parity: device upload of the seeded inputs and
the tolerance the comparisons use.

Tolerance (fixed for the bf16 path as max-abs 2e-2 together with mean
relative error 5e-3, and 1e-5 for fp32): over all compared elements,
  max |g - r| <= atol  and  sum |g - r| / sum |r| <= rel_l1,
with (atol, rel_l1) = (2e-2, 5e-3) for bf16 and (1e-5, 1e-5) for fp32. A
per-element relative error is not used: near-zero references make it
meaningless.
"""

from __future__ import annotations

import numpy as np
import torch

from synthetic_inputs import Drawn

TOL = {"bf16": (2e-2, 5e-3), "f32": (1e-5, 1e-5)}


def to_dev(d: Drawn) -> torch.Tensor:
    if d.bits is not None:
        return torch.from_numpy(np.ascontiguousarray(d.bits).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(d.f32)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def stats(g: np.ndarray, r: np.ndarray):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    diff = np.abs(g - r)
    return float(diff.max()), float(diff.sum() / max(np.abs(r).sum(), 1e-300))


def assert_close(g, r, dtype: str, what: str = ""):
    atol, rel = TOL[dtype]
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    mx, rl = stats(g, r)
    print(f"[parity] {what}: max_abs={mx:.3e} rel_l1={rl:.3e} (tol {atol:g}, {rel:g})", flush=True)
    assert mx <= atol and rl <= rel, f"{what}: max_abs={mx:.3e} rel_l1={rl:.3e} exceed ({atol}, {rel})"
    return mx, rl


def space_then_time_at_positions(x, grid, split, positions, storage=None, theta=10000.0):
    """The oracle's spatial-then-temporal chain (q = k = RoPE(x), v = x per
    pass, stored intermediates rounded to ``storage``), evaluated only on the
    token rows of the given patch positions in every frame.

    The temporal output at a position needs only the spatial outputs at that
    same position in every frame (its key set), so the chain restricted to
    rows = {t*HW + p : all t, p in positions} is exact on those rows. Returns
    (rows, spatial output at rows, chain output at rows). A CPU test checks
    this against ``oracle.divided`` on small grids.
    """
    import oracle

    x = np.asarray(x, dtype=np.float64)
    T, Hp, Wp = grid
    HW = Hp * Wp
    positions = np.asarray(positions, dtype=np.int64)
    rows = (np.arange(T, dtype=np.int64)[:, None] * HW + positions[None, :]).reshape(-1)
    r0 = oracle.store(oracle.rope3d(x, grid, split, theta), storage)
    x1_rows = oracle.store(oracle.attention(r0, r0, x, grid, "spatial", rows=rows), storage)
    r1_rows = oracle.store(oracle.rope3d_rows(x1_rows, grid, rows, split, theta), storage)
    x1_full = np.zeros_like(x)
    r1_full = np.zeros_like(x)
    x1_full[:, rows] = x1_rows
    r1_full[:, rows] = r1_rows
    x2_rows = oracle.store(oracle.attention(r1_full, r1_full, x1_full, grid, "temporal", rows=rows), storage)
    return rows, x1_rows, x2_rows
