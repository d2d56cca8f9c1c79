"""Pins of the oracle's divided chain (``oracle.divided``, ``oracle.block_input``)
to a brute force that uses neither of them nor any other oracle routine.

The chain is the "time then space" block of the "Video and 3D Generation"
cheatsheet ("Tiny video DiT"; "Functions in the lessons": the divided
attention block) and the block-input order of the 480p block-input workload
(spatial, then temporal). Each pass attends with q = k = RoPE(x) (or x with no
split) and v = x, the order "How AI Generates Video ..." section 5 gives for
attn1 (rotate Q and K, then attend).

The brute force here:
- attends with torch's CPU fp64 ``scaled_dot_product_attention`` under boolean
  block masks (same frame for the spatial pass, same patch position for the
  temporal pass), built from numpy's own C-order unravel of the token index;
- rotates with complex arithmetic: each interleaved feature pair (2j, 2j+1) is
  one complex number, multiplied by exp(i * position * theta^(-2j/d_a)) for
  the axis segment it falls in ("How AI Generates Video ...", section 4: the
  [44, 42, 42] split viewed as 22, 21 and 21 complex pairs);
- patchifies with torch's fp64 ``conv3d`` (stride = kernel);
- rounds stored intermediates to bf16 with torch's own float64 -> bfloat16
  conversion (round to nearest even), independent of the host rounding in
  ``synthetic_inputs``.

The last test plants three mistakes in a chain assembled from the oracle's
parts (order reversed, v taken from the rotated tensor, no rotation on the
second pass) and checks that the brute force tells each of them apart from
the correct chain by far more than the pins' tolerance.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(2024)
# Token values of standard deviation 0.5: with q = k = x a token's score with
# itself is then about 0.25 * sqrt(D) (1.4 at D = 32, 2.8 at D = 128), so
# every pass mixes many tokens while the rotation still moves the scores.
# At standard deviation 1 the self-score dominates and each pass is close to
# the identity (a chain in the wrong order then differs by only ~5e-4); at
# 0.2 the scores are so small that dropping a rotation moves the output by
# only ~4e-5.
STD = 0.5


def _coords(grid):
    T, Hp, Wp = grid
    return np.unravel_index(np.arange(T * Hp * Wp), (T, Hp, Wp))


def _masks(grid):
    t, h, w = _coords(grid)
    same_frame = t[:, None] == t[None, :]
    same_pos = (h[:, None] == h[None, :]) & (w[:, None] == w[None, :])
    return {"spatial": torch.from_numpy(same_frame), "temporal": torch.from_numpy(same_pos),
            "full": None}


def _rotate(x: torch.Tensor, grid, split, theta: float) -> torch.Tensor:
    """x (B, N, heads, D) fp64 -> each pair turned by its axis angle (complex form)."""
    B, N, H, D = x.shape
    pos = [torch.from_numpy(c.astype(np.float64)) for c in _coords(grid)]  # t, h, w per token
    angles = []
    for axis, width in enumerate(split):
        j = torch.arange(width // 2, dtype=torch.float64)
        freq = torch.pow(torch.tensor(float(theta), dtype=torch.float64), -2.0 * j / width)
        angles.append(pos[axis][:, None] * freq[None, :])  # (N, width/2)
    ang = torch.cat(angles, dim=1)  # (N, D/2)
    turn = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]
    xc = torch.view_as_complex(x.reshape(B, N, H, D // 2, 2).contiguous())
    return torch.view_as_real(xc * turn).reshape(B, N, H, D)


def _attend(qk: torch.Tensor, v: torch.Tensor, mask) -> torch.Tensor:
    o = F.scaled_dot_product_attention(qk.permute(0, 2, 1, 3), qk.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3),
                                       attn_mask=mask)
    return o.permute(0, 2, 1, 3).contiguous()


def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16).to(torch.float64)


def brute_chain(x: np.ndarray, grid, order, split=None, theta=10000.0, bf16_store=False) -> np.ndarray:
    masks = _masks(grid)
    cur = torch.from_numpy(np.asarray(x, dtype=np.float64))
    for mode in order:
        qk = _rotate(cur, grid, split, theta) if split is not None else cur
        if bf16_store:
            qk = _bf16(qk)
        cur = _attend(qk, cur, masks[mode])
        if bf16_store:
            cur = _bf16(cur)
    return cur.numpy()


ORDERS = [("temporal", "spatial"), ("spatial", "temporal")]


@pytest.mark.parametrize("order", ORDERS)
def test_tiny_dit_chain_matches_brute_force(order):
    # The tiny video DiT's shape: grid (4, 8, 8), 2 heads x 32.
    grid = (4, 8, 8)
    x = RNG.standard_normal((1, 256, 2, 32)) * STD
    np.testing.assert_allclose(oracle.divided(x, grid, order), brute_chain(x, grid, order),
                               rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("order", ORDERS)
@pytest.mark.parametrize("grid,heads,D,split", [((4, 8, 8), 2, 32, (12, 10, 10)),
                                                ((3, 4, 5), 2, 128, (44, 42, 42)),
                                                ((5, 3, 7), 1, 128, (64, 32, 32))])
def test_chain_with_rope_matches_brute_force(order, grid, heads, D, split):
    N = grid[0] * grid[1] * grid[2]
    x = RNG.standard_normal((2, N, heads, D)) * STD
    np.testing.assert_allclose(oracle.divided(x, grid, order, rope_split=split),
                               brute_chain(x, grid, order, split), rtol=1e-11, atol=1e-12)


def test_chain_theta_reaches_the_rotation():
    grid, split, order = (3, 4, 5), (44, 42, 42), ("spatial", "temporal")
    x = RNG.standard_normal((1, 60, 2, 128)) * STD
    np.testing.assert_allclose(oracle.divided(x, grid, order, rope_split=split, theta=500.0),
                               brute_chain(x, grid, order, split, theta=500.0), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("order", ORDERS)
def test_chain_bf16_storage_matches_brute_force(order):
    # Values drawn as bf16 (as the GPU path consumes them); the oracle rounds
    # the rotated q/k and each pass's output to bf16, the brute force with
    # torch's conversion. Rounding decisions that fall on a tie are a
    # measure-zero event for these random inputs, so the two agree to fp64
    # rounding; a mismatch of one bf16 step would show as ~4e-3.
    grid, split = (3, 5, 6), (44, 42, 42)
    x = _bf16(torch.from_numpy(RNG.standard_normal((1, 90, 2, 128)) * STD)).numpy()
    got = oracle.divided(x, grid, order, rope_split=split, storage="bf16")
    ref = brute_chain(x, grid, order, split, bf16_store=True)
    assert np.abs(got - ref).max() <= 1e-6
    # The rounding is really applied: without it the chain moves by much more.
    loose = brute_chain(x, grid, order, split)
    assert np.abs(loose - ref).max() > 1e-4


def test_block_input_matches_brute_force():
    # Latent (1, 4, 6, 8, 10) through 1x2x2 bricks to a (6, 4, 5) grid of
    # width 64 = 2 heads x 32, then RoPE [12, 10, 10] and spatial -> temporal.
    lat = RNG.standard_normal((1, 4, 6, 8, 10)) * 10.0
    w = RNG.standard_normal((64, 4, 1, 2, 2)) * 0.02
    b = RNG.standard_normal(64) * 0.02
    grid, split = (6, 4, 5), (12, 10, 10)
    got = oracle.block_input(lat, w, grid, 2, 32, split, bias=b)
    tok = F.conv3d(torch.from_numpy(lat), torch.from_numpy(w), torch.from_numpy(b), stride=(1, 2, 2))
    tok = tok.flatten(2).transpose(1, 2).reshape(1, 120, 2, 32).numpy()
    ref = brute_chain(tok, grid, ("spatial", "temporal"), split)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_brute_force_rejects_planted_chain_mistakes():
    grid, split, order = (3, 4, 5), (44, 42, 42), ("spatial", "temporal")
    x = RNG.standard_normal((1, 60, 2, 128)) * STD
    ref = brute_chain(x, grid, order, split)

    def chain(order_, v_rotated=False, rotate_second=True):
        cur = x
        for i, mode in enumerate(order_):
            qk = oracle.rope3d(cur, grid, split) if (i == 0 or rotate_second) else cur
            cur = oracle.attention(qk, qk, qk if v_rotated else cur, grid, mode)
        return cur

    np.testing.assert_allclose(chain(order), ref, rtol=1e-11, atol=1e-12)
    # Each mistake moves the output by at least 1e-3 (measured: 1e-2 to 1.3),
    # eight orders of magnitude past the 1e-11 the pins above allow.
    for name, bad in (("order reversed", chain(order[::-1])),
                      ("v = RoPE(x)", chain(order, v_rotated=True)),
                      ("no RoPE on the second pass", chain(order, rotate_second=False))):
        assert np.abs(bad - ref).max() > 1e-3, name


@pytest.mark.parametrize("storage", [None, "bf16"])
def test_row_restricted_chain_equals_divided(storage):
    # The full-size GPU test of the block-input chain evaluates the oracle's
    # chain only at a few patch positions; on a small grid that restriction
    # equals the whole chain at those rows.
    from tests.parity_util import space_then_time_at_positions
    grid, split = (4, 5, 6), (44, 42, 42)
    x = RNG.standard_normal((1, 120, 2, 128)) * STD
    if storage == "bf16":
        x = _bf16(torch.from_numpy(x)).numpy()
    rows, x1, x2 = space_then_time_at_positions(x, grid, split, [0, 7, 29], storage)
    whole = oracle.divided(x, grid, ("spatial", "temporal"), rope_split=split, storage=storage)
    first = oracle.divided(x, grid, ("spatial",), rope_split=split, storage=storage)
    np.testing.assert_allclose(x2, whole[:, rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(x1, first[:, rows], rtol=1e-12, atol=1e-14)
