"""Pins of the fp64 oracle to things other than itself.

- Library routines that the oracle does not call: torch's CPU fp64
  scaled_dot_product_attention (with boolean block masks for the divided
  passes) and conv3d.
- Closed forms and invariants the mathematics fixes: constant values, zero
  queries, single-key sets, the peaky limit, joint key/value permutation,
  the RoPE angle law and its relative-offset property.
- The pages' own worked values: the token order of the attention probe
  (query 4082 at (2, 18, 26) of the 17-frame grid) and the RoPE split error.

Each case is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign, index or axis, a transposed operand) fails at least one of them.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


RNG = np.random.default_rng(12345)


def _grid_coords(T, Hp, Wp):
    """(t, h, w) of every token, from numpy's own C-order unravel."""
    t, h, w = np.unravel_index(np.arange(T * Hp * Wp), (T, Hp, Wp))
    return t, h, w


def _sdpa(q, k, v, mask=None, scale=None):
    """torch CPU fp64 SDPA on (B, N, heads, D) arrays; mask (N, N) True = attend."""
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def _qkv(B, N, H, D, std=1.0):
    return [RNG.standard_normal((B, N, H, D)) * std for _ in range(3)]


# ----------------------------------------------------------------------------
# Attention against the library routine
# ----------------------------------------------------------------------------

GRIDS = [(1, 1, 1), (2, 3, 5), (3, 4, 4), (4, 8, 8), (5, 3, 7)]


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("D", [32, 128])
def test_full_matches_sdpa(grid, D):
    T, Hp, Wp = grid
    N = T * Hp * Wp
    q, k, v = _qkv(2, N, 3, D)
    got = oracle.attention(q, k, v, grid, "full")
    np.testing.assert_allclose(got, _sdpa(q, k, v), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("grid", GRIDS)
def test_divided_passes_match_masked_sdpa(grid):
    T, Hp, Wp = grid
    N = T * Hp * Wp
    t, h, w = _grid_coords(T, Hp, Wp)
    same_frame = t[:, None] == t[None, :]
    same_pos = (h[:, None] == h[None, :]) & (w[:, None] == w[None, :])
    q, k, v = _qkv(2, N, 2, 64)
    np.testing.assert_allclose(oracle.attention(q, k, v, grid, "spatial"),
                               _sdpa(q, k, v, same_frame), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle.attention(q, k, v, grid, "temporal"),
                               _sdpa(q, k, v, same_pos), rtol=1e-12, atol=1e-13)


def test_explicit_scale_matches_sdpa():
    grid = (2, 3, 4)
    q, k, v = _qkv(1, 24, 2, 32)
    np.testing.assert_allclose(oracle.attention(q, k, v, grid, "full", scale=0.3),
                               _sdpa(q, k, v, scale=0.3), rtol=1e-12, atol=1e-13)


def test_row_sampling_matches_all_rows():
    grid = (3, 5, 6)
    N = 90
    q, k, v = _qkv(2, N, 2, 32)
    rows = np.array([0, 7, 31, 89], dtype=np.int64)
    for mode in ("full", "spatial", "temporal"):
        whole = oracle.attention(q, k, v, grid, mode)
        part = oracle.attention(q, k, v, grid, mode, rows=rows)
        np.testing.assert_array_equal(part, whole[:, rows])


# ----------------------------------------------------------------------------
# Closed forms and invariants
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["full", "spatial", "temporal"])
def test_constant_values(mode):
    grid = (3, 4, 5)
    q, k, _ = _qkv(1, 60, 2, 32)
    c = RNG.standard_normal((1, 1, 2, 32))
    v = np.broadcast_to(c, (1, 60, 2, 32)).copy()
    got = oracle.attention(q, k, v, grid, mode)
    np.testing.assert_allclose(got, v, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("mode", ["full", "spatial", "temporal"])
def test_zero_query_gives_mean_of_key_set(mode):
    grid = (3, 4, 5)
    T, Hp, Wp = grid
    _, k, v = _qkv(1, 60, 1, 32)
    q = np.zeros_like(k)
    got = oracle.attention(q, k, v, grid, mode)
    vv = v.reshape(T, Hp * Wp, 32)
    if mode == "full":
        want = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
    elif mode == "spatial":
        want = np.broadcast_to(vv.mean(axis=1, keepdims=True), vv.shape).reshape(v.shape)
    else:
        want = np.broadcast_to(vv.mean(axis=0, keepdims=True), vv.shape).reshape(v.shape)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_single_key_sets_return_v_exactly():
    # T = 1: the temporal key set of a token is the token itself.
    q, k, v = _qkv(2, 12, 2, 32)
    np.testing.assert_array_equal(oracle.attention(q, k, v, (1, 3, 4), "temporal"), v)
    # Hp = Wp = 1: the spatial key set is the token itself.
    q, k, v = _qkv(2, 5, 2, 32)
    np.testing.assert_array_equal(oracle.attention(q, k, v, (5, 1, 1), "spatial"), v)


def test_degenerate_axes_reduce_to_full():
    q, k, v = _qkv(1, 12, 2, 32)
    full = oracle.attention(q, k, v, (1, 3, 4), "full")
    np.testing.assert_array_equal(oracle.attention(q, k, v, (1, 3, 4), "spatial"), full)
    full = oracle.attention(q, k, v, (12, 1, 1), "full")
    np.testing.assert_array_equal(oracle.attention(q, k, v, (12, 1, 1), "temporal"), full)


def test_peaky_limit_is_argmax_value():
    # With a huge scale the softmax puts all mass on the largest logit; a
    # missing or wrong-signed max subtraction overflows instead.
    grid = (2, 3, 4)
    q, k, v = _qkv(1, 24, 2, 32)
    got = oracle.attention(q, k, v, grid, "full", scale=1e4)
    logits = np.einsum("bnhd,bmhd->bhnm", q, k)
    arg = logits.argmax(axis=-1)  # (b, h, n)
    want = np.empty_like(v)
    for h in range(2):
        want[0, :, h] = v[0, arg[0, h], h]
    np.testing.assert_array_equal(got, want)
    assert np.isfinite(got).all()


def test_joint_key_value_permutation():
    grid = (2, 4, 5)
    q, k, v = _qkv(1, 40, 2, 32)
    perm = RNG.permutation(40)
    a = oracle.attention(q, k, v, grid, "full")
    b = oracle.attention(q, k[:, perm], v[:, perm], grid, "full")
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_outputs_within_value_range():
    grid = (3, 4, 5)
    q, k, v = _qkv(1, 60, 2, 32, std=3.0)
    for mode in ("full", "spatial", "temporal"):
        o = oracle.attention(q, k, v, grid, mode)
        assert (o <= v.max(axis=1, keepdims=True) + 1e-12).all()
        assert (o >= v.min(axis=1, keepdims=True) - 1e-12).all()


def test_token_order_of_the_probe(page_values):
    # The 17-frame grid (5, 30, 52): a value equal to a token's own grid
    # coordinate is returned unchanged by every pass whose key set shares
    # that coordinate, and query 4082 sits at (t, h, w) = (2, 18, 26).
    T, Hp, Wp = 5, 30, 52
    N = T * Hp * Wp
    t, h, w = _grid_coords(T, Hp, Wp)
    q = RNG.standard_normal((1, N, 1, 8))
    k = RNG.standard_normal((1, N, 1, 8))
    v = np.zeros((1, N, 1, 8))
    v[0, :, 0, 0], v[0, :, 0, 1], v[0, :, 0, 2] = t, h, w
    probe = int(page_values["probe_token_index"][0])
    rows = np.array([0, probe, N - 1], dtype=np.int64)
    sp = oracle.attention(q, k, v, (T, Hp, Wp), "spatial", rows=rows)
    tm = oracle.attention(q, k, v, (T, Hp, Wp), "temporal", rows=rows)
    np.testing.assert_allclose(sp[0, :, 0, 0], t[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(tm[0, :, 0, 1], h[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(tm[0, :, 0, 2], w[rows], rtol=0, atol=1e-12)
    assert (t[probe], h[probe], w[probe]) == (2, 18, 26)


def test_divided_chain_order_and_degenerate_cases():
    grid = (3, 2, 2)
    x = RNG.standard_normal((1, 12, 2, 16))
    ts = oracle.divided(x, grid, ("temporal", "spatial"))
    st = oracle.divided(x, grid, ("spatial", "temporal"))
    assert np.abs(ts - st).max() > 1e-3  # the passes do not commute
    # T = 1: time-then-space is the spatial pass alone, which is full attention.
    x1 = RNG.standard_normal((1, 6, 2, 16))
    np.testing.assert_allclose(oracle.divided(x1, (1, 2, 3), ("temporal", "spatial")),
                               _sdpa(x1, x1, x1), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# Patchify
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape,patch", [((1, 4, 8, 16, 16), (2, 2, 2)),
                                         ((2, 3, 5, 6, 10), (1, 2, 2)),
                                         ((1, 2, 5, 7, 9), (2, 3, 2))])
def test_patchify_matches_conv3d(shape, patch):
    B, C, Tl, Hl, Wl = shape
    x = RNG.standard_normal(shape)
    w = RNG.standard_normal((24, C) + patch) * 0.02
    b = RNG.standard_normal(24)
    got = oracle.patchify(x, w, b)
    ref = F.conv3d(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b), stride=patch)
    ref = ref.flatten(2).transpose(1, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_patchify_one_hot():
    C, pt, ph, pw = 3, 2, 2, 3
    T, Hp, Wp = 2, 3, 2
    w = RNG.standard_normal((10, C, pt, ph, pw))
    for (c, t, h, ww, i, j, kk) in [(0, 0, 0, 0, 0, 0, 0), (2, 1, 2, 1, 1, 1, 2), (1, 0, 1, 1, 1, 0, 1)]:
        x = np.zeros((1, C, T * pt, Hp * ph, Wp * pw))
        x[0, c, t * pt + i, h * ph + j, ww * pw + kk] = 1.0
        tok = oracle.patchify(x, w)
        n = (t * Hp + h) * Wp + ww
        np.testing.assert_array_equal(tok[0, n], w[:, c, i, j, kk])
        others = np.delete(tok[0], n, axis=0)
        assert not others.any()


def test_patchify_drops_remainder():
    x = RNG.standard_normal((1, 2, 5, 7, 9))
    w = RNG.standard_normal((6, 2, 2, 2, 2))
    np.testing.assert_array_equal(oracle.patchify(x, w), oracle.patchify(x[:, :, :4, :6, :8], w))


# ----------------------------------------------------------------------------
# 3D RoPE
# ----------------------------------------------------------------------------

SPLIT = (44, 42, 42)
THETA = 10000.0


def test_rope_identity_at_origin():
    x = RNG.standard_normal((2, 1, 3, 128))
    np.testing.assert_array_equal(oracle.rope3d(x, (1, 1, 1), SPLIT), x)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_rope_angle_law(axis):
    # Put e_{2j} into every pair of every segment; the rotated pair is
    # (cos phi, sin phi) with phi = p_axis * f_{axis, j}. The law the pages fix:
    # f_{a,0} = 1, f_{a,j+1} / f_{a,j} = theta^(-2/d_a), and phi linear in p.
    grid = (5, 6, 7)
    T, Hp, Wp = grid
    t, h, w = _grid_coords(*grid)
    pos = (t, h, w)[axis]
    x = np.zeros((1, T * Hp * Wp, 1, 128))
    x[..., 0::2] = 1.0
    y = oracle.rope3d(x, grid, SPLIT)
    start = sum(SPLIT[:axis])
    d_a = SPLIT[axis]
    seg = y[0, :, 0, start:start + d_a]
    c, s = seg[:, 0::2], seg[:, 1::2]
    np.testing.assert_allclose(c * c + s * s, 1.0, rtol=0, atol=1e-14)
    # At position 1 on this axis every angle is < pi and atan2 recovers it.
    n1 = np.where(pos == 1)[0][0]
    f = np.arctan2(s[n1], c[n1])
    np.testing.assert_allclose(f[0], 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(f[1:] / f[:-1], THETA ** (-2.0 / d_a), rtol=1e-12)
    assert f.size == d_a // 2
    # Linear in position: angle at p equals p * angle at 1 (mod 2 pi).
    for n in range(0, T * Hp * Wp, 17):
        p = pos[n]
        np.testing.assert_allclose(c[n], np.cos(p * f), rtol=0, atol=1e-12)
        np.testing.assert_allclose(s[n], np.sin(p * f), rtol=0, atol=1e-12)
    # Tokens at position 0 on this axis leave this segment untouched.
    z = np.where(pos == 0)[0]
    np.testing.assert_array_equal(seg[z], x[0, z, 0, start:start + d_a])


def test_rope_relative_offset_property():
    # The pages' demonstration: (t,h,w) pairs (1,10,20)->(3,12,25) and
    # (2,15,30)->(4,17,35) share the offset (2,2,5) and give the same q.k.
    grid = (5, 18, 37)
    T, Hp, Wp = grid
    N = T * Hp * Wp
    qb = RNG.standard_normal(128)
    kb = RNG.standard_normal(128)
    x = np.broadcast_to(qb, (1, N, 1, 128)).copy()
    xk = np.broadcast_to(kb, (1, N, 1, 128)).copy()
    rq = oracle.rope3d(x, grid, SPLIT)[0, :, 0]
    rk = oracle.rope3d(xk, grid, SPLIT)[0, :, 0]
    idx = lambda t, h, w: (t * Hp + h) * Wp + w  # noqa: E731
    a = rq[idx(1, 10, 20)] @ rk[idx(3, 12, 25)]
    b = rq[idx(2, 15, 30)] @ rk[idx(4, 17, 35)]
    assert abs(a - b) < 1e-12
    c = rq[idx(2, 15, 30)] @ rk[idx(4, 17, 36)]  # a different offset differs
    assert abs(a - c) > 1e-6


def test_rope_preserves_pair_norms():
    grid = (3, 4, 5)
    x = RNG.standard_normal((2, 60, 3, 128))
    y = oracle.rope3d(x, grid, SPLIT)
    np.testing.assert_allclose(y[..., 0::2] ** 2 + y[..., 1::2] ** 2,
                               x[..., 0::2] ** 2 + x[..., 1::2] ** 2, rtol=1e-13)


@pytest.mark.parametrize("split", [(44, 42, 40), (44, 44, 42), (43, 43, 42), (0, 64, 62)])
def test_rope_bad_split_raises(split):
    x = RNG.standard_normal((1, 6, 1, 128))
    if sum(split) == 128 and all(s % 2 == 0 for s in split):
        oracle.rope3d(x, (1, 2, 3), split)  # a legal split with an empty axis
        return
    with pytest.raises(oracle.RopeSplitError):
        oracle.rope3d(x, (1, 2, 3), split)


# ----------------------------------------------------------------------------
# Cross-attention (video queries against text keys)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("Nq,Nk,D", [(7, 5, 32), (40, 64, 128), (33, 1, 64)])
def test_cross_matches_sdpa(Nq, Nk, D):
    q = RNG.standard_normal((2, Nq, 3, D))
    k = RNG.standard_normal((2, Nk, 3, D))
    v = RNG.standard_normal((2, Nk, 3, D))
    np.testing.assert_allclose(oracle.cross_attention(q, k, v), _sdpa(q, k, v), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle.cross_attention(q, k, v, scale=0.7), _sdpa(q, k, v, scale=0.7),
                               rtol=1e-12, atol=1e-13)


def test_cross_closed_forms():
    q = RNG.standard_normal((1, 9, 2, 16))
    k = RNG.standard_normal((1, 6, 2, 16))
    v = RNG.standard_normal((1, 6, 2, 16))
    # One key: every query returns it exactly.
    np.testing.assert_array_equal(oracle.cross_attention(q, k[:, :1], v[:, :1]),
                                  np.broadcast_to(v[:, :1], q.shape))
    # Zero queries: the mean of the values.
    np.testing.assert_allclose(oracle.cross_attention(np.zeros_like(q), k, v),
                               np.broadcast_to(v.mean(axis=1, keepdims=True), q.shape), rtol=1e-12, atol=1e-14)
    # Same keys as the queries' own token set: cross equals full attention.
    x = RNG.standard_normal((1, 12, 2, 16))
    np.testing.assert_allclose(oracle.cross_attention(x, x, x), oracle.attention(x, x, x, (1, 3, 4), "full"),
                               rtol=1e-13, atol=1e-14)
    rows = np.array([0, 5, 8], dtype=np.int64)
    np.testing.assert_array_equal(oracle.cross_attention(q, k, v, rows=rows), oracle.cross_attention(q, k, v)[:, rows])


# ----------------------------------------------------------------------------
# Windowed spacetime attention
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("grid,window", [((4, 6, 7), (2, 3, 3)), ((5, 4, 9), (3, 4, 2)), ((3, 5, 5), (1, 2, 5)),
                                         ((2, 3, 4), (5, 5, 5))])
def test_window_matches_masked_sdpa(grid, window):
    T, Hp, Wp = grid
    wt, wh, ww = window
    N = T * Hp * Wp
    t, h, w = _grid_coords(T, Hp, Wp)
    same = ((t[:, None] // wt == t[None, :] // wt) & (h[:, None] // wh == h[None, :] // wh)
            & (w[:, None] // ww == w[None, :] // ww))
    q, k, v = _qkv(2, N, 2, 32)
    np.testing.assert_allclose(oracle.window_attention(q, k, v, grid, window), _sdpa(q, k, v, same),
                               rtol=1e-12, atol=1e-13)


def test_window_special_cases():
    grid = (3, 4, 5)
    T, Hp, Wp = grid
    q, k, v = _qkv(1, 60, 2, 32)
    np.testing.assert_allclose(oracle.window_attention(q, k, v, grid, (1, Hp, Wp)),
                               oracle.attention(q, k, v, grid, "spatial"), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.window_attention(q, k, v, grid, (T, 1, 1)),
                               oracle.attention(q, k, v, grid, "temporal"), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.window_attention(q, k, v, grid, (T, Hp, Wp)),
                               oracle.attention(q, k, v, grid, "full"), rtol=1e-13, atol=1e-15)
    # 1x1x1 windows: each token attends to itself only.
    np.testing.assert_array_equal(oracle.window_attention(q, k, v, grid, (1, 1, 1)), v)
    rows = np.array([0, 17, 59], dtype=np.int64)
    np.testing.assert_array_equal(oracle.window_attention(q, k, v, grid, (2, 3, 2), rows=rows),
                                  oracle.window_attention(q, k, v, grid, (2, 3, 2))[:, rows])


# ----------------------------------------------------------------------------
# QKV projection with Q/K RMSNorm and RoPE
# ----------------------------------------------------------------------------

def test_rope_rows_match_grid_rope():
    grid = (3, 4, 5)
    x = RNG.standard_normal((2, 60, 2, 32))
    rows = np.array([0, 7, 23, 59], dtype=np.int64)
    full = oracle.rope3d(x, grid, (12, 10, 10))
    np.testing.assert_array_equal(oracle.rope3d_rows(x[:, rows], grid, rows, (12, 10, 10)), full[:, rows])


def test_rmsnorm_matches_torch_and_closed_forms():
    x = RNG.standard_normal((3, 5, 128))
    g = RNG.standard_normal(128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(x, g, 1e-6), ref, rtol=1e-12, atol=1e-13)
    # Unit gain, eps = 0: the mean square of every output row is exactly 1,
    # and scaling the input by a positive factor changes nothing.
    y = oracle.rmsnorm(x, np.ones(128), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * x, np.ones(128), 0.0), y, rtol=1e-13)
    # A constant row c: every output is sign(c) * |c| / sqrt(c^2 + eps) * gain.
    c, eps = -0.3, 1e-2
    np.testing.assert_allclose(oracle.rmsnorm(np.full((1, 8), c), np.arange(1, 9), eps),
                               [np.arange(1, 9) * c / np.sqrt(c * c + eps)], rtol=1e-14)


def test_qkv_proj_matches_torch_linear():
    grid, heads, D = (2, 3, 4), 2, 32
    dim = heads * D
    x = RNG.standard_normal((2, 24, dim))
    w = 0.02 * RNG.standard_normal((3 * dim, dim))
    b = 0.1 * RNG.standard_normal(3 * dim)
    q, k, v = oracle.qkv_proj(x, w, b, None, None, grid, heads, D)
    lin = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b)).numpy()
    got = np.concatenate([t.reshape(2, 24, dim) for t in (q, k, v)], axis=-1)
    np.testing.assert_allclose(got, lin, rtol=1e-12, atol=1e-14)


def test_qkv_proj_composition():
    # Identity blocks: q and k are the normalised (and rotated) tokens, v the
    # tokens themselves; sampled rows equal the same rows of the whole output.
    grid, heads, D = (2, 3, 5), 2, 32
    dim = heads * D
    x = RNG.standard_normal((1, 30, dim))
    w = np.concatenate([np.eye(dim)] * 3)
    gq, gk = RNG.standard_normal(dim), RNG.standard_normal(dim)
    split = (12, 10, 10)
    q, k, v = oracle.qkv_proj(x, w, None, gq, gk, grid, heads, D, split, eps=1e-6)
    xh = x.reshape(1, 30, heads, D)
    np.testing.assert_array_equal(v, xh)
    np.testing.assert_allclose(q, oracle.rope3d(oracle.rmsnorm(xh, gq.reshape(heads, D), 1e-6), grid, split),
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(k, oracle.rope3d(oracle.rmsnorm(xh, gk.reshape(heads, D), 1e-6), grid, split),
                               rtol=1e-13, atol=1e-14)
    rows = np.array([1, 17, 29], dtype=np.int64)
    for a, b_ in zip(oracle.qkv_proj(x, w, None, gq, gk, grid, heads, D, split, rows=rows), (q, k, v)):
        np.testing.assert_allclose(a, b_[:, rows], rtol=1e-14, atol=1e-15)
    # Per-head normalisation: each head of q has mean square 1 before the
    # rotation (unit gain, eps = 0), and the rotation keeps every pair's norm.
    q1, _, _ = oracle.qkv_proj(x, w, None, np.ones(dim), np.ones(dim), grid, heads, D, split, eps=0.0)
    np.testing.assert_allclose(np.mean(q1 * q1, axis=-1), 1.0, rtol=1e-12)
