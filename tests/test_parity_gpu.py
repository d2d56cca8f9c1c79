"""GPU parity: every HIP entry point against the fp64 oracle, through the C ABI.

Small shapes are compared element by element over whole outputs; they span
several key tiles and query blocks and end in ragged tails. The full-size
workloads (480p full, 480p divided, 720p full, block input) run in the same
launch configuration as the benchmark and are compared on sampled query rows
(every row of a sampled query costs the oracle 4*N*head_dim FLOP), or in full
where the oracle is cheap (temporal pass, patchify, RoPE).
"""

import numpy as np
import pytest
import torch

import oracle
import spacetime_attention_amd as vd
from synthetic_inputs import (CROSS_WORKLOADS, QKV_WORKLOADS, WORKLOADS, CrossWorkload, QkvWorkload, bf16_bits,
                              bf16_to_f32, draw, round_bf16, sample_rows, small_grid)
from tests.parity_util import assert_close, space_then_time_at_positions, stats, to_dev, to_host

pytestmark = pytest.mark.gpu

PASSES = {"full": vd.attn_full, "spatial": vd.attn_spatial, "temporal": vd.attn_temporal}


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _qkv(w, q_scale=1.0):
    d = w.draw_qkv(q_scale)
    return d, [to_dev(d[n]) for n in ("q", "k", "v")]


# ----------------------------------------------------------------------------
# Small shapes, whole outputs
# ----------------------------------------------------------------------------

SMALL = [
    # (name, B, grid, heads, D)
    ("ragged_231", 2, (3, 7, 11), 2, 128),
    ("ragged_d64", 1, (5, 6, 9), 3, 64),
    ("multi_tile_1000", 1, (4, 10, 25), 2, 128),
    ("single_frame", 1, (1, 9, 15), 2, 128),
    ("long_time_40", 1, (40, 2, 3), 2, 128),
    ("one_token_frames", 2, (7, 1, 1), 2, 128),
    # 100 tokens: only the first four 32-query wavefronts of an 8-wave
    # workgroup have queries, so one group of the full pass's two phase
    # groups runs alone; 2 key tiles.
    ("first_group_only_100", 1, (4, 5, 5), 2, 128),
    # 620 tokens: three query blocks (256, 256, 108), 10 key tiles.
    ("three_blocks_620", 2, (5, 4, 31), 2, 128),
    # head_dim 64 over several key tiles: 250-token frames (4 tiles, the
    # last with 58 keys, so its second 32-key block is ragged).
    ("multi_tile_d64", 1, (3, 10, 25), 2, 64),
    # head_dim 32 (16 rows per 1 KB tile load; the full pass on the 4-wave
    # tile): ragged tiles, several key tiles, two clips with three query
    # blocks, and the temporal kernel's 32-row slices (T = 7, 30, 33, 40).
    ("ragged_d32", 2, (3, 7, 11), 2, 32),
    ("multi_tile_d32", 1, (3, 10, 25), 2, 32),
    ("two_clips_d32", 2, (5, 4, 31), 2, 32),
    ("time_30_d32", 1, (30, 2, 3), 2, 32),
    ("time_33_d32", 1, (33, 2, 3), 2, 32),
    ("long_time_40_d32", 1, (40, 2, 3), 3, 32),
]


@pytest.mark.parametrize("mode", ["full", "spatial", "temporal"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_bf16(case, mode):
    name, B, grid, heads, D = case
    _announce(f"small bf16 {name} {mode} B={B} grid={grid} heads={heads} D={D}")
    w = small_grid(name, B, *grid, heads, D, "bf16", seed=100 + len(name))
    d, (q, k, v) = _qkv(w)
    got = to_host(PASSES[mode](q, k, v, grid))
    torch.cuda.synchronize()
    ref = oracle.attention(d["q"].f32, d["k"].f32, d["v"].f32, grid, mode)
    assert_close(got, ref, "bf16", f"{name}/{mode}")


@pytest.mark.parametrize("mode", ["full", "spatial", "temporal"])
def test_peaky_bf16(mode):
    # Q and K with standard deviation 4: logits of standard deviation 16,
    # which exercises the running-maximum updates.
    grid = (3, 8, 13)
    _announce(f"peaky bf16 {mode} grid={grid}")
    w = small_grid("peaky", 1, *grid, 2, 128, "bf16", seed=7)
    d, (q, k, v) = _qkv(w, q_scale=4.0)
    got = to_host(PASSES[mode](q, k, v, grid))
    ref = oracle.attention(d["q"].f32, d["k"].f32, d["v"].f32, grid, mode)
    assert_close(got, ref, "bf16", f"peaky/{mode}")


@pytest.mark.parametrize("mode", ["full", "spatial"])
def test_rising_logits_bf16(mode):
    # Key norms ramp up 30x along the token order, so the largest score keeps
    # growing from one key tile to the next by far more than the kernel lets
    # its reference maximum lag: the reference is raised on many tiles.
    grid = (4, 10, 25)
    _announce(f"rising logits bf16 {mode} grid={grid}")
    w = small_grid("rising", 1, *grid, 2, 128, "bf16", seed=17)
    d = w.draw_qkv()
    ramp = (1.0 + 30.0 * np.arange(w.N, dtype=np.float32) / w.N)[None, :, None, None]
    kb = bf16_bits(d["k"].f32 * ramp)
    k_f32 = bf16_to_f32(kb).reshape(d["k"].f32.shape)
    q = to_dev(d["q"])
    k = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).cuda()
    v = to_dev(d["v"])
    got = to_host(PASSES[mode](q, k, v, grid))
    ref = oracle.attention(d["q"].f32, k_f32, d["v"].f32, grid, mode)
    assert_close(got, ref, "bf16", f"rising/{mode}")


def test_single_key_sets_are_exact():
    # T = 1: the temporal key set is the query itself; Hp = Wp = 1: so is the
    # spatial one. The softmax weight is exactly 1 and the output is V bit for bit.
    _announce("single-key sets")
    w = small_grid("t1", 2, 1, 5, 13, 2, 128, "bf16", seed=3)
    d, (q, k, v) = _qkv(w)
    assert torch.equal(vd.attn_temporal(q, k, v, (1, 5, 13)), v)
    w = small_grid("hw1", 2, 9, 1, 1, 2, 128, "bf16", seed=4)
    d, (q, k, v) = _qkv(w)
    assert torch.equal(vd.attn_spatial(q, k, v, (9, 1, 1)), v)


@pytest.mark.parametrize("mode", ["full", "spatial", "temporal"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_small_f32(mode, D):
    grid = (3, 5, 7)
    _announce(f"small f32 {mode} D={D}")
    w = small_grid("f32", 2, *grid, 2, D, "f32", seed=11)
    d, (q, k, v) = _qkv(w)
    got = to_host(PASSES[mode](q, k, v, grid))
    ref = oracle.attention(d["q"].f32, d["k"].f32, d["v"].f32, grid, mode)
    assert_close(got, ref, "f32", f"f32/{mode}/D{D}")


def test_deterministic_and_in_bounds():
    # Two runs agree bit for bit (no LDS race), and guard bands around the
    # output stay untouched (no stray writes).
    grid = (3, 7, 11)
    _announce("determinism and guard bands")
    w = small_grid("guard", 1, *grid, 2, 128, "bf16", seed=21)
    d, (q, k, v) = _qkv(w)
    n = q.numel()
    for fn in PASSES.values():
        buf = torch.full((n + 2 * 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
        out = buf[4096:4096 + n].view_as(q)
        fn(q, k, v, grid, out=out)
        again = fn(q, k, v, grid)
        torch.cuda.synchronize()
        assert torch.equal(out, again)
        assert bool((buf[:4096] == 7.0).all()) and bool((buf[4096 + n:] == 7.0).all())


# ----------------------------------------------------------------------------
# Tiny video DiT (fp32): patchify, each pass, and time-then-space
# ----------------------------------------------------------------------------

def test_tiny_dit_f32():
    w = WORKLOADS["tiny"]
    _announce("tiny video DiT fp32")
    d = w.draw_latent()
    x, wt = to_dev(d["x"]), to_dev(d["w"])
    grid = (w.T, w.Hp, w.Wp)
    tok = vd.patchify(x, wt, heads=w.heads, head_dim=w.head_dim)
    ref_tok = oracle.patchify(d["x"].f32, d["w"].f32)
    assert tuple(tok.shape) == (1, 256, 64)
    assert_close(to_host(tok), ref_tok, "f32", "tiny/patchify")
    # Time then space, q = k = v = tokens split into 2 heads of 32.
    xs = tok.view(1, 256, 2, 32)
    got = to_host(vd.divided(xs, grid, order=("temporal", "spatial")))
    ref = oracle.divided(ref_tok.reshape(1, 256, 2, 32), grid, ("temporal", "spatial"))
    assert_close(got, ref, "f32", "tiny/time-then-space")
    for mode, fn in PASSES.items():
        assert_close(to_host(fn(xs, xs, xs, grid)), oracle.attention(ref_tok.reshape(1, 256, 2, 32),
                     ref_tok.reshape(1, 256, 2, 32), ref_tok.reshape(1, 256, 2, 32), grid, mode),
                     "f32", f"tiny/{mode}")


# ----------------------------------------------------------------------------
# RoPE and patchify, small and ragged
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_small(dtype):
    grid = (5, 7, 9)
    _announce(f"rope small {dtype}")
    x = draw(31, [("x", (2, 315, 3, 128), 1.0)], dtype)["x"]
    xd = to_dev(x)
    got = to_host(vd.rope3d(xd, grid, (44, 42, 42)))
    ref = oracle.rope3d(x.f32, grid, (44, 42, 42))
    assert_close(got, ref, dtype, f"rope/{dtype}")
    # In place gives the same result.
    vd.rope3d(xd, grid, (44, 42, 42), out=xd)
    assert_close(to_host(xd), ref, dtype, f"rope-inplace/{dtype}")


def test_rope_other_split():
    grid = (3, 4, 6)
    _announce("rope split 12/10/10 at head_dim 32 (fp32)")
    x = draw(32, [("x", (1, 72, 2, 32), 1.0)], "f32")["x"]
    got = to_host(vd.rope3d(to_dev(x), grid, (12, 10, 10)))
    assert_close(got, oracle.rope3d(x.f32, grid, (12, 10, 10)), "f32", "rope/12-10-10")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_patchify_small(dtype):
    _announce(f"patchify small {dtype}")
    d = draw(41, [("x", (2, 3, 5, 9, 13), 1.0), ("w", (64, 3, 2, 2, 3), 0.02), ("b", (64,), 0.1)], dtype)
    x, wt, b = (to_dev(d[n]) for n in ("x", "w", "b"))
    got = to_host(vd.patchify(x, wt, b, heads=2, head_dim=32))
    ref = oracle.patchify(d["x"].f32, d["w"].f32, d["b"].f32)
    assert got.shape == ref.shape == (2, 2 * 4 * 4, 64)
    assert_close(got, ref, dtype, f"patchify/{dtype}")


def test_patchify_general_gather_chunks():
    # Three-wide bricks take the general gather; 384 output channels are three
    # 128-channel chunks, so both chunk groups of a workgroup work, the first
    # group twice.
    _announce("patchify general gather, 3 chunks")
    d = draw(43, [("x", (2, 4, 4, 7, 9), 1.0), ("w", (384, 4, 2, 2, 3), 0.02), ("b", (384,), 0.1)], "bf16")
    x, wt, b = (to_dev(d[n]) for n in ("x", "w", "b"))
    got = to_host(vd.patchify(x, wt, b, heads=3, head_dim=128))
    ref = oracle.patchify(d["x"].f32, d["w"].f32, d["b"].f32)
    assert got.shape == ref.shape == (2, 2 * 3 * 3, 384)
    assert_close(got, ref, "bf16", "patchify/general/3 chunks")


@pytest.mark.parametrize("C,dout", [(16, 384), (12, 640), (16, 1536)])
def test_patchify_bias_chunks(C, dout):
    # Several 128-channel chunks with a bias (each chunk's bias is fetched
    # one chunk ahead), a 1x2x2 brick, and a token count that leaves the last
    # 32-token block ragged (3 x 7 x 5 = 105 tokens).
    _announce(f"patchify bias chunks C={C} dout={dout}")
    d = draw(43, [("x", (1, C, 3, 14, 10), 1.0), ("w", (dout, C, 1, 2, 2), 0.02), ("b", (dout,), 0.1)], "bf16")
    x, wt, b = (to_dev(d[n]) for n in ("x", "w", "b"))
    got = to_host(vd.patchify(x, wt, b, heads=dout // 128, head_dim=128))
    ref = oracle.patchify(d["x"].f32, d["w"].f32, d["b"].f32)
    assert got.shape == ref.shape == (1, 105, dout)
    assert_close(got, ref, "bf16", f"patchify/C{C}/dout{dout}")


@pytest.mark.parametrize("C,pt,ph,pw,dout,B", [
    (4, 1, 2, 2, 256, 1),    # K = 16: one 32-wide k step, half of it padding
    (8, 1, 2, 2, 128, 2),    # K = 32: exactly one k step; two clips
    (3, 1, 2, 2, 448, 1),    # K = 12: W rows not a multiple of 8 elements; 7 channel steps
    (16, 2, 2, 2, 256, 1),   # K = 128: beyond the per-wavefront kernel's two k steps
    (8, 1, 2, 6, 384, 1),    # K = 96, six-wide bricks: general gather of the chunked kernel
    (4, 1, 2, 2, 200, 1),    # 200 channels: the last 64-channel step holds 8
    (16, 1, 2, 2, 840, 2),   # 840 channels: a third channel group of 72 (a full step and 8)
])
def test_patchify_patch_lengths(C, pt, ph, pw, dout, B):
    # Patch lengths on both sides of 64 (the largest the per-wavefront kernel
    # takes) and of 32, over a 2 x 5 x 7 token grid: 70 tokens, so the second
    # 64-token block is ragged.
    _announce(f"patchify patch length {C * pt * ph * pw}: C={C} brick {pt}x{ph}x{pw} dout={dout} B={B}")
    d = draw(44 + C + pw, [("x", (B, C, 2 * pt, 5 * ph, 7 * pw), 1.0), ("w", (dout, C, pt, ph, pw), 0.05),
                           ("b", (dout,), 0.1)], "bf16")
    x, wt, b = (to_dev(d[n]) for n in ("x", "w", "b"))
    heads = dout // 64 if dout % 64 == 0 else dout // 8
    got = to_host(vd.patchify(x, wt, b, heads=heads, head_dim=dout // heads))
    ref = oracle.patchify(d["x"].f32, d["w"].f32, d["b"].f32)
    assert got.shape == ref.shape == (B, 70, dout)
    assert_close(got, ref, "bf16", f"patchify/K{C * pt * ph * pw}")


def test_patchify_480p_frames():
    # The 480p block input at full size: latent (1,16,21,60,104) -> 32,760
    # tokens of 1,536 (the last 64-token block holds 56). Three whole latent
    # frames are checked against the oracle run on those frames alone
    # (patchify is local in t).
    _announce("patchify 480p full size: latent (1,16,21,60,104) -> [1,32760,1536], frames 0, 9, 20")
    d = draw(47, [("x", (1, 16, 21, 60, 104), 1.0), ("w", (1536, 16, 1, 2, 2), 0.05), ("b", (1536,), 0.1)],
             "bf16")
    x, wt, b = (to_dev(d[n]) for n in ("x", "w", "b"))
    got = vd.patchify(x, wt, b, heads=12, head_dim=128)
    hw = 30 * 52
    for t in (0, 9, 20):
        ref = oracle.patchify(d["x"].f32[:, :, t:t + 1], d["w"].f32, d["b"].f32)
        assert_close(to_host(got[:, t * hw:(t + 1) * hw]), ref, "bf16", f"patchify/480p/frame{t}")


# ----------------------------------------------------------------------------
# Full-size workloads, sampled
# ----------------------------------------------------------------------------

def _sampled_attention(wname, mode, stride, q_scale=1.0, offset=None):
    w = WORKLOADS[wname]
    grid = (w.T, w.Hp, w.Wp)
    _announce(f"{wname} {mode} full size, rows every {stride}, q/k std {q_scale}")
    d, (q, k, v) = _qkv(w, q_scale)
    got = PASSES[mode](q, k, v, grid)
    rows = sample_rows(w.N, stride, offset=stride // 3 if offset is None else offset)
    got_rows = to_host(got[:, torch.from_numpy(rows).cuda()])
    ref = oracle.attention(d["q"].f32, d["k"].f32, d["v"].f32, grid, mode, rows=rows)
    return assert_close(got_rows, ref, "bf16", f"{wname}/{mode}/std{q_scale}")


def test_480p_full_sampled():
    _sampled_attention("480p_full", "full", 512)


@pytest.mark.parametrize("D,mode,stride", [(32, "full", 1637), (32, "spatial", 389), (32, "temporal", 97),
                                            (64, "full", 1637), (64, "spatial", 389), (64, "temporal", 97)])
def test_480p_grid_small_heads_sampled(D, mode, stride):
    # head_dim 32 and 64 at the 480p token grid (1536 / D heads keep the
    # width): the full pass's whole-clip key loop (head_dim 64 on the 8-wave
    # ping-pong, 32 on the 4-wave tile), every 1,560-key frame of the spatial
    # pass, and the 21-frame temporal sequences.
    grid = (21, 30, 52)
    heads = 1536 // D
    _announce(f"480p grid, {heads} heads x {D}, {mode}, rows every {stride}")
    w = small_grid(f"d{D}_480p", 1 if mode == "full" else 2, *grid, heads, D, "bf16", seed=33 + D)
    d, (q, k, v) = _qkv(w)
    got = PASSES[mode](q, k, v, grid)
    rows = sample_rows(w.N, stride, offset=stride // 2)
    ref = oracle.attention(d["q"].f32, d["k"].f32, d["v"].f32, grid, mode, rows=rows)
    assert_close(to_host(got[:, torch.from_numpy(rows).cuda()]), ref, "bf16", f"480p_d{D}/{mode}")


def test_480p_divided_spatial_sampled():
    _sampled_attention("480p_divided", "spatial", 97)


def test_480p_divided_temporal_whole():
    w = WORKLOADS["480p_divided"]
    grid = (w.T, w.Hp, w.Wp)
    _announce("480p divided temporal, every row")
    d, (q, k, v) = _qkv(w)
    got = to_host(vd.attn_temporal(q, k, v, grid))
    ref = oracle.attention(d["q"].f32, d["k"].f32, d["v"].f32, grid, "temporal")
    assert_close(got, ref, "bf16", "480p_divided/temporal")


def test_720p_full_sampled():
    # 259 query rows (every 293rd token from 97, plus the last) of all 40
    # heads: about 4e11 oracle FLOP.
    _sampled_attention("720p_full", "full", 293, offset=97)


@pytest.mark.parametrize("wname,mode,stride", [("480p_full", "full", 509), ("480p_divided", "spatial", 97)])
def test_480p_peaky_sampled(wname, mode, stride):
    # Q and K of standard deviation 4 (logits of standard deviation 16) at
    # the full size: the reference maximum is raised on many of the 512 key
    # tiles of a full-attention row, and on the 25 of a frame.
    _sampled_attention(wname, mode, stride, q_scale=4.0)


@pytest.mark.parametrize("wname,mode,stride", [("480p_full", "full", 509), ("480p_divided", "spatial", 97)])
def test_480p_rising_logits_sampled(wname, mode, stride):
    # Key norms ramp up 30x along each clip (full) or each clip's token order
    # (spatial: frame by frame), so the largest score keeps growing across
    # the key tiles of a row and the reference is raised far into the row.
    w = WORKLOADS[wname]
    grid = (w.T, w.Hp, w.Wp)
    _announce(f"{wname} {mode} rising logits full size, rows every {stride}")
    d = w.draw_qkv()
    ramp = (1.0 + 30.0 * np.arange(w.N, dtype=np.float32) / w.N)[None, :, None, None]
    kb = bf16_bits(d["k"].f32 * ramp)
    k_f32 = bf16_to_f32(kb).reshape(d["k"].f32.shape)
    q, v = to_dev(d["q"]), to_dev(d["v"])
    k = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).cuda()
    got = PASSES[mode](q, k, v, grid)
    rows = sample_rows(w.N, stride, offset=stride // 2)
    got_rows = to_host(got[:, torch.from_numpy(rows).cuda()])
    ref = oracle.attention(d["q"].f32, k_f32, d["v"].f32, grid, mode, rows=rows)
    assert_close(got_rows, ref, "bf16", f"{wname}/{mode}/rising")


@pytest.mark.parametrize("mode", ["full", "spatial", "temporal"])
@pytest.mark.parametrize("scale", [0.05, 0.3])
def test_explicit_scale(mode, scale):
    # A positive scale replaces 1/sqrt(head_dim) (0.088 at 128) in every pass.
    grid = (3, 10, 25)
    _announce(f"explicit scale {scale} {mode} grid={grid}")
    w = small_grid("scale", 1, *grid, 2, 128, "bf16", seed=57)
    d, (q, k, v) = _qkv(w)
    got = to_host(PASSES[mode](q, k, v, grid, scale=scale))
    ref = oracle.attention(d["q"].f32, d["k"].f32, d["v"].f32, grid, mode, scale=scale)
    assert_close(got, ref, "bf16", f"scale{scale}/{mode}")


@pytest.mark.parametrize("mode", ["full", "spatial", "temporal"])
def test_nan_and_inf_propagate(mode):
    """NaN and Inf inputs are not errors: they reach exactly the outputs whose
    key sets hold them, as in the oracle (an Inf score makes its row NaN, a
    -Inf score gets weight 0, NaN or Inf in V reaches that feature of every
    query that sees the key). Everything else stays finite and in tolerance.
    Non-finite data cannot make a kernel access memory differently."""
    grid = (3, 7, 11)
    N = 231
    _announce(f"NaN/Inf propagation {mode} grid={grid}")
    w = small_grid("nonfinite", 1, *grid, 2, 128, "bf16", seed=61)
    d = w.draw_qkv()
    q, k, v = (d[n].f32.copy() for n in ("q", "k", "v"))
    q[0, 40, 0, 5] = np.nan          # one query row of head 0
    k[0, 100, 1, 7] = np.inf         # one key of head 1: +-Inf scores
    k[0, 150, 0, 3] = -np.inf        # one key of head 0
    v[0, 200, 0, 9] = np.nan         # one value feature of head 0
    v[0, 77, 1, 30] = np.inf         # one value feature of head 1
    dev = [torch.from_numpy(bf16_bits(t).view(np.int16)).view(torch.bfloat16).cuda() for t in (q, k, v)]
    got = to_host(PASSES[mode](*dev, grid))
    ref = oracle.attention(q, k, v, grid, mode)
    for name, pred in (("nan", np.isnan), ("+inf", np.isposinf), ("-inf", np.isneginf)):
        assert np.array_equal(pred(got), pred(ref)), f"{mode}: {name} pattern differs"
    assert np.isnan(ref).any() and np.isinf(ref).any()
    fin = np.isfinite(ref)
    assert fin.sum() > 0.3 * ref.size
    mx, rl = stats(got[fin], ref[fin])
    print(f"[parity] nonfinite/{mode}: finite part max_abs={mx:.3e} rel_l1={rl:.3e}", flush=True)
    assert mx <= 2e-2 and rl <= 5e-3


# ----------------------------------------------------------------------------
# RoPE applied inside the attention kernel
# ----------------------------------------------------------------------------

ROPE_PASSES = {"full": vd.attn_full_rope, "spatial": vd.attn_spatial_rope, "temporal": vd.attn_temporal_rope}
ROPE_SMALL = [
    # (name, B, grid, heads, D, split)
    # 750 tokens: ragged last key tile and query block.
    ("rope_ragged_750", 1, (3, 10, 25), 2, 128, (44, 42, 42)),
    # two clips: the second clip's rows start at token row N, spatial
    # segments at every frame of both clips.
    ("rope_two_clips_620", 2, (5, 4, 31), 2, 128, (44, 42, 42)),
    # 35-token frames: one 64-key tile spans two frame boundaries, so the
    # per-tile step of the key positions carries into t and h.
    ("rope_small_frames_140", 2, (4, 5, 7), 2, 128, (44, 42, 42)),
    # a single row per frame: the w index is always 0 and t steps by 64 / Wp.
    ("rope_one_row_frames", 1, (30, 1, 9), 2, 128, (44, 42, 42)),
    # 40 frames: the temporal kernel's two-block form (T > 32).
    ("rope_long_time_40", 1, (40, 2, 3), 2, 128, (44, 42, 42)),
    ("rope_d64", 1, (5, 6, 9), 3, 64, (24, 20, 20)),
    ("rope_d32", 1, (5, 6, 9), 3, 32, (12, 10, 10)),
    ("rope_two_clips_d32", 2, (5, 4, 31), 2, 32, (12, 10, 10)),
    ("rope_uneven_split", 1, (3, 7, 11), 2, 128, (64, 32, 32)),
    ("rope_no_time_part", 1, (3, 7, 11), 2, 128, (0, 64, 64)),
]


def _rope_ref(d, grid, split, mode, rows=None):
    qr = oracle.rope3d(d["q"].f32, grid, split)
    kr = oracle.rope3d(d["k"].f32, grid, split)
    return oracle.attention(qr, kr, d["v"].f32, grid, mode, rows=rows)


@pytest.mark.parametrize("mode", ["full", "spatial", "temporal"])
@pytest.mark.parametrize("case", ROPE_SMALL, ids=[c[0] for c in ROPE_SMALL])
def test_attn_rope_small(case, mode):
    """attention(RoPE(q), RoPE(k), v) with the rotation inside the kernel,
    against the oracle's RoPE followed by its attention."""
    name, B, grid, heads, D, split = case
    _announce(f"attn {mode} with fused RoPE {name} B={B} grid={grid} heads={heads} D={D} split={split}")
    w = small_grid(name, B, *grid, heads, D, "bf16", seed=200 + len(name))
    d, (q, k, v) = _qkv(w)
    q0, k0 = q.clone(), k.clone()
    got = to_host(ROPE_PASSES[mode](q, k, v, grid, split))
    torch.cuda.synchronize()
    assert_close(got, _rope_ref(d, grid, split, mode), "bf16", f"{name}/{mode}+rope")
    # q and k in memory are left unrotated.
    assert torch.equal(q.view(torch.int16), q0.view(torch.int16))
    assert torch.equal(k.view(torch.int16), k0.view(torch.int16))


@pytest.mark.parametrize("mode", ["full", "spatial", "temporal"])
def test_attn_rope_peaky(mode):
    """Q and K of standard deviation 4 (logits of standard deviation 16):
    the running maximum is raised often, on rotated operands. The kernel
    stores the rotated Q and K in bf16 (as the separate RoPE pass does), so
    the oracle's rotated values are rounded to bf16 before its attention:
    at these logit sizes that rounding alone moves the oracle's own output
    by 0.10-0.14 (max-abs, full and spatial), past the 2e-2 bound."""
    grid, split = (3, 8, 13), (44, 42, 42)
    _announce(f"peaky attn {mode} with fused RoPE grid={grid}")
    w = small_grid("rope_peaky", 1, *grid, 2, 128, "bf16", seed=9)
    d, (q, k, v) = _qkv(w, q_scale=4.0)
    got = to_host(ROPE_PASSES[mode](q, k, v, grid, split))
    qr = round_bf16(oracle.rope3d(d["q"].f32, grid, split).astype(np.float32))
    kr = round_bf16(oracle.rope3d(d["k"].f32, grid, split).astype(np.float32))
    ref = oracle.attention(qr, kr, d["v"].f32, grid, mode)
    assert_close(got, ref, "bf16", f"peaky/{mode}+rope")


@pytest.mark.parametrize("order", [("spatial", "temporal"), ("temporal", "spatial")])
def test_divided_chain_with_rope_bf16(order):
    """The binding's divided() chain with RoPE in bf16 (its temporal pass
    rotates inside the kernel, its spatial pass after a separate RoPE
    pass) against the oracle's chain with every stored intermediate, the
    rotated q/k included, rounded to bf16."""
    grid, split = (5, 6, 9), (44, 42, 42)
    _announce(f"divided chain {order} with RoPE, bf16, grid={grid}")
    w = small_grid("divided_rope", 1, *grid, 2, 128, "bf16", seed=41)
    d = w.draw_qkv()
    x = to_dev(d["q"])
    got = to_host(vd.divided(x, grid, order=order, split=split))
    ref = oracle.divided(d["q"].f32, grid, order, rope_split=split, storage="bf16")
    assert_close(got, ref, "bf16", f"divided/{'-'.join(order)}+rope")


def test_divided_chain_without_rope_bf16():
    """divided() with no split in bf16: q = k = v = x for each pass, and
    each pass's output stored in bf16 before the next reads it."""
    grid = (5, 6, 9)
    _announce(f"divided chain without RoPE, bf16, grid={grid}")
    w = small_grid("divided_plain", 1, *grid, 2, 128, "bf16", seed=43)
    d = w.draw_qkv()
    for order in (("spatial", "temporal"), ("temporal", "spatial")):
        got = to_host(vd.divided(to_dev(d["q"]), grid, order=order))
        ref = oracle.divided(d["q"].f32, grid, order, storage="bf16")
        assert_close(got, ref, "bf16", f"divided/{'-'.join(order)}")


def test_attn_rope_theta_and_scale():
    """Another base and an explicit softmax scale reach the kernel."""
    grid, split = (3, 10, 25), (44, 42, 42)
    _announce("attn full with fused RoPE, theta 500, scale 0.05")
    w = small_grid("rope_theta", 1, *grid, 2, 128, "bf16", seed=233)
    d, (q, k, v) = _qkv(w)
    got = to_host(vd.attn_full_rope(q, k, v, grid, split, theta=500.0, scale=0.05))
    qr = oracle.rope3d(d["q"].f32, grid, split, theta=500.0)
    kr = oracle.rope3d(d["k"].f32, grid, split, theta=500.0)
    ref = oracle.attention(qr, kr, d["v"].f32, grid, "full", scale=0.05)
    assert_close(got, ref, "bf16", "full+rope/theta500")


@pytest.mark.parametrize("wname,mode,stride", [("480p_full", "full", 512), ("480p_divided", "spatial", 97),
                                               ("480p_divided", "temporal", 89)])
def test_480p_attn_rope_sampled(wname, mode, stride):
    w = WORKLOADS[wname]
    grid, split = (w.T, w.Hp, w.Wp), (44, 42, 42)
    _announce(f"{wname} {mode} with fused RoPE, full size, rows every {stride}")
    d, (q, k, v) = _qkv(w)
    got = ROPE_PASSES[mode](q, k, v, grid, split)
    rows = sample_rows(w.N, stride, offset=stride // 5)
    got_rows = to_host(got[:, torch.from_numpy(rows).cuda()])
    assert_close(got_rows, _rope_ref(d, grid, split, mode, rows=rows), "bf16", f"{wname}/{mode}+rope")


def test_block_input_path():
    """Latent (1,16,21,60,104) -> patchify -> RoPE -> spatial -> temporal."""
    w = WORKLOADS["block_input"]
    grid = (w.T, w.Hp, w.Wp)
    split = w.rope_split
    _announce("block input path")
    d = w.draw_latent()
    x, wt = to_dev(d["x"]), to_dev(d["w"])
    tok = vd.patchify(x, wt, heads=w.heads, head_dim=w.head_dim)
    ref_tok = oracle.patchify(d["x"].f32, d["w"].f32)
    assert_close(to_host(tok), ref_tok, "bf16", "block/patchify")

    x0 = tok.view(1, w.N, w.heads, w.head_dim)
    r0 = vd.rope3d(x0, grid, split)
    ref_r0 = oracle.rope3d(ref_tok.reshape(1, w.N, w.heads, w.head_dim), grid, split)
    assert_close(to_host(r0), ref_r0, "bf16", "block/rope")

    x1 = vd.attn_spatial(r0, r0, x0, grid)
    r1 = vd.rope3d(x1, grid, split)
    x2 = vd.attn_temporal(r1, r1, x1, grid)
    torch.cuda.synchronize()

    # Oracle chain restricted to a few patch positions: their temporal outputs
    # need the spatial outputs of every frame at those positions.
    HW = w.Hp * w.Wp
    positions = np.array([0, 777, HW - 1], dtype=np.int64)
    rows = (np.arange(w.T)[:, None] * HW + positions[None, :]).reshape(-1)
    xr = ref_tok.reshape(1, w.N, w.heads, w.head_dim)
    sp_rows = oracle.attention(ref_r0, ref_r0, xr, grid, "spatial", rows=rows)
    x1_full = np.zeros_like(xr)
    x1_full[:, rows] = sp_rows
    r1_full = oracle.rope3d(x1_full, grid, split)
    ref_x2 = oracle.attention(r1_full, r1_full, x1_full, grid, "temporal", rows=rows)
    got_x2 = to_host(x2[:, torch.from_numpy(rows).cuda()])
    assert_close(to_host(x1[:, torch.from_numpy(rows).cuda()]), sp_rows, "bf16", "block/spatial")
    assert_close(got_x2, ref_x2, "bf16", "block/spatial-then-temporal")


def test_block_input_divided():
    """The block-input workload through the binding's own divided() chain at
    the full 480p size: latent (1,16,21,60,104) -> patchify -> spatial pass
    on RoPE'd q/k (separate RoPE pass) -> temporal pass with RoPE inside the
    kernel. The oracle chain rounds the stored tokens, rotated q/k and the
    spatial output to bf16 as the GPU stores them, and is evaluated at every
    frame of four patch positions (two interior, the first and the last)."""
    w = WORKLOADS["block_input"]
    grid = (w.T, w.Hp, w.Wp)
    split = w.rope_split
    _announce("block input through divided(), spatial then temporal, full size")
    d = w.draw_latent()
    x, wt = to_dev(d["x"]), to_dev(d["w"])
    tok = vd.patchify(x, wt, heads=w.heads, head_dim=w.head_dim)
    x0 = tok.view(1, w.N, w.heads, w.head_dim)
    got = vd.divided(x0, grid, order=("spatial", "temporal"), split=split)
    torch.cuda.synchronize()
    ref_tok = oracle.store(oracle.patchify(d["x"].f32, d["w"].f32), "bf16")
    HW = w.Hp * w.Wp
    positions = np.array([0, 777, 1234, HW - 1], dtype=np.int64)
    rows, _, ref = space_then_time_at_positions(ref_tok.reshape(1, w.N, w.heads, w.head_dim), grid, split,
                                                positions, storage="bf16")
    assert_close(to_host(got[:, torch.from_numpy(rows).cuda()]), ref, "bf16", "block/divided()")


# ----------------------------------------------------------------------------
# Cross-attention (video queries, text keys)
# ----------------------------------------------------------------------------

CROSS_SMALL = [("cross_231x77", 2, 231, 77, 2, 128), ("cross_1000x512", 1, 1000, 512, 2, 128),
               ("cross_d64", 1, 300, 130, 3, 64), ("cross_one_key", 2, 150, 1, 2, 128),
               # head_dim 64 over five key tiles, the last with 20 keys (a
               # fully masked second 32-key block).
               ("cross_d64_5tiles", 1, 400, 276, 2, 64),
               ("cross_d32", 1, 300, 130, 3, 32), ("cross_d32_5tiles", 2, 400, 276, 2, 32)]


@pytest.mark.parametrize("case", CROSS_SMALL, ids=[c[0] for c in CROSS_SMALL])
def test_cross_small_bf16(case):
    name, B, Nq, Nk, heads, D = case
    _announce(f"cross bf16 {name}")
    w = CrossWorkload(name, B, Nq, Nk, heads, D, "bf16", seed=60 + Nk)
    d = w.draw()
    q, k, v = (to_dev(d[n]) for n in ("q", "k", "v"))
    got = vd.attn_cross(q, k, v)
    if Nk == 1:  # a single key: every query returns it bit for bit
        assert torch.equal(got, v.expand_as(got))
        return
    ref = oracle.cross_attention(d["q"].f32, d["k"].f32, d["v"].f32)
    assert_close(to_host(got), ref, "bf16", f"{name}")


def test_cross_peaky_bf16():
    _announce("cross peaky")
    w = CrossWorkload("cross_peaky", 1, 400, 200, 2, 128, "bf16", seed=77)
    d = w.draw(q_scale=4.0)
    q, k, v = (to_dev(d[n]) for n in ("q", "k", "v"))
    ref = oracle.cross_attention(d["q"].f32, d["k"].f32, d["v"].f32)
    assert_close(to_host(vd.attn_cross(q, k, v)), ref, "bf16", "cross/peaky")


@pytest.mark.parametrize("D", [32, 64, 128])
def test_cross_f32(D):
    _announce(f"cross f32 D={D}")
    w = CrossWorkload("cross_f32", 2, 70, 45, 2, D, "f32", seed=78)
    d = w.draw()
    q, k, v = (to_dev(d[n]) for n in ("q", "k", "v"))
    ref = oracle.cross_attention(d["q"].f32, d["k"].f32, d["v"].f32)
    assert_close(to_host(vd.attn_cross(q, k, v)), ref, "f32", f"cross/f32/D{D}")


def test_cross_480p_sampled():
    w = CROSS_WORKLOADS["cross_480p"]
    _announce("cross 480p: 32,760 video queries x 512 text keys, rows every 127")
    d = w.draw()
    q, k, v = (to_dev(d[n]) for n in ("q", "k", "v"))
    got = vd.attn_cross(q, k, v)
    rows = sample_rows(w.Nq, 127, offset=3)
    ref = oracle.cross_attention(d["q"].f32, d["k"].f32, d["v"].f32, rows=rows)
    assert_close(to_host(got[:, torch.from_numpy(rows).cuda()]), ref, "bf16", "cross_480p")


# ----------------------------------------------------------------------------
# Windowed spacetime attention
# ----------------------------------------------------------------------------

WINDOW_SMALL = [
    # (name, B, grid, window, heads, D)
    ("ragged_edges", 2, (5, 9, 13), (2, 4, 5), 2, 128),
    ("multi_tile", 1, (4, 12, 20), (3, 7, 9), 2, 128),
    ("d64", 1, (6, 7, 11), (4, 3, 6), 3, 64),
    ("frame_window", 1, (3, 9, 15), (1, 9, 15), 2, 128),
    ("time_column", 1, (9, 3, 4), (9, 1, 1), 2, 128),
    ("larger_than_grid", 1, (3, 5, 7), (8, 16, 16), 2, 128),
    ("one_token", 1, (2, 3, 5), (1, 1, 1), 2, 128),
    ("thin_rows", 1, (2, 20, 70), (1, 1, 67), 2, 64),
    ("d32", 1, (6, 7, 11), (4, 3, 6), 3, 32),
    ("thin_rows_d32", 2, (2, 20, 70), (1, 1, 67), 2, 32),
]


@pytest.mark.parametrize("case", WINDOW_SMALL, ids=[c[0] for c in WINDOW_SMALL])
def test_window_small_bf16(case):
    name, B, grid, window, heads, D = case
    _announce(f"window bf16 {name} B={B} grid={grid} window={window} heads={heads} D={D}")
    w = small_grid(name, B, *grid, heads, D, "bf16", seed=200 + len(name))
    d, (q, k, v) = _qkv(w)
    got = to_host(vd.attn_window(q, k, v, grid, window))
    ref = oracle.window_attention(d["q"].f32, d["k"].f32, d["v"].f32, grid, window)
    assert_close(got, ref, "bf16", f"window/{name}")


def test_window_peaky_bf16():
    grid, window = (4, 9, 14), (3, 5, 6)
    _announce(f"window peaky bf16 grid={grid} window={window}")
    w = small_grid("wpeaky", 1, *grid, 2, 128, "bf16", seed=8)
    d, (q, k, v) = _qkv(w, q_scale=4.0)
    got = to_host(vd.attn_window(q, k, v, grid, window))
    ref = oracle.window_attention(d["q"].f32, d["k"].f32, d["v"].f32, grid, window)
    assert_close(got, ref, "bf16", "window/peaky")


def test_window_one_token_is_exact_and_in_bounds():
    # 1x1x1 windows: each output is its own V bit for bit; guard bands around
    # the output stay untouched.
    grid = (3, 5, 7)
    _announce("window 1x1x1 exactness and guard bands")
    w = small_grid("w111", 2, *grid, 2, 128, "bf16", seed=9)
    d, (q, k, v) = _qkv(w)
    n = q.numel()
    buf = torch.full((n + 2 * 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[4096:4096 + n].view_as(q)
    vd.attn_window(q, k, v, grid, (1, 1, 1), out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, v)
    assert bool((buf[:4096] == 7.0).all()) and bool((buf[4096 + n:] == 7.0).all())


@pytest.mark.parametrize("D", [32, 64, 128])
def test_window_f32(D):
    grid, window = (5, 6, 7), (2, 4, 3)
    _announce(f"window f32 D={D} grid={grid} window={window}")
    w = small_grid("wf32", 2, *grid, 2, D, "f32", seed=12)
    d, (q, k, v) = _qkv(w)
    got = to_host(vd.attn_window(q, k, v, grid, window))
    ref = oracle.window_attention(d["q"].f32, d["k"].f32, d["v"].f32, grid, window)
    assert_close(got, ref, "f32", f"window/f32/D{D}")


@pytest.mark.parametrize("window,stride", [(None, 61), ((4, 8, 8), 89)])
def test_480p_window_sampled(window, stride):
    # The benchmark's 3 x 15 x 26 windows (which tile the grid exactly), and
    # 4 x 8 x 8 windows, which leave clipped windows on every edge of it.
    w = WORKLOADS["480p_window"]
    grid = (w.T, w.Hp, w.Wp)
    window = window or w.window
    _announce(f"480p window {window} full size, rows every {stride}")
    d, (q, k, v) = _qkv(w)
    got = vd.attn_window(q, k, v, grid, window)
    rows = sample_rows(w.N, stride, offset=stride // 3)
    got_rows = to_host(got[:, torch.from_numpy(rows).cuda()])
    ref = oracle.window_attention(d["q"].f32, d["k"].f32, d["v"].f32, grid, window, rows=rows)
    assert_close(got_rows, ref, "bf16", f"480p_window/{window}")


# ----------------------------------------------------------------------------
# QKV projection with per-head Q/K RMSNorm and 3D RoPE
# ----------------------------------------------------------------------------

QKV_SMALL = [
    # (name, B, grid, heads, head_dim, dtype, split, bias, norm)
    ("ragged_tokens", 2, (3, 5, 7), 2, 128, "bf16", (44, 42, 42), True, True),
    ("odd_heads_no_rope", 1, (2, 4, 9), 3, 128, "bf16", None, False, True),
    ("multi_tile", 1, (4, 10, 25), 4, 128, "bf16", (44, 42, 42), True, True),
    ("plain_projection", 1, (1, 16, 16), 2, 128, "bf16", None, True, False),
    ("tiny_width_f32", 1, (4, 8, 8), 2, 32, "f32", (12, 10, 10), True, True),
    ("f32_d128", 2, (2, 3, 5), 2, 128, "f32", (44, 42, 42), False, True),
    # Splits other than (44, 42, 42), one with no time pairs.
    ("split_64_32_32", 1, (3, 6, 10), 2, 128, "bf16", (64, 32, 32), True, True),
    ("split_0_64_64", 1, (2, 5, 12), 2, 128, "bf16", (0, 64, 64), False, True),
    # A wide grid: w positions up to 199, so the w-axis angles reach many
    # revolutions before their reduction.
    ("wide_grid_rope", 1, (1, 2, 200), 2, 128, "bf16", (44, 42, 42), True, True),
    # Five heads: 1,920 channels in 7.5 tiles of 256, so one tile holds the
    # last Q heads and the first K heads and another the last K heads and
    # the first V heads (per-channel bias, gain and rotation across them).
    ("five_heads_rope", 1, (3, 4, 10), 5, 128, "bf16", (44, 42, 42), True, True),
]


def _qkv_case(w, d, split, use_bias, norm, rows=None):
    dev = {n: to_dev(d[n]) for n in d}
    grid = (w.T, w.Hp, w.Wp)
    got = vd.qkv_proj(dev["x"], dev["w"], dev["bias"] if use_bias else None, dev["gq"] if norm else None,
                      dev["gk"] if norm else None, grid=grid, heads=w.heads, head_dim=w.head_dim, split=split)
    ref = oracle.qkv_proj(d["x"].f32, d["w"].f32, d["bias"].f32 if use_bias else None,
                          d["gq"].f32 if norm else None, d["gk"].f32 if norm else None, grid, w.heads, w.head_dim,
                          split, rows=rows)
    return got, ref


@pytest.mark.parametrize("case", QKV_SMALL, ids=[c[0] for c in QKV_SMALL])
def test_qkv_proj_small(case):
    name, B, grid, heads, D, dtype, split, use_bias, norm = case
    _announce(f"qkv_proj {name} B={B} grid={grid} heads={heads} D={D} {dtype} split={split}")
    w = QkvWorkload(name, B, *grid, heads, D, dtype, seed=300 + len(name))
    got, ref = _qkv_case(w, w.draw(), split, use_bias, norm)
    for t, g, r in zip("qkv", got, ref):
        assert_close(to_host(g), r, dtype, f"qkv/{name}/{t}")


def test_qkv_proj_480p_sampled():
    w = QKV_WORKLOADS["qkv_480p"]
    _announce("qkv_proj 480p: [1,32760,1536] x [4608,1536], rows every 61")
    d = w.draw()
    rows = sample_rows(w.N, 61, offset=20)
    got, ref = _qkv_case(w, d, w.rope_split, True, True, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    for t, g, r in zip("qkv", got, ref):
        assert_close(to_host(g[:, idx]), r, "bf16", f"qkv_480p/{t}")


def test_qkv_proj_14b_width():
    # The 14B model's width (40 heads x 128, dim 5,120): 80 K stages and 60
    # channel tiles, on a small grid whose token count leaves a ragged tile.
    w = QkvWorkload("qkv_14b", 1, 5, 16, 20, 40, 128, "bf16", seed=31, rope_split=(44, 42, 42))
    _announce("qkv_proj 14B width: [1,1600,5120] x [15360,5120]")
    rows = sample_rows(w.N, 37, offset=5)
    got, ref = _qkv_case(w, w.draw(), w.rope_split, True, True, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    for t, g, r in zip("qkv", got, ref):
        assert_close(to_host(g[:, idx]), r, "bf16", f"qkv_14b/{t}")


def test_attn1_input_chain():
    # The self-attention input path of one block, end to end: patchify of a
    # latent, projection to Q/K/V with per-head RMSNorm and RoPE on Q and K,
    # then full 3D attention; the oracle chains its own routines in fp64.
    grid, heads, D, C = (3, 6, 8), 2, 128, 16
    dim = heads * D
    _announce(f"attn1 chain: latent (1,{C},3,12,16) -> [1,144,{dim}] -> qkv -> full attention")
    d = draw(51, [("x", (1, C, 3, 12, 16), 1.0), ("pw", (dim, C, 1, 2, 2), 0.02), ("w", (3 * dim, dim), 0.02),
                  ("b", (3 * dim,), 0.02)], "bf16")
    g = draw(52, [("gq", (dim,), 0.02), ("gk", (dim,), 0.02)], "f32")
    gq, gk = (round_bf16(g[n].f32 + np.float32(1.0)) for n in ("gq", "gk"))
    dev = {n: to_dev(d[n]) for n in d}
    gq_d, gk_d = (torch.from_numpy(bf16_bits(t).view(np.int16)).view(torch.bfloat16).cuda() for t in (gq, gk))
    tok = vd.patchify(dev["x"], dev["pw"], heads=heads, head_dim=D)
    q, k, v = vd.qkv_proj(tok, dev["w"], dev["b"], gq_d, gk_d, grid=grid, heads=heads, head_dim=D,
                          split=(44, 42, 42))
    got = to_host(vd.attn_full(q, k, v, grid))
    rtok = oracle.patchify(d["x"].f32, d["pw"].f32)
    rq, rk, rv = oracle.qkv_proj(rtok, d["w"].f32, d["b"].f32, gq, gk, grid, heads, D, (44, 42, 42))
    ref = oracle.attention(rq, rk, rv, grid, "full")
    assert_close(got, ref, "bf16", "attn1_chain")


@pytest.mark.parametrize("T", [24, 25, 32, 33, 64])
def test_temporal_block_boundaries(T):
    # The temporal kernel picks its layout by T: up to 24, up to 32, up to 64
    # frames (two 32-key blocks); each side of every boundary, up to the
    # 64-frame limit.
    grid = (T, 3, 5)
    _announce(f"temporal bf16 T={T} grid={grid}")
    w = small_grid(f"t{T}", 2, *grid, 3, 128, "bf16", seed=400 + T)
    d, (q, k, v) = _qkv(w)
    got = to_host(vd.attn_temporal(q, k, v, grid))
    ref = oracle.attention(d["q"].f32, d["k"].f32, d["v"].f32, grid, "temporal")
    assert_close(got, ref, "bf16", f"temporal/T{T}")
