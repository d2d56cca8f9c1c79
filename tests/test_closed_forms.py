"""Closed-form counts of the pages against the values the pages print.

Every expected value comes from tests/golden/page_values.txt, which cites
the passage that prints it.
"""

import math

import pytest

from oracle import closed_forms as cf


def _int(page_values, key):
    return int(page_values[key][0])


def _tuple(page_values, key):
    return tuple(int(v) for v in page_values[key][0].split(","))


def test_token_counts(page_values):
    assert cf.spacetime_tokens(81, 480, 832) == _int(page_values, "tokens_81f_480p")
    assert cf.spacetime_tokens(81, 720, 1280) == _int(page_values, "tokens_81f_720p")
    assert cf.spacetime_tokens(17, 480, 832) == _int(page_values, "tokens_17f_480p")
    assert cf.spacetime_grid(81, 480, 832) == _tuple(page_values, "grid_81f_480p")
    assert cf.spacetime_grid(17, 480, 832) == _tuple(page_values, "grid_17f_480p")
    T, Hp, Wp = cf.spacetime_grid(81, 480, 832)
    assert Hp * Wp == _int(page_values, "tokens_per_slice_480p")


def test_tiny_grid(page_values):
    # (1,4,8,16,16) through a Conv3d with kernel = stride = (2,2,2).
    T, Hp, Wp = 8 // 2, 16 // 2, 16 // 2
    assert (T, Hp, Wp) == _tuple(page_values, "grid_tiny")
    # The cheatsheet's count_tokens with its patch sizes: the same formula.
    assert cf.count_tokens(8, 16, 16, 2, 2, 2) == 256
    assert cf.count_tokens(16, 64, 64) == 8 * 8 * 8  # defaults p_t=2, p_h=p_w=8


@pytest.mark.parametrize("frames,key", [(81, "latent_frames_81"), (17, "latent_frames_17"),
                                        (72, "latent_frames_72"), (96, "latent_frames_96")])
def test_latent_frames(page_values, frames, key):
    want = _int(page_values, key)
    # 72 and 96 are printed by the ceil(F/4) rule; 81 and 17 by 1 + (F-1)//4.
    if frames in (81, 17):
        assert cf.latent_frames(frames) == want
    assert cf.latent_frames_ceil(frames) == want


def test_latent_frame_rules_agree():
    # The two rules of the pages agree for every frame count.
    for f in range(1, 400):
        assert cf.latent_frames(f) == cf.latent_frames_ceil(f)


def test_latent_and_raw_sizes(page_values):
    assert 1 * 16 * 21 * 60 * 104 == _int(page_values, "latent_values_81f")
    assert 1 * 16 * 5 * 60 * 104 == _int(page_values, "latent_values_17f")
    assert 1 * 3 * 81 * 480 * 832 == _int(page_values, "raw_values_81f")
    assert 81 * 480 * 832 == _int(page_values, "raw_pixels_81f")


def test_pair_counts(page_values):
    npix = _int(page_values, "raw_pixels_81f")
    assert cf.full_pairs(npix) == _int(page_values, "raw_pairs_81f")
    assert cf.fp16_bytes(cf.full_pairs(npix)) == _int(page_values, "raw_fp16_bytes_81f")
    n = cf.spacetime_tokens(81, 480, 832)
    assert cf.full_pairs(n) == _int(page_values, "token_pairs_81f")
    assert cf.full_pairs(cf.spacetime_tokens(17, 480, 832)) == _int(page_values, "token_pairs_17f")
    ratio = cf.full_pairs(npix) / cf.full_pairs(n)
    assert round(ratio, 1) == float(page_values["pair_reduction"][0])
    assert round(cf.fp16_bytes(cf.full_pairs(n)) / 1e9, 2) == float(page_values["token_fp16_gb"][0])


@pytest.mark.parametrize("res,h,w", [("480p", 480, 832), ("720p", 720, 1280)])
def test_forward_flops_prints(page_values, res, h, w):
    # The 14B model of "Video Diffusion Models, in depth", Step 2: 14e9
    # weights, 40 layers of width 5,120.
    n = cf.spacetime_tokens(81, h, w)
    dense, attn = cf.dense_flop(14e9, n), cf.attention_flop(n, 5120, 40)
    share = attn / (dense + attn)
    total = 100 * (dense + attn)
    assert round(share, 2) == float(page_values[f"attn_share_{res}"][0])
    assert float(f"{total:.1e}") == float(page_values[f"flops_per_clip_{res}"][0])


def test_divided_cost():
    T, Hp, Wp = cf.spacetime_grid(81, 480, 832)
    HW = Hp * Wp
    N = T * HW
    # (HW)*T^2 + T*(HW)^2 = N^2/HW + N^2/T, an identity of the two terms.
    assert cf.divided_pairs(T, HW) == N * N // HW + N * N // T
    assert cf.divided_pairs(T, HW) == 687_960 + 51_105_600
    # The attention FLOP counts follow the 4*N^2*dim convention per pass.
    D, H = 128, 12
    assert cf.attention_flops_full(1, H, N, D) == 4 * H * D * cf.full_pairs(N)
    assert (cf.attention_flops_spatial(1, H, T, HW, D) + cf.attention_flops_temporal(1, H, T, HW, D)
            == 4 * H * D * cf.divided_pairs(T, HW))
    # The page's per-layer count uses dim = heads * head_dim: the same count.
    assert cf.attention_flop(N, H * D, 1) == cf.attention_flops_full(1, H, N, D)


def test_probe_token_index(page_values):
    T, Hp, Wp = _tuple(page_values, "grid_17f_480p")
    t, h, w = 2, 18, 26
    assert (t * Hp + h) * Wp + w == _int(page_values, "probe_token_index")


def test_rope_split_and_width(page_values):
    split = _tuple(page_values, "rope_split_128")
    pairs = _tuple(page_values, "rope_pairs_128")
    heads, hd = _tuple(page_values, "wan13_heads_dim")
    assert sum(split) == hd == 128
    assert tuple(s // 2 for s in split) == pairs
    assert heads * hd == 1536
    assert math.prod((1, 16, 1, 2, 2)) == 64  # one 16-channel 1x2x2 brick is 64 numbers
