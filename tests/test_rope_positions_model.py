"""Model of how the attention kernels with RoPE inside track key positions.

The full and spatial kernels rotate each K tile in LDS: a lane's load i
fills key row r = RPL*(wave*LOADS + i) + lane/CH of every 64-key tile, and
the lane carries that row's grid position (t, h, w) from one tile to the
next by adding 64 = dt*Hp*Wp + dh*Wp + dw with one carry per digit. This
model replays that stepping for many grid shapes and checks it against the
position computed directly from the token index, for every key that
exists (rows past the segment's last key are zeros and may hold any
position). It models the index arithmetic only; the GPU tests check the
kernels' results.
"""
import random

import pytest

KBN = 64


def direct(n, Hp, Wp):
    return n // (Hp * Wp), (n // Wp) % Hp, n % Wp


def replay(T, Hp, Wp, korg, Lk, D, NW):
    CH = D // 8
    loads = KBN * CH // (NW * 64)
    rpl = 64 // CH
    HW = Hp * Wp
    N = T * HW
    dt, dh, dw = KBN // HW, (KBN % HW) // Wp, KBN % Wp
    ntiles = (Lk + KBN - 1) // KBN
    for wave in range(NW):
        for lane in range(64):
            for i in range(loads):
                r = rpl * (wave * loads + i) + lane // CH
                t, h, w = direct((korg + r) % N, Hp, Wp)
                for tile in range(ntiles):
                    j = tile * KBN + r
                    if j < Lk:
                        assert (t, h, w) == direct((korg + j) % N, Hp, Wp), (T, Hp, Wp, korg, j)
                    # one tile step, as the kernel takes it
                    w += dw
                    c1 = w >= Wp
                    w -= Wp if c1 else 0
                    h += dh + c1
                    c2 = h >= Hp
                    h -= Hp if c2 else 0
                    t += dt + c2


GRIDS = [(21, 30, 52), (4, 5, 7), (30, 1, 9), (3, 7, 11), (5, 4, 31), (2, 1, 1), (3, 1, 100), (2, 9, 64),
         (1, 8, 8), (7, 2, 32)]


@pytest.mark.parametrize("D,NW", [(128, 8), (128, 4), (64, 8), (64, 4)])
@pytest.mark.parametrize("grid", GRIDS[1:])
def test_full_and_spatial_positions(grid, D, NW):
    T, Hp, Wp = grid
    HW, N = Hp * Wp, T * Hp * Wp
    for b in range(2):                       # full pass: segment = clip b
        replay(T, Hp, Wp, b * N, N, D, NW)
    for seg in range(2 * T):                 # spatial pass: segment = frame seg % T of clip seg // T
        replay(T, Hp, Wp, seg * HW, HW, D, NW)


def test_480p_grid_spatial_positions():
    T, Hp, Wp = GRIDS[0]
    for seg in (0, 1, 20, 21, 41):
        replay(T, Hp, Wp, seg * Hp * Wp, Hp * Wp, 128, 4)


def test_random_grids():
    rng = random.Random(5)
    for _ in range(40):
        T, Hp, Wp = rng.randint(1, 6), rng.randint(1, 40), rng.randint(1, 90)
        D, NW = rng.choice([(128, 8), (128, 4), (64, 8), (64, 4)])
        replay(T, Hp, Wp, 0, T * Hp * Wp, D, NW)
        seg = rng.randrange(2 * T)
        replay(T, Hp, Wp, seg * Hp * Wp, Hp * Wp, D, NW)
