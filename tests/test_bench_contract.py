"""bench.py's host-side contract, checked without a GPU: it refuses more than
one GPU with a message before touching the device, its peak constant is the
published figure, and its window FLOP count matches a brute-force sum over
the clipped windows."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                       env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_published_peak():
    # 256 compute units x 2.4 GHz x 4,096 dense bf16 FLOP per CU per clock.
    assert abs(bench.PEAK_BF16_TFLOPS - 2516.5824) < 1e-6
    assert bench.PEAK_HBM_GBS == 8000.0


class _W:
    def __init__(self, B, T, Hp, Wp, heads, head_dim):
        self.B, self.T, self.Hp, self.Wp, self.heads, self.head_dim = B, T, Hp, Wp, heads, head_dim


@pytest.mark.parametrize("grid,window", [((21, 30, 52), (3, 15, 26)), ((21, 30, 52), (4, 8, 8)),
                                         ((5, 9, 13), (2, 4, 5)), ((3, 5, 7), (8, 16, 16))])
def test_window_flop_matches_brute_force(grid, window):
    w = _W(1, *grid, 12, 128)
    T, Hp, Wp = grid
    wt, wh, ww = window
    count = {}
    for t in range(T):
        for h in range(Hp):
            for x in range(Wp):
                key = (t // wt, h // wh, x // ww)
                count[key] = count.get(key, 0) + 1
    expected = 4.0 * w.B * w.heads * w.head_dim * sum(n * n for n in count.values())
    assert bench.window_flop(w, window) == expected
