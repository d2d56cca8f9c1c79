"""The C ABI loads, exports every function include/vdit.h declares, and rejects
bad arguments before it enqueues anything. No call here reaches the GPU: each
one returns from the argument checks, which run before any HIP call."""

import ctypes
import os
import re

import pytest

import spacetime_attention_amd as vd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "vdit.h")).read()
    return sorted(set(re.findall(r"\b(vdit_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vd.LIB_PATH):
        from spacetime_attention_amd import build
        build.build()
    return vd.load_library()


def test_exports_every_declared_function(lib):
    declared = _declared()
    assert declared == sorted(vd.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in enumerate(vd.STATUS):
        assert vd.status_str(code).startswith(name)


# Fake, never-dereferenced addresses: every case below fails a check first.
P = 1 << 20
Q, K, V, O = P, 2 * P << 8, 3 * P << 8, 4 * P << 8


@pytest.mark.parametrize("fn", ["vdit_attn_full", "vdit_attn_spatial", "vdit_attn_temporal"])
def test_attention_argument_errors(lib, fn):
    f = getattr(lib, fn)
    ok = dict(q=Q, k=K, v=V, o=O, B=1, heads=2, T=3, Hp=4, Wp=5, D=128, scale=0.0, dt=vd.BF16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["B"], a["heads"], a["T"], a["Hp"], a["Wp"], a["D"],
                 a["scale"], a["dt"], None)

    assert call(q=None) == 1                      # VDIT_E_NULL
    assert call(o=None) == 1
    assert call(B=0) == 2                         # VDIT_E_SHAPE
    assert call(Wp=-1) == 2
    assert call(T=1 << 16, Hp=1 << 16, Wp=1 << 16) == 2  # overflow
    assert call(T=64, Hp=256, Wp=256, heads=16) == 2     # one batch over 2 GiB in bf16
    assert call(D=96) == 3                        # VDIT_E_HEAD_DIM
    assert call(D=48) == 3                        # 32, 64 and 128 only
    assert call(dt=vd.F32, D=48) == 3
    assert call(q=Q + 8) == 5                     # VDIT_E_ALIGN
    assert call(o=Q + 16) == 6                    # VDIT_E_ALIAS (o inside q)
    assert call(dt=7) == 7                        # VDIT_E_DTYPE
    if fn == "vdit_attn_temporal":
        assert call(T=65) == 2


@pytest.mark.parametrize("fn", ["vdit_attn_full_rope", "vdit_attn_spatial_rope", "vdit_attn_temporal_rope"])
def test_attention_rope_argument_errors(lib, fn):
    f = getattr(lib, fn)
    ok = dict(q=Q, k=K, v=V, o=O, B=1, heads=2, T=3, Hp=4, Wp=5, D=128, split=(44, 42, 42), theta=10000.0,
              scale=0.0, dt=vd.BF16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["B"], a["heads"], a["T"], a["Hp"], a["Wp"], a["D"],
                 *a["split"], a["theta"], a["scale"], a["dt"], None)

    assert call(q=None) == 1                      # VDIT_E_NULL
    assert call(B=0) == 2                         # VDIT_E_SHAPE
    assert call(T=64, Hp=256, Wp=256, heads=16) == 2
    assert call(D=96) == 3                        # VDIT_E_HEAD_DIM
    assert call(dt=vd.F32) == 7                   # bf16 only
    assert call(dt=7) == 7
    assert call(split=(44, 42, 40)) == 4          # VDIT_E_ROPE_SPLIT: parts do not sum to D
    assert call(split=(43, 43, 42)) == 4          # odd part
    assert call(D=64, split=(44, 42, 42)) == 4
    assert call(theta=0.0) == 2
    assert call(theta=float("inf")) == 2
    assert call(q=Q + 8) == 5                     # VDIT_E_ALIGN
    assert call(o=K + 16) == 6                    # VDIT_E_ALIAS
    if fn == "vdit_attn_temporal_rope":
        assert call(T=65) == 2


def test_rope_argument_errors(lib):
    f = lib.vdit_rope3d

    def call(x=Q, y=O, B=1, heads=12, T=2, Hp=3, Wp=4, D=128, dt_=44, dh=42, dw=42, theta=10000.0, dt=vd.BF16):
        return f(x, y, B, heads, T, Hp, Wp, D, dt_, dh, dw, theta, dt, None)

    assert call(x=None) == 1
    assert call(dw=40) == 4                       # VDIT_E_ROPE_SPLIT: parts do not sum to D
    assert call(dt_=43, dh=43) == 4               # odd part
    assert call(D=100, dt_=34, dh=34, dw=32) == 3 # head_dim not a multiple of 8
    assert call(theta=0.0) == 2
    assert call(y=Q + 16) == 6                    # partial overlap
    assert call(y=Q + 8) == 5


def test_patchify_argument_errors(lib):
    f = lib.vdit_patchify

    def call(x=Q, w=K, b=None, o=O, B=1, C=16, pt=1, ph=2, pw=2, Tl=21, Hl=60, Wl=104, heads=12, T=21,
             Hp=30, Wp=52, D=128, dt=vd.BF16):
        return f(x, w, b, o, B, C, pt, ph, pw, Tl, Hl, Wl, heads, T, Hp, Wp, D, dt, None)

    assert call(x=None) == 1
    assert call(Hp=31) == 2                       # grid is not the convolution's
    assert call(Tl=22, T=22, pt=2) == 2
    assert call(C=200) == 2                       # patch longer than the bf16 kernel holds
    assert call(heads=1, D=12) == 2               # output width not a multiple of 8
    assert call(o=Q + 16) == 6
    assert call(w=K + 4) == 5


def test_cross_argument_errors(lib):
    f = lib.vdit_attn_cross

    def call(q=Q, k=K, v=V, o=O, B=1, heads=2, Nq=100, Nk=20, D=128, scale=0.0, dt=vd.BF16):
        return f(q, k, v, o, B, heads, Nq, Nk, D, scale, dt, None)

    assert call(k=None) == 1
    assert call(Nk=0) == 2
    assert call(Nq=-3) == 2
    assert call(D=48) == 3
    assert call(v=V + 8) == 5
    assert call(o=K + 16) == 6                    # o overlaps k
    assert call(dt=9) == 7


def test_window_argument_errors(lib):
    f = lib.vdit_attn_window

    def call(q=Q, k=K, v=V, o=O, B=1, heads=2, T=3, Hp=4, Wp=5, D=128, wt=2, wh=2, ww=2, scale=0.0,
             dt=vd.BF16):
        return f(q, k, v, o, B, heads, T, Hp, Wp, D, wt, wh, ww, scale, dt, None)

    assert call(o=None) == 1
    assert call(wt=0) == 2                        # a window extent below 1
    assert call(ww=-2) == 2
    assert call(T=0) == 2
    assert call(T=64, Hp=256, Wp=256, heads=16) == 2  # one batch over 2 GiB in bf16
    assert call(D=48) == 3
    assert call(dt=vd.F32, D=80) == 3
    assert call(k=K + 8) == 5
    assert call(o=V + 16) == 6
    assert call(dt=5) == 7


def test_qkv_proj_argument_errors(lib):
    f = lib.vdit_qkv_proj
    G = 5 * P << 8

    def call(x=Q, w=K, b=None, gq=None, gk=None, q=O, k=V + (1 << 24), v=G, B=1, T=2, Hp=3, Wp=4, heads=2, D=128,
             dt_=44, dh=42, dw=42, theta=10000.0, eps=1e-6, dt=vd.BF16):
        return f(x, w, b, gq, gk, q, k, v, B, T, Hp, Wp, heads, D, dt_, dh, dw, theta, eps, dt, None)

    assert call(x=None) == 1
    assert call(v=None) == 1
    assert call(T=0) == 2
    assert call(eps=-1.0) == 2
    assert call(theta=0.0) == 2
    assert call(D=64, dt_=24, dh=20, dw=20) == 3      # bf16 takes head_dim 128 only
    assert call(dt=vd.F32, D=300, dt_=100, dh=100, dw=100) == 3
    assert call(dw=40) == 4                          # split does not sum to head_dim
    assert call(dt_=0, dh=0, dw=0, w=K + 8) == 5     # an all-zero split (no rotation) passes that check
    assert call(w=K + 8) == 5
    assert call(q=Q + 16) == 6                       # output overlaps x
    assert call(k=O + 64) == 6                       # outputs overlap each other
    assert call(dt=3) == 7
