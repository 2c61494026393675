"""The C-ABI library loads, exports every declared symbol, and validates on the host (CPU only).

No call here reaches a kernel launch: every call is rejected by host-side
validation before the library touches the GPU.
"""
import ctypes
import math
import os
import re

import pytest

import block_sparse_attention_fractal_amd as nabla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nabla.h")
OK, INVALID, UNSUP, WS = 0, 1, 2, 3
BF16, FP32 = 1, 0
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nabla_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nabla.LIB_PATH):
        from block_sparse_attention_fractal_amd import build
        build.build()
    return nabla.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == {"nabla_abi_version", "nabla_status_string", "nabla_fractal_permute",
                          "nabla_sta_mask", "nabla_block_mask_workspace", "nabla_block_mask",
                          "nabla_sparse_attn_fwd", "nabla_sparse_attn_workspace",
                          "nabla_sparse_attn_fwd_lse", "nabla_sparse_attn_bwd_workspace",
                          "nabla_sparse_attn_bwd", "nabla_block_mask_topk",
                          "nabla_block_mask_grid", "nabla_sparse_attn_workspace_grid",
                          "nabla_sparse_attn_fwd_grid", "nabla_quant_qkv_workspace",
                          "nabla_quant_qkv", "nabla_sparse_attn_q8_workspace",
                          "nabla_sparse_attn_fwd_q8", "nabla_sparse_attn_bwd_grid",
                          "nabla_quant_qkv_grid", "nabla_sparse_attn_fwd_q8_grid",
                          "nabla_block_mask_natural", "nabla_sparse_attn_fwd_natural",
                          "nabla_quant_qkv_natural", "nabla_sparse_attn_fwd_q8_natural",
                          "nabla_sparse_attn_fwd_noalloc"}
    raw = ctypes.CDLL(nabla.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_version_and_status_strings(L):
    assert L.nabla_abi_version() == 11
    for s in range(5):
        assert L.nabla_status_string(s)
    assert L.nabla_status_string(99) == b"unknown status"


def test_workspace_size(L):
    # pooled q and k; rows of 513-2048 blocks add the block scores
    assert L.nabla_block_mask_workspace(1, 61440, 16, 128) == 2 * 16 * 960 * 128 * 4 + 16 * 960 * 960 * 4
    assert L.nabla_block_mask_workspace(1, 8192, 8, 128) == 2 * 8 * 128 * 128 * 4
    assert L.nabla_block_mask_workspace(2, 2049 * 64, 1, 64) == 2 * 2 * 2049 * 64 * 4
    assert L.nabla_block_mask_workspace(1, 100, 16, 128) == 0
    assert L.nabla_block_mask_workspace(0, 64, 1, 64) == 0


def test_block_mask_validation(L):
    f = L.nabla_block_mask
    good = dict(q=FAKE, k=FAKE, dt=BF16, B=1, S=8192, h=8, D=128, sta=None, thr=0.9,
                kv_nb=FAKE, kv_inds=FAKE, ws=FAKE, wsb=1 << 40)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["q"], a["k"], a["dt"], a["B"], a["S"], a["h"], a["D"], a["sta"], a["thr"],
                 a["kv_nb"], a["kv_inds"], a["ws"], a["wsb"], None)

    assert call(q=None) == INVALID
    assert call(kv_inds=None) == INVALID
    assert call(dt=7) == INVALID
    assert call(S=8192 + 32) == INVALID          # S % 64 != 0 (the page requires it)
    assert call(B=0) == INVALID
    assert call(h=-1) == INVALID
    for thr in (-0.01, 1.01, math.nan, math.inf):
        assert call(thr=thr) == INVALID
    assert call(D=96) == UNSUP
    assert call(S=64 * 4097) == UNSUP            # longer rows than the selection kernel holds
    assert call(B=8192, S=64) == UNSUP           # B * heads = 65536: more than a grid's y extent
    assert call(ws=None) == WS
    assert call(wsb=L.nabla_block_mask_workspace(1, 8192, 8, 128) - 1) == WS


def test_block_mask_topk_validation(L):
    f = L.nabla_block_mask_topk

    def call(q=FAKE, dt=BF16, B=1, S=8192, D=128, ratio=0.1, kv_nb=FAKE, ws=FAKE, wsb=1 << 40):
        return f(q, FAKE, dt, B, S, 8, D, None, ratio, kv_nb, FAKE, ws, wsb, None)

    assert call(q=None) == INVALID
    assert call(kv_nb=None) == INVALID
    assert call(dt=7) == INVALID
    assert call(S=8192 + 32) == INVALID
    for r in (-0.01, 1.01, math.nan):
        assert call(ratio=r) == INVALID
    assert call(D=96) == UNSUP
    assert call(S=64 * 2049) == UNSUP            # one wave holds a row of up to 2048 blocks
    assert call(ws=None) == WS
    assert call(wsb=L.nabla_block_mask_workspace(1, 8192, 8, 128) - 1) == WS


def test_grid_entry_points_validation(L):
    g = L.nabla_block_mask_grid

    def mask(q=FAKE, T=2, H=44, W=76, thr=0.9, ratio=-1.0, ws=FAKE, wsb=1 << 40):
        return g(q, FAKE, BF16, 1, T, H, W, 8, 128, None, thr, ratio, FAKE, FAKE, ws, wsb, None)

    assert mask(q=None) == INVALID
    assert mask(T=0) == INVALID
    assert mask(H=0) == INVALID
    assert mask(thr=1.5) == INVALID               # the CDF estimator checks thr
    assert mask(ratio=1.5) == INVALID             # the top-k variant checks its ratio
    assert mask(ratio=math.nan) == INVALID
    S = 2 * 6 * 10 * 64                           # 44 x 76 -> 6 x 10 patches
    assert mask(wsb=L.nabla_block_mask_workspace(1, S, 8, 128) - 1) == WS
    f = L.nabla_sparse_attn_fwd_grid

    def fwd(q=FAKE, T=2, H=44, W=76, D=128, o=FAKE, ws=FAKE, wsb=1 << 40):
        return f(q, FAKE, FAKE, BF16, 1, T, H, W, 8, D, FAKE, FAKE, 0.0, o, None, ws, wsb, None)

    assert fwd(q=None) == INVALID
    assert fwd(o=None) == INVALID
    assert fwd(W=-3) == INVALID
    assert fwd(D=96) == UNSUP
    need = L.nabla_sparse_attn_workspace_grid(1, 2, 44, 76, 8)
    assert need == L.nabla_sparse_attn_workspace(1, S, 8, 2, 6, 10) > 0
    assert fwd(wsb=need - 1) == WS
    assert L.nabla_sparse_attn_workspace_grid(1, 0, 44, 76, 8) == 0


def test_natural_entry_points_validation(L):
    g = L.nabla_block_mask_natural

    def mask(q=FAKE, T=2, H=48, W=80, heads=8, D=128, dt=BF16, thr=0.9, ratio=-1.0, ws=FAKE,
             wsb=1 << 40):
        return g(q, FAKE, dt, 1, T, H, W, heads, D, None, thr, ratio, FAKE, FAKE, ws, wsb, None)

    assert mask(q=None) == INVALID
    assert mask(T=0) == INVALID
    assert mask(dt=7) == INVALID
    assert mask(ratio=math.nan) == INVALID
    assert mask(thr=-0.5) == INVALID
    assert mask(H=44) == UNSUP                    # partial patches: permute + the grid calls
    assert mask(W=76) == UNSUP
    assert mask(W=8 * 65536, heads=8, D=128) == UNSUP   # rows of a patch 2^32 bytes apart
    S = 2 * 6 * 10 * 64
    assert mask(wsb=L.nabla_block_mask_workspace(1, S, 8, 128) - 1) == WS
    f = L.nabla_sparse_attn_fwd_natural

    def fwd(q=FAKE, T=2, H=48, W=80, D=128, dt=BF16, o=FAKE, ws=FAKE, wsb=1 << 40):
        return f(q, FAKE, FAKE, dt, 1, T, H, W, 8, D, FAKE, FAKE, 0.0, o, None, ws, wsb, None)

    assert fwd(q=None) == INVALID
    assert fwd(o=None) == INVALID
    assert fwd(T=-1) == INVALID
    assert fwd(dt=5) == INVALID
    assert fwd(H=20) == UNSUP
    assert fwd(D=96) == UNSUP
    need = L.nabla_sparse_attn_workspace_grid(1, 2, 48, 80, 8)
    assert need > 0
    assert fwd(wsb=need - 1) == WS


def test_sparse_attn_noalloc_validation(L):
    """The no-allocation forward validates like nabla_sparse_attn_fwd, and rejects shapes whose
    schedule does not fit its static 1 MiB scratch, all before touching the GPU."""
    f = L.nabla_sparse_attn_fwd_noalloc

    def call(q=FAKE, o=FAKE, B=1, S=61440, heads=16, D=128, tiles=(16, 6, 10), dt=BF16,
             scale=0.0):
        return f(q, FAKE, FAKE, dt, B, S, heads, D, FAKE, FAKE, scale, *tiles, o, None)

    assert call(q=None) == INVALID
    assert call(o=None) == INVALID
    assert call(dt=9) == INVALID
    assert call(S=1000) == INVALID
    assert call(scale=math.nan) == INVALID
    assert call(tiles=(16, 6, 9)) == INVALID
    assert call(D=96) == UNSUP
    # 546 (b, head) slices of the 720p tile grid: 546 * 240 groups > 131 008
    assert L.nabla_sparse_attn_workspace(546, 61440, 1, 16, 6, 10) > (1 << 20)
    assert call(B=546, heads=1) == WS
    assert L.nabla_sparse_attn_workspace(1, 61440, 545, 16, 6, 10) <= (1 << 20)
    # unknown grid (groups of 4 consecutive blocks): 33 sequences of 4096 blocks = 33 792 groups
    # fit, 33 * 4 = 132 sequences do not
    assert L.nabla_sparse_attn_workspace(132, 4096 * 64, 1, 0, 0, 0) > (1 << 20)
    assert call(B=132, S=4096 * 64, heads=1, tiles=(0, 0, 0)) == WS


def test_sparse_attn_workspace_size(L):
    # 720p tile grid 16 x 6 x 10: 8 * 6 * 5 = 240 groups per head
    ng = 16 * 240
    rnd = lambda x: (x + 255) // 256 * 256
    assert L.nabla_sparse_attn_workspace(1, 61440, 16, 16, 6, 10) == 256 + 2 * rnd(4 * ng)
    # unknown grid: groups of 4 consecutive blocks
    assert L.nabla_sparse_attn_workspace(2, 64 * 10, 3, 0, 0, 0) == 256 + 2 * rnd(4 * 2 * 3 * 3)
    assert L.nabla_sparse_attn_workspace(1, 61440, 16, 16, 6, 9) == 0   # grid != S/64
    assert L.nabla_sparse_attn_workspace(1, 100, 16, 0, 0, 0) == 0


def test_sparse_attn_validation(L):
    f = L.nabla_sparse_attn_fwd

    def call(q=FAKE, dt=BF16, B=1, S=8192, h=8, D=128, kv_nb=FAKE, scale=0.0, o=FAKE,
             tiles=(8, 4, 4), ws=FAKE, wsb=1 << 40):
        return f(q, FAKE, FAKE, dt, B, S, h, D, kv_nb, FAKE, scale, *tiles, o, ws, wsb, None)

    assert call(q=None) == INVALID
    assert call(o=None) == INVALID
    assert call(kv_nb=None) == INVALID
    assert call(S=100) == INVALID
    assert call(scale=math.nan) == INVALID
    assert call(tiles=(8, 4, 3)) == INVALID      # grid does not multiply to S/64
    assert call(tiles=(0, 4, 4)) == INVALID
    assert call(tiles=(-8, -4, 4)) == INVALID
    assert call(D=32) == UNSUP
    assert call(D=256) == UNSUP
    assert call(S=64 * 4097, tiles=(0, 0, 0)) == UNSUP
    assert call(ws=None) == WS
    assert call(wsb=L.nabla_sparse_attn_workspace(1, 8192, 8, 8, 4, 4) - 1) == WS


def test_sparse_attn_fwd_lse_validation(L):
    f = L.nabla_sparse_attn_fwd_lse

    def call(q=FAKE, o=FAKE, lse=FAKE, S=8192, D=128, ws=FAKE, wsb=1 << 40):
        return f(q, FAKE, FAKE, BF16, 1, S, 8, D, FAKE, FAKE, 0.0, 8, 4, 4, o, lse, ws, wsb, None)

    assert call(q=None) == INVALID
    assert call(o=None) == INVALID
    assert call(S=100) == INVALID
    assert call(D=96) == UNSUP
    assert call(ws=None) == WS
    assert call(lse=None, ws=None) == WS   # lse NULL: the plain forward's checks


def test_sparse_attn_bwd_workspace_size(L):
    rnd = lambda x: (x + 255) // 256 * 256
    bh, S, nb = 16, 61440, 960
    want = rnd(4 * bh * S) + rnd(4 * bh * nb) + rnd(4 * bh * nb * nb) + rnd(bh * nb * nb) + \
        2 * rnd(4 * bh * nb)
    assert L.nabla_sparse_attn_bwd_workspace(1, S, 16) == want
    assert L.nabla_sparse_attn_bwd_workspace(1, 100, 16) == 0
    assert L.nabla_sparse_attn_bwd_workspace(1, 64 * 4097, 1) == 0
    assert L.nabla_sparse_attn_bwd_workspace(0, 64, 1) == 0


def test_sparse_attn_bwd_validation(L):
    f = L.nabla_sparse_attn_bwd

    def call(q=FAKE, o=FAKE, dout=FAKE, lse=FAKE, dt=BF16, B=1, S=8192, D=128, scale=0.0,
             dq=FAKE, dv=FAKE, ws=FAKE, wsb=1 << 40):
        return f(q, FAKE, FAKE, o, dout, lse, dt, B, S, 8, D, FAKE, FAKE, scale, dq, FAKE, dv,
                 ws, wsb, None)

    for kw in ({"q": None}, {"o": None}, {"dout": None}, {"lse": None}, {"dq": None},
               {"dv": None}, {"S": 100}, {"B": 0}, {"scale": math.nan}, {"dt": 5}):
        assert call(**kw) == INVALID, kw
    assert call(dt=FP32) == UNSUP
    assert call(D=96) == UNSUP
    assert call(S=64 * 4097) == UNSUP
    assert call(ws=None) == WS
    assert call(wsb=L.nabla_sparse_attn_bwd_workspace(1, 8192, 8) - 1) == WS
    g = L.nabla_sparse_attn_bwd_grid

    def gcall(T=2, H=12, W=20, q=FAKE, dt=BF16, D=128, ws=FAKE, wsb=1 << 40):
        return g(q, FAKE, FAKE, FAKE, FAKE, FAKE, dt, 1, T, H, W, 8, D, FAKE, FAKE, 0.0, FAKE,
                 FAKE, FAKE, ws, wsb, None)

    for kw in ({"T": 0}, {"H": 0}, {"W": -1}, {"q": None}):
        assert gcall(**kw) == INVALID, kw
    assert gcall(dt=FP32) == UNSUP
    assert gcall(D=96) == UNSUP
    S = 2 * 2 * 3 * 64  # 2 frames of 2 x 3 patches (12 x 20 latents)
    assert gcall(wsb=L.nabla_sparse_attn_bwd_workspace(1, S, 8) - 1) == WS


def test_quant_workspace_size(L):
    rnd = lambda x: (x + 255) // 256 * 256
    assert L.nabla_quant_qkv_workspace(1, 61440, 16, 128) == \
        rnd(4 * 16 * 960 * 128) + rnd(4 * 16 * 60 * 128)
    assert L.nabla_quant_qkv_workspace(2, 640, 3, 64) == rnd(4 * 6 * 10 * 64) + rnd(4 * 6 * 1 * 64)
    assert L.nabla_quant_qkv_workspace(1, 100, 16, 128) == 0
    assert L.nabla_sparse_attn_q8_workspace(1, 61440, 16, 16, 6, 10) == \
        L.nabla_sparse_attn_workspace(1, 61440, 16, 16, 6, 10)
    assert L.nabla_sparse_attn_q8_workspace(1, 61440, 16, 16, 6, 9) == 0


def test_quant_validation(L):
    f = L.nabla_quant_qkv

    def call(q=FAKE, v=FAKE, dt=BF16, S=8192, D=128, q8=FAKE, km=FAKE, ws=FAKE, wsb=1 << 40):
        return f(q, FAKE, v, dt, 1, S, 8, D, q8, FAKE, FAKE, FAKE, FAKE, FAKE, km, ws, wsb, None)

    assert call(q=None) == INVALID
    assert call(v=None) == INVALID
    assert call(q8=None) == INVALID
    assert call(km=None) == INVALID
    assert call(dt=7) == INVALID
    assert call(S=100) == INVALID
    assert call(D=96) == UNSUP
    assert call(ws=None) == WS
    assert call(wsb=L.nabla_quant_qkv_workspace(1, 8192, 8, 128) - 1) == WS
    g = L.nabla_quant_qkv_grid

    def gcall(T=2, H=12, W=20, q=FAKE, dt=BF16, D=128, wsb=1 << 40):
        return g(q, FAKE, FAKE, dt, 1, T, H, W, 8, D, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                 FAKE, wsb, None)

    for kw in ({"T": 0}, {"H": 0}, {"W": -2}, {"q": None}, {"dt": 7}):
        assert gcall(**kw) == INVALID, kw
    assert gcall(D=96) == UNSUP
    assert gcall(wsb=L.nabla_quant_qkv_workspace(1, 2 * 2 * 3 * 64, 8, 128) - 1) == WS
    n = L.nabla_quant_qkv_natural

    def ncall(T=2, H=48, W=80, wsb=1 << 40):
        return n(FAKE, FAKE, FAKE, BF16, 1, T, H, W, 8, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                 FAKE, FAKE, wsb, None)

    assert ncall(T=0) == INVALID
    assert ncall(H=44) == UNSUP
    # more than 4096 blocks in a sequence: the natural-order block addressing is not exact
    assert ncall(T=69, H=48, W=80) == UNSUP        # 69 * 60 = 4140 blocks
    assert ncall(T=1, H=8, W=8 * 4097) == UNSUP    # one row of 4097 patches
    assert ncall(T=68, wsb=L.nabla_quant_qkv_workspace(1, 68 * 48 * 80, 8, 128) - 1) == WS


def test_sparse_attn_q8_validation(L):
    f = L.nabla_sparse_attn_fwd_q8

    def call(q8=FAKE, v8=FAKE, S=8192, D=128, kv_nb=FAKE, scale=0.0, tiles=(8, 4, 4), o=FAKE,
             ws=FAKE, wsb=1 << 40):
        return f(q8, FAKE, FAKE, FAKE, v8, FAKE, 1, S, 8, D, kv_nb, FAKE, scale, *tiles, o, ws,
                 wsb, None)

    assert call(q8=None) == INVALID
    assert call(v8=None) == INVALID
    assert call(kv_nb=None) == INVALID
    assert call(o=None) == INVALID
    assert call(S=100) == INVALID
    assert call(scale=math.nan) == INVALID
    assert call(tiles=(8, 4, 3)) == INVALID
    assert call(D=32) == UNSUP
    assert call(S=64 * 4097, tiles=(0, 0, 0)) == UNSUP
    assert call(ws=None) == WS
    assert call(wsb=L.nabla_sparse_attn_q8_workspace(1, 8192, 8, 8, 4, 4) - 1) == WS
    g = L.nabla_sparse_attn_fwd_q8_grid

    def gcall(T=2, H=12, W=20, q8=FAKE, D=128, scale=0.0, wsb=1 << 40):
        return g(q8, FAKE, FAKE, FAKE, FAKE, FAKE, 1, T, H, W, 8, D, FAKE, FAKE, scale, FAKE,
                 FAKE, wsb, None)

    for kw in ({"T": 0}, {"W": 0}, {"q8": None}, {"scale": math.nan}):
        assert gcall(**kw) == INVALID, kw
    assert gcall(D=32) == UNSUP
    assert gcall(wsb=L.nabla_sparse_attn_q8_workspace(1, 2 * 2 * 3 * 64, 8, 2, 2, 3) - 1) == WS


def test_permute_and_sta_validation(L):
    p = L.nabla_fractal_permute
    assert p(None, FAKE, BF16, 1, 2, 16, 16, 2, 64, 0, None) == INVALID
    assert p(FAKE, FAKE, BF16, 1, 2, 12, 0, 2, 64, 0, None) == INVALID    # W < 1
    assert p(FAKE, FAKE, BF16, 0, 2, 12, 20, 2, 64, 0, None) == INVALID   # B < 1
    assert p(FAKE, FAKE, BF16, 1, 0, 16, 16, 2, 64, 0, None) == INVALID
    assert p(FAKE, FAKE, BF16, 1, 2, 16, 16, 1, 2, 0, None) == UNSUP      # 4-byte rows
    assert p(FAKE, FAKE, BF16, 1, 16384, 256, 256, 1, 64, 0, None) == UNSUP  # 2^24 patches
    s = L.nabla_sta_mask
    assert s(None, 2, 2, 2, 1, 1, 1, None) == INVALID
    assert s(FAKE, 2, 0, 2, 1, 1, 1, None) == INVALID
    assert s(FAKE, 2, 2, 2, -1, 1, 1, None) == INVALID


def test_binding_has_no_cpu_path():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 128, 1, 64)
    with pytest.raises(TypeError):
        nabla.nabla_block_mask(q, q, None, 0.9)
    with pytest.raises(TypeError):
        nabla.nabla_fractal_permute(torch.zeros(1, 1, 8, 8, 1, 64))
    kv = torch.zeros(1, 1, 2, dtype=torch.int32)
    with pytest.raises(ValueError):
        nabla.nabla_sparse_attn_fwd(q, q, q, kv, kv, causal=True)
    with pytest.raises(TypeError):
        nabla.nabla_sparse_attn_fwd(q, q, q, kv, kv)
    lse = torch.zeros(1, 1, 128)
    with pytest.raises(TypeError):
        nabla.nabla_sparse_attn_bwd(q, q, q, q, q, lse, kv, kv)
