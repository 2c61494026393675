"""Padded tile grids (H or W not multiples of 8) on the HIP path against the oracle.

The fractal layout pads each frame to whole 8 x 8 patches; padding positions are 0
and are not tokens: blocks average their tokens only, and padding is never a key.
Permute and lists are compared bit for bit; attention within max-abs 2e-2 and
mean-abs 2e-3 on the rows of real tokens (padding rows are dropped by the inverse
permute).  Grids of whole patches must give exactly the plain calls' results.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_fractal_amd as nabla
from block_sparse_attention_fractal_amd import synth

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


_CACHE = {}


def case(name, orc, dev):
    if name in _CACHE:
        return _CACHE[name]
    _CACHE.clear()
    w = synth.WORKLOADS[name]
    say("[grid case]", w.describe())
    q, k, v = synth.make_qkv(w)
    g = {n: torch.from_numpy(a).to(torch.bfloat16).to(dev) for n, a in (("q", q), ("k", k), ("v", v))}
    f = {n: orc.fractal_permute(a) for n, a in (("q", q), ("k", k), ("v", v))}
    c = dict(w=w, nat=dict(q=q, k=k, v=v), frac=f, gnat=g)
    _CACHE[name] = c
    return c


@pytest.mark.parametrize("T,H,W,dt", [(3, 44, 76, torch.bfloat16), (2, 13, 21, torch.float32),
                                      (1, 8, 9, torch.bfloat16), (2, 7, 8, torch.float32)])
def test_padded_permute_bit_exact(orc, dev, T, H, W, dt):
    rng = np.random.default_rng(81)
    x = rng.standard_normal((2, T, H, W, 2, 64)).astype(np.float32)
    gx = torch.from_numpy(x).to(dt).to(dev)
    xv = gx.float().cpu().numpy()
    y = nabla.nabla_fractal_permute(gx)
    torch.cuda.synchronize()
    want = orc.fractal_permute(xv)
    assert y.shape == want.shape
    assert np.array_equal(y.float().cpu().numpy(), want)  # padding rows 0 included
    back = nabla.nabla_fractal_permute(y, grid=(T, H, W), inverse=True)
    assert torch.equal(back, gx)


@pytest.mark.parametrize("ratio", [None, 0.25])
def test_padded_estimator_full_parity(orc, dev, ratio):
    c = case("small_pad", orc, dev)
    w = c["w"]
    qf = nabla.nabla_fractal_permute(c["gnat"]["q"])
    kf = nabla.nabla_fractal_permute(c["gnat"]["k"])
    sta = nabla.nabla_sta_mask(w.tiles, w.sta, dev)
    kv_nb, kv_inds = nabla.nabla_block_mask(qf, kf, sta, w.thr, topk_ratio=ratio,
                                            grid=(w.T, w.H, w.W))
    torch.cuda.synchronize()
    o = orc.block_mask_grid(c["frac"]["q"], c["frac"]["k"], (w.T, w.H, w.W),
                            orc.sta_mask(*w.tiles, *w.sta), w.thr, topk_ratio=ratio)
    g_nb, g_inds = kv_nb.cpu().numpy().reshape(-1), kv_inds.cpu().numpy().reshape(-1, w.nb)
    o_nb, o_inds = o["kv_nb"].reshape(-1), o["kv_inds"].reshape(-1, w.nb)
    for r in range(g_nb.size):
        n = int(o_nb[r])
        assert int(g_nb[r]) == n and np.array_equal(g_inds[r, :n], o_inds[r, :n]), r
    say("[padded estimator ratio=%s] %d rows bit-exact" % (ratio, g_nb.size))


def test_padded_attention_full_parity(orc, dev):
    c = case("small_pad", orc, dev)
    w = c["w"]
    qf, kf, vf = (nabla.nabla_fractal_permute(c["gnat"][n]) for n in ("q", "k", "v"))
    o_lists = orc.block_mask_grid(c["frac"]["q"], c["frac"]["k"], (w.T, w.H, w.W),
                                  orc.sta_mask(*w.tiles, *w.sta), w.thr)
    kv_nb = torch.from_numpy(o_lists["kv_nb"]).to(dev)
    kv_inds = torch.from_numpy(o_lists["kv_inds"]).to(dev)
    lse = torch.empty((w.B, w.heads, w.S), dtype=torch.float32, device=dev)
    out = nabla.nabla_sparse_attn_fwd(qf, kf, vf, kv_nb, kv_inds, grid=(w.T, w.H, w.W), lse=lse)
    torch.cuda.synchronize()
    ids, o = orc.attention_grid(c["frac"]["q"], c["frac"]["k"], c["frac"]["v"], (w.T, w.H, w.W),
                                o_lists["kv_nb"], o_lists["kv_inds"])
    want = orc.rows_to_tokens(o, ids, w.B, w.S, w.heads, w.D)
    got = out.float().cpu().numpy().astype(np.float64)
    valid = orc.token_valid(w.T, w.H, w.W)
    err = np.abs(got[:, valid] - want[:, valid])
    say("[padded attention] max %.3g mean %.3g over %d token rows" % (err.max(), err.mean(), valid.sum()))
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(lse.cpu().numpy()))
    # the natural-order output through the inverse permute holds exactly the token rows
    o_nat = nabla.nabla_fractal_permute(out, grid=(w.T, w.H, w.W), inverse=True)
    assert o_nat.shape[1:4] == (w.T, w.H, w.W)


def test_whole_patch_grid_equals_plain(orc, dev):
    """On a grid of whole patches the grid entry points give exactly the plain calls' results."""
    c = case("small", orc, dev)
    w = c["w"]
    qf, kf, vf = (nabla.nabla_fractal_permute(c["gnat"][n]) for n in ("q", "k", "v"))
    sta = nabla.nabla_sta_mask(w.tiles, w.sta, dev)
    a = nabla.nabla_block_mask(qf, kf, sta, w.thr)
    b = nabla.nabla_block_mask(qf, kf, sta, w.thr, grid=(w.T, w.H, w.W))
    assert torch.equal(a[0], b[0])
    live = torch.arange(w.nb, device=dev)[None, None, None, :] < a[0][..., None]  # the lists
    assert torch.equal(torch.where(live, a[1], 0), torch.where(live, b[1], 0))
    o1 = nabla.nabla_sparse_attn_fwd(qf, kf, vf, *a, tiles=w.tiles)
    o2 = nabla.nabla_sparse_attn_fwd(qf, kf, vf, *a, grid=(w.T, w.H, w.W))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_padded_720p_sampled(orc, dev):
    """A 720p-sized padded grid (16 x 44 x 76 latents: 6 x 10 patches per frame, the last row
    and column partial): lists bit-exact and attention within tolerance on sampled rows."""
    c = case("720p_pad", orc, dev)
    w = c["w"]
    qf, kf, vf = (nabla.nabla_fractal_permute(c["gnat"][n]) for n in ("q", "k", "v"))
    sta = nabla.nabla_sta_mask(w.tiles, w.sta, dev)
    kv_nb, kv_inds = nabla.nabla_block_mask(qf, kf, sta, w.thr, grid=(w.T, w.H, w.W))
    out = nabla.nabla_sparse_attn_fwd(qf, kf, vf, kv_nb, kv_inds, grid=(w.T, w.H, w.W))
    torch.cuda.synchronize()
    rng = np.random.default_rng(82)
    Tt, Ht, Wt = w.tiles
    ids = []
    for h in range(w.heads):
        # partial-patch blocks (last patch row / column) and random ones
        part = [i for i in range(w.nb) if (i // Wt) % Ht == Ht - 1 or i % Wt == Wt - 1]
        pick = set(rng.choice(part, 3, replace=False).tolist()) | set(rng.choice(w.nb, 3).tolist())
        ids += [h * w.nb + i for i in sorted(pick)]
    ids = np.array(ids, np.int64)
    o = orc.block_mask_grid(c["frac"]["q"], c["frac"]["k"], (w.T, w.H, w.W),
                            orc.sta_mask(*w.tiles, *w.sta), w.thr, row_ids=ids)
    g_nb = kv_nb.cpu().numpy().reshape(-1)
    g_inds = kv_inds.cpu().numpy().reshape(-1, w.nb)
    for n_, r in enumerate(ids):
        n = int(o["kv_nb"][n_])
        assert int(g_nb[r]) == n and np.array_equal(g_inds[r, :n], o["kv_inds"][n_, :n])
    _, oo = orc.attention_grid(c["frac"]["q"], c["frac"]["k"], c["frac"]["v"], (w.T, w.H, w.W),
                               kv_nb.cpu().numpy(), kv_inds.cpu().numpy(), row_ids=ids)
    got = out.float().cpu().numpy()
    valid = orc.token_valid(w.T, w.H, w.W)
    errs = []
    for n_, r in enumerate(ids):
        h, i = divmod(int(r), w.nb)
        vr = valid[64 * i:64 * (i + 1)]
        errs.append(np.abs(got[0, 64 * i:64 * (i + 1), h][vr] - oo[n_][vr]))
    e = np.concatenate([x.ravel() for x in errs])
    say("[padded 720p] %d sampled blocks: max %.3g mean %.3g" % (ids.size, e.max(), e.mean()))
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS
