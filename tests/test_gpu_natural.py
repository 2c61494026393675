"""The natural-order entry points: the fractal permute folded into the kernels' addressing.

nabla_block_mask_natural takes q, k as [B, T, H, W, heads, D] (H, W multiples of 8) and
must give the oracle estimator's lists on the permuted q, k. Lists are compared bit for
bit outside the cut's rounding band, and must be exactly nabla_block_mask's lists on the
GPU permute. nabla_sparse_attn_fwd_natural must give:
  * o in natural order within max-abs 2e-2 and mean-abs 2e-3 of the oracle's attention;
  * o bit for bit equal to the inverse permute of nabla_sparse_attn_fwd_lse's output on
    the permuted inputs (the same kernel arithmetic on the same rows);
  * the same lse.
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


def to_np(t):
    return t.float().cpu().numpy()


def lists_vs_oracle(g_nb, g_inds, o, thr, band_fn, label):
    """Bit-exact lists outside the oracle's rounding band of the cut; at most 1 band row off."""
    g_nb, o_nb = g_nb.reshape(-1), o["kv_nb"].reshape(-1)
    nb = g_inds.shape[-1]
    g_inds, o_inds = g_inds.reshape(-1, nb), o["kv_inds"].reshape(-1, nb)
    band = band_fn(o["diag"], thr).reshape(-1) if thr is not None else np.zeros(g_nb.size, bool)
    off = 0
    for r in range(g_nb.size):
        n = int(o_nb[r])
        same = int(g_nb[r]) == n and np.array_equal(g_inds[r, :n], o_inds[r, :n])
        if band[r]:
            off += not same
            continue
        assert same, "%s: row %d differs (gpu n=%d, oracle n=%d)" % (label, r, g_nb[r], n)
    say("[%s] rows %d, band rows %d, off in band %d" % (label, g_nb.size, int(band.sum()), off))
    assert off <= 1, label


def same_lists(a_nb, a_inds, b_nb, b_inds, label):
    """The used part of every row is identical (the rest of a row is unspecified)."""
    a_nb, b_nb = a_nb.cpu().numpy().reshape(-1), b_nb.cpu().numpy().reshape(-1)
    nb = a_inds.shape[-1]
    a_inds, b_inds = a_inds.cpu().numpy().reshape(-1, nb), b_inds.cpu().numpy().reshape(-1, nb)
    assert np.array_equal(a_nb, b_nb), label
    for r in range(a_nb.size):
        n = int(a_nb[r])
        assert np.array_equal(a_inds[r, :n], b_inds[r, :n]), "%s row %d" % (label, r)


def natural_inputs(shape, dt, seed, dev):
    rng = np.random.default_rng(seed)
    xs = [rng.standard_normal(shape).astype(np.float32) for _ in range(3)]
    g = [torch.from_numpy(x).to(dt).to(dev) for x in xs]
    return g, [to_np(t) for t in g]  # the oracle sees the values the GPU holds


def run_both(orc, dev, g, vals, tiles, sta_win, thr, ratio):
    """Natural calls, the permuted calls, and the oracle on the permuted values."""
    B, T, H, W, heads, D = g[0].shape
    sta_g = None if sta_win is None else nabla.nabla_sta_mask(tiles, sta_win, dev)
    nb_n, inds_n = nabla.nabla_block_mask_natural(g[0], g[1], sta_g, thr, topk_ratio=ratio)
    lse_n = torch.empty((B, heads, T * H * W), dtype=torch.float32, device=dev)
    o_n = nabla.nabla_sparse_attn_fwd_natural(*g, nb_n, inds_n, lse=lse_n)
    qf, kf, vf = (nabla.nabla_fractal_permute(t) for t in g)
    nb_f, inds_f = nabla.nabla_block_mask(qf, kf, sta_g, thr, topk_ratio=ratio)
    lse_f = torch.empty_like(lse_n)
    o_f = nabla.nabla_sparse_attn_fwd(qf, kf, vf, nb_f, inds_f, tiles=tiles, lse=lse_f)
    o_fn = nabla.nabla_fractal_permute(o_f, grid=(T, H, W), inverse=True)
    torch.cuda.synchronize()
    same_lists(nb_n, inds_n, nb_f, inds_f, "natural vs permuted lists")
    assert torch.equal(o_n, o_fn), "natural o differs from the permuted path's"
    assert torch.equal(lse_n, lse_f), "natural lse differs from the permuted path's"
    frac = [orc.fractal_permute(x) for x in vals]
    return dict(nb=nb_n, inds=inds_n, o=o_n, frac=frac)


@pytest.mark.parametrize("shape,dt,ratio,seed", [
    ((1, 2, 16, 16, 2, 64), torch.float32, None, 91),
    ((2, 3, 24, 40, 3, 128), torch.bfloat16, None, 92),
    ((1, 4, 16, 24, 2, 128), torch.bfloat16, 0.3, 93),
    ((2, 2, 8, 56, 1, 64), torch.float32, 0.5, 94),
])
def test_natural_full_parity(orc, dev, shape, dt, ratio, seed):
    B, T, H, W, heads, D = shape
    tiles = (T, H // 8, W // 8)
    sta_win, thr = (1, 1, 1), 0.9
    say("[natural] shape", shape, dt, "topk", ratio, "seed", seed)
    g, vals = natural_inputs(shape, dt, seed, dev)
    r = run_both(orc, dev, g, vals, tiles, sta_win, thr, ratio)
    sta_o = orc.sta_mask(*tiles, *sta_win)
    if ratio is None:
        o = orc.block_mask(r["frac"][0], r["frac"][1], sta_o, thr)
        lists_vs_oracle(r["nb"].cpu().numpy(), r["inds"].cpu().numpy(), o, thr, orc.band_rows,
                        "natural lists")
    else:
        o = orc.block_mask_topk(r["frac"][0], r["frac"][1], sta_o, ratio)
        lists_vs_oracle(r["nb"].cpu().numpy(), r["inds"].cpu().numpy(), o, None, None,
                        "natural top-k lists")
    g_nb, g_inds = r["nb"].cpu().numpy(), r["inds"].cpu().numpy()
    ids, oo = orc.attention(*r["frac"], g_nb, g_inds)
    S = T * H * W
    want = orc.fractal_permute(orc.rows_to_tokens(oo, ids, B, S, heads, D), inverse=True,
                               grid=(T, H, W))
    err = np.abs(to_np(r["o"]).astype(np.float64) - want)
    say("[natural attn] max-abs %.3e mean-abs %.3e" % (err.max(), err.mean()))
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


def test_natural_720p(orc, dev):
    w = synth.WORKLOADS["720p"]
    say("[natural 720p]", w.describe())
    q, k, v = synth.make_qkv(w)
    g = [torch.from_numpy(a).to(torch.bfloat16).to(dev) for a in (q, k, v)]
    vals = [to_np(t) for t in g]
    r = run_both(orc, dev, g, vals, w.tiles, w.sta, w.thr, None)
    # sampled rows against the oracle, read back from natural order
    g_nb, g_inds = r["nb"].cpu().numpy(), r["inds"].cpu().numpy()
    rng = np.random.default_rng(95)
    nb = w.nb
    ids = np.sort(rng.choice(w.B * w.heads * nb, size=24, replace=False))
    rid, oo = orc.attention(*r["frac"], g_nb, g_inds, row_ids=ids)
    fr = orc.fractal_permute(to_np(r["o"]))  # o moved to fractal order on the CPU
    sel = []
    for rr in rid:
        b, rem = divmod(int(rr), w.heads * nb)
        h, i = divmod(rem, nb)
        sel.append(fr[b, 64 * i:64 * (i + 1), h, :])
    err = np.abs(np.stack(sel).astype(np.float64) - oo)
    say("[natural 720p attn] max-abs %.3e mean-abs %.3e" % (err.max(), err.mean()))
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


def test_natural_rejects_partial_patches(dev):
    x = torch.zeros((1, 2, 12, 16, 1, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        nabla.nabla_block_mask_natural(x, x)
    L = nabla.lib()
    st = L.nabla_block_mask_natural(nabla._p(x), nabla._p(x), 1, 1, 2, 12, 16, 1, 64, None,
                                    0.9, -1.0, nabla._p(x), nabla._p(x), nabla._p(x), 1 << 20,
                                    None)
    assert nabla.STATUS[st] == "NABLA_ERR_UNSUPPORTED"


@pytest.mark.parametrize("shape,dt,seed", [((2, 3, 24, 40, 3, 128), torch.bfloat16, 96),
                                           ((1, 2, 16, 16, 2, 64), torch.float32, 97)])
def test_natural_quantized(orc, dev, shape, dt, seed):
    """nabla_quant_qkv on natural q, k, v: the oracle's codes (bit-exact) and those of the
    permuted call; nabla_sparse_attn_fwd_q8_natural: the permuted call's o, inverse-permuted."""
    B, T, H, W, heads, D = shape
    tiles = (T, H // 8, W // 8)
    say("[natural q8] shape", shape, dt, "seed", seed)
    g, vals = natural_inputs(shape, dt, seed, dev)
    qz_n = nabla.nabla_quant_qkv(*g)
    qf = [nabla.nabla_fractal_permute(t) for t in g]
    qz_f = nabla.nabla_quant_qkv(*qf)
    sta = nabla.nabla_sta_mask(tiles, (1, 1, 1), dev)
    kv_nb, kv_inds = nabla.nabla_block_mask(qf[0], qf[1], sta, 0.9)
    o_n = nabla.nabla_sparse_attn_fwd_q8(qz_n, kv_nb, kv_inds, natural=(T, H, W))
    o_f = nabla.nabla_sparse_attn_fwd_q8(qz_f, kv_nb, kv_inds, tiles=tiles)
    o_fn = nabla.nabla_fractal_permute(o_f, grid=(T, H, W), inverse=True)
    torch.cuda.synchronize()
    oz = orc.quant_qkv(*[orc.fractal_permute(x) for x in vals])
    for gk, okey in (("q8", "q8"), ("q_scale", "qs"), ("k8", "k8"), ("k_scale", "ks"),
                     ("v8", "v8"), ("v_scale", "vs"), ("k_mean", "km")):
        a = qz_n[gk].cpu().numpy()
        assert np.array_equal(a.view(np.uint8), oz[okey].view(np.uint8)), gk
        assert torch.equal(qz_n[gk], qz_f[gk]), gk
    assert o_n.shape == (B, T, H, W, heads, D)
    assert torch.equal(o_n, o_fn), "natural q8 o differs from the permuted path's"
