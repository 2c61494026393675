"""Parity of the quantized variant (INT8 Q and K per block, FP8 e4m3 V per channel and
FP8 weights) with the CPU oracle, through the C ABI.

The quantizer's codes and scales must equal the oracle's bit for bit (fixed rounding
and summation order on both sides).  The attention is compared with the oracle's
attention on the same codes.  Both round every weight to e4m3, but against different
references (the oracle against the row maximum m, the kernel against a reference up to
log 4 below it), so the two weight sets are rounded on different grids.

Tolerance, derived from that rounding.  In the normal range an e4m3 rounding changes a
weight by at most 2^-4 of itself, so the two weights of a key differ by at most 2^-3 of
the exact weight P_c = exp(z_c - m).  To first order the normalized average then moves
by at most 2^-3 * sum_c P_c |v_c - o| / sum_c P_c <= 2^-3 * sigma, sigma the
P-weighted standard deviation of v in that channel.  Weights below e4m3's normal range
(P < 2^-6 / 112 on the kernel's side) are rounded with an absolute error of at most
2^-10 / 112 of the row's largest weight, at most (n_small * 1.1e-5 / sum P) * max|v - o|
in o.  The bf16 output and fp32 sums add 2^-8 |o|.  Every element must lie within 1.1x
that bound (the factor covers second-order terms), and the mean error must stay below
3e-3 (the rounding errors are independent from key to key and average out; measured
~2e-3).  A wrong index, scale or transpose moves o by about sigma itself, 8x the bound.
The lists always come from the oracle or the host, never from the HIP path.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_fractal_amd as nabla
from block_sparse_attention_fractal_amd import synth

pytestmark = pytest.mark.gpu

MEAN_ABS = 3e-3
QUANT_KEYS = ("q8", "q_scale", "k8", "k_scale", "v8", "v_scale", "k_mean")
ORC_KEYS = ("q8", "qs", "k8", "ks", "v8", "vs", "km")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


_CACHE = {}


def case(name, orc, dev):
    """Fractal-ordered inputs of a named workload (oracle arrays and GPU tensors), the GPU's
    and the oracle's codes, and the oracle's kv lists."""
    if name in _CACHE:
        return _CACHE[name]
    _CACHE.clear()
    w = synth.WORKLOADS[name]
    say("[q8 case] generating", w.describe())
    q, k, v = synth.make_qkv(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    frac = {n: orc.fractal_permute(a).reshape(w.B, w.S, w.heads, w.D)
            for n, a in (("q", q), ("k", k), ("v", v))}
    del q, k, v
    g = {n: torch.from_numpy(a).to(tdt).to(dev) for n, a in frac.items()}
    say("[q8 case] quantizing on the GPU")
    gz = nabla.nabla_quant_qkv(g["q"], g["k"], g["v"])
    torch.cuda.synchronize()
    say("[q8 case] oracle quantizer")
    oz = orc.quant_qkv(frac["q"], frac["k"], frac["v"])
    say("[q8 case] oracle lists")
    sta = None if w.sta is None else orc.sta_mask(*w.tiles, *w.sta)
    m = orc.block_mask(frac["q"], frac["k"], sta, w.thr)
    c = dict(w=w, frac=frac, g=g, gz=gz, oz=oz, kv_nb=m["kv_nb"], kv_inds=m["kv_inds"])
    _CACHE[name] = c
    return c


def q8_bound(orc, oz, kv_nb, kv_inds, row_ids, o, scale=0.0, valid=None):
    """Per-element bound [len(row_ids), 64, D] on |o_kernel - o_oracle| (module docstring).
    valid: bool [S] of a padded layout (padding positions are never keys), or None."""
    q8, k8 = oz["q8"], oz["k8"]
    B, heads, nb, _, D = q8.shape
    if not scale or scale <= 0:
        scale = 1.0 / np.sqrt(D)
    vdec = orc.fp8_e4m3_value(oz["v8"]) * oz["vs"][:, :, None, :, None]   # [B,h,nb,D,64]
    out = np.empty(o.shape)
    for n, rid in enumerate(row_ids):
        bh, i = divmod(int(rid), nb)
        b, h = divmod(bh, heads)
        cnt = int(kv_nb[b, h, i])
        if cnt == 0:
            out[n] = 1e-6
            continue
        blocks = kv_inds[b, h, i, :cnt]
        kk = k8[b, h, blocks].reshape(-1, D).astype(np.int64)             # [keys, D]
        dots = q8[b, h, i].astype(np.int64) @ kk.T                          # [64, keys]
        z = scale * float(oz["qs"][b, h, i]) * (dots * np.repeat(oz["ks"][b, h, blocks], 64))
        if valid is not None:
            keys = (64 * blocks[:, None] + np.arange(64)[None, :]).ravel()
            z = np.where(valid[keys][None, :], z, -np.inf)
        P = np.exp(z - z.max(axis=1, keepdims=True))
        sp = P.sum(axis=1, keepdims=True)
        v = vdec[b, h, blocks].transpose(0, 2, 1).reshape(-1, D)            # [keys, D]
        ev2 = (P @ (v * v)) / sp
        sigma = np.sqrt(np.maximum(ev2 - o[n] ** 2, 0.0))
        nsmall = (P < 2.0 ** -6 / 112).sum(axis=1, keepdims=True)
        spread = np.abs(v).max(axis=0)[None, :] + np.abs(o[n])
        out[n] = 1.1 * (2.0 ** -3 * sigma + nsmall * 1.1e-5 * spread / sp + 2.0 ** -8 * np.abs(o[n])) + 1e-5
    return out


def check(got, want, bound, label, mean_abs=MEAN_ABS):
    err = np.abs(got.astype(np.float64) - want)
    ratio = err / bound
    say("[%s] max-abs %.3e mean-abs %.3e over %d values (mean |o| %.3e); max err/bound %.3f"
        % (label, err.max(), err.mean(), err.size, np.abs(want).mean(), ratio.max()))
    assert ratio.max() <= 1.0 and err.mean() <= mean_abs, label


def rows_of(out, ids, w):
    got = out.float().cpu().numpy()
    nb = w.nb
    sel = []
    for rr in ids:
        b, rem = divmod(int(rr), w.heads * nb)
        h, i = divmod(rem, nb)
        sel.append(got[b, 64 * i:64 * (i + 1), h, :])
    return np.stack(sel)


@pytest.mark.parametrize("name", ["tiny", "small", "720p"])
def test_quant_bit_exact(orc, dev, name):
    c = case(name, orc, dev)
    say("[q8 quant]", name)
    for gk, ok in zip(QUANT_KEYS, ORC_KEYS):
        got = c["gz"][gk].cpu().numpy()
        want = c["oz"][ok]
        assert got.shape == want.shape, gk
        if got.dtype == np.float32:
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), gk
        else:
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), gk


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_q8_attention_full_parity(orc, dev, name):
    c = case(name, orc, dev)
    w = c["w"]
    say("[q8 attn-full]", name)
    out = nabla.nabla_sparse_attn_fwd_q8(c["gz"], torch.from_numpy(c["kv_nb"]).to(dev),
                                         torch.from_numpy(c["kv_inds"]).to(dev), tiles=w.tiles)
    torch.cuda.synchronize()
    ids, oo = orc.attention_q8(c["oz"], c["kv_nb"], c["kv_inds"])
    bound = q8_bound(orc, c["oz"], c["kv_nb"], c["kv_inds"], ids, oo)
    check(rows_of(out, ids, w), oo, bound, "%s q8 attn" % name)


@pytest.mark.parametrize("name", ["720p", "long"])
def test_q8_attention_sampled_parity(orc, dev, name):
    """The bench's launch configuration (full workload, tile grid known), sampled rows."""
    c = case(name, orc, dev)
    w = c["w"]
    say("[q8 attn-sampled]", name)
    out = nabla.nabla_sparse_attn_fwd_q8(c["gz"], torch.from_numpy(c["kv_nb"]).to(dev),
                                         torch.from_numpy(c["kv_inds"]).to(dev), tiles=w.tiles)
    torch.cuda.synchronize()
    rng = np.random.default_rng(21)
    kv_nb = c["kv_nb"]
    ids = []
    for b in range(w.B):
        for h in range(w.heads):
            row = kv_nb[b, h]
            pick = {0, w.nb - 1, int(np.argmin(row)), int(np.argmax(row))}
            ids += [(b * w.heads + h) * w.nb + i for i in sorted(pick)]
    ids = np.array(ids, np.int64)
    ids = ids[rng.choice(ids.size, size=min(ids.size, 40), replace=False)]
    rid, oo = orc.attention_q8(c["oz"], kv_nb, c["kv_inds"], row_ids=ids)
    bound = q8_bound(orc, c["oz"], kv_nb, c["kv_inds"], rid, oo)
    check(rows_of(out, rid, w), oo, bound, "%s q8 attn sampled" % name)


def test_q8_against_unquantized_attention(orc, dev):
    """The quantized output stays close to the plain attention on the unquantized inputs."""
    c = case("small", orc, dev)
    w = c["w"]
    out = nabla.nabla_sparse_attn_fwd_q8(c["gz"], torch.from_numpy(c["kv_nb"]).to(dev),
                                         torch.from_numpy(c["kv_inds"]).to(dev), tiles=w.tiles)
    torch.cuda.synchronize()
    ids, oo = orc.attention(c["frac"]["q"], c["frac"]["k"], c["frac"]["v"], c["kv_nb"],
                            c["kv_inds"])
    want = orc.rows_to_tokens(oo, ids, w.B, w.S, w.heads, w.D)
    got = out.float().cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    cos = (got * want).sum() / np.sqrt((got * got).sum() * (want * want).sum())
    say("[q8 vs unquantized] relative L2 %.4f cosine %.6f" % (rel, cos))
    assert cos > 0.995 and rel < 0.1


def test_q8_random_lists_and_edges(orc, dev):
    """Host lists: empty rows (o = 0), single blocks, full rows, any order; D = 64 and 128,
    fp32 and bf16 inputs, known and unknown tile grids, an explicit scale."""
    rng = np.random.default_rng(22)
    for D, dtype, tiles, scale in ((128, torch.bfloat16, (5, 1, 4), None),
                                   (64, torch.bfloat16, None, None),
                                   (64, torch.float32, (1, 4, 5), 0.2),
                                   (128, torch.bfloat16, (5, 2, 2), None)):
        B, S, h = 2, 1280, 3
        nb = S // 64
        say("[q8 random] D", D, dtype, "tiles", tiles, "scale", scale)
        q, k, v = (rng.standard_normal((B, S, h, D)).astype(np.float32) for _ in range(3))
        if dtype == torch.bfloat16:
            q, k, v = synth.round_bf16(q), synth.round_bf16(k), synth.round_bf16(v)
        kv_nb, kv_inds = synth.random_lists(rng, B, h, nb, 0.3)
        kv_nb[0, 0, 0] = 0
        kv_nb[0, 1, 3] = 1
        kv_nb[1, 2, 5] = nb
        kv_inds[1, 2, 5] = rng.permutation(nb)
        kv_inds[0, 2, 7, :kv_nb[0, 2, 7]] = kv_inds[0, 2, 7, :kv_nb[0, 2, 7]][::-1].copy()
        g = [torch.from_numpy(a).to(dtype).to(dev) for a in (q, k, v)]
        gz = nabla.nabla_quant_qkv(*g)
        out = nabla.nabla_sparse_attn_fwd_q8(gz, torch.from_numpy(kv_nb).to(dev),
                                             torch.from_numpy(kv_inds).to(dev), scale=scale,
                                             tiles=tiles)
        torch.cuda.synchronize()
        oz = orc.quant_qkv(q, k, v)
        for gk, ok in zip(QUANT_KEYS, ORC_KEYS):
            gv = gz[gk].cpu().numpy()
            assert np.array_equal(gv.view(np.uint8), oz[ok].view(np.uint8)), gk
        sc = 0.0 if scale is None else scale
        ids, oo = orc.attention_q8(oz, kv_nb, kv_inds, scale=sc)
        got = out.float().cpu().numpy()
        assert np.all(got[0, 0:64, 0] == 0)
        nbk = S // 64
        sel = np.stack([got[r // (h * nbk), 64 * (r % nbk):64 * (r % nbk + 1), (r // nbk) % h]
                        for r in ids])
        check(sel, oo, q8_bound(orc, oz, kv_nb, kv_inds, ids, oo, sc),
              "q8 random D=%d %s tiles=%s" % (D, dtype, tiles))


def test_q8_run_twice_bitwise(orc, dev):
    c = case("small", orc, dev)
    w = c["w"]
    say("[q8 determinism]")
    gz2 = nabla.nabla_quant_qkv(c["g"]["q"], c["g"]["k"], c["g"]["v"])
    for key in QUANT_KEYS:
        assert torch.equal(gz2[key], c["gz"][key])
    lists = (torch.from_numpy(c["kv_nb"]).to(dev), torch.from_numpy(c["kv_inds"]).to(dev))
    o1 = nabla.nabla_sparse_attn_fwd_q8(c["gz"], *lists, tiles=w.tiles)
    o2 = nabla.nabla_sparse_attn_fwd_q8(c["gz"], *lists, tiles=w.tiles)
    assert torch.equal(o1, o2)
    o3 = nabla.nabla_sparse_attn_fwd_q8(c["gz"], *lists)  # other grouping, same result
    assert torch.equal(o1, o3)


# ---- padded fractal layouts (H or W not a multiple of 8): padding is not a token

@pytest.mark.parametrize("T,H,W,h,D,seed", [(2, 12, 20, 2, 128, 61), (1, 20, 28, 3, 64, 62)])
def test_q8_padded_quantizer_and_attention(orc, dev, T, H, W, h, D, seed):
    """The grid entry points on a padded layout whose padding positions hold a large value
    (7.0) that must be ignored: codes and scales bit-exact against oracle.quant_qkv(grid=...),
    attention within the e4m3 bound of oracle.attention_q8(grid=...) on every element."""
    rng = np.random.default_rng(seed)
    grid = (T, H, W)
    nat = [rng.standard_normal((1, T, H, W, h, D)).astype(np.float32) for _ in range(3)]
    valid = orc.token_valid(T, H, W)
    frac = []
    for a in nat:
        x = orc.fractal_permute(a)
        x[:, ~valid] = 7.0
        frac.append(torch.from_numpy(x).to(torch.bfloat16))
    S = frac[0].shape[1]
    nb = S // 64
    say("[q8 padded] T=%d H=%d W=%d heads=%d D=%d (S=%d)" % (T, H, W, h, D, S))
    gz = nabla.nabla_quant_qkv(*[t.to(dev) for t in frac], grid=grid)
    torch.cuda.synchronize()
    oz = orc.quant_qkv(*[t.float().numpy() for t in frac], grid=grid)
    for gk, ok in zip(QUANT_KEYS, ORC_KEYS):
        a = gz[gk].cpu().numpy()
        assert np.array_equal(a.view(np.uint8), oz[ok].view(np.uint8)), gk
    kv_nb, kv_inds = synth.random_lists(rng, 1, h, nb, 0.5)
    kv_nb[0, 0, 0] = 0
    kv_nb[0, h - 1, nb - 1] = nb
    o = nabla.nabla_sparse_attn_fwd_q8(gz, torch.from_numpy(kv_nb).to(dev),
                                       torch.from_numpy(kv_inds).to(dev), grid=grid)
    torch.cuda.synchronize()
    ids, want = orc.attention_q8(oz, kv_nb, kv_inds, grid=grid)
    gt = o.float().cpu().numpy()
    got = np.stack([gt[0, 64 * (int(r) % nb):64 * (int(r) % nb + 1), int(r) // nb] for r in ids])
    bound = q8_bound(orc, oz, kv_nb, kv_inds, ids, want, valid=valid)
    check(got, want, bound, "q8 padded")


def test_q8_grid_of_whole_patches_is_plain(orc, dev):
    """On a grid of whole patches the grid entry points give the plain calls' bits."""
    rng = np.random.default_rng(63)
    T, H, W, h, D = 2, 16, 8, 2, 128
    S = T * H * W
    g = [torch.from_numpy(rng.standard_normal((1, S, h, D)).astype(np.float32)).to(torch.bfloat16).to(dev)
         for _ in range(3)]
    za = nabla.nabla_quant_qkv(*g, grid=(T, H, W))
    zb = nabla.nabla_quant_qkv(*g)
    for n in QUANT_KEYS:
        assert torch.equal(za[n], zb[n]), n
    kv_nb, kv_inds = synth.random_lists(rng, 1, h, S // 64, 0.5)
    nb_t, inds_t = torch.from_numpy(kv_nb).to(dev), torch.from_numpy(kv_inds).to(dev)
    oa = nabla.nabla_sparse_attn_fwd_q8(za, nb_t, inds_t, grid=(T, H, W))
    ob = nabla.nabla_sparse_attn_fwd_q8(za, nb_t, inds_t, tiles=(T, H // 8, W // 8))
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
