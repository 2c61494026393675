"""Parity of the HIP path (through the C ABI) with the CPU oracle, on seeded inputs.

Integer outputs (fractal permutation, STA mask, kv_nb and the kv_inds sets)
must match bit for bit on every row.  Rows whose CDF lies within 1e-6 of the cut
("band" rows, where several selections are defensible) are counted and listed
for every run; both sides compute the softmax with one exp method and exact
fixed-point sums, so band rows must match as well.  The attention output (bf16
MFMA, fp32 accumulation) must stay within max-abs 2e-2 and mean-abs 2e-3 of
the fp64 oracle.  The lists are compared on every row of every workload (tiny,
small, 720p, the long clip and all fifteen runs of the 720p sparsity sweep) and
of row lengths that hit each column-group count of the selection kernel with a
partial last group;
the attention in full on tiny and small and on sampled query blocks (first and
last, fewest and most kept blocks, random) on the larger shapes.
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


def case(name, orc, dev, w=None):
    """Inputs of a workload (named, or given): natural numpy arrays, oracle fractal arrays, GPU
    tensors.  Workloads that draw the same tensors (the sweep's thr / STA runs) share them."""
    w = synth.WORKLOADS[name] if w is None else w
    key = (w.B, w.T, w.H, w.W, w.heads, w.D, w.dtype, w.gen, w.seed, w.sigma_f, w.sigma_n)
    if key in _CACHE:
        _CACHE[key] = _CACHE.pop(key)  # most recently used last
        return dict(_CACHE[key], w=w)
    while len(_CACHE) >= 2:  # keep the two most recent input sets (host fp32 + GPU bf16)
        _CACHE.pop(next(iter(_CACHE)))
    say("[case] generating", w.describe())
    q, k, v = synth.make_qkv(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = {n: torch.from_numpy(a).to(tdt).to(dev) for n, a in (("q", q), ("k", k), ("v", v))}
    f = {n: orc.fractal_permute(a).reshape(w.B, w.S, w.heads, w.D)
         for n, a in (("q", q), ("k", k), ("v", v))}
    c = dict(w=w, nat=dict(q=q, k=k, v=v), frac=f, gnat=g)
    _CACHE[key] = c
    return c


def to_np(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def sample_rows(kv_nb, rng, per_head=6):
    """Row ids per (b, h): first, last, fewest and most kept blocks, and random rows."""
    B, H, nb = kv_nb.shape
    ids = []
    for b in range(B):
        for h in range(H):
            row = kv_nb[b, h]
            pick = {0, nb - 1, int(np.argmin(row)), int(np.argmax(row))}
            pick |= set(rng.choice(nb, size=per_head, replace=False).tolist())
            ids += [(b * H + h) * nb + i for i in sorted(pick)]
    return np.array(ids, np.int64)


def rows_equal(g_nb, g_inds, o_nb, o_inds):
    """bool per row: equal kv_nb and equal kv_inds prefixes (both sides write them ascending)."""
    g_nb = g_nb.reshape(-1)
    o_nb = o_nb.reshape(-1)
    nb = g_inds.shape[-1]
    g_inds = g_inds.reshape(-1, nb)
    o_inds = o_inds.reshape(-1, nb)
    live = np.arange(nb)[None, :] < o_nb[:, None]
    return (g_nb == o_nb) & np.all((g_inds == o_inds) | ~live, axis=1)


def compare_lists(g_nb, g_inds, o_nb, o_inds, band, label, ids=None):
    """kv_nb and the kv_inds sets bit-exact on every row.  The band rows (CDF within 1e-6 of
    the cut) are counted and listed first; they must match too (one exp method and exact
    sums on both sides).  ids: the global row ids of sampled rows (None: rows in order)."""
    same = rows_equal(g_nb, g_inds, o_nb, o_inds)
    band = band.reshape(-1)
    rid = np.arange(same.size) if ids is None else np.asarray(ids)
    bad = np.flatnonzero(~same)
    say("[%s] rows=%d band rows=%d %s; differing rows=%d (in band %d)"
        % (label, same.size, int(band.sum()), rid[band][:32].tolist(), bad.size,
           int((~same & band).sum())))
    assert bad.size == 0, "%s: rows %s differ (band: %s)" % (label, rid[bad][:16].tolist(),
                                                             band[bad][:16].tolist())
    return int(band.sum())


# ------------------------------------------------------------------ permute + STA
@pytest.mark.parametrize("name", ["tiny", "small", "720p"])
def test_fractal_permute_bit_exact(orc, dev, name):
    c = case(name, orc, dev)
    w = c["w"]
    say("[permute]", name)
    for n in ("q", "k", "v"):
        y = nabla.nabla_fractal_permute(c["gnat"][n])
        torch.cuda.synchronize()
        want = c["frac"][n]
        got = to_np(y)
        assert got.shape == want.shape
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), n
        back = nabla.nabla_fractal_permute(y, grid=(w.T, w.H, w.W), inverse=True)
        assert torch.equal(back, c["gnat"][n])


@pytest.mark.parametrize("tiles,win", [((2, 2, 2), (1, 1, 1)), ((8, 4, 4), (1, 1, 1)),
                                       ((16, 6, 10), (2, 1, 1)), ((16, 6, 10), (1, 1, 1)),
                                       ((31, 6, 10), (2, 1, 1)), ((5, 3, 7), (0, 2, 1))])
def test_sta_mask_bit_exact(orc, dev, tiles, win):
    say("[sta]", tiles, win)
    got = nabla.nabla_sta_mask(tiles, win, dev).cpu().numpy()
    assert np.array_equal(got, orc.sta_mask(*tiles, *win))


# ------------------------------------------------------------------ estimator
def run_mask(c, orc, dev, thr, sta_win, rows=None, rng=None):
    w = c["w"]
    qf = nabla.nabla_fractal_permute(c["gnat"]["q"])
    kf = nabla.nabla_fractal_permute(c["gnat"]["k"])
    sta_g = None if sta_win is None else nabla.nabla_sta_mask(w.tiles, sta_win, dev)
    kv_nb, kv_inds = nabla.nabla_block_mask(qf, kf, sta_g, thr)
    torch.cuda.synchronize()
    g_nb, g_inds = kv_nb.cpu().numpy(), kv_inds.cpu().numpy()
    sta_o = None if sta_win is None else orc.sta_mask(*w.tiles, *sta_win)
    if rows == "all":
        o = orc.block_mask(c["frac"]["q"], c["frac"]["k"], sta_o, thr)
        band = orc.band_rows(o["diag"], thr)
        return (qf, kf), (g_nb, g_inds), (o["kv_nb"], o["kv_inds"]), band, None
    ids = sample_rows(g_nb, rng)
    o = orc.block_mask(c["frac"]["q"], c["frac"]["k"], sta_o, thr, row_ids=ids)
    band = orc.band_rows(o["diag"], thr)
    nb = w.nb
    return ((qf, kf), (g_nb.reshape(-1)[ids], g_inds.reshape(-1, nb)[ids]),
            (o["kv_nb"], o["kv_inds"]), band, ids)


@pytest.mark.parametrize("name,thr,sta", [
    ("tiny", 0.9, (1, 1, 1)), ("tiny", 0.9, None), ("tiny", 0.5, None), ("tiny", 0.0, None),
    ("tiny", 1.0, None), ("small", 0.9, (1, 1, 1)), ("small", 0.5, None), ("small", 0.95, (0, 0, 0)),
])
def test_block_mask_full_parity(orc, dev, name, thr, sta):
    c = case(name, orc, dev)
    say("[mask-full]", name, "thr", thr, "sta", sta)
    _, g, o, band, _ = run_mask(c, orc, dev, thr, sta, rows="all")
    compare_lists(*g, *o, band, "%s thr=%g sta=%s" % (name, thr, sta))
    if thr == 1.0:
        assert np.all(g[0] == c["w"].nb)


def test_block_mask_uniform_ties(orc, dev):
    """Q = 0: every score is exactly 0, so the order is decided by the index tie-break alone."""
    B, S, h, D = 1, 8192, 2, 128
    rng = np.random.default_rng(12)
    k = synth.round_bf16(rng.standard_normal((B, S, h, D)).astype(np.float32))
    q = np.zeros_like(k)
    gq = torch.zeros((B, S, h, D), dtype=torch.bfloat16, device=dev)
    gk = torch.from_numpy(k).to(torch.bfloat16).to(dev)
    for thr in (0.5, 0.7, 0.9, 0.95):
        say("[mask-ties] thr", thr)
        kv_nb, kv_inds = nabla.nabla_block_mask(gq, gk, None, thr)
        o = orc.block_mask(q, k, None, thr)
        compare_lists(kv_nb.cpu().numpy(), kv_inds.cpu().numpy(), o["kv_nb"], o["kv_inds"],
                      np.zeros(o["kv_nb"].shape, bool), "ties thr=%g" % thr)
        want = {0.5: 65, 0.7: 90, 0.9: 116, 0.95: 122}[thr]
        assert np.all(kv_nb.cpu().numpy() == want)


@pytest.mark.parametrize("nb", [960, 1100, 1880])
def test_block_mask_long_row_degenerate(orc, dev, nb):
    """The degenerate selections on rows of one wave (960 blocks) and of a pair of waves (1100
    and 1880 blocks): Q = 0 (every score 0: one histogram bin, the order decided by the index
    tie-break through the refinement passes), thr = 0 (only the arg-max and the band) and
    thr = 1 (every block), against the oracle on every row."""
    B, h, D = 1, 2, 128
    S = nb * 64
    rng = np.random.default_rng(40 + nb)
    k = synth.round_bf16(rng.standard_normal((B, S, h, D)).astype(np.float32))
    q = synth.round_bf16(rng.standard_normal((B, S, h, D)).astype(np.float32))
    ii = np.arange(nb)
    sta = (np.abs(ii[:, None] - ii[None, :]) <= 1).astype(np.uint8)
    gk = torch.from_numpy(k).to(torch.bfloat16).to(dev)
    gsta = torch.from_numpy(sta).to(dev)
    for label, qq, thr, st in (("ties", np.zeros_like(q), 0.9, None), ("thr0", q, 0.0, sta),
                               ("thr1", q, 1.0, None)):
        say("[mask-degenerate] nb", nb, label)
        gq = torch.from_numpy(qq).to(torch.bfloat16).to(dev)
        kv_nb, kv_inds = nabla.nabla_block_mask(gq, gk, None if st is None else gsta, thr)
        o = orc.block_mask(qq, k, st, thr)
        compare_lists(kv_nb.cpu().numpy(), kv_inds.cpu().numpy(), o["kv_nb"], o["kv_inds"],
                      orc.band_rows(o["diag"], thr), "degenerate nb=%d %s" % (nb, label))
        if label == "thr1":
            assert np.all(kv_nb.cpu().numpy() == nb)


def test_block_mask_long_rows_repeatable(orc, dev):
    """Rows of a pair of waves (1880 blocks) whose cut bins need refinement passes, five calls
    in a row: the lists are the same on every call (the waves' decisions come from shared LDS
    values around barriers).  Every kv block's tokens equal one of 8 vectors, so a row's
    scores take 8 values and each of them is held by about 235 blocks (ties broken by index)."""
    B, h, D, nb = 1, 4, 128, 1880
    S = nb * 64
    rng = np.random.default_rng(77)
    kvec = synth.round_bf16(rng.standard_normal((8, h, D)).astype(np.float32))
    k = np.ascontiguousarray(kvec[(np.arange(S) // 64) % 8][None])  # [1, S, h, D]
    q = synth.round_bf16(rng.standard_normal((B, S, h, D)).astype(np.float32))
    gq, gk = (torch.from_numpy(a).to(torch.bfloat16).to(dev) for a in (q, k))
    first = None
    for rep in range(5):
        kv_nb, kv_inds = nabla.nabla_block_mask(gq, gk, None, 0.9)
        g_nb, g_inds = kv_nb.cpu().numpy(), kv_inds.cpu().numpy()
        if first is None:
            first = (g_nb, g_inds)
            o = orc.block_mask(q, k, None, 0.9)
            compare_lists(g_nb, g_inds, o["kv_nb"], o["kv_inds"], orc.band_rows(o["diag"], 0.9),
                          "tied kv blocks nb=%d" % nb)
            continue
        same = rows_equal(g_nb, g_inds, *first)
        say("[mask-repeat] call", rep, "differing rows", int((~same).sum()))
        assert same.all(), "call %d: rows %s differ" % (rep, np.flatnonzero(~same)[:16].tolist())


# ------------------------------------------------------------------ attention
@pytest.mark.parametrize("nb,D,dtype,B,h", [
    (1, 128, "bf16", 1, 2),      # one column group, one block
    (65, 128, "bf16", 2, 2),     # 2 groups, the second holds one block; batch offset
    (300, 128, "bf16", 1, 2),    # 8 groups, eight rows per wave (two row quads on the matrix cores)
    (513, 128, "bf16", 1, 2),    # the shortest rows of the two-launch path: score tiles of one row / block
    (600, 128, "bf16", 1, 3),    # three heads: score tiles and selection rows of several heads
    (700, 128, "bf16", 2, 4),    # four heads, two batches: (b, head) offsets of the score buffer
    (897, 128, "bf16", 1, 2),    # 15 groups, the last holds one block
    (960, 128, "fp32", 1, 2),    # fp32 inputs, 15 groups
    (1000, 64, "bf16", 1, 2),    # 16 groups, D = 64 (q pooled by the pooling pass)
    (1024, 64, "bf16", 1, 6),    # six heads, D = 64, 16 full groups
    (1025, 128, "bf16", 1, 2),   # 32 groups over a pair of waves: the second wave holds one block
    (1857, 128, "bf16", 1, 2),   # 30 groups, 15 per wave of the pair
    (1921, 128, "fp32", 1, 2),   # 32 groups, fp32 inputs
    (2048, 64, "bf16", 2, 3),    # the longest rows of the two-launch path, D = 64, (b, head) offsets
    (2049, 128, "bf16", 1, 2),   # rows of more than 2048 blocks: one workgroup of eight waves per row
    (4096, 64, "fp32", 1, 1),    # the longest rows the estimator takes
])
def test_block_mask_row_lengths(orc, dev, nb, D, dtype, B, h):
    """Rows of every column-group count of the selection kernel, each with a partial last
    group, against the oracle estimator on every row (fractal-order call, band STA), with
    several head counts and batches on the two-launch path."""
    S = nb * 64
    rng = np.random.default_rng(1000 + nb)
    # a shared direction per head plus noise: scores spread, so the cut moves between rows
    base = rng.standard_normal((1, 1, h, D)).astype(np.float32)
    q = (rng.standard_normal((B, S, h, D)) + 2.0 * base).astype(np.float32)
    k = (rng.standard_normal((B, S, h, D)) + 1.5 * base * rng.standard_normal((B, S, h, 1))).astype(np.float32)
    if dtype == "bf16":
        q, k = synth.round_bf16(q), synth.round_bf16(k)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gq, gk = (torch.from_numpy(a).to(tdt).to(dev) for a in (q, k))
    ii = np.arange(nb)
    sta = (np.abs(ii[:, None] - ii[None, :]) <= 2).astype(np.uint8)
    for thr in (0.9, 0.5):
        say("[mask-rows] nb", nb, "D", D, dtype, "B", B, "heads", h, "thr", thr)
        kv_nb, kv_inds = nabla.nabla_block_mask(gq, gk, torch.from_numpy(sta).to(dev), thr)
        o = orc.block_mask(q, k, sta, thr)
        band = orc.band_rows(o["diag"], thr)
        compare_lists(kv_nb.cpu().numpy(), kv_inds.cpu().numpy(), o["kv_nb"], o["kv_inds"], band,
                      "rows nb=%d D=%d %s h=%d thr=%g" % (nb, D, dtype, h, thr))


def check_attention(got, want, label):
    err = np.abs(got.astype(np.float64) - want)
    say("[%s] max-abs %.3e mean-abs %.3e over %d values" % (label, err.max(), err.mean(), err.size))
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, label


@pytest.mark.parametrize("name,thr,sta", [("tiny", 0.9, (1, 1, 1)), ("tiny", 0.5, None),
                                          ("small", 0.9, (1, 1, 1))])
def test_attention_full_parity(orc, dev, name, thr, sta):
    c = case(name, orc, dev)
    w = c["w"]
    say("[attn-full]", name, "thr", thr, "sta", sta)
    (qf, kf), g, o, band, _ = run_mask(c, orc, dev, thr, sta, rows="all")
    compare_lists(*g, *o, band, "%s lists" % name)
    vf = nabla.nabla_fractal_permute(c["gnat"]["v"])
    kv_nb = torch.from_numpy(g[0]).to(dev)
    kv_inds = torch.from_numpy(g[1]).to(dev)
    out = nabla.nabla_sparse_attn_fwd(qf, kf, vf, kv_nb, kv_inds, tiles=w.tiles)
    torch.cuda.synchronize()
    ids, oo = orc.attention(c["frac"]["q"], c["frac"]["k"], c["frac"]["v"], g[0], g[1])
    want = orc.rows_to_tokens(oo, ids, w.B, w.S, w.heads, w.D)
    check_attention(to_np(out), want, "%s attn" % name)
    # inverse permutation of O back to the natural grid
    o_nat = nabla.nabla_fractal_permute(out, grid=(w.T, w.H, w.W), inverse=True)
    assert torch.equal(nabla.nabla_fractal_permute(o_nat), out)


def test_attention_random_lists_and_edges(orc, dev):
    """User-supplied lists: empty rows (O = 0), single blocks, full rows, any order."""
    rng = np.random.default_rng(15)
    for D, dtype, tiles in ((128, torch.bfloat16, (5, 1, 4)), (64, torch.bfloat16, None),
                            (128, torch.float32, (1, 4, 5)), (128, torch.bfloat16, (5, 2, 2))):
        B, S, h = 2, 1280, 3
        nb = S // 64
        say("[attn-random] D", D, dtype, "tiles", tiles)
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
        out = nabla.nabla_sparse_attn_fwd(*g, torch.from_numpy(kv_nb).to(dev),
                                          torch.from_numpy(kv_inds).to(dev), tiles=tiles)
        torch.cuda.synchronize()
        qq, kk, vv = (to_np(t) for t in g)  # the values the kernel sees
        ids, oo = orc.attention(qq, kk, vv, kv_nb, kv_inds)
        want = orc.rows_to_tokens(oo, ids, B, S, h, D)
        got = to_np(out)
        assert np.all(got[0, 0:64, 0] == 0)
        check_attention(got, want, "random lists D=%d %s tiles=%s" % (D, dtype, tiles))


def test_attention_sta_only_window(orc, dev):
    """Lists built from the STA window alone give attention restricted to the window."""
    c = case("small", orc, dev)
    w = c["w"]
    say("[attn-sta-only]")
    sta = orc.sta_mask(*w.tiles, *w.sta)
    nb = w.nb
    kv_nb = np.broadcast_to(sta.sum(1).astype(np.int32), (w.B, w.heads, nb)).copy()
    kv_inds = np.zeros((w.B, w.heads, nb, nb), np.int32)
    for i in range(nb):
        sel = np.flatnonzero(sta[i])
        kv_inds[:, :, i, :sel.size] = sel
    qf, kf, vf = (nabla.nabla_fractal_permute(c["gnat"][n]) for n in ("q", "k", "v"))
    out = nabla.nabla_sparse_attn_fwd(qf, kf, vf, torch.from_numpy(kv_nb).to(dev),
                                      torch.from_numpy(kv_inds).to(dev), tiles=w.tiles)
    torch.cuda.synchronize()
    ids, oo = orc.attention(c["frac"]["q"], c["frac"]["k"], c["frac"]["v"], kv_nb, kv_inds)
    check_attention(to_np(out), orc.rows_to_tokens(oo, ids, w.B, w.S, w.heads, w.D),
                    "sta-only")


def test_run_twice_bitwise(orc, dev):
    c = case("small", orc, dev)
    w = c["w"]
    say("[determinism]")
    qf, kf, vf = (nabla.nabla_fractal_permute(c["gnat"][n]) for n in ("q", "k", "v"))
    sta = nabla.nabla_sta_mask(w.tiles, w.sta, dev)
    a = nabla.nabla_block_mask(qf, kf, sta, 0.9)
    b = nabla.nabla_block_mask(qf, kf, sta, 0.9)
    assert torch.equal(a[0], b[0])
    for r in range(a[0].numel()):
        n = int(a[0].view(-1)[r])
        assert torch.equal(a[1].view(-1, w.nb)[r, :n], b[1].view(-1, w.nb)[r, :n])
    o1 = nabla.nabla_sparse_attn_fwd(qf, kf, vf, *a, tiles=w.tiles)
    o2 = nabla.nabla_sparse_attn_fwd(qf, kf, vf, *a, tiles=w.tiles)
    assert torch.equal(o1, o2)
    # grouping only changes which blocks share tiles on chip, not the result
    o3 = nabla.nabla_sparse_attn_fwd(qf, kf, vf, *a)
    assert torch.equal(o1, o3)


def test_gpu_errors(dev):
    q = torch.zeros(1, 100, 1, 64, device=dev, dtype=torch.bfloat16)
    with pytest.raises(nabla.NablaError) as e:
        nabla.nabla_block_mask(q, q, None, 0.9)
    assert e.value.status == 1
    q = torch.zeros(1, 128, 1, 64, device=dev, dtype=torch.bfloat16)
    with pytest.raises(nabla.NablaError) as e:
        nabla.nabla_block_mask(q, q, None, float("nan"))
    assert e.value.status == 1
    q = torch.zeros(1, 128, 1, 96, device=dev, dtype=torch.bfloat16)
    with pytest.raises(nabla.NablaError) as e:
        nabla.nabla_block_mask(q, q, None, 0.9)
    assert e.value.status == 2


# ------------------------------------------------------------------ every row at full size
@pytest.mark.parametrize("name", ["long", "720p"])
def test_attention_sampled_parity(orc, dev, name):
    c = case(name, orc, dev)
    w = c["w"]
    say("[attn-sampled]", name)
    (qf, kf), _, _, _, _ = run_mask(c, orc, dev, w.thr, w.sta, rng=np.random.default_rng(13))
    sta_g = nabla.nabla_sta_mask(w.tiles, w.sta, dev)
    kv_nb, kv_inds = nabla.nabla_block_mask(qf, kf, sta_g, w.thr)
    vf = nabla.nabla_fractal_permute(c["gnat"]["v"])
    out = nabla.nabla_sparse_attn_fwd(qf, kf, vf, kv_nb, kv_inds, tiles=w.tiles)
    torch.cuda.synchronize()
    g_nb = kv_nb.cpu().numpy()
    rng = np.random.default_rng(14)
    ids = sample_rows(g_nb, rng, per_head=0)
    ids = ids[rng.choice(ids.size, size=min(ids.size, 48), replace=False)]
    rid, oo = orc.attention(c["frac"]["q"], c["frac"]["k"], c["frac"]["v"], g_nb,
                            kv_inds.cpu().numpy(), row_ids=ids)
    got = to_np(out)
    nb = w.nb
    sel = []
    for rr in rid:
        b, rem = divmod(int(rr), w.heads * nb)
        h, i = divmod(rem, nb)
        sel.append(got[b, 64 * i:64 * (i + 1), h, :])
    check_attention(np.stack(sel), oo, "%s attn sampled" % name)


@pytest.mark.parametrize("name", ["720p", "long"])
def test_block_mask_every_row_large(orc, dev, name):
    """The 720p and long-clip workloads: every row of kv_nb and kv_inds, from the fractal-order
    call and from the natural-order call that the bench times (the permute folded into the
    pooling)."""
    c = case(name, orc, dev)
    w = c["w"]
    say("[mask-all-rows]", w.describe())
    _, g, o, band, _ = run_mask(c, orc, dev, w.thr, w.sta, rows="all")
    compare_lists(*g, *o, band, "%s fractal-order call" % name)
    sta_g = nabla.nabla_sta_mask(w.tiles, w.sta, dev)
    n_nb, n_inds = nabla.nabla_block_mask_natural(c["gnat"]["q"], c["gnat"]["k"], sta_g, w.thr)
    torch.cuda.synchronize()
    compare_lists(n_nb.cpu().numpy(), n_inds.cpu().numpy(), *o, band, "%s natural-order call" % name)


def sweep_params():
    return [pytest.param(w, id=w.name) for w in synth.sweep_workloads()]


@pytest.mark.parametrize("w", sweep_params())
def test_sweep_run_parity(orc, dev, w):
    """Each of the fifteen 720p sweep runs (thr 0.5 / 0.7 / 0.9 / 0.95 x STA off / (1,1,1) /
    (2,1,1) on the seed-2 tensors, and the iid, noise 0.1 and sigma_f 1 / noise 0.1
    generators), in the launch configuration the bench times (natural-order calls): kv_nb and
    kv_inds on every row against the oracle estimator, then the attention on 48 sampled query
    blocks, the fewest- and most-kept rows, the first and the last among them."""
    c = case(None, orc, dev, w=w)
    say("[sweep]", w.describe())
    sta_g = None if w.sta is None else nabla.nabla_sta_mask(w.tiles, w.sta, dev)
    kv_nb, kv_inds = nabla.nabla_block_mask_natural(c["gnat"]["q"], c["gnat"]["k"], sta_g, w.thr)
    o = nabla.nabla_sparse_attn_fwd_natural(c["gnat"]["q"], c["gnat"]["k"], c["gnat"]["v"],
                                            kv_nb, kv_inds)
    torch.cuda.synchronize()
    g_nb, g_inds = kv_nb.cpu().numpy(), kv_inds.cpu().numpy()
    sta_o = None if w.sta is None else orc.sta_mask(*w.tiles, *w.sta)
    m = orc.block_mask(c["frac"]["q"], c["frac"]["k"], sta_o, w.thr)
    band = orc.band_rows(m["diag"], w.thr)
    compare_lists(g_nb, g_inds, m["kv_nb"], m["kv_inds"], band, w.name)
    say("[sweep] %s density %.4f" % (w.name, g_nb.sum() / float(w.B * w.heads * w.nb ** 2)))
    flat = g_nb.reshape(-1)
    rng = np.random.default_rng(16)
    ids = {0, flat.size - 1, int(np.argmin(flat)), int(np.argmax(flat))}
    while len(ids) < 48:
        ids.add(int(rng.integers(flat.size)))
    ids = np.array(sorted(ids), np.int64)
    rid, oo = orc.attention(c["frac"]["q"], c["frac"]["k"], c["frac"]["v"], m["kv_nb"],
                            m["kv_inds"], row_ids=ids)
    got = orc.fractal_permute(to_np(o)).reshape(w.B, w.S, w.heads, w.D)  # natural -> fractal
    sel = []
    for rr in rid:
        b, rem = divmod(int(rr), w.heads * w.nb)
        h, i = divmod(rem, w.nb)
        sel.append(got[b, 64 * i:64 * (i + 1), h, :])
    check_attention(np.stack(sel), oo, "%s attn sampled" % w.name)
