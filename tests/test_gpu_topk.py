"""Parity of the HIP top-k estimator variant (nabla_block_mask_topk) with the oracle.

Both sides pool in the same fixed fp32 order, subtract the same smooth-k mean and
form the scores by the same sequential fma chain, so the selected sets are compared
bit for bit on every row (no band: unit weights and integer ranks, no softmax).
Inputs are the oracle's fractal-ordered arrays uploaded as they are.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_fractal_amd as nabla
from block_sparse_attention_fractal_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


_CACHE = {}


def inputs(name, orc, dev):
    if name in _CACHE:
        return _CACHE[name]
    _CACHE.clear()
    w = synth.WORKLOADS[name]
    say("[topk case]", w.describe())
    q, k, _ = synth.make_qkv(w)
    f = lambda a: orc.fractal_permute(a).reshape(w.B, w.S, w.heads, w.D)
    qf, kf = f(q), f(k)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gq = torch.from_numpy(np.ascontiguousarray(qf)).to(tdt).to(dev)
    gk = torch.from_numpy(np.ascontiguousarray(kf)).to(tdt).to(dev)
    # the oracle sees exactly the values the GPU reads
    c = (w, gq.float().cpu().numpy(), gk.float().cpu().numpy(), gq, gk)
    _CACHE[name] = c
    return c


def compare(g_nb, g_inds, o_nb, o_inds, label):
    g_nb, o_nb = g_nb.reshape(-1), o_nb.reshape(-1)
    nb = g_inds.shape[-1]
    g_inds, o_inds = g_inds.reshape(-1, nb), o_inds.reshape(-1, nb)
    for r in range(g_nb.size):
        n = int(o_nb[r])
        assert int(g_nb[r]) == n, "%s row %d: gpu %d oracle %d" % (label, r, g_nb[r], n)
        assert np.array_equal(g_inds[r, :n], o_inds[r, :n]), "%s row %d" % (label, r)
    say("[%s] %d rows bit-exact" % (label, g_nb.size))


@pytest.mark.parametrize("name", ["tiny", "small"])
@pytest.mark.parametrize("ratio,use_sta", [(0.1, False), (0.5, True), (0.0, True), (0.0, False),
                                           (1.0, False), (0.33, True)])
def test_topk_full_parity(orc, dev, name, ratio, use_sta):
    w, q, k, gq, gk = inputs(name, orc, dev)
    sta_o = orc.sta_mask(*w.tiles, *w.sta) if use_sta else None
    sta_g = nabla.nabla_sta_mask(w.tiles, w.sta, dev) if use_sta else None
    kv_nb, kv_inds = nabla.nabla_block_mask(gq, gk, sta_g, topk_ratio=ratio)
    torch.cuda.synchronize()
    o = orc.block_mask_topk(q, k, sta_o, ratio)
    compare(kv_nb.cpu().numpy(), kv_inds.cpu().numpy(), o["kv_nb"], o["kv_inds"],
            "%s ratio %g sta %s" % (name, ratio, use_sta))
    if not use_sta:
        assert np.all(kv_nb.cpu().numpy() == orc.topk_count(w.nb, ratio))


@pytest.mark.parametrize("name,ratio", [("720p", 0.1), ("720p", 0.25), ("long", 0.1)])
def test_topk_sampled_parity(orc, dev, name, ratio):
    """Large shapes (CPT 16 and 32 selection paths) on sampled rows: first, last, random."""
    w, q, k, gq, gk = inputs(name, orc, dev)
    sta_g = nabla.nabla_sta_mask(w.tiles, w.sta, dev)
    kv_nb, kv_inds = nabla.nabla_block_mask(gq, gk, sta_g, topk_ratio=ratio)
    torch.cuda.synchronize()
    g_nb, g_inds = kv_nb.cpu().numpy(), kv_inds.cpu().numpy()
    rng = np.random.default_rng(61)
    nb = w.nb
    ids = []
    for h in range(w.heads):
        pick = {0, nb - 1} | set(rng.choice(nb, 6, replace=False).tolist())
        ids += [h * nb + i for i in sorted(pick)]
    ids = np.array(ids, np.int64)
    o = orc.block_mask_topk(q, k, orc.sta_mask(*w.tiles, *w.sta), ratio, row_ids=ids)
    compare(g_nb.reshape(-1)[ids], g_inds.reshape(-1, nb)[ids], o["kv_nb"], o["kv_inds"],
            "%s ratio %g sampled" % (name, ratio))


def test_topk_ties(orc, dev):
    """Q = 0: every score is 0; the k highest block indices are kept (lower indices dropped
    first on equal scores)."""
    w, q, k, gq, gk = inputs("small", orc, dev)
    kv_nb, kv_inds = nabla.nabla_block_mask(torch.zeros_like(gq), gk, None, topk_ratio=0.25)
    torch.cuda.synchronize()
    kk = orc.topk_count(w.nb, 0.25)
    assert np.all(kv_nb.cpu().numpy() == kk)
    assert np.all(kv_inds.cpu().numpy()[..., :kk] == np.arange(w.nb - kk, w.nb))
