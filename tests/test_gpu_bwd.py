"""Parity of the HIP training pass (forward lse + backward, through the C ABI) with the oracle.

The oracle computes lse, dq, dk and dv of the dense masked softmax attention in fp64
(oracle.attention_bwd / attention_dq / attention_lse).  The HIP path takes bf16 q, k, v
and dO, rounds the weights P and dS = P (dP - Delta) to bf16 as MFMA operands and
accumulates in fp32; Delta comes from the forward's bf16 output.

Tolerance (derived from that arithmetic, independent of the data's scale): each
gradient element is a sum of products of which one factor was rounded to bf16
(relative error <= 2^-9) plus an error of the same order through Delta, so relative
to the gradient's own magnitude we allow max|err| <= 2e-2 * max|g| and
mean|err| <= 1e-2 * mean|g| (errors of a wrong index, sign or missing term are O(1)
in these measures).  lse is an fp32 log of bf16-product sums: |err| <= 2e-2 absolute
(the scores themselves carry bf16 input rounding, as in the forward).

Inputs are seeded (numpy); the lists come from the host (random, window or the
oracle's own estimator), never from the HIP path.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_fractal_amd as nabla
from block_sparse_attention_fractal_amd import synth

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN, LSE_ABS = 2e-2, 1e-2, 2e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def bf16_round(a):
    """numpy fp32 -> the fp32 values of its bf16 rounding (RNE), and the bf16 bytes."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.float().numpy(), t


def random_lists(rng, B, h, nb, empty=(), full=()):
    kv_nb = np.zeros((B, h, nb), np.int32)
    kv_inds = np.zeros((B, h, nb, nb), np.int32)
    for b in range(B):
        for hh in range(h):
            for i in range(nb):
                n = int(rng.integers(1, nb + 1))
                if (b, hh, i) in empty:
                    n = 0
                if (b, hh, i) in full:
                    n = nb
                kv_nb[b, hh, i] = n
                kv_inds[b, hh, i] = rng.permutation(nb)
    return kv_nb, kv_inds


def run_gpu(dev, tq, tk, tv, tdo, kv_nb, kv_inds, scale=None, grid=None):
    g = lambda t: t.to(dev)
    q, k, v, do = g(tq), g(tk), g(tv), g(tdo)
    nb_t = torch.from_numpy(kv_nb).to(dev)
    inds_t = torch.from_numpy(kv_inds).to(dev)
    B, S, h, D = q.shape
    lse = torch.empty((B, h, S), dtype=torch.float32, device=dev)
    o = nabla.nabla_sparse_attn_fwd(q, k, v, nb_t, inds_t, scale=scale, lse=lse, grid=grid)
    dq, dk, dv = nabla.nabla_sparse_attn_bwd(q, k, v, o, do, lse, nb_t, inds_t, scale=scale,
                                             grid=grid)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return dict(lse=lse.cpu().numpy().astype(np.float64), dq=f(dq), dk=f(dk), dv=f(dv), o=o)


def rel_check(got, want, label):
    err = np.abs(got - want)
    mx, mn = float(err.max()), float(err.mean())
    ref_mx, ref_mn = float(np.abs(want).max()), float(np.abs(want).mean())
    say("[%s] max err %.3g (max|g| %.3g, ratio %.3g)  mean err %.3g (mean|g| %.3g, ratio %.3g)"
        % (label, mx, ref_mx, mx / max(ref_mx, 1e-30), mn, ref_mn, mn / max(ref_mn, 1e-30)))
    assert mx <= REL_MAX * ref_mx, label
    assert mn <= REL_MEAN * ref_mn, label


def lse_check(got, want, label):
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got)), label
    if fin.any():
        e = float(np.abs(got[fin] - want[fin]).max())
        say("[%s] lse max err %.3g" % (label, e))
        assert e <= LSE_ABS, label
    assert np.all(got[~fin] == -np.inf), label


@pytest.mark.parametrize("D,S,h,seed,B", [(128, 1024, 2, 31, 1), (64, 1344, 3, 32, 1),
                                           (128, 256, 1, 33, 1), (128, 512, 3, 34, 2),
                                           (64, 384, 2, 35, 2)])
def test_bwd_full_parity_random_lists(orc, dev, D, S, h, seed, B):
    """Every lse, dq, dk, dv element against the oracle on random lists: ragged counts, any
    order, one empty row, one row that lists every block; batches of two give the (b, head)
    offsets of every kernel."""
    rng = np.random.default_rng(seed)
    nb = S // 64
    say("[bwd full] B=%d D=%d S=%d heads=%d seed=%d" % (B, D, S, h, seed))
    arrs = [bf16_round(rng.standard_normal((B, S, h, D)).astype(np.float32)) for _ in range(4)]
    (q, tq), (k, tk), (v, tv), (do, tdo) = arrs
    kv_nb, kv_inds = random_lists(rng, B, h, nb, empty={(0, h - 1, nb // 2)}, full={(0, 0, 1)})
    got = run_gpu(dev, tq, tk, tv, tdo, kv_nb, kv_inds)
    want = orc.attention_bwd(q, k, v, do, kv_nb, kv_inds)
    lse_check(got["lse"], want["lse"], "lse")
    for n in ("dq", "dk", "dv"):
        rel_check(got[n], want[n], n)
    # the empty row's dq is exactly zero
    i0 = nb // 2
    assert np.all(got["dq"][0, 64 * i0:64 * (i0 + 1), h - 1] == 0.0)


def test_bwd_unlisted_keys_and_scale(orc, dev):
    """Key blocks that no list holds get dk = dv = 0; an explicit scale is honoured."""
    rng = np.random.default_rng(34)
    B, S, h, D = 1, 512, 2, 128
    nb = S // 64
    arrs = [bf16_round(rng.standard_normal((B, S, h, D)).astype(np.float32)) for _ in range(4)]
    (q, tq), (k, tk), (v, tv), (do, tdo) = arrs
    kv_nb = np.full((B, h, nb), 3, np.int32)
    kv_inds = np.zeros((B, h, nb, nb), np.int32)
    for i in range(nb):  # every row lists blocks 1, 4, 6 only
        kv_inds[0, :, i] = [6, 1, 4] + [x for x in range(nb) if x not in (1, 4, 6)]
    got = run_gpu(dev, tq, tk, tv, tdo, kv_nb, kv_inds, scale=0.05)
    want = orc.attention_bwd(q, k, v, do, kv_nb, kv_inds, scale=0.05)
    for j in range(nb):
        if j in (1, 4, 6):
            continue
        assert np.all(got["dk"][0, 64 * j:64 * (j + 1)] == 0.0)
        assert np.all(got["dv"][0, 64 * j:64 * (j + 1)] == 0.0)
    lse_check(got["lse"], want["lse"], "lse scale")
    for n in ("dq", "dk", "dv"):
        rel_check(got[n], want[n], n + " scale")


def test_bwd_estimator_lists_small(orc, dev):
    """The small workload with the oracle estimator's lists (thr 0.9, STA (1,1,1)) and a seeded
    dO: every gradient element."""
    w = synth.WORKLOADS["small"]
    say("[bwd small]", w.describe())
    qn, kn, vn = synth.make_qkv(w)
    f = lambda a: orc.fractal_permute(a).reshape(w.B, w.S, w.heads, w.D)
    q, tq = bf16_round(f(qn))
    k, tk = bf16_round(f(kn))
    v, tv = bf16_round(f(vn))
    do, tdo = bf16_round(np.random.default_rng(41).standard_normal(q.shape).astype(np.float32))
    m = orc.block_mask(q, k, orc.sta_mask(*w.tiles, *w.sta), w.thr)
    got = run_gpu(dev, tq, tk, tv, tdo, m["kv_nb"], m["kv_inds"])
    want = orc.attention_bwd(q, k, v, do, m["kv_nb"], m["kv_inds"])
    lse_check(got["lse"], want["lse"], "lse small")
    for n in ("dq", "dk", "dv"):
        rel_check(got[n], want[n], n + " small")


def test_bwd_720p_sampled_and_sums(orc, dev):
    """720p with the oracle estimator's lists: lse and dq on sampled query blocks, dk and dv on
    sampled key blocks (among them the key block that the most query blocks list) against the
    oracle, element by element; per (b, h) the sum of dv over all keys equals the sum of dO over
    all rows, and the sum of dk is 0 (properties of the exact gradient at any size)."""
    w = synth.WORKLOADS["720p"]
    say("[bwd 720p]", w.describe())
    qn, kn, vn = synth.make_qkv(w)
    f = lambda a: orc.fractal_permute(a).reshape(w.B, w.S, w.heads, w.D)
    q, tq = bf16_round(f(qn))
    k, tk = bf16_round(f(kn))
    v, tv = bf16_round(f(vn))
    do, tdo = bf16_round(np.random.default_rng(42).standard_normal(q.shape).astype(np.float32))
    say("[bwd 720p] oracle estimator")
    m = orc.block_mask(q, k, orc.sta_mask(*w.tiles, *w.sta), w.thr)
    say("[bwd 720p] gpu")
    got = run_gpu(dev, tq, tk, tv, tdo, m["kv_nb"], m["kv_inds"])
    rng = np.random.default_rng(43)
    nb = w.nb
    ids = []
    for hh in range(w.heads):
        row = m["kv_nb"][0, hh]
        pick = {0, nb - 1, int(np.argmin(row)), int(np.argmax(row))} | set(rng.choice(nb, 2).tolist())
        ids += [hh * nb + i for i in sorted(pick)]
    ids = np.array(ids, np.int64)
    say("[bwd 720p] oracle on %d sampled q-blocks" % ids.size)
    _, lse_o = orc.attention_lse(q, k, m["kv_nb"], m["kv_inds"], row_ids=ids)
    _, dq_o = orc.attention_dq(q, k, v, do, m["kv_nb"], m["kv_inds"], row_ids=ids)
    lse_g = np.stack([got["lse"][0, int(r) // nb, 64 * (int(r) % nb):64 * (int(r) % nb + 1)] for r in ids])
    dq_g = np.stack([got["dq"][0, 64 * (int(r) % nb):64 * (int(r) % nb + 1), int(r) // nb] for r in ids])
    lse_check(lse_g, lse_o, "lse 720p sampled")
    rel_check(dq_g, dq_o, "dq 720p sampled")
    # dk, dv: key block j of head h gathers from every query block whose list holds j
    held = np.zeros((w.heads, nb), np.int64)  # how many query blocks list each key block
    for hh in range(w.heads):
        for i in range(nb):
            held[hh, m["kv_inds"][0, hh, i, :m["kv_nb"][0, hh, i]]] += 1
    h_top = int(np.argmax(held.max(1)))
    h_other = (h_top + 1 + int(rng.integers(w.heads - 1))) % w.heads
    # the most and the least listed key blocks of that head, and a random one of another head
    # (each costs the oracle a full row pass of every query block that lists it)
    cols = {h_top * nb + int(np.argmax(held[h_top])), h_top * nb + int(np.argmin(held[h_top])),
            h_other * nb + int(rng.integers(nb))}
    cols = np.array(sorted(cols), np.int64)
    say("[bwd 720p] oracle dk, dv on %d key blocks (listed by %s query blocks)"
        % (cols.size, [int(held.reshape(-1)[c]) for c in cols]))
    _, dk_o, dv_o = orc.attention_dkdv(q, k, v, do, m["kv_nb"], m["kv_inds"], cols)
    key_rows = lambda g: np.stack([g[0, 64 * (int(c) % nb):64 * (int(c) % nb + 1), int(c) // nb]
                                   for c in cols])
    rel_check(key_rows(got["dk"]), dk_o, "dk 720p sampled key blocks")
    rel_check(key_rows(got["dv"]), dv_o, "dv 720p sampled key blocks")
    sum_do = do.astype(np.float64).sum(1)  # [B, h, D]; every 720p row lists >= 1 block
    sum_dv = got["dv"].sum(1)
    sum_dk = got["dk"].sum(1)
    scale_ref = np.abs(got["dv"]).sum(1).max()
    e_dv = float(np.abs(sum_dv - sum_do).max())
    e_dk = float(np.abs(sum_dk).max())
    say("[bwd 720p] |sum dv - sum dO| max %.3g, |sum dk| max %.3g (sum |dv| up to %.3g)"
        % (e_dv, e_dk, scale_ref))
    # each of the S terms carries a bf16 rounding of relative size <= 2^-9
    assert e_dv <= 2.0 ** -8 * scale_ref
    assert e_dk <= 2.0 ** -8 * np.abs(got["dk"]).sum(1).max()


def test_bwd_deterministic(dev):
    """Two runs give the same bits (no atomics in the backward)."""
    rng = np.random.default_rng(44)
    B, S, h, D = 1, 2048, 2, 128
    arrs = [bf16_round(rng.standard_normal((B, S, h, D)).astype(np.float32))[1] for _ in range(4)]
    kv_nb, kv_inds = random_lists(rng, B, h, S // 64)
    a = run_gpu(dev, *arrs, kv_nb, kv_inds)
    b = run_gpu(dev, *arrs, kv_nb, kv_inds)
    for n in ("lse", "dq", "dk", "dv"):
        assert np.array_equal(a[n], b[n]), n


# ---- padded fractal layouts (H or W not a multiple of 8): padding is never a key

def padded_inputs(orc, rng, B, T, H, W, h, D):
    """Natural-order seeded q, k, v, dO permuted by the oracle (padding rows 0), bf16."""
    nat = [rng.standard_normal((B, T, H, W, h, D)).astype(np.float32) for _ in range(4)]
    return [bf16_round(orc.fractal_permute(a)) for a in nat]


@pytest.mark.parametrize("T,H,W,h,D,seed", [(2, 12, 20, 2, 128, 51), (1, 20, 28, 3, 64, 52)])
def test_bwd_padded_full_parity(orc, dev, T, H, W, h, D, seed):
    """Every lse, dq, dk, dv element of the padded training pass (nabla_sparse_attn_fwd_grid +
    nabla_sparse_attn_bwd_grid) against oracle.attention_bwd_grid on random lists; padding
    positions get exactly zero dk and dv (they are never keys) and zero dq (dO = 0 there)."""
    rng = np.random.default_rng(seed)
    B = 1
    (q, tq), (k, tk), (v, tv), (do, tdo) = padded_inputs(orc, rng, B, T, H, W, h, D)
    S = q.shape[1]
    nb = S // 64
    say("[bwd padded] T=%d H=%d W=%d heads=%d D=%d (S=%d)" % (T, H, W, h, D, S))
    kv_nb, kv_inds = random_lists(rng, B, h, nb, empty={(0, h - 1, 0)}, full={(0, 0, nb - 1)})
    got = run_gpu(dev, tq, tk, tv, tdo, kv_nb, kv_inds, grid=(T, H, W))
    want = orc.attention_bwd_grid(q, k, v, do, (T, H, W), kv_nb, kv_inds)
    lse_check(got["lse"], want["lse"], "lse padded")
    for n in ("dq", "dk", "dv"):
        rel_check(got[n], want[n], n + " padded")
    pad = ~orc.token_valid(T, H, W)
    for n in ("dq", "dk", "dv"):
        assert np.all(got[n][0, pad] == 0.0), n


def test_bwd_padded_estimator_lists(orc, dev):
    """The padded small workload (4 frames of 20 x 28 latents) with the oracle's padded
    estimator lists: every gradient element."""
    w = synth.WORKLOADS["small_pad"]
    say("[bwd padded estimator]", w.describe())
    grid = (w.T, w.H, w.W)
    qn, kn, vn = synth.make_qkv(w)
    q, tq = bf16_round(orc.fractal_permute(qn))
    k, tk = bf16_round(orc.fractal_permute(kn))
    v, tv = bf16_round(orc.fractal_permute(vn))
    don = np.random.default_rng(53).standard_normal(qn.shape).astype(np.float32)
    do, tdo = bf16_round(orc.fractal_permute(don))
    Ht, Wt = (w.H + 7) // 8, (w.W + 7) // 8
    m = orc.block_mask_grid(q, k, grid, orc.sta_mask(w.T, Ht, Wt, *w.sta), w.thr)
    got = run_gpu(dev, tq, tk, tv, tdo, m["kv_nb"], m["kv_inds"], grid=grid)
    want = orc.attention_bwd_grid(q, k, v, do, grid, m["kv_nb"], m["kv_inds"])
    lse_check(got["lse"], want["lse"], "lse padded small")
    for n in ("dq", "dk", "dv"):
        rel_check(got[n], want[n], n + " padded small")


def test_bwd_grid_of_whole_patches_is_plain(dev):
    """On a grid of whole patches the grid entry point gives the plain call's bits."""
    rng = np.random.default_rng(54)
    T, H, W, h, D = 2, 16, 24, 2, 128
    S = T * H * W
    arrs = [bf16_round(rng.standard_normal((1, S, h, D)).astype(np.float32))[1] for _ in range(4)]
    kv_nb, kv_inds = random_lists(rng, 1, h, S // 64)
    a = run_gpu(dev, *arrs, kv_nb, kv_inds, grid=(T, H, W))
    b = run_gpu(dev, *arrs, kv_nb, kv_inds)
    for n in ("lse", "dq", "dk", "dv"):
        assert np.array_equal(a[n], b[n]), n
