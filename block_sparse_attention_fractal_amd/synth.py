"""Seeded synthetic video-shaped inputs and the named workloads.

This module holds no arithmetic of the method: it draws random tensors and
describes workload shapes.  Both the HIP path's tests and the oracle's tests
take their inputs from here.

Generator (numpy PCG64, ``default_rng(seed)``), tensors in natural order
[B, T, H, W, heads, D]:

* ``iid``: Q, K, V ~ N(0, 1), drawn in that order.
* ``smooth``: a low-frequency spatio-temporal field shared by Q and K plus
  independent noise,  Q = F + sigma_n N,  K = F + sigma_n N',  V ~ N(0, 1), with
  F_{h,c}(t, y, x) = (sigma_f / 2) sum_{m<8} a_m cos(2 pi (f_t t/T + f_y y/H
  + f_x x/W) + phi_m),  a ~ N(0,1), f ~ U(-1,1) cycles per extent,
  phi ~ U(0, 2 pi), drawn per (head, channel) in the order a, f, phi; then
  Q noise, K noise, V.  E[F^2] = sigma_f^2.

These stand in for the latents of the video models the pages evaluate
(Wan 2.1 at 720p, a 2B DiT at 512^2); no dataset or weights are used.
``bf16`` tensors are rounded to bfloat16 (nearest-even) and returned as the
fp32 values they hold.
"""
import dataclasses
import math

import numpy as np

TILE = 8      # spatial patch edge: a 1 x 8 x 8 tile is one 64-token block
BLOCK = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    D: int
    T: int
    H: int
    W: int
    dtype: str                 # "bf16" | "fp32"
    gen: str                   # "iid" | "smooth"
    seed: int
    thr: float = 0.9
    sta: tuple = (1, 1, 1)     # (win_t, win_h, win_w); None = STA off
    sigma_f: float = 0.75
    sigma_n: float = 0.5

    @property
    def tiles(self):
        """(T, ceil(H/8), ceil(W/8)): the patch grid; partial patches when 8 does not divide H, W."""
        return (self.T, -(-self.H // TILE), -(-self.W // TILE))

    @property
    def S(self):
        """Length of the fractal layout (padded to whole patches)."""
        Tt, Ht, Wt = self.tiles
        return Tt * Ht * Wt * BLOCK

    @property
    def tokens(self):
        return self.T * self.H * self.W

    @property
    def padded(self):
        return self.H % TILE != 0 or self.W % TILE != 0

    @property
    def nb(self):
        return self.S // BLOCK

    def describe(self):
        sta = "off" if self.sta is None else "|dt|<=%d,|dh|<=%d,|dw|<=%d" % self.sta
        return ("%s: B=%d heads=%d D=%d T=%d H=%d W=%d (S=%d, nb=%d) %s %s seed=%d thr=%g STA %s"
                % (self.name, self.B, self.heads, self.D, self.T, self.H, self.W, self.S,
                   self.nb, self.dtype, self.gen, self.seed, self.thr, sta))


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, 2, 16, 16, "fp32", "iid", 0, 0.9, (1, 1, 1)),
    "small": Workload("small", 1, 8, 128, 8, 32, 32, "bf16", "smooth", 1, 0.9, (1, 1, 1)),
    "720p": Workload("720p", 1, 16, 128, 16, 48, 80, "bf16", "smooth", 2, 0.9, (2, 1, 1)),
    "long": Workload("long", 1, 16, 128, 31, 48, 80, "bf16", "smooth", 3, 0.9, (2, 1, 1)),
    # H, W not multiples of 8: the last patch row / column of each frame is partial
    "small_pad": Workload("small_pad", 1, 4, 128, 4, 20, 28, "bf16", "smooth", 7, 0.9, (1, 1, 1)),
    "720p_pad": Workload("720p_pad", 1, 16, 128, 16, 44, 76, "bf16", "smooth", 8, 0.9, (2, 1, 1)),
}


def sweep_workloads():
    """The 720p sparsity sweep: thr x STA window on the seed-2 tensors, plus generator variants."""
    base = WORKLOADS["720p"]
    out = []
    for thr in (0.5, 0.7, 0.9, 0.95):
        for sta in (None, (1, 1, 1), (2, 1, 1)):
            tag = "off" if sta is None else "%d%d%d" % sta
            out.append(dataclasses.replace(base, name="sweep_thr%g_sta%s" % (thr, tag), thr=thr,
                                           sta=sta))
    out.append(dataclasses.replace(base, name="sweep_iid", gen="iid", seed=4))
    out.append(dataclasses.replace(base, name="sweep_noise0.1", sigma_n=0.1, seed=5))
    out.append(dataclasses.replace(base, name="sweep_sf1_noise0.1", sigma_f=1.0, sigma_n=0.1,
                                   seed=6))
    return out


def round_bf16(x):
    """Round fp32 values to bfloat16, nearest-even, in place; returns the fp32 array (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    lsb += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return x


def _smooth_field(rng, T, H, W, heads, D, sigma_f):
    M = 8
    a = rng.standard_normal((heads, D, M))
    f = rng.uniform(-1.0, 1.0, size=(heads, D, M, 3))
    phi = rng.uniform(0.0, 2.0 * math.pi, size=(heads, D, M))
    F = np.zeros((T, H, W, heads, D), dtype=np.float32)
    ys = (np.arange(H, dtype=np.float32) / np.float32(H))[:, None, None, None]
    xs = (np.arange(W, dtype=np.float32) / np.float32(W))[None, :, None, None]
    two_pi = np.float32(2.0 * math.pi)
    ang = np.empty((H, W, heads, D), np.float32)
    cb = np.empty_like(ang)
    sb = np.empty_like(ang)
    tmp = np.empty_like(ang)
    for m in range(M):
        fy = (two_pi * f[:, :, m, 1]).astype(np.float32)
        fx = (two_pi * f[:, :, m, 2]).astype(np.float32)
        np.multiply(ys, fy, out=ang)
        np.multiply(xs, fx, out=tmp)
        ang += tmp
        np.cos(ang, out=cb)
        np.sin(ang, out=sb)
        amp = 0.5 * sigma_f * a[:, :, m]
        for t in range(T):
            ang_a = 2.0 * math.pi * f[:, :, m, 0] * (t / T) + phi[:, :, m]
            ca = (amp * np.cos(ang_a)).astype(np.float32)
            sa = (amp * np.sin(ang_a)).astype(np.float32)
            np.multiply(cb, ca, out=tmp)      # amp cos(ang_a) cos(ang_b)
            F[t] += tmp
            np.multiply(sb, sa, out=tmp)      # amp sin(ang_a) sin(ang_b)
            F[t] -= tmp
    return F


def make_qkv(w: Workload, B=None):
    """Natural-order q, k, v [B, T, H, W, heads, D] as fp32 arrays (bf16-exact for bf16)."""
    B = w.B if B is None else B
    rng = np.random.default_rng(w.seed)
    shape = (B, w.T, w.H, w.W, w.heads, w.D)
    if w.gen == "iid":
        q = rng.standard_normal(shape, dtype=np.float32)
        k = rng.standard_normal(shape, dtype=np.float32)
    elif w.gen == "smooth":
        F = np.stack([_smooth_field(rng, w.T, w.H, w.W, w.heads, w.D, w.sigma_f)
                      for _ in range(B)]) if B > 1 else \
            _smooth_field(rng, w.T, w.H, w.W, w.heads, w.D, w.sigma_f)[None]
        sn = np.float32(w.sigma_n)
        q = rng.standard_normal(shape, dtype=np.float32)
        q *= sn
        q += F
        k = rng.standard_normal(shape, dtype=np.float32)
        k *= sn
        k += F
        del F
    else:
        raise ValueError("unknown generator %r" % w.gen)
    v = rng.standard_normal(shape, dtype=np.float32)
    if w.dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


def random_lists(rng, B, heads, nb, density):
    """Random kv lists (each row: a random subset, ascending) for attention-only tests."""
    kv_nb = np.zeros((B, heads, nb), np.int32)
    kv_inds = np.zeros((B, heads, nb, nb), np.int32)
    for b in range(B):
        for h in range(heads):
            for i in range(nb):
                n = int(rng.binomial(nb, density))
                sel = np.sort(rng.choice(nb, size=n, replace=False)).astype(np.int32)
                kv_nb[b, h, i] = n
                kv_inds[b, h, i, :n] = sel
                rest = np.setdiff1d(np.arange(nb, dtype=np.int32), sel)
                kv_inds[b, h, i, n:] = rest
    return kv_nb, kv_inds
