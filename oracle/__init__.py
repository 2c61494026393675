"""CPU oracle for the NABLA hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it and
shares no code with it.  The arithmetic lives in ``nabla_oracle.c`` (fp32
estimator with a fixed reduction order, fp64 attention); this module only
marshals numpy arrays through ctypes.

Pages followed: FastVideo API page "nabla" (nablaT_v2 source; the
NablaAttentionImpl.forward source; the NablaAttentionMetadata fields) and the
"NABLA: Neighborhood Adaptive Block-Level Attention" summary page (Technical
Summary, Methodology).

The training pass (attention_lse, attention_dq, attention_bwd, and attention_bwd_grid
on padded layouts) is the gradient of that dense masked attention; it is pinned
against torch's fp64 autograd (over the natural token order for padded grids) and
closed forms.

The quantized variant (fp8_e4m3, quant_qkv, attention_q8) follows the sibling
"sla" backend page's SageSLA forward: INT8 Q and K per 64-token block after the
mean of K is subtracted, FP8 e4m3 V per channel, FP8 P; the encoders are pinned
against torch's float8_e4m3fn cast and round-trip bounds, the attention against
closed forms and the plain attention on the dequantized codes.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against closed forms, brute force, invariants or library routines
(nothing here is "parity unpinned").
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liborc_nabla.so")

BLOCK = 64
FIX_BITS = 48

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.orc_set_threads.argtypes = [i32]
    lib.orc_get_threads.restype = i32
    lib.orc_fractal_index.argtypes = [i32, i32, i32, i32, i32]
    lib.orc_fractal_index.restype = i64
    lib.orc_fractal_permute.argtypes = [P, P, i64, i32, i32, i32, i32, i32, i32, i32]
    lib.orc_sta_mask.argtypes = [P, i32, i32, i32, i32, i32, i32]
    lib.orc_pool.argtypes = [P, P, i32, i32, i32, i32]
    lib.orc_fractal_len.argtypes = [i32, i32, i32]
    lib.orc_fractal_len.restype = i64
    lib.orc_token_valid.argtypes = [i64, i32, i32]
    lib.orc_token_valid.restype = i32
    lib.orc_pool_grid.argtypes = [P, P, i32, i32, i32, i32, i32, i32]
    lib.orc_block_mask_grid.argtypes = [P, P, i32, i32, i32, i32, i32, i32, P, f64, P, i64, P, P,
                                        P, P]
    lib.orc_block_mask_grid.restype = i32
    lib.orc_block_mask_topk_grid.argtypes = [P, P, i32, i32, i32, i32, i32, i32, P, f64, P, i64,
                                             P, P]
    lib.orc_block_mask_topk_grid.restype = i32
    lib.orc_attention_grid.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, P, P, f64, P, i64, P]
    lib.orc_attention_grid.restype = i32
    lib.orc_scores.argtypes = [P, P, P, i32, i32, i32, i32]
    lib.orc_nexp.argtypes = [ctypes.c_float]
    lib.orc_nexp.restype = ctypes.c_float
    lib.orc_nexp_vec.argtypes = [P, P, i64]
    lib.orc_softmax_row.argtypes = [P, i32, P, P, P, P]
    lib.orc_cut_fixed.argtypes = [f64]
    lib.orc_cut_fixed.restype = i64
    lib.orc_select_row.argtypes = [P, i32, f64, P, P]
    lib.orc_block_mask.argtypes = [P, P, i32, i32, i32, i32, P, f64, P, i64, P, P, P, P]
    lib.orc_block_mask.restype = i32
    lib.orc_attention.argtypes = [P, P, P, i32, i32, i32, i32, P, P, f64, P, i64, P]
    lib.orc_attention.restype = i32
    lib.orc_topk_count.argtypes = [i32, f64]
    lib.orc_topk_count.restype = i32
    lib.orc_block_mask_topk.argtypes = [P, P, i32, i32, i32, i32, P, f64, P, i64, P, P]
    lib.orc_block_mask_topk.restype = i32
    lib.orc_attention_lse.argtypes = [P, P, i32, i32, i32, i32, P, P, f64, P, i64, P]
    lib.orc_attention_lse.restype = i32
    lib.orc_attention_dq.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, f64, P, i64, P]
    lib.orc_attention_dq.restype = i32
    lib.orc_attention_bwd.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, f64, P, P, P, P]
    lib.orc_attention_bwd.restype = i32
    lib.orc_attention_bwd_grid.argtypes = [P, P, P, P] + [i32] * 6 + [P, P, f64, P, P, P, P]
    lib.orc_attention_bwd_grid.restype = i32
    lib.orc_attention_dkdv.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, f64, P, i64, P, P]
    lib.orc_attention_dkdv.restype = i32
    lib.orc_fp8_e4m3.argtypes = [f64]
    lib.orc_fp8_e4m3.restype = ctypes.c_uint8
    lib.orc_fp8_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_fp8_e4m3_value.restype = f64
    lib.orc_fp8_e4m3_vec.argtypes = [P, P, i64]
    lib.orc_quant_qkv.argtypes = [P, P, P, i32, i32, i32, i32, P, P, P, P, P, P, P]
    lib.orc_quant_qkv.restype = i32
    lib.orc_attention_q8.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, P, P, f64, P, i64, P]
    lib.orc_attention_q8.restype = i32
    lib.orc_quant_qkv_grid.argtypes = [P, P, P] + [i32] * 6 + [P] * 7
    lib.orc_quant_qkv_grid.restype = i32
    lib.orc_attention_q8_grid.argtypes = [P] * 6 + [i32] * 6 + [P, P, f64, P, i64, P]
    lib.orc_attention_q8_grid.restype = i32
    _lib = lib
    return lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def set_threads(n: int) -> int:
    lib = _load()
    lib.orc_set_threads(int(n))
    return lib.orc_get_threads()


def get_threads() -> int:
    return _load().orc_get_threads()


# ---------------------------------------------------------------- O1 permute
def fractal_index(t, y, x, H, W) -> int:
    return _load().orc_fractal_index(t, y, x, H, W)


def fractal_len(T, H, W) -> int:
    """Sequence length of the fractal order of a T x H x W grid (padded to whole 8 x 8 patches)."""
    return _load().orc_fractal_len(T, H, W)


def token_valid(T, H, W):
    """bool [S]: which fractal positions of one sequence are tokens (False = patch padding)."""
    S = fractal_len(T, H, W)
    lib = _load()
    return np.array([bool(lib.orc_token_valid(s, H, W)) for s in range(S)])


def fractal_permute(x, inverse=False, grid=None):
    """Forward: x natural [B,T,H,W,heads,D] -> fractal [B,S,heads,D], S = fractal_len(T,H,W)
    (padding rows of partial patches are 0).  Inverse: x fractal [B,S,heads,D] with
    grid=(T,H,W) (or a natural-shaped array of a grid of whole patches) -> natural.
    Any fixed-size dtype (the permutation moves bytes).
    """
    x = np.ascontiguousarray(x)
    if not inverse:
        B, T, H, W, heads, D = x.shape
        y = np.empty((B, fractal_len(T, H, W), heads, D), dtype=x.dtype)
    else:
        if x.ndim == 6:
            B, T, H, W, heads, D = x.shape
        else:
            B, _, heads, D = x.shape
            T, H, W = grid
        y = np.empty((B, T, H, W, heads, D), dtype=x.dtype)
    _load().orc_fractal_permute(_ptr(x), _ptr(y), x.itemsize, B, T, H, W, heads, D, int(inverse))
    return y


# ---------------------------------------------------------------- O2 STA
def sta_mask(Tt, Ht, Wt, wt, wh, ww):
    nb = Tt * Ht * Wt
    out = np.empty((nb, nb), dtype=np.uint8)
    _load().orc_sta_mask(_ptr(out), Tt, Ht, Wt, wt, wh, ww)
    return out


# ---------------------------------------------------------------- O3-O5
def pool(x):
    """x [B,S,heads,D] (fp32 values) -> [B,heads,S/64,D] fp32."""
    x = _f32(x)
    B, S, heads, D = x.shape
    out = np.empty((B, heads, S // BLOCK, D), dtype=np.float32)
    _load().orc_pool(_ptr(x), _ptr(out), B, S, heads, D)
    return out


def pool_grid(x, grid):
    """x fractal [B,S,heads,D] of a padded T x H x W grid -> [B,heads,nb,D]: means over tokens only."""
    x = _f32(x)
    B, S, heads, D = x.shape
    T, H, W = grid
    out = np.empty((B, heads, S // BLOCK, D), dtype=np.float32)
    _load().orc_pool_grid(_ptr(x), _ptr(out), B, T, H, W, heads, D)
    return out


def scores(qa, ka):
    qa, ka = _f32(qa), _f32(ka)
    B, heads, nb, D = qa.shape
    out = np.empty((B, heads, nb, nb), dtype=np.float32)
    _load().orc_scores(_ptr(qa), _ptr(ka), _ptr(out), B, heads, nb, D)
    return out


def nexp(x):
    x = _f32(x)
    y = np.empty_like(x)
    _load().orc_nexp_vec(_ptr(x), _ptr(y), x.size)
    return y


def softmax_row(s):
    """Returns (e, p, P, Z): exp weights, fp32 probabilities, their 2^-48 fixed-point values, Z."""
    s = _f32(s)
    nb = s.shape[0]
    e = np.empty(nb, np.float32)
    p = np.empty(nb, np.float32)
    P = np.empty(nb, np.int64)
    Z = np.zeros(1, np.float64)
    _load().orc_softmax_row(_ptr(s), nb, _ptr(e), _ptr(p), _ptr(P), _ptr(Z))
    return e, p, P, float(Z[0])


def cut_fixed(thr) -> int:
    return _load().orc_cut_fixed(float(thr))


def select_row(s, thr):
    """Returns (kept uint8 [nb], diag int64 [3] = (i0, c_{i0-1}, c_{i0}))."""
    s = _f32(s)
    nb = s.shape[0]
    kept = np.empty(nb, np.uint8)
    diag = np.empty(3, np.int64)
    _load().orc_select_row(_ptr(s), nb, float(thr), _ptr(kept), _ptr(diag))
    return kept, diag


# ---------------------------------------------------------------- O3-O9
def block_mask(q, k, sta, thr, want_nabla=False, row_ids=None):
    """The estimator.  q, k [B,S,heads,D] fp32 values; sta [nb,nb] uint8 or None.

    Returns dict with kv_nb [B,h,nb] int32, kv_inds [B,h,nb,nb] int32
    (kept ascending, then dropped ascending), diag [B,h,nb,3] int64 and,
    if asked, mnabla [B,h,nb,nb] uint8 (mask before the STA union).  With
    ``row_ids`` (ids (b*heads + h)*nb + i) only those rows are evaluated and
    the outputs are [len(row_ids), ...].
    """
    q, k = _f32(q), _f32(k)
    B, S, heads, D = q.shape
    nb = S // BLOCK
    if row_ids is None:
        lead = (B, heads, nb)
        n = B * heads * nb
        rid = None
    else:
        rid = np.ascontiguousarray(row_ids, dtype=np.int64)
        lead = (rid.size,)
        n = rid.size
    kv_nb = np.empty(lead, np.int32)
    kv_inds = np.empty(lead + (nb,), np.int32)
    diag = np.empty(lead + (3,), np.int64)
    mn = np.empty(lead + (nb,), np.uint8) if want_nabla else None
    st = None if sta is None else np.ascontiguousarray(sta, dtype=np.uint8)
    rc = _load().orc_block_mask(_ptr(q), _ptr(k), B, S, heads, D, _ptr(st), float(thr),
                                _ptr(rid), n, _ptr(kv_nb), _ptr(kv_inds), _ptr(mn), _ptr(diag))
    if rc != 0:
        raise ValueError("oracle block_mask: bad argument")
    out = {"kv_nb": kv_nb, "kv_inds": kv_inds, "diag": diag}
    if want_nabla:
        out["mnabla"] = mn
    return out


def block_mask_grid(q, k, grid, sta, thr, topk_ratio=None, row_ids=None):
    """Either estimator on the padded fractal layout of grid = (T, H, W): pooled means over
    tokens only.  Returns dict(kv_nb, kv_inds) (and diag for the CDF estimator)."""
    q, k = _f32(q), _f32(k)
    B, S, heads, D = q.shape
    T, H, W = grid
    nb = S // BLOCK
    if row_ids is None:
        lead, n, rid = (B, heads, nb), B * heads * nb, None
    else:
        rid = np.ascontiguousarray(row_ids, dtype=np.int64)
        lead, n = (rid.size,), rid.size
    kv_nb = np.empty(lead, np.int32)
    kv_inds = np.empty(lead + (nb,), np.int32)
    st = None if sta is None else np.ascontiguousarray(sta, dtype=np.uint8)
    lib = _load()
    if topk_ratio is None:
        diag = np.empty(lead + (3,), np.int64)
        rc = lib.orc_block_mask_grid(_ptr(q), _ptr(k), B, T, H, W, heads, D, _ptr(st), float(thr),
                                     _ptr(rid), n, _ptr(kv_nb), _ptr(kv_inds), None, _ptr(diag))
        out = {"kv_nb": kv_nb, "kv_inds": kv_inds, "diag": diag}
    else:
        rc = lib.orc_block_mask_topk_grid(_ptr(q), _ptr(k), B, T, H, W, heads, D, _ptr(st),
                                          float(topk_ratio), _ptr(rid), n, _ptr(kv_nb),
                                          _ptr(kv_inds))
        out = {"kv_nb": kv_nb, "kv_inds": kv_inds}
    if rc != 0:
        raise ValueError("oracle block_mask_grid: bad argument")
    return out


def attention_grid(q, k, v, grid, kv_nb, kv_inds, row_ids=None, scale=0.0):
    """attention() on the padded fractal layout of grid = (T, H, W): padding is never a key."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, S, heads, D = q.shape
    T, H, W = grid
    nb = S // BLOCK
    if row_ids is None:
        row_ids = np.arange(B * heads * nb, dtype=np.int64)
    row_ids = np.ascontiguousarray(row_ids, dtype=np.int64)
    kv_nb, kv_inds = _lists(kv_nb, kv_inds)
    o = np.zeros((row_ids.size, BLOCK, D), np.float64)
    rc = _load().orc_attention_grid(_ptr(q), _ptr(k), _ptr(v), B, T, H, W, heads, D, _ptr(kv_nb),
                                    _ptr(kv_inds), float(scale), _ptr(row_ids), row_ids.size,
                                    _ptr(o))
    if rc != 0:
        raise ValueError("oracle attention_grid: bad argument")
    return row_ids, o


def topk_count(nb, ratio) -> int:
    return _load().orc_topk_count(int(nb), float(ratio))


def block_mask_topk(q, k, sta, ratio, row_ids=None):
    """The top-k estimator variant (smooth-k, pooled scores, the ratio * nb largest per row,
    STA union).  Returns dict(kv_nb, kv_inds) shaped like block_mask's."""
    q, k = _f32(q), _f32(k)
    B, S, heads, D = q.shape
    nb = S // BLOCK
    if row_ids is None:
        lead, n, rid = (B, heads, nb), B * heads * nb, None
    else:
        rid = np.ascontiguousarray(row_ids, dtype=np.int64)
        lead, n = (rid.size,), rid.size
    kv_nb = np.empty(lead, np.int32)
    kv_inds = np.empty(lead + (nb,), np.int32)
    st = None if sta is None else np.ascontiguousarray(sta, dtype=np.uint8)
    rc = _load().orc_block_mask_topk(_ptr(q), _ptr(k), B, S, heads, D, _ptr(st), float(ratio),
                                     _ptr(rid), n, _ptr(kv_nb), _ptr(kv_inds))
    if rc != 0:
        raise ValueError("oracle block_mask_topk: bad argument")
    return {"kv_nb": kv_nb, "kv_inds": kv_inds}


def band_rows(diag, thr, width=1e-6):
    """Rows whose CDF at the cut (c_{i0-1} or c_{i0}) lies within ``width`` of fl32(1-thr)."""
    cut = float(np.float32(1.0 - thr))
    c_prev = diag[..., 1].astype(np.float64) / 2.0 ** FIX_BITS
    c_at = diag[..., 2].astype(np.float64) / 2.0 ** FIX_BITS
    return (np.abs(c_prev - cut) < width) | (np.abs(c_at - cut) < width)


# ---------------------------------------------------------------- O10
def attention(q, k, v, kv_nb, kv_inds, row_ids=None, scale=0.0):
    """Dense fp64 attention with disallowed 64x64 blocks at -inf.

    q, k, v [B,S,heads,D] fp32 values; row_ids: q-block row ids
    (b*heads + h)*nb + i (all rows if None).  Returns (row_ids, o) with
    o [len(row_ids), 64, D] fp64.
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, S, heads, D = q.shape
    nb = S // BLOCK
    if row_ids is None:
        row_ids = np.arange(B * heads * nb, dtype=np.int64)
    row_ids = np.ascontiguousarray(row_ids, dtype=np.int64)
    kv_nb = np.ascontiguousarray(kv_nb, dtype=np.int32)
    kv_inds = np.ascontiguousarray(kv_inds, dtype=np.int32)
    o = np.zeros((row_ids.size, BLOCK, D), np.float64)
    rc = _load().orc_attention(_ptr(q), _ptr(k), _ptr(v), B, S, heads, D, _ptr(kv_nb),
                               _ptr(kv_inds), float(scale), _ptr(row_ids), row_ids.size, _ptr(o))
    if rc != 0:
        raise ValueError("oracle attention: bad argument")
    return row_ids, o


# ---------------------------------------------------------------- O11 training pass
def _lists(kv_nb, kv_inds):
    return (np.ascontiguousarray(kv_nb, dtype=np.int32),
            np.ascontiguousarray(kv_inds, dtype=np.int32))


def _rows(row_ids, B, heads, nb):
    if row_ids is None:
        row_ids = np.arange(B * heads * nb, dtype=np.int64)
    return np.ascontiguousarray(row_ids, dtype=np.int64)


def attention_lse(q, k, kv_nb, kv_inds, row_ids=None, scale=0.0):
    """Natural-log log-sum-exp of the scaled allowed scores of every row of the listed
    q-blocks.  Returns (row_ids, lse [len(row_ids), 64] fp64)."""
    q, k = _f32(q), _f32(k)
    B, S, heads, D = q.shape
    row_ids = _rows(row_ids, B, heads, S // BLOCK)
    kv_nb, kv_inds = _lists(kv_nb, kv_inds)
    lse = np.zeros((row_ids.size, BLOCK), np.float64)
    rc = _load().orc_attention_lse(_ptr(q), _ptr(k), B, S, heads, D, _ptr(kv_nb), _ptr(kv_inds),
                                   float(scale), _ptr(row_ids), row_ids.size, _ptr(lse))
    if rc != 0:
        raise ValueError("oracle attention_lse: bad argument")
    return row_ids, lse


def attention_dq(q, k, v, dout, kv_nb, kv_inds, row_ids=None, scale=0.0):
    """dq of every row of the listed q-blocks.  Returns (row_ids, dq [n, 64, D] fp64)."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, S, heads, D = q.shape
    row_ids = _rows(row_ids, B, heads, S // BLOCK)
    kv_nb, kv_inds = _lists(kv_nb, kv_inds)
    dq = np.zeros((row_ids.size, BLOCK, D), np.float64)
    rc = _load().orc_attention_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, S, heads, D,
                                  _ptr(kv_nb), _ptr(kv_inds), float(scale), _ptr(row_ids),
                                  row_ids.size, _ptr(dq))
    if rc != 0:
        raise ValueError("oracle attention_dq: bad argument")
    return row_ids, dq


def attention_bwd(q, k, v, dout, kv_nb, kv_inds, scale=0.0):
    """The full training pass: dict(lse [B,heads,S], dq, dk, dv [B,S,heads,D]), fp64."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, S, heads, D = q.shape
    kv_nb, kv_inds = _lists(kv_nb, kv_inds)
    lse = np.zeros((B, heads, S), np.float64)
    dq, dk, dv = (np.zeros((B, S, heads, D), np.float64) for _ in range(3))
    rc = _load().orc_attention_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, S, heads, D,
                                   _ptr(kv_nb), _ptr(kv_inds), float(scale), _ptr(lse), _ptr(dq),
                                   _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle attention_bwd: bad argument")
    return {"lse": lse, "dq": dq, "dk": dk, "dv": dv}


def attention_dkdv(q, k, v, dout, kv_nb, kv_inds, col_ids, scale=0.0):
    """dk and dv of the 64 keys of each listed key block id (b*heads + h)*nb + j, from every
    query row whose block lists j.  Returns (col_ids, dk [n, 64, D], dv [n, 64, D]) fp64."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, S, heads, D = q.shape
    kv_nb, kv_inds = _lists(kv_nb, kv_inds)
    col_ids = np.ascontiguousarray(col_ids, dtype=np.int64)
    dk = np.zeros((col_ids.size, BLOCK, D), np.float64)
    dv = np.zeros((col_ids.size, BLOCK, D), np.float64)
    rc = _load().orc_attention_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, S, heads, D,
                                    _ptr(kv_nb), _ptr(kv_inds), float(scale), _ptr(col_ids),
                                    col_ids.size, _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle attention_dkdv: bad argument")
    return col_ids, dk, dv


def attention_bwd_grid(q, k, v, dout, grid, kv_nb, kv_inds, scale=0.0):
    """attention_bwd() on the padded fractal layout of grid = (T, H, W): the gradients of
    attention_grid's output; padding positions are never keys (their dk, dv are 0)."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, S, heads, D = q.shape
    T, H, W = grid
    kv_nb, kv_inds = _lists(kv_nb, kv_inds)
    lse = np.zeros((B, heads, S), np.float64)
    dq, dk, dv = (np.zeros((B, S, heads, D), np.float64) for _ in range(3))
    rc = _load().orc_attention_bwd_grid(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), B, T, H, W,
                                        heads, D, _ptr(kv_nb), _ptr(kv_inds), float(scale),
                                        _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle attention_bwd_grid: bad argument")
    return {"lse": lse, "dq": dq, "dk": dk, "dv": dv}


def rows_to_tokens(o_rows, row_ids, B, S, heads, D):
    """Scatter [n,64,D] q-block rows into a dense [B,S,heads,D] fp64 array (NaN elsewhere)."""
    nb = S // BLOCK
    out = np.full((B, S, heads, D), np.nan)
    for n, rid in enumerate(np.asarray(row_ids)):
        b, rem = divmod(int(rid), heads * nb)
        h, i = divmod(rem, nb)
        out[b, i * BLOCK:(i + 1) * BLOCK, h, :] = o_rows[n]
    return out


# ---------------------------------------------------------------- O12 quantized variant
def fp8_e4m3(x):
    """OCP FP8 e4m3fn codes (uint8) of float64 values, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, np.uint8)
    _load().orc_fp8_e4m3_vec(_ptr(x), _ptr(y), x.size)
    return y


def fp8_e4m3_value(codes):
    """float64 values of e4m3fn codes."""
    lib = _load()
    table = np.array([lib.orc_fp8_e4m3_value(c) for c in range(256)])
    return table[np.asarray(codes, dtype=np.uint8)]


def quant_qkv(q, k, v, grid=None):
    """INT8 q, k per 64-token block (k after subtracting its sequence mean), FP8 e4m3 v per
    channel.  q, k, v [B,S,heads,D] fp32 values.  Returns dict(q8, qs, k8, ks, v8, vs, km):
    q8, k8 [B,heads,nb,64,D] int8; qs, ks [B,heads,nb] fp32; v8 [B,heads,nb,D,64] uint8 codes;
    vs, km [B,heads,D] fp32.  grid=(T, H, W): the padded fractal layout of that grid, whose
    padding positions are not tokens (left out of the mean and the maxima, codes 0)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, S, heads, D = q.shape
    nb = S // BLOCK
    out = {"q8": np.empty((B, heads, nb, BLOCK, D), np.int8), "qs": np.empty((B, heads, nb), np.float32),
           "k8": np.empty((B, heads, nb, BLOCK, D), np.int8), "ks": np.empty((B, heads, nb), np.float32),
           "v8": np.empty((B, heads, nb, D, BLOCK), np.uint8), "vs": np.empty((B, heads, D), np.float32),
           "km": np.empty((B, heads, D), np.float32)}
    outs = [_ptr(out[n]) for n in ("q8", "qs", "k8", "ks", "v8", "vs", "km")]
    if grid is None:
        rc = _load().orc_quant_qkv(_ptr(q), _ptr(k), _ptr(v), B, S, heads, D, *outs)
    else:
        rc = _load().orc_quant_qkv_grid(_ptr(q), _ptr(k), _ptr(v), B, *grid, heads, D, *outs)
    if rc != 0:
        raise ValueError("oracle quant_qkv: bad argument")
    return out


def attention_q8(qz, kv_nb, kv_inds, row_ids=None, scale=0.0, grid=None):
    """The block-sparse attention on quant_qkv()'s codes (FP8 P, fp64 sums).
    Returns (row_ids, o [len(row_ids), 64, D] fp64) like attention().  grid=(T, H, W): the
    padded fractal layout of that grid (padding positions are never keys)."""
    q8 = np.ascontiguousarray(qz["q8"], dtype=np.int8)
    B, heads, nb, _, D = q8.shape
    S = nb * BLOCK
    arrs = [np.ascontiguousarray(qz[n], dtype=t) for n, t in
            (("qs", np.float32), ("k8", np.int8), ("ks", np.float32), ("v8", np.uint8),
             ("vs", np.float32))]
    row_ids = _rows(row_ids, B, heads, nb)
    kv_nb, kv_inds = _lists(kv_nb, kv_inds)
    o = np.zeros((row_ids.size, BLOCK, D), np.float64)
    if grid is None:
        rc = _load().orc_attention_q8(_ptr(q8), *[_ptr(a) for a in arrs], B, S, heads, D,
                                      _ptr(kv_nb), _ptr(kv_inds), float(scale), _ptr(row_ids),
                                      row_ids.size, _ptr(o))
    else:
        rc = _load().orc_attention_q8_grid(_ptr(q8), *[_ptr(a) for a in arrs], B, *grid, heads,
                                           D, _ptr(kv_nb), _ptr(kv_inds), float(scale),
                                           _ptr(row_ids), row_ids.size, _ptr(o))
    if rc != 0:
        raise ValueError("oracle attention_q8: bad argument")
    return row_ids, o


def dequant_qkv(qz):
    """The values the codes stand for, as fp64 [B,S,heads,D] arrays (q, k - k_mean, v)."""
    B, heads, nb, _, D = qz["q8"].shape
    S = nb * BLOCK
    q = (qz["q8"].astype(np.float64) * qz["qs"][..., None, None]).reshape(B, heads, S, D)
    k = (qz["k8"].astype(np.float64) * qz["ks"][..., None, None]).reshape(B, heads, S, D)
    vv = fp8_e4m3_value(qz["v8"]) * qz["vs"][:, :, None, :, None]      # [B,h,nb,D,64]
    v = vv.transpose(0, 1, 2, 4, 3).reshape(B, heads, S, D)
    return tuple(np.ascontiguousarray(x.transpose(0, 2, 1, 3)) for x in (q, k, v))
