"""MI355X-native NABLA hot path.

Python binding of ``libnabla.so`` (``include/nabla.h``): argument marshalling
only.  Every step runs in the library's HIP kernels; PyTorch provides device
memory and the current stream.  There is no CPU path: a missing library or a
tensor that is not on the GPU raises.

Calls (same names as the C ABI):
  nabla_fractal_permute(x, grid=None, inverse=False)
  nabla_sta_mask(tiles, window, device)
  nabla_block_mask(q, k, sta, thr=0.9)          -> (kv_nb, kv_inds)
  nabla_sparse_attn_fwd(q, k, v, kv_nb, kv_inds, scale=None, causal=False, tiles=None,
                        workspace=None, out=None) -> o
  nabla_quant_qkv(q, k, v)                      -> dict of INT8 / FP8 codes and scales
  nabla_sparse_attn_fwd_q8(qz, kv_nb, kv_inds, scale=None, tiles=None) -> o (bf16)
"""
import ctypes
import os

import torch

__all__ = ["nabla_fractal_permute", "nabla_sta_mask", "nabla_block_mask",
           "nabla_block_mask_workspace", "nabla_sparse_attn_fwd", "nabla_sparse_attn_workspace",
           "nabla_sparse_attn_bwd", "nabla_sparse_attn_bwd_workspace", "fractal_len",
           "nabla_quant_qkv", "nabla_sparse_attn_fwd_q8", "nabla_block_mask_natural",
           "nabla_sparse_attn_fwd_natural", "nabla_sparse_attn_fwd_noalloc",
           "NablaError", "lib",
           "LIB_PATH", "STATUS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnabla.so")
STATUS = {0: "NABLA_OK", 1: "NABLA_ERR_INVALID_ARG", 2: "NABLA_ERR_UNSUPPORTED",
          3: "NABLA_ERR_WORKSPACE", 4: "NABLA_ERR_HIP"}
_FP32, _BF16 = 0, 1
BLOCK = 64

_lib = None


class NablaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s (%s)" % (what, STATUS.get(status, status),
                                          lib().nabla_status_string(status).decode()))


def lib():
    """The loaded libnabla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libnabla.so is not built (%s); run "
                           "`python -m block_sparse_attention_fractal_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I, D, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_float, ctypes.c_size_t
    L.nabla_abi_version.restype = I
    L.nabla_status_string.argtypes = [I]
    L.nabla_status_string.restype = ctypes.c_char_p
    L.nabla_fractal_permute.argtypes = [P, P, I, I, I, I, I, I, I, I, P]
    L.nabla_fractal_permute.restype = I
    L.nabla_sta_mask.argtypes = [P, I, I, I, I, I, I, P]
    L.nabla_sta_mask.restype = I
    L.nabla_block_mask_workspace.argtypes = [I, I, I, I]
    L.nabla_block_mask_workspace.restype = Z
    L.nabla_block_mask.argtypes = [P, P, I, I, I, I, I, P, D, P, P, P, Z, P]
    L.nabla_block_mask.restype = I
    L.nabla_block_mask_topk.argtypes = [P, P, I, I, I, I, I, P, D, P, P, P, Z, P]
    L.nabla_block_mask_topk.restype = I
    L.nabla_block_mask_grid.argtypes = [P, P, I, I, I, I, I, I, I, P, D, D, P, P, P, Z, P]
    L.nabla_block_mask_grid.restype = I
    L.nabla_sparse_attn_workspace_grid.argtypes = [I, I, I, I, I]
    L.nabla_sparse_attn_workspace_grid.restype = Z
    L.nabla_sparse_attn_fwd_grid.argtypes = [P, P, P, I, I, I, I, I, I, I, P, P, F, P, P, P, Z, P]
    L.nabla_sparse_attn_fwd_grid.restype = I
    L.nabla_block_mask_natural.argtypes = [P, P, I, I, I, I, I, I, I, P, D, D, P, P, P, Z, P]
    L.nabla_block_mask_natural.restype = I
    L.nabla_sparse_attn_fwd_natural.argtypes = [P, P, P] + [I] * 7 + [P, P, F, P, P, P, Z, P]
    L.nabla_sparse_attn_fwd_natural.restype = I
    L.nabla_quant_qkv_natural.argtypes = [P, P, P] + [I] * 7 + [P] * 7 + [P, Z, P]
    L.nabla_quant_qkv_natural.restype = I
    L.nabla_sparse_attn_fwd_q8_natural.argtypes = [P] * 6 + [I] * 6 + [P, P, F, P, P, Z, P]
    L.nabla_sparse_attn_fwd_q8_natural.restype = I
    L.nabla_sparse_attn_workspace.argtypes = [I, I, I, I, I, I]
    L.nabla_sparse_attn_workspace.restype = Z
    L.nabla_sparse_attn_fwd.argtypes = [P, P, P, I, I, I, I, I, P, P, F, I, I, I, P, P, Z, P]
    L.nabla_sparse_attn_fwd.restype = I
    L.nabla_sparse_attn_fwd_noalloc.argtypes = [P, P, P, I, I, I, I, I, P, P, F, I, I, I, P, P]
    L.nabla_sparse_attn_fwd_noalloc.restype = I
    L.nabla_sparse_attn_fwd_lse.argtypes = [P, P, P, I, I, I, I, I, P, P, F, I, I, I, P, P, P, Z,
                                            P]
    L.nabla_sparse_attn_fwd_lse.restype = I
    L.nabla_sparse_attn_bwd_workspace.argtypes = [I, I, I]
    L.nabla_sparse_attn_bwd_workspace.restype = Z
    L.nabla_sparse_attn_bwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, F, P, P, P, P, Z, P]
    L.nabla_sparse_attn_bwd.restype = I
    L.nabla_sparse_attn_bwd_grid.argtypes = [P] * 6 + [I] * 7 + [P, P, F, P, P, P, P, Z, P]
    L.nabla_sparse_attn_bwd_grid.restype = I
    L.nabla_quant_qkv_workspace.argtypes = [I, I, I, I]
    L.nabla_quant_qkv_workspace.restype = Z
    L.nabla_quant_qkv.argtypes = [P, P, P, I, I, I, I, I, P, P, P, P, P, P, P, P, Z, P]
    L.nabla_quant_qkv.restype = I
    L.nabla_sparse_attn_q8_workspace.argtypes = [I, I, I, I, I, I]
    L.nabla_sparse_attn_q8_workspace.restype = Z
    L.nabla_sparse_attn_fwd_q8.argtypes = [P, P, P, P, P, P, I, I, I, I, P, P, F, I, I, I, P, P, Z,
                                           P]
    L.nabla_sparse_attn_fwd_q8.restype = I
    L.nabla_quant_qkv_grid.argtypes = [P, P, P] + [I] * 7 + [P] * 7 + [P, Z, P]
    L.nabla_quant_qkv_grid.restype = I
    L.nabla_sparse_attn_fwd_q8_grid.argtypes = [P] * 6 + [I] * 6 + [P, P, F, P, P, Z, P]
    L.nabla_sparse_attn_fwd_q8_grid.restype = I
    _lib = L
    return L


def _check(status, what):
    if status != 0:
        raise NablaError(status, what)


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor (no CPU path)" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _out(t, name, shape, dtype, device):
    """A caller-supplied output tensor: on `device`, contiguous, of exactly `dtype` and `shape`
    (the kernels write that many elements; anything smaller would be overrun)."""
    _dev(t, name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, not %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, not %s" % (name, tuple(shape), tuple(t.shape)))
    if t.device != device:
        raise ValueError("%s must be on %s, not %s" % (name, device, t.device))
    return t


def _same_device(device, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError("%s must be on %s, not %s" % (name, device, t.device))


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _FP32
    raise TypeError("unsupported dtype %s (bfloat16 or float32)" % t.dtype)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _workspace(ws, need, device):
    """The caller's workspace (a uint8 GPU tensor on `device`; its size is checked by the
    library) or a new one of `need` bytes."""
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _dev(ws, "workspace")
    if ws.dtype != torch.uint8:
        raise TypeError("workspace must be uint8")
    _same_device(device, workspace=ws)
    return ws


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def fractal_len(T, H, W):
    """Tokens of the fractal layout of a T x H x W grid: T * ceil(H/8) * ceil(W/8) * 64."""
    return T * ((H + 7) // 8) * ((W + 7) // 8) * BLOCK


def nabla_fractal_permute(x, grid=None, inverse=False, out=None):
    """Fractal token order (8 x 8 patches -> runs of 64 tokens).

    Forward: x [B, T, H, W, heads, D] -> [B, fractal_len(T, H, W), heads, D]; when 8 does
    not divide H or W the partial patches are padded with zeros.
    Inverse: x [B, S, heads, D] with grid=(T, H, W) -> [B, T, H, W, heads, D].
    """
    _dev(x, "x")
    if not inverse:
        B, T, H, W, heads, D = x.shape
        shape = (B, fractal_len(T, H, W), heads, D)
    else:
        B, S, heads, D = x.shape
        T, H, W = grid
        if fractal_len(T, H, W) != S:
            raise ValueError("grid %s does not match S=%d" % (grid, S))
        shape = (B, T, H, W, heads, D)
    y = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else \
        _out(out, "out", shape, x.dtype, x.device)
    _check(lib().nabla_fractal_permute(_p(x), _p(y), _dtype_code(x), B, T, H, W, heads, D,
                                       int(bool(inverse)), _stream(x)), "nabla_fractal_permute")
    return y


def nabla_sta_mask(tiles, window, device="cuda"):
    """STA block mask [nb, nb] uint8 for a (Tt, Ht, Wt) tile grid and (win_t, win_h, win_w)."""
    Tt, Ht, Wt = tiles
    nb = Tt * Ht * Wt
    sta = torch.empty((nb, nb), dtype=torch.uint8, device=device)
    _check(lib().nabla_sta_mask(_p(sta), Tt, Ht, Wt, *window, _stream(sta)), "nabla_sta_mask")
    return sta


def nabla_block_mask_workspace(B, S, heads, D):
    return lib().nabla_block_mask_workspace(B, S, heads, D)


def nabla_block_mask(q, k, sta=None, thr=0.9, workspace=None, out=None, topk_ratio=None,
                     grid=None):
    """NABLA estimator: q, k [B, S, heads, D] -> (kv_nb [B,heads,nb] int32, kv_inds [B,heads,nb,nb] int32).

    The first kv_nb entries of each kv_inds row are the kept blocks, ascending.
    With topk_ratio set, the top-k variant runs instead (nabla_block_mask_topk:
    smooth-k pooled scores, the int(topk_ratio * nb) largest per row); thr is then
    not used.  grid=(T, H, W): q, k are the padded fractal layout of that latent grid
    (nabla_block_mask_grid: blocks average their tokens only).
    """
    _dev(q, "q")
    _dev(k, "k")
    if q.shape != k.shape or q.dtype != k.dtype:
        raise ValueError("q and k must match in shape and dtype")
    B, S, heads, D = q.shape
    nb = S // BLOCK
    if sta is not None:
        _dev(sta, "sta")
        if sta.dtype != torch.uint8 or sta.numel() != nb * nb:
            raise ValueError("sta must be uint8 with nb*nb = %d elements" % (nb * nb))
    need = lib().nabla_block_mask_workspace(B, S, heads, D)
    ws = _workspace(workspace, need, q.device)
    _same_device(q.device, k=k, sta=sta)
    if out is None:
        kv_nb = torch.empty((B, heads, nb), dtype=torch.int32, device=q.device)
        kv_inds = torch.empty((B, heads, nb, nb), dtype=torch.int32, device=q.device)
    else:
        kv_nb = _out(out[0], "kv_nb", (B, heads, nb), torch.int32, q.device)
        kv_inds = _out(out[1], "kv_inds", (B, heads, nb, nb), torch.int32, q.device)
    if grid is not None:
        T, H, W = grid
        if fractal_len(T, H, W) != S:
            raise ValueError("grid %s does not match S=%d" % (grid, S))
        _check(lib().nabla_block_mask_grid(_p(q), _p(k), _dtype_code(q), B, T, H, W, heads, D,
                                           _p(sta), float(thr),
                                           -1.0 if topk_ratio is None else float(topk_ratio),
                                           _p(kv_nb), _p(kv_inds), _p(ws), ws.numel(),
                                           _stream(q)), "nabla_block_mask_grid")
        return kv_nb, kv_inds
    if topk_ratio is not None:
        _check(lib().nabla_block_mask_topk(_p(q), _p(k), _dtype_code(q), B, S, heads, D, _p(sta),
                                           float(topk_ratio), _p(kv_nb), _p(kv_inds), _p(ws),
                                           ws.numel(), _stream(q)), "nabla_block_mask_topk")
        return kv_nb, kv_inds
    _check(lib().nabla_block_mask(_p(q), _p(k), _dtype_code(q), B, S, heads, D, _p(sta),
                                  float(thr), _p(kv_nb), _p(kv_inds), _p(ws), ws.numel(),
                                  _stream(q)), "nabla_block_mask")
    return kv_nb, kv_inds


def nabla_sparse_attn_workspace(B, S, heads, tiles=None):
    """Bytes of workspace nabla_sparse_attn_fwd needs (0 for invalid sizes)."""
    Tt, Ht, Wt = (0, 0, 0) if tiles is None else tiles
    return lib().nabla_sparse_attn_workspace(B, S, heads, Tt, Ht, Wt)


def nabla_sparse_attn_fwd(q, k, v, kv_nb, kv_inds, scale=None, causal=False, tiles=None,
                          workspace=None, out=None, lse=None, grid=None):
    """Block-sparse attention over the listed 64 x 64 blocks: o [B, S, heads, D] (q's dtype).

    tiles: the (Tt, Ht, Wt) tile grid of the blocks (lets neighbouring query
    blocks share K/V tiles on chip); None if unknown.  workspace: a uint8 GPU
    tensor of at least nabla_sparse_attn_workspace() bytes (allocated if None).
    lse: None, or a float32 GPU tensor [B, heads, S] that receives each row's
    log-sum-exp (natural log), as the backward needs it.  grid=(T, H, W): q, k, v are
    the padded fractal layout of that latent grid (nabla_sparse_attn_fwd_grid: padding
    is never a key; tiles is then implied).
    """
    if causal:
        raise ValueError("causal=True is not available: the block lists define the whole "
                         "mask and carry no causal part")
    for name, t in (("q", q), ("k", k), ("v", v), ("kv_nb", kv_nb), ("kv_inds", kv_inds)):
        _dev(t, name)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must match in shape and dtype")
    if kv_nb.dtype != torch.int32 or kv_inds.dtype != torch.int32:
        raise TypeError("kv_nb and kv_inds must be int32")
    B, S, heads, D = q.shape
    nb = S // BLOCK
    if kv_nb.numel() != B * heads * nb or kv_inds.numel() != B * heads * nb * nb:
        raise ValueError("kv lists do not match q's shape")
    _same_device(q.device, k=k, v=v, kv_nb=kv_nb, kv_inds=kv_inds, lse=lse)
    o = torch.empty_like(q) if out is None else _out(out, "out", q.shape, q.dtype, q.device)
    if grid is not None:
        T, H, W = grid
        if fractal_len(T, H, W) != S:
            raise ValueError("grid %s does not match S=%d" % (grid, S))
        tiles = (T, (H + 7) // 8, (W + 7) // 8)
    Tt, Ht, Wt = (0, 0, 0) if tiles is None else tiles
    workspace = _workspace(workspace, lib().nabla_sparse_attn_workspace(B, S, heads, Tt, Ht, Wt),
                           q.device)
    if lse is not None:
        _dev(lse, "lse")
        if lse.dtype != torch.float32 or lse.numel() != B * heads * S:
            raise ValueError("lse must be float32 with B * heads * S elements")
    if grid is not None:
        _check(lib().nabla_sparse_attn_fwd_grid(_p(q), _p(k), _p(v), _dtype_code(q), B, *grid,
                                                heads, D, _p(kv_nb), _p(kv_inds),
                                                0.0 if scale is None else float(scale), _p(o),
                                                None if lse is None else _p(lse), _p(workspace),
                                                workspace.numel(), _stream(q)),
               "nabla_sparse_attn_fwd_grid")
        return o
    _check(lib().nabla_sparse_attn_fwd_lse(_p(q), _p(k), _p(v), _dtype_code(q), B, S, heads, D,
                                           _p(kv_nb), _p(kv_inds),
                                           0.0 if scale is None else float(scale), Tt, Ht, Wt,
                                           _p(o), None if lse is None else _p(lse),
                                           _p(workspace), workspace.numel(), _stream(q)),
           "nabla_sparse_attn_fwd")
    return o


def nabla_sparse_attn_fwd_noalloc(q, k, v, kv_nb, kv_inds, out, scale=None, tiles=None):
    """nabla_sparse_attn_fwd into the caller's `out` with no allocation at all: the library
    keeps the call's work schedule in a static 1 MiB device array per GPU (calls that overlap
    on one GPU race).  Raises NablaError (NABLA_ERR_WORKSPACE) when the schedule of this
    shape does not fit."""
    for name, t in (("q", q), ("k", k), ("v", v), ("kv_nb", kv_nb), ("kv_inds", kv_inds)):
        _dev(t, name)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must match in shape and dtype")
    if kv_nb.dtype != torch.int32 or kv_inds.dtype != torch.int32:
        raise TypeError("kv_nb and kv_inds must be int32")
    B, S, heads, D = q.shape
    nb = S // BLOCK
    if kv_nb.numel() != B * heads * nb or kv_inds.numel() != B * heads * nb * nb:
        raise ValueError("kv lists do not match q's shape")
    _same_device(q.device, k=k, v=v, kv_nb=kv_nb, kv_inds=kv_inds)
    o = _out(out, "out", q.shape, q.dtype, q.device)
    Tt, Ht, Wt = (0, 0, 0) if tiles is None else tiles
    _check(lib().nabla_sparse_attn_fwd_noalloc(_p(q), _p(k), _p(v), _dtype_code(q), B, S, heads,
                                               D, _p(kv_nb), _p(kv_inds),
                                               0.0 if scale is None else float(scale), Tt, Ht,
                                               Wt, _p(o), _stream(q)),
           "nabla_sparse_attn_fwd_noalloc")
    return o


def _natural_shape(q, name="q"):
    if q.dim() != 6:
        raise ValueError("%s must be natural-order [B, T, H, W, heads, D]" % name)
    B, T, H, W, heads, D = q.shape
    if H % 8 or W % 8:
        raise ValueError("natural-order calls need H and W multiples of 8 (whole patches); "
                         "use nabla_fractal_permute and the grid= calls instead")
    return B, T, H, W, heads, D


def nabla_block_mask_natural(q, k, sta=None, thr=0.9, topk_ratio=None, workspace=None,
                             out=None):
    """Either estimator on q, k in natural order [B, T, H, W, heads, D] (H, W multiples of 8),
    with the fractal permute folded into the pooling (nabla_block_mask_natural): the lists
    over fractal block indices equal nabla_block_mask's on the permuted q and k."""
    _dev(q, "q")
    _dev(k, "k")
    if q.shape != k.shape or q.dtype != k.dtype:
        raise ValueError("q and k must match in shape and dtype")
    B, T, H, W, heads, D = _natural_shape(q)
    nb = T * (H // 8) * (W // 8)
    S = nb * BLOCK
    if sta is not None:
        _dev(sta, "sta")
        if sta.dtype != torch.uint8 or sta.numel() != nb * nb:
            raise ValueError("sta must be uint8 with nb*nb = %d elements" % (nb * nb))
    need = lib().nabla_block_mask_workspace(B, S, heads, D)
    ws = _workspace(workspace, need, q.device)
    _same_device(q.device, k=k, sta=sta)
    if out is None:
        kv_nb = torch.empty((B, heads, nb), dtype=torch.int32, device=q.device)
        kv_inds = torch.empty((B, heads, nb, nb), dtype=torch.int32, device=q.device)
    else:
        kv_nb = _out(out[0], "kv_nb", (B, heads, nb), torch.int32, q.device)
        kv_inds = _out(out[1], "kv_inds", (B, heads, nb, nb), torch.int32, q.device)
    _check(lib().nabla_block_mask_natural(_p(q), _p(k), _dtype_code(q), B, T, H, W, heads, D,
                                          _p(sta), float(thr),
                                          -1.0 if topk_ratio is None else float(topk_ratio),
                                          _p(kv_nb), _p(kv_inds), _p(ws), ws.numel(),
                                          _stream(q)), "nabla_block_mask_natural")
    return kv_nb, kv_inds


def nabla_sparse_attn_fwd_natural(q, k, v, kv_nb, kv_inds, scale=None, workspace=None,
                                  out=None, lse=None):
    """The forward on q, k, v in natural order [B, T, H, W, heads, D] (H, W multiples of 8),
    with the fractal permutes folded into the kernel (nabla_sparse_attn_fwd_natural):
    o in natural order, bit-identical to the inverse permute of nabla_sparse_attn_fwd on
    the permuted inputs; lse (optional, [B, heads, S] fp32) stays in fractal order."""
    for name, t in (("q", q), ("k", k), ("v", v), ("kv_nb", kv_nb), ("kv_inds", kv_inds)):
        _dev(t, name)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must match in shape and dtype")
    if kv_nb.dtype != torch.int32 or kv_inds.dtype != torch.int32:
        raise TypeError("kv_nb and kv_inds must be int32")
    B, T, H, W, heads, D = _natural_shape(q)
    nb = T * (H // 8) * (W // 8)
    S = nb * BLOCK
    if kv_nb.numel() != B * heads * nb or kv_inds.numel() != B * heads * nb * nb:
        raise ValueError("kv lists do not match q's shape")
    _same_device(q.device, k=k, v=v, kv_nb=kv_nb, kv_inds=kv_inds, lse=lse)
    o = torch.empty_like(q) if out is None else _out(out, "out", q.shape, q.dtype, q.device)
    workspace = _workspace(workspace, lib().nabla_sparse_attn_workspace_grid(B, T, H, W, heads),
                           q.device)
    if lse is not None:
        _dev(lse, "lse")
        if lse.dtype != torch.float32 or lse.numel() != B * heads * S:
            raise ValueError("lse must be float32 with B * heads * S elements")
    _check(lib().nabla_sparse_attn_fwd_natural(_p(q), _p(k), _p(v), _dtype_code(q), B, T, H, W,
                                               heads, D, _p(kv_nb), _p(kv_inds),
                                               0.0 if scale is None else float(scale), _p(o),
                                               None if lse is None else _p(lse),
                                               _p(workspace), workspace.numel(), _stream(q)),
           "nabla_sparse_attn_fwd_natural")
    return o


def nabla_sparse_attn_bwd_workspace(B, S, heads):
    """Bytes of workspace nabla_sparse_attn_bwd needs (0 if the sizes are invalid)."""
    return lib().nabla_sparse_attn_bwd_workspace(B, S, heads)


def nabla_sparse_attn_bwd(q, k, v, o, dout, lse, kv_nb, kv_inds, scale=None, workspace=None,
                          dq=None, dk=None, dv=None, grid=None):
    """Gradients (dq, dk, dv) of the block-sparse attention for output gradient dout.

    q, k, v, o, dout: bf16 [B, S, heads, D] GPU tensors (o and lse from
    nabla_sparse_attn_fwd(..., lse=...) on the same inputs, lists and scale).
    grid=(T, H, W): the padded fractal layout of that latent grid
    (nabla_sparse_attn_bwd_grid: padding is never a key; o and lse from
    nabla_sparse_attn_fwd(..., grid=grid)).
    Returns three new tensors (or the given dq, dk, dv).
    """
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("lse", lse),
                    ("kv_nb", kv_nb), ("kv_inds", kv_inds)):
        _dev(t, name)
    if not (q.shape == k.shape == v.shape == o.shape == dout.shape):
        raise ValueError("q, k, v, o, dout must have one shape")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise ValueError("q, k, v, o, dout must have one dtype")
    if kv_nb.dtype != torch.int32 or kv_inds.dtype != torch.int32:
        raise TypeError("kv_nb and kv_inds must be int32")
    B, S, heads, D = q.shape
    nb = S // BLOCK
    if kv_nb.numel() != B * heads * nb or kv_inds.numel() != B * heads * nb * nb:
        raise ValueError("kv lists do not match q's shape")
    if lse.dtype != torch.float32 or lse.numel() != B * heads * S:
        raise ValueError("lse must be float32 with B * heads * S elements")
    if grid is not None and fractal_len(*grid) != S:
        raise ValueError("grid %s does not match S=%d" % (grid, S))
    _same_device(q.device, k=k, v=v, o=o, dout=dout, lse=lse, kv_nb=kv_nb, kv_inds=kv_inds)
    outs = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        outs.append(torch.empty_like(q) if t is None else _out(t, name, q.shape, q.dtype,
                                                                q.device))
    workspace = _workspace(workspace, lib().nabla_sparse_attn_bwd_workspace(B, S, heads),
                           q.device)
    sc = 0.0 if scale is None else float(scale)
    if grid is not None:
        _check(lib().nabla_sparse_attn_bwd_grid(_p(q), _p(k), _p(v), _p(o), _p(dout), _p(lse),
                                                _dtype_code(q), B, *grid, heads, D, _p(kv_nb),
                                                _p(kv_inds), sc, _p(outs[0]), _p(outs[1]),
                                                _p(outs[2]), _p(workspace), workspace.numel(),
                                                _stream(q)),
               "nabla_sparse_attn_bwd_grid")
        return tuple(outs)
    _check(lib().nabla_sparse_attn_bwd(_p(q), _p(k), _p(v), _p(o), _p(dout), _p(lse),
                                       _dtype_code(q), B, S, heads, D, _p(kv_nb), _p(kv_inds),
                                       sc, _p(outs[0]), _p(outs[1]), _p(outs[2]), _p(workspace),
                                       workspace.numel(), _stream(q)),
           "nabla_sparse_attn_bwd")
    return tuple(outs)


def nabla_quant_qkv(q, k, v, workspace=None, grid=None):
    """The quantizer of the quantized variant: q, k, v [B, S, heads, D] (bf16 or fp32) ->
    dict(q8, q_scale, k8, k_scale, v8, v_scale, k_mean) with q8, k8 int8 [B, heads, nb, 64, D]
    (k after subtracting its sequence mean), q_scale, k_scale float32 [B, heads, nb], v8 uint8
    e4m3 codes [B, heads, nb, D, 64] (blocks transposed), v_scale, k_mean float32 [B, heads, D].
    grid=(T, H, W): the padded fractal layout of that latent grid (nabla_quant_qkv_grid:
    padding positions are not tokens).  q, k, v of 6 dims [B, T, H, W, heads, D] (H, W
    multiples of 8): natural order, read in place of their permute (nabla_quant_qkv_natural;
    the same codes).
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        _dev(t, name)
    if not (q.shape == k.shape == v.shape) or not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must match in shape and dtype")
    nat = None
    if q.dim() == 6:
        B, T, H, W, heads, D = _natural_shape(q)
        nat = (T, H, W)
        S = T * H * W
    else:
        B, S, heads, D = q.shape
    nb = S // BLOCK
    dev = q.device
    out = {"q8": torch.empty((B, heads, nb, BLOCK, D), dtype=torch.int8, device=dev),
           "q_scale": torch.empty((B, heads, nb), dtype=torch.float32, device=dev),
           "k8": torch.empty((B, heads, nb, BLOCK, D), dtype=torch.int8, device=dev),
           "k_scale": torch.empty((B, heads, nb), dtype=torch.float32, device=dev),
           "v8": torch.empty((B, heads, nb, D, BLOCK), dtype=torch.uint8, device=dev),
           "v_scale": torch.empty((B, heads, D), dtype=torch.float32, device=dev),
           "k_mean": torch.empty((B, heads, D), dtype=torch.float32, device=dev)}
    _same_device(dev, k=k, v=v)
    workspace = _workspace(workspace, lib().nabla_quant_qkv_workspace(B, S, heads, D), dev)
    codes = [_p(out[n]) for n in ("q8", "q_scale", "k8", "k_scale", "v8", "v_scale", "k_mean")]
    if nat is not None:
        _check(lib().nabla_quant_qkv_natural(_p(q), _p(k), _p(v), _dtype_code(q), B, *nat, heads,
                                             D, *codes, _p(workspace), workspace.numel(),
                                             _stream(q)),
               "nabla_quant_qkv_natural")
        return out
    if grid is not None:
        if fractal_len(*grid) != S:
            raise ValueError("grid %s does not match S=%d" % (grid, S))
        _check(lib().nabla_quant_qkv_grid(_p(q), _p(k), _p(v), _dtype_code(q), B, *grid, heads,
                                          D, *codes, _p(workspace), workspace.numel(),
                                          _stream(q)),
               "nabla_quant_qkv_grid")
        return out
    _check(lib().nabla_quant_qkv(_p(q), _p(k), _p(v), _dtype_code(q), B, S, heads, D, *codes,
                                 _p(workspace), workspace.numel(), _stream(q)),
           "nabla_quant_qkv")
    return out


def nabla_sparse_attn_fwd_q8(qz, kv_nb, kv_inds, scale=None, tiles=None, workspace=None,
                             out=None, grid=None, natural=None):
    """Block-sparse attention of the quantized variant over the listed 64 x 64 blocks, on the
    codes of nabla_quant_qkv (qz): o [B, S, heads, D] bfloat16.  grid=(T, H, W): the padded
    fractal layout of that latent grid (nabla_sparse_attn_fwd_q8_grid: padding is never a
    key; tiles is then implied).  natural=(T, H, W) (H, W multiples of 8): o is written in
    natural order [B, T, H, W, heads, D] (nabla_sparse_attn_fwd_q8_natural)."""
    names = ("q8", "q_scale", "k8", "k_scale", "v8", "v_scale")
    for name in names:
        _dev(qz[name], name)
    _dev(kv_nb, "kv_nb")
    _dev(kv_inds, "kv_inds")
    q8 = qz["q8"]
    if q8.dtype != torch.int8 or q8.dim() != 5 or q8.shape[3] != BLOCK:
        raise ValueError("q8 must be int8 [B, heads, nb, 64, D]")
    B, heads, nb, _, D = q8.shape
    S = nb * BLOCK
    if kv_nb.dtype != torch.int32 or kv_inds.dtype != torch.int32:
        raise TypeError("kv_nb and kv_inds must be int32")
    if kv_nb.numel() != B * heads * nb or kv_inds.numel() != B * heads * nb * nb:
        raise ValueError("kv lists do not match the codes' shape")
    if qz["k8"].shape != q8.shape or qz["v8"].numel() != q8.numel():
        raise ValueError("q8, k8, v8 must have one shape")
    for name, dt, n in (("k8", torch.int8, q8.numel()), ("v8", torch.uint8, q8.numel()),
                        ("q_scale", torch.float32, B * heads * nb),
                        ("k_scale", torch.float32, B * heads * nb),
                        ("v_scale", torch.float32, B * heads * D)):
        if qz[name].dtype != dt or qz[name].numel() != n:
            raise ValueError("%s must be %s with %d elements" % (name, dt, n))
    if natural is not None:
        T, H, W = natural
        if H % 8 or W % 8 or T * H * W != S:
            raise ValueError("natural grid %s must be whole patches with T*H*W = S" % (natural,))
        grid_shape = (B, T, H, W, heads, D)
        tiles = (T, H // 8, W // 8)
    else:
        grid_shape = (B, S, heads, D)
    _same_device(q8.device, kv_nb=kv_nb, kv_inds=kv_inds,
                 **{n: qz[n] for n in names if n != "q8"})
    o = torch.empty(grid_shape, dtype=torch.bfloat16, device=q8.device) if out is None \
        else _out(out, "out", grid_shape, torch.bfloat16, q8.device)
    if grid is not None:
        T, H, W = grid
        if fractal_len(T, H, W) != S:
            raise ValueError("grid %s does not match S=%d" % (grid, S))
        tiles = (T, (H + 7) // 8, (W + 7) // 8)
    Tt, Ht, Wt = (0, 0, 0) if tiles is None else tiles
    workspace = _workspace(workspace,
                           lib().nabla_sparse_attn_q8_workspace(B, S, heads, Tt, Ht, Wt),
                           q8.device)
    if natural is not None:
        _check(lib().nabla_sparse_attn_fwd_q8_natural(*[_p(qz[n]) for n in names], B, *natural,
                                                      heads, D, _p(kv_nb), _p(kv_inds),
                                                      0.0 if scale is None else float(scale),
                                                      _p(o), _p(workspace), workspace.numel(),
                                                      _stream(q8)),
               "nabla_sparse_attn_fwd_q8_natural")
        return o
    if grid is not None:
        _check(lib().nabla_sparse_attn_fwd_q8_grid(*[_p(qz[n]) for n in names], B, *grid, heads,
                                                   D, _p(kv_nb), _p(kv_inds),
                                                   0.0 if scale is None else float(scale), _p(o),
                                                   _p(workspace), workspace.numel(),
                                                   _stream(q8)),
               "nabla_sparse_attn_fwd_q8_grid")
        return o
    _check(lib().nabla_sparse_attn_fwd_q8(*[_p(qz[n]) for n in names], B, S, heads, D,
                                          _p(kv_nb), _p(kv_inds),
                                          0.0 if scale is None else float(scale), Tt, Ht, Wt,
                                          _p(o), _p(workspace), workspace.numel(), _stream(q8)),
           "nabla_sparse_attn_fwd_q8")
    return o
