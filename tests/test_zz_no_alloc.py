"""The no-allocation forward (nabla_sparse_attn_fwd_noalloc, through the C ABI) against the
forward with a caller workspace (nabla_sparse_attn_fwd) on the same inputs and lists.

Both run the same kernels on the same schedule, so the outputs must be equal bit for bit.
Two calls in a row, the second on a smaller input, show that the static scratch keeps no
state a later call depends on (the schedule's counter is reset by the plan kernel of every
call).
"""
import ctypes
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import block_sparse_attention_fractal_amd as nabla
from block_sparse_attention_fractal_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def P(t):
    return ctypes.c_void_p(t.data_ptr())


def inputs(dev, B, T, Ht, Wt, heads, D, seed):
    rng = np.random.default_rng(seed)
    S = T * Ht * Wt * 64
    nb = S // 64
    q, k, v = (synth.round_bf16(rng.standard_normal((B, S, heads, D)).astype(np.float32))
               for _ in range(3))
    kv_nb, kv_inds = synth.random_lists(rng, B, heads, nb, 0.3)
    kv_nb[0, 0, 1] = 0          # an empty row: o = 0
    kv_nb[-1, -1, nb - 1] = nb  # a row that lists every block
    g = [torch.from_numpy(a).to(torch.bfloat16).to(dev) for a in (q, k, v)]
    return g, torch.from_numpy(kv_nb).to(dev), torch.from_numpy(kv_inds).to(dev), (T, Ht, Wt)


def test_noalloc_matches_workspace_call_twice():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    dev = torch.device("cuda:0")
    L = nabla.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    # the second call is smaller (fewer heads, frames and blocks) than the first
    for B, T, Ht, Wt, heads, D, seed in ((2, 6, 3, 4, 4, 128, 61), (1, 3, 2, 3, 2, 64, 62)):
        (q, k, v), kv_nb, kv_inds, tiles = inputs(dev, B, T, Ht, Wt, heads, D, seed)
        S = q.shape[1]
        say("[noalloc] B=%d S=%d heads=%d D=%d tiles=%s" % (B, S, heads, D, tiles))
        o_ref = torch.empty_like(q)
        ws = torch.empty(L.nabla_sparse_attn_workspace(B, S, heads, *tiles), dtype=torch.uint8,
                         device=dev)
        rc = L.nabla_sparse_attn_fwd(P(q), P(k), P(v), 1, B, S, heads, D, P(kv_nb), P(kv_inds),
                                     0.0, *tiles, P(o_ref), P(ws), ws.numel(), stream)
        assert rc == 0
        o = torch.full_like(q, float("nan"))
        rc = L.nabla_sparse_attn_fwd_noalloc(P(q), P(k), P(v), 1, B, S, heads, D, P(kv_nb),
                                             P(kv_inds), 0.0, *tiles, P(o), stream)
        assert rc == 0
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)
        assert torch.all(o[0, 64:128, 0] == 0)
        # the Python wrapper of the same call
        o2 = nabla.nabla_sparse_attn_fwd_noalloc(q, k, v, kv_nb, kv_inds, torch.empty_like(q),
                                                 tiles=tiles)
        torch.cuda.synchronize()
        assert torch.equal(o2, o_ref)
    # a shape whose schedule does not fit the static scratch is rejected before any launch
    rc = L.nabla_sparse_attn_fwd_noalloc(P(q), P(k), P(v), 1, 546, 61440, 1, 128, P(kv_nb),
                                         P(kv_inds), 0.0, 16, 6, 10, P(o), stream)
    assert rc == 3
