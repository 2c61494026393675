#!/usr/bin/env python3
"""Benchmark of the NABLA hot path on one MI355X.

One step = the whole path over one batch of synthetic video-shaped inputs
already resident in HBM (natural token order):
  STA block mask -> fractal permute of q, k, v -> nabla_block_mask (pool,
  scores, softmax, CDF cut, STA union, kv lists) -> nabla_sparse_attn_fwd ->
  inverse permute of o.
The default workload is the 720p shape (B=1, 16 heads, D=128, 16 x 48 x 80
latents = 61440 tokens, 960 blocks, thr 0.9, STA |dt|<=2, |dh|<=1, |dw|<=1).

Prints one JSON line.  ``value`` is the effective throughput of the step:
kept-block attention FLOPs (4 * 64 * 64 * D per kept (query block, kv block)
pair) divided by the step time.  ``roofline`` describes the dominant kernel
(the sparse attention forward) from HIP events around its launches in the
timed steps; ``cpu_baseline`` is the CPU oracle on the host cores, on a
bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NABLA sparse attn fwd effective TFLOP/s + mask ms at 720p shape, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (int8: 5000 TOP/s)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
ATTN_SRC = [os.path.join(ROOT, "block_sparse_attention_fractal_amd", "csrc", f)
            for f in ("sparse_attn.hip", "attn_tile.h", "nabla_device.h")]
PMC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_720p_pmc.txt")
Q8_SRC = [os.path.join(ROOT, "block_sparse_attention_fractal_amd", "csrc", f)
          for f in ("sparse_attn_q8.hip", "attn_tile.h", "nabla_device.h")]
Q8_PMC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_q8_720p_pmc.txt")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="720p", help="tiny | small | 720p | long | small_pad | 720p_pad")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=768,
                    help="query blocks in the oracle attention sample")
    ap.add_argument("--sweep", action="store_true",
                    help="the sparsity sweep on the 720p shape and the long clip, one line per run")
    ap.add_argument("--topk", type=float, default=None, metavar="RATIO",
                    help="the top-k estimator variant with this ratio instead of NABLA's CDF cut "
                         "(a variant line, not the headline)")
    ap.add_argument("--q8", action="store_true",
                    help="the quantized variant: INT8 Q K^T / FP8 P V attention on the codes of "
                         "nabla_quant_qkv (quantizer inside the step; a variant line)")
    ap.add_argument("--bwd", action="store_true",
                    help="the training pass instead: forward with lse, then the backward (one line)")
    ap.add_argument("--separate-permutes", action="store_true",
                    help="permute q, k, v and o with nabla_fractal_permute around fractal-order "
                         "calls, instead of the natural-order calls that fold the permutes into "
                         "the estimator's and the attention's addressing (grids of whole "
                         "patches; padded grids always permute)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def src_sha(paths):
    """Hash of the attention kernel's sources (the kernel file and the headers it includes)."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(pmc_file=PMC_FILE, src=ATTN_SRC):
    """HBM bytes per attention launch from the committed PMC summary, if it matches this source."""
    if not os.path.exists(pmc_file):
        return None
    kv = {}
    for line in open(pmc_file):
        if "=" in line and not line.lstrip().startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_sha") != src_sha(src):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def lists_vs_oracle(m, g_nb, g_inds, thr):
    """The GPU lists against the oracle estimator's (m): kv_nb and the kv_inds sets on every
    row; rows whose CDF lies within 1e-6 of the cut (band rows) are counted, listed, and
    compared separately."""
    import oracle
    band = oracle.band_rows(m["diag"], thr).reshape(-1)
    o_nb = m["kv_nb"].reshape(-1)
    nb = g_inds.shape[-1]
    live = np.arange(nb)[None, :] < o_nb[:, None]
    same = (g_nb.reshape(-1) == o_nb) & np.all(
        (g_inds.reshape(-1, nb) == m["kv_inds"].reshape(-1, nb)) | ~live, axis=1)
    return {"band_rows": int(band.sum()),
            "band_row_ids": np.flatnonzero(band)[:64].tolist(),
            "lists_match_gpu": bool(same[~band].all()),
            "lists_match_gpu_in_band": bool(same[band].all()),
            "rows_compared": int(same.size)}


def cpu_baseline(w, q, k, v, sta_np, g_nb, g_inds, rows, flops_per_pair):
    """The oracle (untuned) on the host: full estimator, attention on a row sample."""
    import oracle
    from block_sparse_attention_fractal_amd import synth  # noqa: F401  (inputs only)
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    f = lambda a: oracle.fractal_permute(a).reshape(w.B, w.S, w.heads, w.D)
    t0 = time.perf_counter()
    qf, kf, vf = f(q), f(k), f(v)
    t_perm = time.perf_counter() - t0
    t0 = time.perf_counter()
    m = oracle.block_mask(qf, kf, sta_np, w.thr)
    t_mask = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    total_rows = w.B * w.heads * w.nb
    ids = np.sort(rng.choice(total_rows, size=min(rows, total_rows), replace=False))
    t0 = time.perf_counter()
    oracle.attention(qf, kf, vf, m["kv_nb"], m["kv_inds"], row_ids=ids)
    t_attn_sample = time.perf_counter() - t0
    sample_pairs = int(m["kv_nb"].reshape(-1)[ids].sum())
    all_pairs = int(m["kv_nb"].sum())
    t_attn_full = t_attn_sample * all_pairs / max(sample_pairs, 1)
    t_step = t_perm + t_mask + t_attn_full
    return {
        "value": all_pairs * flops_per_pair / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.get_threads(),
        "kind": "oracle",
        "sample": ("full permute (%.2f s) and full estimator (%.2f s, %d rows) measured; "
                   "attention measured on %d of %d query blocks (%.2f s, %d of %d kept pairs) "
                   "and scaled by kept pairs to %.1f s"
                   % (t_perm, t_mask, total_rows, ids.size, total_rows, t_attn_sample,
                      sample_pairs, all_pairs, t_attn_full)),
        "mask_ms": t_mask * 1e3,
        **lists_vs_oracle(m, g_nb, g_inds, w.thr),
    }


def measure(torch, nabla, w, qkv, steps, warmup, topk_ratio=None, quant=False, fold=True):
    """Run the path on workload w for `steps` timed steps; return the measurement dict.
    With topk_ratio the top-k estimator variant replaces NABLA's CDF estimator; with quant
    the quantizer and the INT8 / FP8 attention replace the bf16 attention.  fold: on a grid
    of whole patches (bf16 or fp32 attention), the natural-order calls read q, k, v and write
    o where the fractal permutes would have moved them (the same rows, the same results)."""
    import ctypes
    dev = torch.device("cuda:0")
    q, k, v = qkv
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gq, gk, gv = (torch.from_numpy(a).to(tdt).to(dev) for a in (q, k, v))
    B, S, H, D, nb = w.B, w.S, w.heads, w.D, w.nb
    qf = torch.empty((B, S, H, D), dtype=tdt, device=dev)
    kf, vf, of = torch.empty_like(qf), torch.empty_like(qf), torch.empty_like(qf)
    o_nat = torch.empty_like(gq)
    sta = torch.empty((nb, nb), dtype=torch.uint8, device=dev)
    kv_nb = torch.empty((B, H, nb), dtype=torch.int32, device=dev)
    kv_inds = torch.empty((B, H, nb, nb), dtype=torch.int32, device=dev)
    ws = torch.empty(nabla.nabla_block_mask_workspace(B, S, H, D), dtype=torch.uint8, device=dev)
    ws_attn = torch.empty(nabla.nabla_sparse_attn_workspace(B, S, H, w.tiles), dtype=torch.uint8,
                          device=dev)
    L = nabla.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    dt_code = 1 if tdt == torch.bfloat16 else 0
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    sta_p = P(sta) if w.sta is not None else None
    if quant:
        qz = {"q8": torch.empty((B, H, nb, 64, D), dtype=torch.int8, device=dev),
              "k8": torch.empty((B, H, nb, 64, D), dtype=torch.int8, device=dev),
              "v8": torch.empty((B, H, nb, D, 64), dtype=torch.uint8, device=dev)}
        for n in ("qs", "ks"):
            qz[n] = torch.empty((B, H, nb), dtype=torch.float32, device=dev)
        for n in ("vs", "km"):
            qz[n] = torch.empty((B, H, D), dtype=torch.float32, device=dev)
        ws_q = torch.empty(L.nabla_quant_qkv_workspace(B, S, H, D), dtype=torch.uint8, device=dev)
        ws_q8 = torch.empty(L.nabla_sparse_attn_q8_workspace(B, S, H, *w.tiles), dtype=torch.uint8,
                            device=dev)

    def check(rc, what):
        if rc != 0:
            raise nabla.NablaError(rc, what)

    fold = fold and not w.padded

    def step(rec=None):
        """One pass of the path; rec collects (start, end) event pairs per stage."""
        e = [ev() for _ in range(6)] if rec is not None else None
        if e: e[0].record(stream)
        if w.sta is not None:
            check(L.nabla_sta_mask(P(sta), *w.tiles, *w.sta, sp), "sta")
        for src, dst in ((gq, qf), (gk, kf), (gv, vf)) if not fold else ():
            check(L.nabla_fractal_permute(P(src), P(dst), dt_code, B, w.T, w.H, w.W, H, D, 0, sp),
                  "permute")
        if e: e[1].record(stream)
        if fold:
            check(L.nabla_block_mask_natural(P(gq), P(gk), dt_code, B, w.T, w.H, w.W, H, D, sta_p,
                                             w.thr, -1.0 if topk_ratio is None else topk_ratio,
                                             P(kv_nb), P(kv_inds), P(ws), ws.numel(), sp),
                  "mask")
        elif w.padded:  # partial patches: the grid entry points
            check(L.nabla_block_mask_grid(P(qf), P(kf), dt_code, B, w.T, w.H, w.W, H, D, sta_p,
                                          w.thr, -1.0 if topk_ratio is None else topk_ratio,
                                          P(kv_nb), P(kv_inds), P(ws), ws.numel(), sp), "mask")
        elif topk_ratio is None:
            check(L.nabla_block_mask(P(qf), P(kf), dt_code, B, S, H, D, sta_p, w.thr, P(kv_nb),
                                     P(kv_inds), P(ws), ws.numel(), sp), "mask")
        else:
            check(L.nabla_block_mask_topk(P(qf), P(kf), dt_code, B, S, H, D, sta_p, topk_ratio,
                                          P(kv_nb), P(kv_inds), P(ws), ws.numel(), sp), "mask")
        if e: e[2].record(stream)
        codes = [P(qz[n]) for n in ("q8", "qs", "k8", "ks", "v8", "vs")] if quant else None
        if quant and fold:
            check(L.nabla_quant_qkv_natural(P(gq), P(gk), P(gv), dt_code, B, w.T, w.H, w.W, H, D,
                                            *codes, P(qz["km"]), P(ws_q), ws_q.numel(), sp),
                  "quant")
        elif quant and w.padded:
            check(L.nabla_quant_qkv_grid(P(qf), P(kf), P(vf), dt_code, B, w.T, w.H, w.W, H, D,
                                         *codes, P(qz["km"]), P(ws_q), ws_q.numel(), sp), "quant")
        elif quant:
            check(L.nabla_quant_qkv(P(qf), P(kf), P(vf), dt_code, B, S, H, D, *codes,
                                    P(qz["km"]), P(ws_q), ws_q.numel(), sp), "quant")
        if e: e[3].record(stream)
        if quant and fold:
            check(L.nabla_sparse_attn_fwd_q8_natural(*codes, B, w.T, w.H, w.W, H, D, P(kv_nb),
                                                     P(kv_inds), 0.0, P(o_nat), P(ws_q8),
                                                     ws_q8.numel(), sp), "attn q8")
        elif quant and w.padded:
            check(L.nabla_sparse_attn_fwd_q8_grid(*codes, B, w.T, w.H, w.W, H, D, P(kv_nb),
                                                  P(kv_inds), 0.0, P(of), P(ws_q8),
                                                  ws_q8.numel(), sp), "attn q8")
        elif quant:
            check(L.nabla_sparse_attn_fwd_q8(*codes, B, S, H, D, P(kv_nb), P(kv_inds), 0.0,
                                             *w.tiles, P(of), P(ws_q8), ws_q8.numel(), sp),
                  "attn q8")
        elif fold:
            check(L.nabla_sparse_attn_fwd_natural(P(gq), P(gk), P(gv), dt_code, B, w.T, w.H, w.W,
                                                  H, D, P(kv_nb), P(kv_inds), 0.0, P(o_nat), None,
                                                  P(ws_attn), ws_attn.numel(), sp), "attn")
        elif w.padded:
            check(L.nabla_sparse_attn_fwd_grid(P(qf), P(kf), P(vf), dt_code, B, w.T, w.H, w.W, H,
                                               D, P(kv_nb), P(kv_inds), 0.0, P(of), None,
                                               P(ws_attn), ws_attn.numel(), sp), "attn")
        else:
            check(L.nabla_sparse_attn_fwd(P(qf), P(kf), P(vf), dt_code, B, S, H, D, P(kv_nb),
                                          P(kv_inds), 0.0, *w.tiles, P(of), P(ws_attn),
                                          ws_attn.numel(), sp), "attn")
        if e: e[4].record(stream)
        if not fold:
            check(L.nabla_fractal_permute(P(of), P(o_nat), dt_code, B, w.T, w.H, w.W, H, D, 1, sp),
                  "unpermute")
        if e:
            e[5].record(stream)
            rec.append(e)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps; per-stage HIP events are recorded on
    # the launch stream inside the same steps
    rec = []
    t0 = time.perf_counter()
    for _ in range(steps):
        step(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = np.array([[a.elapsed_time(b) for a, b in zip(e[:-1], e[1:])] for e in rec])
    g_nb = kv_nb.cpu().numpy()
    g_inds = kv_inds.cpu().numpy()
    pairs = int(g_nb.sum())
    flops_per_pair = 4.0 * 64 * 64 * D
    esz = 2 if tdt == torch.bfloat16 else 4
    mask_ms = float(np.mean(stage[:, 1]))
    quant_ms = float(np.mean(stage[:, 2]))
    attn_ms = float(np.mean(stage[:, 3]))
    mask_bytes = 2.0 * B * S * H * D * esz + 4.0 * B * H * nb + 4.0 * pairs + nb * nb
    sta_pairs = int(sta.sum().item()) * B * H if w.sta is not None else 0
    return {
        "ms_per_step": wall * 1e3 / steps,
        "perm_ms": float(np.mean(stage[:, 0] + stage[:, 4])),
        "mask_ms": mask_ms,
        "quant_ms": quant_ms,
        "attn_ms": attn_ms,
        "pairs": pairs,
        "flops_per_pair": flops_per_pair,
        "attn_flops": pairs * flops_per_pair,
        "density": pairs / float(B * H * nb * nb),
        "sta_density": sta_pairs / float(B * H * nb * nb),
        "mask_gbs": mask_bytes / (mask_ms * 1e-3) / 1e9,
        "g_nb": g_nb,
        "g_inds": g_inds,
        "sta_np": None if w.sta is None else sta.cpu().numpy(),
        "dtype": "bf16" if tdt == torch.bfloat16 else "fp32",
        "fold": fold,
    }


def sweep(torch, nabla, synth, steps, warmup, quant=False, oracle_lists=True):
    """The sparsity sweep on the 720p shape and the long clip: one JSON line per run (with
    quant, the quantizer and the quantized attention in place of the bf16 attention).  With
    oracle_lists, each run's lists are also compared with the oracle estimator's on every row
    (band rows counted and listed)."""
    cache = {}
    runs = synth.sweep_workloads() + [synth.WORKLOADS["long"]]
    for w in runs:
        key = (w.T, w.H, w.W, w.heads, w.D, w.gen, w.seed, w.sigma_f, w.sigma_n, w.dtype)
        if key not in cache:
            cache.clear()
            print("[bench] generating %s" % w.describe(), file=sys.stderr, flush=True)
            cache[key] = synth.make_qkv(w)
        m = measure(torch, nabla, w, cache[key], steps, warmup, quant=quant)
        line = {"workload": w.describe(), "attention": "int8/fp8" if quant else "bf16",
                "density": round(m["density"], 5),
                "sta_density": round(m["sta_density"], 5), "kept_pairs": m["pairs"],
                "mask_ms": round(m["mask_ms"], 4), "mask_gbs": round(m["mask_gbs"], 1),
                "attn_ms": round(m["attn_ms"], 4),
                "attn_tflops": round(m["attn_flops"] / (m["attn_ms"] * 1e-3) / 1e12, 2),
                "permute_ms": round(m["perm_ms"], 4), "ms_per_step": round(m["ms_per_step"], 4),
                **({"quant_ms": round(m["quant_ms"], 4)} if quant else {}),
                "value": round(m["attn_flops"] / (m["ms_per_step"] * 1e-3) / 1e12, 3)}
        if oracle_lists:
            import oracle
            oracle.set_threads(len(os.sched_getaffinity(0)))
            q, k, _ = cache[key]
            f = lambda a: oracle.fractal_permute(a).reshape(w.B, w.S, w.heads, w.D)
            orc = oracle.block_mask(f(q), f(k), m["sta_np"], w.thr)
            line.update(lists_vs_oracle(orc, m["g_nb"], m["g_inds"], w.thr))
        print(json.dumps(line), flush=True)


def train_pass(torch, nabla, synth, w, steps, warmup):
    """The training pass on workload w: nabla_sparse_attn_fwd with lse, then
    nabla_sparse_attn_bwd for a seeded dO, on the estimator's lists (the grid entry
    points on a padded layout); one JSON line.

    Backward FLOPs are the algorithmic five products per kept pair (S = Q K^T again,
    dP = dO V^T, dV += P^T dO, dK += dS^T Q, dQ += dS K), 10 * 64 * 64 * D; the kernels
    recompute S and dP in both gradient kernels (seven products), which is not counted."""
    dev = torch.device("cuda:0")
    q, k, v = synth.make_qkv(w)
    g = [torch.from_numpy(a).to(torch.bfloat16).to(dev) for a in (q, k, v)]
    qf, kf, vf = (nabla.nabla_fractal_permute(t) for t in g)
    # a padded layout (partial patches) goes through the grid entry points
    grid = (w.T, w.H, w.W) if w.padded else None
    sta = nabla.nabla_sta_mask(w.tiles, w.sta, dev) if w.sta is not None else None
    kv_nb, kv_inds = nabla.nabla_block_mask(qf, kf, sta, w.thr, grid=grid)
    rng = np.random.default_rng(w.seed + 1000)
    # dO drawn in natural order and permuted, so it is 0 at padding positions
    dnat = torch.from_numpy(rng.standard_normal(q.shape, dtype=np.float32)).to(torch.bfloat16)
    dout = nabla.nabla_fractal_permute(dnat.to(dev))
    B, S, H, D = qf.shape
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    o = torch.empty_like(qf)
    dq, dk, dv = torch.empty_like(qf), torch.empty_like(qf), torch.empty_like(qf)
    ws_f = torch.empty(nabla.nabla_sparse_attn_workspace(B, S, H, w.tiles), dtype=torch.uint8,
                       device=dev)
    ws_b = torch.empty(nabla.nabla_sparse_attn_bwd_workspace(B, S, H), dtype=torch.uint8,
                       device=dev)
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def one(rec=None):
        e = [ev() for _ in range(3)] if rec is not None else None
        if e: e[0].record(stream)
        nabla.nabla_sparse_attn_fwd(qf, kf, vf, kv_nb, kv_inds, tiles=w.tiles, workspace=ws_f,
                                    out=o, lse=lse, grid=grid)
        if e: e[1].record(stream)
        nabla.nabla_sparse_attn_bwd(qf, kf, vf, o, dout, lse, kv_nb, kv_inds, workspace=ws_b,
                                    dq=dq, dk=dk, dv=dv, grid=grid)
        if e:
            e[2].record(stream)
            rec.append(e)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    rec = []
    t0 = time.perf_counter()
    for _ in range(steps):
        one(rec)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in rec]))
    bwd_ms = float(np.mean([b.elapsed_time(c) for _, b, c in rec]))
    pairs = int(kv_nb.sum().item())
    f_fwd = 4.0 * 64 * 64 * D * pairs
    f_bwd = 10.0 * 64 * 64 * D * pairs
    bwd_tf = f_bwd / (bwd_ms * 1e-3) / 1e12
    out = {
        "metric": "NABLA sparse attn training pass (fwd with lse + bwd) effective TFLOP/s, 1 MI355X",
        "value": round((f_fwd + f_bwd) / (wall * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(wall, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded smooth spatio-temporal field + noise, video-shaped; dO ~ N(0,1))",
        "config": {"workload": w.describe(), "kept_pairs": pairs,
                   "density": round(pairs / float(B * H * w.nb * w.nb), 5)},
        "fwd_lse_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2), "bwd_tflops": round(bwd_tf, 2),
        "roofline": {"bound": "mfma", "achieved": round(bwd_tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "nabla_sparse_attn_bwd (all its kernels)",
                     "per_launch": {"flops": f_bwd, "kept_pairs": pairs}},
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(the path shards by (batch, head) across GPUs; that is not built here)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import block_sparse_attention_fractal_amd as nabla
    from block_sparse_attention_fractal_amd import synth
    if args.sweep:
        sweep(torch, nabla, synth, args.steps, args.warmup, quant=args.q8,
              oracle_lists=not args.no_cpu_baseline)
        return
    if args.bwd:
        w = synth.WORKLOADS[args.workload]
        print("[bench] training pass %s" % w.describe(), file=sys.stderr, flush=True)
        train_pass(torch, nabla, synth, w, args.steps, args.warmup)
        return

    w = synth.WORKLOADS[args.workload]
    print("[bench] %s" % w.describe(), file=sys.stderr, flush=True)
    q, k, v = synth.make_qkv(w)
    m = measure(torch, nabla, w, (q, k, v), args.steps, args.warmup, topk_ratio=args.topk,
                quant=args.q8, fold=not args.separate_permutes)
    attn_tflops = m["attn_flops"] / (m["attn_ms"] * 1e-3) / 1e12
    # the committed PMC summaries cover the 720p workload with the natural-order calls only
    pmc_case = w.name == "720p" and m["fold"] and args.topk is None
    traffic = None
    if pmc_case:
        traffic = read_traffic(Q8_PMC_FILE, Q8_SRC) if args.q8 else read_traffic()
    kname = "sparse_attn_kernel<%d, %s, %s, %s>" % (
        w.D, "bf16" if w.dtype == "bf16" else "float", str(w.padded).lower(),
        str(m["fold"]).lower())
    metric = METRIC if args.topk is None else (
        "NABLA path with the top-k estimator (ratio %g): sparse attn fwd effective TFLOP/s + "
        "mask ms at %s shape, 1 MI355X" % (args.topk, w.name))
    if args.q8:
        metric = ("NABLA path with the quantized attention (INT8 Q K^T, FP8 P V): sparse attn fwd "
                  "effective TFLOP/s + mask ms at %s shape, 1 MI355X" % w.name)
    out = {
        "metric": metric,
        "value": round(m["attn_flops"] / (m["ms_per_step"] * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m["dtype"],
        "data": "synthetic (seeded smooth spatio-temporal field + noise, video-shaped)",
        "config": {"workload": w.describe(), "B": w.B, "heads": w.heads, "head_dim": w.D,
                   "T": w.T, "H": w.H, "W": w.W, "seq_len": w.S, "blocks": w.nb, "thr": w.thr,
                   "sta_window": list(w.sta) if w.sta else None, "kept_pairs": m["pairs"],
                   "density": round(m["density"], 5),
                   "permutes": "folded into the kernels' addressing (natural-order calls)"
                   if m["fold"] else "nabla_fractal_permute kernels"},
        "mask_ms": round(m["mask_ms"], 4),
        "attn_ms": round(m["attn_ms"], 4),
        "permute_ms": round(m["perm_ms"], 4),
        "attn_tflops": round(attn_tflops, 2),
        "mask_gbs": round(m["mask_gbs"], 1),
        "mask_hbm_frac": round(m["mask_gbs"] / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": kname,
                     "per_launch": {"flops": m["attn_flops"], "kept_pairs": m["pairs"]}},
    }
    if args.q8:
        out["dtype"] = "int8 (Q K^T) / fp8 e4m3 (P V)"
        out["quant_ms"] = round(m["quant_ms"], 4)
        out["roofline"].update({"peak": PEAK_FP8_TFLOPS,
                                "frac": round(attn_tflops / PEAK_FP8_TFLOPS, 4),
                                "kernel": "sparse_attn_q8_kernel<%d, %s>" % (
                                    w.D, str(w.padded).lower())})
    if not args.no_cpu_baseline and args.topk is None and not args.q8 and not w.padded:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, m["sta_np"], m["g_nb"], m["g_inds"],
                                           args.cpu_rows, m["flops_per_pair"])
        out["band_rows"] = out["cpu_baseline"]["band_rows"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
