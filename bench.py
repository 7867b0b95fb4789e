"""Benchmark of the sparse-weight matmul hot path on one MI355X.

Default workload (``--workload decode``) prints one JSON line with:

* ``value``: decode on the q_proj shape -- W 4096x4096 fp16 at 50% per-row
  magnitude pruning, compressed to the tiled column-bitmap format.  One step =
  three sparse products with N = 1, 8 and 16 tokens; ``value`` = algorithmic
  bytes of the sparse products (kept values, bitmaps and tile pointers without
  run padding, + X + Y) / their GPU time, in GB/s, inputs resident in HBM.  The
  same step is timed with the in-house dense GEMM on the masked W stored dense,
  for the speedup.  ``roofline`` is the N = 16 launch against 8 TB/s and
  against the library's streaming kernel at the same byte count and rotation.
* ``prefill``: up/gate 11008x4096 at 50%, N = 4096, through the workspace
  route, the on-chip kernel and the dense kernel, with an MFMA roofline on
  useful (2 nnz N) and executed (2 M K N) FLOPs and the oracle timed on the
  host on a 512-token slice.
* ``layer``: the seven Llama-2-7B-shaped linears back to back, N = 16 and
  4096, rotated over 5 compressed and 3 dense copies of the layer.
* ``device``: name, CU count, clocks, ROCm and HIP versions.

Timing: launches are captured once into HIP graphs (torch.cuda.CUDAGraph) and
replayed, so host launch overhead does not starve the GPU; HIP events on the
launch stream bracket the replays (one event pair per replay for the
median / p10 / p90).  Copies of the weight are rotated so the working set
exceeds 1 GiB (4x the 256 MB Infinity Cache) and every launch streams its
weight from HBM.

Other workloads: ``spmspv`` (down_proj 4096x11008, SiLU-gated x with |x|<0.3
zeroed, N = 1, 2, 4), ``prefill`` (up/gate 11008x4096, N = 512/2048/4096,
sparsity 0.5/0.6/0.7), ``layer`` (the layer block alone), ``mlp`` (decode FFN
block), ``wide`` (other shapes and sparsities), ``calib`` (copy of known size
for the counter scale).  Each prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 1 << 30


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def fmt_bytes(info):
    """Resident bytes of a format's device sections (tile pointers, bitmaps,
    padded value runs)."""
    return int(info["bytes_tile_ptr"] + info["bytes_bits"] + info["bytes_values"])


def fmt_alg_bytes(info):
    """Algorithmic bytes of a format: tile pointers, bitmaps and the kept fp16
    values; the run padding is not counted."""
    return int(info["bytes_tile_ptr"] + info["bytes_bits"] + 2 * info["nnz"])


def pct(ts):
    """median / p10 / p90 of a list of per-launch times (ms) -> dict in us."""
    a = np.asarray(ts, dtype=np.float64) * 1e3
    return {"median_us": float(np.median(a)), "p10_us": float(np.percentile(a, 10)),
            "p90_us": float(np.percentile(a, 90)), "replays": int(a.size)}


def device_info(torch):
    """Device name, CU count, clocks, LDS, L2 and the ROCm / HIP versions."""
    import ctypes
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count,
            "hbm_bytes": int(p.total_memory), "hip": torch.version.hip, "torch": torch.__version__}
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm"] = None
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        for key, attr in (("clock_khz", 5), ("mem_clock_khz", 60), ("lds_per_block", 74), ("l2_bytes", 19)):
            # hipDeviceAttributeClockRate, MemoryClockRate, MaxSharedMemoryPerBlock, L2CacheSize
            if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) == 0:
                info[key] = int(v.value)
    except OSError:
        pass
    return info


def blas_vendor():
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name')} {b.get('version')}"
    except Exception:
        return None


class Graphs:
    """Capture launch sequences into HIP graphs and time their replays with events."""

    def __init__(self, torch):
        self.torch = torch

    def capture(self, fns):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for fn in fns:
                fn()
        g.replay()
        torch.cuda.synchronize()
        return g

    def time(self, g, reps=1):
        torch = self.torch
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps  # ms per replay

    def samples(self, g, reps, per):
        """ms per launch of each of `reps` replays (one event pair per replay of
        a graph of `per` launches)."""
        torch = self.torch
        s = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        ev[0].record(s)
        for r in range(reps):
            g.replay()
            ev[r + 1].record(s)
        ev[-1].synchronize()
        return [ev[r].elapsed_time(ev[r + 1]) / per for r in range(reps)]

    def interleaved(self, graphs, reps, pers, warm=3):
        """ms per launch of `reps` replays of each graph (`pers[i]` launches in
        graph i), sampled in turn: one replay of every graph per round, after
        `warm` untimed rounds, so that all of them run in the same clock and
        power state (a route timed alone right after host-side work runs on a
        cooler, slower chip)."""
        torch = self.torch
        s = torch.cuda.current_stream()
        for _ in range(warm):
            for g in graphs:
                g.replay()
        torch.cuda.synchronize()
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
              for _ in graphs]
        for r in range(reps):
            for i, g in enumerate(graphs):
                ev[i][r][0].record(s)
                g.replay()
                ev[i][r][1].record(s)
        torch.cuda.synchronize()
        return [[ev[i][r][0].elapsed_time(ev[i][r][1]) / pers[i] for r in range(reps)] for i in range(len(graphs))]


def rotating_formats(swm, W, mask, min_bytes=ROTATE_BYTES):
    """Copies of the compressed W whose resident bytes add up to >= min_bytes;
    returns them and the format's algorithmic bytes (no run padding)."""
    f0 = swm.sparse_compress(W, mask)
    copies = max(2, int(np.ceil(min_bytes / fmt_bytes(f0.info))))
    blob = f0.export()
    return [f0] + [swm.format_import(blob) for _ in range(copies - 1)], fmt_alg_bytes(f0.info)


def rotating_dense(torch, W, min_bytes=ROTATE_BYTES):
    Wd = torch.from_numpy(W).cuda()
    copies = max(2, int(np.ceil(min_bytes / (W.size * 2))))
    return [Wd] + [Wd.clone() for _ in range(copies - 1)]


def profiled_traffic(profile_md):
    """HBM bytes per launch from a committed counter summary, if the kernel
    sources it was taken on are the ones built now; else None."""
    import hashlib
    import re
    try:
        text = open(os.path.join(ROOT, "profiles", profile_md)).read()
        meta = json.loads(re.search(r"<!-- bench-traffic: (\{.*\}) -->", text).group(1))
        sources = meta.get("sources") or [[meta["source"], meta["source_sha256"]]]
        for path, sha in sources:
            if hashlib.sha256(open(os.path.join(ROOT, path), "rb").read()).hexdigest() != sha:
                return None
    except (OSError, AttributeError, ValueError, KeyError, TypeError):
        return None
    return int(meta["traffic_bytes_per_launch"])


def stream_achievable(torch, swm, G, nbytes, min_bytes=ROTATE_BYTES):
    """Read bandwidth of the library's streaming kernel for `nbytes` per launch
    under the same rotation (>= 1 GiB of distinct buffers): the best launch
    shape of a small sweep.  The 'achievable' reference beside the 8 TB/s peak."""
    nb = (int(nbytes) + 255) // 256 * 256
    copies = max(2, int(np.ceil(min_bytes / nb)))
    buf = torch.empty(copies * nb, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    out = torch.empty(4096 * 4, dtype=torch.int32, device="cuda")
    views = [buf[i * nb:i * nb + (nbytes // 16) * 16] for i in range(copies)]
    best = None
    for unroll in (4, 8, 16):
        for blocks in (256, 512, 1024, 2048):
            fns = [lambda v=v: swm.hbm_stream(v, unroll, blocks, out) for v in views]
            for f in fns[:2]:
                f()
            t = G.time(G.capture(fns), 3) / copies
            if best is None or t < best[0]:
                best = (t, unroll, blocks)
    del buf
    t, unroll, blocks = best
    return {"GBps": (nbytes // 16) * 16 / (t * 1e-3) / 1e9, "us": t * 1e3, "bytes": int(nbytes),
            "unroll": unroll, "blocks": blocks, "copies": copies}


def threads_used():
    try:
        from threadpoolctl import threadpool_info
        return int(max([d.get("num_threads", 1) for d in threadpool_info()] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_oracle(W, mask, X_list, units, unit, budget_s=20.0):
    """The oracle as it stands (oracle.masked_matmul: the masked weight in
    float64, then the product) on the host cores: one warm-up call, then the
    median of up to 3 timed calls per sample."""
    import oracle
    t_tot, u_tot = 0.0, 0.0
    for X, u in zip(X_list, units):
        oracle.masked_matmul(W, mask, X)
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.masked_matmul(W, mask, X)
            ts.append(time.perf_counter() - t0)
            if sum(ts) > budget_s:
                break
        t_tot += float(np.median(ts))
        u_tot += u
    return {"value": u_tot / t_tot, "unit": unit, "cores": threads_used(), "kind": "oracle", "blas": blas_vendor()}


# ------------------------------------------------------------------ decode (default)
def bench_decode(args, torch, swm, wl, G):
    _log("workload: decode q_proj 4096x4096, 50%")
    W, mask, X = wl.decode_qproj(16)
    fmts, fa = rotating_formats(swm, W, mask)
    fb = fmt_bytes(fmts[0].info)
    Wds = rotating_dense(torch, W)
    C, CD = len(fmts), len(Wds)
    _log(f"format {fb / 1e6:.2f} MB resident ({fa / 1e6:.2f} MB algorithmic), {C} sparse / {CD} dense rotating copies")
    Xd = torch.from_numpy(X).cuda()
    Ns = (1, 8, 16)
    M, K = W.shape
    Ys = {n: torch.empty((n, M), dtype=torch.float16, device="cuda") for n in Ns}
    alg = {n: fa + 2 * K * n + 2 * M * n for n in Ns}
    dense_b = {n: 2 * M * K + 2 * K * n + 2 * M * n for n in Ns}

    def sp(i, n):
        return lambda: swm.spmm(fmts[i % C], Xd[:n], Ys[n])

    def de(i, n):
        return lambda: swm.dense_gemm(Wds[i % CD], Xd[:n], Ys[n])

    for r in range(2):  # untimed: warms the code paths
        for n in Ns:
            sp(r, n)()
            de(r, n)()
    torch.cuda.synchronize()
    per_n, per_n_d, dist = {}, {}, {}
    for n in Ns:
        gs = G.capture([sp(i, n) for i in range(C)])
        gd = G.capture([de(i, n) for i in range(CD)])
        ts = G.samples(gs, 20, C)
        per_n[n] = float(np.mean(ts))
        dist[n] = pct(ts)
        per_n_d[n] = G.time(gd, 5) / CD
    # The contract's steps: W warmup steps, then exactly K timed steps.
    g_warm = G.capture([sp(s * 3 + j, n) for s in range(args.warmup) for j, n in enumerate(Ns)])
    g_steps = G.capture([sp(s * 3 + j, n) for s in range(args.steps) for j, n in enumerate(Ns)])
    g_dsteps = G.capture([de(s * 3 + j, n) for s in range(args.steps) for j, n in enumerate(Ns)])
    g_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_total = G.time(g_steps, 1)
    wall = time.perf_counter() - t0
    ms_dense = G.time(g_dsteps, 1)
    ms_step = ms_total / args.steps
    value = sum(alg.values()) / (ms_step * 1e-3) / 1e9
    detail = {str(n): {"sparse_us": per_n[n] * 1e3, "sparse_dist": dist[n], "dense_us": per_n_d[n] * 1e3,
                       "speedup_vs_dense": per_n_d[n] / per_n[n],
                       "sparse_GBps_alg": alg[n] / (per_n[n] * 1e-3) / 1e9,
                       "sparse_frac_hbm": alg[n] / (per_n[n] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "dense_GBps": dense_b[n] / (per_n_d[n] * 1e-3) / 1e9} for n in Ns}
    dom = 16
    ach = alg[dom] / (per_n[dom] * 1e-3) / 1e9
    _log("stream calibration at the decode launch's byte count")
    st = stream_achievable(torch, swm, G, alg[dom])
    _log("stream calibration at the dense baseline launch's byte count")
    st_d = stream_achievable(torch, swm, G, dense_b[dom])
    dense_ach = dense_b[dom] / (per_n_d[dom] * 1e-3) / 1e9
    out = {
        "metric": "decode SpMM HBM throughput on compressed bytes (q_proj 4096x4096, 50%)",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic (seeded N(0,1) fp16 W and X, 50% per-row magnitude pruning)",
        "config": {"workload": "decode q_proj 4096x4096, 50% unstructured, N in {1,8,16} per step",
                   "format": "SWM-TCB v2 tm=16 tk=64", "format_resident_bytes": fb,
                   "format_alg_bytes": fa, "rotating_copies": C},
        "speedup_vs_dense": ms_dense / ms_total,
        "dense_ms_per_step": ms_dense / args.steps,
        "dense_baseline": {"kernel": "dense_small_kernel, N=16", "bytes_per_launch": dense_b[dom],
                           "GBps": dense_ach, "frac_hbm": dense_ach / HBM_PEAK_GBS,
                           "achievable": st_d["GBps"], "frac_of_achievable": dense_ach / st_d["GBps"]},
        "detail": detail,
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS,
                     "traffic": profiled_traffic("decode_seq_kernel_qproj_pmc.md"),
                     "kernel": "decode_seq_kernel, N=16", "alg_bytes_per_launch": alg[dom],
                     "avg_launch_us": per_n[dom] * 1e3, "launch_dist": dist[dom],
                     "achievable": st["GBps"], "frac_of_achievable": ach / st["GBps"],
                     "achievable_kernel": st},
        "timed_wall_s": wall,
    }
    if not args.no_cpu:
        _log("timing the CPU oracle")
        cb = cpu_oracle(W, mask, [X[:n] for n in Ns], [alg[n] for n in Ns], "B")
        cb["value"] = cb["value"] / 1e9
        cb["unit"] = "GB/s"
        cb["sample"] = "one full decode step (N = 1, 8, 16), oracle.masked_matmul (float64 masking included), median of 3"
        out["cpu_baseline"] = cb
    return out


def prefill_block(args, torch, swm, wl, G):
    """Config-4 headline point: up/gate 11008x4096 at 50%, N = 4096, through
    swm_spmm_ws (W expanded once, dense MFMA), the on-chip kernel and the
    dense kernel; MFMA roofline on useful and executed FLOPs."""
    _log("prefill block: up/gate 11008x4096, 50%, N = 4096")
    n = 4096
    W, mask, X = wl.prefill_upgate(0.5, n)
    M, K = W.shape
    nnz = int(mask.sum())
    f = swm.sparse_compress(W, mask)
    Wd = torch.from_numpy(W).cuda()
    Xd = torch.from_numpy(X).cuda()
    ws = torch.empty(max(swm.spmm_workspace_bytes(f, n), 256), dtype=torch.uint8, device="cuda")
    y = torch.empty((n, M), dtype=torch.float16, device="cuda")
    swm.spmm(f, Xd, y)
    swm.spmm_ws(f, Xd, ws, y)
    swm.dense_gemm(Wd, Xd, y)
    torch.cuda.synchronize()
    reps = 4

    # The block follows host-side work (the oracle's timing), during which
    # the GPU's clocks drop: the routes are sampled in turn after common
    # warm-up rounds, so that none of them is timed on a cooler chip.
    gr = [G.capture([fn] * reps) for fn in (lambda: swm.spmm_ws(f, Xd, ws, y), lambda: swm.spmm(f, Xd, y),
                                            lambda: swm.dense_gemm(Wd, Xd, y),
                                            lambda: swm.decompress(f, ws.view(torch.float16)[:M * K].view(M, K)))]
    d_ws, d_on, d_de, d_dc = (pct(t) for t in G.interleaved(gr, 10, [reps] * 4, warm=5))
    useful, executed = 2.0 * nnz * n, 2.0 * M * K * n
    t_ws, t_on, t_de = d_ws["median_us"] * 1e-6, d_on["median_us"] * 1e-6, d_de["median_us"] * 1e-6
    blk = {
        "workload": "prefill up/gate 11008x4096, 50% per-row magnitude pruning, N = 4096",
        "spmm_ws": d_ws, "onchip": d_on, "dense": d_de, "expand_only": d_dc,
        "useful_TFLOPs_ws": useful / t_ws / 1e12, "useful_TFLOPs_onchip": useful / t_on / 1e12,
        "dense_TFLOPs": executed / t_de / 1e12,
        "speedup_ws_vs_dense": t_de / t_ws, "speedup_onchip_vs_dense": t_de / t_on,
        "roofline": {"bound": "mfma", "unit": "TFLOP/s", "peak": MFMA_F16_PEAK_TFLOPS,
                     "kernel": "swm_spmm_ws (decompress_kernel + dense_kernel), N=4096",
                     "achieved": useful / t_ws / 1e12, "frac": useful / t_ws / 1e12 / MFMA_F16_PEAK_TFLOPS,
                     "executed_TFLOPs": executed / t_ws / 1e12,
                     "frac_executed": executed / t_ws / 1e12 / MFMA_F16_PEAK_TFLOPS,
                     "useful_flops_per_launch": useful, "executed_flops_per_launch": executed,
                     "traffic": profiled_traffic("prefill_upgate_n4096_traffic.md")},
    }
    if not args.no_cpu:
        _log("timing the CPU oracle on a 512-token slice")
        cb = cpu_oracle(W, mask, [X[:512]], [2.0 * nnz * 512], "FLOP")
        cb["value"] = cb["value"] / 1e12
        cb["unit"] = "TFLOP/s"
        cb["sample"] = "512 of the 4096 tokens, oracle.masked_matmul (float64 masking included), median of 3, useful FLOPs"
        blk["cpu_baseline"] = cb
    del f, Wd, ws, y
    torch.cuda.empty_cache()
    return blk


def layer_copies(swm, torch, parts, min_sparse=5, min_dense=3, smfmac=False):
    """Linears given as (W, mask, X): >= min_sparse compressed copies and
    >= min_dense dense copies of each (rotated so that each layer pass streams
    its weights from HBM: 5 x 228 MB and 3 x 405 MB are above 4x the 256 MB
    Infinity Cache).  smfmac: every copy also keeps the 2:4 layers."""
    fmts, dens, xs, shapes, alg = [], [], [], [], 0
    for W, mask, X in parts:
        f0 = swm.sparse_compress(W, mask, smfmac=smfmac)
        blob = f0.export()
        copies = [swm.format_import(blob) for _ in range(min_sparse - 1)]
        if smfmac:
            for c in copies:
                c.enable_smfmac()
        fmts.append([f0] + copies)
        Wd = torch.from_numpy(W).cuda()
        dens.append([Wd] + [Wd.clone() for _ in range(min_dense - 1)])
        xs.append(torch.from_numpy(X).cuda())
        shapes.append(W.shape)
        alg += fmt_alg_bytes(f0.info)
    return fmts, dens, xs, shapes, alg


def layer_pass(args, torch, swm, G, parts, CS, CD, smfmac=False):
    """One layer pass = each of `parts` once, back to back on one stream,
    sparse through spmm_ws and dense through dense_gemm, at N = 16 and 4096."""
    fmts, dens, xs, shapes, fa = layer_copies(swm, torch, parts, CS, CD, smfmac)
    ws = torch.empty(max(max(swm.spmm_workspace_bytes(f[0], 4096) for f in fmts), 256), dtype=torch.uint8,
                     device="cuda")
    L = len(parts)
    blk = {"launches_per_pass": L, "format_alg_bytes": fa}
    for n in (16, 4096):
        ys = [torch.empty((n, shp[0]), dtype=torch.float16, device="cuda") for shp in shapes]

        def sp(c, i):
            return lambda: swm.spmm_ws(fmts[i][c], xs[i][:n], ws, ys[i])

        def de(c, i):
            return lambda: swm.dense_gemm(dens[i][c], xs[i][:n], ys[i])
        for i in range(L):
            sp(0, i)()
            de(0, i)()
        torch.cuda.synchronize()
        gs = G.capture([sp(c, i) for c in range(CS) for i in range(L)])
        gd = G.capture([de(c, i) for c in range(CD) for i in range(L)])
        reps = 10 if n == 16 else 3
        ts, td = G.interleaved([gs, gd], reps, [CS, CD], warm=3 if n == 16 else 1)
        ds, dd = pct(ts), pct(td)
        alg = fa + sum(2 * (shp[0] + shp[1]) * n for shp in shapes)
        e = {"sparse_layer": ds, "dense_layer": dd, "speedup_vs_dense": dd["median_us"] / ds["median_us"],
             "route": "decode kernels" if n <= 32 else
                      ("swm_spmm_ws (resident 2:4 layers, v_smfmac)" if smfmac else
                       "swm_spmm_ws (expand + dense MFMA; one shared workspace)")}
        if n == 16:
            e["alg_bytes"] = alg
            e["GBps_alg"] = alg / (ds["median_us"] * 1e-6) / 1e9
            e["frac_hbm"] = e["GBps_alg"] / HBM_PEAK_GBS
        else:
            useful = sum(2.0 * f[0].info["nnz"] * n for f in fmts)
            e["useful_TFLOPs"] = useful / (ds["median_us"] * 1e-6) / 1e12
        blk[str(n)] = e
        del ys
    del fmts, dens, xs, ws
    torch.cuda.empty_cache()
    return blk


def layer_block(args, torch, swm, wl, G):
    """Config 5: the seven linears back to back on one stream, N = 16 and 4096,
    rotated over 5 compressed / 3 dense copies of the layer; then the same
    layer with q/k/v and gate/up row-stacked (four launches a pass, as
    inference engines run it; the dense side stacked the same way)."""
    CS, CD = 5, 3
    _log("layer block: 7 linears, 5 compressed / 3 dense rotating copies")
    parts = [wl.layer_linear(i, 4096) for i in range(7)]
    blk = layer_pass(args, torch, swm, G, parts, CS, CD)
    blk.update({"workload": "Llama-2-7B layer: q/k/v/o 4096x4096, gate/up 11008x4096, down 4096x11008, 50%",
                "rotation": {"compressed_layer_copies": CS, "dense_layer_copies": CD}})
    _log("layer block: stacked projections qkv / o / gate_up / down")
    fused = [wl.stack_linears([parts[i] for i in idx]) for _, idx in wl.LAYER_FUSED]
    del parts
    fb = layer_pass(args, torch, swm, G, fused, CS, CD)
    fb["workload"] = "the same layer as qkv 12288x4096, o 4096x4096, gate_up 22016x4096, down 4096x11008"
    blk["stacked_projections"] = fb
    _log("layer block: the same seven linears pruned 2:4, sparse-matrix-core route")
    parts = [wl.layer_linear_2_4(i, 4096) for i in range(7)]
    b24 = layer_pass(args, torch, swm, G, parts, CS, CD, smfmac=True)
    b24["workload"] = ("the seven linears pruned 2:4 along K; handles keep the 2:4 layers (SWM_CFG_SMFMAC): "
                       "decode kernels at N = 16, v_smfmac at N = 4096")
    blk["pruned_2_4"] = b24
    return blk


def bench_default(args, torch, swm, wl, G):
    out = bench_decode(args, torch, swm, wl, G)
    if not args.decode_only:
        out["prefill"] = prefill_block(args, torch, swm, wl, G)
        out["layer"] = layer_block(args, torch, swm, wl, G)
    out["device"] = device_info(torch)
    return out


# ------------------------------------------------------------------ spMspV
def bench_spmspv(args, torch, swm, wl, G):
    _log("workload: spMspV down_proj 4096x11008, 50%, SiLU-gated x")
    W, mask, x = wl.spmspv_down(4, args.tau)
    fmts, fb = rotating_formats(swm, W, mask)
    Wds = rotating_dense(torch, W)
    C, CD = len(fmts), len(Wds)
    M, K = W.shape
    _log(f"column-run encoding for {C} rotated copies")
    cr_bytes = [f.enable_skipping() for f in fmts]
    resident = fmt_bytes(fmts[0].info) + cr_bytes[0]
    xd = torch.from_numpy(x).cuda()
    # the same activations before zeroing: the fused-threshold call drops |x| < tau itself
    x_raw = wl.silu_gated_sparse(wl.CFG_SPMSPV, 0, 4, K, 0.0)
    xrd = torch.from_numpy(x_raw).cuda()
    # kept entries per (256-row block, column): the runs the skipping kernel reads
    Mb = -(-M // 256)
    mpad = np.zeros((Mb * 256, K), dtype=bool)
    mpad[:M] = mask
    counts = mpad.reshape(Mb, 256, K).sum(axis=1)        # (Mb, K)
    run_bytes = 2 * counts + 32 + 4                        # kept values + 4 bitmap words + pointer (no padding)
    out = {"metric": "decode spMspV HBM throughput on algorithmic bytes", "unit": "GB/s", "n_gpus": 1,
           "higher_is_better": True, "dtype": "f16", "data": "synthetic", "detail": {},
           "config": {"workload": "spMspV down_proj 4096x11008, 50% unstructured, x = SiLU(g)*u, |x| < tau zeroed",
                      "tau": args.tau, "column_run_bytes": cr_bytes[0], "tiled_format_alg_bytes": fb,
                      "resident_bytes_per_handle": resident, "dense_weight_bytes": 2 * M * K}}
    for n in (1, 2, 4):
        active = np.any(x[:n] != 0, axis=0)
        alg = int(run_bytes[:, active].sum()) + 2 * K * n + 2 * M * n
        y = torch.empty((n, M), dtype=torch.float16, device="cuda")
        for i in range(2):
            swm.spmspv(fmts[i], xd[:n], y)
            swm.spmm(fmts[i], xd[:n], y)
            swm.dense_gemm(Wds[i], xd[:n], y)
        torch.cuda.synchronize()
        t_skip = G.time(G.capture([lambda i=i: swm.spmspv(fmts[i % C], xd[:n], y) for i in range(C)]), 3) / C
        t_full = G.time(G.capture([lambda i=i: swm.spmm(fmts[i % C], xd[:n], y) for i in range(C)]), 3) / C
        t_dense = G.time(G.capture([lambda i=i: swm.dense_gemm(Wds[i % CD], xd[:n], y) for i in range(CD)]), 3) / CD
        t_thr = G.time(G.capture([lambda i=i: swm.spmspv_threshold(fmts[i % C], xrd[:n], args.tau, y)
                                  for i in range(C)]), 3) / C
        t_cr = G.time(G.capture([lambda i=i: swm.spmspv_threshold(fmts[i % C], xd[:n], 0.0, y)
                                 for i in range(C)]), 3) / C
        out["detail"][str(n)] = {
            "fused_threshold_us": t_thr * 1e3, "column_run_kernel_us": t_cr * 1e3,
            "spmspv_route": "column-run skipping kernel" if n <= 2 else "full product (tiled)",
            "zero_frac": float(np.mean(x[:n] == 0)), "inactive_cols": float(1 - active.mean()),
            "spmspv_us": t_skip * 1e3, "spmm_us": t_full * 1e3, "dense_us": t_dense * 1e3,
            "alg_bytes": alg, "spmspv_GBps_alg": alg / (t_skip * 1e-3) / 1e9,
            "speedup_vs_dense": t_dense / t_skip, "speedup_vs_spmm": t_full / t_skip}
    d1 = out["detail"]["1"]
    out["value"] = d1["spmspv_GBps_alg"]
    out["roofline"] = {"bound": "hbm", "achieved": d1["spmspv_GBps_alg"], "peak": 8000.0, "unit": "GB/s",
                       "frac": d1["spmspv_GBps_alg"] / 8000.0, "traffic": None,
                       "kernel": "spmspv_cr_kernel, n=1", "alg_bytes_per_launch": d1["alg_bytes"],
                       "avg_launch_us": d1["spmspv_us"]}
    return out


# ------------------------------------------------------------------ decode FFN block
def bench_mlp(args, torch, swm, wl, G):
    """Decode FFN block of the Llama-2-7B-shaped layer (gate/up 11008x4096, down
    4096x11008, 50%): gate and up in one launch with the SiLU * mul epilogue
    and the threshold tau, then the skipping down projection; against the
    same chain unfused (two sparse products, SiLU * mul and the threshold as
    torch element-wise ops, the full sparse down product) and the dense chain
    (in-house dense kernel, same element-wise ops)."""
    _log("workload: decode FFN block, fused gate/up + threshold + skipping down")
    F = torch.nn.functional
    tau = args.tau
    Wg, mg, X = wl.layer_linear(4, 16)
    Wu, mu, _ = wl.layer_linear(5, 16)
    Wd, md, _ = wl.layer_linear(6, 1)
    fgs, fbg = rotating_formats(swm, Wg, mg)
    fus, fbu = rotating_formats(swm, Wu, mu)
    fds, fbd = rotating_formats(swm, Wd, md)
    _log(f"column-run encoding for {len(fds)} rotated down copies")
    for f in fds:
        f.enable_skipping()
    dgs, dus, dds = rotating_dense(torch, Wg), rotating_dense(torch, Wu), rotating_dense(torch, Wd)
    C, CD = min(len(fgs), len(fus), len(fds)), min(len(dgs), len(dus), len(dds))
    M, K = Wg.shape
    Xd = torch.from_numpy(X).cuda()
    out = {"metric": "decode FFN block time (gate/up fused with SiLU*mul and threshold, skipping down)",
           "unit": "us", "n_gpus": 1, "higher_is_better": False, "dtype": "f16", "data": "synthetic",
           "detail": {}, "config": {"workload": "Llama-2-7B FFN block, gate/up 11008x4096 + down 4096x11008, "
                                                "50% unstructured", "tau": tau}}
    for n in (1, 4, 16):
        H = torch.empty((n, M), dtype=torch.float16, device="cuda")
        g = torch.empty((n, M), dtype=torch.float16, device="cuda")
        u = torch.empty((n, M), dtype=torch.float16, device="cuda")
        y = torch.empty((n, K), dtype=torch.float16, device="cuda")
        x = Xd[:n]

        def epilogue():
            h = (F.silu(g.float()) * u.float()).half()
            return torch.where(h.abs() >= tau, h, torch.zeros_like(h))

        def glu(i):
            swm.gate_up_silu(fgs[i], fus[i], x, tau, H)

        def fused(i):
            swm.gate_up_silu(fgs[i], fus[i], x, tau, H)
            swm.spmspv(fds[i], H, y)

        def fused_full(i):
            swm.gate_up_silu(fgs[i], fus[i], x, tau, H)
            swm.spmm(fds[i], H, y)

        def two(i):
            swm.spmm(fgs[i], x, g)
            swm.spmm(fus[i], x, u)

        def unfused(i):
            swm.spmm(fgs[i], x, g)
            swm.spmm(fus[i], x, u)
            swm.spmm(fds[i], epilogue(), y)

        def dense(i):
            swm.dense_gemm(dgs[i], x, g)
            swm.dense_gemm(dus[i], x, u)
            swm.dense_gemm(dds[i], epilogue(), y)

        for i in range(2):
            fused(i), fused_full(i), unfused(i), dense(i)
        torch.cuda.synchronize()
        t = {name: G.time(G.capture([lambda i=i, fn=fn: fn(i % cc) for i in range(cc)]), 3) / cc * 1e3
             for name, fn, cc in (("fused_glu", glu, C), ("two_spmm", two, C), ("fused_chain", fused, C),
                                  ("fused_full_chain", fused_full, C), ("unfused_chain", unfused, C),
                                  ("dense_chain", dense, CD))}
        best = min(t["fused_chain"], t["fused_full_chain"])
        glu_alg = fbg + fbu + 2 * K * n + 2 * M * n
        swm.gate_up_silu(fgs[0], fus[0], x, tau, H)
        torch.cuda.synchronize()
        out["detail"][str(n)] = {
            "fused_glu_us": t["fused_glu"], "two_spmm_us": t["two_spmm"],
            "fused_glu_GBps_alg": glu_alg / (t["fused_glu"] * 1e-6) / 1e9,
            "fused_skip_chain_us": t["fused_chain"], "fused_full_chain_us": t["fused_full_chain"],
            "best_fused_chain_us": best, "unfused_chain_us": t["unfused_chain"],
            "dense_chain_us": t["dense_chain"], "h_zero_frac": float((H == 0).float().mean()),
            "h_inactive_cols": float((H == 0).all(dim=0).float().mean()),
            "speedup_vs_unfused": t["unfused_chain"] / best, "speedup_vs_dense": t["dense_chain"] / best}
        _log(f"n={n}: fused {t['fused_chain']:.2f} / {t['fused_full_chain']:.2f} us (skipping / full down), "
             f"unfused {t['unfused_chain']:.2f} us, dense {t['dense_chain']:.2f} us")
    out["prefill"] = mlp_prefill(args, torch, swm, wl, G)
    out["value"] = out["detail"]["1"]["best_fused_chain_us"]
    d1 = out["detail"]["1"]
    out["roofline"] = {"bound": "hbm", "achieved": d1["fused_glu_GBps_alg"], "peak": 8000.0, "unit": "GB/s",
                       "frac": d1["fused_glu_GBps_alg"] / 8000.0, "traffic": None,
                       "kernel": "decode_seq_kernel (gated), gate+up, n=1",
                       "alg_bytes_per_launch": fbg + fbu + 2 * K + 2 * M, "avg_launch_us": d1["fused_glu_us"]}
    return out


def mlp_prefill(args, torch, swm, wl, G, Ns=(512, 2048, 4096)):
    """The same FFN block at prefill token counts: gate and up through
    swm_gate_up_silu_ws (both expanded as interleaved rows, one dense MFMA
    product with the gated epilogue), then the down projection through
    swm_spmm_ws; against the dense baseline with the same gated epilogue
    (swm_dense_gate_up_silu on the interleaved masked weights, then
    swm_dense_gemm), and against both unfused (two products, SiLU * mul and
    the threshold as torch element-wise ops).  One call per graph replay,
    median of 10."""
    F = torch.nn.functional
    tau = args.tau
    nmax = max(Ns)
    _log(f"FFN block at prefill sizes (N = {', '.join(map(str, Ns))})")
    Wg, mg, X = wl.layer_linear(4, nmax)
    Wu, mu, _ = wl.layer_linear(5, nmax)
    Wd, md, _ = wl.layer_linear(6, 1)
    fg, fu, fd = swm.sparse_compress(Wg, mg), swm.sparse_compress(Wu, mu), swm.sparse_compress(Wd, md)
    dg, du, dd = (torch.from_numpy(w).cuda() for w in (Wg, Wu, Wd))
    M, K = Wg.shape
    W2 = np.empty((2 * M, K), dtype=np.float16)
    W2[0::2], W2[1::2] = Wg, Wu  # gate row m at 2m, up row m at 2m + 1
    d2 = torch.from_numpy(W2).cuda()
    del W2
    nnz = int(mg.sum()) + int(mu.sum())
    Xd = torch.from_numpy(X).cuda()
    wsb = max(swm.gate_up_silu_workspace_bytes(fg, fu, nmax), swm.spmm_workspace_bytes(fd, nmax), 256)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    res = {"workload": "Llama-2-7B FFN block, gate/up 11008x4096 + down 4096x11008, 50%, prefill", "tau": tau}
    for n in Ns:
        x = Xd[:n]
        H = torch.empty((n, M), dtype=torch.float16, device="cuda")
        g = torch.empty((n, M), dtype=torch.float16, device="cuda")
        u = torch.empty((n, M), dtype=torch.float16, device="cuda")
        y = torch.empty((n, K), dtype=torch.float16, device="cuda")

        def epilogue():
            h = (F.silu(g.float()) * u.float()).half()
            return torch.where(h.abs() >= tau, h, torch.zeros_like(h))

        fns = {
            "fused_glu": lambda: swm.gate_up_silu_ws(fg, fu, x, ws, tau, H),
            "two_spmm_ws_eltwise": lambda: (swm.spmm_ws(fg, x, ws, g), swm.spmm_ws(fu, x, ws, u), epilogue()),
            "dense_fused_glu": lambda: swm.dense_gate_up_silu(d2, x, tau, H),
            "dense_two_eltwise": lambda: (swm.dense_gemm(dg, x, g), swm.dense_gemm(du, x, u), epilogue()),
            "fused_chain": lambda: (swm.gate_up_silu_ws(fg, fu, x, ws, tau, H), swm.spmm_ws(fd, H, ws, y)),
            "unfused_chain": lambda: (swm.spmm_ws(fg, x, ws, g), swm.spmm_ws(fu, x, ws, u),
                                      swm.spmm_ws(fd, epilogue(), ws, y)),
            "dense_fused_chain": lambda: (swm.dense_gate_up_silu(d2, x, tau, H), swm.dense_gemm(dd, H, y)),
            "dense_chain": lambda: (swm.dense_gemm(dg, x, g), swm.dense_gemm(du, x, u),
                                    swm.dense_gemm(dd, epilogue(), y)),
        }
        for fn in fns.values():
            fn()
        torch.cuda.synchronize()
        graphs = [G.capture([fn]) for fn in fns.values()]
        d = {name: pct(t) for name, t in zip(fns, G.interleaved(graphs, 10, [1] * len(graphs)))}
        t = {k: v["median_us"] for k, v in d.items()}
        res[str(n)] = {**{k + "_us": v for k, v in t.items()},
                       "glu_useful_TFLOPs": 2.0 * nnz * n / (t["fused_glu"] * 1e-6) / 1e12,
                       "glu_speedup_vs_unfused": t["two_spmm_ws_eltwise"] / t["fused_glu"],
                       "glu_speedup_vs_dense_fused": t["dense_fused_glu"] / t["fused_glu"],
                       "chain_speedup_vs_unfused": t["unfused_chain"] / t["fused_chain"],
                       "chain_speedup_vs_dense_fused": t["dense_fused_chain"] / t["fused_chain"]}
        _log(f"prefill n={n}: gate/up fused {t['fused_glu']:.1f} us (dense fused {t['dense_fused_glu']:.1f}), "
             f"two spmm_ws + eltwise {t['two_spmm_ws_eltwise']:.1f}, two dense + eltwise "
             f"{t['dense_two_eltwise']:.1f}; chain fused {t['fused_chain']:.1f} (dense fused "
             f"{t['dense_fused_chain']:.1f}) / unfused {t['unfused_chain']:.1f} / dense unfused "
             f"{t['dense_chain']:.1f} us")
        del H, g, u, y
    del ws, d2
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ prefill
def bench_prefill(args, torch, swm, wl, G):
    _log("workload: prefill up/gate 11008x4096")
    out = {"metric": "prefill SpMM useful TFLOP/s (2*nnz*N / t)", "unit": "TFLOP/s", "n_gpus": 1,
           "higher_is_better": True, "dtype": "f16", "data": "synthetic", "detail": {}}
    Ns = [int(v) for v in args.prefill_n.split(",")]
    sps = [float(v) for v in args.prefill_s.split(",")]
    Xfull = None
    for s in sps:
        W, mask, X = wl.prefill_upgate(s, max(Ns))
        if Xfull is None:
            Xfull = torch.from_numpy(X).cuda()
        f = swm.sparse_compress(W, mask)
        Wd = torch.from_numpy(W).cuda()
        M, K = W.shape
        nnz = int(mask.sum())
        # workspace of spmm_ws: W expanded once per call for N >= 1024
        ws = torch.empty(max(swm.spmm_workspace_bytes(f, max(Ns)), 256), dtype=torch.uint8, device="cuda")
        reps = 5
        Wx = torch.empty_like(Wd)
        swm.decompress(f, Wx)
        torch.cuda.synchronize()
        t_dc = G.time(G.capture([lambda: swm.decompress(f, Wx)] * reps), 3) / reps
        del Wx
        out["detail"][f"s{s}_decompress"] = {
            "us": t_dc * 1e3, "alg_GBs": (fmt_alg_bytes(f.query()) + 2 * M * K) / (t_dc * 1e-3) / 1e9}
        for n in Ns:
            y = torch.empty((n, M), dtype=torch.float16, device="cuda")
            swm.spmm(f, Xfull[:n], y)
            swm.spmm_ws(f, Xfull[:n], ws, y)
            swm.dense_gemm(Wd, Xfull[:n], y)
            torch.cuda.synchronize()
            t_sp = G.time(G.capture([lambda: swm.spmm(f, Xfull[:n], y)] * reps), 3) / reps
            t_ws = G.time(G.capture([lambda: swm.spmm_ws(f, Xfull[:n], ws, y)] * reps), 3) / reps
            t_de = G.time(G.capture([lambda: swm.dense_gemm(Wd, Xfull[:n], y)] * reps), 3) / reps
            useful = 2.0 * nnz * n
            dense_fl = 2.0 * M * K * n
            out["detail"][f"s{s}_n{n}"] = {
                "spmm_ws_us": t_ws * 1e3, "ws_speedup_vs_dense": t_de / t_ws,
                "ws_route": "expand + dense MFMA" if swm.spmm_workspace_bytes(f, n) else "on-chip",
                "ws_useful_TFLOPs": useful / (t_ws * 1e-3) / 1e12,
                "onchip_us": t_sp * 1e3, "onchip_speedup_vs_dense": t_de / t_sp,
                "onchip_useful_TFLOPs": useful / (t_sp * 1e-3) / 1e12,
                "onchip_dense_equiv_TFLOPs": dense_fl / (t_sp * 1e-3) / 1e12,
                "dense_us": t_de * 1e3, "dense_TFLOPs": dense_fl / (t_de * 1e-3) / 1e12}
        del f, Wd, ws
    k0 = f"s{sps[0]}_n{Ns[-1]}"
    out["value"] = out["detail"][k0]["ws_useful_TFLOPs"]
    return out


# ------------------------------------------------------------------ layer
def bench_layer(args, torch, swm, wl, G):
    blk = layer_block(args, torch, swm, wl, G)
    return {"metric": "layer time, 7 linears back to back (N = 16)", "unit": "us", "n_gpus": 1,
            "higher_is_better": False, "dtype": "f16", "data": "synthetic",
            "value": blk["16"]["sparse_layer"]["median_us"], "detail": blk}


# ------------------------------------------------------------------ copy calibration
def bench_calib(args, torch, swm, wl, G):
    """A plain device copy of known size: its FETCH_SIZE / WRITE_SIZE counter
    readings scale the counters of the other kernels to bytes."""
    nbytes = 256 << 20
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t = G.time(G.capture([lambda: dst.copy_(src)] * 5), 3) / 5
    return {"metric": "device copy bandwidth (read + write)", "value": 2 * nbytes / (t * 1e-3) / 1e9,
            "unit": "GB/s", "n_gpus": 1, "higher_is_better": True, "dtype": "i32", "data": "synthetic",
            "config": {"workload": f"copy of {nbytes} bytes, 5 per graph replay"}}


# ------------------------------------------------------------------ wider workloads
def bench_wide(args, torch, swm, wl, G):
    """q_proj decode at 60% / 70% and with a 2:4 mask (N = 1, 16), and the
    moderate-sparsity paper's Fig. 1 shape 65536x16384 at N = 32 (and 16),
    each against the in-house dense kernel on W (.) mask."""
    _log("workload: wider shapes and sparsities")
    out = {"metric": "sparse speedup over the in-house dense kernel", "unit": "x", "n_gpus": 1,
           "higher_is_better": True, "dtype": "f16", "data": "synthetic", "detail": {},
           "config": {"workload": "q_proj 4096x4096 at 50% (N = 24, 32), 60% / 70% / 2:4 (N = 1, 16); down / up at 50% (N = 1, 16); 65536x16384 at 50% (N = 16, 32)"}}

    def measure(name, W, mask, X, Ns, rotate=True):
        M, K = W.shape
        if rotate:
            fmts, fb = rotating_formats(swm, W, mask)
            Wds = rotating_dense(torch, W)
        else:
            f0 = swm.sparse_compress(W, mask)
            fmts, fb = [f0], fmt_alg_bytes(f0.info)
            Wds = [torch.from_numpy(W).cuda()]
        C, CD = len(fmts), len(Wds)
        Xd = torch.from_numpy(X).cuda()
        for n in Ns:
            y = torch.empty((n, M), dtype=torch.float16, device="cuda")
            for i in range(2):
                swm.spmm(fmts[i % C], Xd[:n], y)
                swm.dense_gemm(Wds[i % CD], Xd[:n], y)
            torch.cuda.synchronize()
            reps = max(C, 4)
            t_sp = G.time(G.capture([lambda i=i: swm.spmm(fmts[i % C], Xd[:n], y) for i in range(reps)]), 3) / reps
            t_de = G.time(G.capture([lambda i=i: swm.dense_gemm(Wds[i % CD], Xd[:n], y) for i in range(reps)]), 3) / reps
            alg = fb + 2 * K * n + 2 * M * n
            out["detail"][f"{name} N={n}"] = {
                "sparse_us": t_sp * 1e3, "dense_us": t_de * 1e3, "speedup_vs_dense": t_de / t_sp,
                "format_MB": fb / 1e6, "sparse_GBps_alg": alg / (t_sp * 1e-3) / 1e9,
                "useful_TFLOPs": 2 * int(mask.sum()) * n / (t_sp * 1e-3) / 1e12}
            _log(f"{name} N={n}: sparse {t_sp * 1e3:.2f} us, dense {t_de * 1e3:.2f} us")
        del fmts, Wds
        torch.cuda.empty_cache()

    W, mask, X = wl.decode_qproj(32)
    measure("q_proj s=0.5", W, mask, X, (24, 32))
    for i, name in ((6, "down_proj 4096x11008 s=0.5"), (5, "up_proj 11008x4096 s=0.5")):
        W, mask, X = wl.layer_linear(i, 16)
        measure(name, W, mask, X, (1, 16))
    for s in (0.6, 0.7):
        W, mask, X = wl.decode_qproj_sparsity(s, 16)
        measure(f"q_proj s={s}", W, mask, X, (1, 16))
    W, mask, X = wl.decode_qproj_2_4(16)
    measure("q_proj 2:4", W, mask, X, (1, 16))
    W, mask, X = wl.fig1_shape()
    measure("fig1 65536x16384 s=0.5", W, mask, X, (16, 32), rotate=False)
    sp = [v["speedup_vs_dense"] for v in out["detail"].values()]
    out["value"] = float(np.exp(np.mean(np.log(sp))))  # geometric mean over the lines
    return out


# ------------------------------------------------------------------ prefill on the sparse matrix cores
def bench_smfmac(args, torch, swm, wl, G):
    """The 2:4 + residual route (W compacted into the 2:4 operand layout once,
    at compress time; spmm_ws then runs v_smfmac) against the expansion route
    (expand W to dense per call, then the dense MFMA kernel) and the dense
    kernel on W (.) mask: q_proj 4096x4096 with a 2:4 mask (no residual
    layer) and up/gate 11008x4096 at 50/60/70% forced onto the route with
    its residual layer."""
    _log("workload: prefill on the sparse matrix cores")
    out = {"metric": "prefill useful TFLOP/s on the sparse matrix cores", "unit": "TFLOP/s", "n_gpus": 1,
           "higher_is_better": True, "dtype": "f16", "data": "synthetic", "detail": {}}
    reps = 4
    cases = [("q_proj 2:4", wl.decode_qproj_2_4(1)[:2], (4096,) if args.quick else (1024, 2048, 4096))]
    for sp in (() if args.quick else (0.5, 0.6, 0.7)):
        W, mask, _ = wl.prefill_upgate(sp, 1)
        cases.append((f"up/gate {int(sp * 100)}%", (W, mask), (2048, 4096)))
    Xall = torch.from_numpy(wl.activations(wl.CFG_PREFILL, 0, 4096, 11008)).cuda()
    for name, (W, mask), Ns in cases:
        M, K = W.shape
        nnz = int(mask.sum())
        f = swm.sparse_compress(W, mask, smfmac=True)
        Wd = torch.from_numpy(W).cuda()
        Wx = torch.empty_like(Wd)
        for n in Ns:
            X = Xall[:n, :K].contiguous()
            y = torch.empty((n, M), dtype=torch.float16, device="cuda")
            ws = torch.empty(max(swm.spmm_workspace_bytes(f, n), 256), dtype=torch.uint8, device="cuda")
            def route():
                swm.spmm_ws(f, X, ws, y)
            def expand():
                swm.decompress(f, Wx)
                swm.dense_gemm(Wx, X, y)
            def dense():
                swm.dense_gemm(Wd, X, y)
            for fn in (route, expand, dense):
                fn()
            torch.cuda.synchronize()
            t = {nm: pct(G.samples(G.capture([fn] * reps), 8, reps))["median_us"]
                 for nm, fn in (("smfmac_route", route), ("expand_route", expand), ("dense", dense))}
            useful = 2.0 * nnz * n
            e = {k + "_us": v for k, v in t.items()}
            e.update({"useful_TFLOPs": useful / (t["smfmac_route"] * 1e-6) / 1e12,
                      "speedup_vs_dense": t["dense"] / t["smfmac_route"],
                      "speedup_vs_expand": t["expand_route"] / t["smfmac_route"]})
            out["detail"][f"{name} N={n}"] = e
            _log(f"{name} N={n}: smfmac route {t['smfmac_route']:.1f} us, expand route {t['expand_route']:.1f} us, "
                 f"dense {t['dense']:.1f} us")
            del ws, y
        del f, Wd, Wx
        torch.cuda.empty_cache()
    out["value"] = out["detail"]["q_proj 2:4 N=4096"]["useful_TFLOPs"]
    return out


# ------------------------------------------------------------------ batch-aware skipping experiment
def group_tokens(zero, size, greedy=True, seed=0):
    """Partition the tokens (rows of the boolean zero-pattern matrix) into
    groups of `size`: greedy by the number of columns zero in every member
    (the columns a group's skipping call can drop), or at random."""
    T = zero.shape[0]
    left = list(range(T))
    if size == 1:
        return [[t] for t in left]
    if not greedy:
        left = list(np.random.default_rng(seed).permutation(T))
        return [left[i:i + size] for i in range(0, T, size)]
    groups = []
    while left:
        best = None
        for a in left:  # seed each group with the token pair sharing the most zeros
            for b in left:
                if a < b:
                    c = int(np.count_nonzero(zero[a] & zero[b]))
                    if best is None or c > best[0]:
                        best = (c, [a, b])
        g = best[1] if best else [left[0]]
        common = np.logical_and.reduce(zero[g], axis=0)
        while len(g) < size and len(g) < len(left):
            c, t = max((int(np.count_nonzero(common & zero[t])), t) for t in left if t not in g)
            g.append(t)
            common &= zero[t]
        groups.append(g)
        left = [t for t in left if t not in g]
    return groups


def bench_batchskip(args, torch, swm, wl, G):
    """Batch-aware skipping for 16 decode tokens on the down_proj shape
    ("Reduced Matrix Multiplication" blog page, Sec. 6.2: group tokens by
    channel pattern so skipping survives in a batch): the tokens are split
    into groups (greedy by shared zero columns, or random) and every group
    runs the column-run skipping kernel, each group reading the active runs
    of W again; against one full product of all 16 tokens."""
    _log("workload: batch-aware skipping, 16 tokens, down_proj 4096x11008")
    T = 16
    W, mask, _ = wl.spmspv_down(1, args.tau)
    M, K = W.shape
    fmts, fa = rotating_formats(swm, W, mask)
    for f in fmts:
        f.enable_skipping()
    C = len(fmts)
    x = wl.silu_gated_sparse(wl.CFG_SPMSPV, 1, T, K, args.tau)
    zero = x == 0
    xd = torch.from_numpy(x).cuda()
    y = torch.empty((T, M), dtype=torch.float16, device="cuda")
    out = {"metric": "batch-aware skipping: time for 16 decode tokens", "unit": "us", "n_gpus": 1,
           "higher_is_better": False, "dtype": "f16", "data": "synthetic", "detail": {},
           "config": {"workload": "down_proj 4096x11008 50%, 16 tokens of x = SiLU(g)*u with |x| < tau zeroed",
                      "tau": args.tau, "zero_frac": float(zero.mean()),
                      "inactive_cols_all16": float(np.logical_and.reduce(zero, axis=0).mean())}}
    swm.spmm(fmts[0], xd, y)
    torch.cuda.synchronize()
    full = G.time(G.capture([lambda i=i: swm.spmm(fmts[i % C], xd, y) for i in range(C)]), 5) / C
    out["detail"]["full product, N=16"] = {"us": full * 1e3, "calls": 1}
    for size in (1, 2, 4):
        for greedy in ((True, False) if size > 1 else (True,)):
            groups = group_tokens(zero, size, greedy)
            idx = [torch.tensor(g, device="cuda") for g in groups]
            xs = [xd.index_select(0, t).contiguous() for t in idx]   # gathered once, outside the timing
            ys = [torch.empty((len(g), M), dtype=torch.float16, device="cuda") for g in groups]
            inact = [float(np.logical_and.reduce(zero[g], axis=0).mean()) for g in groups]

            def run(i):
                for xg, yg in zip(xs, ys):
                    swm.spmspv_threshold(fmts[i % C], xg, 0.0, yg)
            run(0)
            torch.cuda.synchronize()
            t = G.time(G.capture([lambda i=i: run(i) for i in range(C)]), 3) / C
            name = f"groups of {size}" + ("" if size == 1 else (", greedy" if greedy else ", random"))
            out["detail"][name] = {"us": t * 1e3, "calls": len(groups), "vs_full": full / t,
                                   "mean_inactive_cols": float(np.mean(inact)),
                                   "min_inactive_cols": float(np.min(inact)), "max_inactive_cols": float(np.max(inact))}
            _log(f"{name}: {t * 1e3:.1f} us in {len(groups)} calls (full product {full * 1e3:.1f} us), "
                 f"inactive columns per group {np.mean(inact):.3f}")
    out["value"] = min(v["us"] for v in out["detail"].values())
    return out


# ------------------------------------------------------------------ decode across shapes (also the profiling driver)
def bench_decodeshapes(args, torch, swm, wl, G):
    """Decode SpMM on the layer's shapes (q_proj 4096x4096, up 11008x4096, down
    4096x11008, 50%) at N = 1 and 16, each against the library's streaming
    kernel at the same algorithmic byte count and rotation, and the dense
    kernel.  Short: also the driver for kernel traces and counter passes."""
    _log("workload: decode across the layer's shapes")
    out = {"metric": "decode HBM throughput on algorithmic bytes across shapes", "unit": "GB/s", "n_gpus": 1,
           "higher_is_better": True, "dtype": "f16", "data": "synthetic", "detail": {}}
    reps = args.reps
    for i, name in ((0, "q_proj 4096x4096"), (5, "up 11008x4096"), (6, "down 4096x11008")):
        W, mask, X = wl.layer_linear(i, 16)
        fmts, fa = rotating_formats(swm, W, mask)
        Wds = rotating_dense(torch, W)
        C, CD = len(fmts), len(Wds)
        M, K = W.shape
        Xd = torch.from_numpy(X).cuda()
        for n in (1, 16):
            y = torch.empty((n, M), dtype=torch.float16, device="cuda")
            for f in fmts[:2]:
                swm.spmm(f, Xd[:n], y)
            swm.dense_gemm(Wds[0], Xd[:n], y)
            torch.cuda.synchronize()
            ds = pct(G.samples(G.capture([lambda i=i: swm.spmm(fmts[i % C], Xd[:n], y) for i in range(C)]), reps, C))
            dd = pct(G.samples(G.capture([lambda i=i: swm.dense_gemm(Wds[i % CD], Xd[:n], y) for i in range(CD)]),
                               reps, CD))
            alg = fa + 2 * K * n + 2 * M * n
            st = stream_achievable(torch, swm, G, alg) if not args.no_stream else None
            e = {"sparse": ds, "dense": dd, "alg_bytes": alg,
                 "GBps_alg": alg / (ds["median_us"] * 1e-6) / 1e9,
                 "speedup_vs_dense": dd["median_us"] / ds["median_us"]}
            if st:
                e["stream"] = st
                e["frac_of_stream"] = st["us"] / ds["median_us"]
            out["detail"][f"{name} N={n}"] = e
            _log(f"{name} N={n}: sparse {ds['median_us']:.2f} us ({e['GBps_alg']:.0f} GB/s), dense "
                 f"{dd['median_us']:.2f} us" + (f", stream {st['us']:.2f} us" if st else ""))
        del fmts, Wds
        torch.cuda.empty_cache()
    out["value"] = out["detail"]["q_proj 4096x4096 N=16"]["GBps_alg"]
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "spmspv", "prefill", "layer", "wide", "mlp", "calib", "decodeshapes",
                             "batchskip", "smfmac"])
    ap.add_argument("--reps", type=int, default=20, help="graph replays per timing (decodeshapes)")
    ap.add_argument("--no-stream", action="store_true", help="decodeshapes without the streaming-kernel sweep")
    ap.add_argument("--quick", action="store_true", help="smfmac: only q_proj 2:4 at N = 4096 (profiling driver)")
    ap.add_argument("--tau", type=float, default=0.3)
    ap.add_argument("--prefill-n", default="512,2048,4096")
    ap.add_argument("--prefill-s", default="0.5,0.6,0.7")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--decode-only", action="store_true", help="default workload without the prefill and layer blocks")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported: the library "
              "has no multi-GPU path (the sharding design is described in the docs)", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_weight_matmul_amd as swm
    import swm_workloads as wl
    swm.load()
    torch.cuda.set_device(0)
    G = Graphs(torch)
    fn = {"decode": bench_default, "spmspv": bench_spmspv, "prefill": bench_prefill, "layer": bench_layer,
          "wide": bench_wide, "mlp": bench_mlp, "calib": bench_calib, "decodeshapes": bench_decodeshapes,
          "batchskip": bench_batchskip, "smfmac": bench_smfmac}
    out = fn[args.workload](args, torch, swm, wl, G)
    out.setdefault("n_gpus", 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
