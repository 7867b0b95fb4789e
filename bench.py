"""Benchmark of the sparse-weight matmul hot path on one MI355X.

Default workload (``--workload decode``): the q_proj shape -- W 4096x4096 fp16
at 50% per-row magnitude pruning, compressed to the tiled column-bitmap format.
One step = three sparse products with N = 1, 8 and 16 tokens.  The same step
is timed with the in-house dense GEMM on the masked W stored dense, for the
speedup.  ``value`` = algorithmic bytes of the sparse products (compressed
weight + X + Y) / their GPU time, in GB/s, inputs resident in HBM.

Timing: launches are captured once into HIP graphs (torch.cuda.CUDAGraph) and
replayed, so host launch overhead does not starve the GPU; HIP events on the
launch stream bracket the replays.  Copies of the weight are rotated so the
working set exceeds 1 GiB (4x the 256 MB Infinity Cache) and every launch
streams its weight from HBM.

Other workloads: ``spmspv`` (down_proj 4096x11008, SiLU-gated x with |x|<0.3
zeroed, N = 1 and 4), ``prefill`` (up/gate 11008x4096, N = 512/2048/4096,
sparsity 0.5/0.6/0.7), ``layer`` (seven Llama-2-7B linears back to back, N =
16 and 4096).  Each prints one JSON line.
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
    return int(info["bytes_tile_ptr"] + info["bytes_bits"] + info["bytes_values"])


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


def rotating_formats(swm, W, mask, min_bytes=ROTATE_BYTES):
    f0 = swm.sparse_compress(W, mask)
    fb = fmt_bytes(f0.info)
    copies = max(2, int(np.ceil(min_bytes / fb)))
    blob = f0.export()
    return [f0] + [swm.format_import(blob) for _ in range(copies - 1)], fb


def rotating_dense(torch, W, min_bytes=ROTATE_BYTES):
    Wd = torch.from_numpy(W).cuda()
    copies = max(2, int(np.ceil(min_bytes / (W.size * 2))))
    return [Wd] + [Wd.clone() for _ in range(copies - 1)]


def profiled_traffic(profile_md):
    """HBM bytes per launch from a committed counter summary, if the kernel
    source it was taken on is the one built now; else None."""
    import hashlib
    import re
    try:
        text = open(os.path.join(ROOT, "profiles", profile_md)).read()
        meta = json.loads(re.search(r"<!-- bench-traffic: (\{.*\}) -->", text).group(1))
        src = open(os.path.join(ROOT, meta["source"]), "rb").read()
    except (OSError, AttributeError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != meta["source_sha256"]:
        return None
    return int(meta["traffic_bytes_per_launch"])


def threads_used():
    try:
        from threadpoolctl import threadpool_info
        return int(max([d.get("num_threads", 1) for d in threadpool_info()] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_oracle(W, mask, X_list, units, unit, budget_s=20.0):
    """The oracle (numpy float64 masked-W @ X, as it stands) on the host cores."""
    import oracle
    Wm = np.where(mask, W.astype(np.float64), 0.0)  # untimed preparation
    t_tot, u_tot = 0.0, 0.0
    for X, u in zip(X_list, units):
        oracle.masked_matmul(W[:4], mask[:4], X[:1])
        X64 = X.astype(np.float64)
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            _ = Wm @ X64.T
            ts.append(time.perf_counter() - t0)
            if sum(ts) > budget_s:
                break
        t_tot += float(np.median(ts))
        u_tot += u
    return {"value": u_tot / t_tot, "unit": unit, "cores": threads_used(), "kind": "oracle"}


# ------------------------------------------------------------------ decode (default)
def bench_decode(args, torch, swm, wl, G):
    _log("workload: decode q_proj 4096x4096, 50%")
    W, mask, X = wl.decode_qproj(16)
    fmts, fb = rotating_formats(swm, W, mask)
    Wds = rotating_dense(torch, W)
    C, CD = len(fmts), len(Wds)
    _log(f"format {fb / 1e6:.2f} MB, {C} sparse / {CD} dense rotating copies")
    Xd = torch.from_numpy(X).cuda()
    Ns = (1, 8, 16)
    M, K = W.shape
    Ys = {n: torch.empty((n, M), dtype=torch.float16, device="cuda") for n in Ns}
    alg = {n: fb + 2 * K * n + 2 * M * n for n in Ns}
    dense_b = {n: 2 * M * K + 2 * K * n + 2 * M * n for n in Ns}

    def sp(i, n):
        return lambda: swm.spmm(fmts[i % C], Xd[:n], Ys[n])

    def de(i, n):
        return lambda: swm.dense_gemm(Wds[i % CD], Xd[:n], Ys[n])

    for r in range(2):  # untimed: builds workspaces, warms the code paths
        for n in Ns:
            sp(r, n)()
            de(r, n)()
    torch.cuda.synchronize()
    per_n, per_n_d = {}, {}
    for n in Ns:
        gs = G.capture([sp(i, n) for i in range(C)])
        gd = G.capture([de(i, n) for i in range(CD)])
        per_n[n] = G.time(gs, 3) / C
        per_n_d[n] = G.time(gd, 3) / CD
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
    detail = {str(n): {"sparse_us": per_n[n] * 1e3, "dense_us": per_n_d[n] * 1e3,
                       "speedup_vs_dense": per_n_d[n] / per_n[n],
                       "sparse_GBps_alg": alg[n] / (per_n[n] * 1e-3) / 1e9,
                       "sparse_frac_hbm": alg[n] / (per_n[n] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "dense_GBps": dense_b[n] / (per_n_d[n] * 1e-3) / 1e9} for n in Ns}
    dom = 16
    ach = alg[dom] / (per_n[dom] * 1e-3) / 1e9
    out = {
        "metric": "decode SpMM HBM throughput on compressed bytes (q_proj 4096x4096, 50%)",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic (seeded N(0,1) fp16 W and X, 50% per-row magnitude pruning)",
        "config": {"workload": "decode q_proj 4096x4096, 50% unstructured, N in {1,8,16} per step",
                   "format": "SWM-TCB v2 tm=16 tk=64", "format_bytes": fb, "rotating_copies": C},
        "speedup_vs_dense": ms_dense / ms_total,
        "dense_ms_per_step": ms_dense / args.steps,
        "detail": detail,
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS,
                     "traffic": profiled_traffic("decode_seq_kernel_qproj_pmc.md"),
                     "kernel": "decode_seq_kernel, N=16", "alg_bytes_per_launch": alg[dom],
                     "avg_launch_us": per_n[dom] * 1e3},
        "timed_wall_s": wall,
    }
    if not args.no_cpu:
        _log("timing the CPU oracle")
        cb = cpu_oracle(W, mask, [X[:n] for n in Ns], [alg[n] for n in Ns], "B")
        cb["value"] = cb["value"] / 1e9
        cb["unit"] = "GB/s"
        cb["sample"] = "one full decode step (N = 1, 8, 16), numpy float64 masked-W @ X, median of 3"
        out["cpu_baseline"] = cb
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
                      "tau": args.tau, "column_run_bytes": cr_bytes[0], "tiled_format_bytes": fb}}
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
        out["detail"][str(n)] = {
            "fused_threshold_us": t_thr * 1e3,
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
    out["value"] = out["detail"]["1"]["best_fused_chain_us"]
    d1 = out["detail"]["1"]
    out["roofline"] = {"bound": "hbm", "achieved": d1["fused_glu_GBps_alg"], "peak": 8000.0, "unit": "GB/s",
                       "frac": d1["fused_glu_GBps_alg"] / 8000.0, "traffic": None,
                       "kernel": "decode_seq_kernel (gated), gate+up, n=1",
                       "alg_bytes_per_launch": fbg + fbu + 2 * K + 2 * M, "avg_launch_us": d1["fused_glu_us"]}
    return out


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
            "us": t_dc * 1e3, "alg_GBs": (fmt_bytes(f.query()) + 2 * M * K) / (t_dc * 1e-3) / 1e9}
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
    _log("workload: Llama-2-7B-shaped layer, 7 linears")
    out = {"metric": "layer time, 7 linears back to back", "unit": "us", "n_gpus": 1,
           "higher_is_better": False, "dtype": "f16", "data": "synthetic", "detail": {}}
    lin = []
    for i in range(7):
        W, mask, X = wl.layer_linear(i, 4096)
        f = swm.sparse_compress(W, mask)
        lin.append((f, torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda(), W.shape))
    # one workspace shared by the seven linears (calls ordered on one stream)
    ws = torch.empty(max(max(swm.spmm_workspace_bytes(f, 4096) for (f, _, _, _) in lin), 256),
                     dtype=torch.uint8, device="cuda")
    for n in (16, 4096):
        ys = [torch.empty((n, shp[0]), dtype=torch.float16, device="cuda") for (_, _, _, shp) in lin]
        for (f, Wd, Xd, _), y in zip(lin, ys):
            swm.spmm(f, Xd[:n], y)
            swm.spmm_ws(f, Xd[:n], ws, y)
            swm.dense_gemm(Wd, Xd[:n], y)
        torch.cuda.synchronize()
        gs = G.capture([lambda f=f, Xd=Xd, y=y: swm.spmm(f, Xd[:n], y) for (f, _, Xd, _), y in zip(lin, ys)])
        gw = G.capture([lambda f=f, Xd=Xd, y=y: swm.spmm_ws(f, Xd[:n], ws, y) for (f, _, Xd, _), y in zip(lin, ys)])
        gd = G.capture([lambda Wd=Wd, Xd=Xd, y=y: swm.dense_gemm(Wd, Xd[:n], y) for (_, Wd, Xd, _), y in zip(lin, ys)])
        ts, tw, td = G.time(gs, 5), G.time(gw, 5), G.time(gd, 5)
        out["detail"][str(n)] = {"sparse_us": ts * 1e3, "spmm_ws_us": tw * 1e3, "dense_us": td * 1e3,
                                 "speedup_vs_dense": td / ts, "ws_speedup_vs_dense": td / tw,
                                 "note": "no rotation: the compressed layer (228 MB) fits the 256 MB "
                                         "Infinity Cache, the dense one (405 MB) does not; spmm_ws "
                                         "shares one workspace across the seven linears"}
    out["value"] = out["detail"]["16"]["sparse_us"]
    return out


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
            fmts, fb = [f0], fmt_bytes(f0.info)
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["decode", "spmspv", "prefill", "layer", "wide", "mlp", "calib"])
    ap.add_argument("--tau", type=float, default=0.3)
    ap.add_argument("--prefill-n", default="512,2048,4096")
    ap.add_argument("--prefill-s", default="0.5,0.6,0.7")
    ap.add_argument("--no-cpu", action="store_true")
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
    fn = {"decode": bench_decode, "spmspv": bench_spmspv, "prefill": bench_prefill, "layer": bench_layer,
          "wide": bench_wide, "mlp": bench_mlp, "calib": bench_calib}
    out = fn[args.workload](args, torch, swm, wl, G)
    out.setdefault("n_gpus", 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
