"""Benchmark of the sparse-weight matmul hot path on one MI355X.

Default workload: decode on the q_proj shape -- W 4096x4096 fp16, 50% per-row
magnitude pruning, compressed to the tiled column-bitmap format; one step is
three sparse products with N = 1, 8 and 16 tokens.  The same step is timed for
the in-house dense GEMM on the same (masked, dense-stored) W for the speedup.

value = algorithmic bytes moved by the sparse products (compressed weight
+ X + Y) / their time, in GB/s, inputs resident in HBM.  Copies of the weight
are rotated so that the working set exceeds 1 GiB (4x the 256 MB Infinity
Cache) and every launch streams its weight from HBM.

Other workloads (--workload): spmspv (down_proj, SiLU-gated x, N=1 and 4),
prefill (up/gate 11008x4096, N = 512/2048/4096, s = 0.5/0.6/0.7),
layer (seven Llama-2-7B linears back to back, N = 16 and 4096).
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


def _fmt_bytes(info):
    return int(info["bytes_tile_ptr"] + info["bytes_bits"] + info["bytes_values"])


class Timer:
    """HIP events on the launch stream (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, reps):
        torch = self.torch
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for r in range(reps):
            fn(r)
        e1.record(s)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps  # ms per call


def cpu_oracle_baseline(W, mask, X_list, alg_bytes_list, budget_s=20.0):
    """Time the oracle (numpy fp64 product of the masked W) on the host cores."""
    import oracle
    from threadpoolctl import threadpool_info
    Wm = np.where(mask, W.astype(np.float64), 0.0)  # precomputed, untimed
    times, nbytes = [], 0
    for X, ab in zip(X_list, alg_bytes_list):
        X64 = X.astype(np.float64)
        oracle.masked_matmul(W[:8], mask[:8], X[:1])  # warm the code path
        t = []
        for _ in range(3):
            t0 = time.perf_counter()
            _ = Wm @ X64.T
            t.append(time.perf_counter() - t0)
        times.append(float(np.median(t)))
        nbytes += ab
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    return {"value": nbytes / sum(times) / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": "the full decode step (N = 1, 8, 16) as numpy float64 masked-W @ X, median of 3"}


def bench_decode(args, torch, swm, wl):
    _log("building q_proj workload")
    W, mask, X = wl.decode_qproj(16)
    f0 = swm.sparse_compress(W, mask)
    info = f0.info
    fbytes = _fmt_bytes(info)
    blob = f0.export()
    copies = max(2, int(np.ceil(ROTATE_BYTES / fbytes)))
    _log(f"format {fbytes / 1e6:.2f} MB, {copies} rotating copies")
    fmts = [f0] + [swm.format_import(blob) for _ in range(copies - 1)]
    Wd = torch.from_numpy(W).cuda()
    dcopies = max(2, int(np.ceil(ROTATE_BYTES / (W.size * 2))))
    Wds = [Wd] + [Wd.clone() for _ in range(dcopies - 1)]
    Xd = torch.from_numpy(X).cuda()
    Ns = (1, 8, 16)
    Ys = {n: torch.empty((n, 4096), dtype=torch.float16, device="cuda") for n in Ns}
    M, K = W.shape
    alg = {n: fbytes + 2 * K * n + 2 * M * n for n in Ns}
    dense_bytes = {n: 2 * M * K + 2 * K * n + 2 * M * n for n in Ns}
    timer = Timer(torch)

    def sparse_step(r):
        for n in Ns:
            swm.spmm(fmts[(r * 3 + n) % copies], Xd[:n], Ys[n])

    def dense_step(r):
        for n in Ns:
            swm.dense_gemm(Wds[(r * 3 + n) % dcopies], Xd[:n], Ys[n])

    # warmup
    for r in range(args.warmup):
        sparse_step(r)
        dense_step(r)
    torch.cuda.synchronize()
    per_n, per_n_dense = {}, {}
    reps_n = max(50, args.steps * 5)
    for n in Ns:
        per_n[n] = timer.run(lambda r, n=n: swm.spmm(fmts[r % copies], Xd[:n], Ys[n]), reps_n)
        per_n_dense[n] = timer.run(lambda r, n=n: swm.dense_gemm(Wds[r % dcopies], Xd[:n], Ys[n]), reps_n)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_sparse = timer.run(sparse_step, args.steps)
    wall = time.perf_counter() - t0
    ms_dense = timer.run(dense_step, args.steps)
    total_alg = sum(alg.values())
    value = total_alg / (ms_sparse * 1e-3) / 1e9
    detail = {
        str(n): {"sparse_us": per_n[n] * 1e3, "dense_us": per_n_dense[n] * 1e3,
                 "speedup_vs_dense": per_n_dense[n] / per_n[n],
                 "sparse_GBps_alg": alg[n] / (per_n[n] * 1e-3) / 1e9,
                 "dense_GBps": dense_bytes[n] / (per_n_dense[n] * 1e-3) / 1e9}
        for n in Ns
    }
    dom_n = 16
    achieved = alg[dom_n] / (per_n[dom_n] * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": None,
            "kernel": "decode_kernel (spmm, N=16)", "alg_bytes_per_launch": alg[dom_n]}
    out = {
        "metric": "decode SpMM HBM throughput on compressed bytes (q_proj 4096x4096, 50%)",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_sparse, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic (seeded N(0,1) fp16, 50% per-row magnitude pruning)",
        "config": {"workload": "decode q_proj 4096x4096, 50% unstructured, N in {1,8,16}",
                   "format": "SWM-TCB v1 tm=64 tk=64", "format_bytes": fbytes,
                   "rotating_copies": copies},
        "speedup_vs_dense": ms_dense / ms_sparse,
        "dense_ms_per_step": ms_dense,
        "detail": detail,
        "roofline": roof,
        "wall_s_timed_region": wall,
    }
    if not args.no_cpu:
        _log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_oracle_baseline(W, mask, [X[:n] for n in Ns], [alg[n] for n in Ns])
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["decode"])
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the product path has no multi-GPU code)", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_weight_matmul_amd as swm
    import swm_workloads as wl
    swm.load()
    torch.cuda.set_device(0)
    out = bench_decode(args, torch, swm, wl)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
