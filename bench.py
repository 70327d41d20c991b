"""Benchmark: batch-1 AQLM GEMV over the Llama-2-7B linear-layer set (scheme 2x8).

One step = aqlm_gemv on each of the seven Llama-2-7B linear layers
(q, k, v, o: 4096x4096; gate, up: 11008x4096; down: 4096x11008), scheme 2x8
(two 8-bit codebooks, codeword length 8), one activation row, on seeded
synthetic weights. The codes, scales, activations and outputs are rotated
over enough distinct copies (>= 1 GiB of codes) that every step reads its
codes from HBM, not from the 256 MiB last-level cache; the 8 KiB codebooks
are shared.

Reported value: achieved HBM GB/s = (codes + x + y bytes of the seven layers)
/ time per step, timed with HIP events on the stream the kernels run on,
bracketed by device synchronisation. Also reported: microseconds per layer,
the roofline object of the GEMV kernel and the CPU oracle timed on a bounded
sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "AQLM GEMV µs/layer + achieved HBM GB/s (% of peak), Llama-2-7B shapes, batch 1"
WORKLOAD = "llama2_7b_2x8"
HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 1 << 30
GEMV_KERNEL = "gemv_fast_kernel<2x8, batch 1>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_2x8_llama2_7b_b1_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "additive_codebook_matmul_amd", "csrc", "gemv.hip")


def _parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--layer-iters", type=int, default=200,
                   help="launches per layer for the per-layer timing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def _source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic():
    """HBM bytes per step from rocprofv3 counters, if taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != _source_hash():
        return None
    return t.get("bytes_per_step")


def cpu_baseline(layers_np, budget_s: float = 12.0):
    """The CPU oracle (decode in float32, product in float64) on the same layers."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the interpreter's one thread
        blas_threads = 1
    done_bytes = 0
    done_layers = 0
    t0 = time.perf_counter()
    while True:
        for (layer, d, x, nbytes) in layers_np:
            oracle.forward(x, d.codes, d.codebooks, d.scales)
            done_bytes += nbytes
            done_layers += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    _ = np
    return {
        "value": round(done_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{done_layers} layer products of the seven Llama-2-7B 2x8 layers at batch 1 "
                  f"(whole passes over the layer set, {dt:.1f} s); numpy decode is single-threaded, "
                  f"the float64 product uses BLAS with up to {blas_threads} threads",
    }


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from additive_codebook_matmul_amd import AqlmLayer, load_library
    from additive_codebook_matmul_amd import workloads as WL

    load_library()
    dev = torch.device("cuda:0")
    wl = WL.WORKLOADS[WORKLOAD]

    layers_np = []
    for layer in wl.layers:
        d = WL.make_layer(layer)
        x = WL.make_x(layer, 1)
        b = WL.workload_bytes(layer, 1)
        layers_np.append((layer, d, x, b["codes"] + b["x"] + b["y"]))
    code_bytes = sum(d.codes.nbytes for (_, d, _, _) in layers_np)
    copies = max(2, -(-ROTATE_BYTES // code_bytes))

    # device copies: copy c of layer l
    base = []
    for (layer, d, x, _) in layers_np:
        base.append((torch.from_numpy(d.codes).to(dev), torch.from_numpy(d.codebooks).to(dev),
                     torch.from_numpy(d.scales).to(dev), torch.from_numpy(x).to(dev)))
    rot = []
    for c in range(copies):
        row = []
        for (codes, books, scales, x) in base:
            L = AqlmLayer(codes.clone(), books, scales.clone())
            xx = x.clone()
            yy = torch.empty((1, L.out_features), dtype=torch.float16, device=dev)
            row.append((L, xx, yy))
        rot.append(row)
    torch.cuda.synchronize()

    def step(i):
        for (L, xx, yy) in rot[i % copies]:
            L.gemv(xx, out=yy)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps

    # per-layer timing: the same layer launched back to back over the rotated copies
    us_layer, gbps_layer = {}, {}
    for li, (layer, _, _, nbytes) in enumerate(layers_np):
        for i in range(10):
            L, xx, yy = rot[i % copies][li]
            L.gemv(xx, out=yy)
        torch.cuda.synchronize()
        start.record()
        for i in range(args.layer_iters):
            L, xx, yy = rot[i % copies][li]
            L.gemv(xx, out=yy)
        end.record()
        torch.cuda.synchronize()
        us = start.elapsed_time(end) * 1e3 / args.layer_iters
        us_layer[layer.name] = round(us, 3)
        gbps_layer[layer.name] = round(nbytes / us / 1e3, 1)

    step_bytes = sum(nb for (_, _, _, nb) in layers_np)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    launches = len(layers_np)
    traffic = _traffic()
    roofline = {
        "bound": "hbm",
        "kernel": GEMV_KERNEL,
        "achieved": round(value, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(value / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "bytes_per_launch_avg": step_bytes // launches,
        "avg_launch_us": round(ms_per_step * 1e3 / launches, 3),
    }

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD,
            "scheme": "2x8 (M=2, B=8, g=8)",
            "batch": 1,
            "layers": {l.name: [l.out_features, l.in_features] for (l, _, _, _) in layers_np},
            "bytes_per_step": step_bytes,
            "rotated_copies": copies,
            "us_per_layer": us_layer,
            "gbps_per_layer": gbps_layer,
            "pct_of_peak_per_layer": {k: round(100 * v / HBM_PEAK_GBPS, 1)
                                      for k, v in gbps_layer.items()},
            "accumulate": "fp32",
        },
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers_np)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
