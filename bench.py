"""Benchmark: batch-1 AQLM GEMV over the Llama-2-7B linear-layer set (scheme 2x8).

One step = the seven Llama-2-7B linear layers of one transformer block
(q, k, v, o: 4096x4096; gate, up: 11008x4096; down: 4096x11008), scheme 2x8
(two 8-bit codebooks, codeword length 8), one activation row, seeded
synthetic weights, issued the way a decode step can issue them: q, k and v
share their input and go out as one aqlm_gemv_batched call, then o, then gate
and up (shared input) as one batched call, then down. The codes, scales,
activations and outputs are rotated over enough distinct copies (>= 1 GiB of
codes) that every step reads its codes from HBM, not from the 256 MiB
last-level cache; the 8 KiB codebooks are shared.

Reported value: achieved HBM GB/s = (codes + x + y bytes of the seven layers)
/ time per step, timed with HIP events on the stream the kernels run on,
bracketed by device synchronisation. Also reported: microseconds per layer
launched alone, the whole block as a single batched call, the roofline
object of the dominant kernel (the grouped GEMV of the q,k,v and gate,up
calls), the CPU oracle timed on a bounded sample of the same workload, and
the host library's GEMV (aqlm_host_gemv, table lookup on the CPU cores) on the
same seven layers.

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
GEMV_KERNEL = "gemv_2x8_mfma_group_kernel (grouped 2x8 GEMV on the matrix cores, batch 1)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_2x8_llama2_7b_b1_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "additive_codebook_matmul_amd", "csrc", "gemv_mfma.hip")


def _parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--layer-iters", type=int, default=200,
                   help="launches per layer for the per-layer timing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-host-gemv", action="store_true",
                   help="skip timing the host library's GEMV on the CPU cores")
    p.add_argument("--workload", default=WORKLOAD,
                   help="llama2_7b_2x8 (default: the headline step), or per-layer tables for "
                        "single_2x8_512x1024, llama2_7b_1x16, llama2_70b_1x16, gemm_mlp, "
                        "general_schemes, dequant, or the toy encoder's kernels: encode")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run device-to-device copies of MIB MiB (for scaling the HBM "
                        "byte counters of a profiler) and exit")
    return p.parse_args()


def copy_calibration(mib: int) -> None:
    """Plain copies of a known size: the reference for FETCH_SIZE / WRITE_SIZE readings."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 4}), flush=True)


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
    return t.get("bytes_per_launch")


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


def host_gemv_context(layers_np, budget_s: float = 2.0):
    """The host library (aqlm_host_gemv) over the same seven layers at batch 1."""
    from additive_codebook_matmul_amd import host
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    for (_, d, x, _) in layers_np:  # warm the code pages and the thread pool
        host.host_gemv(d.codes, d.codebooks, d.scales, x, threads=threads)
    passes, t0 = 0, time.perf_counter()
    while True:
        for (_, d, x, _) in layers_np:
            host.host_gemv(d.codes, d.codebooks, d.scales, x, threads=threads)
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / passes
    step_bytes = sum(nb for (_, _, _, nb) in layers_np)
    return {
        "value": round(step_bytes / dt / 1e9, 3),
        "unit": "GB/s",
        "us_per_step": round(dt * 1e6, 1),
        "threads": threads,
        "isa": host.host_isa(),
        "kind": "host library aqlm_host_gemv (float32 lookup tables for 8-bit codebooks)",
        "sample": f"{passes} passes over the seven layers, codes in host memory",
    }


def _capture(torch, fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _time_graph(torch, g, reps):
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / reps


def per_layer_tables(args):
    """Per-layer launch times for the other workloads (one JSON line each).

    Every layer is launched back to back over rotated copies of its codes
    (>= 1 GiB) inside a HIP graph; the time per launch is the graph's time over
    the launch count. GEMV and dequant rows report HBM GB/s (codes + x + y, or
    codes + W written); GEMM rows also report fp16 matrix-core TFLOP/s.
    """
    import torch
    from additive_codebook_matmul_amd import AqlmLayer, load_library
    from additive_codebook_matmul_amd import workloads as WL
    load_library()
    dev = torch.device("cuda:0")
    name = args.workload
    wl = WL.WORKLOADS["llama2_7b_2x8" if name == "dequant" else name]
    rows = []
    for layer in wl.layers:
        d = WL.make_layer(layer)
        if layer.packed:
            codes = torch.from_numpy(WL.pack_codes(d.codes, layer.scheme.B).view("int32")).to(dev)
        else:
            codes = torch.from_numpy(d.codes.view("int16") if d.codes.dtype.name == "uint16"
                                     else d.codes).to(dev)
        books = torch.from_numpy(d.codebooks).to(dev)
        scales = torch.from_numpy(d.scales).to(dev)
        kw = {"in_features": layer.in_features} if layer.packed else {}
        batches = (1,) if name == "dequant" else wl.batches
        for batch in batches:
            b = WL.workload_bytes(layer, batch)
            copies = max(2, min(64, -(-ROTATE_BYTES // b["codes"])))
            if batch > 8:
                copies = max(2, min(copies, 8))
            Ls = [AqlmLayer(codes.clone(), books, scales, **kw) for _ in range(copies)]
            x = torch.from_numpy(WL.make_x(layer, batch)).to(dev)
            op = "dequant" if name == "dequant" else ("gemm" if batch > 8 else "gemv")
            if op == "dequant":
                w = torch.empty((layer.out_features, layer.in_features), dtype=torch.float16, device=dev)
                fn = lambda: [L.dequant(out=w) for L in Ls]
                nbytes = b["codes"] + 2 * layer.out_features * layer.in_features
            else:
                y = torch.empty((batch, layer.out_features), dtype=torch.float16, device=dev)
                fn = lambda op=op: [getattr(L, op)(x, out=y) for L in Ls]
                nbytes = b["codes"] + b["x"] + b["y"]
            g = _capture(torch, fn)
            reps = max(2, 200 // copies)
            us = 1e3 * _time_graph(torch, g, reps) / copies
            row = {"layer": layer.name, "out": layer.out_features, "in": layer.in_features,
                   "scheme": layer.scheme.name, "packed_codes": layer.packed, "batch": batch,
                   "us": round(us, 3),
                   "hbm_gbps": round(nbytes / us / 1e3, 1),
                   "pct_hbm_peak": round(100 * nbytes / us / 1e3 / HBM_PEAK_GBPS, 2)}
            if op == "gemm":
                flops = 2 * batch * layer.out_features * layer.in_features
                row["tflops"] = round(flops / us / 1e6, 2)
                row["pct_fp16_mfma_peak"] = round(100 * flops / us / 1e6 / 2500.0, 2)
            rows.append(row)
            print(json.dumps({"workload": name, **row}), flush=True)
            del Ls, g
            torch.cuda.empty_cache()
    return rows


VALU_PEAK_TOPS = 78.6  # fp32 VALU ops/s: 157.3 TFLOP/s counts an FMA as two


def encode_tables(args):
    """Toy encoder kernels on a 4096 x 4096 dense float16 layer (2M group
    vectors of 8): per-launch time of the nearest-codeword search for 256 and
    65536 codewords (bound by VALU issue: 3g float32 operations per vector and
    codeword, against 78.6 T operations/s), of the centroid update, and the
    whole 2x8 encode with ten Lloyd iterations per codebook."""
    import torch
    from additive_codebook_matmul_amd import encode as ENC
    from additive_codebook_matmul_amd import load_library
    from additive_codebook_matmul_amd import workloads as WL
    load_library()
    dev = torch.device("cuda:0")
    out = n_in = 4096
    g = 8
    n = out * n_in // g
    W = torch.from_numpy(WL.make_dense_weight(out, n_in, seed=99)).to(dev)
    scales, vecs = ENC.normalize(W)
    v = vecs.view(n, g)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return 1e3 * t0.elapsed_time(t1) / reps

    rows = []
    for K, reps in ((256, 20), (65536, 2)):
        idx = torch.from_numpy(WL.kmeans_init_indices(n, K, 1, seed=3)[0]).to(dev)
        cents = torch.empty((K, g), dtype=torch.float32, device=dev)
        ENC._check(ENC._lib().aqlm_encode_init(v.data_ptr(), n, g, idx.data_ptr(), K,
                                               cents.data_ptr(), None))
        codes = torch.empty((n, 1), dtype=torch.uint8 if K == 256 else torch.int16, device=dev)
        us = timed(lambda: ENC.assign(v, cents, codes, 1, 0), reps)
        ops = 3 * g * n * K
        rows.append({"kernel": "aqlm_encode_assign", "vectors": n, "g": g, "K": K, "us": round(us, 1),
                     "tops": round(ops / us / 1e6, 2),
                     "pct_valu_peak": round(100 * ops / us / 1e6 / VALU_PEAK_TOPS, 1)})
        ws = torch.empty(K * (g + 1), dtype=torch.int64, device=dev)
        us = timed(lambda: ENC.update(v, codes, 1, 0, cents, ws), reps)
        rows.append({"kernel": "aqlm_encode_update", "vectors": n, "g": g, "K": K, "us": round(us, 1),
                     "gbps": round((n * g * 4 + n * codes.element_size()) / us / 1e3, 1)})
    init = WL.kmeans_init_indices(n, 256, 2, seed=5)
    t0 = time.perf_counter()
    ENC.encode_layer(W, 2, 8, 8, 10, init)
    torch.cuda.synchronize()
    rows.append({"kernel": "encode_layer (2x8, 10 Lloyd iterations per codebook)", "out": out,
                 "in": n_in, "ms": round(1e3 * (time.perf_counter() - t0), 1)})
    for r in rows:
        print(json.dumps({"workload": "encode", **r}), flush=True)
    return rows


def main():
    args = _parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.workload == "encode":
        encode_tables(args)
        return
    if args.workload != WORKLOAD:
        per_layer_tables(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from additive_codebook_matmul_amd import AqlmLayer, gemv_batched, load_library
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
    names = [l.name for (l, _, _, _) in layers_np]
    idx = {n: i for i, n in enumerate(names)}
    rot = []
    for c in range(copies):
        row = []
        for (codes, books, scales, x) in base:
            L = AqlmLayer(codes.clone(), books, scales.clone())
            yy = torch.empty((1, L.out_features), dtype=torch.float16, device=dev)
            row.append((L, x.clone(), yy))
        # q, k, v share one input, as do gate and up
        row[idx["k"]] = (row[idx["k"]][0], row[idx["q"]][1], row[idx["k"]][2])
        row[idx["v"]] = (row[idx["v"]][0], row[idx["q"]][1], row[idx["v"]][2])
        row[idx["up"]] = (row[idx["up"]][0], row[idx["gate"]][1], row[idx["up"]][2])
        rot.append(row)
    torch.cuda.synchronize()

    calls = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gate_up", ["gate", "up"]), ("down", ["down"])]
    call_bytes = {cn: sum(layers_np[idx[n]][3] for n in members) for cn, members in calls}
    for cn, members in calls:  # shared inputs are read once per call
        if len(members) > 1:
            call_bytes[cn] -= (len(members) - 1) * 2 * layers_np[idx[members[0]]][0].in_features

    def issue(i, cn, members):
        row = rot[i % copies]
        if len(members) == 1:
            L, xx, yy = row[idx[members[0]]]
            L.gemv(xx, out=yy)
        else:
            items = [row[idx[m]] for m in members]
            gemv_batched([it[0] for it in items], [it[1] for it in items],
                         [it[2] for it in items])

    def step(i):
        for cn, members in calls:
            issue(i, cn, members)

    def capture(fn):
        """A HIP graph of fn's launches (outputs are preallocated: nothing allocates)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def time_graph(g, reps):
        """Mean milliseconds per replay, HIP events on the replay stream."""
        g.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    # one graph holds one step on each rotated copy; a replay is `copies` steps
    step_graph = capture(lambda: [step(i) for i in range(copies)])
    for _ in range(max(1, args.warmup // copies)):
        step_graph.replay()
    reps = max(1, -(-args.steps // copies))
    torch.cuda.synchronize()
    ms_per_step = time_graph(step_graph, reps) / copies
    steps_timed = reps * copies

    # eager issue of the same step (host launch overhead included), for context
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    eager_ms_per_step = t0.elapsed_time(t1) / args.steps

    # per call and per layer: graphs of back-to-back launches over the copies
    call_us = {}
    for cn, members in calls:
        g = capture(lambda cn=cn, members=members: [issue(i, cn, members) for i in range(copies)])
        call_us[cn] = 1e3 * time_graph(g, max(1, args.layer_iters // copies)) / copies
    us_layer, gbps_layer = {}, {}
    for li, (layer, _, _, nbytes) in enumerate(layers_np):
        def one_layer(li=li):
            for i in range(copies):
                L, xx, yy = rot[i][li]
                L.gemv(xx, out=yy)
        g = capture(one_layer)
        us = 1e3 * time_graph(g, max(1, args.layer_iters // copies)) / copies
        us_layer[layer.name] = round(us, 3)
        gbps_layer[layer.name] = round(nbytes / us / 1e3, 1)

    # the whole block as one batched call (independent inputs)
    def one_call_all():
        for i in range(copies):
            row = rot[i]
            gemv_batched([r[0] for r in row], [r[1] for r in row], [r[2] for r in row])
    g = capture(one_call_all)
    one_call_us = 1e3 * time_graph(g, max(1, args.layer_iters // copies)) / copies

    # dominant kernel: the grouped GEMV of the q,k,v and gate,up calls, launched
    # back to back (one launch per call) inside the timed graph
    def dominant():
        for i in range(copies):
            issue(i, "qkv", ["q", "k", "v"])
            issue(i, "gate_up", ["gate", "up"])
    g = capture(dominant)
    dom_ms = time_graph(g, max(1, args.layer_iters // copies))
    dom_launches = 2 * copies

    step_bytes = sum(call_bytes.values())
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dom_bytes = call_bytes["qkv"] + call_bytes["gate_up"]
    dom_avg_us = 1e3 * dom_ms / dom_launches
    achieved = (dom_bytes / 2) / (dom_avg_us * 1e-6) / 1e9
    traffic = _traffic()
    roofline = {
        "bound": "hbm",
        "kernel": GEMV_KERNEL,
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "bytes_per_launch_avg": dom_bytes // 2,
        "avg_launch_us": round(dom_avg_us, 3),
    }

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps_timed,
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
            "step_calls": {cn: members for cn, members in calls},
            "us_per_call": {k: round(v, 3) for k, v in call_us.items()},
            "us_per_layer": us_layer,
            "gbps_per_layer": gbps_layer,
            "pct_of_peak_per_layer": {k: round(100 * v / HBM_PEAK_GBPS, 1)
                                      for k, v in gbps_layer.items()},
            "accumulate": "fp32",
            "issue": "HIP graph of the step's launches (eager issue in eager_ms_per_step)",
            "eager_ms_per_step": round(eager_ms_per_step, 5),
            "block_as_one_call_us": round(one_call_us, 3),
            "block_as_one_call_gbps": round(sum(nb for (_, _, _, nb) in layers_np) / one_call_us / 1e3, 1),
        },
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers_np)
    if not args.no_host_gemv:
        result["host_gemv"] = host_gemv_context(layers_np)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
