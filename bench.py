"""Benchmark: batch-1 AQLM GEMV over Llama-2-7B-shaped linear layers.

One step is one decode token through the linear layers of Llama-2-7B: 32
transformer blocks of seven layers each (q, k, v, o: 4096x4096; gate, up:
11008x4096; down: 4096x11008), batch 1, seeded synthetic weights. Each block
has its own copy of the codes and scales in HBM (32 distinct buffers of the
seeded block, 1.54 GB of codes per step, far above the 256 MiB last-level
cache), so every step reads its codes from HBM; the codebooks are shared, as
the workload statement puts them in L2. A block issues its layers the way a
decode step can: q, k and v share their input and go out as one
aqlm_gemv_batched call, then o, then gate and up (shared input) as one
batched call, then down. The step is captured once as a HIP graph; the timed
region is exactly --steps replays of it, bracketed by device synchronisation
and timed with HIP events on the replay stream.

Reported value: achieved HBM GB/s of the scheme-2x8 step (two 8-bit
codebooks, codeword length 8) = (codes + x + y bytes of the 224 layers) /
time per step. The same step is measured for scheme 1x16 (one 16-bit
codebook of 1 MiB) under "schemes", with its own roofline object. Also
reported, per scheme: microseconds per layer and per call, the block as one
batched call, and the roofline of the dominant kernel; for context: the
pure-read and random-gather ceilings measured here with the benchmark's own
kernels (libaqlm_ceiling.so), dense float16 torch.nn.functional.linear at the
same shapes, the CPU oracle on a bounded sample (decode and product timed
separately), and the host library's GEMV.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --workload NAME   (per-layer tables of the other workloads)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "AQLM GEMV µs/layer + achieved HBM GB/s (% of peak), Llama-2-7B shapes, batch 1"
WORKLOAD = "llama2_7b_2x8"
HBM_PEAK_GBPS = 8000.0
CLOCK_GHZ = 2.4  # MI355X peak engine clock, for per-clock rates
ROTATE_BYTES = 1 << 30
MODEL_BLOCKS = 32  # transformer blocks of Llama-2-7B
CALLS = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")), ("down", ("down",)))
CSRC = os.path.join(ROOT, "additive_codebook_matmul_amd", "csrc")
CEILING_LIB = os.path.join(ROOT, "additive_codebook_matmul_amd", "libaqlm_ceiling.so")

# Per scheme: the workload, the launches that make up its dominant kernel (a
# call of several layers is one grouped launch where the grouped kernel serves
# it), that kernel's name and source, and the HBM counter summary of it.
SCHEME_SPECS = {
    "2x8": {
        "workload": "llama2_7b_2x8",
        "scheme": "2x8 (M=2, B=8, g=8)",
        "kernel": "gemv_2x8_rows_kernel (2x8 GEMV on the matrix cores, one output row per "
                  "wavefront, batch 1; the grouped q,k,v and gate,up calls)",
        "dominant": (("q", "k", "v"), ("gate", "up")),
        "source": "gemv_mfma.hip",
        "traffic": os.path.join(ROOT, "profiles", "gemv_2x8_llama2_7b_b1_traffic.json"),
    },
    "1x16": {
        "workload": "llama2_7b_1x16",
        "scheme": "1x16 (M=1, B=16, g=8, 1 MiB codebook)",
        "kernel": "gemv_1x16_slice_kernel (codebook split over the LDS of 8 workgroups, batch 1); "
                  "a launch is timed with the launch that adds its member sums",
        "dominant": (("q", "k", "v"), ("gate", "up"), ("down",)),
        "source": "gemv_slice.hip",
        "traffic": os.path.join(ROOT, "profiles", "gemv_1x16_llama2_7b_b1_traffic.json"),
    },
}


def _parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20,
                   help="timed steps (one step: 32 blocks x 7 layers, one token)")
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--layer-iters", type=int, default=200,
                   help="launches per layer (at least two replays of the rotated copies) for "
                        "the per-layer tables of --workload")
    p.add_argument("--schemes", default="2x8,1x16",
                   help="schemes of the headline run; the first one listed gives the "
                        "reported value (default 2x8)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-host-gemv", action="store_true",
                   help="skip timing the host library's GEMV on the CPU cores")
    p.add_argument("--graph-ms", type=float, default=2.0,
                   help="minimum milliseconds of replays behind each per-call and per-layer "
                        "figure (0: two replays, for profiler runs)")
    p.add_argument("--no-context", action="store_true",
                   help="skip the ceilings and the dense float16 comparator")
    p.add_argument("--cold-codebooks", action="store_true",
                   help="also time each scheme's step with a copy of every layer's codebooks "
                        "per block (codebooks read cold, like the codes): a secondary figure")
    p.add_argument("--workload", default=WORKLOAD,
                   help="llama2_7b_2x8 (default: the headline step), or per-layer tables for "
                        "single_2x8_512x1024, llama2_7b_1x16, llama2_70b_1x16, gemm_mlp, "
                        "general_schemes, dequant, or the toy encoder's kernels: encode")
    p.add_argument("--batches", default="",
                   help="comma-separated activation-row counts for a per-layer table in place of "
                        "the workload's own (e.g. 512,1024,2048 for gemm_mlp)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run device-to-device copies of MIB MiB (for scaling the HBM "
                        "byte counters of a profiler) and exit")
    return p.parse_args()


def _source_hash(name: str) -> str:
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(spec):
    """HBM bytes per launch from rocprofv3 counters, if taken on this kernel source."""
    try:
        with open(spec["traffic"]) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != _source_hash(spec["source"]):
        return None
    return t.get("bytes_per_launch")


def _median_time(fn, runs=3):
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts)


CPU_RUNS = 8  # timed runs per layer and oracle step


def cpu_baseline(layers_np):
    """The CPU oracle on the seven layers of one block: O1 decode (numpy,
    float32, single-threaded) and O2 product (float64 BLAS) timed separately
    per layer, median of CPU_RUNS runs each (about 11 s of CPU work in all)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the interpreter's one thread
        blas_threads = 1
    t_dec = t_prod = 0.0
    block_bytes = 0
    t0 = time.perf_counter()
    per_layer = {}
    for (layer, d, x, nbytes) in layers_np:
        w = oracle.decode(d.codes, d.codebooks, d.scales)
        td = _median_time(lambda: oracle.decode(d.codes, d.codebooks, d.scales), CPU_RUNS)
        tp = _median_time(lambda: oracle.product(x, w), CPU_RUNS)
        t_dec += td
        t_prod += tp
        block_bytes += nbytes
        per_layer[layer.name] = {"decode_ms": round(1e3 * td, 1), "product_ms": round(1e3 * tp, 1)}
    wall = time.perf_counter() - t0
    return {
        "value": round(block_bytes / (t_dec + t_prod) / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"one Llama-2-7B block (seven layers, batch 1) of the scheme: O1 decode "
                  f"{1e3 * t_dec:.0f} ms, O2 product {1e3 * t_prod:.0f} ms per block, each the "
                  f"median of {CPU_RUNS} runs per layer ({wall:.1f} s in all); decode is single-threaded "
                  f"numpy, the float64 product uses BLAS with up to {blas_threads} threads",
        "per_layer": per_layer,
    }


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
    if name == "dequant":
        # the 7B layer sets of both schemes and the 1x16 g16 MLP layers
        layers = (WL.WORKLOADS["llama2_7b_2x8"].layers + WL.WORKLOADS["llama2_7b_1x16"].layers
                  + tuple(l for l in WL.WORKLOADS["gemm_mlp"].layers if l.scheme == WL.S1x16g16))
    else:
        layers = WL.WORKLOADS[name].layers
        wl = WL.WORKLOADS[name]
    rows = []
    for layer in layers:
        d = WL.make_layer(layer)
        if layer.packed:
            codes = torch.from_numpy(WL.pack_codes(d.codes, layer.scheme.B).view("int32")).to(dev)
        else:
            codes = torch.from_numpy(d.codes.view("int16") if d.codes.dtype.name == "uint16"
                                     else d.codes).to(dev)
        books = torch.from_numpy(d.codebooks).to(dev)
        scales = torch.from_numpy(d.scales).to(dev)
        kw = {"in_features": layer.in_features} if layer.packed else {}
        batches = (1,) if name == "dequant" else (
            tuple(int(v) for v in args.batches.split(",")) if args.batches else wl.batches)
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
            reps = max(2, args.layer_iters // copies)
            us = 1e3 * _time_graph(torch, g, reps) / copies
            row = {"layer": layer.name, "out": layer.out_features, "in": layer.in_features,
                   "scheme": layer.scheme.name, "packed_codes": layer.packed, "batch": batch,
                   "us": round(us, 3),
                   "hbm_gbps": round(nbytes / us / 1e3, 1),
                   "pct_hbm_peak": round(100 * nbytes / us / 1e3 / HBM_PEAK_GBPS, 2)}
            if op == "dequant" and not args.no_context:
                wbytes = 2 * layer.out_features * layer.in_features
                wc = write_ceiling_us(torch, w, wbytes, copies, reps)
                row["write_ceiling_us"] = round(wc, 3)
                row["write_ceiling_gbps"] = round(wbytes / wc / 1e3, 1)
                row["pct_of_write_ceiling"] = round(100 * wc / us, 1)
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



def _layers_np(wname):
    from additive_codebook_matmul_amd import workloads as WL
    out = []
    for layer in WL.WORKLOADS[wname].layers:
        d = WL.make_layer(layer)
        x = WL.make_x(layer, 1)
        b = WL.workload_bytes(layer, 1)
        out.append((layer, d, x, b["codes"] + b["x"] + b["y"]))
    return out


GRAPH_MS = 2.0  # set from --graph-ms


def _graph_ms(torch, g):
    """Mean milliseconds per replay of graph g over at least GRAPH_MS of replays."""
    one = _time_graph(torch, g, 1)
    reps = max(2, int(GRAPH_MS / max(one, 1e-3)) + 1)
    return _time_graph(torch, g, reps)


def scheme_step(torch, name, args, layers_np):
    """The 32-block decode step of one scheme: timed steps, per-call and
    per-layer times, the block as one call, and the dominant kernel's roofline."""
    from additive_codebook_matmul_amd import AqlmLayer, gemv_batched
    spec = SCHEME_SPECS[name]
    dev = torch.device("cuda:0")
    idx = {l.name: i for i, (l, _, _, _) in enumerate(layers_np)}
    base = [(torch.from_numpy(d.codes.view("int16") if d.codes.dtype.name == "uint16" else d.codes)
             .to(dev), torch.from_numpy(d.codebooks).to(dev), torch.from_numpy(d.scales).to(dev),
             torch.from_numpy(x).to(dev)) for (_, d, x, _) in layers_np]
    def make_blocks(cold_books):
        """MODEL_BLOCKS copies of the block's layers, each with codes, scales, x
        and y of its own; the codebooks are shared (warm, the primary figure)
        or, with cold_books, copied per block as well."""
        out = []
        for _ in range(MODEL_BLOCKS):
            row = {}
            for (layer, _, _, _), (codes, books, scales, x) in zip(layers_np, base):
                L = AqlmLayer(codes.clone(), books.clone() if cold_books else books,
                              scales.clone())
                row[layer.name] = [L, x.clone(), torch.empty((1, L.out_features),
                                                             dtype=torch.float16, device=dev)]
            # q, k and v share one input, as do gate and up
            for a, b in (("k", "q"), ("v", "q"), ("up", "gate")):
                row[a][1] = row[b][1]
            out.append(row)
        torch.cuda.synchronize()
        return out

    blocks = make_blocks(False)
    nbytes = {l.name: nb for (l, _, _, nb) in layers_np}
    in2 = {l.name: 2 * l.in_features for (l, _, _, _) in layers_np}

    def call_bytes(members):  # a shared input is read once per call
        return sum(nbytes[m] for m in members) - (len(members) - 1) * in2[members[0]]

    def issue(row, members):
        if len(members) == 1:
            L, xx, yy = row[members[0]]
            L.gemv(xx, out=yy)
        else:
            gemv_batched([row[m][0] for m in members], [row[m][1] for m in members],
                         [row[m][2] for m in members])

    def step(rows):
        for row in rows:
            for _, members in CALLS:
                issue(row, members)

    step_graph = _capture(torch, lambda: step(blocks))
    for _ in range(args.warmup):
        step_graph.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step_graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    block_bytes = sum(call_bytes(m) for _, m in CALLS)
    step_bytes = MODEL_BLOCKS * block_bytes

    def over_blocks(fn):
        g = _capture(torch, lambda: [fn(row) for row in blocks])
        return 1e3 * _graph_ms(torch, g) / MODEL_BLOCKS

    us_call = {cn: over_blocks(lambda row, m=m: issue(row, m)) for cn, m in CALLS}
    us_layer = {n: over_blocks(lambda row, n=n: issue(row, (n,))) for n in idx}
    one_call_us = over_blocks(lambda row: issue(row, tuple(idx)))
    # the block's layers each in a call of its own: four fewer launches saved
    dom_us = over_blocks(lambda row: [issue(row, m) for m in spec["dominant"]])
    dom_launches = len(spec["dominant"])
    dom_bytes = sum(call_bytes(m) for m in spec["dominant"])
    avg_us = dom_us / dom_launches
    achieved = (dom_bytes / dom_launches) / (avg_us * 1e-6) / 1e9
    layer_gbps = {n: nbytes[n] / us_layer[n] / 1e3 for n in idx}
    one_call_bytes = sum(nbytes.values())
    # secondary, on request: every block with codebooks of its own, cold like
    # its codes
    book_bytes = sum(int(base[i][1].numel()) * 2 for i in range(len(base)))
    cold_ms = None
    if args.cold_codebooks:
        cold = make_blocks(True)
        cold_graph = _capture(torch, lambda: step(cold))
        cold_ms = _graph_ms(torch, cold_graph)
        del cold, cold_graph
        torch.cuda.empty_cache()
    res = {
        "workload": spec["workload"],
        "scheme": spec["scheme"],
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "ms_per_step": round(ms_per_step, 5),
        "pct_hbm_peak": round(100 * step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "bytes_per_step": step_bytes,
        "block_step_us": round(1e3 * ms_per_step / MODEL_BLOCKS, 3),
        "us_per_call": {k: round(v, 3) for k, v in us_call.items()},
        "us_per_layer": {k: round(v, 3) for k, v in us_layer.items()},
        "gbps_per_layer": {k: round(v, 1) for k, v in layer_gbps.items()},
        "pct_of_peak_per_layer": {k: round(100 * v / HBM_PEAK_GBPS, 1) for k, v in layer_gbps.items()},
        "block_as_one_call_us": round(one_call_us, 3),
        "block_as_one_call_gbps": round(one_call_bytes / one_call_us / 1e3, 1),
        "cold_codebooks": None if cold_ms is None else {
            "block_step_us": round(1e3 * cold_ms / MODEL_BLOCKS, 3),
            "gbps": round(step_bytes / (cold_ms * 1e-3) / 1e9, 1),
            "codebook_bytes_per_block": book_bytes,
            "note": "secondary: the same step with a copy of each layer's codebooks per block "
                    "(read cold, like the codes); gbps counts codes + x + y only",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": spec["kernel"],
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": _traffic(spec),
            "bytes_per_launch_avg": dom_bytes // dom_launches,
            "avg_launch_us": round(avg_us, 3),
            "launches_timed": dom_launches * MODEL_BLOCKS,
        },
    }
    del blocks, step_graph
    torch.cuda.empty_cache()
    return res


def _ceiling_lib():
    if not os.path.exists(CEILING_LIB):
        raise RuntimeError(f"{CEILING_LIB} not built (python -m additive_codebook_matmul_amd.build)")
    lib = ctypes.CDLL(CEILING_LIB)
    lib.aqlm_ceiling_blocks.restype = ctypes.c_int
    lib.aqlm_ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    lib.aqlm_ceiling_gather.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.aqlm_ceiling_write.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_void_p]
    lib.aqlm_ceiling_lds_bytes.argtypes = [ctypes.c_int]
    lib.aqlm_ceiling_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
    return lib


# aqlm_ceiling_lds modes: (name, bytes per lane access, what it stands for)
LDS_MODES = (
    ("read_b128_conflict_free", 16, "2x8 GEMV/GEMM A-operand reads from the bank-spread table"),
    ("read_b128_four_addresses", 16, "2x8 GEMV activation fragments at one activation row"),
    ("read_b64_random_128kib", 8, "codebook-sliced 1x16 GEMV lookups"),
    ("read_b128_random_8kib", 16, "2x8 decode from an 8 KiB codebook copy (decoded-tile GEMM fill)"),
    ("write_b128_conflict_free", 16, "tile and table writes"),
)


def lds_rates(torch, iters=1000):
    """LDS access rates of the kernels' patterns (aqlm_ceiling_lds): clocks of
    LDS time per wavefront access and bytes per clock per CU, with the shader
    clock measured inside the kernel (core-clock cycles over the 100 MHz
    real-time counter)."""
    lib = _ceiling_lib()
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = {}
    for mode, (name, width, what) in enumerate(LDS_MODES):
        blocks = cus  # one workgroup of sixteen wavefronts per CU
        sink = torch.zeros(blocks, dtype=torch.int32, device=dev)
        clocks = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(2):  # the first launch warms up; the second is reported
            t0.record()
            if lib.aqlm_ceiling_lds(mode, blocks, iters, sink.data_ptr(), clocks.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream) != 0:
                raise RuntimeError("aqlm_ceiling_lds failed")
            t1.record()
            torch.cuda.synchronize()
        wall_s = t0.elapsed_time(t1) * 1e-3
        c = clocks.view(blocks, 2).cpu().double()
        cyc = float(c[:, 0].median())
        ghz = float((c[:, 0] / (c[:, 1] * 10.0)).median())
        accesses = 16 * 16 * iters  # wavefront accesses per CU
        clk = cyc / accesses
        # the same from the launch's wall time (launch overhead included)
        clk_wall = wall_s * ghz * 1e9 / accesses
        out[name] = {"clk_per_wavefront_access": round(clk, 3),
                     "bytes_per_clk_per_cu": round(64 * width / clk, 1),
                     "lane_accesses_per_clk_per_cu": round(64 / clk, 2),
                     "clk_per_wavefront_access_from_launch_time": round(clk_wall, 3),
                     "wavefronts_per_cu": 16, "shader_clock_ghz": round(ghz, 3),
                     "pattern_of": what}
        del sink, clocks
    return out


def write_ceiling_us(torch, buf, nbytes, copies, reps):
    """Pure-write time of nbytes into buf (16-byte non-temporal stores, the
    dequant kernel's), launched `copies` times back to back in a HIP graph as
    the dequant rows are: the fastest of 1, 2, 4 and 8 stores per thread."""
    lib = _ceiling_lib()
    best = None
    for pt in (1, 2, 4, 8):
        def fn(pt=pt):
            for _ in range(copies):
                if lib.aqlm_ceiling_write(buf.data_ptr(), nbytes, pt,
                                          torch.cuda.current_stream().cuda_stream) != 0:
                    raise RuntimeError("aqlm_ceiling_write failed")
        g = _capture(torch, fn)
        us = 1e3 * _time_graph(torch, g, reps) / copies
        best = us if best is None else min(best, us)
        del g
    return best


def ceilings(torch, sizes):
    """Pure-read ceiling at each byte count (cold: rotated buffers of >= 1 GiB
    in all, one launch per buffer, inside a HIP graph; the fastest of 1..16
    loads per thread), and the random 16-byte gather rate from a 1 MiB table
    (the 1x16 codebook's size)."""
    lib = _ceiling_lib()
    dev = torch.device("cuda:0")
    sink = torch.zeros(max(lib.aqlm_ceiling_blocks(), (1 << 31) // 4096 + 1), dtype=torch.int32,
                       device=dev)
    stream = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731
    out = {}
    for label, nb in sizes.items():
        nb = (nb + 15) // 16 * 16
        copies = max(2, min(256, -(-ROTATE_BYTES // nb)))
        bufs = [torch.full((nb,), 1, dtype=torch.uint8, device=dev) for _ in range(copies)]
        best = None
        for per_thread in (1, 2, 4, 8, 16):
            def reads(bufs=bufs, nb=nb, pt=per_thread):
                for b in bufs:
                    if lib.aqlm_ceiling_read(b.data_ptr(), nb, pt, sink.data_ptr(), stream()) != 0:
                        raise RuntimeError("aqlm_ceiling_read failed")
            g = _capture(torch, reads)
            us = 1e3 * _graph_ms(torch, g) / copies
            if best is None or us < best[0]:
                best = (us, per_thread)
            del g
        us, pt = best
        out[label] = {"bytes": nb, "us": round(us, 3), "gbps": round(nb / us / 1e3, 1),
                      "pct_hbm_peak": round(100 * nb / us / 1e3 / HBM_PEAK_GBPS, 1),
                      "loads_per_thread": pt}
        del bufs
        torch.cuda.empty_cache()
    table = torch.full((1 << 20,), 1, dtype=torch.uint8, device=dev)
    per_lane = 256
    lanes = lib.aqlm_ceiling_blocks() * 256

    def gathers():
        if lib.aqlm_ceiling_gather(table.data_ptr(), 16, per_lane, sink.data_ptr(), stream()) != 0:
            raise RuntimeError("aqlm_ceiling_gather failed")
    g = _capture(torch, gathers)
    us = 1e3 * _graph_ms(torch, g)
    rate = lanes * per_lane / (us * 1e-6)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    return {
        "read": out,
        "lds": lds_rates(torch),
        "kernel": "aqlm_ceiling_read: 16-byte non-temporal loads, each byte once, a block of "
                  "256 threads per 4096 * loads_per_thread bytes",
        "gather_1mib": {"gathers_per_s": round(rate / 1e9, 2), "unit_rate": "G per s",
                        "per_clk_per_cu": round(rate / (cus * CLOCK_GHZ * 1e9), 3),
                        "code_gbps_at_one_gather_per_2_byte_code": round(2 * rate / 1e9, 1),
                        "kernel": "aqlm_ceiling_gather: random 16-byte loads from a 1 MiB table"},
    }


def dense_fp16(torch, layers_np):
    """torch.nn.functional.linear in float16 at the same seven shapes, batch 1,
    on weights 8x the size of the 2-bit codes (rotated copies, >= 1 GiB)."""
    import torch.nn.functional as F
    dev = torch.device("cuda:0")
    wbytes = sum(2 * l.out_features * l.in_features for (l, _, _, _) in layers_np)
    copies = max(2, -(-ROTATE_BYTES // wbytes))
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    ws = [[(torch.randn((l.out_features, l.in_features), generator=gen, device=dev) * 0.02)
           .to(torch.float16) for (l, _, _, _) in layers_np] for _ in range(copies)]
    xs = [torch.from_numpy(x).to(dev) for (_, _, x, _) in layers_np]

    def blockstep():
        for c in range(copies):
            for w, x in zip(ws[c], xs):
                F.linear(x, w)
    g = None
    try:
        g = _capture(torch, blockstep)
        us = 1e3 * _graph_ms(torch, g) / copies
        how = "HIP graph"
    except Exception as e:  # a BLAS path that cannot be captured: time it eagerly
        torch.cuda.synchronize()
        blockstep()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(5):
            blockstep()
        t1.record()
        torch.cuda.synchronize()
        us = 1e3 * t0.elapsed_time(t1) / (5 * copies)
        how = f"eager launches (graph capture failed: {type(e).__name__})"
    xy = sum(2 * (l.in_features + l.out_features) for (l, _, _, _) in layers_np)
    res = {"block_us": round(us, 3), "gbps": round((wbytes + xy) / us / 1e3, 1),
           "pct_hbm_peak": round(100 * (wbytes + xy) / us / 1e3 / HBM_PEAK_GBPS, 1),
           "weight_bytes_per_block": wbytes, "issue": how,
           "op": "torch.nn.functional.linear, float16 weights [out, in], one activation row"}
    del ws, g
    torch.cuda.empty_cache()
    return res


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
    if args.steps < 1:
        print("--steps must be at least 1", file=sys.stderr)
        sys.exit(2)
    global GRAPH_MS
    GRAPH_MS = max(0.0, args.graph_ms)

    import torch

    from additive_codebook_matmul_amd import load_library

    load_library()
    names = [s for s in args.schemes.split(",") if s]
    if not names or any(n not in SCHEME_SPECS for n in names) or len(set(names)) != len(names):
        print(f"--schemes: a comma-separated list of {', '.join(SCHEME_SPECS)}", file=sys.stderr)
        sys.exit(2)
    layers_by_scheme = {n: _layers_np(SCHEME_SPECS[n]["workload"]) for n in names}
    schemes = {}
    for n in names:
        print(f"[bench] scheme {n}: {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr,
              flush=True)
        schemes[n] = scheme_step(torch, n, args, layers_by_scheme[n])
    # the first scheme listed (2x8 by default) gives the reported value
    head = schemes[names[0]]
    layers_np = layers_by_scheme[names[0]]
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": head["workload"],
            "scheme": head["scheme"],
            "batch": 1,
            "blocks_per_step": MODEL_BLOCKS,
            "layers": {l.name: [l.out_features, l.in_features] for (l, _, _, _) in layers_np},
            "bytes_per_step": head["bytes_per_step"],
            "step": "one token through the linear layers of 32 Llama-2-7B blocks (224 launches' "
                    "worth of layers, 128 calls), each block's codes in buffers of their own",
            "step_calls": {cn: list(m) for cn, m in CALLS},
            "block_step_us": head["block_step_us"],
            "us_per_call": head["us_per_call"],
            "us_per_layer": head["us_per_layer"],
            "gbps_per_layer": head["gbps_per_layer"],
            "pct_of_peak_per_layer": head["pct_of_peak_per_layer"],
            "block_as_one_call_us": head["block_as_one_call_us"],
            "block_as_one_call_gbps": head["block_as_one_call_gbps"],
            "accumulate": "fp32",
            "issue": "HIP graph of the step's launches, replayed once per timed step",
        },
        "roofline": head["roofline"],
        "schemes": schemes,
        "rooflines": {n: s["roofline"] for n, s in schemes.items()},
    }
    if not args.no_context:
        print("[bench] ceilings and dense fp16", file=sys.stderr, flush=True)
        sizes = {"layer_4096x4096": layers_np[0][3], "layer_11008x4096": layers_np[4][3],
                 "call_qkv": 3 * layers_np[0][3], "call_gate_up": 2 * layers_np[4][3],
                 "block": sum(nb for (_, _, _, nb) in layers_np),
                 "step_32_blocks": MODEL_BLOCKS * sum(nb for (_, _, _, nb) in layers_np)}
        result["ceiling"] = ceilings(torch, sizes)
        blk = result["ceiling"]["read"]["block"]["us"]
        for n, s in schemes.items():
            s["block_as_one_call_pct_of_read_ceiling"] = round(100 * blk / s["block_as_one_call_us"], 1)
        result["dense_fp16"] = dense_fp16(torch, layers_np)
    if not args.no_cpu_baseline:
        print("[bench] cpu oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(layers_np)
    if not args.no_host_gemv:
        result["host_gemv"] = host_gemv_context(layers_np)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
