"""The entry points captured into a HIP graph (torch.cuda.CUDAGraph, as the
benchmark times them) give on every replay exactly the bits of the same calls
issued eagerly: GEMV (single and grouped), the GEMM with and without its
workspace (split-K included, the workspace coming from the graph's memory
pool; the one-tile form reading x in place, through the GEMV and the GEMM;
the decoded-tile kernel at 2048 rows, for 2x8 and 1x16 g16), and dequant. Eager work runs between the replays, and every replay is
checked. Nothing here clears memory with a memset node: the kernels write
every output element and the workspace form rewrites its workspace each call.
"""
import numpy as np
import pytest
import torch

from additive_codebook_matmul_amd import _lib, workloads as WL
from gpu_util import bits, dev_layer, dev_x, device

pytestmark = pytest.mark.gpu


def _calls():
    s2, s16 = WL.S2x8, WL.S1x16g16
    c, b, sc, x = WL.small_case(1000, 8192, s2, 40, seed=3)        # split-K at 40 rows
    big = dev_layer(c, b, sc)
    c2, b2, sc2, x2 = WL.small_case(300, 2048, s16, 40, seed=4)
    small = dev_layer(c2, b2, sc2)
    c3, b3, sc3, _ = WL.small_case(512, 2048, s2, 1, seed=5)
    third = dev_layer(c3, b3, sc3)
    c5, b5, sc5, x5 = WL.small_case(7000, 2048, WL.S1x16g16, 16, seed=6)
    in_place = dev_layer(c5, b5, sc5)                              # one tile, x read in place
    # the decoded-tile kernel: 20 x 8 = 160 blocks of 128 rows x 256 activation rows
    c6, b6, sc6, x6 = WL.small_case(2560, 128, s2, 2048, seed=7)
    tile_2x8 = dev_layer(c6, b6, sc6)
    c7, b7, sc7, _ = WL.small_case(2560, 128, s16, 1, seed=8)
    tile_g16 = dev_layer(c7, b7, sc7)
    xt = dev_x(x6)
    xb, xs, x16 = dev_x(x), dev_x(x2), dev_x(x5)
    x4 = dev_x(x2[:4])
    assert in_place.workspace_bytes(16) == 0
    assert big.workspace_bytes(40) > 8192 * 48 * 2 + 512   # the split form is exercised
    outs = {
        "gemv": torch.empty((4, 300), dtype=torch.float16, device=device()),
        "gemv_batched_a": torch.empty((4, 300), dtype=torch.float16, device=device()),
        "gemv_batched_b": torch.empty((4, 512), dtype=torch.float16, device=device()),
        "gemm_ws_big": torch.empty((40, 1000), dtype=torch.float16, device=device()),
        "gemm_ws_small": torch.empty((40, 300), dtype=torch.float16, device=device()),
        "gemm_plain": torch.empty((40, 1000), dtype=torch.float16, device=device()),
        "dequant": torch.empty((300, 2048), dtype=torch.float16, device=device()),
        "gemv_in_place": torch.empty((4, 7000), dtype=torch.float16, device=device()),
        "gemm_in_place": torch.empty((16, 7000), dtype=torch.float16, device=device()),
        "gemm_tile_2x8": torch.empty((2048, 2560), dtype=torch.float16, device=device()),
        "gemm_tile_g16": torch.empty((2048, 2560), dtype=torch.float16, device=device()),
    }

    def run():
        small.gemv(x4, out=outs["gemv"])
        _lib.gemv_batched([small, third], [x4, x4], [outs["gemv_batched_a"], outs["gemv_batched_b"]])
        big.gemm(xb, out=outs["gemm_ws_big"])
        small.gemm(xs, out=outs["gemm_ws_small"])
        big.gemm(xb, out=outs["gemm_plain"], workspace=False)
        small.dequant(out=outs["dequant"])
        in_place.gemv(x16[:4], out=outs["gemv_in_place"])
        in_place.gemm(x16, out=outs["gemm_in_place"])
        tile_2x8.gemm(xt, out=outs["gemm_tile_2x8"])
        tile_g16.gemm(xt, out=outs["gemm_tile_g16"], workspace=False)

    return run, outs, big, xb


def test_graph_replays_match_eager():
    run, outs, big, xb = _calls()
    run()
    torch.cuda.synchronize()
    eager = {k: bits(v) for k, v in outs.items()}
    for v in outs.values():
        v.fill_(0.0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    scratch = torch.empty((40, 1000), dtype=torch.float16, device=device())
    for rep in range(4):
        for v in outs.values():
            v.fill_(-1.0)                      # every replay must rewrite every element
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert np.array_equal(bits(v), eager[k]), f"replay {rep}: {k}"
        big.gemm(xb, out=scratch)              # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(bits(scratch), eager["gemm_ws_big"])
    del g
    torch.cuda.empty_cache()
