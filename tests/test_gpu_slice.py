"""GPU parity of the codebook-sliced 1x16 GEMV (aqlm_gemv_ws at one activation row).

The kernel splits the 1 MiB codebook over the LDS of eight workgroups and
adds their partial sums in a second launch; a call runs it when its eligible
1x16 layers hold at least 2^22 codes. It is checked on its own shapes, all
above that: rows not a multiple of anything (8200), rows whose codes end
inside a 1 KiB chunk (11008 and 2112 inputs), two and seven chunks per row
(8192 and 28672 inputs), against the oracle at the product tolerance and the
tighter gate, with one-hot probes, a grouped call of layers that are below
the threshold alone, repeated calls, and calls mixed with other schemes.
"""
import numpy as np
import pytest
import torch

import oracle
from additive_codebook_matmul_amd import _lib, gemv_batched, workloads as WL
from gpu_util import assert_product, bits, dev_layer, dev_x

pytestmark = pytest.mark.gpu

SHAPES = [(8200, 4096), (3100, 11008), (1200, 28672), (16000, 2112), (4200, 8192)]


def _case(out, n_in, seed):
    return WL.small_case(out, n_in, WL.S1x16, 1, seed=seed)


@pytest.mark.parametrize("out,n_in", SHAPES)
def test_sliced_gemv_matches_oracle(out, n_in):
    codes, books, scales, x = _case(out, n_in, seed=out + n_in)
    L = dev_layer(codes, books, scales)
    assert _lib.gemv_workspace_bytes([L], 1) == (8 * out * 4 + 255) // 256 * 256
    y = L.gemv(dev_x(x))
    y_ref, bound = oracle.forward(x, codes, books, scales)
    assert_product(y, y_ref, bound, f"sliced gemv {out}x{n_in}")
    # the workspace-free kernel agrees to the same tolerance
    assert_product(L.gemv(dev_x(x), workspace=False), y_ref, bound, f"gather gemv {out}x{n_in}")
    # repeated calls give the same bits
    assert np.array_equal(bits(y), bits(L.gemv(dev_x(x))))


@pytest.mark.parametrize("out,n_in", SHAPES[:3])
def test_sliced_gemv_one_hot(out, n_in):
    """x = e_i returns column i of W exactly (a half-codeword dotted with a
    one-hot half of x, summed with zeros, times the scale, rounded once)."""
    codes, books, scales, _ = _case(out, n_in, seed=7 * out)
    L = dev_layer(codes, books, scales)
    w = oracle.decode(codes, books, scales).astype(np.float32)
    rng = np.random.default_rng(out)
    cols = np.unique(np.concatenate([[0, 7, 8, n_in // 2, n_in - 8, n_in - 1],
                                     rng.choice(n_in, 26, replace=False)]))
    for c in cols:
        x = np.zeros((1, n_in), dtype=np.float16)
        x[0, c] = 1
        y = L.gemv(dev_x(x)).cpu().numpy().astype(np.float32)[0]
        assert np.array_equal(y, w[:, c]), (out, n_in, int(c))


def test_sliced_gemv_grouped_call():
    """Layers too small to take the sliced kernel alone (4.9 M codes together)
    and a 2x8 layer in one call: the 1x16 outputs meet the oracle's tolerance
    and repeat bit for bit; the 2x8 layer's bits equal aqlm_gemv_batched
    without a workspace."""
    cases = [(_case(2100, 8192, 1)), (_case(1600, 11008, 2)), (_case(1025, 4096, 3))]
    Ls = [dev_layer(c, b, s) for (c, b, s, _) in cases]
    xs = [dev_x(x) for (_, _, _, x) in cases]
    for L in Ls:
        assert _lib.gemv_workspace_bytes([L], 1) == 0
    assert _lib.gemv_workspace_bytes(Ls, 1) > 0
    c8, b8, s8, x8 = WL.small_case(4096, 4096, WL.S2x8, 1, seed=4)
    L8 = dev_layer(c8, b8, s8)
    ys = gemv_batched(Ls + [L8], xs + [dev_x(x8)])
    again = gemv_batched(Ls + [L8], xs + [dev_x(x8)])
    for y, y2 in zip(ys, again):
        assert np.array_equal(bits(y), bits(y2))
    assert np.array_equal(bits(ys[-1]), bits(gemv_batched([L8], [dev_x(x8)], workspace=False)[0]))
    for (c, b, s, x), y in zip(cases, ys):
        y_ref, bound = oracle.forward(x, c, b, s)
        assert_product(y, y_ref, bound, "grouped sliced gemv")


def test_sliced_gemv_in_a_graph():
    """Captured in a HIP graph (workspace from the graph's pool), replayed with
    new activations: every replay matches the eager result for its input."""
    codes, books, scales, _ = _case(8200, 4096, seed=11)
    L = dev_layer(codes, books, scales)
    assert _lib.gemv_workspace_bytes([L], 1) > 0
    xs = [dev_x(WL.make_x_only(1, 4096, seed=s)) for s in range(3)]
    xin = xs[0].clone()
    yout = torch.empty((1, 8200), dtype=torch.float16, device=xin.device)
    eager = [bits(L.gemv(x)) for x in xs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        L.gemv(xin, out=yout)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.gemv(xin, out=yout)
    for k in (0, 1, 2, 1):
        xin.copy_(xs[k])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(yout), eager[k]), k
