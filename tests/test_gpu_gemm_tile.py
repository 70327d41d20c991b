"""GPU parity of the decoded-tile GEMM (gemm_tile.hip) for the 2x8, 1x16 and
1x16 g16 schemes: the binding's gemm without workspace (aqlm_gemm) above 128
activation rows for 1x16 and 1x16 g16, and for 2x8 from 512 rows on layers
whose grid of 128-row x 256-row blocks has at least 160 blocks, i.e. the
calls that run it (with a workspace, the calls whose timing model prefers it
to the workspace form run it too).

Checked against the oracle at the product tolerance and the tighter gate on
sampled activation rows (first, last and seeded others): whole 128-row and
256-row blocks, ragged rows and activation rows, 1, 3 and 5 K blocks (the
tails of the unrolled K loops), rows not a multiple of four
(the unpacked store path), the 11008x4096 MLP shape; one-hot activations
return the decoded columns to within one float16 ulp; repeated calls give
the same bits; nothing past y is written; bit-packed codes give the element
layout's bits; 2x8 codebooks large enough for the float16 codeword sum to
overflow take the halved table.
"""
import numpy as np
import pytest
import torch

import oracle
from additive_codebook_matmul_amd import AqlmLayer, workloads as WL
from gpu_util import assert_product, bits, dev_layer, dev_x, device
from test_gpu_overflow import _large_layer

pytestmark = pytest.mark.gpu

SCHEMES = {"2x8": WL.S2x8, "1x16": WL.S1x16, "1x16g16": WL.S1x16g16}

# (out, in, batch): blocks of 128 rows x 256 activation rows, at least 160
CASES = [(4096, 512, 2048),    # 32 x 8 whole blocks
         (4100, 1024, 1800),   # 33 x 8: a 4-row last row block, an 8-row last token block
         (4098, 512, 2000),    # rows not a multiple of 4: unpacked stores
         (11008, 1024, 600),   # 86 x 3 from 600 rows: an 88-row last token block
         (11008, 4096, 2048)]  # the MLP shape


def _tokens(batch, n=64, seed=1):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, batch - 1], rng.choice(batch, n - 2, replace=False)]))


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("out,n_in,batch", CASES)
def test_tile_gemm_matches_oracle(out, n_in, batch, scheme):
    codes, books, scales, x = WL.small_case(out, n_in, SCHEMES[scheme], batch,
                                            seed=out + n_in + batch)
    L = dev_layer(codes, books, scales)
    toks = _tokens(batch)
    y_ref, bound = oracle.forward(x[toks], codes, books, scales)
    for ws in (True, False):  # without a workspace: the tile kernel
        y = L.gemm(dev_x(x), workspace=ws).cpu().numpy()
        assert_product(y[toks], y_ref, bound, f"tile gemm {scheme} {out}x{n_in} b{batch} ws={ws}")


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("n_in", [64, 192, 320])
def test_tile_gemm_short_k(scheme, n_in):
    """1, 3 and 5 K blocks of 64 inputs: the K loops' tails (the fill loop is
    unrolled by four, the multiply loop by two) and a K loop that is only its
    prologue. 2560 rows x 2048 activation rows: 20 x 8 = 160 blocks."""
    out, batch = 2560, 2048
    codes, books, scales, x = WL.small_case(out, n_in, SCHEMES[scheme], batch, seed=n_in + 7)
    L = dev_layer(codes, books, scales)
    toks = _tokens(batch)
    y_ref, bound = oracle.forward(x[toks], codes, books, scales)
    y = L.gemm(dev_x(x), workspace=False).cpu().numpy()
    assert_product(y[toks], y_ref, bound, f"tile gemm {scheme} {out}x{n_in} b{batch}")


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("out,n_in,batch", [(11008, 256, 511),   # 2x8: wide tiles below 512 rows
                                            (11008, 256, 512),   # decoded tile: 86 x 2 = 172 blocks
                                            (2560, 64, 4096)])   # 20 x 16 blocks, grid y 16
def test_tile_gemm_routing_edges(scheme, out, n_in, batch):
    """Both sides of the 2x8 512-row edge of aqlm_gemm, and 4096 activation
    rows; with and without a workspace."""
    codes, books, scales, x = WL.small_case(out, n_in, SCHEMES[scheme], batch, seed=batch + 3)
    L = dev_layer(codes, books, scales)
    toks = _tokens(batch)
    y_ref, bound = oracle.forward(x[toks], codes, books, scales)
    for ws in (True, False):
        y = L.gemm(dev_x(x), workspace=ws).cpu().numpy()
        assert_product(y[toks], y_ref, bound, f"gemm {scheme} {out}x{n_in} b{batch} ws={ws}")


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_tile_gemm_one_hot(scheme):
    """Activation row i is e_(c_i): row i of y is column c_i of W, to within one
    float16 ulp (the tile multiplies the float16 codeword or codeword sum and
    scales the float32 total; one nonzero product per output)."""
    out, n_in, batch = 4096, 512, 2048
    codes, books, scales, _ = WL.small_case(out, n_in, SCHEMES[scheme], 1, seed=21)
    L = dev_layer(codes, books, scales)
    w_ref = oracle.decode(codes, books, scales).astype(np.float32)
    cols = (np.arange(batch) * 37 + 5) % n_in
    cols[:4] = (0, 7, n_in - 8, n_in - 1)
    x = np.zeros((batch, n_in), dtype=np.float16)
    x[np.arange(batch), cols] = 1
    y = L.gemm(dev_x(x), workspace=False).cpu().numpy().astype(np.float32)
    ref = w_ref[:, cols].T
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float32)
    bad = np.argwhere(np.abs(y - ref) > ulp)
    assert bad.size == 0, bad[:8]


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_tile_gemm_deterministic_and_in_bounds(scheme):
    out, n_in, batch = 4100, 512, 1800
    codes, books, scales, x = WL.small_case(out, n_in, SCHEMES[scheme], batch, seed=33)
    L = dev_layer(codes, books, scales)
    canary = np.float16(-12345.0)
    ybuf = torch.full((batch * out + 64,), float(canary), dtype=torch.float16, device=device())
    y = ybuf[: batch * out].view(batch, out)
    L.gemm(dev_x(x), out=y, workspace=False)
    first = bits(y)
    assert torch.all(ybuf[batch * out:] == float(canary))
    L.gemm(dev_x(x), out=y, workspace=False)
    assert np.array_equal(first, bits(y))


def test_tile_gemm_large_codebooks():
    """Planted (32768, 32768), (65504, 65504) and (65504, -32768) codeword pairs
    at s = 0.25 on every row: finite outputs within the product tolerance."""
    codes, books, scales, x, _ = _large_layer(4096, 512, 2048, seed=9)
    L = dev_layer(codes, books, scales)
    y = L.gemm(dev_x(x), workspace=False).cpu().numpy()
    assert np.isfinite(y.astype(np.float32)).all()
    toks = _tokens(2048)
    y_ref, bound = oracle.forward(x[toks], codes, books, scales)
    assert_product(y[toks], y_ref, bound, "tile gemm, large codebooks")


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_tile_gemm_bit_packed_codes(scheme):
    """The bit-packed flag (8- and 16-bit codes: the stream holds the element
    layout's bytes) takes the same tile kernel and gives the same bits.
    2560 x 128 at 2048 rows: 20 x 8 = 160 blocks."""
    s = SCHEMES[scheme]
    out, n_in, batch = 2560, 128, 2048
    codes, books, scales, x = WL.small_case(out, n_in, s, batch, seed=44)
    plain = dev_layer(codes, books, scales)
    packed = AqlmLayer(torch.from_numpy(WL.pack_codes(codes, s.B).view(np.int32)).to(device()),
                       torch.from_numpy(books).to(device()), torch.from_numpy(scales).to(device()),
                       in_features=n_in)
    xd = dev_x(x)
    assert np.array_equal(bits(packed.gemm(xd, workspace=False)), bits(plain.gemm(xd, workspace=False)))
