"""GPU: aqlm_gemv_batched equals aqlm_gemv layer by layer (bit for bit) and the oracle."""
import numpy as np
import pytest
import torch

import oracle
from additive_codebook_matmul_amd import gemv_batched, workloads as WL
from gpu_util import assert_product, bits, dev_layer, dev_x

pytestmark = pytest.mark.gpu


def _layers(wname):
    wl = WL.WORKLOADS[wname]
    out = []
    for layer in wl.layers:
        d = WL.make_layer(layer)
        out.append((layer, d, dev_layer(d.codes, d.codebooks, d.scales)))
    return out


@pytest.mark.parametrize("batch", [1, 2])
def test_batched_matches_single_launches_llama2_7b(batch):
    layers = _layers("llama2_7b_2x8")
    xs = [dev_x(WL.make_x(l, batch)) for (l, _, _) in layers]
    ys = gemv_batched([L for (_, _, L) in layers], xs, workspace=False)
    for (layer, d, L), x, y in zip(layers, xs, ys):
        y1 = L.gemv(x, workspace=False)
        assert np.array_equal(bits(y), bits(y1)), layer.name
    # and against the oracle on two of them
    for i in (0, 6):
        layer, d, L = layers[i]
        xn = WL.make_x(layer, batch)
        y_ref, bound = oracle.forward(xn, d.codes, d.codebooks, d.scales)
        assert_product(ys[i], y_ref, bound, f"batched {layer.name}")


def test_batched_1x16_llama2_7b_both_entry_points():
    """The 1x16 layer set at one row: aqlm_gemv_batched equals aqlm_gemv bit
    for bit (no workspace: the gather kernel); the workspace call (the q,k,v
    and gate,up calls are large enough for the codebook-sliced kernel) meets
    the oracle on every layer."""
    layers = _layers("llama2_7b_1x16")
    xs = [dev_x(WL.make_x(l, 1)) for (l, _, _) in layers]
    Ls = [L for (_, _, L) in layers]
    ys = gemv_batched(Ls, xs, workspace=False)
    for (layer, d, L), x, y in zip(layers, xs, ys):
        assert np.array_equal(bits(y), bits(L.gemv(x, workspace=False))), layer.name
    for names in (("q", "k", "v"), ("gate", "up")):
        idx = [i for i, (l, _, _) in enumerate(layers) if l.name in names]
        yw = gemv_batched([Ls[i] for i in idx], [xs[i] for i in idx])
        for i, y in zip(idx, yw):
            layer, d, _ = layers[i]
            y_ref, bound = oracle.forward(WL.make_x(layer, 1), d.codes, d.codebooks, d.scales)
            assert_product(y, y_ref, bound, f"workspace call {layer.name}")


def test_batched_shared_x_and_mixed_schemes():
    """q/k/v-style groups share one x; a 1x16 layer in the list takes its own launch."""
    rng_layers = []
    for i, (out, n_in, s) in enumerate([(300, 1024, WL.S2x8), (512, 1024, WL.S2x8),
                                        (96, 1024, WL.S1x16), (257, 1024, WL.S2x8),
                                        (64, 8 * 13, WL.S2x8)]):
        codes, books, scales, _ = WL.small_case(out, n_in, s, 1, seed=40 + i)
        rng_layers.append((codes, books, scales, dev_layer(codes, books, scales)))
    x_shared = WL.make_x_only(2, 1024, seed=9)
    x_odd = WL.make_x_only(2, 8 * 13, seed=10)
    xs = [dev_x(x_shared)] * 4 + [dev_x(x_odd)]
    ys = gemv_batched([L for (*_, L) in rng_layers], xs)
    for (codes, books, scales, L), x, y in zip(rng_layers, [x_shared] * 4 + [x_odd], ys):
        y_ref, bound = oracle.forward(x, codes, books, scales)
        assert_product(y, y_ref, bound, "batched mixed")
        assert np.array_equal(bits(y), bits(L.gemv(dev_x(x))))


@pytest.mark.parametrize("batch", [3, 5, 8])
def test_batched_mixed_routes_bit_identical(batch):
    """Layers that take the four GEMV routes (the matrix-core 2x8 GEMV, 2x8 rows
    too long for it on the GEMM tiles from three rows, 1x16 g16 on the GEMM
    tiles, short 1x16 rows on the lookup GEMV) in one grouped call: every
    output equals its single-layer aqlm_gemv bit for bit and the oracle."""
    specs = [(256, 4096, WL.S2x8), (200, 11008, WL.S2x8), (160, 2048, WL.S1x16g16),
             (96, 1024, WL.S1x16)]
    items = []
    for i, (out, n_in, s) in enumerate(specs):
        codes, books, scales, x = WL.small_case(out, n_in, s, batch, seed=70 + i)
        items.append((codes, books, scales, x, dev_layer(codes, books, scales)))
    ys = gemv_batched([it[4] for it in items], [dev_x(it[3]) for it in items])
    for (codes, books, scales, x, L), y in zip(items, ys):
        assert np.array_equal(bits(y), bits(L.gemv(dev_x(x)))), L.out_features
        y_ref, bound = oracle.forward(x, codes, books, scales)
        assert_product(y, y_ref, bound, f"batched mixed routes b{batch}")


def test_batched_many_layers_splits_launches():
    """More layers than one grouped launch holds."""
    items = []
    for i in range(20):
        codes, books, scales, x = WL.small_case(64 + 8 * i, 512, WL.S2x8, 1, seed=100 + i)
        items.append((codes, books, scales, x, dev_layer(codes, books, scales)))
    ys = gemv_batched([it[4] for it in items], [dev_x(it[3]) for it in items])
    for (codes, books, scales, x, L), y in zip(items, ys):
        y_ref, bound = oracle.forward(x, codes, books, scales)
        assert_product(y, y_ref, bound, "batched x20")
