"""GPU parity of the toy encoder kernels (include/aqlm_encode.h) with the CPU
oracle of the toy encoder: every kernel bit for bit on seeded inputs (ties,
empty clusters, zero rows, float16 edge values), whole small layers encoded
identically (codes, codebooks, scales), and a Llama-2-7B-sized layer checked on
sampled vectors (its codes are the oracle's nearest codewords for the
codebooks the GPU learned) plus a reconstruction sanity bound."""
import numpy as np
import pytest
import torch

import oracle
from oracle import encoder_oracle as E
from additive_codebook_matmul_amd import encode as ENC
from additive_codebook_matmul_amd import workloads as WL
from gpu_util import dev_layer, device

pytestmark = pytest.mark.gpu


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def _bits16(t):
    return t.detach().cpu().numpy().view(np.uint16)


def test_normalize_bit_exact():
    W = WL.make_dense_weight(37, 200, seed=1)
    W[3] = 0                                   # a zero row: scale 1
    W[5, 7] = np.float16(-0.5)                 # the largest magnitude is negative
    W[6] = np.float16(2.0 ** -20)              # subnormal row
    W[6, 11] = np.float16(-2.0 ** -24)
    scales, vecs = ENC.normalize(_t(W))
    s_ref = E.row_scales(W)
    v_ref = E.normalize(W, s_ref, 8).reshape(37, 200)
    assert np.array_equal(_bits16(scales), s_ref.view(np.uint16))
    assert np.array_equal(vecs.cpu().numpy().view(np.uint32), v_ref.view(np.uint32))


@pytest.mark.parametrize("K,g", [(256, 8), (256, 16), (4096, 8), (65536, 8), (512, 16)])
def test_assign_bit_exact(K, g):
    rng = np.random.default_rng(K + g)
    n = 3000
    vecs = rng.normal(0, 0.3, size=(n, g)).astype(np.float32)
    cents = rng.normal(0, 0.3, size=(K, g)).astype(np.float32)
    cents[7] = cents[3]                        # duplicates: the lower code must win
    vecs[:5] = cents[3]                        # exact hits on the duplicated centroid
    vecs[5:9] = cents[K - 1]
    M, m = 3, 1
    codes = torch.zeros((n, M), dtype=torch.uint8 if K == 256 else torch.int16, device=device())
    res = torch.empty((n, g), dtype=torch.float32, device=device())
    ENC.assign(_t(vecs), _t(cents), codes, M, m, residual=res)
    c_ref, _ = E.assign(vecs, cents)
    got = codes.cpu().numpy().view(np.uint8 if K == 256 else np.uint16).astype(np.int64)
    assert np.array_equal(got[:, m], c_ref)
    assert np.all(got[:, [0, 2]] == 0)         # other codebooks' slots untouched
    r_ref = vecs - cents[c_ref]
    assert np.array_equal(res.cpu().numpy().view(np.uint32), r_ref.view(np.uint32))
    assert got[0, m] == 3 and got[5, m] == K - 1


def test_assign_in_place_residual():
    rng = np.random.default_rng(4)
    vecs = rng.normal(0, 0.3, size=(700, 8)).astype(np.float32)
    cents = rng.normal(0, 0.3, size=(256, 8)).astype(np.float32)
    v = _t(vecs)
    codes = torch.empty((700, 1), dtype=torch.uint8, device=device())
    ENC.assign(v, _t(cents), codes, 1, 0, residual=v)
    c_ref, _ = E.assign(vecs, cents)
    assert np.array_equal(v.cpu().numpy().view(np.uint32), (vecs - cents[c_ref]).view(np.uint32))


@pytest.mark.parametrize("K,g", [(256, 8), (256, 16), (4096, 8), (65536, 16)])
def test_update_bit_exact(K, g):
    rng = np.random.default_rng(K * 3 + g)
    n = 5000
    vecs = rng.uniform(-1, 1, size=(n, g)).astype(np.float32)
    vecs[:10] *= np.float32(2.0 ** -30)        # components below the fixed-point step
    codes = rng.integers(0, min(K, 300), size=n)
    codes[codes == 5] = 6                      # centroid 5 stays empty
    M, m = 2, 1
    packed = np.zeros((n, M), dtype=np.uint8 if K == 256 else np.uint16)
    packed[:, m] = codes
    old = rng.normal(0, 1, size=(K, g)).astype(np.float32)
    cents = _t(old)
    ws = torch.empty(K * (g + 1), dtype=torch.int64, device=device())
    ENC.update(_t(vecs), _t(packed.view(np.int16) if K > 256 else packed), M, m, cents, ws)
    ref = E.update_centroids(vecs, codes, old)
    got = cents.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(got[5], old[5])


def test_round_bit_exact():
    vals = np.array([0.1, -0.3333, 65519.0, 65520.0, 1e-8, -2.0 ** -25, 3 * 2.0 ** -26, 1 + 2.0 ** -11,
                     1 + 3 * 2.0 ** -11, -0.0, 1e6, 2.0 ** -14 - 2.0 ** -26], dtype=np.float32)
    x = np.resize(vals, 64).astype(np.float32)
    books = torch.empty(64, dtype=torch.float16, device=device())
    rounded = torch.empty(64, dtype=torch.float32, device=device())
    lib = ENC._lib()
    src = _t(x)
    assert lib.aqlm_encode_round(src.data_ptr(), 64, books.data_ptr(), rounded.data_ptr(), None) == 0
    torch.cuda.synchronize()
    with np.errstate(over="ignore"):  # 65520 and 1e6 round to infinity on purpose
        want = x.astype(np.float16)
    assert np.array_equal(_bits16(books), want.view(np.uint16))
    assert np.array_equal(rounded.cpu().numpy().view(np.uint32), want.astype(np.float32).view(np.uint32))


SMALL = [(32, 256, 2, 8, 8, 4), (16, 128, 1, 12, 8, 3), (24, 256, 2, 8, 16, 3), (8, 64, 3, 9, 8, 2),
         (4, 64, 1, 16, 8, 2), (40, 96, 2, 10, 16, 2)]


@pytest.mark.parametrize("out,n_in,M,B,g,iters", SMALL)
def test_encode_layer_matches_oracle(out, n_in, M, B, g, iters):
    W = WL.make_dense_weight(out, n_in, seed=out * 31 + n_in)
    init = WL.kmeans_init_indices(out * n_in // g, 2 ** B, M, seed=B * 7 + g)
    codes, books, scales = ENC.encode_layer(_t(W), M, B, g, iters, init)
    c_ref, b_ref, s_ref = E.encode(W, M, B, g, iters, init)
    assert np.array_equal(_bits16(scales), s_ref.view(np.uint16))
    assert np.array_equal(_bits16(books), b_ref.view(np.uint16))
    got = codes.cpu().numpy()
    got = got.view(np.uint16) if B > 8 else got
    assert np.array_equal(got, c_ref)
    # the GPU's own decode of what it encoded reproduces the oracle's decode
    w_gpu = dev_layer(c_ref, b_ref, s_ref).dequant().cpu().numpy()
    assert np.array_equal(w_gpu.view(np.uint16), oracle.decode(c_ref, b_ref, s_ref).view(np.uint16))


def test_encode_llama_sized_layer():
    """4096 x 4096, scheme 2x8, ten Lloyd iterations per codebook: the codes of
    4096 sampled vectors are the oracle's greedy nearest codewords for the
    codebooks the GPU learned, and the layer decodes close to W."""
    out = n_in = 4096
    W = WL.make_dense_weight(out, n_in, seed=99)
    n = out * n_in // 8
    init = WL.kmeans_init_indices(n, 256, 2, seed=5)
    codes, books, scales = ENC.encode_layer(_t(W), 2, 8, 8, 10, init)
    codes_np, books_np, scales_np = codes.cpu().numpy(), books.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(scales_np.view(np.uint16), E.row_scales(W).view(np.uint16))
    rows = np.random.default_rng(0).choice(out, size=8, replace=False)
    r = E.normalize(W[rows], scales_np[rows], 8)
    got = codes_np[rows].reshape(-1, 2).astype(np.int64)
    for m in range(2):
        cb = books_np[m].astype(np.float32)
        c_ref, _ = E.assign(r, cb)
        assert np.array_equal(got[:, m], c_ref)
        r = r - cb[c_ref]
    w_q = dev_layer(codes_np, books_np, scales_np).dequant().cpu().numpy().astype(np.float64)
    rel = np.mean((w_q - W.astype(np.float64)) ** 2) / np.mean(W.astype(np.float64) ** 2)
    assert rel < 0.15, rel
    torch.cuda.empty_cache()
