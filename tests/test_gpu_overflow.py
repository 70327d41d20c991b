"""2x8 layers with codewords so large that the float16 sum of a group's two
codewords overflows while the decoded weights s * (C_0 + C_1) stay finite.

The decode rule sums the codewords in float32 and applies the row scale before
the one round to float16, so C_0 = C_1 = 32768 with s = 0.25 decodes to 16384
and C_0 = C_1 = 65504 with s = 0.25 to 32752. The matrix-core tiles add the two
codewords in float16 before the scale; for such codebooks they must halve the
table and double the totals (exact for normal values) instead of producing
infinities. Every product entry point and each of its kernels is driven here:
the GEMV tile (1 and 8 rows, single and grouped calls), the skinny GEMM tile
(16 and 128 rows), the wide GEMM tile (300 rows), and the workspace form (one
activation tile read in place at 16 rows, re-laid activations at 128 rows,
K split across workgroups at 40 rows).
"""
import numpy as np
import pytest
import oracle
from additive_codebook_matmul_amd import gemv_batched, workloads as WL
from gpu_util import assert_product, bits, dev_layer, dev_x

pytestmark = pytest.mark.gpu

BIG = np.float16(32768.0)   # 0x7800, the smallest half that triggers the guard
TOP = np.float16(65504.0)   # 0x7BFF, the largest finite half


def _large_layer(out, n_in, batch, seed):
    """A seeded 2x8 layer whose every row holds three planted groups: (C_0[7],
    C_1[9]) = (32768, 32768), (C_0[200], C_1[201]) = (65504, 65504) and
    (C_0[50], C_1[60]) = (65504, -32768); scales 0.25, activations / 64 so
    that the products stay inside float16. Codebook values below 2^-13 in
    magnitude are zeroed, so halving the table is exact everywhere and the
    one-hot probes can ask for the decoded column to within one ulp."""
    codes, books, scales, x = WL.small_case(out, n_in, WL.S2x8, batch, seed=seed)
    books = books.copy()
    books[np.abs(books.astype(np.float32)) < 2.0 ** -13] = 0
    books[0, 7], books[1, 9] = BIG, BIG
    books[0, 200], books[1, 201] = TOP, TOP
    books[0, 50], books[1, 60] = TOP, -BIG
    codes = codes.copy()
    J = n_in // 8
    o = np.arange(out)
    j1 = (o * 7) % J
    j2 = (j1 + 1 + (o % (J - 2))) % J
    j3 = (j1 + J // 2) % J
    j3 = np.where((j3 == j2), (j3 + 1) % J, j3)
    j3 = np.where((j3 == j1), (j3 + 1) % J, j3)
    codes[o, j1] = (7, 9)
    codes[o, j2] = (200, 201)
    codes[o, j3] = (50, 60)
    scales = np.full(out, 0.25, dtype=np.float16)
    x = (x.astype(np.float32) / 64).astype(np.float16)
    w = oracle.decode(codes, books, scales)
    assert np.isfinite(w.astype(np.float32)).all()
    assert (np.abs(w.astype(np.float32)) == 32752).any()
    return codes, books, scales, x, w


def _check(y, x, codes, books, scales, what):
    y = y.cpu().numpy()
    assert np.isfinite(y.astype(np.float32)).all(), f"{what}: non-finite outputs"
    y_ref, bound = oracle.forward(x, codes, books, scales)
    assert_product(y, y_ref, bound, what)


@pytest.mark.parametrize("batch", [1, 8])
def test_large_codebooks_gemv(batch):
    codes, books, scales, x, _ = _large_layer(300, 1024, batch, seed=1)
    L = dev_layer(codes, books, scales)
    _check(L.gemv(dev_x(x)), x, codes, books, scales, f"gemv b{batch}")
    # grouped call: bit-identical to the single calls
    c2, b2, s2, x2, _ = _large_layer(300, 1024, batch, seed=2)
    L2 = dev_layer(c2, b2, s2)
    ys = gemv_batched([L, L2], [dev_x(x), dev_x(x2)])
    assert np.array_equal(bits(ys[0]), bits(L.gemv(dev_x(x))))
    assert np.array_equal(bits(ys[1]), bits(L2.gemv(dev_x(x2))))
    _check(ys[1], x2, c2, b2, s2, f"gemv_batched b{batch}")


@pytest.mark.parametrize("out,n_in,batch,ws", [
    (300, 1024, 16, False), (300, 1024, 128, False), (300, 1024, 300, False),  # skinny, wide
    (7000, 2112, 16, True),    # workspace form, one activation tile read in place
    (300, 1024, 128, True),    # workspace form, re-laid activations
    (100, 16384, 40, True),    # workspace form, K split across workgroups
])
def test_large_codebooks_gemm(out, n_in, batch, ws):
    codes, books, scales, x, _ = _large_layer(out, n_in, batch, seed=out + batch)
    L = dev_layer(codes, books, scales)
    if ws and (out, batch) != (7000, 16):
        assert L.workspace_bytes(batch) > 0
    _check(L.gemm(dev_x(x), workspace=ws), x, codes, books, scales,
           f"gemm {out}x{n_in} b{batch} ws={ws}")


@pytest.mark.parametrize("out,n_in,rows,ws", [(300, 1024, 8, False), (300, 1024, 16, False),
                                              (300, 1024, 300, False), (7000, 2112, 16, True),
                                              (300, 1024, 128, True)])
def test_large_codebooks_one_hot(out, n_in, rows, ws):
    """x = e_i returns column i of W to within one float16 ulp, also where the
    planted groups make it 16384 or 32752."""
    codes, books, scales, _, w = _large_layer(out, n_in, 1, seed=3)
    L = dev_layer(codes, books, scales)
    J = n_in // 8
    j1 = 0
    j2 = 1 % J
    cols = np.unique(np.array([8 * j1, 8 * j1 + 7, 8 * j2 + 3, 8 * (J // 2) + 5, n_in - 1,
                               8 * 7 + 2, 8 * 14 + 6, 8 * (J // 2 + 1)]))
    x = np.zeros((rows, n_in), dtype=np.float16)
    x[np.arange(len(cols)), cols] = 1
    fn = L.gemv if rows <= 8 else (lambda v: L.gemm(v, workspace=ws))
    yfull = fn(dev_x(x)).cpu().numpy().astype(np.float32)
    y = yfull[: len(cols)]
    ref = w.astype(np.float32)[:, cols].T
    assert np.abs(ref).max() >= 16384
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float32)
    assert np.all(np.abs(y - ref) <= ulp), (out, n_in, rows, ws)
    assert np.all(yfull[len(cols):] == 0)  # the all-zero activation rows


def test_codebooks_just_below_the_guard():
    """Largest half 32752 (0x77FF): the plain float16 sum reaches 65504 and
    stays finite, so the table is used as staged."""
    codes, books, scales, x = WL.small_case(300, 1024, WL.S2x8, 8, seed=9)
    books = books.copy()
    books[0, 3], books[1, 4] = np.float16(32752.0), np.float16(32752.0)
    codes = codes.copy()
    codes[:, 5] = (3, 4)
    scales = np.full(300, 0.125, dtype=np.float16)
    x = (x.astype(np.float32) / 256).astype(np.float16)
    L = dev_layer(codes, books, scales)
    for y, what in ((L.gemv(dev_x(x)), "gemv b8"), (L.gemm(dev_x(x[:1]).repeat(16, 1)), "gemm b16")):
        xx = x if what == "gemv b8" else np.repeat(x[:1], 16, axis=0)
        _check(y, xx, codes, books, scales, what)
