"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Decoded weights (aqlm_dequant) must match bit for bit; products (aqlm_gemv,
aqlm_gemm) must lie within 1e-2 * sum_i |x_i w_i| of the float64 oracle for
every output, and within the tighter 1e-3 gate. Sizes: small ragged layers
that span several tiles and a tail, and every layer of the five workloads at
full size on every row (the 70B-shaped layers in chunks of 2048 rows, the
2048-row products on sampled activation rows). One-hot probes (64 columns per
workload layer, group edges and row tails included) check single columns of W
to within one float16 ulp, which the loose tolerance cannot.
"""
import functools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from additive_codebook_matmul_amd import AqlmLayer, _lib, workloads as WL
from gpu_util import (assert_bit_exact, assert_product, bits, dev_layer, dev_x, device,
                      to_dev_codes)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCHEMES = {"2x8": WL.S2x8, "1x16": WL.S1x16, "1x16g16": WL.S1x16g16}

# (out, groups): single row/group, ragged rows and groups, multiples of the
# 16-byte code chunk (8 groups) with and without row tails, several tiles, and
# whole 256-input chunks (the mid-batch GEMM) with ragged rows.
SMALL_SHAPES = [(1, 1), (7, 5), (64, 8), (255, 13), (300, 64), (33, 172), (513, 24), (257, 9),
                (70, 200), (77, 96), (1000, 32), (90, 48)]


def _small(scheme, out, J, batch, seed):
    return WL.small_case(out, J * scheme.g, scheme, batch, seed)


@pytest.fixture(scope="module", autouse=True)
def _announce():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield


# ---------------------------------------------------------------------------
# small, ragged
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("sname", list(SCHEMES))
@pytest.mark.parametrize("out,J", SMALL_SHAPES)
def test_small_dequant_bit_exact(sname, out, J):
    s = SCHEMES[sname]
    codes, books, scales, _ = _small(s, out, J, 1, seed=out * 131 + J)
    w = dev_layer(codes, books, scales).dequant()
    assert_bit_exact(w.cpu().numpy(), oracle.decode(codes, books, scales), f"{sname} {out}x{J}")


@pytest.mark.parametrize("sname", list(SCHEMES))
@pytest.mark.parametrize("out,J", SMALL_SHAPES)
def test_small_gemv(sname, out, J):
    s = SCHEMES[sname]
    codes, books, scales, x = _small(s, out, J, 8, seed=out * 17 + J)
    layer = dev_layer(codes, books, scales)
    for batch in range(1, 9):
        y = layer.gemv(dev_x(x[:batch]))
        y_ref, bound = oracle.forward(x[:batch], codes, books, scales)
        assert_product(y, y_ref, bound, f"gemv {sname} {out}x{J} b{batch}")


@pytest.mark.parametrize("sname", list(SCHEMES))
@pytest.mark.parametrize("out,J", SMALL_SHAPES)
def test_small_gemm(sname, out, J):
    s = SCHEMES[sname]
    codes, books, scales, x = _small(s, out, J, 130, seed=out * 23 + J)
    layer = dev_layer(codes, books, scales)
    for batch in (1, 5, 16, 17, 32, 33, 64, 65, 100, 128, 130):
        y_ref, bound = oracle.forward(x[:batch], codes, books, scales)
        for ws in (True, False):
            y = layer.gemm(dev_x(x[:batch]), workspace=ws)
            assert_product(y, y_ref, bound, f"gemm {sname} {out}x{J} b{batch} ws={ws}")


# ---------------------------------------------------------------------------
# golden values on the GPU
# ---------------------------------------------------------------------------
def _golden_cases():
    with open(os.path.join(GOLDEN, "hand_worked_groups.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_hand_worked(case):
    M, B, g = case["M"], case["B"], case["g"]
    books = np.zeros((M, 2 ** B, g), dtype=np.float16)
    for m, rows in case["codebook_rows"].items():
        for c, vals in rows.items():
            books[int(m), int(c)] = np.asarray(vals, dtype=np.float16)
    codes = np.asarray(case["codes"], dtype=np.uint8 if B == 8 else np.uint16)
    scales = np.asarray(case["scales"], dtype=np.float16)
    x = np.asarray(case["x"], dtype=np.float16)
    layer = dev_layer(codes, books, scales)
    w = layer.dequant().cpu().numpy()
    if "expected_w_bits" in case:
        exp = np.array([[int(h, 16) for h in r] for r in case["expected_w_bits"]], dtype=np.uint16)
    else:
        exp = bits(np.asarray(case["expected_w"], dtype=np.float16))
    assert np.array_equal(bits(w), exp)
    expected_y = np.asarray(case["expected_y"], dtype=np.float64)
    for fn in (layer.gemv, layer.gemm):
        y = fn(dev_x(x)).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, expected_y), (fn.__name__, y, expected_y)


def _rounding_cases():
    with open(os.path.join(GOLDEN, "rounding_cases.json")) as f:
        return [c for c in json.load(f)["cases"] if len(c["codewords"]) in (1, 2)]


@pytest.mark.parametrize("case", _rounding_cases(), ids=lambda c: c["name"])
def test_golden_rounding_dequant(case):
    """The golden single-weight decodes, placed in a real 2x8 or 1x16 layer."""
    cw = [int(h, 16) for h in case["codewords"]]
    if len(cw) == 2:
        books = np.zeros((2, 256, 8), dtype=np.uint16)
        books[0, 7, 3], books[1, 9, 3] = cw
        codes = np.array([[[7, 9]]], dtype=np.uint8)
    else:
        books = np.zeros((1, 65536, 8), dtype=np.uint16)
        books[0, 40000, 3] = cw[0]
        codes = np.array([[[40000]]], dtype=np.uint16)
    scales = np.array([int(case["scale"], 16)], dtype=np.uint16).view(np.float16)
    w = dev_layer(codes, books.view(np.float16), scales).dequant()
    assert int(bits(w)[0, 3]) == int(case["expected"], 16), case["name"]


# ---------------------------------------------------------------------------
# the workloads at full size
# ---------------------------------------------------------------------------
@functools.lru_cache(maxsize=4)
def _layer_data(wname, lname):
    wl = WL.WORKLOADS[wname]
    layer = next(l for l in wl.layers if l.name == lname)
    return layer, WL.make_layer(layer)


def _sample_rows(out, n=1024, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, out - 2, out - 1],
                                     rng.choice(out, size=min(out, n), replace=False)]))
    return rows[(rows >= 0) & (rows < out)]


BIG = "llama2_70b_1x16"  # layers of up to 235 M weights: checked in row chunks below
LAYER_IDS = [(w.name, l.name) for w in WL.WORKLOADS.values() for l in w.layers if w.name != BIG]


@pytest.mark.parametrize("wname,lname", LAYER_IDS, ids=lambda v: str(v))
def test_workload_dequant_bit_exact(wname, lname):
    layer, d = _layer_data(wname, lname)
    gl = dev_layer(d.codes, d.codebooks, d.scales)
    w = gl.dequant()
    assert_bit_exact(w.cpu().numpy(), oracle.decode(d.codes, d.codebooks, d.scales),
                     f"{wname}/{lname}")
    del w
    torch.cuda.empty_cache()


GEMV_IDS = [(w.name, l.name, b) for w in WL.WORKLOADS.values() if w.index <= 4 and w.name != BIG
            for l in w.layers for b in w.batches]


@pytest.mark.parametrize("wname,lname,batch", GEMV_IDS, ids=lambda v: str(v))
def test_workload_gemv(wname, lname, batch):
    layer, d = _layer_data(wname, lname)
    x = WL.make_x(layer, batch)
    y = dev_layer(d.codes, d.codebooks, d.scales).gemv(dev_x(x)).cpu().numpy()
    y_ref, bound = oracle.forward(x, d.codes, d.codebooks, d.scales)
    assert_product(y, y_ref, bound, f"{wname}/{lname} b{batch}")


def _probe_columns(n_in, g, n=64, seed=0):
    """n input columns for one-hot probes: the first and last column of the
    first, second and middle groups, the row tail (the last group whole), and
    seeded random columns for the rest."""
    J = n_in // g
    fixed = [0, g - 1, g, 2 * g - 1, (J // 2) * g, (J // 2) * g + g - 1]
    fixed += list(range(n_in - g, n_in))
    fixed = sorted(set(c for c in fixed if 0 <= c < n_in))
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(n_in), fixed)
    extra = rng.choice(rest, size=max(0, min(n, n_in) - len(fixed)), replace=False)
    return np.sort(np.concatenate([fixed, extra]).astype(np.int64))


def _one_hot_check(L, cols, ref_cols, what):
    """x = e_c for every probe column c: y[:, o] must be W16[o, c] to within one
    float16 ulp, through the GEMV (8 columns per call) and through the GEMM's
    matrix-core tiles (all columns in one call, with and without a workspace)."""
    n_in = L.in_features
    x = np.zeros((len(cols), n_in), dtype=np.float16)
    x[np.arange(len(cols)), cols] = 1
    ref = ref_cols.T.astype(np.float32)  # [len(cols), out]
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float32)
    for b0 in range(0, len(cols), 8):
        y = L.gemv(dev_x(x[b0:b0 + 8])).cpu().numpy().astype(np.float32)
        bad = np.abs(y - ref[b0:b0 + 8]) > ulp[b0:b0 + 8]
        assert not bad.any(), f"{what} gemv: column {cols[b0 + np.argwhere(bad)[0][0]]}"
    if not L.general:
        for ws in (True, False):
            y = L.gemm(dev_x(x), workspace=ws).cpu().numpy().astype(np.float32)
            bad = np.abs(y - ref) > ulp
            assert not bad.any(), f"{what} gemm ws={ws}: column {cols[np.argwhere(bad)[0][0]]}"


ONE_HOT_IDS = [(w.name, l.name) for w in WL.WORKLOADS.values() if w.name != BIG
               for l in w.layers if not l.packed]


@pytest.mark.parametrize("wname,lname", ONE_HOT_IDS, ids=lambda v: str(v))
def test_workload_one_hot_probes(wname, lname):
    """64 one-hot probes per workload layer, including the first and last
    column of groups and the row tail: the loose product tolerance cannot see
    a single dropped or misplaced group at these widths, these probes can."""
    layer, d = _layer_data(wname, lname)
    cols = _probe_columns(layer.in_features, layer.scheme.g, seed=layer.seed)
    ref = oracle.decode(d.codes, d.codebooks, d.scales)[:, cols]
    _one_hot_check(dev_layer(d.codes, d.codebooks, d.scales), cols, ref, f"{wname}/{lname}")


@pytest.mark.parametrize("lname", [l.name for l in WL.WORKLOADS[BIG].layers])
def test_llama2_70b_layer_every_row(lname):
    """The Llama-2-70B-shaped layers checked on every row, in chunks of 2048
    rows (one oracle decode pass per layer): aqlm_dequant bit-exact, aqlm_gemv
    at batch 1 within tolerance, and 64 one-hot probes."""
    layer, d = _layer_data(BIG, lname)
    out = layer.out_features
    L = dev_layer(d.codes, d.codebooks, d.scales)
    w_gpu = L.dequant()
    x = WL.make_x(layer, 1)
    y_gpu = L.gemv(dev_x(x)).cpu().numpy()
    cols = _probe_columns(layer.in_features, layer.scheme.g, seed=layer.seed)
    ref_cols = np.empty((out, len(cols)), dtype=np.float16)
    for r0 in range(0, out, 2048):
        rows = np.arange(r0, min(out, r0 + 2048))
        ref = oracle.decode_rows(d.codes, d.codebooks, d.scales, rows)
        assert_bit_exact(w_gpu[r0:r0 + len(rows)].cpu().numpy(), ref, f"{BIG}/{lname} rows {r0}+")
        y_ref, bound = oracle.product(x, ref)
        assert_product(y_gpu[:, rows], y_ref, bound, f"{BIG}/{lname} gemv rows {r0}+")
        ref_cols[rows] = ref[:, cols]
    del w_gpu
    torch.cuda.empty_cache()
    _one_hot_check(L, cols, ref_cols, f"{BIG}/{lname}")


@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_rows_per_wavefront_same_bits(batch):
    """The 1x16 GEMV kernel gives each wavefront 1, 2 or 4 rows by the layer's
    row count (1024, 4096 and 12288 rows here); a row's sum, and so its bits,
    must not depend on that. The taller layers repeat the 1024-row codes."""
    c, b, sc, x = WL.small_case(1024, 1024, WL.S1x16, batch, seed=11)
    y0 = dev_layer(c, b, sc).gemv(dev_x(x), workspace=False).cpu().numpy()
    y_ref, bound = oracle.forward(x, c, b, sc)
    assert_product(y0, y_ref, bound, f"1024 rows b{batch}")
    for k in (4, 12):
        yk = dev_layer(np.tile(c, (k, 1, 1)), b, np.tile(sc, k)).gemv(
            dev_x(x), workspace=False).cpu().numpy()
        for i in range(k):
            assert_bit_exact(yk[:, i * 1024:(i + 1) * 1024], y0, f"{1024 * k} rows, copy {i}")


def test_sliced_gemv_rows_same_bits_wherever_they_sit():
    """The codebook-sliced kernel (aqlm_gemv_ws, 1x16, one row) splits rows
    over 32 teams by the layer's row count; a row's bits must not depend on
    which team, wavefront or ring slot computes it. The taller layers repeat
    the 8200-row codes (16400 and 16401 rows: a ragged last team)."""
    c, b, sc, x = WL.small_case(8200, 4096, WL.S1x16, 1, seed=12)
    L0 = dev_layer(c, b, sc)
    assert _lib.gemv_workspace_bytes([L0], 1) > 0
    y0 = L0.gemv(dev_x(x)).cpu().numpy()
    y_ref, bound = oracle.forward(x, c, b, sc)
    assert_product(y0, y_ref, bound, "8200 rows, sliced")
    for k, extra in ((2, 0), (2, 1)):
        ck = np.concatenate([np.tile(c, (k, 1, 1)), c[:extra]])
        sk = np.concatenate([np.tile(sc, k), sc[:extra]])
        yk = dev_layer(ck, b, sk).gemv(dev_x(x)).cpu().numpy()
        for i in range(k):
            assert_bit_exact(yk[:, i * 8200:(i + 1) * 8200], y0, f"{8200 * k + extra} rows, copy {i}")


# the workload's batches plus batches of the workspace GEMM (1..16 rows: one
# activation tile on the 11008-row layers, the skinny tile on the others;
# 33..128 rows:
# three row tiles per workgroup on the 11008-row layers, whose last row block
# is a third full, a half chunk at the end of the 11008-input rows; 200 rows:
# two blocks of 128 activation rows on the layers whose wide grid would be
# small)
GEMM_IDS = [(l.name, b) for l in WL.WORKLOADS["gemm_mlp"].layers
            for b in sorted(set(WL.WORKLOADS["gemm_mlp"].batches) | {1, 8, 33, 64, 100, 200})]


@pytest.mark.parametrize("lname,batch", GEMM_IDS, ids=lambda v: str(v))
def test_workload_gemm(lname, batch):
    layer, d = _layer_data("gemm_mlp", lname)
    x = WL.make_x(layer, batch)
    L = dev_layer(d.codes, d.codebooks, d.scales)
    toks = np.arange(batch) if batch <= 128 else np.unique(np.concatenate(
        [[0, batch - 1], np.random.default_rng(1).choice(batch, 62, replace=False)]))
    y_ref, bound = oracle.forward(x[toks], d.codes, d.codebooks, d.scales)
    for ws in ((True, False) if batch <= 128 else (True,)):
        y = L.gemm(dev_x(x), workspace=ws).cpu().numpy()
        assert_product(y[toks], y_ref, bound, f"gemm {lname} b{batch} ws={ws}")


@pytest.mark.parametrize("sname", list(SCHEMES))
@pytest.mark.parametrize("out,n_in,batch", [(100, 16384, 40), (40, 32768, 128), (1000, 8192, 20),
                                            (1035, 16384, 70)])
def test_gemm_split_k(sname, out, n_in, batch):
    """Few output rows over a long K: the workspace form splits K across
    workgroups, which write float32 partial tiles that a second launch adds in
    part order. 1035 rows take three row tiles per workgroup with a ragged last
    block. Two calls in a row give the same bits."""
    s = SCHEMES[sname]
    codes, books, scales, x = WL.small_case(out, n_in, s, batch, seed=out + batch)
    layer = dev_layer(codes, books, scales)
    y_ref, bound = oracle.forward(x, codes, books, scales)
    ws = torch.empty(layer.workspace_bytes(batch), dtype=torch.uint8, device=device())
    nt = -(-batch // 16)
    assert ws.numel() > n_in * 16 * (nt if nt <= 4 else 8 if nt > 6 else 6) * 2 + 512  # K is split
    ys = []
    for _ in range(2):
        y = torch.empty((batch, out), dtype=torch.float16, device=device())
        assert _lib.raw_call("aqlm_gemm_ws", layer._struct, dev_x(x).data_ptr(), batch,
                             y.data_ptr(), ws.data_ptr(), ws.numel(), None) == 0
        torch.cuda.synchronize()
        assert_product(y, y_ref, bound, f"split-K gemm {sname} {out}x{n_in} b{batch}")
        ys.append(bits(y))
    assert np.array_equal(ys[0], ys[1])


# GEMV calls that run on the 16-row GEMM tiles (2x8 rows too long to stage 5..8
# activation rows on chip, 1x16 once batch x in reaches 32768, 1x16 g16 from
# two rows) give exactly the bits of aqlm_gemm at that batch; the neighbours
# on the GEMV side of each threshold are checked against the oracle too.
@pytest.mark.parametrize("sname,out,n_in,batch,tiles", [
    ("2x8", 4096, 11008, 4, False), ("2x8", 4096, 11008, 5, True), ("2x8", 4096, 11008, 8, True),
    ("1x16", 1000, 11008, 2, False), ("1x16", 1000, 11008, 3, True),
    ("1x16", 1000, 4096, 7, False), ("1x16", 1000, 4096, 8, True),
    ("1x16g16", 300, 4096, 1, False), ("1x16g16", 300, 4096, 2, True),
    # layers whose GEMM tile is the workspace form's one activation tile read in place
    ("1x16g16", 11008, 4096, 2, True), ("1x16", 11008, 4096, 8, True), ("2x8", 7000, 2112, 3, True)])
def test_gemv_on_gemm_tiles(sname, out, n_in, batch, tiles):
    s = SCHEMES[sname]
    codes, books, scales, x = WL.small_case(out, n_in, s, batch, seed=out + n_in + batch)
    layer = dev_layer(codes, books, scales)
    y = layer.gemv(dev_x(x))
    rows = _sample_rows(out, n=256)
    y_ref, bound = oracle.forward_rows(x, codes, books, scales, rows)
    assert_product(y.cpu().numpy()[:, rows], y_ref, bound, f"gemv {sname} {out}x{n_in} b{batch}")
    if tiles:
        assert np.array_equal(bits(y), bits(layer.gemm(dev_x(x), workspace=False)))


@pytest.mark.parametrize("batch", [3, 7, 16])
def test_gemm_one_tile_in_place(batch):
    """Up to 16 rows, on layers with enough row blocks, the product runs one
    activation tile of the workspace form reading x in place: no workspace,
    the same bits with and without one. 2112 inputs leave a quarter-full last
    super-chunk; 7000 rows a ragged last row block."""
    s = SCHEMES["2x8"]
    codes, books, scales, x = WL.small_case(7000, 2112, s, batch, seed=batch)
    layer = dev_layer(codes, books, scales)
    assert layer.workspace_bytes(batch) == 0
    y = layer.gemm(dev_x(x), workspace=False)
    assert np.array_equal(bits(y), bits(layer.gemm(dev_x(x), workspace=True)))
    rows = _sample_rows(7000, n=512)
    y_ref, bound = oracle.forward_rows(x, codes, books, scales, rows)
    assert_product(y.cpu().numpy()[:, rows], y_ref, bound, f"one tile in place b{batch}")


@pytest.mark.parametrize("sname", list(SCHEMES))
def test_dedicated_schemes_bit_packed(sname):
    """The bit-packed flag on a dedicated scheme (8- or 16-bit codes, where the
    stream holds the element layout's bytes) gives the element layout's bits
    on every entry point and route."""
    s = SCHEMES[sname]
    out, n_in = 300, 64 * s.g
    codes, books, scales, x = WL.small_case(out, n_in, s, 130, seed=21)
    plain = dev_layer(codes, books, scales)
    words = WL.pack_codes(codes, s.B)
    packed = AqlmLayer(torch.from_numpy(words.view(np.int32)).to(device()),
                       torch.from_numpy(books).to(device()), torch.from_numpy(scales).to(device()),
                       in_features=n_in)
    assert np.array_equal(bits(packed.dequant()), bits(plain.dequant()))
    for batch in (1, 2, 5, 8):
        xb = dev_x(x[:batch])
        assert np.array_equal(bits(packed.gemv(xb)), bits(plain.gemv(xb))), batch
    for batch in (16, 64, 130):
        xb = dev_x(x[:batch])
        for ws in (True, False):
            assert np.array_equal(bits(packed.gemm(xb, workspace=ws)),
                                  bits(plain.gemm(xb, workspace=ws))), (batch, ws)
    y_ref, bound = oracle.forward(x[:8], codes, books, scales)
    assert_product(packed.gemv(dev_x(x[:8])), y_ref, bound, f"packed {sname} gemv b8")


# ---------------------------------------------------------------------------
# probes the loose tolerance cannot replace
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("sname,out,n_in", [("2x8", 4096, 4096), ("1x16", 4096, 11008),
                                            ("1x16g16", 1000, 2048), ("2x8", 300, 520)])
def test_one_hot_probes(sname, out, n_in):
    """x = e_i returns column i of W: the lookup path to within one float16 ulp,
    exactly for the decode-then-dot order (first/last column of groups, row tail)."""
    s = SCHEMES[sname]
    codes, books, scales, _ = WL.small_case(out, n_in, s, 1, seed=out + n_in)
    layer = dev_layer(codes, books, scales)
    w_ref = oracle.decode(codes, books, scales).astype(np.float32)
    cols = np.unique(np.array([0, s.g - 1, s.g, n_in // 2, n_in // 2 + 1, n_in - s.g,
                               n_in - 2, n_in - 1]))
    for fn in (layer.gemv, layer.gemm):
        for c0 in range(0, len(cols), 8):
            cc = cols[c0:c0 + 8]
            x = np.zeros((len(cc), n_in), dtype=np.float16)
            x[np.arange(len(cc)), cc] = 1
            y = fn(dev_x(x)).cpu().numpy().astype(np.float32)
            ref = w_ref[:, cc].T
            ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float32)
            assert np.all(np.abs(y - ref) <= ulp), (fn.__name__, sname, cc)


@pytest.mark.parametrize("sname", list(SCHEMES))
def test_deterministic(sname):
    s = SCHEMES[sname]
    codes, books, scales, x = WL.small_case(2000, 2048, s, 64, seed=5)
    layer = dev_layer(codes, books, scales)
    gemm_plain = lambda v: layer.gemm(v, workspace=False)  # noqa: E731
    for name, fn, xb in (("gemv", layer.gemv, x[:8]), ("gemm_ws", layer.gemm, x),
                         ("gemm", gemm_plain, x)):
        a = bits(fn(dev_x(xb)))
        b = bits(fn(dev_x(xb)))
        assert np.array_equal(a, b), name


@pytest.mark.parametrize("sname", list(SCHEMES))
def test_outputs_stay_in_bounds(sname):
    """Canary words after y and W stay untouched."""
    s = SCHEMES[sname]
    out, n_in = 300, 13 * s.g
    codes, books, scales, x = WL.small_case(out, n_in, s, 8, seed=7)
    layer = dev_layer(codes, books, scales)
    canary = np.float16(-12345.0)
    ybuf = torch.full((8 * out + 64,), float(canary), dtype=torch.float16, device=device())
    for fn in ("gemv", "gemm"):
        y = ybuf[: 8 * out].view(8, out)
        getattr(layer, fn)(dev_x(x), out=y)
        assert torch.all(ybuf[8 * out:] == float(canary)), fn
    wbuf = torch.full((out * n_in + 64,), float(canary), dtype=torch.float16, device=device())
    layer.dequant(out=wbuf[: out * n_in].view(out, n_in))
    assert torch.all(wbuf[out * n_in:] == float(canary))


@pytest.mark.parametrize("sname", list(SCHEMES))
def test_workspace_form_stays_in_bounds(sname):
    """The workspace form writes y and at most its workspace: canary words after
    both stay untouched (ragged rows and activation rows, split and unsplit)."""
    s = SCHEMES[sname]
    canary = np.float16(-12345.0)
    for out, n_in, batch in ((300, 64 * s.g, 37), (20, 512 * s.g, 70)):
        codes, books, scales, x = WL.small_case(out, n_in, s, batch, seed=out)
        layer = dev_layer(codes, books, scales)
        need = layer.workspace_bytes(batch)
        assert need > 0
        ybuf = torch.full((batch * out + 64,), float(canary), dtype=torch.float16, device=device())
        wbuf = torch.full(((need + 256) // 2,), float(canary), dtype=torch.float16, device=device())
        assert _lib.raw_call("aqlm_gemm_ws", layer._struct, dev_x(x).data_ptr(), batch,
                             ybuf.data_ptr(), wbuf.data_ptr(), need, None) == 0
        torch.cuda.synchronize()
        assert torch.all(ybuf[batch * out:] == float(canary))
        assert torch.all(wbuf[(need + 1) // 2:] == float(canary))
        y_ref, bound = oracle.forward(x, codes, books, scales)
        assert_product(ybuf[: batch * out].view(batch, out), y_ref, bound, f"{sname} {out}x{n_in}")


def test_zero_batch_is_noop():
    codes, books, scales, x = WL.small_case(16, 64, WL.S2x8, 1, seed=1)
    layer = dev_layer(codes, books, scales)
    y = torch.full((0, 16), 1.0, dtype=torch.float16, device=device())
    assert layer.gemv(dev_x(x[:0])).shape == (0, 16)
    assert layer.gemm(dev_x(x[:0])).shape == (0, 16)
