"""Host (CPU) GEMV library, aqlm_host_gemv (include/aqlm_host.h), against the
CPU oracle: every scheme family on small ragged layers, both instruction-set
forms, thread-count independence, the golden hand-worked and rounding cases
(a one-hot activation returns the decoded weight exactly), argument errors,
and Llama-2-7B layers at full size. No GPU involved.
"""
import ctypes
import json
import os

import numpy as np
import pytest

import oracle
from additive_codebook_matmul_amd import workloads as WL
from additive_codebook_matmul_amd import host
from additive_codebook_matmul_amd._lib import AqlmLayerStruct
from gpu_util import REL_TOL, TIGHT_TOL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
S = WL.Scheme
SCHEMES = [S(2, 8, 8), S(1, 16, 8), S(1, 16, 16), S(3, 8, 8), S(4, 8, 16), S(1, 12, 8),
           S(2, 12, 16), S(8, 8, 16), S(5, 9, 8), S(1, 8, 8)]
SHAPES = [(1, 1), (7, 5), (65, 9), (130, 17)]


@pytest.fixture(scope="module", autouse=True)
def _host_library():
    if not os.path.exists(host.HOST_LIB_PATH):
        from additive_codebook_matmul_amd.build import build_host_library
        build_host_library(verbose=False)
    host.load_host_library()


@pytest.fixture(params=["avx2", "scalar"])
def isa(request, monkeypatch):
    if request.param == "scalar":
        monkeypatch.setenv("AQLM_HOST_ISA", "scalar")
        assert host.host_isa() == "scalar"
    else:
        monkeypatch.delenv("AQLM_HOST_ISA", raising=False)
        if host.host_isa() != "avx2":
            pytest.skip("this CPU lacks AVX2/FMA/F16C")
    return request.param


def _check(y, y_ref, bound, what):
    ok = oracle.within_tolerance(y, y_ref, bound, rel=REL_TOL)
    assert ok.all(), f"{what}: {int((~ok).sum())} outputs outside 1e-2*sum|xw|"
    err = np.abs(y.astype(np.float64) - y_ref)
    rel = np.where(bound > 0, err / np.where(bound > 0, bound, 1), err)
    assert rel.max() <= TIGHT_TOL, f"{what}: tight gate {rel.max():.3e}"


@pytest.mark.parametrize("scheme", SCHEMES, ids=lambda s: s.name)
@pytest.mark.parametrize("out,J", SHAPES)
def test_host_small(scheme, out, J, isa):
    codes, books, scales, x = WL.small_case(out, J * scheme.g, scheme, 8, seed=out * 7 + J)
    w = oracle.decode(codes, books, scales)
    for batch in (1, 3, 8):
        y = host.host_gemv(codes, books, scales, x[:batch], threads=3)
        y_ref, bound = oracle.product(x[:batch], w)
        _check(y, y_ref, bound, f"{scheme.name} {out}x{J} b{batch} {isa}")


@pytest.mark.parametrize("scheme", [S(1, 12, 8), S(2, 10, 16), S(3, 9, 8), S(2, 8, 8), S(1, 16, 8)],
                         ids=lambda s: s.name)
def test_host_packed_codes(scheme, isa):
    """Bit-packed code streams, unpacked on the oracle's side by its own reader."""
    codes, books, scales, x = WL.small_case(65, 9 * scheme.g, scheme, 8, seed=13)
    words = WL.pack_codes(codes, scheme.B)
    unpacked = oracle.unpack_codes(words, 65, 9, scheme.M, scheme.B)
    w = oracle.decode(unpacked, books, scales)
    for batch in (1, 8):
        y = host.host_gemv(words, books, scales, x[:batch], threads=2)
        y_ref, bound = oracle.product(x[:batch], w)
        _check(y, y_ref, bound, f"packed {scheme.name} b{batch} {isa}")


@pytest.mark.parametrize("scheme", [S(2, 8, 8), S(1, 16, 8), S(3, 10, 16)], ids=lambda s: s.name)
def test_host_threads_do_not_change_bits(scheme):
    codes, books, scales, x = WL.small_case(300, 40 * scheme.g, scheme, 8, seed=5)
    ys = [host.host_gemv(codes, books, scales, x, threads=t).view(np.uint16) for t in (1, 3, 8)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden("hand_worked_groups.json"), ids=lambda c: c["name"])
def test_host_golden_hand_worked(case, isa):
    M, B, g = case["M"], case["B"], case["g"]
    books = np.zeros((M, 2 ** B, g), dtype=np.float16)
    for m, rows in case["codebook_rows"].items():
        for c, vals in rows.items():
            books[int(m), int(c)] = np.asarray(vals, dtype=np.float16)
    codes = np.asarray(case["codes"], dtype=np.uint8 if B == 8 else np.uint16)
    scales = np.asarray(case["scales"], dtype=np.float16)
    x = np.asarray(case["x"], dtype=np.float16)
    y = host.host_gemv(codes, books, scales, x).astype(np.float64)
    assert np.array_equal(y, np.asarray(case["expected_y"], dtype=np.float64)), (y, case["expected_y"])


@pytest.mark.parametrize("case", [c for c in _golden("rounding_cases.json") if len(c["codewords"]) in (1, 2)],
                         ids=lambda c: c["name"])
def test_host_rounding_one_hot(case, isa):
    """x = e_3 returns the decoded weight of column 3: the table and the
    direct forms both multiply the exact float32 codeword sum by 1 and round
    scale * sum once, so the golden single-weight decodes come out exactly
    (compared as numbers: the zero products of the other columns may flip
    the sign of a zero)."""
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
    x = np.zeros((1, 8), dtype=np.float16)
    x[0, 3] = 1
    y = host.host_gemv(codes, books.view(np.float16), scales, x)
    want = np.array([int(case["expected"], 16)], dtype=np.uint16).view(np.float16)
    assert y[0, 0].astype(np.float32) == want[0].astype(np.float32) or (
        np.isnan(y[0, 0]) and np.isnan(want[0])), case["name"]


def _call_raw(st, x, batch, y):
    lib = host.load_host_library()
    return lib.aqlm_host_gemv(ctypes.byref(st) if st is not None else None, x, batch, y, 1)


def test_host_errors():
    codes, books, scales, x = WL.small_case(4, 16, S(2, 8, 8), 2, seed=1)
    y = np.empty((2, 4), dtype=np.float16)

    def st(M=2, B=8, g=8, out=4, n_in=16, flags=0, codes_p=codes.ctypes.data):
        return AqlmLayerStruct(out, n_in, M, B, g, flags, codes_p, books.ctypes.data,
                               scales.ctypes.data)
    xp, yp = x.ctypes.data, y.ctypes.data
    assert _call_raw(st(), xp, 2, yp) == 0
    assert _call_raw(st(), xp, 0, None) == 0               # batch 0: no-op
    assert _call_raw(None, xp, 2, yp) == 1                 # NULL layer
    assert _call_raw(st(codes_p=None), xp, 2, yp) == 1     # NULL codes
    assert _call_raw(st(), None, 2, yp) == 1               # NULL x
    assert _call_raw(st(n_in=12), xp, 2, yp) == 2          # in % g
    assert _call_raw(st(out=0), xp, 2, yp) == 2
    assert _call_raw(st(flags=2), xp, 2, yp) == 2
    for M, B, g in ((0, 8, 8), (9, 8, 8), (2, 7, 8), (2, 17, 8), (2, 8, 4), (2, 8, 32)):
        assert _call_raw(st(M, B, g), xp, 2, yp) == 3
    assert _call_raw(st(), xp, 9, yp) == 5
    assert _call_raw(st(), xp, -1, yp) == 5
    with pytest.raises(ValueError):
        host.host_gemv(codes.astype(np.uint16), books, scales, x)


@pytest.mark.parametrize("wname,lname", [("llama2_7b_2x8", "q"), ("llama2_7b_2x8", "down"),
                                         ("llama2_7b_1x16", "q")])
def test_host_workload_layers(wname, lname):
    layer = next(l for l in WL.WORKLOADS[wname].layers if l.name == lname)
    d = WL.make_layer(layer)
    x = WL.make_x(layer, 1)
    y = host.host_gemv(d.codes, d.codebooks, d.scales, x)
    y_ref, bound = oracle.forward(x, d.codes, d.codebooks, d.scales)
    _check(y, y_ref, bound, f"{wname} {lname}")
