"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each pin takes an implementation namespace with the oracle's interface
(decode, decode_rows, forward, product, bits_per_weight,
packed_bits_per_weight) and raises AssertionError when it disagrees with:
hand-worked golden values, exact IEEE-754 rational arithmetic, closed
forms, reductions to textbook special cases, or invariants of the product.
The same pins are run against planted-mistake copies of the oracle to show
that each plausible mistake is caught by at least one of them.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

from ieee_exact import decode_group_bits, from_f16_bits, value

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16(v):
    return np.asarray(v, dtype=np.float16)


def _bits(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def _golden_layer(case):
    M, B, g = case["M"], case["B"], case["g"]
    books = np.zeros((M, 2 ** B, g), dtype=np.float16)
    for m, rows in case["codebook_rows"].items():
        for c, vals in rows.items():
            books[int(m), int(c)] = _f16(vals)
    dt = np.uint8 if B == 8 else np.uint16
    codes = np.asarray(case["codes"], dtype=dt)
    scales = _f16(case["scales"])
    x = _f16(case["x"])
    return codes, books, scales, x


# --------------------------------------------------------------------------
# golden, hand-worked
# --------------------------------------------------------------------------
def pin_hand_worked(impl):
    """Golden layers worked by hand (layout, additive rule, per-row scale, product)."""
    for case in _load("hand_worked_groups.json")["cases"]:
        codes, books, scales, x = _golden_layer(case)
        w = impl.decode(codes, books, scales)
        if "expected_w_bits" in case:
            exp = np.array([[int(h, 16) for h in row] for row in case["expected_w_bits"]],
                           dtype=np.uint16)
            assert np.array_equal(_bits(w), exp), (case["name"], _bits(w), exp)
        else:
            exp = _f16(case["expected_w"])
            assert np.array_equal(_bits(w), _bits(exp)), (case["name"], w, exp)
        y, bound = impl.forward(x, codes, books, scales)
        assert np.array_equal(y, np.asarray(case["expected_y"], dtype=np.float64)), \
            (case["name"], y, case["expected_y"])


def pin_rounding_cases(impl):
    """Golden single-weight decodes: ties, scale placement, subnormals, signs, order."""
    for case in _load("rounding_cases.json")["cases"]:
        cw = [int(h, 16) for h in case["codewords"]]
        M = len(cw)
        books = np.zeros((M, 256, 1), dtype=np.uint16)
        for m in range(M):
            books[m, 7, 0] = cw[m]
        books = books.view(np.float16)
        codes = np.full((1, 1, M), 7, dtype=np.uint8)
        scales = np.array([int(case["scale"], 16)], dtype=np.uint16).view(np.float16)
        with np.errstate(over="ignore"):
            w = impl.decode(codes, books, scales)
        got = int(_bits(w)[0, 0])
        assert got == int(case["expected"], 16), (case["name"], hex(got), case["expected"])


# --------------------------------------------------------------------------
# exact arithmetic (brute force over rationals)
# --------------------------------------------------------------------------
def _special_codebooks(rng, M, B, g):
    """Codebooks mixing normal values with subnormals, signed zeros and large values."""
    n = 2 ** B
    books = rng.normal(0, 0.02, size=(M, n, g)).astype(np.float16)
    bits = books.view(np.uint16)
    pick = rng.random(size=bits.shape)
    bits[pick < 0.08] = rng.integers(0, 1024, size=int((pick < 0.08).sum())).astype(np.uint16)
    neg = (pick >= 0.08) & (pick < 0.12)
    bits[neg] |= 0x8000
    bits[(pick >= 0.12) & (pick < 0.14)] = 0x8000
    big = (pick >= 0.14) & (pick < 0.16)
    bits[big] = rng.integers(0x6000, 0x7000, size=int(big.sum())).astype(np.uint16)
    return books


def pin_brute_force_decode(impl):
    """Vectorised decode == exact per-element IEEE emulation, bit for bit."""
    rng = np.random.default_rng(12345)
    for (M, B, g, out, J, span) in ((2, 8, 8, 3, 4, 64), (1, 16, 8, 2, 3, 64),
                                    (1, 16, 16, 2, 2, 64), (3, 8, 4, 2, 3, 64),
                                    (1, 8, 1, 4, 5, 64),
                                    # general schemes: more codebooks, wider codes
                                    (4, 8, 8, 2, 3, 256), (8, 8, 16, 2, 2, 256),
                                    (1, 12, 8, 3, 3, 4096), (2, 12, 16, 2, 2, 4096),
                                    (3, 10, 8, 2, 3, 1024), (5, 16, 8, 2, 2, 65536)):
        books = _special_codebooks(rng, M, B, g)
        codes = rng.integers(0, min(2 ** B, span), size=(out, J, M)).astype(
            np.uint8 if B == 8 else np.uint16)
        if span > 256:
            codes[0, 0, :] = 2 ** B - 1   # the last codeword of every codebook
        scales = rng.uniform(0.5, 1.5, size=out).astype(np.float16)
        scales[0] = np.float16(0.0009765625)   # push products into the subnormal range
        with np.errstate(over="ignore"):
            w = _bits(impl.decode(codes, books, scales))
        bb = books.view(np.uint16)
        sb = scales.view(np.uint16)
        for o in range(out):
            for j in range(J):
                cws = [[int(v) for v in bb[m, codes[o, j, m]]] for m in range(M)]
                exp = decode_group_bits(cws, int(sb[o]))
                got = [int(v) for v in w[o, j * g:(j + 1) * g]]
                assert got == exp, ((M, B, g), o, j, [hex(v) for v in got], [hex(v) for v in exp])


def pin_brute_force_product(impl):
    """float64 product == exact rational dot product, within float64 rounding."""
    rng = np.random.default_rng(777)
    for (M, B, g, out, J, batch) in ((2, 8, 8, 5, 6, 3), (1, 16, 8, 4, 4, 2),
                                     (1, 16, 16, 3, 3, 1)):
        codes = rng.integers(0, 2 ** B, size=(out, J, M)).astype(np.uint8 if B == 8 else np.uint16)
        books = rng.normal(0, 0.02, size=(M, 2 ** B, g)).astype(np.float16)
        scales = rng.uniform(0.5, 1.5, size=out).astype(np.float16)
        x = rng.standard_normal((batch, J * g)).astype(np.float16)
        w = impl.decode(codes, books, scales)
        y, bound = impl.forward(x, codes, books, scales)
        K = J * g
        xb, wb = x.view(np.uint16), np.asarray(w, dtype=np.float16).view(np.uint16)
        for b in range(batch):
            for o in range(out):
                exact = sum(value(from_f16_bits(int(xb[b, i]))) * value(from_f16_bits(int(wb[o, i])))
                            for i in range(K))
                absb = sum(abs(value(from_f16_bits(int(xb[b, i]))) * value(from_f16_bits(int(wb[o, i]))))
                           for i in range(K))
                assert abs(Fraction(float(y[b, o])) - exact) <= Fraction(K, 2 ** 52) * absb, (b, o)
                assert abs(Fraction(float(bound[b, o])) - absb) <= Fraction(K, 2 ** 52) * absb, (b, o)


# --------------------------------------------------------------------------
# closed forms and special cases
# --------------------------------------------------------------------------
def pin_scalar_lut_special_case(impl):
    """M = 1, g = 1 is scalar lookup-table quantization: W[o, i] = fp16(s_o * T[c_oi])."""
    rng = np.random.default_rng(5)
    out, n_in = 7, 19
    table = rng.normal(0, 0.5, size=(1, 256, 1)).astype(np.float16)
    codes = rng.integers(0, 256, size=(out, n_in, 1)).astype(np.uint8)
    scales = rng.uniform(0.5, 1.5, size=out).astype(np.float16)
    w_expected = (table[0, codes[:, :, 0], 0].astype(np.float32)
                  * scales.astype(np.float32)[:, None]).astype(np.float16)
    w = impl.decode(codes, table, scales)
    assert np.array_equal(_bits(w), _bits(w_expected))
    x = rng.standard_normal((2, n_in)).astype(np.float16)
    y, _ = impl.forward(x, codes, table, scales)
    # for g = 1 the product is a plain matrix-vector product
    y_expected = np.array([[sum(float(x[b, i]) * float(w_expected[o, i]) for i in range(n_in))
                            for o in range(out)] for b in range(2)])
    assert np.allclose(y, y_expected, rtol=0, atol=1e-12)


def pin_constant_codes(impl):
    """All codes equal c*: every group of row o decodes to the same g weights, and
    y_o = sum_j <x_j, that group>."""
    rng = np.random.default_rng(9)
    M, B, g, out, J = 2, 8, 8, 4, 6
    books = rng.normal(0, 0.02, size=(M, 2 ** B, g)).astype(np.float16)
    cstar = (17, 201)
    codes = np.empty((out, J, M), dtype=np.uint8)
    codes[:, :, 0], codes[:, :, 1] = cstar
    scales = rng.uniform(0.5, 1.5, size=out).astype(np.float16)
    w = impl.decode(codes, books, scales)
    bb, sb = books.view(np.uint16), scales.view(np.uint16)
    x = rng.standard_normal((1, J * g)).astype(np.float16)
    y, _ = impl.forward(x, codes, books, scales)
    for o in range(out):
        group = decode_group_bits([[int(v) for v in bb[m, cstar[m]]] for m in range(M)], int(sb[o]))
        assert [int(v) for v in _bits(w)[o]] == group * J
        gv = [float(value(from_f16_bits(h))) for h in group]
        y_closed = sum(float(x[0, j * g + k]) * gv[k] for j in range(J) for k in range(g))
        assert abs(y[0, o] - y_closed) <= 1e-12 * (1 + abs(y_closed))


def pin_zero_second_codebook(impl):
    """With the second codebook all +0, 2x8 decodes like the first codebook alone
    (a -0 codeword entry turns into +0, equal in value)."""
    rng = np.random.default_rng(21)
    out, J = 5, 7
    books = rng.normal(0, 0.02, size=(2, 256, 8)).astype(np.float16)
    books[1] = 0
    codes = rng.integers(0, 256, size=(out, J, 2)).astype(np.uint8)
    scales = rng.uniform(0.5, 1.5, size=out).astype(np.float16)
    w2 = impl.decode(codes, books, scales)
    w1 = impl.decode(codes[:, :, :1].copy(), books[:1].copy(), scales)
    assert np.array_equal(w2.astype(np.float32), w1.astype(np.float32))


def pin_one_hot_columns(impl):
    """x = e_i selects column i of W: y[:, o] == W[o, i] exactly."""
    rng = np.random.default_rng(31)
    for (M, B, g) in ((2, 8, 8), (1, 16, 8), (1, 16, 16)):
        out, J = 6, 3
        codes = rng.integers(0, 2 ** B, size=(out, J, M)).astype(np.uint8 if B == 8 else np.uint16)
        books = rng.normal(0, 0.02, size=(M, 2 ** B, g)).astype(np.float16)
        scales = rng.uniform(0.5, 1.5, size=out).astype(np.float16)
        K = J * g
        x = np.eye(K, dtype=np.float16)
        y, bound = impl.forward(x, codes, books, scales)
        w = impl.decode(codes, books, scales).astype(np.float64)
        assert np.array_equal(y, w.T)
        assert np.array_equal(bound, np.abs(w.T))


def pin_linearity(impl):
    """y(2^k x) = 2^k y(x) exactly; y(x1 + x2) = y(x1) + y(x2) to float64 rounding;
    doubling the scales doubles every normal decoded weight exactly."""
    rng = np.random.default_rng(41)
    codes = rng.integers(0, 256, size=(8, 16, 2)).astype(np.uint8)
    books = rng.normal(0, 0.02, size=(2, 256, 8)).astype(np.float16)
    scales = rng.uniform(0.5, 1.5, size=8).astype(np.float16)
    x = rng.standard_normal((3, 128)).astype(np.float16)
    y, bound = impl.forward(x, codes, books, scales)
    y4, _ = impl.forward((x.astype(np.float32) * 4).astype(np.float16), codes, books, scales)
    assert np.array_equal(y4, 4 * y)
    x1 = (x.astype(np.float32) * 0.5).astype(np.float16)
    x2 = (x.astype(np.float32) - x1.astype(np.float32)).astype(np.float16)
    y1, _ = impl.forward(x1, codes, books, scales)
    y2, _ = impl.forward(x2, codes, books, scales)
    ysum, bsum = impl.forward((x1.astype(np.float32) + x2.astype(np.float32)).astype(np.float16),
                              codes, books, scales)
    assert np.all(np.abs(ysum - (y1 + y2)) <= 1e-13 * (1 + bsum))
    w = impl.decode(codes, books, scales).astype(np.float32)
    w2 = impl.decode(codes, books, (scales.astype(np.float32) * 2).astype(np.float16)).astype(np.float32)
    normal = np.abs(w) >= 2.0 ** -14
    assert np.array_equal(w2[normal], 2 * w[normal])
    assert normal.mean() > 0.9


def pin_bits_per_weight(impl):
    """The closed form equals the stored bytes, gives 8x compression at 2 code bits,
    and reproduces 2.07 bits for a Llama-2-70B-shaped block of 1x16 g8 layers."""
    for (out, n_in, M, B, g) in ((512, 1024, 2, 8, 8), (4096, 4096, 2, 8, 8),
                                 (11008, 4096, 1, 16, 8), (4096, 11008, 1, 16, 16),
                                 (64, 64, 3, 8, 4)):
        codes = np.zeros((out, n_in // g, M), dtype=np.uint8 if B == 8 else np.uint16)
        books = np.zeros((M, 2 ** B, g), dtype=np.float16)
        scales = np.zeros(out, dtype=np.float16)
        measured = impl.packed_bits_per_weight(codes, books, scales)
        closed = impl.bits_per_weight(out, n_in, M, B, g)
        assert abs(measured - closed) <= 1e-12 * closed, (out, n_in, M, B, g, measured, closed)
    # codes wider than 8 bits sit in 16-bit elements: the stored size follows
    # the container, and equals the nominal one when B fills whole bytes
    for (out, n_in, M, B, g) in ((64, 128, 1, 12, 8), (32, 256, 2, 10, 16), (16, 64, 3, 8, 8),
                                 (16, 64, 2, 16, 16), (8, 64, 8, 9, 8)):
        codes = np.zeros((out, n_in // g, M), dtype=np.uint8 if B == 8 else np.uint16)
        books = np.zeros((M, 2 ** B, g), dtype=np.float16)
        scales = np.zeros(out, dtype=np.float16)
        measured = impl.packed_bits_per_weight(codes, books, scales)
        stored = impl.stored_bits_per_weight(out, n_in, M, B, g)
        assert abs(measured - stored) <= 1e-12 * stored, (out, n_in, M, B, g, measured, stored)
        nominal = impl.bits_per_weight(out, n_in, M, B, g)
        assert (abs(stored - nominal) <= 1e-12 * nominal) == (B % 8 == 0)
    # 2 code bits per weight against 16-bit weights: the "up to ~8x" compression
    big = impl.bits_per_weight(1 << 20, 1 << 20, 2, 8, 8)
    assert abs(16 / big - 8.0) < 1e-3
    assert impl.bits_per_weight(512, 1024, 2, 8, 8) == 2.140625
    shapes = ((8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192),
              (28672, 8192), (28672, 8192), (8192, 28672))
    bits = sum(impl.bits_per_weight(o, i, 1, 16, 8) * o * i for o, i in shapes)
    n = sum(o * i for o, i in shapes)
    assert round(bits / n, 2) == 2.07


def pin_unpack_codes(impl):
    """Bit-packed codes: a hand-packed stream, an independent bit-by-bit
    reader, and the byte / halfword layouts that B = 8 and 16 must reproduce."""
    got = impl.unpack_codes(np.array([0xFF123ABC, 0x0000000F], dtype=np.uint32), 1, 1, 3, 12)
    assert got.tolist() == [[[0xABC, 0x123, 0xFFF]]]
    rng = np.random.default_rng(21)
    for B in (9, 10, 11, 12, 13, 15):
        out, J, M = 5, 7, 3
        n = out * J * M
        words = rng.integers(0, 2 ** 32, size=(n * B + 31) // 32, dtype=np.uint64).astype(np.uint32)
        bits = [(int(words[p // 32]) >> (p % 32)) & 1 for p in range(n * B)]
        want = [sum(bits[i * B + t] << t for t in range(B)) for i in range(n)]
        assert impl.unpack_codes(words, out, J, M, B).reshape(-1).tolist() == want
    c8 = rng.integers(0, 256, size=(3, 4, 2), dtype=np.uint8)
    assert np.array_equal(impl.unpack_codes(c8.reshape(-1).view(np.uint32), 3, 4, 2, 8), c8)
    c16 = rng.integers(0, 65536, size=(3, 4, 2), dtype=np.uint16)
    assert np.array_equal(impl.unpack_codes(c16.reshape(-1).view(np.uint32), 3, 4, 2, 16), c16)


ALL_PINS = [
    pin_hand_worked, pin_rounding_cases, pin_brute_force_decode, pin_brute_force_product,
    pin_scalar_lut_special_case, pin_constant_codes, pin_zero_second_codebook,
    pin_one_hot_columns, pin_linearity, pin_bits_per_weight, pin_unpack_codes,
]
