"""Oracle pins (CPU only): the oracle against facts that do not come from itself."""
import types

import numpy as np
import pytest

import oracle
from oracle import aqlm_oracle as O
import oracle_pins as P
from additive_codebook_matmul_amd import workloads as WL


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(O)


# ---------------------------------------------------------------------------
# Planted mistakes: each copy of the oracle below carries one plausible error;
# the pin suite must reject every one of them.
# ---------------------------------------------------------------------------
def _impl(decode_rows=None, product=None, unpack=None):
    ns = types.SimpleNamespace()
    dr = decode_rows or O.decode_rows
    pr = product or O.product

    def decode(codes, books, scales):
        return dr(codes, books, scales, np.arange(np.asarray(codes).shape[0]))

    def forward(x, codes, books, scales):
        return pr(x, decode(codes, books, scales))

    ns.decode_rows, ns.decode, ns.forward, ns.product = dr, decode, forward, pr
    ns.bits_per_weight, ns.packed_bits_per_weight = O.bits_per_weight, O.packed_bits_per_weight
    ns.stored_bits_per_weight = O.stored_bits_per_weight
    ns.unpack_codes = unpack or O.unpack_codes
    return ns


def _gather(codes, books, rows):
    idx = np.asarray(codes)[rows].astype(np.int64)
    b32 = np.asarray(books).astype(np.float32)
    return [b32[m][idx[:, :, m]] for m in range(b32.shape[0])]


def _finish(acc, scales, rows, g):
    return acc.reshape(len(rows), -1)


def m_swapped_codebooks(codes, books, scales, rows):
    rows = np.asarray(rows)
    idx = np.asarray(codes)[rows].astype(np.int64)
    b32 = np.asarray(books).astype(np.float32)
    M = b32.shape[0]
    acc = b32[0][idx[:, :, M - 1]]
    for m in range(1, M):
        acc = acc + b32[m][idx[:, :, M - 1 - m]]
    acc = acc * np.asarray(scales)[rows].astype(np.float32)[:, None, None]
    return acc.astype(np.float16).reshape(len(rows), -1)


def m_fp16_sum_then_scale(codes, books, scales, rows):
    rows = np.asarray(rows)
    g = _gather(codes, books, rows)
    acc = g[0].astype(np.float16)
    for t in g[1:]:
        acc = (acc + t.astype(np.float16)).astype(np.float16)
    acc = (acc * np.asarray(scales)[rows][:, None, None]).astype(np.float16)
    return acc.reshape(len(rows), -1)


def m_no_scale(codes, books, scales, rows):
    rows = np.asarray(rows)
    g = _gather(codes, books, rows)
    acc = g[0]
    for t in g[1:]:
        acc = acc + t
    return acc.astype(np.float16).reshape(len(rows), -1)


def m_first_codebook_only(codes, books, scales, rows):
    rows = np.asarray(rows)
    g = _gather(codes, books, rows)
    acc = g[0] * np.asarray(scales)[rows].astype(np.float32)[:, None, None]
    return acc.astype(np.float16).reshape(len(rows), -1)


def m_strided_columns(codes, books, scales, rows):
    w = O.decode_rows(codes, books, scales, rows)
    J = np.asarray(codes).shape[1]
    g = np.asarray(books).shape[2]
    # column k*J + j instead of j*g + k
    return w.reshape(len(rows), J, g).transpose(0, 2, 1).reshape(len(rows), J * g)


def m_zero_init(codes, books, scales, rows):
    rows = np.asarray(rows)
    g = _gather(codes, books, rows)
    acc = np.zeros_like(g[0])
    for t in g:
        acc = acc + t
    acc = acc * np.asarray(scales)[rows].astype(np.float32)[:, None, None]
    return acc.astype(np.float16).reshape(len(rows), -1)


def m_descending_order(codes, books, scales, rows):
    rows = np.asarray(rows)
    g = _gather(codes, books, rows)
    acc = g[-1]
    for t in reversed(g[:-1]):
        acc = acc + t
    acc = acc * np.asarray(scales)[rows].astype(np.float32)[:, None, None]
    return acc.astype(np.float16).reshape(len(rows), -1)


def m_flush_subnormals(codes, books, scales, rows):
    w = O.decode_rows(codes, books, scales, rows)
    w = w.copy()
    w[np.abs(w.astype(np.float32)) < 2.0 ** -14] = 0
    return w


def m_truncate_round(codes, books, scales, rows):
    rows = np.asarray(rows)
    g = _gather(codes, books, rows)
    acc = g[0]
    for t in g[1:]:
        acc = acc + t
    acc = acc * np.asarray(scales)[rows].astype(np.float32)[:, None, None]
    # round toward zero: clear the 13 low mantissa bits of float32 before narrowing
    b = acc.view(np.uint32) & np.uint32(0xFFFFE000)
    return b.view(np.float32).astype(np.float16).reshape(len(rows), -1)


def m_scale_by_group(codes, books, scales, rows):
    rows = np.asarray(rows)
    g = _gather(codes, books, rows)
    acc = g[0]
    for t in g[1:]:
        acc = acc + t
    s = np.asarray(scales).astype(np.float32)
    J = acc.shape[1]
    sj = s[np.arange(J) % s.shape[0]]
    acc = acc * sj[None, :, None]
    return acc.astype(np.float16).reshape(len(rows), -1)


def m_low_byte_codes(codes, books, scales, rows):
    # wide codes truncated to their low byte
    c = np.asarray(codes)
    return O.decode_rows((c.astype(np.int64) & 0xFF).astype(c.dtype), books, scales, rows)


def m_first_two_codebooks(codes, books, scales, rows):
    rows = np.asarray(rows)
    g = _gather(codes, books, rows)
    acc = g[0]
    for t in g[1:2]:
        acc = acc + t
    acc = acc * np.asarray(scales)[rows].astype(np.float32)[:, None, None]
    return acc.astype(np.float16).reshape(len(rows), -1)


def p_drop_last_column(x, w16):
    x = np.asarray(x)[:, :-1]
    w16 = np.asarray(w16)[:, :-1]
    return O.product(x, w16)


def p_transposed_rows(x, w16):
    y, b = O.product(x, w16)
    return y[:, ::-1].copy(), b[:, ::-1].copy()


def p_fp32_accumulate_in_fp16(x, w16):
    x64 = np.asarray(x).astype(np.float16)
    w = np.asarray(w16).astype(np.float16)
    y = np.zeros((x64.shape[0], w.shape[0]), dtype=np.float16)
    for i in range(w.shape[1]):
        y = (y + x64[:, i:i + 1] * w[None, :, i]).astype(np.float16)
    _, b = O.product(x, w16)
    return y.astype(np.float64), b


def u_msb_first(words, out, J, M, B):
    w = np.asarray(words, dtype=np.uint32)
    bits = np.unpackbits(w.view(np.uint8), bitorder="big")
    n = out * J * M
    codes = [int("".join(str(b) for b in bits[i * B:(i + 1) * B]), 2) for i in range(n)]
    return np.array(codes, dtype=np.uint8 if B == 8 else np.uint16).reshape(out, J, M)


def u_byte_aligned(words, out, J, M, B):
    # each code padded to whole bytes: the unpacked element layout read from the stream
    w = np.asarray(words, dtype=np.uint32).view(np.uint8)
    step = (B + 7) // 8
    n = out * J * M
    raw = np.zeros(n * step, dtype=np.uint8)
    raw[:min(n * step, w.size)] = w[:n * step]
    vals = raw.reshape(n, step).astype(np.uint32)
    codes = vals[:, 0] | (vals[:, 1] << 8 if step > 1 else 0)
    return (codes & ((1 << B) - 1)).astype(np.uint8 if B == 8 else np.uint16).reshape(out, J, M)


MUTANTS = {
    "swapped_codebooks": _impl(decode_rows=m_swapped_codebooks),
    "fp16_sum_then_scale": _impl(decode_rows=m_fp16_sum_then_scale),
    "no_scale": _impl(decode_rows=m_no_scale),
    "first_codebook_only": _impl(decode_rows=m_first_codebook_only),
    "strided_columns": _impl(decode_rows=m_strided_columns),
    "zero_initialised_sum": _impl(decode_rows=m_zero_init),
    "descending_codebook_order": _impl(decode_rows=m_descending_order),
    "flush_subnormals": _impl(decode_rows=m_flush_subnormals),
    "truncating_round": _impl(decode_rows=m_truncate_round),
    "scale_indexed_by_group": _impl(decode_rows=m_scale_by_group),
    "wide_codes_low_byte": _impl(decode_rows=m_low_byte_codes),
    "first_two_codebooks_only": _impl(decode_rows=m_first_two_codebooks),
    "product_drops_last_column": _impl(product=p_drop_last_column),
    "product_rows_reversed": _impl(product=p_transposed_rows),
    "product_accumulates_in_fp16": _impl(product=p_fp32_accumulate_in_fp16),
    "packed_codes_msb_first": _impl(unpack=u_msb_first),
    "packed_codes_byte_aligned": _impl(unpack=u_byte_aligned),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name):
    impl = MUTANTS[name]
    caught = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the planted mistake {name}"


# ---------------------------------------------------------------------------
# oracle plumbing
# ---------------------------------------------------------------------------
def test_decode_chunking_is_bit_neutral():
    codes, books, scales, _ = WL.small_case(37, 64, WL.S2x8, 1, seed=3)
    a = O.decode(codes, books, scales, chunk_rows=5)
    b = O.decode(codes, books, scales, chunk_rows=4096)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    rows = np.array([36, 0, 17])
    assert np.array_equal(O.decode_rows(codes, books, scales, rows).view(np.uint16),
                          a[rows].view(np.uint16))


def test_signed_code_storage_is_read_bitwise():
    codes, books, scales, x = WL.small_case(9, 32, WL.S1x16, 2, seed=4)
    signed = codes.view(np.int16)
    assert np.array_equal(O.decode(signed, books, scales).view(np.uint16),
                          O.decode(codes, books, scales).view(np.uint16))


def test_format_errors():
    codes, books, scales, _ = WL.small_case(4, 16, WL.S2x8, 1, seed=5)
    with pytest.raises(ValueError):
        O.check_format(codes[:, :, :1], books, scales)
    with pytest.raises(ValueError):
        O.check_format(codes, books.astype(np.float32), scales)
    with pytest.raises(ValueError):
        O.check_format(codes, books, scales[:3])


def test_within_tolerance_rejects_nan_and_large_error():
    y_ref = np.array([[1.0, 2.0, 3.0]])
    bound = np.array([[10.0, 10.0, 10.0]])
    ok = O.within_tolerance(np.array([[1.05, np.nan, 3.2]]), y_ref, bound)
    assert ok.tolist() == [[True, False, False]]


# ---------------------------------------------------------------------------
# generator statistics (the synthetic inputs have the stated distributions)
# ---------------------------------------------------------------------------
def test_generator_statistics():
    for scheme, M in ((WL.S2x8, 2), (WL.S1x16, 1)):
        codes, books, scales, x = WL.small_case(2048, 1024, scheme, 1, seed=99)
        w = O.decode(codes, books, scales).astype(np.float64)
        expected = 0.02 * np.sqrt(M) * np.sqrt(13.0 / 12.0)
        assert abs(w.std() / expected - 1) < 0.03, (scheme, w.std(), expected)
        hist = np.bincount(codes.reshape(-1).astype(np.int64), minlength=2 ** scheme.B)
        n = codes.size / 2 ** scheme.B
        chi2 = ((hist - n) ** 2 / n).sum()
        dof = 2 ** scheme.B - 1
        assert abs(chi2 - dof) < 6 * np.sqrt(2 * dof)
        assert scales.min() >= 0.5 and scales.max() <= 1.5
        assert abs(float(x.astype(np.float64).std()) - 1) < 0.1


def test_batch_variants_share_weights():
    layer = WL.WORKLOADS["llama2_7b_1x16"].layers[0]
    small = WL.Layer(layer.name, 64, 128, layer.scheme, layer.seed)
    x1 = WL.make_x(small, 1)
    x8 = WL.make_x(small, 8)
    assert np.array_equal(x1[0], x8[0])
