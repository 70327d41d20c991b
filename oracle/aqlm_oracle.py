"""CPU oracle for the additive multi-codebook quantized linear layer (AQLM).

TEST INFRASTRUCTURE ONLY. This module exists to check the HIP library. Only
the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the library never calls it and never falls back to it. It imports numpy
and nothing else: no code is shared with the HIP kernels or their binding.

What it computes, and where that comes from:

* The representation. A layer's weight matrix is stored as sums of learned
  codebook vectors: every weight vector is the sum of one codeword chosen
  from each of M codebooks ("Additive quantization that actually survives
  one-bit weights", section "What it does"; "AQLM (additive / multi-codebook
  quantization)", field "Activation scheme"; "Extreme Compression of Large
  Language Models via Additive Quantization" paper record, method paragraph).
  The pages name 8- and 16-dimensional codewords ("Additive quantization that
  actually survives one-bit weights", "Key highlights" and "Caveats").

* Readings where the pages are silent (each is listed with its reason in the
  design notes of the repository):
    - a weight group is g consecutive input columns of one output row:
      group j of row o covers columns j*g .. j*g+g-1, element k <-> column j*g+k;
    - codes are unsigned indices laid out [out, in/g, M] (m fastest), one
      per storage element (uint8 for B = 8, uint16 for 8 < B <= 16, no bit
      packing), codebooks [M, 2**B, g], one float16 scale per output row;
    - decode: the M codewords are widened to float32 and summed in ascending
      m, the accumulator starting from the m = 0 codeword (not from +0.0);
      the sum is multiplied by the row's scale in float32; the result is
      rounded once, to nearest-even, to float16 (subnormals kept, overflow
      to infinity);
    - activations stay float16 and the product y = x . W^T is accumulated in
      float32 or better ("AQLM (additive / multi-codebook quantization)",
      fields "Bits" and "Activation scheme": weight-only, activations fp16).

* The product reference is the plain definition y[b, o] = sum_i x[b, i] W[o, i]
  evaluated in float64 on the float16 decoded weights, together with
  bound[b, o] = sum_i |x[b, i] W[o, i]|, the scale for the acceptance
  tolerance |y - y_ref| <= rel * bound.

* Storage cost: bits per weight of the packed format, M*B/g for the codes
  plus the codebooks and the per-row scales spread over the out*in weights
  (the pages call the effective bit width non-integer and give about 8x
  compression at 2 bits per weight: "AQLM (additive / multi-codebook
  quantization)", notes; paper record, claims paragraph).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "check_format", "decode", "decode_rows", "product", "forward",
    "forward_rows", "within_tolerance", "bits_per_weight", "stored_bits_per_weight",
    "packed_bits_per_weight", "unpack_codes",
]


def unpack_codes(words, out, J, M, B):
    """Codes [out, J, M] from their bit-packed storage: code i of the flattened
    array is bits i*B .. i*B+B-1 of the little-endian 32-bit word stream,
    least significant bit first (the library's reading of a packed format the
    pages leave unstated)."""
    w = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    n = out * J * M
    if w.size * 32 < n * B:
        raise ValueError("packed stream too short")
    bit = np.arange(n, dtype=np.uint64) * np.uint64(B)
    k = (bit >> np.uint64(5)).astype(np.int64)
    nxt = np.where(k + 1 < w.size, w[np.minimum(k + 1, w.size - 1)], np.uint64(0))
    win = w[k] | (nxt << np.uint64(32))
    codes = (win >> (bit & np.uint64(31))) & np.uint64((1 << B) - 1)
    return codes.astype(np.uint8 if B == 8 else np.uint16).reshape(out, J, M)


def check_format(codes, codebooks, scales):
    """Validate the packed triple and return (out, in, M, B, g)."""
    codes = np.asarray(codes)
    codebooks = np.asarray(codebooks)
    scales = np.asarray(scales)
    if codes.ndim != 3 or codebooks.ndim != 3 or scales.ndim != 1:
        raise ValueError("codes must be [out, in/g, M], codebooks [M, 2**B, g], scales [out]")
    out, J, M = codes.shape
    Mc, ncode, g = codebooks.shape
    if Mc != M:
        raise ValueError("codes and codebooks disagree on the number of codebooks")
    if ncode & (ncode - 1) or ncode < 2:
        raise ValueError("codebook size must be a power of two")
    B = ncode.bit_length() - 1
    if codebooks.dtype != np.float16 or scales.dtype != np.float16:
        raise ValueError("codebooks and scales must be float16")
    if codes.dtype.kind not in "ui":
        raise ValueError("codes must be integers")
    if scales.shape[0] != out:
        raise ValueError("one scale per output row")
    return out, J * g, M, B, g


def _unsigned(codes: np.ndarray, B: int) -> np.ndarray:
    """Read codes as unsigned B-bit indices (signed storage is reinterpreted bitwise)."""
    if codes.dtype.kind == "i":
        codes = codes.view(np.dtype(f"u{codes.dtype.itemsize}"))
    idx = codes.astype(np.int64)
    if idx.size and int(idx.max()) >= (1 << B):
        raise ValueError("code out of range for the codebook size")
    return idx


def decode_rows(codes, codebooks, scales, rows) -> np.ndarray:
    """Decoded float16 weights W[rows, :] (see the module docstring for the rule)."""
    out, n_in, M, B, g = check_format(codes, codebooks, scales)
    rows = np.asarray(rows, dtype=np.int64)
    idx = _unsigned(np.asarray(codes)[rows], B)              # [r, J, M]
    books32 = np.asarray(codebooks).astype(np.float32)       # exact widening
    acc = books32[0][idx[:, :, 0]]                           # [r, J, g], m = 0 term
    for m in range(1, M):                                    # ascending m, fp32 adds
        acc = acc + books32[m][idx[:, :, m]]
    s32 = np.asarray(scales)[rows].astype(np.float32)
    acc = acc * s32[:, None, None]                           # one fp32 multiply
    w16 = acc.astype(np.float16)                             # one RNE round to fp16
    return w16.reshape(rows.shape[0], n_in)


def decode(codes, codebooks, scales, chunk_rows: int = 2048) -> np.ndarray:
    """Decoded float16 weight matrix W [out, in], built in row chunks."""
    out, n_in, _, _, _ = check_format(codes, codebooks, scales)
    w = np.empty((out, n_in), dtype=np.float16)
    for r0 in range(0, out, chunk_rows):
        r1 = min(out, r0 + chunk_rows)
        w[r0:r1] = decode_rows(codes, codebooks, scales, np.arange(r0, r1))
    return w


def product(x, w16):
    """y_ref = x . W^T in float64 and bound = |x| . |W|^T (both [batch, out])."""
    x64 = np.asarray(x).astype(np.float64)
    w64 = np.asarray(w16).astype(np.float64)
    if x64.ndim != 2 or w64.ndim != 2 or x64.shape[1] != w64.shape[1]:
        raise ValueError("x must be [batch, in] and W [out, in]")
    y_ref = x64 @ w64.T
    bound = np.abs(x64) @ np.abs(w64).T
    return y_ref, bound


def forward(x, codes, codebooks, scales, chunk_rows: int = 2048):
    """(y_ref, bound) of the quantized layer applied to x [batch, in]."""
    out = np.asarray(codes).shape[0]
    x = np.asarray(x)
    y_ref = np.empty((x.shape[0], out), dtype=np.float64)
    bound = np.empty_like(y_ref)
    for r0 in range(0, out, chunk_rows):
        r1 = min(out, r0 + chunk_rows)
        w = decode_rows(codes, codebooks, scales, np.arange(r0, r1))
        y_ref[:, r0:r1], bound[:, r0:r1] = product(x, w)
    return y_ref, bound


def forward_rows(x, codes, codebooks, scales, rows):
    """(y_ref, bound) for the given output rows only: columns follow `rows`."""
    w = decode_rows(codes, codebooks, scales, rows)
    return product(x, w)


def within_tolerance(y, y_ref, bound, rel: float = 1e-2) -> np.ndarray:
    """Elementwise acceptance: finite and |y - y_ref| <= rel * bound."""
    y64 = np.asarray(y).astype(np.float64)
    ok = np.isfinite(y64) & (np.abs(y64 - y_ref) <= rel * bound)
    return ok


def bits_per_weight(out_features: int, in_features: int, M: int, B: int, g: int) -> float:
    """Closed form: code bits M*B/g, plus 16-bit codebooks and per-row scales amortised."""
    return (M * B / g
            + 16.0 * M * (2 ** B) * g / (out_features * in_features)
            + 16.0 / in_features)


def stored_bits_per_weight(out_features: int, in_features: int, M: int, B: int, g: int) -> float:
    """As bits_per_weight, but with each code in its storage element: one byte
    per code for B <= 8, two bytes for 8 < B <= 16 (codes are not bit-packed)."""
    code_bits = 8 * ((B + 7) // 8)
    return (M * code_bits / g
            + 16.0 * M * (2 ** B) * g / (out_features * in_features)
            + 16.0 / in_features)


def packed_bits_per_weight(codes, codebooks, scales) -> float:
    """Bits per weight measured from the stored arrays' sizes."""
    out, n_in, _, _, _ = check_format(codes, codebooks, scales)
    total = np.asarray(codes).nbytes + np.asarray(codebooks).nbytes + np.asarray(scales).nbytes
    return 8.0 * total / (out * n_in)
