"""CPU oracle of the toy AQLM encoder: row scales, residual k-means codebooks
and greedy code assignment under the plain (unweighted) squared error.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the
smoke check and the benchmark's CPU-baseline leg may use it; the library
never does. numpy only; no code is shared with the HIP kernels.

Where it comes from. The pages describe AQLM as classic additive
quantization (codes chosen by nearest-neighbour style search over sums of
codewords) adapted to LLM weights, with codebooks and codes learned by beam
search and Adam, and report that a residual K-means initialisation of the
codebooks beats a random one ("Extreme Compression of Large Language Models
via Additive Quantization" summary: "Approach"; table "Measured effects
reported in the paper", row on residual K-means initialisation; "Limitations"
on beam search and the Adam codebook update). This toy encoder keeps the
parts that need no calibration data and no training: the input-aware
objective, the Adam updates and the fine-tuning are left out, and the code
assignment is greedy (a beam of width one).

Readings where the pages are silent (each listed in the design notes):
  * row scale: the largest magnitude of the row, as float16 (exact), or 1 for
    a row of zeros; the row is divided by it in float32 (correctly rounded),
    so every normalised weight lies in [-1, 1];
  * group vectors: group j of row o is the g consecutive normalised weights
    j*g .. j*g+g-1, vector index o * (in / g) + j;
  * squared error of vector v against codeword c: float32, terms (v_k - c_k)^2
    added in ascending k, each operation rounded to float32 (no fused
    multiply-add); the nearest codeword is the one with the smallest error,
    the lowest index on a tie. The GPU takes the same decision in the same
    precision, so codes compare exactly;
  * k-means (Lloyd): K = 2**B initial centroids are the vectors at K seeded
    distinct indices (an input: the draw itself lives with the seeded input
    generators); each iteration assigns every vector to its nearest centroid,
    then moves each centroid to the mean of its vectors. The mean is taken
    exactly in 24-bit fixed point: each component is rounded to a multiple of
    2**-24 (nearest, ties to even), the integer sums are exact, and the sum
    times 2**-24 divided by the count is rounded once to float32; a centroid
    with no vectors keeps its place;
  * residual codebooks: codebook m is learned by k-means on the residuals left
    by codebooks 0 .. m-1; after its k-means it is rounded to float16 (the
    packed format's precision), the codes of codebook m are the nearest
    rounded codewords, and the residual drops that codeword (float32
    subtraction) before codebook m + 1 is learned.
"""
from __future__ import annotations

import numpy as np

from .aqlm_oracle import decode

__all__ = ["row_scales", "normalize", "sq_errors", "assign", "update_centroids", "kmeans",
           "encode", "reconstruction_mse", "FIXED_POINT_BITS"]

FIXED_POINT_BITS = 24


def row_scales(W16):
    """Per-row scale: max |W[o, :]| (float16, exact), 1 for an all-zero row."""
    W16 = np.asarray(W16, dtype=np.float16)
    s = np.abs(W16).max(axis=1)
    return np.where(s == 0, np.float16(1), s).astype(np.float16)


def normalize(W16, scales, g):
    """Group vectors [out * in/g, g] float32: W / scale, correctly rounded."""
    W = np.asarray(W16, dtype=np.float16).astype(np.float32)
    s = np.asarray(scales, dtype=np.float16).astype(np.float32)
    v = W / s[:, None]
    return v.reshape(-1, g)


def sq_errors(vecs, cents):
    """float32 squared errors [n, K], terms added in ascending k, no fusion."""
    vecs = np.asarray(vecs, dtype=np.float32)
    cents = np.asarray(cents, dtype=np.float32)
    d = vecs[:, None, 0] - cents[None, :, 0]
    acc = d * d
    for k in range(1, vecs.shape[1]):
        d = vecs[:, None, k] - cents[None, :, k]
        acc = acc + d * d
    return acc


def assign(vecs, cents, chunk=4096):
    """Nearest centroid of every vector (lowest index on ties) and its error."""
    vecs = np.asarray(vecs, dtype=np.float32)
    n = vecs.shape[0]
    codes = np.empty(n, dtype=np.int64)
    best = np.empty(n, dtype=np.float32)
    for i in range(0, n, chunk):
        e = sq_errors(vecs[i:i + chunk], cents)
        codes[i:i + chunk] = np.argmin(e, axis=1)  # first minimum = lowest index
        best[i:i + chunk] = e[np.arange(e.shape[0]), codes[i:i + chunk]]
    return codes, best


def update_centroids(vecs, codes, cents):
    """Centroid = mean of its vectors, exact in 24-bit fixed point, then
    rounded once to float32; empty clusters keep their centroid."""
    vecs = np.asarray(vecs, dtype=np.float32)
    K, g = cents.shape
    q = np.rint(vecs.astype(np.float64) * 2.0 ** FIXED_POINT_BITS).astype(np.int64)
    sums = np.zeros((K, g), dtype=np.int64)
    np.add.at(sums, codes, q)
    counts = np.bincount(codes, minlength=K).astype(np.int64)
    new = np.array(cents, dtype=np.float32, copy=True)
    hit = counts > 0
    mean = (sums[hit].astype(np.float64) * 2.0 ** -FIXED_POINT_BITS) / counts[hit][:, None]
    new[hit] = mean.astype(np.float32)
    return new


def kmeans(vecs, init_idx, iters):
    """Lloyd iterations from the vectors at init_idx; returns float32 centroids."""
    vecs = np.asarray(vecs, dtype=np.float32)
    cents = vecs[np.asarray(init_idx)].copy()
    for _ in range(iters):
        codes, _ = assign(vecs, cents)
        cents = update_centroids(vecs, codes, cents)
    return cents


def encode(W16, M, B, g, iters, init_indices):
    """Toy encoder: (codes [out, in/g, M], codebooks [M, 2**B, g] float16,
    scales [out] float16). init_indices[m] are the K seeded starting vectors
    of codebook m's k-means."""
    W16 = np.asarray(W16, dtype=np.float16)
    out, n_in = W16.shape
    if n_in % g:
        raise ValueError("in must be a multiple of g")
    scales = row_scales(W16)
    r = normalize(W16, scales, g)
    K = 2 ** B
    codes = np.empty((r.shape[0], M), dtype=np.uint8 if B == 8 else np.uint16)
    books = np.empty((M, K, g), dtype=np.float16)
    for m in range(M):
        cents = kmeans(r, init_indices[m], iters)
        books[m] = cents.astype(np.float16)
        cr = books[m].astype(np.float32)
        c, _ = assign(r, cr)
        codes[:, m] = c
        r = r - cr[c]
    return codes.reshape(out, n_in // g, M), books, scales


def reconstruction_mse(W16, codes, codebooks, scales):
    """Mean squared difference (float64) between W and the decoded layer."""
    W = np.asarray(W16, dtype=np.float16).astype(np.float64)
    Wq = decode(codes, codebooks, scales).astype(np.float64)
    return float(np.mean((Wq - W) ** 2))
