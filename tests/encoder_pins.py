"""Pins of the toy-encoder oracle (oracle/encoder_oracle.py) to facts that do
not come from the oracle itself: hand-worked values, exact arithmetic on
dyadic inputs, brute-force search in float64 with the float32 rounding bound,
the plain mean, k-means on well-separated clusters with known answers, the
Lloyd descent property, and round trips whose error is fixed by the float16
format. Each pin takes an implementation namespace E with the oracle's
functions, so that copies carrying planted mistakes can be run through them.
"""
import numpy as np

FP32_EPS = 2.0 ** -23


def _rng(seed):
    return np.random.default_rng(seed)


def pin_row_scales_hand_worked(E):
    W = np.array([[0.5, -2.0, 1.0, 0.0], [0, 0, 0, 0], [-0.25, 0.125, 0.0, -0.0]], dtype=np.float16)
    s = E.row_scales(W)
    assert s.dtype == np.float16
    assert np.array_equal(s.astype(np.float32), np.array([2.0, 1.0, 0.25], dtype=np.float32))


def pin_normalize_hand_worked(E):
    W = np.array([[0.5, -2.0, 1.0, 0.25], [3.0, 1.5, -0.75, 0.0]], dtype=np.float16)
    s = np.array([2.0, 3.0], dtype=np.float16)
    v = E.normalize(W, s, 2)
    want = np.array([[0.25, -1.0], [0.5, 0.125], [1.0, 0.5], [-0.25, 0.0]], dtype=np.float32)
    assert v.shape == (4, 2) and v.dtype == np.float32
    assert np.array_equal(v, want)


def pin_normalize_is_correctly_rounded_quotient(E):
    W = _rng(1).normal(0, 0.02, size=(5, 16)).astype(np.float16)
    s = np.abs(W).max(axis=1).astype(np.float16)
    v = E.normalize(W, s, 8).reshape(5, 16).astype(np.float64)
    exact = W.astype(np.float64) / s.astype(np.float64)[:, None]
    assert np.all(np.abs(v - exact) <= 0.5 * FP32_EPS * np.abs(exact) + 1e-45)
    assert np.all(np.abs(v) <= 1.0)


def pin_sq_errors_exact_on_dyadics(E):
    # multiples of 1/64 in [-2, 2]: every difference, square and partial sum is exact
    r = _rng(2)
    v = (r.integers(-128, 129, size=(6, 8)) / 64.0).astype(np.float32)
    c = (r.integers(-128, 129, size=(9, 8)) / 64.0).astype(np.float32)
    exact = ((v.astype(np.float64)[:, None, :] - c.astype(np.float64)[None, :, :]) ** 2).sum(-1)
    assert np.array_equal(E.sq_errors(v, c).astype(np.float64), exact)


def pin_sq_errors_within_rounding_bound(E):
    r = _rng(3)
    v = r.normal(0, 0.3, size=(20, 16)).astype(np.float32)
    c = r.normal(0, 0.3, size=(11, 16)).astype(np.float32)
    exact = ((v.astype(np.float64)[:, None, :] - c.astype(np.float64)[None, :, :]) ** 2).sum(-1)
    d = E.sq_errors(v, c).astype(np.float64)
    assert np.all(np.abs(d - exact) <= 20 * FP32_EPS * exact)


def pin_assign_brute_force(E):
    r = _rng(4)
    v = r.normal(0, 0.2, size=(200, 8)).astype(np.float32)
    c = r.normal(0, 0.2, size=(37, 8)).astype(np.float32)
    codes, best = E.assign(v, c)
    ex = ((v.astype(np.float64)[:, None, :] - c.astype(np.float64)[None, :, :]) ** 2).sum(-1)
    order = np.sort(ex, axis=1)
    clear = order[:, 1] - order[:, 0] > 40 * FP32_EPS * order[:, 1]
    assert clear.sum() > 150
    assert np.array_equal(codes[clear], np.argmin(ex, axis=1)[clear])
    assert np.all(np.abs(best.astype(np.float64) - ex[np.arange(200), codes]) <= 20 * FP32_EPS * ex[np.arange(200), codes] + 1e-30)
    for i in range(200):  # never worse than the exact optimum beyond rounding
        assert ex[i, codes[i]] <= order[i, 0] * (1 + 40 * FP32_EPS) + 1e-30


def pin_assign_ties_take_lowest_index(E):
    c = np.array([[1, 0, 0, 0, 0, 0, 0, 0], [0, 0.5, 0, 0, 0, 0, 0, 0], [0.25, 0, 0, 0, 0, 0, 0, 0],
                  [0, 0.5, 0, 0, 0, 0, 0, 0], [0.25, 0, 0, 0, 0, 0, 0, 0]], dtype=np.float32)
    v = np.array([[0.25, 0, 0, 0, 0, 0, 0, 0], [0, 0.5, 0, 0, 0, 0, 0, 0],
                  [0.125, 0.25, 0, 0, 0, 0, 0, 0]], dtype=np.float32)
    codes, _ = E.assign(v, c)
    # v0 equals rows 2 and 4; v1 equals rows 1 and 3; v2 is at squared distance
    # 1/64 + 1/16 from rows 1, 2, 3 and 4 alike
    assert codes.tolist() == [2, 1, 1]


def pin_update_is_the_mean(E):
    r = _rng(5)
    v = (r.integers(-512, 513, size=(40, 8)) / 1024.0).astype(np.float32)
    codes = r.integers(0, 6, size=40)
    codes[codes == 4] = 0            # cluster 4 stays empty
    old = np.full((6, 8), 7.0, dtype=np.float32)
    new = E.update_centroids(v, codes, old)
    for k in range(6):
        members = v[codes == k].astype(np.float64)
        if len(members) == 0:
            assert np.array_equal(new[k], old[k])
        else:
            mean = members.mean(axis=0)
            assert np.all(np.abs(new[k].astype(np.float64) - mean) <= 0.5 * FP32_EPS * np.abs(mean) + 1e-12)


def pin_update_quantises_to_fixed_point(E):
    # two vectors whose mean needs more than 24 fractional bits: the fixed-point
    # sum rounds each component to a multiple of 2^-24 first
    tiny = np.float32(2.0 ** -26)
    v = np.array([[tiny] * 8, [0.0] * 8], dtype=np.float32)
    new = E.update_centroids(v, np.array([0, 0]), np.zeros((1, 8), dtype=np.float32))
    assert np.all(new == 0.0)        # 2^-26 rounds to 0 in 2^-24 steps
    v = np.array([[3 * 2.0 ** -25] * 8, [0.0] * 8], dtype=np.float32)
    new = E.update_centroids(v, np.array([0, 0]), np.zeros((1, 8), dtype=np.float32))
    assert np.all(new == np.float32(2.0 ** -24))  # 3*2^-25 = 1.5*2^-24 -> 2*2^-24 (ties to even), mean 2^-24


def _separated_clusters(seed, K=4, per=25, g=8):
    r = _rng(seed)
    centers = np.zeros((K, g))
    for k in range(K):
        centers[k, k % g] = 0.5 if k < g else -0.5
    labels = np.repeat(np.arange(K), per)
    pts = centers[labels] + r.uniform(-0.01, 0.01, size=(K * per, g))
    perm = r.permutation(K * per)
    return pts[perm].astype(np.float32), labels[perm], centers


def pin_kmeans_recovers_separated_clusters(E):
    v, labels, _ = _separated_clusters(6)
    init = np.array([np.flatnonzero(labels == k)[0] for k in range(4)])
    for iters in (1, 3):
        cents = E.kmeans(v, init, iters)
        codes, _ = E.assign(v, cents)
        assert np.array_equal(codes, labels)
        for k in range(4):
            mean = v[labels == k].astype(np.float64).mean(axis=0)
            assert np.all(np.abs(cents[k] - mean) <= 1e-6)


def pin_kmeans_objective_never_rises(E):
    r = _rng(7)
    v = r.normal(0, 0.3, size=(500, 8)).astype(np.float32)
    init = r.choice(500, size=16, replace=False)
    prev = None
    for iters in range(6):
        cents = E.kmeans(v, init, iters).astype(np.float64)
        obj = ((v.astype(np.float64)[:, None, :] - cents[None]) ** 2).sum(-1).min(axis=1).sum()
        if prev is not None:
            assert obj <= prev * (1 + 1e-6)
        prev = obj
    assert prev < ((v.astype(np.float64)[:, None, :] - v[init].astype(np.float64)[None]) ** 2
                   ).sum(-1).min(axis=1).sum()


def pin_encode_each_vector_its_own_codeword(E):
    # fewer group vectors than codewords and every vector a starting point:
    # k-means keeps each vector as its own centroid, so the only error left is
    # the float16 rounding of the codeword and of scale * codeword
    W = _rng(8).normal(0, 0.02, size=(6, 32)).astype(np.float16)
    n = W.size // 8
    init = [np.resize(np.arange(n), 256)]
    codes, books, scales = E.encode(W, 1, 8, 8, 2, init)
    from oracle.aqlm_oracle import decode
    Wq = decode(codes, books, scales).astype(np.float64)
    ulp = np.spacing(np.abs(W).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(Wq - W.astype(np.float64)) <= 2 * ulp)
    assert np.array_equal(scales, np.abs(W).max(axis=1))


def pin_encode_codes_are_greedy_nearest(E):
    W = _rng(9).normal(0, 0.02, size=(16, 64)).astype(np.float16)
    n = W.size // 8
    r = _rng(10)
    init = [r.choice(n, 32, replace=False).astype(np.int64) for _ in range(2)]
    # B = 8 needs 256 starting vectors: repeat the 32 (the duplicates stay unused)
    init = [np.resize(i, 256) for i in init]
    codes, books, scales = E.encode(W, 2, 8, 8, 3, init)
    assert codes.shape == (16, 8, 2) and codes.dtype == np.uint8 and books.dtype == np.float16
    res = (W.astype(np.float64) / scales.astype(np.float64)[:, None]).reshape(-1, 8)
    for m in range(2):
        cb = books[m].astype(np.float64)
        ex = ((res[:, None, :] - cb[None]) ** 2).sum(-1)
        order = np.sort(ex, axis=1)
        clear = order[:, 1] - order[:, 0] > 1e-5 * order[:, 1]
        got = codes.reshape(-1, 2)[:, m].astype(np.int64)
        assert clear.sum() > n // 2
        assert np.array_equal(got[clear], np.argmin(ex, axis=1)[clear])
        res = res - cb[got]


def pin_encode_second_codebook_helps(E):
    W = _rng(11).normal(0, 0.02, size=(32, 128)).astype(np.float16)
    n = W.size // 8
    init = [np.resize(_rng(12 + m).permutation(n), 256) for m in range(2)]
    from oracle.aqlm_oracle import decode
    errs = []
    for M in (1, 2):
        codes, books, scales = E.encode(W, M, 8, 8, 4, init[:M])
        errs.append(np.mean((decode(codes, books, scales).astype(np.float64) - W.astype(np.float64)) ** 2))
    assert errs[1] < 0.7 * errs[0]


ALL_PINS = [
    pin_row_scales_hand_worked, pin_normalize_hand_worked, pin_normalize_is_correctly_rounded_quotient,
    pin_sq_errors_exact_on_dyadics, pin_sq_errors_within_rounding_bound, pin_assign_brute_force,
    pin_assign_ties_take_lowest_index, pin_update_is_the_mean, pin_update_quantises_to_fixed_point,
    pin_kmeans_recovers_separated_clusters, pin_kmeans_objective_never_rises,
    pin_encode_each_vector_its_own_codeword, pin_encode_codes_are_greedy_nearest,
    pin_encode_second_codebook_helps,
]
