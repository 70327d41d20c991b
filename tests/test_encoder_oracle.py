"""Toy-encoder oracle pins (CPU only), and planted mistakes that the pins must
reject."""
import types

import numpy as np
import pytest

import encoder_pins as P
from oracle import encoder_oracle as E


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_encoder_oracle_pin(pin):
    pin(E)


def _impl(**over):
    """A copy of the encoder oracle with some functions replaced; the others
    are rebuilt on top of the replacements in the oracle's own order."""
    ns = types.SimpleNamespace()
    ns.row_scales = over.get("row_scales", E.row_scales)
    ns.normalize = over.get("normalize", E.normalize)
    ns.sq_errors = over.get("sq_errors", E.sq_errors)

    def assign(vecs, cents, chunk=4096):
        e = ns.sq_errors(vecs, cents)
        c = np.argmin(e, axis=1)
        return c, e[np.arange(e.shape[0]), c]
    ns.assign = over.get("assign", assign)
    ns.update_centroids = over.get("update_centroids", E.update_centroids)

    def kmeans(vecs, init_idx, iters):
        cents = np.asarray(vecs, dtype=np.float32)[np.asarray(init_idx)].copy()
        for _ in range(iters):
            codes, _ = ns.assign(vecs, cents)
            cents = ns.update_centroids(vecs, codes, cents)
        return cents
    ns.kmeans = over.get("kmeans", kmeans)

    def encode(W16, M, B, g, iters, init_indices, residual=True):
        W16 = np.asarray(W16, dtype=np.float16)
        out, n_in = W16.shape
        scales = ns.row_scales(W16)
        v = ns.normalize(W16, scales, g)
        r = v
        codes = np.empty((r.shape[0], M), dtype=np.uint8 if B == 8 else np.uint16)
        books = np.empty((M, 2 ** B, g), dtype=np.float16)
        for m in range(M):
            cents = ns.kmeans(r if residual else v, init_indices[m], iters)
            books[m] = cents.astype(np.float16)
            cr = books[m].astype(np.float32)
            c, _ = ns.assign(r, cr)
            codes[:, m] = c
            r = r - cr[c]
        return codes.reshape(out, n_in // g, M), books, scales
    ns.encode = over.get("encode", encode)
    return ns


def m_mean_abs_scale(W16):
    s = np.abs(np.asarray(W16, dtype=np.float32)).mean(axis=1)
    return np.where(s == 0, 1, s).astype(np.float16)


def m_multiply_not_divide(W16, scales, g):
    return (np.asarray(W16, np.float32) * np.asarray(scales, np.float32)[:, None]).reshape(-1, g)


def m_column_major_groups(W16, scales, g):
    v = np.asarray(W16, np.float32) / np.asarray(scales, np.float32)[:, None]
    return v.T.reshape(-1, g)


def m_l1_distance(vecs, cents):
    return np.abs(np.asarray(vecs, np.float32)[:, None, :] - np.asarray(cents, np.float32)[None]).sum(-1)


def m_dropped_last_dim(vecs, cents):
    return E.sq_errors(np.asarray(vecs)[:, :-1], np.asarray(cents)[:, :-1])


def m_highest_index_on_ties(vecs, cents, chunk=4096):
    e = E.sq_errors(vecs, cents)
    c = e.shape[1] - 1 - np.argmin(e[:, ::-1], axis=1)
    return c, e[np.arange(e.shape[0]), c]


def m_first_member(vecs, codes, cents):
    new = np.array(cents, dtype=np.float32, copy=True)
    for k in range(new.shape[0]):
        idx = np.flatnonzero(codes == k)
        if len(idx):
            new[k] = vecs[idx[0]]
    return new


def m_empty_to_zero(vecs, codes, cents):
    new = E.update_centroids(vecs, codes, cents)
    counts = np.bincount(codes, minlength=new.shape[0])
    new[counts == 0] = 0
    return new


def m_sum_not_mean(vecs, codes, cents):
    new = np.array(cents, dtype=np.float32, copy=True)
    for k in range(new.shape[0]):
        idx = codes == k
        if idx.any():
            new[k] = np.asarray(vecs, np.float64)[idx].sum(axis=0)
    return new


def m_no_update(vecs, init_idx, iters):
    return np.asarray(vecs, dtype=np.float32)[np.asarray(init_idx)].copy()


def _no_residual_encode():
    base = _impl()

    def encode(W16, M, B, g, iters, init_indices):
        return base.encode(W16, M, B, g, iters, init_indices, residual=False)
    return encode


MUTANTS = {
    "scale_is_mean_magnitude": _impl(row_scales=m_mean_abs_scale),
    "normalise_multiplies": _impl(normalize=m_multiply_not_divide),
    "groups_taken_down_columns": _impl(normalize=m_column_major_groups),
    "l1_distance": _impl(sq_errors=m_l1_distance),
    "distance_drops_last_dimension": _impl(sq_errors=m_dropped_last_dim),
    "ties_take_highest_index": _impl(assign=m_highest_index_on_ties),
    "centroid_is_first_member": _impl(update_centroids=m_first_member),
    "empty_cluster_reset_to_zero": _impl(update_centroids=m_empty_to_zero),
    "centroid_is_sum": _impl(update_centroids=m_sum_not_mean),
    "kmeans_never_updates": _impl(kmeans=m_no_update),
    "every_codebook_learned_on_the_weights": _impl(encode=_no_residual_encode()),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_encoder_pins_reject_planted_mistake(name):
    impl = MUTANTS[name]
    caught = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the planted mistake {name}"


def test_init_indices_are_distinct_or_cover_every_vector():
    from additive_codebook_matmul_amd import workloads as WL
    a = WL.kmeans_init_indices(1000, 256, 2, seed=3)
    assert len(a) == 2 and all(len(np.unique(i)) == 256 and i.max() < 1000 for i in a)
    b = WL.kmeans_init_indices(100, 256, 1, seed=3)[0]
    assert set(b.tolist()) == set(range(100)) and len(b) == 256
