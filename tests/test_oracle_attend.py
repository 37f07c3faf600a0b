"""Pins of the oracle's compensated attention and the whole path (CPU only).

Expected values come from torch's own scaled_dot_product_attention (dense
softmax attention, fp64 on the CPU) in the cases where the method must
reduce to it: everything selected (density 1), keys and values constant in
every key cluster, singleton key clusters. Jensen's inequality and
permutation equivariance pin the compensation term's direction and indexing.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp
import torch

from oracle import svgear_oracle as O


def sdpa(q, k, v, scale):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), scale=scale)[0, 0].numpy()


def _setup(rng, n, d, cq, ck, spread=1.0):
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d)) * spread
    v = rng.standard_normal((n, d))
    lq = rng.integers(0, cq, n).astype(np.int32)
    lk = rng.integers(0, ck, n).astype(np.int32)
    lk[lk == 1] = 2                                     # key cluster 1 empty
    pq, qo = O.permute(lq, cq)
    pk, ko = O.permute(lk, ck)
    return q, k, v, pq, qo, pk, ko


def _attend_perm(q, k, v, pq, qo, pk, ko, mask, scale):
    qp, kp, vp = O.gather(q, pq), O.gather(k, pk), O.gather(v, pk)
    kc, vc = O.segment_means(kp, ko), O.segment_means(vp, ko)
    return O.unpermute(O.attend(qp, kp, vp, qo, ko, kc, vc, mask, scale), pq)


def test_density_one_is_dense_attention():
    rng = np.random.default_rng(1)
    q, k, v, pq, qo, pk, ko = _setup(rng, 300, 16, 7, 11)
    mask = np.ones((7, 11), dtype=np.uint8)
    got = _attend_perm(q, k, v, pq, qo, pk, ko, mask, 0.25)
    np.testing.assert_allclose(got, sdpa(q, k, v, 0.25), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(O.dense_attention(q, k, v, 0.25), sdpa(q, k, v, 0.25),
                               rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("frac", [0.0, 0.3, 0.7])
def test_constant_clusters_make_compensation_exact(frac):
    # keys and values identical inside every key cluster: the centroid term is
    # exact, so any selection gives dense attention.
    rng = np.random.default_rng(2)
    q, k, v, pq, qo, pk, ko = _setup(rng, 240, 8, 5, 9)
    lk = np.empty(240, dtype=np.int64)
    lk[pk] = np.repeat(np.arange(9), np.diff(ko))
    kpts, vpts = rng.standard_normal((9, 8)), rng.standard_normal((9, 8))
    k, v = kpts[lk], vpts[lk]
    mask = (rng.random((5, 9)) < frac).astype(np.uint8)
    got = _attend_perm(q, k, v, pq, qo, pk, ko, mask, 0.35)
    np.testing.assert_allclose(got, sdpa(q, k, v, 0.35), rtol=1e-11, atol=1e-12)


def test_singleton_key_clusters_are_dense_at_any_selection():
    rng = np.random.default_rng(3)
    n = 64
    q, k, v = (rng.standard_normal((n, 8)) for _ in range(3))
    lq = rng.integers(0, 4, n).astype(np.int32)
    pq, qo = O.permute(lq, 4)
    pk, ko = O.permute(np.arange(n, dtype=np.int32), n)
    mask = (rng.random((4, n)) < 0.2).astype(np.uint8)
    got = _attend_perm(q, k, v, pq, qo, pk, ko, mask, 0.3)
    np.testing.assert_allclose(got, sdpa(q, k, v, 0.3), rtol=1e-11, atol=1e-12)


def test_density_zero_is_centroid_softmax_with_log_count_bias():
    # nothing selected: each non-empty key cluster acts as one key k-bar with
    # value v-bar repeated |k_c| times -> dense attention over the expanded
    # centroid table.
    rng = np.random.default_rng(4)
    q, k, v, pq, qo, pk, ko = _setup(rng, 200, 8, 6, 10)
    mask = np.zeros((6, 10), dtype=np.uint8)
    got = _attend_perm(q, k, v, pq, qo, pk, ko, mask, 0.5)
    kp, vp = O.gather(k, pk), O.gather(v, pk)
    kc, vc = O.segment_means(kp, ko), O.segment_means(vp, ko)
    counts = np.diff(ko)
    kexp, vexp = np.repeat(kc, counts, axis=0), np.repeat(vc, counts, axis=0)
    np.testing.assert_allclose(got, sdpa(q, kexp, vexp, 0.5), rtol=1e-11, atol=1e-12)


def test_jensen_centroid_mass_below_block_mass():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((50, 8))
    for _ in range(10):
        blk = rng.standard_normal((int(rng.integers(2, 20)), 8)) * 2
        lhs = blk.shape[0] * np.exp(0.4 * q @ blk.mean(axis=0))
        rhs = np.exp(0.4 * q @ blk.T).sum(axis=1)
        assert np.all(lhs <= rhs * (1 + 1e-12))


def test_permutation_equivariance():
    rng = np.random.default_rng(6)
    q, k, v, pq, qo, pk, ko = _setup(rng, 150, 8, 5, 8)
    mask = (rng.random((5, 8)) < 0.5).astype(np.uint8)
    base = _attend_perm(q, k, v, pq, qo, pk, ko, mask, 0.3)
    # relabel tokens: same clusters, different token order -> rows move with q
    sig = rng.permutation(150)
    lq = np.empty(150, np.int32); lq[pq] = np.repeat(np.arange(5), np.diff(qo))
    lk = np.empty(150, np.int32); lk[pk] = np.repeat(np.arange(8), np.diff(ko))
    pq2, qo2 = O.permute(lq[sig], 5)
    pk2, ko2 = O.permute(lk[sig], 8)
    got = _attend_perm(q[sig], k[sig], v[sig], pq2, qo2, pk2, ko2, mask, 0.3)
    np.testing.assert_allclose(got, base[sig], rtol=1e-11, atol=1e-12)


def test_whole_path_density_one_is_dense():
    rng = np.random.default_rng(7)
    n, d = 256, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    init_q = q[rng.choice(n, 6, replace=False)]
    init_k = k[rng.choice(n, 9, replace=False)]
    res = O.routed_attention_head(q, k, v, 6, 9, n, 5, init_q, init_k, 1 / math.sqrt(d))
    np.testing.assert_allclose(res.o, sdpa(q, k, v, 1 / math.sqrt(d)), rtol=1e-11, atol=1e-12)
    assert np.all(res.sel_keys == n)


def test_whole_path_routes_to_the_spread_cluster():
    # Two key clusters: one tight (keys nearly equal), one spread out. With a
    # budget that covers exactly one of them, every query cluster must pick
    # the spread one, even though the tight one carries more attention mass.
    rng = np.random.default_rng(8)
    d = 8
    tight = np.ones(d) * 0.6 + 1e-3 * rng.standard_normal((40, d))
    spread = rng.standard_normal((40, d)) * 1.5
    k = np.concatenate([tight, spread])
    v = rng.standard_normal((80, d))
    q = np.abs(rng.standard_normal((30, d)))
    lk = np.array([0] * 40 + [1] * 40, dtype=np.int32)
    lq = np.zeros(30, dtype=np.int32)
    res = O.routed_attention_head(q, k, v, 1, 2, 40, 1, None, None, 0.35, labels_q=lq, labels_k=lk)
    assert list(res.sel_mask[0]) == [0, 1]
    assert res.ratio[0, 1] > 100 * res.ratio[0, 0]


# ---------------------------------------------------------------- map error (Section 5.3)
def _head(rng, n, ck, d, tight=False):
    counts = rng.multinomial(n, np.ones(ck) / ck)
    off = np.concatenate([[0], np.cumsum(counts)])
    kc = rng.normal(size=(ck, d))
    kp = np.repeat(kc, counts, axis=0)
    if not tight:
        kp = kp + 0.5 * rng.normal(size=kp.shape)
    kbar = np.stack([kp[off[j]:off[j + 1]].mean(0) if counts[j] else kc[j] for j in range(ck)])
    return off, kp, kbar


def test_map_error_full_mask_is_exact():
    rng = np.random.default_rng(80)
    off, kp, kbar = _head(rng, 60, 5, 4)
    qp = rng.normal(size=(20, 4))
    qo = np.array([0, 8, 20])
    for comp in (True, False):
        err, zf, zs = O.attention_map_error(qp, kp, qo, off, kbar, np.ones((2, 5), np.uint8),
                                            0.8, compensate=comp)
        assert np.all(err < 1e-30)
        np.testing.assert_allclose(zs, zf, rtol=1e-14)


def test_map_error_identical_keys_compensate_exactly():
    # keys equal to their centroid: every skipped block's centroid weight is the
    # exact weight, so the compensated map is the full map at any mask
    rng = np.random.default_rng(81)
    off, kp, kbar = _head(rng, 50, 6, 3, tight=True)
    qp = rng.normal(size=(15, 3))
    qo = np.array([0, 5, 15])
    mask = rng.integers(0, 2, (2, 6)).astype(np.uint8)
    err, zf, zs = O.attention_map_error(qp, kp, qo, off, kbar, mask, 1.1, compensate=True)
    assert np.all(err < 1e-28)
    np.testing.assert_allclose(zs, zf, rtol=1e-13)


def test_map_error_drop_everything_is_the_squared_map():
    rng = np.random.default_rng(82)
    off, kp, kbar = _head(rng, 40, 4, 5)
    qp = rng.normal(size=(9, 5))
    qo = np.array([0, 9])
    err, zf, zs = O.attention_map_error(qp, kp, qo, off, kbar, np.zeros((1, 4), np.uint8), 0.6,
                                        compensate=False)
    s = 0.6 * qp @ kp.T
    a = np.exp(s - logsumexp(s, axis=1, keepdims=True))
    np.testing.assert_allclose(err, (a ** 2).sum(1), rtol=1e-13)
    assert np.all(zs == 0)
    np.testing.assert_allclose(zf, np.exp(logsumexp(s, axis=1) - s.max(1)), rtol=1e-13)


def test_map_error_drop_one_block_closed_form():
    # dropping block B leaves the rest renormalised: with P = mass of B in the
    # full row, err = sum_{j in B} a_j^2 + (1/(1-P) - 1)^2 sum_{j not in B} a_j^2
    rng = np.random.default_rng(83)
    off, kp, kbar = _head(rng, 30, 3, 4)
    qp = rng.normal(size=(7, 4))
    mask = np.array([[1, 0, 1]], np.uint8)
    err, _, _ = O.attention_map_error(qp, kp, np.array([0, 7]), off, kbar, mask, 0.9,
                                      compensate=False)
    s = 0.9 * qp @ kp.T
    a = np.exp(s - logsumexp(s, axis=1, keepdims=True))
    inb = np.zeros(kp.shape[0], bool)
    inb[off[1]:off[2]] = True
    P = a[:, inb].sum(1)
    want = (a[:, inb] ** 2).sum(1) + (1 / (1 - P) - 1) ** 2 * (a[:, ~inb] ** 2).sum(1)
    np.testing.assert_allclose(err, want, rtol=1e-11)


def test_block_scores_are_centroid_softmax_mass():
    rng = np.random.default_rng(84)
    qc, kc = rng.normal(size=(3, 6)), rng.normal(size=(5, 6))
    off = np.array([0, 4, 4, 9, 10, 16])
    sc = O.block_scores(qc, kc, off, 0.5)
    n = np.diff(off)
    logits = 0.5 * qc @ kc.T
    live = n > 0
    want = np.exp(logits[:, live] + np.log(n[live])[None, :]
                  - logsumexp(logits[:, live] + np.log(n[live])[None, :], axis=1, keepdims=True))
    np.testing.assert_allclose(sc[:, live], want, rtol=1e-13)
    assert np.all(sc[:, ~live] == -1)
