"""Pins of the oracle's error probe and greedy router (CPU only).

The probe is pinned by a two-key closed form (written with cosh, not with
the oracle's expression), by the zero-error cases the method names (a block
whose keys are identical, singleton key clusters), by the log-sum-exp of
scipy, and by the covariance form of the raw-logit variant. The router is
pinned by brute-force subset enumeration, the budget extremes, and a
hand-worked skip-and-continue case.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import svgear_oracle as O


def test_probe_two_key_closed_form():
    # One query centroid q = (1, 0), scale 1. Key cluster 0 holds (a+dl, 0)
    # and (a-dl, 0): logits a+dl and a-dl around the centroid logit a. Key
    # cluster 1 holds (b, 1) and (b, -1): both logits equal b, so its error
    # is exactly zero.
    a, dl, b = 0.7, 0.45, 1.3
    kp = np.array([[a + dl, 0.0], [a - dl, 0.0], [b, 1.0], [b, -1.0]])
    off = np.array([0, 2, 4])
    kc = np.array([[a, 0.0], [b, 0.0]])
    ratio, log_norm = O.probe(np.array([[1.0, 0.0]]), kp, kc, off, 1.0)
    m = max(a + dl, b)
    z = (2 * math.exp(a) * math.cosh(dl) + 2 * math.exp(b)) * math.exp(-m)
    # (e^dl - 1)^2 + (e^-dl - 1)^2 = 2 cosh(2 dl) - 4 cosh(dl) + 2
    num = math.exp(2 * (a - m)) * (2 * math.cosh(2 * dl) - 4 * math.cosh(dl) + 2)
    assert ratio[0, 0] == pytest.approx(num / (2 * z * z), rel=1e-13)
    assert ratio[0, 1] == 0.0
    assert log_norm[0] == pytest.approx(math.log(2 * math.exp(a) * math.cosh(dl) + 2 * math.exp(b)),
                                        rel=1e-14)


def _clustered(rng, nk, d, ck, cq):
    labels = np.sort(rng.integers(0, ck, nk))
    kp = rng.standard_normal((nk, d))
    counts = np.bincount(labels, minlength=ck)
    off = np.concatenate([[0], np.cumsum(counts)])
    kc = O.segment_means(kp, off)
    qc = rng.standard_normal((cq, d))
    return qc, kp, kc, off


def test_probe_identical_keys_give_zero_error():
    rng = np.random.default_rng(11)
    qc, kp, kc, off = _clustered(rng, 200, 16, 9, 5)
    for j in (2, 6):                                  # collapse two clusters to one point
        kp[off[j]:off[j + 1]] = rng.standard_normal(16)
    kc = O.segment_means(kp, off)
    ratio, _ = O.probe(qc, kp, kc, off, 0.25)
    for j in (2, 6):
        if off[j + 1] > off[j]:
            # zero up to the rounding of the mean of identical rows
            assert np.all(ratio[:, j] <= 1e-20 * ratio.max())
    others = [j for j in range(9) if j not in (2, 6) and off[j + 1] - off[j] > 1]
    assert np.all(ratio[:, others] > 0)


def test_probe_singleton_clusters_give_zero_ratio():
    rng = np.random.default_rng(12)
    kp = rng.standard_normal((30, 8))
    off = np.arange(31)
    ratio, _ = O.probe(rng.standard_normal((4, 8)), kp, kp.copy(), off, 0.3)
    assert np.all(ratio == 0.0)


def test_probe_empty_cluster_marked_and_log_norm_is_logsumexp():
    rng = np.random.default_rng(13)
    qc, kp, kc, off = _clustered(rng, 120, 8, 6, 3)
    off = np.concatenate([off[:3], [off[3]], off[3:]])   # insert an empty cluster at index 3
    kc = O.segment_means(kp, off)
    ratio, log_norm = O.probe(qc, kp, kc, off, 0.5)
    assert np.all(ratio[:, 3] == -1.0)
    np.testing.assert_allclose(log_norm, logsumexp(0.5 * qc @ kp.T, axis=1), rtol=1e-14)


def test_probe_permuting_keys_inside_a_cluster_changes_nothing():
    rng = np.random.default_rng(14)
    qc, kp, kc, off = _clustered(rng, 150, 8, 7, 4)
    r1, l1 = O.probe(qc, kp, kc, off, 0.4)
    kp2 = kp.copy()
    for j in range(7):
        seg = kp2[off[j]:off[j + 1]]
        kp2[off[j]:off[j + 1]] = seg[rng.permutation(seg.shape[0])]
    r2, l2 = O.probe(qc, kp2, kc, off, 0.4)
    np.testing.assert_allclose(r1, r2, rtol=1e-12, atol=0)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)


def test_probe_logit_mode_is_quadratic_form_of_cluster_covariance():
    # raw-logit gap: mean_j (scale q.(k_j - kbar))^2 = scale^2 q^T Cov_c q
    rng = np.random.default_rng(15)
    qc, kp, kc, off = _clustered(rng, 160, 6, 5, 3)
    ratio, _ = O.probe(qc, kp, kc, off, 0.7, mode="logit")
    for j in range(5):
        seg = kp[off[j]:off[j + 1]]
        if seg.shape[0] < 2:
            continue
        cov = np.cov(seg.T, bias=True)
        np.testing.assert_allclose(ratio[:, j], 0.49 * np.einsum("cd,de,ce->c", qc, cov, qc),
                                   rtol=1e-10)


def test_probe_centroid_logit_is_mean_of_block_logits():
    # The centroid logit is the mean of the block's raw logits (k-bar is the
    # mean key), so it never exceeds the block's largest logit: exp(s~ - m) <= 1.
    rng = np.random.default_rng(16)
    qc, kp, kc, off = _clustered(rng, 100, 8, 6, 4)
    s = qc @ kp.T
    st = qc @ kc.T
    for j in range(6):
        if off[j + 1] > off[j]:
            np.testing.assert_allclose(st[:, j], s[:, off[j]:off[j + 1]].mean(axis=1), rtol=1e-12)
            assert np.all(st[:, j] <= s[:, off[j]:off[j + 1]].max(axis=1) + 1e-12)


# ---------------------------------------------------------------- value-aware probe
def _clustered_kv(rng, ck, n_per, d, dv):
    counts = rng.integers(0, n_per, ck)
    counts[0] = max(counts[0], 2)
    off = np.concatenate([[0], np.cumsum(counts)])
    kp = rng.normal(size=(off[-1], d))
    vp = rng.normal(size=(off[-1], dv))
    kc = np.stack([kp[off[j]:off[j + 1]].mean(0) if counts[j] else np.zeros(d)
                   for j in range(ck)])
    vc = np.stack([vp[off[j]:off[j + 1]].mean(0) if counts[j] else np.zeros(dv)
                   for j in range(ck)])
    return off, kp, kc, vp, vc


def test_probe_values_with_values_at_their_means_scales_probe():
    # v_j = vbar for every key: the gap is (p - p~) vbar, so the value-aware
    # ratio is ||vbar_c'||^2 times the weight-gap ratio of the same block.
    rng = np.random.default_rng(70)
    off, kp, kc, vp, vc = _clustered_kv(rng, 9, 12, 8, 5)
    kappa = np.repeat(np.arange(9), np.diff(off))
    qc = rng.normal(size=(4, 8))
    rv, lv = O.probe_values(qc, kp, kc, vc[kappa], vc, off, 0.7)
    r, ln = O.probe(qc, kp, kc, off, 0.7)
    live = np.diff(off) > 0
    np.testing.assert_allclose(rv[:, live], r[:, live] * (vc[live] ** 2).sum(1)[None, :],
                               rtol=1e-12, atol=1e-300)
    assert np.all(rv[:, ~live] == -1)
    np.testing.assert_allclose(lv, ln, rtol=1e-14)


def test_probe_values_identical_keys_leave_the_value_spread():
    # All keys of a cluster equal: p = p~ = softmax weight of that key, so the
    # ratio is p^2 times the block's mean squared value deviation.
    rng = np.random.default_rng(71)
    ck, d, dv = 6, 5, 3
    counts = np.array([3, 1, 4, 2, 5, 2])
    off = np.concatenate([[0], np.cumsum(counts)])
    kc = rng.normal(size=(ck, d))
    kp = np.repeat(kc, counts, axis=0)
    vp = rng.normal(size=(off[-1], dv))
    vc = np.stack([vp[off[j]:off[j + 1]].mean(0) for j in range(ck)])
    qc = rng.normal(size=(3, d))
    rv, _ = O.probe_values(qc, kp, kc, vp, vc, off, 1.3)
    logits = 1.3 * qc @ kc.T                              # [3, ck], one per cluster
    lse = logsumexp(logits + np.log(counts)[None, :], axis=1, keepdims=True)
    pw = np.exp(logits - lse)                             # each key's softmax weight
    spread = np.array([((vp[off[j]:off[j + 1]] - vc[j]) ** 2).sum(1).mean() for j in range(ck)])
    np.testing.assert_allclose(rv, pw ** 2 * spread[None, :], rtol=1e-11)
    assert np.all(rv[:, 1] == 0)  # a one-key cluster is its own mean


def test_probe_values_invariant_to_order_inside_clusters():
    rng = np.random.default_rng(72)
    off, kp, kc, vp, vc = _clustered_kv(rng, 7, 10, 6, 4)
    qc = rng.normal(size=(3, 6))
    perm = np.arange(off[-1])
    for j in range(7):
        a, b = off[j], off[j + 1]
        perm[a:b] = a + rng.permutation(b - a)
    r1, _ = O.probe_values(qc, kp, kc, vp, vc, off, 0.9)
    r2, _ = O.probe_values(qc, kp[perm], kc, vp[perm], vc, off, 0.9)
    np.testing.assert_allclose(r1, r2, rtol=1e-12)


# ---------------------------------------------------------------- route
def test_route_budget_extremes():
    rng = np.random.default_rng(21)
    counts = np.array([5, 0, 7, 3, 9, 1])
    off = np.concatenate([[0], np.cumsum(counts)])
    ratio = rng.random((4, 6))
    ratio[:, 1] = -1
    mask, lst, cnt, keys = O.route(ratio, off, int(off[-1]))
    assert np.all(mask[:, [0, 2, 3, 4, 5]] == 1) and np.all(mask[:, 1] == 0)
    assert np.all(keys == off[-1]) and np.all(cnt == 5)
    np.testing.assert_array_equal(lst[0], [0, 2, 3, 4, 5, -1])
    mask, lst, cnt, keys = O.route(ratio, off, 0)
    assert mask.sum() == 0 and np.all(lst == -1) and np.all(cnt == 0) and np.all(keys == 0)


def test_route_skip_and_continue_by_hand():
    counts = np.array([4, 6, 2, 3])
    off = np.concatenate([[0], np.cumsum(counts)])
    ratio = np.array([[0.9, 0.8, 0.1, 0.5]])
    # budget 9: take 0 (4 keys), 1 does not fit (4+6>9), take 3 (7), then 2 (9)
    mask, lst, cnt, keys = O.route(ratio, off, 9)
    np.testing.assert_array_equal(mask[0], [1, 0, 1, 1])
    np.testing.assert_array_equal(lst[0], [0, 2, 3, -1])
    assert cnt[0] == 3 and keys[0] == 9
    mask, _, _, keys = O.route(ratio, off, 9, fill="stop")
    np.testing.assert_array_equal(mask[0], [1, 0, 0, 0])
    assert keys[0] == 4


def test_route_empty_query_cluster_selects_nothing():
    # A query cluster without queries owns no attention row: with the query
    # offsets given it selects nothing (empty mask row, list all -1, zero
    # count and keys), whatever its ratios; the worked case above still holds
    # for the live query cluster next to it.
    counts = np.array([4, 6, 2, 3])
    off = np.concatenate([[0], np.cumsum(counts)])
    ratio = np.array([[0.9, 0.8, 0.1, 0.5], [0.9, 0.8, 0.1, 0.5]])
    q_off = np.array([0, 0, 5])  # query cluster 0 empty, cluster 1 holds five queries
    mask, lst, cnt, keys = O.route(ratio, off, 9, q_offsets=q_off)
    np.testing.assert_array_equal(mask, [[0, 0, 0, 0], [1, 0, 1, 1]])
    np.testing.assert_array_equal(lst, [[-1, -1, -1, -1], [0, 2, 3, -1]])
    np.testing.assert_array_equal(cnt, [0, 3])
    np.testing.assert_array_equal(keys, [0, 9])


def test_route_ties_prefer_lower_index():
    counts = np.array([2, 2, 2, 2])
    off = np.concatenate([[0], np.cumsum(counts)])
    ratio = np.array([[0.5, 0.7, 0.5, 0.5]])
    mask, _, _, _ = O.route(ratio, off, 4)
    np.testing.assert_array_equal(mask[0], [1, 1, 0, 0])


@pytest.mark.parametrize("seed", range(6))
def test_route_equal_sizes_is_optimal_subset(seed):
    # With equal key-cluster sizes the greedy pick maximises the covered block
    # error (sum of ratio * size) among all subsets that fit; check by
    # enumerating every subset.
    rng = np.random.default_rng(seed)
    ck, n = 10, 3
    off = np.arange(0, (ck + 1) * n, n)
    ratio = rng.random((3, ck))
    budget = int(rng.integers(0, ck * n + 1))
    mask, _, _, keys = O.route(ratio, off, budget)
    for c in range(3):
        best = -1.0
        for r in range(ck + 1):
            for sub in itertools.combinations(range(ck), r):
                if n * len(sub) <= budget:
                    best = max(best, float(sum(ratio[c, j] * n for j in sub)))
        got = float(sum(ratio[c, j] * n for j in range(ck) if mask[c, j]))
        assert got == pytest.approx(best, rel=1e-12)
        assert keys[c] <= budget


def test_route_never_exceeds_budget_random():
    rng = np.random.default_rng(30)
    for _ in range(20):
        counts = rng.integers(0, 40, 25)
        off = np.concatenate([[0], np.cumsum(counts)])
        ratio = rng.random((6, 25))
        budget = int(rng.integers(0, off[-1] + 1))
        mask, lst, cnt, keys = O.route(ratio, off, budget)
        for c in range(6):
            assert keys[c] == int(counts[mask[c] == 1].sum()) <= budget
            assert cnt[c] == mask[c].sum()
            assert list(lst[c, :cnt[c]]) == sorted(np.nonzero(mask[c])[0])
            # no unselected non-empty cluster would still fit
            left = budget - keys[c]
            assert not np.any((mask[c] == 0) & (counts > 0) & (counts <= left))


# ---------------------------------------------------------------- global route
@pytest.mark.parametrize("seed", range(4))
def test_route_global_one_query_cluster_is_route(seed):
    # With one query cluster of n queries every block costs n * |k_c'|, so a
    # head-wide budget of n * B entries selects what the per-cluster route
    # selects with B keys.
    rng = np.random.default_rng(40 + seed)
    counts = rng.integers(0, 30, 40)
    off = np.concatenate([[0], np.cumsum(counts)])
    ratio = rng.random((1, 40))
    ratio[0, counts == 0] = -1
    ratio[0, rng.integers(0, 40, 6)] = 0.5  # ties
    n = int(rng.integers(1, 50))
    budget = int(rng.integers(0, off[-1] + 1))
    for fill in ("skip", "stop"):
        m1, l1, c1, k1 = O.route(ratio, off, budget, fill=fill)
        m2, l2, c2, k2, used = O.route_global(ratio, [0, n], off, n * budget, fill=fill)
        np.testing.assert_array_equal(m1, m2)
        np.testing.assert_array_equal(l1, l2)
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(k1, k2)
        assert used == n * int(k1[0])


def test_route_global_budget_extremes_and_empty_clusters():
    rng = np.random.default_rng(41)
    nq = np.array([3, 0, 5, 2])
    nk = np.array([5, 0, 7, 3, 9, 1])
    qo = np.concatenate([[0], np.cumsum(nq)])
    ko = np.concatenate([[0], np.cumsum(nk)])
    ratio = rng.random((4, 6))
    ratio[:, 1] = -1
    mask, lst, cnt, keys, used = O.route_global(ratio, qo, ko, int(qo[-1] * ko[-1]))
    live = (nq[:, None] > 0) & (nk[None, :] > 0)
    np.testing.assert_array_equal(mask, live.astype(np.uint8))
    assert used == int(qo[-1] * ko[-1])
    np.testing.assert_array_equal(keys, np.where(nq > 0, ko[-1], 0))
    np.testing.assert_array_equal(lst[1], [-1] * 6)
    mask, lst, cnt, keys, used = O.route_global(ratio, qo, ko, 0)
    assert mask.sum() == 0 and np.all(lst == -1) and used == 0 and np.all(keys == 0)


@pytest.mark.parametrize("seed", range(5))
def test_route_global_equal_costs_is_optimal_subset(seed):
    # Equal block costs: the greedy pick maximises the covered error
    # (sum of ratio * cost) among all block sets that fit; enumerate them.
    rng = np.random.default_rng(50 + seed)
    cq, ck, a, b = 3, 4, 2, 3
    qo, ko = np.arange(0, (cq + 1) * a, a), np.arange(0, (ck + 1) * b, b)
    ratio = rng.random((cq, ck))
    budget = int(rng.integers(0, cq * ck * a * b + 1))
    mask, _, _, _, used = O.route_global(ratio, qo, ko, budget)
    blocks = [(c, j) for c in range(cq) for j in range(ck)]
    best = -1.0
    for r in range(len(blocks) + 1):
        if r * a * b > budget:
            break
        for sub in itertools.combinations(blocks, r):
            best = max(best, float(sum(ratio[c, j] for c, j in sub)))
    got = float(sum(ratio[c, j] for c, j in blocks if mask[c, j]))
    assert got == pytest.approx(best, rel=1e-12)
    assert used <= budget


def test_route_global_never_exceeds_budget_random():
    rng = np.random.default_rng(60)
    for _ in range(20):
        nq, nk = rng.integers(0, 20, 7), rng.integers(0, 30, 11)
        qo = np.concatenate([[0], np.cumsum(nq)])
        ko = np.concatenate([[0], np.cumsum(nk)])
        ratio = rng.random((7, 11))
        budget = int(rng.integers(0, qo[-1] * ko[-1] + 1))
        mask, lst, cnt, keys, used = O.route_global(ratio, qo, ko, budget)
        cost = nq[:, None] * nk[None, :]
        assert used == int((cost * mask).sum()) <= budget
        np.testing.assert_array_equal(keys, (nk[None, :] * mask).sum(axis=1))
        np.testing.assert_array_equal(cnt, mask.sum(axis=1))
        # no unselected live block would still fit
        left = budget - used
        assert not np.any((mask == 0) & (cost > 0) & (cost <= left))
