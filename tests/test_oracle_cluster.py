"""Pins of the oracle's k-means and permutation (CPU only).

What fixes the expected values here is mathematics, not the oracle: the
definition of a nearest centroid written as an explicit distance, a planted
partition that Lloyd's iteration must recover, the monotone decrease of the
k-means objective, and Python's own stable sort.
"""
import numpy as np
import pytest

from oracle import svgear_oracle as O
from sparse_attention_video_means_amd import synth


def _blobs(n, d, k, sigma, seed):
    rng = np.random.default_rng(seed)
    centres = rng.standard_normal((k, d))
    z = rng.integers(0, k, n)
    return centres[z] + sigma * rng.standard_normal((n, d)), z, centres


def test_assign_is_nearest_centroid_by_explicit_distance():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((300, 8))
    mu = rng.standard_normal((13, 8))
    lab = O.kmeans_assign(x, mu)
    for n in range(x.shape[0]):
        dist = [float(np.sum((x[n] - mu[c]) ** 2)) for c in range(mu.shape[0])]
        assert lab[n] == int(np.argmin(dist))


def test_assign_ties_go_to_lowest_index():
    x = np.array([[0.0, 0.0], [1.0, 1.0], [5.0, 5.0]])
    mu = np.array([[9.0, 9.0], [1.0, 1.0], [1.0, 1.0], [0.0, 0.0], [0.0, 0.0]])
    assert list(O.kmeans_assign(x, mu)) == [3, 1, 0]


def test_update_means_and_empty_cluster_keeps_centroid():
    x = np.array([[1.0, 0.0], [3.0, 0.0], [0.0, 4.0]])
    labels = np.array([0, 0, 2], dtype=np.int32)
    prev = np.array([[7.0, 7.0], [-5.0, 2.0], [1.0, 1.0]])
    mu, counts = O.kmeans_update(x, labels, prev)
    np.testing.assert_array_equal(counts, [2, 0, 1])
    np.testing.assert_array_equal(mu, [[2.0, 0.0], [-5.0, 2.0], [0.0, 4.0]])


def test_lloyd_recovers_planted_partition():
    # 16 well separated centres in 64 dims, noise 0.3 (the Tiny workload's
    # generator); starting from one member of every planted blob, Lloyd must
    # return exactly the planted partition.
    x, z, _ = _blobs(1024, 64, 16, 0.3, seed=5)
    init = np.stack([x[np.nonzero(z == c)[0][0]] for c in range(16)])
    lab, counts, mu = O.kmeans(x, init, 10)
    np.testing.assert_array_equal(lab, z)
    np.testing.assert_array_equal(counts, np.bincount(z, minlength=16))
    for c in range(16):
        np.testing.assert_allclose(mu[c], x[z == c].mean(axis=0), rtol=0, atol=1e-12)


def test_lloyd_objective_never_increases():
    x, _, _ = _blobs(2000, 16, 40, 0.8, seed=2)
    rng = np.random.default_rng(3)
    mu = x[rng.choice(x.shape[0], 25, replace=False)]
    prev = np.inf
    for _ in range(12):
        lab = O.kmeans_assign(x, mu)
        sse_assign = float(np.sum((x - mu[lab]) ** 2))
        assert sse_assign <= prev + 1e-9
        mu, _ = O.kmeans_update(x, lab, mu)
        prev = float(np.sum((x - mu[lab]) ** 2))
        assert prev <= sse_assign + 1e-9


def test_final_centroids_are_means_of_final_labels():
    x, _, _ = _blobs(500, 8, 10, 1.0, seed=4)
    init = x[:10].copy()
    lab, counts, mu = O.kmeans(x, init, 4)
    for c in range(10):
        if counts[c]:
            np.testing.assert_allclose(mu[c], x[lab == c].mean(axis=0), atol=1e-12)


def test_round_operand_bf16_known_values():
    # bf16 keeps 8 significand bits; 1 + 2^-8 is a tie between 1 and 1 + 2^-7
    # and rounds to even (1.0); 1 + 3*2^-8 rounds up to 1 + 2^-6.
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 3.0e38], dtype=np.float32)
    out = O.round_operand(vals, "bf16")
    assert out[0] == 1.0 and out[1] == 1.0 and out[2] == 1 + 2 ** -6 and out[3] == -2.5
    # agrees with torch's own float -> bfloat16 conversion
    import torch
    t = torch.from_numpy(np.random.default_rng(0).standard_normal(1000).astype(np.float32))
    np.testing.assert_array_equal(O.round_operand(t.numpy(), "bf16"),
                                  t.to(torch.bfloat16).double().numpy())


def test_permute_is_stable_sort():
    rng = np.random.default_rng(7)
    labels = rng.integers(0, 9, 400).astype(np.int32)
    labels[labels == 4] = 5                 # leave cluster 4 empty
    perm, off = O.permute(labels, 9)
    expect = [i for _, i in sorted((int(l), i) for i, l in enumerate(labels))]
    assert list(perm) == expect
    assert off[0] == 0 and off[-1] == 400 and off[4] == off[5]
    for c in range(9):
        assert np.all(labels[perm[off[c]:off[c + 1]]] == c)


def test_unpermute_inverts_gather_and_segment_means():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((97, 5))
    labels = rng.integers(0, 6, 97).astype(np.int32)
    labels[labels == 2] = 3
    perm, off = O.permute(labels, 6)
    xp = O.gather(x, perm)
    np.testing.assert_array_equal(O.unpermute(xp, perm), x)
    means = O.segment_means(xp, off)
    for c in range(6):
        if np.any(labels == c):
            np.testing.assert_allclose(means[c], x[labels == c].mean(axis=0), atol=1e-13)
        else:
            assert np.all(means[c] == 0)


@pytest.mark.parametrize("name", ["tiny"])
def test_synth_tiny_shapes_and_init(name):
    wl = synth.WORKLOADS[name]
    q, k, v = synth.make_qkv(wl)
    assert q.shape == (1, 1024, 64) and q.dtype.is_floating_point
    init = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    assert init.shape == (1, 16, 64)
    # the init rows are rows of the tensor, all distinct
    rows = {tuple(r) for r in q[0].numpy()}
    assert all(tuple(r) in rows for r in init[0].numpy())
    assert len({tuple(r) for r in init[0].numpy()}) == 16
    # generation is reproducible and per head
    q2, _, _ = synth.make_qkv(wl, heads=[0])
    assert (q2 == q).all()


def test_row_spread_decomposes_the_total_sum_of_squares():
    # with exact cluster means: sum_i ||x_i - xbar||^2 = sum_i ||x_i||^2 - sum_c n_c ||xbar_c||^2
    rng = np.random.default_rng(90)
    counts = np.array([4, 1, 0, 7, 3])
    off = np.concatenate([[0], np.cumsum(counts)])
    x = rng.normal(size=(off[-1], 6))
    mu = np.stack([x[off[c]:off[c + 1]].mean(0) if counts[c] else np.zeros(6) for c in range(5)])
    d2 = O.row_spread(x, off, mu)
    assert d2.shape == (off[-1],)
    want = (x ** 2).sum() - (counts[:, None] * mu ** 2).sum()
    assert d2.sum() == pytest.approx(want, rel=1e-12)
    assert d2[off[1]] == 0.0  # a one-row cluster is its own mean
    np.testing.assert_allclose(d2[:4], ((x[:4] - x[:4].mean(0)) ** 2).sum(1), rtol=1e-13)
