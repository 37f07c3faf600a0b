"""GPU edge cases against the CPU oracle, through the C ABI (needs an MI355X).

Cluster assignments are injected (parity "given the same cluster assignment")
so that the cases can force what k-means would rarely produce on its own:
empty query and key clusters, a single cluster, singleton clusters, one row,
N_q != N_k, the maximum cluster count, and a zero budget. Bars as in
test_gpu_parity: permutation, offsets, gathered rows and selections bit-exact;
probe ratios within 2e-2 relative + 1e-4 of the row maximum (empty clusters
exactly -1); attention output relative Frobenius <= 1e-2 and max-abs <= 2e-2
for bf16 (1e-4 for f32).
"""
import math

import numpy as np
import pytest
import torch

from oracle import svgear_oracle as O
from probe_bound import ratio_error_bound
from sparse_attention_video_means_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def sv():
    from sparse_attention_video_means_amd import svgear
    return svgear


def f64(t):
    if t.dtype in (torch.int32, torch.uint8):
        return t.detach().cpu().numpy()
    return t.detach().float().cpu().double().numpy()


def data(h, n, d, dtype, seed, nk=None):
    """Blob-structured Q, K, V ([h, n, d] and [h, nk, d])."""
    nk = n if nk is None else nk
    wl = synth.WORKLOADS["slice"].with_(name="edge", heads=h, n=max(n, nk), d=d, dtype=dtype,
                                        centres=24, seed=seed)
    q, k, v = synth.make_qkv(wl)
    return q[:, :n].contiguous(), k[:, :nk].contiguous(), v[:, :nk].contiguous()


def check_path(q, k, v, lq, lk, cq, ck, budget, *, expect_empty=None):
    """Run permute -> probe -> route -> attend -> unpermute on injected labels
    and compare every step with the oracle."""
    S = sv()
    d = q.shape[2]
    scale = 1 / math.sqrt(d)
    f32 = q.dtype == torch.float32
    rt, at = (1e-4, 1e-4) if f32 else (1e-2, 2e-2)
    print(f"[edges] H={q.shape[0]} Nq={q.shape[1]} Nk={k.shape[1]} d={d} Cq={cq} Ck={ck} "
          f"budget={budget} dtype={q.dtype}", flush=True)
    res = S.routed_attention(q.to(DEV), k.to(DEV), v.to(DEV), cq, ck, budget, 0, None, None,
                             scale, labels_q=torch.from_numpy(lq).to(DEV),
                             labels_k=torch.from_numpy(lk).to(DEV))
    torch.cuda.synchronize()
    for h in range(q.shape[0]):
        pq, qo = O.permute(lq[h], cq)
        pk, ko = O.permute(lk[h], ck)
        np.testing.assert_array_equal(f64(res["perm_q"][h]), pq)
        np.testing.assert_array_equal(f64(res["q_off"][h]), qo)
        np.testing.assert_array_equal(f64(res["perm_k"][h]), pk)
        np.testing.assert_array_equal(f64(res["k_off"][h]), ko)
        assert torch.equal(res["qp"][h].cpu(), q[h][torch.from_numpy(pq).long()])
        assert torch.equal(res["kp"][h].cpu(), k[h][torch.from_numpy(pk).long()])
        assert torch.equal(res["vp"][h].cpu(), v[h][torch.from_numpy(pk).long()])
        qbar = O.segment_means(f64(q[h])[pq], qo)
        kbar = O.segment_means(f64(k[h])[pk], ko)
        vbar = O.segment_means(f64(v[h])[pk], ko)
        for got, want in ((res["q_bar"], qbar), (res["k_bar"], kbar), (res["v_bar"], vbar)):
            np.testing.assert_allclose(f64(got[h]), want, rtol=2e-6, atol=2e-6)
        # probe on the GPU's own centroids and permuted keys
        ratio, _ = O.probe(f64(res["q_bar"][h]), f64(res["kp"][h]), f64(res["k_bar"][h]), ko,
                           scale)
        got = f64(res["ratio"][h])
        empty_k = np.diff(ko) == 0
        assert np.all(got[:, empty_k] == -1.0)
        bound = ratio_error_bound(f64(res["q_bar"][h]), f64(res["kp"][h]), f64(res["k_bar"][h]),
                                  ko, scale, "bf16" if q.dtype == torch.bfloat16 else "f32")
        ok = np.abs(got - ratio) <= bound
        assert ok.all(), f"{(~ok).sum()} ratios outside the rounding bound"
        # route: bit-exact on the GPU ratios (empty query clusters select nothing)
        mask, lst, cnt, keys = O.route(got, ko, budget, q_offsets=qo)
        np.testing.assert_array_equal(f64(res["sel_mask"][h]), mask)
        np.testing.assert_array_equal(f64(res["sel_list"][h]), lst)
        np.testing.assert_array_equal(f64(res["sel_count"][h]), cnt)
        np.testing.assert_array_equal(f64(res["sel_keys"][h]), keys)
        assert not mask[:, empty_k].any() and np.all(keys <= budget)
        # attend on the GPU selection
        want = O.attend(f64(res["qp"][h]), f64(res["kp"][h]), f64(res["vp"][h]), qo, ko,
                        f64(res["k_bar"][h]), f64(res["v_bar"][h]), f64(res["sel_mask"][h]),
                        scale)
        op = f64(res["op"][h])
        assert np.isfinite(op).all()
        err = np.linalg.norm(op - want) / max(np.linalg.norm(want), 1e-30)
        assert err <= rt, err
        assert np.max(np.abs(op - want)) <= at
        np.testing.assert_array_equal(f64(res["o"][h])[pq], op)
        if expect_empty is not None:
            assert (np.diff(qo) == 0).sum() >= expect_empty[0]
            assert empty_k.sum() >= expect_empty[1]
    return res


def test_empty_query_and_key_clusters():
    rng = np.random.default_rng(11)
    q, k, v = data(2, 3000, 128, "bf16", 11)
    cq, ck = 40, 96
    lq = rng.choice(np.arange(1, 30), size=(2, 3000)).astype(np.int32)       # 0 and 30..39 empty
    used = np.array([c for c in range(ck) if c % 3 and c != ck - 1])        # every third + last empty
    lk = rng.choice(used, size=(2, 3000)).astype(np.int32)
    check_path(q, k, v, lq, lk, cq, ck, budget=600, expect_empty=(11, 33))


def test_single_cluster_is_pure_compensation():
    q, k, v = data(1, 700, 64, "bf16", 12)
    lz = np.zeros((1, 700), np.int32)
    res = check_path(q, k, v, lz, lz, 1, 1, budget=350)
    # the only key cluster (700 keys) exceeds the budget: every query sees one
    # centroid term, so the output is the mean value row
    assert int(res["sel_count"].sum()) == 0
    vbar = f64(v[0]).mean(axis=0)
    np.testing.assert_allclose(f64(res["o"][0]), np.broadcast_to(vbar, (700, 64)), atol=2e-2)


def test_single_cluster_full_budget_is_dense():
    q, k, v = data(1, 513, 128, "bf16", 13)
    lz = np.zeros((1, 513), np.int32)
    res = check_path(q, k, v, lz, lz, 1, 1, budget=513)
    want = O.dense_attention(f64(q[0]), f64(k[0]), f64(v[0]), 1 / math.sqrt(128))
    got = f64(res["o"][0])
    assert np.linalg.norm(got - want) / np.linalg.norm(want) <= 1e-2


def test_one_row():
    q, k, v = data(2, 1, 128, "bf16", 14)
    lz = np.zeros((2, 1), np.int32)
    check_path(q, k, v, lz, lz, 1, 1, budget=0)
    check_path(q, k, v, lz, lz, 1, 1, budget=1)


def test_singleton_clusters_f32():
    q, k, v = data(1, 5, 64, "f32", 15)
    lab = np.array([[3, 0, 4, 1, 2]], np.int32)
    res = check_path(q, k, v, lab, lab, 5, 5, budget=2)
    # singleton key clusters have zero error; ties go to the lower index
    assert np.all(f64(res["ratio"][0]) == 0.0)
    assert np.array_equal(f64(res["sel_list"][0])[:, :2], np.tile([0, 1], (5, 1)))


def test_nq_differs_from_nk():
    rng = np.random.default_rng(16)
    q, k, v = data(2, 1000, 128, "bf16", 16, nk=2600)
    lq = rng.integers(0, 12, size=(2, 1000)).astype(np.int32)
    lk = rng.integers(0, 50, size=(2, 2600)).astype(np.int32)
    check_path(q, k, v, lq, lk, 12, 50, budget=390)


def test_maximum_cluster_count():
    rng = np.random.default_rng(17)
    q, k, v = data(1, 4500, 64, "bf16", 17)
    lq = rng.integers(0, 1024, size=(1, 4500)).astype(np.int32)
    lk = rng.integers(0, 1024, size=(1, 4500)).astype(np.int32)
    check_path(q, k, v, lq, lk, 1024, 1024, budget=450)


def test_zero_budget_is_centroid_softmax():
    rng = np.random.default_rng(18)
    q, k, v = data(1, 2000, 128, "bf16", 18)
    lq = rng.integers(0, 20, size=(1, 2000)).astype(np.int32)
    lk = rng.integers(0, 64, size=(1, 2000)).astype(np.int32)
    res = check_path(q, k, v, lq, lk, 20, 64, budget=0)
    assert int(res["sel_count"].sum()) == 0


@pytest.mark.parametrize("n,d,c,dtype", [(700, 64, 1, "bf16"), (4500, 64, 1024, "bf16"),
                                         (1500, 128, 1024, "f32")])
def test_cluster_extreme_counts(n, d, c, dtype):
    """k-means with one cluster and with the maximum cluster count: labels are
    nearest centroids, centroids are the means of the labels (empty keep theirs)."""
    q, _, _ = data(1, n, d, dtype, 19)
    init = synth.kmeans_init(q, c, 0, 0)
    cen = init.to(DEV)
    print(f"[edges] cluster N={n} d={d} C={c} {dtype}", flush=True)
    labels, counts = sv().svgear_cluster(q.to(DEV), cen, 2)
    torch.cuda.synchronize()
    lab = f64(labels[0])
    assert lab.min() >= 0 and lab.max() < c
    np.testing.assert_array_equal(f64(counts[0]), np.bincount(lab, minlength=c))
    x = f64(q[0])
    mu = f64(cen[0])
    nz = np.bincount(lab, minlength=c) > 0
    means = O.segment_means(x[np.argsort(lab, kind="stable")],
                            np.concatenate([[0], np.cumsum(np.bincount(lab, minlength=c))]))
    np.testing.assert_allclose(mu[nz], means[nz], rtol=2e-6, atol=2e-6)


def test_running_maximum_jumps_inside_a_tile():
    """Logits that rise by far more than the kernel's rescale slack from one
    32-key half of a tile to the next (and from tile to tile): every jump
    forces the running maximum up while earlier weights are still being
    accumulated, in the same order the kernel walks the keys."""
    n, d = 320, 128
    rng = np.random.default_rng(20)
    step = np.repeat(np.arange(n // 32), 32).astype(np.float32)        # +1 every 32 keys
    k = np.zeros((1, n, d), np.float32)
    k[0, :, 0] = 4.0 * step                                            # q.k rises 4*40*tau per half
    k[0, :, 1:] = 0.1 * rng.standard_normal((n, d - 1))
    q = np.zeros((1, 96, d), np.float32)
    q[0, :, 0] = 40.0
    q[0, :, 1:] = 0.1 * rng.standard_normal((96, d - 1))
    v = rng.standard_normal((1, n, d)).astype(np.float32)
    to = lambda a: torch.from_numpy(a).to(torch.bfloat16)
    zq, zk = np.zeros((1, 96), np.int32), np.zeros((1, n), np.int32)
    # one key cluster, fully selected: the exact tiles walk the keys in order
    res = check_path(to(q), to(k), to(v), zq, zk, 1, 1, budget=n)
    assert int(res["sel_count"].sum()) == 1
    # two key clusters, the rising one skipped: its centroid term is the
    # largest logit and arrives after the exact tiles
    lk = (np.arange(n) >= 64).astype(np.int32)[None]
    res = check_path(to(q), to(k), to(v), zq, lk, 1, 2, budget=64)
    assert int(res["sel_mask"][0, 0, 0]) == 1 and int(res["sel_mask"][0, 0, 1]) == 0


def test_selection_larger_than_a_source_row_window():
    """More exact keys than one window of the kernel's source-row table holds
    (8192 positions for bf16, 1024 for f32), so the table is refilled
    mid-stream, across clusters of uneven size."""
    rng = np.random.default_rng(21)
    q, k, v = data(1, 20000, 128, "bf16", 21)
    lq = rng.integers(0, 6, size=(1, 20000)).astype(np.int32)
    sizes = rng.zipf(1.3, size=40).astype(np.float64)
    p = sizes / sizes.sum()
    lk = rng.choice(40, size=(1, 20000), p=p).astype(np.int32)
    res = check_path(q, k, v, lq, lk, 6, 40, budget=12000)
    assert int(res["sel_keys"].max()) > 8192
    qf, kf, vf = data(1, 3000, 64, "f32", 22)
    lqf = rng.integers(0, 3, size=(1, 3000)).astype(np.int32)
    lkf = rng.integers(0, 9, size=(1, 3000)).astype(np.int32)
    res = check_path(qf, kf, vf, lqf, lkf, 3, 9, budget=2500)
    assert int(res["sel_keys"].max()) > 1024


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_partial_query_blocks(dtype, d):
    """Query clusters of every size around the kernel's query-block and
    wavefront boundaries (blocks of 256 queries for bf16 and 64 for f32,
    wavefronts of 32 and 16): full, half-full and nearly empty last blocks.
    One key cluster is shorter than half a tile, and in the second run it is
    the only key cluster, so every exact tile is mostly filler."""
    rng = np.random.default_rng(23)
    sizes_q = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 384, 385]
    lq = np.concatenate([np.full(s, c, np.int32) for c, s in enumerate(sizes_q)])
    n = lq.size
    lq = rng.permutation(lq)[None]
    sizes_k = [20, 300, 77, 1000, 5, 431] + [0] * 2
    sizes_k[-1] = n - sum(sizes_k)
    lk = rng.permutation(np.concatenate([np.full(s, c, np.int32)
                                         for c, s in enumerate(sizes_k)]))[None]
    q, k, v = data(1, n, d, dtype, 23)
    check_path(q, k, v, lq, lk, len(sizes_q), len(sizes_k), budget=1400)
    # a single selected key cluster shorter than a half tile and nothing to
    # compensate: the second half of the only tile is all filler
    lk1 = np.zeros((1, n), np.int32)
    k1, v1 = k[:, :20].contiguous(), v[:, :20].contiguous()
    check_path(q, k1, v1, lq, lk1[:, :20], len(sizes_q), 1, budget=20)
