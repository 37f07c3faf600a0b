"""GPU parity of svgear_route_global against the CPU oracle (needs an MI355X).

The router is integer work on a given ratio array, so the GPU must reproduce
the oracle's mask, lists, counts, keys and used entries bit for bit when both
see the same f32 ratios. Cases: ratios with many exact ties (the order then
falls back to the block index), empty query and key clusters, budgets from 0
to the whole map, one query cluster (where it must equal the per-cluster
route), the largest map (1024 x 1024 blocks), and the whole path on a small
workload with the global router, checked against the oracle given the GPU's
cluster labels.
"""
import math

import numpy as np
import pytest
import torch

from oracle import svgear_oracle as O
from sparse_attention_video_means_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def sv():
    from sparse_attention_video_means_amd import svgear
    return svgear


def sizes_to_offsets(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def case(rng, H, cq, ck, n_q, n_k, tie_levels=None, empty_frac=0.1):
    qo, ko, ratio = [], [], []
    for _ in range(H):
        nq = rng.multinomial(n_q, rng.dirichlet(np.ones(cq)))
        nk = rng.multinomial(n_k, rng.dirichlet(np.ones(ck)))
        nq[rng.random(cq) < empty_frac] = 0
        nk[rng.random(ck) < empty_frac] = 0
        r = rng.random((cq, ck)).astype(np.float32)
        if tie_levels:
            r = (np.floor(r * tie_levels) / tie_levels).astype(np.float32)
        r[:, nk == 0] = -1.0
        qo.append(sizes_to_offsets(nq))
        ko.append(sizes_to_offsets(nk))
        ratio.append(r)
    return np.stack(qo), np.stack(ko), np.stack(ratio)


def check(qo, ko, ratio, budget):
    H, cq, ck = ratio.shape
    print(f"[route_global] H={H} Cq={cq} Ck={ck} budget={budget}", flush=True)
    mask, lst, cnt, keys, used = sv().svgear_route_global(
        torch.from_numpy(ratio).to(DEV), torch.from_numpy(qo).to(DEV),
        torch.from_numpy(ko).to(DEV), budget)
    torch.cuda.synchronize()
    for h in range(H):
        m, l, c, k, u = O.route_global(ratio[h].astype(np.float64), qo[h], ko[h], budget)
        np.testing.assert_array_equal(mask[h].cpu().numpy(), m)
        np.testing.assert_array_equal(lst[h].cpu().numpy(), l)
        np.testing.assert_array_equal(cnt[h].cpu().numpy(), c)
        np.testing.assert_array_equal(keys[h].cpu().numpy(), k)
        assert int(used[h]) == u <= budget
    return mask, used


@pytest.mark.parametrize("frac", [0.0, 0.02, 0.1, 0.37, 1.0])
def test_budgets_with_ties_and_empty_clusters(frac):
    rng = np.random.default_rng(int(frac * 1000) + 3)
    qo, ko, ratio = case(rng, 3, 100, 500, 7000, 9000, tie_levels=7)
    budget = int(math.floor(frac * 7000 * 9000))
    mask, used = check(qo, ko, ratio, budget)
    if frac == 1.0:
        for h in range(3):
            live = (np.diff(qo[h])[:, None] > 0) & (np.diff(ko[h])[None, :] > 0)
            np.testing.assert_array_equal(mask[h].cpu().numpy(), live.astype(np.uint8))
    if frac == 0.0:
        assert int(mask.sum()) == 0 and int(used.sum()) == 0


def test_distinct_ratios_realistic_sizes():
    rng = np.random.default_rng(11)
    qo, ko, ratio = case(rng, 4, 100, 500, 75600, 75600, empty_frac=0.02)
    check(qo, ko, ratio, int(math.floor(0.1 * 75600 * 75600)))


def test_one_query_cluster_equals_per_cluster_route():
    rng = np.random.default_rng(12)
    qo, ko, ratio = case(rng, 2, 1, 300, 500, 20000, tie_levels=50, empty_frac=0.05)
    qo[:, 1] = 500
    B = 4321
    mask, _ = check(qo, ko, ratio, 500 * B)
    m2, _, _, _ = sv().svgear_route(torch.from_numpy(ratio).to(DEV), torch.from_numpy(ko).to(DEV),
                                    B)
    assert torch.equal(mask, m2)


def test_largest_map():
    rng = np.random.default_rng(13)
    qo, ko, ratio = case(rng, 1, 1024, 1024, 200000, 200000, tie_levels=1000, empty_frac=0.01)
    check(qo, ko, ratio, int(0.2 * 200000 * 200000))


def test_whole_path_with_global_routing():
    wl = synth.WORKLOADS["slice"].with_(heads=2, n=6000, seed=5)
    q, k, v = synth.make_qkv(wl)
    iq = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    ik = synth.kmeans_init(k, wl.ck, wl.seed, 1)
    budget = int(math.floor(wl.rho * wl.n * wl.n))
    print(f"[route_global] whole path H={wl.heads} N={wl.n} budget={budget}", flush=True)
    res = sv().routed_attention(q.to(DEV), k.to(DEV), v.to(DEV), wl.cq, wl.ck, budget, wl.iters,
                                iq.to(DEV), ik.to(DEV), routing="global")
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(wl.d)
    f64 = lambda t: t.detach().float().cpu().double().numpy()
    for h in range(wl.heads):
        qo, ko = res["q_off"][h].cpu().numpy(), res["k_off"][h].cpu().numpy()
        m, l, c, kk, u = O.route_global(f64(res["ratio"][h]), qo, ko, budget)
        np.testing.assert_array_equal(res["sel_mask"][h].cpu().numpy(), m)
        np.testing.assert_array_equal(res["sel_keys"][h].cpu().numpy(), kk)
        assert int(res["used_entries"][h]) == u <= budget
        want = O.attend(f64(res["qp"][h]), f64(res["kp"][h]), f64(res["vp"][h]), qo, ko,
                        f64(res["k_bar"][h]), f64(res["v_bar"][h]), m, scale)
        got = f64(res["op"][h])
        err = np.linalg.norm(got - want) / np.linalg.norm(want)
        assert err <= 1e-2, err
        assert np.max(np.abs(got - want)) <= 2e-2
