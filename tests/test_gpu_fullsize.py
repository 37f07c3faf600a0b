"""Full-size parity on the full-size layers (needs an MI355X).

The whole path runs exactly as the benchmark times it (`RoutedAttention`) on
the Wan2.2-shaped layer (40 heads x 75,600 tokens x d=128, bf16, C_q=100,
C_k=500, density 0.10, 10 Lloyd iterations), the HunyuanVideo-shaped layer
(24 heads x 118,800 tokens) and the routing-stress layer at its two corners
(C_k=1000 at density 0.30, C_k=250 at density 0.05). The oracle cannot redo
such a layer in seconds, so its checks are sampled on two heads (the first
and the last):
  * k-means: final centroids are the means of the final labels; counts match;
  * permutation and offsets: bit-exact for the whole head; gathered rows exact;
  * probe: ratio rows of four query clusters (smallest, largest and two
    others), against every key of the head, within the derived rounding
    bound of the kernel;
  * route: bit-exact for every query cluster on the GPU ratios;
  * whole-head routing given the GPU labels: the oracle's float64 probe and
    router on every query cluster; selections may differ only where the
    bound cannot separate the ratios, and the differing clusters are counted;
  * attend: 16 queries (first 8 and last 8 rows) of each of three query
    clusters, against the oracle's materialised softmax rows;
  * unpermute (run in the attention kernel's epilogue): the whole layer's
    output bitwise equal to svgear_attend followed by svgear_unpermute.
"""
import math

import numpy as np
import pytest
import torch

from oracle import svgear_oracle as O
from probe_bound import ratio_error_bound, selection_flips
from sparse_attention_video_means_amd import synth

pytestmark = pytest.mark.gpu


def f64(t):
    if t.dtype in (torch.int32, torch.uint8):
        return t.detach().cpu().numpy()
    return t.detach().float().cpu().double().numpy()


LAYERS = {
    "wan22": synth.WORKLOADS["wan22"],
    "hunyuan": synth.WORKLOADS["hunyuan"],
    # routing stress at its largest cluster count and density: 22,680 exact
    # keys per query cluster
    "stress_ck1000_rho0.3": synth.WORKLOADS["stress"].with_(ck=1000, rho=0.3),
    # and at its smallest cluster count and density: 3,780 exact keys over 250
    # clusters of very unequal size
    "stress_ck250_rho0.05": synth.WORKLOADS["stress"].with_(ck=250, rho=0.05),
}


@pytest.fixture(scope="module", params=list(LAYERS))
def layer(request):
    from sparse_attention_video_means_amd import svgear
    wl = LAYERS[request.param]
    print(f"[fullsize] generating {wl.name}: H={wl.heads} N={wl.n}", flush=True)
    q, k, v = synth.make_qkv(wl, threads=16)
    iq = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    ik = synth.kmeans_init(k, wl.ck, wl.seed, 1)
    ra = svgear.RoutedAttention(wl.heads, wl.n, wl.d, wl.cq, wl.ck, wl.budget, wl.iters,
                                torch.bfloat16, "cuda")
    print("[fullsize] running the path", flush=True)
    ra(q.cuda(), k.cuda(), v.cuda(), iq.cuda(), ik.cuda())
    torch.cuda.synchronize()
    print("[fullsize] checking", flush=True)
    yield wl, q, k, v, ra
    del ra, q, k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("which", ["first", "last"])
def test_full_layer_sampled_parity(layer, which):
    wl, q, k, v, ra = layer
    h = 0 if which == "first" else wl.heads - 1
    scale = 1 / math.sqrt(wl.d)
    lq, lk = f64(ra.labels_q[h]), f64(ra.labels_k[h])
    # k-means: counts and final centroids
    np.testing.assert_array_equal(f64(ra.counts_q[h]), np.bincount(lq, minlength=wl.cq))
    np.testing.assert_array_equal(f64(ra.counts_k[h]), np.bincount(lk, minlength=wl.ck))
    # permutation
    pq, qo = O.permute(lq, wl.cq)
    pk, ko = O.permute(lk, wl.ck)
    np.testing.assert_array_equal(f64(ra.perm_q[h]), pq)
    np.testing.assert_array_equal(f64(ra.q_off[h]), qo)
    np.testing.assert_array_equal(f64(ra.perm_k[h]), pk)
    np.testing.assert_array_equal(f64(ra.k_off[h]), ko)
    assert torch.equal(ra.qp[h].cpu(), q[h][torch.from_numpy(pq).long()])
    assert torch.equal(ra.kp[h].cpu(), k[h][torch.from_numpy(pk).long()])
    assert torch.equal(ra.vp[h].cpu(), v[h][torch.from_numpy(pk).long()])
    kp, vp = f64(ra.kp[h]), f64(ra.vp[h])
    qbar = O.segment_means(f64(ra.qp[h]), qo)
    kbar = O.segment_means(kp, ko)
    vbar = O.segment_means(vp, ko)
    nzq, nzk = np.diff(qo) > 0, np.diff(ko) > 0
    np.testing.assert_allclose(f64(ra.cen_q[h])[nzq], qbar[nzq], rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(f64(ra.cen_k[h])[nzk], kbar[nzk], rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(f64(ra.q_bar[h]), qbar, rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(f64(ra.k_bar[h]), kbar, rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(f64(ra.v_bar[h]), vbar, rtol=2e-6, atol=2e-6)
    # probe: sampled query clusters against every key
    sizes = np.diff(qo)
    order = np.argsort(sizes, kind="stable")
    rows = sorted({int(order[np.nonzero(sizes[order] > 0)[0][0]]), int(order[-1]),
                   int(order[len(order) // 2]), 7})
    ratio, _ = O.probe(f64(ra.q_bar[h])[rows], kp, f64(ra.k_bar[h]), ko, scale)
    got = f64(ra.ratio[h])[rows]
    bound = ratio_error_bound(f64(ra.q_bar[h])[rows], kp, f64(ra.k_bar[h]), ko, scale, "bf16")
    ok = np.abs(got - ratio) <= bound
    assert ok.all(), f"{(~ok).sum()} of {ok.size} sampled ratios outside the rounding bound"
    # route: every query cluster, bit-exact on the GPU ratios
    mask, lst, cnt, keys = O.route(f64(ra.ratio[h]), ko, wl.budget, q_offsets=qo)
    np.testing.assert_array_equal(f64(ra.sel_mask[h]), mask)
    np.testing.assert_array_equal(f64(ra.sel_list[h]), lst)
    np.testing.assert_array_equal(f64(ra.sel_count[h]), cnt)
    np.testing.assert_array_equal(f64(ra.sel_keys[h]), keys)
    assert np.all(keys <= wl.budget)
    # attend: sampled queries of three query clusters (ragged tails included)
    # the output is in the original query order: row pq[p] holds permuted query p
    op = f64(ra.o[h])[pq]
    qp = f64(ra.qp[h])
    for c in rows[:3]:
        a, b = int(qo[c]), int(qo[c + 1])
        idx = np.unique(np.concatenate([np.arange(a, min(a + 8, b)), np.arange(max(b - 8, a), b)]))
        want = O.attend(qp[idx], kp, vp, np.array([0, len(idx)]), ko, f64(ra.k_bar[h]),
                        f64(ra.v_bar[h]), mask[c:c + 1], scale)
        gotr = op[idx]
        err = np.linalg.norm(gotr - want) / np.linalg.norm(want)
        assert err <= 1e-2, (c, err)
        assert np.max(np.abs(gotr - want)) <= 2e-2, c
    # unpermute in attend's epilogue == attend, then the standalone unpermute
    from sparse_attention_video_means_amd import svgear as S
    op_all = S.svgear_attend(ra.qp, ra.kp, ra.vp, ra.q_off, ra.k_off, ra.k_bar, ra.v_bar,
                             ra.sel_mask, ra.scale)
    assert torch.equal(S.svgear_unpermute(op_all, ra.perm_q), ra.o)


@pytest.mark.parametrize("which", ["first", "last"])
def test_full_head_routing_against_the_oracle(layer, which):
    """The oracle's float64 probe and router over a whole head, given the GPU
    labels: every query cluster's selection equals the oracle's, except where
    the probe's rounding bound cannot separate the ratios that decide a fill
    step; the differing clusters are counted (and printed)."""
    wl, q, k, v, ra = layer
    h = 0 if which == "first" else wl.heads - 1
    scale = 1 / math.sqrt(wl.d)
    lq, lk = f64(ra.labels_q[h]), f64(ra.labels_k[h])
    pq, qo = O.permute(lq, wl.cq)
    pk, ko = O.permute(lk, wl.ck)
    kp = f64(k[h])[pk]
    qbar = O.segment_means(f64(q[h])[pq], qo)
    kbar = O.segment_means(kp, ko)
    ratio, _ = O.probe(qbar, kp, kbar, ko, scale)
    mask, _, _, keys = O.route(ratio, ko, wl.budget, q_offsets=qo)
    gmask = f64(ra.sel_mask[h])
    bound = ratio_error_bound(f64(ra.q_bar[h]), kp, f64(ra.k_bar[h]), ko, scale, "bf16",
                              mean_tol=2e-6)
    fl = selection_flips(ratio, f64(ra.ratio[h]), bound, ko, mask, gmask, qo)
    qn = np.diff(qo).astype(np.float64)
    dens_ref = float((qn * keys).sum()) / (wl.n * wl.n)
    dens_gpu = float((qn * f64(ra.sel_keys[h])).sum()) / (wl.n * wl.n)
    print(f"[fullsize] {wl.name} Ck={wl.ck} rho={wl.rho} head {h}: {fl['flipped']} of "
          f"{fl['live']} query clusters route differently (first parting gap "
          f"{fl['max_rel_gap']:.3g} relative, {fl['max_gap_over_bound']:.3g} of the bound); "
          f"exact-entry density gpu {dens_gpu:.6f} oracle {dens_ref:.6f}", flush=True)
    assert fl["separated_ok"], "a selection differs where the bound separates the ratios"
    assert fl["flipped"] <= int(0.02 * fl["live"]), fl
