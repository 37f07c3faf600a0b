"""GPU parity of every libsvgear call against the CPU oracle (needs an MI355X).

Each call is checked on the same inputs the HIP path received:
  * permutation, offsets, gathered rows, selections, unpermute: bit-exact;
  * k-means: every GPU label is a nearest centroid up to the f32 accumulation
    bound, taken with the centroids at the kernel's operand precision, and the
    centroids are the means of the GPU labels;
  * centroids / means: f32 accumulation tolerance;
  * probe ratios: within the rounding-error bound derived from the kernel's
    f32 steps on the same inputs (tests/probe_bound.py; about 1e-3 relative);
  * whole path given the GPU labels: every query cluster whose selection
    differs from the oracle's may differ only through ratios the bound cannot
    separate; the differing clusters are counted and printed;
  * attention output: relative Frobenius <= 1e-2 and max-abs <= 2e-2 for bf16,
    1e-4 / 1e-4 for f32.
Sizes span several tiles and end in ragged tails.
"""
import math

import numpy as np
import pytest
import torch

from oracle import svgear_oracle as O
from parity_checks import assert_nearest, check_whole_head, f64, operand, rel_fro, tol_out
from probe_bound import ratio_error_bound
from sparse_attention_video_means_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def sv():
    from sparse_attention_video_means_amd import svgear
    return svgear


CASES = {
    "tiny": synth.WORKLOADS["tiny"],
    "blobs_bf16_d128": synth.WORKLOADS["slice"].with_(name="blobs_bf16_d128", heads=2, n=3001,
                                                      cq=24, ck=70, iters=5, centres=64),
    "blobs_bf16_d64": synth.WORKLOADS["slice"].with_(name="blobs_bf16_d64", heads=2, n=2050,
                                                     d=64, cq=10, ck=40, rho=0.2, iters=4,
                                                     centres=32),
    "lattice_bf16": synth.WORKLOADS["wan22"].with_(name="lattice_bf16", heads=2,
                                                   n=5 * 15 * 20, grid=(5, 15, 20), cq=20,
                                                   ck=60, iters=4),
    "stress_bf16": synth.WORKLOADS["stress"].with_(name="stress_bf16", heads=1, n=4100,
                                                   cq=150, ck=200, iters=3, rho=0.3),
    "big_clusters_f32": synth.WORKLOADS["slice"].with_(name="big_clusters_f32", heads=1,
                                                       n=4000, d=128, dtype="f32", cq=3, ck=3,
                                                       iters=2, centres=3, rho=0.4),
}


_CACHE = {}


def run_case(name):
    if name in _CACHE:
        return _CACHE[name]
    wl = CASES[name]
    q, k, v = synth.make_qkv(wl)
    iq = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    ik = synth.kmeans_init(k, wl.ck, wl.seed, 1)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    S = sv()
    res = S.routed_attention(qd, kd, vd, wl.cq, wl.ck, wl.budget, wl.iters, iq.to(DEV),
                             ik.to(DEV), 1 / math.sqrt(wl.d))
    torch.cuda.synchronize()
    out = dict(wl=wl, q=q, k=k, v=v, iq=iq, ik=ik, res=res)
    _CACHE[name] = out
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_cluster_one_lloyd_step(name):
    wl = CASES[name]
    q, _, _ = synth.make_qkv(wl)
    init = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    cen = init.to(DEV)
    labels, counts = sv().svgear_cluster(q.to(DEV), cen, 1)
    torch.cuda.synchronize()
    for h in range(wl.heads):
        x = f64(q[h])
        lab = f64(labels[h])
        flips = assert_nearest(x, init[h].double().numpy(), lab, operand(wl))
        assert flips <= max(2, x.shape[0] // 1000)
        np.testing.assert_array_equal(f64(counts[h]), np.bincount(lab, minlength=wl.cq))
        mu, _ = O.kmeans_update(x, lab, init[h].double().numpy())
        np.testing.assert_allclose(f64(cen[h]), mu, rtol=2e-6, atol=2e-6)


@pytest.mark.parametrize("name", ["tiny", "blobs_bf16_d128", "lattice_bf16"])
def test_cluster_last_step_consistent_and_deterministic(name):
    wl = CASES[name]
    q, _, _ = synth.make_qkv(wl)
    init = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    qd = q.to(DEV)
    prev = init.to(DEV)
    sv().svgear_cluster(qd, prev, wl.iters - 1) if wl.iters > 1 else None
    c1, c2 = init.to(DEV), init.to(DEV)
    l1, n1 = sv().svgear_cluster(qd, c1, wl.iters)
    l2, n2 = sv().svgear_cluster(qd, c2, wl.iters)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(n1, n2) and torch.equal(c1, c2)
    mu_prev = prev if wl.iters > 1 else init.to(DEV)
    for h in range(wl.heads):
        x = f64(q[h])
        lab = f64(l1[h])
        assert_nearest(x, f64(mu_prev[h]), lab, operand(wl))
        means = O.segment_means(x[np.argsort(lab, kind="stable")],
                                np.concatenate([[0], np.cumsum(np.bincount(lab, minlength=wl.cq))]))
        nz = np.bincount(lab, minlength=wl.cq) > 0
        np.testing.assert_allclose(f64(c1[h])[nz], means[nz], rtol=2e-6, atol=2e-6)


def test_cluster_tiny_recovers_planted_blobs():
    # Tiny workload with one initial row per planted centre: the GPU must find
    # the planted partition exactly, like the oracle.
    wl = CASES["tiny"]
    z, _ = synth._latent(wl, 0)
    q, _, _ = synth.make_qkv(wl)
    init = torch.stack([q[0, int(np.nonzero(z == c)[0][0])] for c in range(16)])[None].float()
    labels, counts = sv().svgear_cluster(q.to(DEV), init.to(DEV), 10)
    np.testing.assert_array_equal(f64(labels[0]), z)


@pytest.mark.parametrize("name", list(CASES))
def test_permute_bit_exact_and_means(name):
    c = run_case(name)
    wl, res = c["wl"], c["res"]
    for h in range(wl.heads):
        lq, lk = f64(res["labels_q"][h]), f64(res["labels_k"][h])
        pq, qo = O.permute(lq, wl.cq)
        pk, ko = O.permute(lk, wl.ck)
        np.testing.assert_array_equal(f64(res["perm_q"][h]), pq)
        np.testing.assert_array_equal(f64(res["q_off"][h]), qo)
        np.testing.assert_array_equal(f64(res["perm_k"][h]), pk)
        np.testing.assert_array_equal(f64(res["k_off"][h]), ko)
        assert torch.equal(res["qp"][h].cpu(), c["q"][h][torch.from_numpy(pq).long()])
        assert torch.equal(res["kp"][h].cpu(), c["k"][h][torch.from_numpy(pk).long()])
        assert torch.equal(res["vp"][h].cpu(), c["v"][h][torch.from_numpy(pk).long()])
        for got, x, p, off in ((res["q_bar"], c["q"], pq, qo), (res["k_bar"], c["k"], pk, ko),
                               (res["v_bar"], c["v"], pk, ko)):
            want = O.segment_means(f64(x[h])[p], off)
            np.testing.assert_allclose(f64(got[h]), want, rtol=2e-6, atol=2e-6)


@pytest.mark.parametrize("name", list(CASES))
def test_probe_against_oracle(name):
    c = run_case(name)
    wl, res = c["wl"], c["res"]
    scale = 1 / math.sqrt(wl.d)
    worst = 0.0
    for h in range(wl.heads):
        qb, kp, kb = f64(res["q_bar"][h]), f64(res["kp"][h]), f64(res["k_bar"][h])
        koff = f64(res["k_off"][h])
        ratio, log_norm = O.probe(qb, kp, kb, koff, scale)
        got = f64(res["ratio"][h])
        bound = ratio_error_bound(qb, kp, kb, koff, scale, operand(wl))
        err = np.abs(got - ratio)
        ok = err <= bound
        worst = max(worst, float(np.max(err / np.maximum(bound, 1e-300))))
        assert ok.all(), f"{(~ok).sum()} of {ok.size} ratios outside the bound; worst " \
                         f"{np.max(err / np.maximum(bound, 1e-300))} of it"
        # log_norm moves by at most max_j |error of s_cj|; the kernel carries
        # qbar and (k_j - kbar) as bf16 high part + remainder (about 2^-16
        # relative per factor) and accumulates in f32, so
        # |error| <= scale * 2^-14 * sum_d |qbar_d (k_jd - kbar_d)| + f32 rounding.
        dk = np.abs(kp - np.repeat(kb, np.diff(koff), axis=0))
        unit = 2.0 ** -14 if wl.dtype == "bf16" else 2.0 ** -20
        lbound = scale * unit * (np.abs(qb) @ dk.T).max(axis=1) + 2e-5
        assert np.all(np.abs(f64(res["log_norm"][h]) - log_norm) <= lbound)
    print(f"[parity] probe {name}: largest error {worst:.3g} of the bound", flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_route_bit_exact_on_identical_ratios(name):
    c = run_case(name)
    wl, res = c["wl"], c["res"]
    for h in range(wl.heads):
        mask, lst, cnt, keys = O.route(f64(res["ratio"][h]), f64(res["k_off"][h]), wl.budget,
                                       q_offsets=f64(res["q_off"][h]))
        np.testing.assert_array_equal(f64(res["sel_mask"][h]), mask)
        np.testing.assert_array_equal(f64(res["sel_list"][h]), lst)
        np.testing.assert_array_equal(f64(res["sel_count"][h]), cnt)
        np.testing.assert_array_equal(f64(res["sel_keys"][h]), keys)
        assert np.all(keys <= wl.budget)


@pytest.mark.parametrize("name", list(CASES))
def test_attend_against_oracle(name):
    c = run_case(name)
    wl, res = c["wl"], c["res"]
    rt, at = tol_out(wl)
    for h in range(wl.heads):
        want = O.attend(f64(res["qp"][h]), f64(res["kp"][h]), f64(res["vp"][h]),
                        f64(res["q_off"][h]), f64(res["k_off"][h]), f64(res["k_bar"][h]),
                        f64(res["v_bar"][h]), f64(res["sel_mask"][h]), 1 / math.sqrt(wl.d))
        got = f64(res["op"][h])
        assert rel_fro(got, want) <= rt
        assert np.max(np.abs(got - want)) <= at
        # unpermute is a pure copy
        o = f64(res["o"][h])
        np.testing.assert_array_equal(o[f64(res["perm_q"][h])], got)


@pytest.mark.parametrize("name", list(CASES))
def test_whole_path_given_gpu_labels(name):
    c = run_case(name)
    wl, res = c["wl"], c["res"]
    for h in range(wl.heads):
        check_whole_head(name, wl, c["q"], c["k"], c["v"], res, h, max_flip_frac=0.02)


@pytest.mark.parametrize("name", ["tiny", "blobs_bf16_d128", "blobs_bf16_d64"])
def test_density_one_is_dense_attention(name):
    c = run_case(name)
    wl, res = c["wl"], c["res"]
    S = sv()
    mask, _, _, keys = S.svgear_route(res["ratio"], res["k_off"], wl.n)
    assert int(keys.min()) == wl.n
    op = S.svgear_attend(res["qp"], res["kp"], res["vp"], res["q_off"], res["k_off"],
                         res["k_bar"], res["v_bar"], mask, 1 / math.sqrt(wl.d))
    o = S.svgear_unpermute(op, res["perm_q"])
    rt, at = tol_out(wl)
    for h in range(wl.heads):
        want = O.dense_attention(f64(c["q"][h]), f64(c["k"][h]), f64(c["v"][h]),
                                 1 / math.sqrt(wl.d))
        got = f64(o[h])
        assert rel_fro(got, want) <= rt
        assert np.max(np.abs(got - want)) <= at


def test_whole_path_is_deterministic():
    wl = CASES["blobs_bf16_d128"]
    q, k, v = synth.make_qkv(wl)
    iq = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    ik = synth.kmeans_init(k, wl.ck, wl.seed, 1)
    S = sv()
    outs = []
    for _ in range(2):
        r = S.routed_attention(q.to(DEV), k.to(DEV), v.to(DEV), wl.cq, wl.ck, wl.budget, wl.iters,
                               iq.to(DEV), ik.to(DEV))
        outs.append(r)
    torch.cuda.synchronize()
    for key in ("labels_q", "labels_k", "perm_q", "ratio", "sel_mask", "op", "o"):
        assert torch.equal(outs[0][key], outs[1][key]), key


@pytest.mark.parametrize("name", list(CASES))
def test_attend_unpermute_equals_attend_then_unpermute(name):
    """The unpermutation run in attend's epilogue writes bitwise what attend
    followed by the standalone unpermute writes (§3.1: outputs go back to the
    original token order), for every case's routing."""
    c = run_case(name)
    wl, res = c["wl"], c["res"]
    S = sv()
    args = (res["qp"], res["kp"], res["vp"], res["q_off"], res["k_off"], res["k_bar"],
            res["v_bar"], res["sel_mask"])
    scale = 1 / math.sqrt(wl.d)
    want = S.svgear_unpermute(S.svgear_attend(*args, scale), res["perm_q"])
    got = S.svgear_attend_unpermute(*args, res["perm_q"], scale)
    assert torch.equal(got, want)


def test_attend_unpermute_drops_rows_outside_the_range():
    """Permuted rows whose target lies outside [0, Nq) are not written; every
    other row is."""
    c = run_case("blobs_bf16_d64")
    wl, res = c["wl"], c["res"]
    S = sv()
    args = (res["qp"], res["kp"], res["vp"], res["q_off"], res["k_off"], res["k_bar"],
            res["v_bar"], res["sel_mask"])
    scale = 1 / math.sqrt(wl.d)
    want = S.svgear_unpermute(S.svgear_attend(*args, scale), res["perm_q"])
    perm = res["perm_q"].clone()
    lost = perm[:, :2].clone()
    perm[:, 0] = -1
    perm[:, 1] = wl.n
    out = torch.full_like(want, 7.0)
    S.svgear_attend_unpermute(*args, perm, scale, out=out)
    for h in range(wl.heads):
        kept = torch.ones(wl.n, dtype=torch.bool, device=out.device)
        kept[lost[h].long()] = False
        assert torch.equal(out[h][kept], want[h][kept])
        assert bool((out[h][~kept] == 7.0).all())
