"""GPU parity of svgear_probe_values (the value-aware probe) against the CPU
oracle (needs an MI355X).

Each case runs the path with probe="value" and checks the GPU ratios against
``oracle.probe_values`` on the GPU's own permuted tensors and centroids, with
the probe's bar: 2e-2 relative plus 1e-4 of the row maximum (16-bit split
centroids, f32 sums). Empty key clusters are exactly -1 and one-key clusters
exactly 0. The selection made from the GPU ratios must equal the oracle's
selection from the same ratios bit for bit, and the attention output must
match the oracle given the GPU's labels and selection. A last case places
every value at its cluster mean, where the value-aware ratio is
||vbar||^2 times the weight-gap ratio of the plain probe.
"""
import math

import numpy as np
import pytest
import torch

from oracle import svgear_oracle as O
from sparse_attention_video_means_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    "tiny_f32": synth.WORKLOADS["tiny"],
    "blobs_bf16_d128": synth.WORKLOADS["slice"].with_(name="pv_blobs", heads=2, n=3001, cq=24,
                                                      ck=70, iters=5, centres=64),
    "blobs_bf16_d64": synth.WORKLOADS["slice"].with_(name="pv_d64", heads=1, n=2050, d=64,
                                                     cq=10, ck=40, rho=0.2, iters=4,
                                                     centres=32),
    "lattice_bf16": synth.WORKLOADS["wan22"].with_(name="pv_lattice", heads=2,
                                                   n=5 * 15 * 20, grid=(5, 15, 20), cq=20,
                                                   ck=60, iters=4),
    "stress_bf16": synth.WORKLOADS["stress"].with_(name="pv_stress", heads=1, n=4100, cq=150,
                                                   ck=200, iters=3, rho=0.3),
}


def sv():
    from sparse_attention_video_means_amd import svgear
    return svgear


def f64(t):
    if t.dtype in (torch.int32, torch.uint8):
        return t.detach().cpu().numpy()
    return t.detach().float().cpu().double().numpy()


def probe_ok(got, want):
    rowmax = want.max(axis=1, keepdims=True)
    return np.abs(got - want) <= 2e-2 * np.abs(want) + 1e-4 * rowmax


@pytest.mark.parametrize("name", list(CASES))
def test_value_aware_probe_route_and_attend(name):
    wl = CASES[name]
    q, k, v = synth.make_qkv(wl)
    iq = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    ik = synth.kmeans_init(k, wl.ck, wl.seed, 1)
    scale = 1 / math.sqrt(wl.d)
    print(f"[probe_values] {name}: H={wl.heads} N={wl.n} d={wl.d} {wl.dtype}", flush=True)
    res = sv().routed_attention(q.to(DEV), k.to(DEV), v.to(DEV), wl.cq, wl.ck, wl.budget,
                                wl.iters, iq.to(DEV), ik.to(DEV), scale, probe="value")
    torch.cuda.synchronize()
    rt, at = (1e-2, 2e-2) if wl.dtype == "bf16" else (1e-4, 1e-4)
    for h in range(wl.heads):
        ko = f64(res["k_off"][h])
        qo = f64(res["q_off"][h])
        kp, vp = f64(res["kp"][h]), f64(res["vp"][h])
        kb, vb = f64(res["k_bar"][h]), f64(res["v_bar"][h])
        ratio, log_norm = O.probe_values(f64(res["q_bar"][h]), kp, kb, vp, vb, ko, scale)
        got = f64(res["ratio"][h])
        sizes = np.diff(ko)
        assert np.all(got[:, sizes == 0] == -1.0)
        assert np.all(got[:, sizes == 1] == 0.0)
        ok = probe_ok(got, ratio)
        assert ok.all(), f"{(~ok).sum()} of {ok.size} ratios off; worst " \
                         f"{np.max(np.abs(got - ratio) / (np.abs(ratio) + 1e-30))}"
        np.testing.assert_allclose(f64(res["log_norm"][h]), log_norm, rtol=0, atol=5e-3)
        mask, lst, cnt, keys = O.route(got, ko, wl.budget, q_offsets=qo)
        np.testing.assert_array_equal(f64(res["sel_mask"][h]), mask)
        np.testing.assert_array_equal(f64(res["sel_keys"][h]), keys)
        want = O.attend(f64(res["qp"][h]), kp, vp, qo, ko, kb, vb, mask, scale)
        out = f64(res["op"][h])
        err = np.linalg.norm(out - want) / np.linalg.norm(want)
        assert err <= rt, err
        assert np.max(np.abs(out - want)) <= at


def test_values_at_their_means_scale_the_weight_gap_ratio():
    # vp rows replaced by their cluster's mean (rounded like the inputs): the
    # value-aware ratio is ||vbar||^2 times the plain probe's ratio.
    wl = CASES["blobs_bf16_d128"]
    q, k, v = synth.make_qkv(wl)
    iq = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    ik = synth.kmeans_init(k, wl.ck, wl.seed, 1)
    scale = 1 / math.sqrt(wl.d)
    S = sv()
    res = S.routed_attention(q.to(DEV), k.to(DEV), v.to(DEV), wl.cq, wl.ck, wl.budget, wl.iters,
                             iq.to(DEV), ik.to(DEV), scale)
    H = wl.heads
    ko = res["k_off"].long()
    sizes = (ko[:, 1:] - ko[:, :-1])
    vb_r = res["v_bar"].to(torch.bfloat16)                     # each cluster's mean, as bf16
    idx = torch.repeat_interleave(torch.arange(wl.ck, device=DEV).repeat(H),
                                  sizes.reshape(-1)).reshape(H, -1)
    vp = torch.gather(vb_r, 1, idx.unsqueeze(-1).expand(-1, -1, wl.d)).contiguous()
    vbar = vb_r.float().contiguous()                           # the exact means of those rows
    print("[probe_values] values at their means", flush=True)
    rv, _ = S.svgear_probe_values(res["q_bar"], res["kp"], res["k_bar"], vp, vbar, res["k_off"],
                                  scale)
    rw, _ = S.svgear_probe(res["q_bar"], res["kp"], res["k_bar"], res["k_off"], scale)
    torch.cuda.synchronize()
    for h in range(H):
        live = f64(sizes[h]) > 1
        w = (f64(vbar[h]) ** 2).sum(1)
        want = f64(rw[h])[:, live] * w[None, live]
        got = f64(rv[h])[:, live]
        ok = probe_ok(got, want)
        assert ok.all(), f"{(~ok).sum()} of {ok.size} off"
