"""GPU parity of the error-analysis calls (paper §5.3) against the CPU oracle
(needs an MI355X).

svgear_block_scores must match ``oracle.block_scores`` to f32 accuracy on the
GPU's centroids. svgear_map_error must match ``oracle.attention_map_error``
per query, for masks from the error-aware router, from the score ranking, the
full mask and the empty one, with and without compensation: the squared error
within 2e-2 relative plus 1e-6 of the query's squared full-map norm, and both
normalisers within 1e-4 relative (the logits come from the same bf16 or f32
operands on both sides).
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
    "blobs_bf16": synth.WORKLOADS["slice"].with_(name="an_blobs", heads=2, n=3001, cq=24, ck=70,
                                                 iters=5, centres=64),
    "lattice_bf16_d64": synth.WORKLOADS["wan22"].with_(name="an_lattice", heads=1, d=64,
                                                       n=6 * 12 * 20, grid=(6, 12, 20), cq=16,
                                                       ck=50, iters=4, rho=0.2),
}


def sv():
    from sparse_attention_video_means_amd import svgear
    return svgear


def f64(t):
    if t.dtype in (torch.int32, torch.uint8):
        return t.detach().cpu().numpy()
    return t.detach().float().cpu().double().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_scores_and_map_error(name):
    wl = CASES[name]
    S = sv()
    q, k, v = synth.make_qkv(wl)
    iq = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    ik = synth.kmeans_init(k, wl.ck, wl.seed, 1)
    scale = 1 / math.sqrt(wl.d)
    print(f"[analysis] {name}: H={wl.heads} N={wl.n} d={wl.d} {wl.dtype}", flush=True)
    res = S.routed_attention(q.to(DEV), k.to(DEV), v.to(DEV), wl.cq, wl.ck, wl.budget, wl.iters,
                             iq.to(DEV), ik.to(DEV), scale)
    scores = S.svgear_block_scores(res["q_bar"], res["k_bar"], res["k_off"], scale)
    smask, _, _, _ = S.svgear_route(scores, res["k_off"], wl.budget)
    masks = {"error_aware": res["sel_mask"], "scores": smask,
             "full": torch.ones_like(smask), "empty": torch.zeros_like(smask)}
    out = {}
    for mname, mk in masks.items():
        for comp in (True, False):
            out[mname, comp] = S.svgear_map_error(res["qp"], res["kp"], res["q_off"], res["k_off"],
                                                  res["k_bar"], mk, scale, compensate=comp)
    torch.cuda.synchronize()
    for h in range(wl.heads):
        qo, ko = f64(res["q_off"][h]), f64(res["k_off"][h])
        want_sc = O.block_scores(f64(res["q_bar"][h]), f64(res["k_bar"][h]), ko, scale)
        np.testing.assert_allclose(f64(scores[h]), want_sc, rtol=2e-5, atol=1e-9)
        qp, kp, kb = f64(res["qp"][h]), f64(res["kp"][h]), f64(res["k_bar"][h])
        # each query's squared full-map norm: the error of keeping nothing, uncompensated
        norm2, _, _ = O.attention_map_error(qp, kp, qo, ko, kb, np.zeros((wl.cq, wl.ck), np.uint8),
                                            scale, compensate=False)
        for xp_key, mu_key, off_key in (("qp", "q_bar", "q_off"), ("kp", "k_bar", "k_off")):
            got = f64(S.svgear_row_spread(res[xp_key], res[mu_key], res[off_key])[h])
            want = O.row_spread(f64(res[xp_key][h]), f64(res[off_key][h]), f64(res[mu_key][h]))
            np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-6 * want.max())
        for (mname, comp), (err, zf, zs) in out.items():
            w_err, w_zf, w_zs = O.attention_map_error(qp, kp, qo, ko, kb, f64(masks[mname][h]),
                                                      scale, compensate=comp)
            g_err = f64(err[h])
            ok = np.abs(g_err - w_err) <= 2e-2 * w_err + 1e-6 * norm2
            assert ok.all(), (mname, comp, int((~ok).sum()))
            np.testing.assert_allclose(f64(zf[h]), w_zf, rtol=1e-4)
            np.testing.assert_allclose(f64(zs[h]), w_zs, rtol=1e-4, atol=1e-30)


def test_harness_runs_and_matches_its_budget():
    from sparse_attention_video_means_amd import analysis
    print("[analysis] harness on the tiny workload", flush=True)
    lines = analysis.run("tiny", [0.1, 0.5])
    for line, rho in zip(lines, (0.1, 0.5)):
        for name in ("topp_drop", "topp_comp", "error_aware_comp", "value_aware_comp"):
            rec = line[name]
            assert np.isfinite(rec["mse"]) and rec["mse"] >= 0
            assert 0 < rec["density"] <= rho + 1e-12
        # compensating the same blocks never needs more keys than dropping them
        assert line["topp_comp"]["density"] == line["topp_drop"]["density"]


def test_cq_sweep_runs():
    from sparse_attention_video_means_amd import analysis
    print("[analysis] C_q sweep on a small slice", flush=True)
    lines = analysis.sweep_cq("slice", [8, 32], 0.2, heads=1, n=2048)
    assert lines[0]["delta_q2_mean"] > lines[1]["delta_q2_mean"] > 0
    for line in lines:
        assert line["delta_q2_max"] >= line["delta_q2_mean"]
        assert np.isfinite(line["error_aware_comp"]["mse"])
