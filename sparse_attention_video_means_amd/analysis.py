"""Block-selection error analysis on the GPU (SVG-EAR §5.3, "Strategy of
block selection", Fig. 6a).

For one workload the path runs once up to the probe (k-means of Q and K,
permutation, both probes). Then, for each density rho, the same budget of
floor(rho * N_k) exact keys per query cluster is filled three ways and the
attention map of every head is compared with the full map,
    mse = (1 / (N_q N_k)) sum_i sum_j (A_sparse - A_full)_ij^2,
for
  * top-p: blocks in decreasing centroid-estimated attention mass, skipped
    blocks dropped (SVG2's selection);
  * top-p + compensation: the same blocks, skipped blocks compensated;
  * error-aware routing + compensation (the method), and the same with the
    value-aware probe.
The mean relative change of the softmax normaliser, |Z_sparse / Z_full - 1|,
is reported for every compensated variant (§4.2 reports 4.18% for the method
in a video model). One JSON line per density:

    python -m sparse_attention_video_means_amd.analysis --workload slice \\
        --densities 0.05,0.1,0.2,0.3

With ``--sweep-cq`` the number of query clusters varies instead (§5.3 "Effect
of clustering", Fig. 6b): for each C_q the line gives the queries' clustering
error delta_q^2 (mean squared distance of a query from its cluster mean, and
the maximum) and the map MSE of the method at one density:

    python -m sparse_attention_video_means_amd.analysis --workload slice \\
        --sweep-cq 25,50,100,200,300 --densities 0.1

With ``--turbo`` each setting C_q:C_k:rho (fewer centroids and a lower density
budget, the trade of §5.1's SVG-EAR-turbo) runs the whole routed path as the
benchmark does, timed per stage over a few passes, and reports its map MSE,
normaliser change and exact density next to top-p with compensation at the
same budget:

    python -m sparse_attention_video_means_amd.analysis --workload wan22 \\
        --turbo 100:500:0.1,50:250:0.1,50:250:0.05
"""
from __future__ import annotations

import argparse
import json
import math
import sys

import torch

from . import svgear, synth


def run(workload: str, densities, heads: int | None = None, n: int | None = None):
    wl = synth.WORKLOADS[workload]
    if heads:
        wl = wl.with_(heads=heads)
    if n:
        wl = wl.with_(n=n)
    dev = "cuda"
    q, k, v = synth.make_qkv(wl, threads=16)
    iq = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    ik = synth.kmeans_init(k, wl.ck, wl.seed, 1)
    scale = 1 / math.sqrt(wl.d)
    res = svgear.routed_attention(q.to(dev), k.to(dev), v.to(dev), wl.cq, wl.ck, wl.budget,
                                  wl.iters, iq.to(dev), ik.to(dev), scale)
    qp, kp, q_off, k_off = res["qp"], res["kp"], res["q_off"], res["k_off"]
    ratio_w = res["ratio"]
    ratio_v, _ = svgear.svgear_probe_values(res["q_bar"], kp, res["k_bar"], res["vp"],
                                            res["v_bar"], k_off, scale)
    scores = svgear.svgear_block_scores(res["q_bar"], res["k_bar"], k_off, scale)
    qn = (q_off[:, 1:] - q_off[:, :-1]).double()
    total = float(wl.heads) * wl.n * wl.n
    out = []
    for rho in densities:
        budget = int(math.floor(rho * wl.n))
        line = {"workload": f"{wl.name}: H={wl.heads} N={wl.n} d={wl.d} {wl.dtype} "
                            f"Cq={wl.cq} Ck={wl.ck} iters={wl.iters}",
                "rho": rho, "budget_keys": budget}
        variants = (("topp_drop", scores, False), ("topp_comp", scores, True),
                    ("error_aware_comp", ratio_w, True), ("value_aware_comp", ratio_v, True))
        for name, ratio, comp in variants:
            mask, _, _, keys = svgear.svgear_route(ratio, k_off, budget, q_off)
            err, zf, zs = svgear.svgear_map_error(qp, kp, q_off, k_off, res["k_bar"], mask,
                                                  scale, compensate=comp)
            rec = {"mse": float(err.double().sum()) / total,
                   "density": float((qn * keys.double()).sum()) / total}
            if comp:
                rec["normaliser_change"] = float((zs.double() / zf.double() - 1).abs().mean())
            line[name] = rec
        out.append(line)
        print(json.dumps(line), flush=True)
    return out


def sweep_cq(workload: str, cqs, rho: float, heads: int | None = None, n: int | None = None):
    base = synth.WORKLOADS[workload]
    if heads:
        base = base.with_(heads=heads)
    if n:
        base = base.with_(n=n)
    dev = "cuda"
    q, k, v = synth.make_qkv(base, threads=16)
    ik = synth.kmeans_init(k, base.ck, base.seed, 1)
    scale = 1 / math.sqrt(base.d)
    total = float(base.heads) * base.n * base.n
    budget = int(math.floor(rho * base.n))
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = []
    for cq in cqs:
        wl = base.with_(cq=cq)
        iq = synth.kmeans_init(q, cq, wl.seed, 0)
        res = svgear.routed_attention(qd, kd, vd, cq, wl.ck, budget, wl.iters, iq.to(dev),
                                      ik.to(dev), scale)
        spread = svgear.svgear_row_spread(res["qp"], res["q_bar"], res["q_off"]).double()
        line = {"workload": f"{wl.name}: H={wl.heads} N={wl.n} d={wl.d} {wl.dtype} "
                            f"Ck={wl.ck} iters={wl.iters}",
                "cq": cq, "rho": rho, "budget_keys": budget,
                "delta_q2_mean": float(spread.mean()), "delta_q2_max": float(spread.max())}
        scores = svgear.svgear_block_scores(res["q_bar"], res["k_bar"], res["k_off"], scale)
        for name, ratio in (("error_aware_comp", res["ratio"]), ("topp_comp", scores)):
            mask, _, _, _ = svgear.svgear_route(ratio, res["k_off"], budget, res["q_off"])
            err, zf, zs = svgear.svgear_map_error(res["qp"], res["kp"], res["q_off"], res["k_off"],
                                                  res["k_bar"], mask, scale, compensate=True)
            line[name] = {"mse": float(err.double().sum()) / total,
                          "normaliser_change": float((zs.double() / zf.double() - 1).abs().mean())}
        out.append(line)
        print(json.dumps(line), flush=True)
    return out


def turbo(workload: str, settings, heads: int | None = None, n: int | None = None,
          reps: int = 3):
    base = synth.WORKLOADS[workload]
    if heads:
        base = base.with_(heads=heads)
    if n:
        base = base.with_(n=n)
    dev = "cuda"
    q, k, v = synth.make_qkv(base, threads=16)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    dtype = torch.bfloat16 if base.dtype == "bf16" else torch.float32
    total = float(base.heads) * base.n * base.n
    out = []
    for cq, ck, rho in settings:
        wl = base.with_(cq=cq, ck=ck, rho=rho)
        iq = synth.kmeans_init(q, cq, wl.seed, 0).to(dev)
        ik = synth.kmeans_init(k, ck, wl.seed, 1).to(dev)
        ra = svgear.RoutedAttention(wl.heads, wl.n, wl.d, cq, ck, wl.budget, wl.iters, dtype, dev)
        ra(qd, kd, vd, iq, ik)
        stages = {s: 0.0 for s in ra.STAGES}
        events = []
        for _ in range(reps):
            ra(qd, kd, vd, iq, ik, stage_events=True)
            events.append(ra._events)
        torch.cuda.synchronize()
        for ev in events:
            for i, name in enumerate(ra.STAGES):
                stages[name] += ev[2 * i].elapsed_time(ev[2 * i + 1]) / reps
        core = sum(stages.values())
        qn = (ra.q_off[:, 1:] - ra.q_off[:, :-1]).double()
        line = {"workload": f"{wl.name}: H={wl.heads} N={wl.n} d={wl.d} {wl.dtype} "
                            f"iters={wl.iters}",
                "cq": cq, "ck": ck, "rho": rho, "budget_keys": wl.budget,
                "core_ms": core, "stages_ms": stages}
        scores = svgear.svgear_block_scores(ra.q_bar, ra.k_bar, ra.k_off, ra.scale)
        for name, mask in (("error_aware_comp", ra.sel_mask),
                           ("topp_comp", svgear.svgear_route(scores, ra.k_off, wl.budget, ra.q_off)[0])):
            err, zf, zs = svgear.svgear_map_error(ra.qp, ra.kp, ra.q_off, ra.k_off, ra.k_bar, mask,
                                                  ra.scale, compensate=True)
            keys = mask.to(torch.int64).mul(
                (ra.k_off[:, 1:] - ra.k_off[:, :-1]).to(torch.int64)[:, None, :]).sum(2)
            line[name] = {"mse": float(err.double().sum()) / total,
                          "normaliser_change": float((zs.double() / zf.double() - 1).abs().mean()),
                          "density": float((qn * keys.double()).sum()) / total}
        out.append(line)
        print(json.dumps(line), flush=True)
        del ra
        torch.cuda.empty_cache()
    return out


def parse_turbo(text: str):
    """'C_q:C_k:rho,...' -> [(C_q, C_k, rho), ...]; raises ValueError on a malformed item."""
    settings = []
    for item in text.split(","):
        parts = item.split(":")
        if len(parts) != 3:
            raise ValueError(f"turbo setting {item!r} is not C_q:C_k:rho")
        cq, ck, rho = int(parts[0]), int(parts[1]), float(parts[2])
        if cq < 1 or ck < 1 or not 0.0 <= rho <= 1.0:
            raise ValueError(f"turbo setting {item!r} is out of range")
        settings.append((cq, ck, rho))
    return settings


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="slice", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--densities", default="0.05,0.1,0.2,0.3")
    ap.add_argument("--heads", type=int, default=None, help="use only this many heads")
    ap.add_argument("--n", type=int, default=None, help="override the token count")
    ap.add_argument("--sweep-cq", default=None,
                    help="comma-separated query-cluster counts (uses the first density)")
    ap.add_argument("--turbo", default=None,
                    help="comma-separated C_q:C_k:rho settings, each timed on the whole path")
    args = ap.parse_args(argv)
    settings = parse_turbo(args.turbo) if args.turbo else None
    if not torch.cuda.is_available():
        print("the analysis runs on the GPU kernels; no GPU is visible", file=sys.stderr)
        return 2
    densities = [float(x) for x in args.densities.split(",")]
    if settings:
        turbo(args.workload, settings, args.heads, args.n)
    elif args.sweep_cq:
        sweep_cq(args.workload, [int(x) for x in args.sweep_cq.split(",")], densities[0],
                 args.heads, args.n)
    else:
        run(args.workload, densities, args.heads, args.n)
    return 0


if __name__ == "__main__":
    sys.exit(main())
