#!/usr/bin/env python3
"""Benchmark of the routed sparse-attention path on one MI355X.

One step = one pass of the whole path over one attention layer of the
Wan2.2-shaped workload (40 heads x 75,600 tokens x d=128, bf16, C_q=100,
C_k=500, density 0.10, 10 Lloyd iterations): cluster(Q), cluster(K),
permute(Q), permute(K, V), probe, route, attend with the unpermutation in its
epilogue. Inputs are
generated on the host, copied to the GPU, and resident in HBM before the
timed region starts.

Prints one JSON line. `value` is milliseconds per head-layer for the whole
path (lower is better); the attention kernel's executed-block TFLOP/s and its
fraction of the bf16 matrix-core peak are in `roofline` and `attend`.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="wan22")
    ap.add_argument("--routing", choices=("cluster", "global"), default="cluster",
                    help="exact keys per query cluster (the pages' implementation) or one "
                         "budget of exact entries per head")
    ap.add_argument("--probe", choices=("weight", "value"), default="weight",
                    help="block errors from the weight gap or from the value-aware gap")
    ap.add_argument("--cq", type=int, default=None, help="override the workload's query clusters")
    ap.add_argument("--ck", type=int, default=None, help="override the workload's key clusters")
    ap.add_argument("--rho", type=float, default=None, help="override the workload's density")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run one plain device copy of COPY_BYTES "
                         "(reference kernel for scaling memory counters)")
    return ap.parse_args()


COPY_BYTES = 1 << 30   # size of the --calibrate-copy copy (read once, written once)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_wan22_traffic.json")
ATTEND_SRC = os.path.join(ROOT, "sparse_attention_video_means_amd", "csrc", "svgear_attend.hip")


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary, or
    None when the kernel source or the workload differs from the profiled one."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
        sha = hashlib.sha256(open(ATTEND_SRC, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def algorithmic_flops(ra, d):
    """4d flops per (query, exact key) pair and per (query, centroid) pair."""
    import torch
    qn = (ra.q_off[:, 1:] - ra.q_off[:, :-1]).double()              # [H, Cq]
    kn = (ra.k_off[:, 1:] - ra.k_off[:, :-1])                        # [H, Ck]
    exact = float((qn * ra.sel_keys.double()).sum()) * 4 * d
    nonempty = (kn > 0).unsqueeze(1)                                 # [H, 1, Ck]
    comp_clusters = ((ra.sel_mask == 0) & nonempty).sum(-1).double()  # [H, Cq]
    comp = float((qn * comp_clusters).sum()) * 4 * d
    del torch
    return exact, comp


def time_dense(q, k, v, scale, reps=2):
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    out = {}
    qq, kk, vv = (t.unsqueeze(0) for t in (q, k, v))
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
            b.record()
            torch.cuda.synchronize()
            out["torch_sdpa_ms"] = a.elapsed_time(b) / reps
    except Exception as e:  # noqa: BLE001
        out["torch_sdpa_error"] = str(e)[:200]
    return out


def budget_for(wl, routing):
    """Exact keys per query cluster, or exact (query, key) entries per head."""
    return wl.budget if routing == "cluster" else int(math.floor(wl.rho * wl.n * wl.n))


def cpu_baseline(wl, q, k, v, iq, ik, routing, probe):
    """The CPU oracle (as written, untuned) on head 0 of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import svgear_oracle as O
    f = lambda t: t.float().numpy().astype(np.float64)
    t0 = time.perf_counter()
    O.routed_attention_head(f(q[0]), f(k[0]), f(v[0]), wl.cq, wl.ck, budget_for(wl, routing),
                            wl.iters, f(iq[0]), f(ik[0]), 1 / math.sqrt(wl.d), routing=routing,
                            value_aware=probe == "value")
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": dt * 1e3, "unit": "ms/head-layer", "cores": int(threads), "kind": "oracle",
            "sample": f"head 0 of {wl.heads}: full routed path (k-means x2, permute, probe, route, "
                      f"attend, unpermute) in float64 NumPy, N={wl.n}, d={wl.d}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards by head "
              "and no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)
    import torch

    from sparse_attention_video_means_amd import svgear, synth

    wl = synth.WORKLOADS[args.workload]
    over = {k: v for k, v in (("cq", args.cq), ("ck", args.ck), ("rho", args.rho)) if v is not None}
    if over:
        wl = wl.with_(**over)
    print(f"[bench] generating {wl.name}: H={wl.heads} N={wl.n} d={wl.d} {wl.dtype}",
          file=sys.stderr, flush=True)
    t0 = time.time()
    q, k, v = synth.make_qkv(wl, threads=16)
    iq = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    ik = synth.kmeans_init(k, wl.ck, wl.seed, 1)
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = "cuda"
    qd, kd, vd, iqd, ikd = (t.to(dev) for t in (q, k, v, iq, ik))
    dtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    ra = svgear.RoutedAttention(wl.heads, wl.n, wl.d, wl.cq, wl.ck, budget_for(wl, args.routing),
                                wl.iters, dtype, dev, routing=args.routing, probe=args.probe)
    for _ in range(args.warmup):
        ra(qd, kd, vd, iqd, ikd)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    stage_ms = {s: [] for s in ra.STAGES}
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        ra(qd, kd, vd, iqd, ikd, stage_events=True)
        # stage events of this step are read after the loop from copies
        stage_ms_step = ra._events
        stage_ms.setdefault("_events", []).append(stage_ms_step)
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    for ev in stage_ms.pop("_events"):
        for i, s in enumerate(ra.STAGES):
            stage_ms[s].append(ev[2 * i].elapsed_time(ev[2 * i + 1]))
    stages = {s: sum(x) / len(x) for s, x in stage_ms.items()}
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr,
          flush=True)

    exact, comp = algorithmic_flops(ra, wl.d)
    t_att = stages["attend"] * 1e-3
    att_tflops = (exact + comp) / t_att / 1e12
    exec_tflops = exact / t_att / 1e12
    # clustering and permutation run fused (one call per tensor), so the core
    # stages include the permutation
    core_ms = stages["cluster_permute_q"] + stages["cluster_permute_kv"] + stages["probe"] + \
        stages["route"] + stages["attend"]

    extra = {}
    if not args.no_dense:
        extra = time_dense(qd, kd, vd, 1 / math.sqrt(wl.d))
        # own kernel at density 1 (every block exact) on the same permuted inputs
        ones = torch.ones_like(ra.sel_mask)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        svgear.svgear_attend(ra.qp, ra.kp, ra.vp, ra.q_off, ra.k_off, ra.k_bar, ra.v_bar, ones,
                             ra.scale)
        torch.cuda.synchronize()
        a.record()
        svgear.svgear_attend(ra.qp, ra.kp, ra.vp, ra.q_off, ra.k_off, ra.k_bar, ra.v_bar, ones,
                             ra.scale)
        b.record()
        torch.cuda.synchronize()
        extra["own_density1_ms"] = a.elapsed_time(b)
        dense = [x for x in (extra.get("torch_sdpa_ms"), extra["own_density1_ms"]) if x]
        extra["dense_ms"] = min(dense)
        extra["core_over_dense"] = core_ms / extra["dense_ms"]
        print(f"[bench] dense comparators: {extra}", file=sys.stderr, flush=True)

    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)  # one elementwise kernel: COPY_BYTES read, COPY_BYTES written
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on head 0", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, q, k, v, iq, ik, args.routing, args.probe)

    line = {
        "metric": "routed attn ms/head-layer + executed-block TFLOP/s vs bf16 MFMA peak",
        "value": ms_per_step / wl.heads,
        "unit": "ms/head-layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": False,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: H={wl.heads} N={wl.n} d={wl.d} {wl.dtype} "
                               f"Cq={wl.cq} Ck={wl.ck} rho={wl.rho} iters={wl.iters}"
                               + ("" if args.routing == "cluster" else " global routing")
                               + ("" if args.probe == "weight" else " value-aware probe"),
                   "heads": wl.heads, "n": wl.n, "d": wl.d, "cq": wl.cq, "ck": wl.ck,
                   "rho": wl.rho, "iters": wl.iters, "routing": args.routing,
                   "probe": args.probe,
                   **({"budget_keys": wl.budget} if args.routing == "cluster" else
                      {"budget_entries": budget_for(wl, "global")})},
        "core_ms_per_head_layer": core_ms / wl.heads,
        "stages_ms": stages,
        "attend": {"executed_block_tflops": exec_tflops,
                   "executed_block_frac_of_peak": exec_tflops / PEAK_BF16_TFLOPS,
                   "exact_tflop": exact / 1e12, "compensation_tflop": comp / 1e12},
        "roofline": {"kernel": "attend_kernel<bf16,128>", "bound": "mfma",
                     "achieved": att_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": att_tflops / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(wl.name)
                     if args.routing == "cluster" and args.probe == "weight" else None},
        "cpu_baseline": cpu,
        **({"dense": extra} if extra else {}),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
