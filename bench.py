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

Protocol:
  * `--warmup` untimed steps, then `--steps` steps back to back between two
    HIP events (`ms_per_step`, `value`); every stage is bracketed by events on
    the stream it runs on, and `stages_ms` and the attention roofline use the
    mean over those steps;
  * `stages_ms_median_evicted`: the median of `--stage-reps` single steps,
    each after a 512 MB write that evicts the last-level cache;
  * dense comparators: torch SDPA and our own kernel at density 1 on the same
    shape, each the mean of 5 launches after one warm-up launch;
  * `cpu_baseline`: the float64 CPU oracle on head 0, the median of
    `--cpu-reps` runs after one warm-up, with the CPU model, affinity core
    count and BLAS configuration; `oracle_routing`: the oracle's probe and
    router on the GPU's labels for heads 0 and 1 (selection flips and
    exact-entry densities);
  * `attend.frac_of_peak_at_measured_clock`: the attention rate against the
    bf16 matrix peak at the shader clock the chip holds under matrix load
    (the library's clock probe, run once per line), beside `roofline.frac`
    against the published 2.5 PFLOP/s;
  * `--sweep stress` prints one such line per routing-stress point.
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
    ap.add_argument("--stage-reps", type=int, default=20,
                    help="steps timed one at a time for the per-stage medians, each after "
                         "a write of EVICT_BYTES that evicts the last-level cache")
    ap.add_argument("--cpu-reps", type=int, default=3,
                    help="timed runs of the CPU oracle (after one untimed warm-up run when "
                         "more than one)")
    ap.add_argument("--sweep", choices=("stress",), default=None,
                    help="one line per routing-stress point: density {0.05, 0.10, 0.20, 0.30} "
                         "x C_k {250, 500, 1000}")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run one plain device copy of COPY_BYTES "
                         "(reference kernel for scaling memory counters)")
    return ap.parse_args()


COPY_BYTES = 1 << 30   # size of the --calibrate-copy copy (read once, written once)
EVICT_BYTES = 512 << 20  # written between the per-stage reps (twice the 256 MB last-level cache)
DENSE_REPS = 5
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_wan22_traffic.json")
ATTEND_SRC = os.path.join(ROOT, "sparse_attention_video_means_amd", "csrc", "svgear_attend.hip")


def measured_clock():
    """The shader clock while every matrix core is busy (the library's clock
    probe: 8 blocks of four MFMA wavefronts per compute unit; the timed
    wavefront runs ~1 ms) and the bf16 matrix peak at that clock, 4096 flops
    per clock per compute unit (four SIMDs, a 16x16x32 MFMA every 16 clocks
    each)."""
    import torch

    from sparse_attention_video_means_amd import svgear
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 8 * cus
    svgear.svgear_clock_probe(blocks, 256)
    out = svgear.svgear_clock_probe(blocks, 16384)
    torch.cuda.synchronize()
    o = out.cpu().tolist()
    khz = svgear.svgear_realtime_khz()
    mhz = (o[1] - o[0]) / (o[3] - o[2]) * khz / 1e3
    return {"mhz": mhz, "compute_units": cus, "probe_ms": (o[3] - o[2]) / khz,
            "bf16_peak_tflops": cus * 4096 * mhz * 1e6 / 1e12}


def measured_traffic(workload):
    """HBM bytes of the attention stage (its two launches) from the committed
    counter summary, or None when the kernel source or the workload differs
    from the profiled one."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
        sha = hashlib.sha256(open(ATTEND_SRC, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_stage")


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


def time_dense(q, k, v, scale, reps=DENSE_REPS):
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


def cpu_info():
    """CPU model, affinity core count and the BLAS the oracle's NumPy uses."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    from threadpoolctl import threadpool_info
    blas = [{k: p.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")}
            for p in threadpool_info()]
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)), "blas": blas}


def cpu_baseline(wl, q, k, v, iq, ik, routing, probe, reps):
    """The CPU oracle (as written, untuned) on head 0 of the same workload: one
    untimed warm-up run, then the median of `reps` timed runs (a single timed
    run when reps is 1)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import svgear_oracle as O
    f = lambda t: t.float().numpy().astype(np.float64)
    args = (f(q[0]), f(k[0]), f(v[0]), wl.cq, wl.ck, budget_for(wl, routing), wl.iters,
            f(iq[0]), f(ik[0]), 1 / math.sqrt(wl.d))
    kw = dict(routing=routing, value_aware=probe == "value")
    if reps > 1:
        O.routed_attention_head(*args, **kw)
    times = []
    for _ in range(max(1, reps)):
        t0 = time.perf_counter()
        O.routed_attention_head(*args, **kw)
        times.append(time.perf_counter() - t0)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    info = cpu_info()
    return {"value": float(np.median(times)) * 1e3, "unit": "ms/head-layer", "cores": int(threads),
            "kind": "oracle",
            "sample": f"head 0 of {wl.heads}: full routed path (k-means x2, permute, probe, route, "
                      f"attend, unpermute) in float64 NumPy, N={wl.n}, d={wl.d}; "
                      + (f"median of {reps} runs after 1 warm-up" if reps > 1 else "one run"),
            "runs_ms": [t * 1e3 for t in times], **info}


def oracle_routing_check(wl, q, k, ra, heads=(0, 1)):
    """Selection flips against the oracle's float64 probe and router, given the
    GPU's cluster labels (part of the CPU oracle leg): for each sampled head,
    the query clusters whose selected key clusters differ from the oracle's,
    and both exact-entry densities."""
    import numpy as np

    from oracle import svgear_oracle as O
    scale = 1 / math.sqrt(wl.d)
    out = {"heads": [], "flipped": 0, "query_clusters": 0}
    for h in heads:
        if h >= wl.heads:
            continue
        lq = ra.labels_q[h].cpu().numpy()
        lk = ra.labels_k[h].cpu().numpy()
        pq, qo = O.permute(lq, wl.cq)
        pk, ko = O.permute(lk, wl.ck)
        kp = k[h].float().numpy().astype(np.float64)[pk]
        qbar = O.segment_means(q[h].float().numpy().astype(np.float64)[pq], qo)
        ratio, _ = O.probe(qbar, kp, O.segment_means(kp, ko), ko, scale)
        mask, _, _, keys = O.route(ratio, ko, wl.budget, q_offsets=qo)
        gmask = ra.sel_mask[h].cpu().numpy()
        live = np.diff(qo) > 0
        flipped = int((np.any(mask != gmask, axis=1) & live).sum())
        qn = np.diff(qo).astype(np.float64)
        out["heads"].append({
            "head": h, "flipped": flipped, "query_clusters": int(live.sum()),
            "exact_density_oracle": float((qn * keys).sum()) / (wl.n * wl.n),
            "exact_density_gpu": float((qn * ra.sel_keys[h].cpu().numpy()).sum()) / (wl.n * wl.n)})
        out["flipped"] += flipped
        out["query_clusters"] += int(live.sum())
    return out


def densities(ra, n):
    """Exact-entry density (selected blocks) and computed density (exact entries
    plus one centroid entry per skipped non-empty key cluster and query), over
    all heads."""
    qn = (ra.q_off[:, 1:] - ra.q_off[:, :-1]).double()
    kn = (ra.k_off[:, 1:] - ra.k_off[:, :-1])
    exact = float((qn * ra.sel_keys.double()).sum())
    comp = float((qn * ((ra.sel_mask == 0) & (kn > 0).unsqueeze(1)).sum(-1).double()).sum())
    total = float(ra.H) * n * n
    return {"exact_entry_density": exact / total, "computed_density": (exact + comp) / total}


def stage_medians(ra, qd, kd, vd, iqd, ikd, reps):
    """Per-stage HIP-event medians over `reps` single steps, each preceded by a
    write of EVICT_BYTES so that no step finds the last one's data in the
    last-level cache."""
    import torch
    evict = torch.empty(EVICT_BYTES // 4, dtype=torch.float32, device=qd.device)
    per = {s: [] for s in ra.STAGES}
    for i in range(reps):
        evict.fill_(float(i))
        ra(qd, kd, vd, iqd, ikd, stage_events=True)
        torch.cuda.synchronize()
        for name, ms in ra.last_stage_ms().items():
            per[name].append(ms)
    del evict
    med = {}
    for name, xs in per.items():
        xs = sorted(xs)
        med[name] = xs[len(xs) // 2] if len(xs) % 2 else 0.5 * (xs[len(xs) // 2 - 1] +
                                                                 xs[len(xs) // 2])
    return med


def run(args, wl, q, k, v, iq, ik, qd, kd, vd, iqd, ikd):
    """Times the whole path on one workload and returns the JSON line."""
    import torch

    from sparse_attention_video_means_amd import svgear
    dev = qd.device
    dtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    ra = svgear.RoutedAttention(wl.heads, wl.n, wl.d, wl.cq, wl.ck, budget_for(wl, args.routing),
                                wl.iters, dtype, dev, routing=args.routing, probe=args.probe)
    for _ in range(args.warmup):
        ra(qd, kd, vd, iqd, ikd)
    torch.cuda.synchronize()
    print(f"[bench] {wl.name} Ck={wl.ck} rho={wl.rho}: warmup done", file=sys.stderr, flush=True)

    # the timed region: K whole steps back to back; the stage events are on the
    # stream every kernel runs on
    events = []
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        ra(qd, kd, vd, iqd, ikd, stage_events=True)
        events.append(ra._events)
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    stage_ms = {s: [] for s in ra.STAGES}
    for ev in events:
        for i, name in enumerate(ra.STAGES):
            stage_ms[name].append(ev[2 * i].elapsed_time(ev[2 * i + 1]))
    stages = {name: sum(x) / len(x) for name, x in stage_ms.items()}
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr,
          flush=True)
    medians = stage_medians(ra, qd, kd, vd, iqd, ikd, args.stage_reps) if args.stage_reps > 0 \
        else None

    exact, comp = algorithmic_flops(ra, wl.d)
    t_att = stages["attend"] * 1e-3
    att_tflops = (exact + comp) / t_att / 1e12
    exec_tflops = exact / t_att / 1e12
    # clustering and permutation run fused (one call per tensor), so the core
    # stages include the permutation
    core_ms = sum(stages[n] for n in ("cluster_permute_q", "cluster_permute_kv", "probe", "route",
                                      "attend"))

    extra = {}
    if not args.no_dense:
        extra = time_dense(qd, kd, vd, 1 / math.sqrt(wl.d))
        # own kernel at density 1 (every block exact) on the same permuted inputs
        ones = torch.ones_like(ra.sel_mask)
        svgear.svgear_attend(ra.qp, ra.kp, ra.vp, ra.q_off, ra.k_off, ra.k_bar, ra.v_bar, ones,
                             ra.scale)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(DENSE_REPS):
            svgear.svgear_attend(ra.qp, ra.kp, ra.vp, ra.q_off, ra.k_off, ra.k_bar, ra.v_bar,
                                 ones, ra.scale)
        b.record()
        torch.cuda.synchronize()
        extra["own_density1_ms"] = a.elapsed_time(b) / DENSE_REPS
        extra["reps"] = DENSE_REPS
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

    clock = measured_clock()
    print(f"[bench] shader clock under matrix load: {clock}", file=sys.stderr, flush=True)

    cpu, check = None, None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on head 0", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, q, k, v, iq, ik, args.routing, args.probe, args.cpu_reps)
        if args.routing == "cluster" and args.probe == "weight":
            print("[bench] oracle routing on the GPU labels, heads 0 and 1", file=sys.stderr,
                  flush=True)
            check = oracle_routing_check(wl, q, k, ra)

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
        "stages_ms_median_evicted": medians,
        "densities": densities(ra, wl.n),
        "attend": {"executed_block_tflops": exec_tflops,
                   "executed_block_frac_of_peak": exec_tflops / PEAK_BF16_TFLOPS,
                   "exact_tflop": exact / 1e12, "compensation_tflop": comp / 1e12,
                   "measured_clock_mhz": clock["mhz"],
                   "bf16_peak_tflops_at_measured_clock": clock["bf16_peak_tflops"],
                   "frac_of_peak_at_measured_clock": att_tflops / clock["bf16_peak_tflops"],
                   "executed_block_frac_at_measured_clock":
                       exec_tflops / clock["bf16_peak_tflops"]},
        "roofline": {"kernel": "attend_kernel<bf16,128> (256-query and short-tail launches)",
                     "bound": "mfma",
                     "achieved": att_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": att_tflops / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(wl.name)
                     if args.routing == "cluster" and args.probe == "weight" else None},
        "cpu_baseline": cpu,
        **({"oracle_routing": check} if check else {}),
        **({"dense": extra} if extra else {}),
    }
    del ra
    torch.cuda.empty_cache()
    return line


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path shards by head "
              "and no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)
    import torch

    from sparse_attention_video_means_amd import synth

    wl = synth.WORKLOADS["stress" if args.sweep else args.workload]
    over = {k: v for k, v in (("cq", args.cq), ("ck", args.ck), ("rho", args.rho)) if v is not None}
    if over:
        wl = wl.with_(**over)
    print(f"[bench] generating {wl.name}: H={wl.heads} N={wl.n} d={wl.d} {wl.dtype}",
          file=sys.stderr, flush=True)
    t0 = time.time()
    q, k, v = synth.make_qkv(wl, threads=16)
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = "cuda"
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    points = [(wl.ck, wl.rho)]
    if args.sweep:
        points = [(ck, rho) for ck in (250, 500, 1000) for rho in (0.05, 0.10, 0.20, 0.30)]
    iq = synth.kmeans_init(q, wl.cq, wl.seed, 0)
    for ck, rho in points:
        w = wl.with_(ck=ck, rho=rho)
        ik = synth.kmeans_init(k, w.ck, w.seed, 1)
        line = run(args, w, q, k, v, iq, ik, qd, kd, vd, iq.to(dev), ik.to(dev))
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
