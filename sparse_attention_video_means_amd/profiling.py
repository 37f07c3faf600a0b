"""Summaries of rocprofv3 output for the profile records under profiles/.

    python -m sparse_attention_video_means_amd.profiling kernels TRACE_DIR [PASSES]
        per-kernel table (calls, total ms, average us, share of the traced
        time) from a `rocprofv3 --kernel-trace --stats --output-format csv`
        run; with PASSES, also the time per pass.

    python -m sparse_attention_video_means_amd.profiling traffic FETCH_DIR WRITE_DIR OUT
        HBM bytes of the attention stage (both attention launches of one pass)
        from two counter runs, `rocprofv3 --pmc FETCH_SIZE` and `rocprofv3
        --pmc WRITE_SIZE`, of `bench.py --steps 1 --warmup 0 --stage-reps 0
        --no-cpu-baseline --no-dense --calibrate-copy`. Each counter is scaled
        by what it reports for the calibration copy of that run (one
        elementwise kernel that reads and writes COPY_BYTES), and the record
        keeps the sha256 of the attention source, so that bench.py drops the
        figure once the kernel changes.

Only reads CSV files; runs nothing on the GPU.
"""
import collections
import csv
import glob
import hashlib
import json
import os
import sys

COPY_BYTES = 1 << 30
ATTEND_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "svgear_attend.hip")


def short_name(name: str) -> str:
    """A readable kernel name: the function name without its argument list,
    with the attention kernel's two configurations told apart."""
    base = name.split("(")[0].strip('"')
    if "attend_kernel" in name:
        tail = "short-tail launch" if "AttTailCfg" in name else "256-query launch"
        typ = "bf16" if ("DF16b" in name or "__bf16" in name) else "f32"
        dim = "128" if ("Li128E" in name or ",128" in name) else "64"
        return f"attend_kernel<{typ},{dim}> ({tail})"
    if base.startswith("_Z"):
        # mangled: keep the identifier that follows the namespace
        for marker in ("3svg",):
            i = base.find(marker)
            if i >= 0:
                rest = base[i + len(marker):]
                digits = ""
                while rest and rest[0].isdigit():
                    digits += rest[0]
                    rest = rest[1:]
                if digits:
                    return rest[:int(digits)]
    if base.startswith("void "):
        base = base[5:]
    return base.replace("svg::", "")


def kernel_table(trace_dir: str, passes: int = 0) -> str:
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = list(csv.DictReader(open(files[0])))
    agg = collections.OrderedDict()
    for r in rows:
        k = short_name(r["Name"])
        a = agg.setdefault(k, [0, 0.0])
        a[0] += int(r["Calls"])
        a[1] += float(r["TotalDurationNs"])
    total = sum(v[1] for v in agg.values())
    out = ["| kernel | calls | total ms | avg us | share |" + (" ms / pass |" if passes else ""),
           "|---|---:|---:|---:|---:|" + ("---:|" if passes else "")]
    for k, (calls, ns) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        line = f"| {k} | {calls} | {ns / 1e6:.3f} | {ns / calls / 1e3:.1f} | {100 * ns / total:.1f}% |"
        if passes:
            line += f" {ns / 1e6 / passes:.3f} |"
        out.append(line)
    return "\n".join(out)


def _counter_rows(run_dir: str, counter: str):
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = collections.OrderedDict()  # dispatch -> (kernel name, summed value)
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, v = per.get(d, (r["Kernel_Name"], 0.0))
            per[d] = (name, v + float(r["Counter_Value"]))
    return per


def traffic_record(fetch_dir: str, write_dir: str, workload: str = "wan22") -> dict:
    rec = {"kernel": "attend_kernel<bf16,128> (256-query and short-tail launches of one pass)",
           "workload": workload,
           "source_sha256": hashlib.sha256(open(ATTEND_SRC, "rb").read()).hexdigest(),
           "copy_bytes": COPY_BYTES}
    total = 0.0
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _counter_rows(run_dir, counter)
        # the calibration copy: the elementwise multiply that moves the most bytes
        copies = [v for name, v in per.values() if "elementwise" in name and "Mul" in name]
        if not copies:
            raise SystemExit(f"{counter}: no calibration copy dispatch in {run_dir}")
        copy_kib = max(copies)
        passes = sum(1 for name, _ in per.values()
                     if "attend_kernel" in name and "AttTailCfg" not in name)
        if passes == 0:
            raise SystemExit(f"{counter}: no attention dispatch in {run_dir}")
        att_kib = sum(v for name, v in per.values() if "attend_kernel" in name) / passes
        scale = COPY_BYTES / (copy_kib * 1024.0)
        key = counter.split("_")[0].lower()
        rec[f"{key}_kib_per_stage"] = att_kib
        rec[f"copy_{key}_kib"] = copy_kib
        rec[f"{key}_scale"] = scale
        rec[f"{key}_passes"] = passes
        total += att_kib * 1024.0 * scale
    rec["hbm_bytes_per_stage"] = total
    rec["note"] = ("scale = known bytes of the calibration copy (torch.mul(src, 1.0, out=dst) "
                   "over 2^28 floats: 1 GiB read, 1 GiB written) / the bytes the same counter "
                   "reports for that kernel; bytes per stage = both attention launches of a pass")
    return rec


def main(argv):
    if len(argv) >= 2 and argv[0] == "kernels":
        print(kernel_table(argv[1], int(argv[2]) if len(argv) > 2 else 0))
    elif len(argv) == 4 and argv[0] == "traffic":
        rec = traffic_record(argv[1], argv[2])
        with open(argv[3], "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec, indent=1))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
