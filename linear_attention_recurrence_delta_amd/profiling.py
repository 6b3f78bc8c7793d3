"""Summaries of rocprofv3 output for the committed profiles.

    python -m linear_attention_recurrence_delta_amd.profiling stats KERNEL_STATS_CSV --title T --command C
        -> markdown table of per-kernel launch counts and durations
    python -m linear_attention_recurrence_delta_amd.profiling traffic \
        --fetch CSV --write CSV --copy-fetch CSV --copy-write CSV --copy-bytes N [--out JSON]
        -> HBM bytes per launch of each libgdn kernel
    python -m linear_attention_recurrence_delta_amd.profiling mfma COUNTER_CSV KERNEL_STATS_CSV BENCH_JSON
        -> per kernel: MFMA busy fraction, bf16 MFMA flops executed per launch,
           the rate those flops give over the traced mean duration, and the
           method's algorithmic flops beside them

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same
counter reads for a plain device copy of known size (bench.py
--copy-calibration N reads N bytes and writes N bytes per launch), so that
the reported bytes are in the copy's units.
"""
import argparse
import csv
import hashlib
import json
import os
import re
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))

# kernel -> source file that defines it
SOURCES = {"gdn_k1_chunk_prep": "gdn_prefill.hip", "gdn_k2_inverse_w": "gdn_prefill.hip",
           "gdn_k3_scan": "gdn_prefill.hip", "gdn_kd_decode_step": "gdn_decode.hip",
           "gdn_kd_decode_multi": "gdn_decode.hip", "gdn_kb_dstate": "gdn_backward.hip",
           "gdn_kb_grad": "gdn_backward.hip"}


def source_of(kernel):
    """Source file of a kernel summary name (instance labels ignored)."""
    return SOURCES.get(kernel.split(" [")[0])


# compile-time switches of each kernel, in template-argument order (the bool
# arguments follow the dtype and sizes); a true switch labels the instance
FLAGS = {"gdn_k2_inverse_w": ("prep", "gate-only", "bwd", "window"),
         "gdn_k3_scan": ("gate-only", "save", "window"), "gdn_kd_decode_step": ("prep", "gate-only"),
         "gdn_kd_decode_multi": ("prep", "gate-only")}


def short_name(name):
    """Kernel name without template arguments, with the names of the
    instance's true compile-time switches in brackets (from the mangled
    `Lb1E` / demangled `true` bool arguments)."""
    m = re.search(r"(gdn_k\w+?)(?:I|\(|<|E|$)", name)
    if not m:
        return name.split("(")[0][:60]
    base = m.group(1)
    bools = re.findall(r"Lb([01])E", name) or [("1" if b == "true" else "0")
                                                for b in re.findall(r"\b(true|false)\b", name)]
    on = [f for f, b in zip(FLAGS.get(base, ()), bools) if b == "1"]
    return base + (f" [{', '.join(on)}]" if on else "")


def kernel_stats(path):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append(r)
    out = ["| kernel | calls | avg (us) | min (us) | max (us) | total (us) | % |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        ns = lambda k: float(r[k]) / 1000.0  # noqa: E731
        out.append(f"| {short_name(r['Name'])} | {r['Calls']} | {ns('AverageNs'):.1f} | "
                   f"{ns('MinNs'):.1f} | {ns('MaxNs'):.1f} | {ns('TotalDurationNs'):.1f} | "
                   f"{float(r['Percentage']):.1f} |")
    return "\n".join(out)


def counter_per_kernel(path, counter):
    vals = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}


def copy_counter(path, counter):
    vals = [v for k, v in counter_per_kernel(path, counter).items() if "gdn_" not in k]
    if not vals:
        raise SystemExit(f"no copy kernel in {path}")
    return max(vals)


def traffic(fetch, write, copy_fetch, copy_write, copy_bytes):
    fsc = copy_bytes / (copy_counter(copy_fetch, "FETCH_SIZE") * 1024.0)
    wsc = copy_bytes / (copy_counter(copy_write, "WRITE_SIZE") * 1024.0)
    f = counter_per_kernel(fetch, "FETCH_SIZE")
    w = counter_per_kernel(write, "WRITE_SIZE")
    out = {"_calibration": {"copy_bytes_each_way": copy_bytes, "fetch_scale": round(fsc, 4),
                            "write_scale": round(wsc, 4)}}
    for k in sorted(set(f) & set(w)):
        if source_of(k) is None:
            continue
        src = os.path.join(HERE, "csrc", source_of(k))
        with open(src, "rb") as fh:
            sha = hashlib.sha256(fh.read()).hexdigest()
        fb, wb = f[k] * 1024.0 * fsc, w[k] * 1024.0 * wsc
        out[k] = {"source": source_of(k), "source_sha256": sha, "fetch_kib_raw": f[k],
                  "write_kib_raw": w[k], "fetch_bytes": round(fb), "write_bytes": round(wb),
                  "bytes_per_launch": round(fb + wb)}
    return out


def traffic_table(traffic_path, bench_path):
    """Markdown table: measured HBM bytes per launch (traffic.json) beside the
    algorithmic bytes bench.py counts (its achieved GB/s times the launch's
    mean time), for every kernel in both."""
    with open(traffic_path) as f:
        tr = json.load(f)
    with open(bench_path) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    kernels = dict(line.get("kernels", {}))
    kernels.update(line.get("backward", {}).get("kernels", {}))
    rows = ["| kernel | fetch (GB) | write (GB) | measured total (GB) | algorithmic (GB) | ratio |",
            "|---|---|---|---|---|---|"]
    for k, rec in kernels.items():
        if k not in tr or "hbm_frac" not in rec:
            continue
        alg = rec["hbm_frac"] * PEAK_HBM_BYTES * rec["ms"] * 1e-3
        m = tr[k]
        rows.append(f"| {k} | {m['fetch_bytes'] / 1e9:.3f} | {m['write_bytes'] / 1e9:.3f} | "
                    f"{m['bytes_per_launch'] / 1e9:.3f} | {alg / 1e9:.3f} | {m['bytes_per_launch'] / alg:.2f} |")
    return "\n".join(rows)


PEAK_HBM_BYTES = 8.0e12       # MI355X HBM3E
PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
SIMD_NUM = 256 * 4            # MI355X: 256 CUs of 4 SIMDs


def mean_durations(stats_csv):
    """Kernel summary name -> mean duration (s) from a --stats CSV (the
    calls of instances that share a summary name pooled)."""
    tot, calls = {}, {}
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            k = short_name(r["Name"])
            tot[k] = tot.get(k, 0.0) + float(r["TotalDurationNs"]) * 1e-9
            calls[k] = calls.get(k, 0) + int(r["Calls"])
    return {k: tot[k] / calls[k] for k in tot}


def mfma_table(counter_csv, stats_csv, bench_path):
    """Markdown table of the MFMA counters of each libgdn kernel: MfmaUtil
    (busy MFMA cycles summed over SIMDs / (GRBM_GUI_ACTIVE x SIMD count)),
    MfmaFlopsBF16 (512 x SQ_INSTS_VALU_MFMA_MOPS_BF16: the flops of the bf16
    MFMA instructions the kernel executed, padding included) and the rate
    those give over the kernel's mean traced duration, beside the method's
    algorithmic flops from bench.py's line."""
    util = counter_per_kernel(counter_csv, "MfmaUtil")
    flops = counter_per_kernel(counter_csv, "MfmaFlopsBF16")
    dur = mean_durations(stats_csv)
    with open(bench_path) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    kernels = dict(line.get("kernels", {}))
    kernels.update(line.get("backward", {}).get("kernels", {}))
    rows = ["| kernel | MfmaUtil (%) | bf16 MFMA flops executed (G) | mean traced duration (us) | "
            "executed rate (TFLOP/s) | executed / peak | algorithmic flops (G) | algorithmic / executed |",
            "|---|---|---|---|---|---|---|---|"]
    for k in sorted(set(util) & set(flops)):
        if source_of(k) is None or k not in dur:
            continue
        rate = flops[k] / dur[k]
        rec = kernels.get(k)
        alg = rec["mfma_frac"] * PEAK_BF16_FLOPS * rec["ms"] * 1e-3 if rec and "mfma_frac" in rec else None
        rows.append(f"| {k} | {util[k]:.1f} | {flops[k] / 1e9:.1f} | {dur[k] * 1e6:.1f} | {rate / 1e12:.1f} | "
                    f"{rate / PEAK_BF16_FLOPS:.4f} | " + ("-" if alg is None else f"{alg / 1e9:.1f}") + " | "
                    + ("-" if alg is None or not flops[k] else f"{alg / flops[k]:.2f}") + " |")
    return "\n".join(rows)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--title", default="Kernel trace")
    s.add_argument("--command", default="")
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--out")
    tt = sub.add_parser("traffic-table")
    tt.add_argument("traffic_json")
    tt.add_argument("bench_json")
    mf = sub.add_parser("mfma")
    mf.add_argument("counter_csv")
    mf.add_argument("stats_csv")
    mf.add_argument("bench_json")
    args = ap.parse_args()
    if args.cmd == "mfma":
        print(mfma_table(args.counter_csv, args.stats_csv, args.bench_json))
        return
    if args.cmd == "traffic-table":
        print(traffic_table(args.traffic_json, args.bench_json))
        return
    if args.cmd == "stats":
        print(f"# {args.title}\n\nCommand (MI355X, repo root):\n\n    {args.command}\n")
        print(kernel_stats(args.csv))
    else:
        res = traffic(args.fetch, args.write, args.copy_fetch, args.copy_write, args.copy_bytes)
        text = json.dumps(res, indent=1)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text + "\n")
        print(text)


if __name__ == "__main__":
    main()
