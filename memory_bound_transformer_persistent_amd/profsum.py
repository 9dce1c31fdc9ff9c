"""Summaries of rocprofv3 CSV output for the decode kernel.

Reads the CSV files that `rocprofv3 --output-format csv` writes under a
directory (kernel traces and/or counter collections) and prints a short text
summary: per kernel name, dispatch count and mean/median/min/max duration;
for the decode kernel, the same over the single-token decode launches alone
(prefill launches of many tokens are much longer and are split off by
duration); and, for counter runs, each counter's per-dispatch value.

    python -m memory_bound_transformer_persistent_amd.profsum trace DIR
    python -m memory_bound_transformer_persistent_amd.profsum dispatches DIR
    python -m memory_bound_transformer_persistent_amd.profsum counters DIR [KERNEL]
    python -m memory_bound_transformer_persistent_amd.profsum traffic FETCH_DIR WRITE_DIR \\
        COPY_FETCH_DIR COPY_WRITE_DIR COPY_BYTES KERNEL_SOURCE [WORKLOAD]

The traffic mode turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into HBM
bytes per decode launch, scaled by what the same counters read for a plain
device-to-device copy of COPY_BYTES (read once, written once), and prints
the `key = value` record that bench.py reads (kernel_sha ties it to the
kernel source it was measured on).
"""
import csv
import glob
import hashlib
import os
import statistics
import sys

DECODE_KERNEL = "dec_resident"


def _rows(d, suffix):
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def _name(r):
    return r.get("Kernel_Name") or r.get("KernelName") or r.get("Name") or "?"


def _dur_ns(r):
    return int(r["End_Timestamp"]) - int(r["Start_Timestamp"])


def _stats(v):
    return {"n": len(v), "mean": statistics.fmean(v), "median": statistics.median(v), "min": min(v), "max": max(v)}


def split_decode(durs):
    """Decode launches: those under twice the median (prefill launches are many times longer)."""
    if not durs:
        return []
    m = statistics.median(durs)
    return [x for x in durs if x < 2 * m]


def trace_summary(d):
    rows = _rows(d, "kernel_trace.csv")
    by = {}
    for r in rows:
        by.setdefault(_name(r), []).append(_dur_ns(r))
    lines = [f"{'kernel':60s} {'calls':>6s} {'mean us':>10s} {'median us':>10s} {'min us':>9s} {'max us':>10s}"]
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        s = _stats(v)
        lines.append(f"{k[:60]:60s} {s['n']:6d} {s['mean'] / 1e3:10.1f} {s['median'] / 1e3:10.1f} "
                     f"{s['min'] / 1e3:9.1f} {s['max'] / 1e3:10.1f}")
    for k, v in by.items():
        if DECODE_KERNEL in k:
            dec = split_decode(v)
            if dec:
                s = _stats(dec)
                lines.append(f"{k} single-token decode launches: n={s['n']} mean {s['mean'] / 1e3:.1f} us, "
                             f"median {s['median'] / 1e3:.1f} us, min {s['min'] / 1e3:.1f} us, max {s['max'] / 1e3:.1f} us")
    return "\n".join(lines)


def dispatch_list(d):
    """Every decode-kernel dispatch in start order with its duration: a
    decode-server launch serves many steps, so its duration is per launch."""
    rows = [r for r in _rows(d, "kernel_trace.csv") if DECODE_KERNEL in _name(r)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    t0 = int(rows[0]["Start_Timestamp"]) if rows else 0
    lines = [f"{'#':>4s} {'kernel':28s} {'start ms':>10s} {'duration us':>12s}"]
    for i, r in enumerate(rows):
        lines.append(f"{i:4d} {_name(r)[:28]:28s} {(int(r['Start_Timestamp']) - t0) / 1e6:10.3f} {_dur_ns(r) / 1e3:12.1f}")
    return "\n".join(lines)


def counter_values(d, kernel=DECODE_KERNEL, names=None):
    """{counter: [value per dispatch]} for dispatches of `kernel` (a name substring),
    plus their durations (ns); the matching kernel names are added to `names`."""
    rows = _rows(d, "counter_collection.csv")
    per = {}
    dur = {}
    for r in rows:
        if kernel not in _name(r):
            continue
        if names is not None:
            names.add(_name(r))
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        c = r.get("Counter_Name")
        per.setdefault(c, {}).setdefault(key, 0.0)
        per[c][key] += float(r["Counter_Value"])
        if "Start_Timestamp" in r and r["Start_Timestamp"]:
            dur[key] = _dur_ns(r)
    return per, dur


def decode_counter(d, counter, kernel=DECODE_KERNEL, names=None):
    """Median of `counter` over the single-token decode dispatches of `kernel`."""
    per, dur = counter_values(d, kernel, names)
    vals = per.get(counter, {})
    if not vals:
        raise SystemExit(f"no {counter} values for {kernel} under {d}")
    keys = list(vals)
    if dur:
        keep = set(k for k in keys if k in dur and dur[k] < 2 * statistics.median([dur[x] for x in keys if x in dur]))
        keys = [k for k in keys if k in keep] or keys
    return statistics.median([vals[k] for k in keys]), len(keys)


def largest_counter(d, counter):
    """The largest per-dispatch value of `counter` over all kernels (the copy of the calibration run)."""
    rows = _rows(d, "counter_collection.csv")
    per = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), _name(r))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} values under {d}")
    k = max(per, key=per.get)
    return per[k], k[1]


def traffic(fetch_dir, write_dir, cfetch_dir, cwrite_dir, copy_bytes, kernel_src, workload="dense2b"):
    names = set()
    f_kib, nf = decode_counter(fetch_dir, "FETCH_SIZE", names=names)
    w_kib, nw = decode_counter(write_dir, "WRITE_SIZE")
    cf_kib, cname = largest_counter(cfetch_dir, "FETCH_SIZE")
    cw_kib, _ = largest_counter(cwrite_dir, "WRITE_SIZE")
    kf = copy_bytes / (cf_kib * 1024.0)
    kw = copy_bytes / (cw_kib * 1024.0)
    hbm = f_kib * 1024.0 * kf + w_kib * 1024.0 * kw
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()[:16]
    return "\n".join([
        f"kernel = {', '.join(sorted(names))}",
        f"workload = {workload}",
        f"kernel_sha = {sha}",
        f"decode_dispatches_fetch = {nf}",
        f"decode_dispatches_write = {nw}",
        f"fetch_kib_per_launch = {f_kib:.1f}",
        f"write_kib_per_launch = {w_kib:.1f}",
        f"copy_kernel = {cname[:80]}",
        f"copy_bytes = {copy_bytes}",
        f"copy_fetch_kib = {cf_kib:.1f}",
        f"copy_write_kib = {cw_kib:.1f}",
        f"fetch_scale = {kf:.4f}",
        f"write_scale = {kw:.4f}",
        f"hbm_bytes_per_launch = {hbm:.0f}",
    ])


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace_summary(argv[1]))
    elif len(argv) >= 2 and argv[0] == "dispatches":
        print(dispatch_list(argv[1]))
    elif len(argv) >= 2 and argv[0] == "counters":
        per, dur = counter_values(argv[1], argv[2] if len(argv) > 2 else DECODE_KERNEL)
        for c, v in per.items():
            vals = list(v.values())
            s = _stats(vals)
            print(f"{c}: dispatches {s['n']}, median {s['median']:.1f}, min {s['min']:.1f}, max {s['max']:.1f}")
    elif len(argv) in (7, 8) and argv[0] == "traffic":
        print(traffic(argv[1], argv[2], argv[3], argv[4], int(argv[5]), argv[6], *argv[7:]))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
