"""Summaries of rocprofv3 output for the POET-X layer kernels.

  python -m orthogonal_equivalence_amd.rocprof_summary trace <kernel_stats.csv> \
      --title "..." --command "..." > profile.txt
      per-kernel call counts and durations from a --kernel-trace --stats run.

  python -m orthogonal_equivalence_amd.rocprof_summary traffic \
      --kernel SUBSTR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
      --algorithmic-bytes B --workload "..." --sources FILE... > traffic.json
      HBM bytes per launch of the kernel whose name contains SUBSTR, from one
      FETCH_SIZE and one WRITE_SIZE counter pass (KiB per dispatch, summed over
      the counter instances of a dispatch), each scaled by what the same counter
      reads for a plain device copy of 1 GiB (read 1 GiB, write 1 GiB).

  python -m orthogonal_equivalence_amd.rocprof_summary dispatches \
      --mfma DIR --fetch DIR --write DIR --per-step N --stages NAME... \
      --calibration profiles/dense_fwd_traffic.json --title "..." --command "..." > profile.txt
      the last N dispatches (one step) in launch order: duration, MFMA
      utilisation (the derived MfmaUtil counter: MFMA-busy SIMD cycles over
      active cycles x SIMDs), and HBM bytes read and written (FETCH_SIZE and
      WRITE_SIZE, scaled by the copy calibration) with the rate they imply.

Reads CSV files only; nothing here touches the GPU.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict


def _csv_rows(path_or_dir, name):
    path = path_or_dir
    if os.path.isdir(path_or_dir):
        hits = sorted(glob.glob(os.path.join(path_or_dir, "**", name), recursive=True))
        if not hits:
            raise SystemExit(f"no {name} under {path_or_dir}")
        path = hits[0]
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def short_name(name, width=110):
    name = name.replace("void poetx::(anonymous namespace)::", "").replace("poetx::(anonymous namespace)::", "")
    name = name.replace("unsigned short", "bf16")
    return name if len(name) <= width else name[: width - 3] + "..."


def trace(args):
    rows = _csv_rows(args.stats, "*kernel_stats.csv")
    out = [f"# rocprofv3 kernel-trace summary: {args.title}", "#",
           "# command (from the repository root, TMPDIR=/tmp):", f"#   {args.command}",
           "# durations in microseconds", "",
           f"{'total_us':>11} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}  kernel"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"{float(r['TotalDurationNs']) / 1e3:11.1f} {int(r['Calls']):6d} "
                   f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                   f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}  {short_name(r['Name'])}")
    print("\n".join(out))


def _per_dispatch_kib(d, counter, substr):
    """Mean over the dispatches of kernels matching substr of the summed counter."""
    rows = _csv_rows(d, "*counter_collection.csv")
    per = defaultdict(float)
    names = {}
    for r in rows:
        if r["Counter_Name"] != counter or substr not in r["Kernel_Name"]:
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = r["Kernel_Name"]
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching {substr!r} in {d}")
    vals = list(per.values())
    return sum(vals) / len(vals), len(vals), sorted(set(names.values()))


def sources_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic(args):
    fetch, nf, kn = _per_dispatch_kib(args.fetch, "FETCH_SIZE", args.kernel)
    write, nw, _ = _per_dispatch_kib(args.write, "WRITE_SIZE", args.kernel)
    cf, _, _ = _per_dispatch_kib(args.copy_fetch, "FETCH_SIZE", args.copy_kernel)
    cw, _, _ = _per_dispatch_kib(args.copy_write, "WRITE_SIZE", args.copy_kernel)
    nbytes = 1 << 30
    f_factor = nbytes / 1024.0 / cf
    w_factor = nbytes / 1024.0 / cw
    rd = fetch * 1024.0 * f_factor
    wr = write * 1024.0 * w_factor
    res = {
        "kernel": kn,
        "workload": args.workload,
        "sources_sha256": sources_digest(args.sources),
        "sources": [os.path.relpath(s, args.root) for s in args.sources],
        "dispatches": {"fetch": nf, "write": nw},
        "fetch_size_kib_per_launch": fetch,
        "write_size_kib_per_launch": write,
        "copy_calibration": {"bytes_read": nbytes, "bytes_written": nbytes, "fetch_size_kib": cf,
                             "write_size_kib": cw, "fetch_factor": f_factor, "write_factor": w_factor},
        "bytes_read_per_launch": rd,
        "bytes_written_per_launch": wr,
        "bytes_per_launch": rd + wr,
        "algorithmic_bytes_per_launch": args.algorithmic_bytes,
        "commands": args.command,
    }
    print(json.dumps(res, indent=1))


def _dispatch_rows(d, counter):
    """{Dispatch_Id: (kernel, value summed over rows, start ns, end ns)}."""
    rows = _csv_rows(d, "*counter_collection.csv")
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        k = int(r["Dispatch_Id"])
        v = float(r["Counter_Value"])
        if k in out:
            name, acc, t0, t1 = out[k]
            out[k] = (name, acc + v, t0, t1)
        else:
            out[k] = (r["Kernel_Name"], v, int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
    return out


def dispatches(args):
    mf = _dispatch_rows(args.mfma, "MfmaUtil")
    fe = _dispatch_rows(args.fetch, "FETCH_SIZE")
    wr = _dispatch_rows(args.write, "WRITE_SIZE")
    cal = json.load(open(args.calibration))["copy_calibration"]
    ff, wf = cal["fetch_factor"], cal["write_factor"]
    def last(d):
        return [d[k] for k in sorted(d)][-args.per_step:]
    m, f, w = last(mf), last(fe), last(wr)
    stages = args.stages or [""] * len(m)
    if not (len(m) == len(f) == len(w) == len(stages) == args.per_step):
        raise SystemExit("dispatch counts differ between the passes")
    out = [f"# rocprofv3 counter summary: {args.title}", "#",
           "# commands (from the repository root, TMPDIR=/tmp):"]
    out += [f"#   {c}" for c in args.command]
    out += ["# one step, launch order; duration from the MfmaUtil pass's timestamps; bytes = counter",
            f"# KiB x 1024 x the copy calibration (FETCH x{ff:.3f}, WRITE x{wf:.3f}); rate against 8 TB/s",
            "",
            f"{'stage':12s} {'us':>8s} {'MFMA %':>7s} {'read MB':>9s} {'write MB':>9s} {'TB/s':>6s} {'of 8':>5s}  kernel"]
    tot_us = 0.0
    for st, (name, util, t0, t1), (nf, kf, _, _), (nw, kw, _, _) in zip(stages, m, f, w):
        if not (name == nf == nw):
            raise SystemExit(f"kernel order differs between the passes: {name} / {nf} / {nw}")
        us = (t1 - t0) / 1e3
        tot_us += us
        rd, wb = kf * 1024 * ff, kw * 1024 * wf
        rate = (rd + wb) / (us * 1e-6) / 1e12 if us > 0 else 0.0
        out.append(f"{st:12s} {us:8.1f} {util:7.1f} {rd / 1e6:9.1f} {wb / 1e6:9.1f} {rate:6.2f} "
                   f"{rate / 8.0:5.2f}  {short_name(name, 80)}")
    out.append(f"{'total':12s} {tot_us:8.1f}")
    print("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats")
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    r = sub.add_parser("traffic")
    r.add_argument("--kernel", required=True)
    r.add_argument("--copy-kernel", default="copyBuffer")
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--copy-fetch", required=True)
    r.add_argument("--copy-write", required=True)
    r.add_argument("--algorithmic-bytes", type=float, required=True)
    r.add_argument("--workload", required=True)
    r.add_argument("--sources", nargs="+", required=True)
    r.add_argument("--root", default=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    r.add_argument("--command", action="append", default=[])
    g = sub.add_parser("dispatches")
    g.add_argument("--mfma", required=True)
    g.add_argument("--fetch", required=True)
    g.add_argument("--write", required=True)
    g.add_argument("--per-step", type=int, required=True)
    g.add_argument("--stages", nargs="*", default=None)
    g.add_argument("--calibration", required=True)
    g.add_argument("--title", required=True)
    g.add_argument("--command", action="append", default=[])
    a = ap.parse_args(argv)
    {"trace": trace, "traffic": traffic, "dispatches": dispatches}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())
