"""Turn rocprofv3 output into the short summaries kept under profiles/.

    python -m normalization_ln_forward_amd.profiling stats <kernel_stats.csv> --command "<cmd>"
        Markdown table of per-kernel call count and average / min / max
        duration from `rocprofv3 --kernel-trace --stats --output-format csv`.

    python -m normalization_ln_forward_amd.profiling traffic <fetch_counter_collection.csv>
        <write_counter_collection.csv> --copy-mib N --kernels k1,k2 --command "<cmd>" [--json out]
        HBM bytes per launch of the named kernels from two `rocprofv3 --pmc`
        passes (FETCH_SIZE, then WRITE_SIZE).  Each counter is scaled by what
        it reads for the plain device copy of N MiB the same command ran
        (torch's copy kernel: N MiB read, N MiB written), so the result is in
        bytes whatever unit the counter uses.  With --json, the entries are
        written to that file together with the hash of the kernels' code (comments removed), so
        bench.py reports them only while the kernels are unchanged.

    python -m normalization_ln_forward_amd.profiling counters <counter_collection.csv>...
        --kernels k1,k2 --command "<cmd>"
        Markdown table of the per-dispatch mean of every counter of the named
        kernels, from one or more `rocprofv3 --pmc` passes.
"""
import argparse
import csv
import hashlib
import json
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# Source files whose text determines each kernel's code.
KERNEL_SOURCES = {
    "ln_partial_kernel": ["ln.hip", "common.hpp"],
    "ln_merge_kernel": ["ln.hip", "common.hpp"],
    "ln_normalize_rows_kernel": ["ln.hip", "common.hpp"],
    "ln_normalize_kernel": ["ln.hip", "common.hpp"],
    "ln_single_ctl_kernel": ["ln.hip", "common.hpp"],
    "gn_fast_kernel": ["gn.hip", "common.hpp"],
    "rms_ch_hold_kernel": ["rms.hip", "common.hpp"],
    "fc_mfma_kernel": ["fc.hip", "common.hpp"],
    "fc_dma_kernel": ["fc.hip", "common.hpp"],
    "copy_dense_kernel": ["ref.hip", "common.hpp"],
    "rms_copy_pattern_kernel": ["rms.hip", "common.hpp"],
}


_COMMENTS = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def code_text(text):
    """The text the compiler acts on: comments and blank lines removed, trailing blanks trimmed (so a
    change to comments alone keeps a measurement valid)."""
    text = _COMMENTS.sub("", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_sha(files, read=None):
    """Hash of the code (see code_text) of the named csrc files and of the extra compiler flags each is
    built with; `read(name) -> str` overrides reading them from the package's csrc/."""
    from . import build
    h = hashlib.sha256()
    for f in files:
        if read is None:
            with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
                text = fh.read()
        else:
            text = read(f)
        h.update(code_text(text).encode("utf-8"))
        h.update(" ".join(build.EXTRA_FLAGS.get(f, [])).encode("utf-8"))
    return h.hexdigest()[:16]


def short_name(name):
    m = re.search(r"normfwd::(\w+)(<[^(]*>)?", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    m = re.search(r"(\w+)\(", name)
    return (m.group(1) if m else name)[:60]


def stats_markdown(path, command):
    rows = list(csv.DictReader(open(path)))
    out = [f"Command: `{command}`", "",
           "| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    return "\n".join(out) + "\n"


def _counter_rows(path, counter):
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def _copy_value(per, copy_mib):
    """Median counter value over the copy-reference dispatches (torch copy kernels of copy_mib)."""
    vals = []
    for name, vs in per.items():
        if "copy" in name.lower() and "normfwd" not in name:
            vals.extend(vs)
    if not vals:
        raise SystemExit("no copy-reference dispatch found")
    # the reference copies are the largest copy dispatches in the run
    vals.sort()
    top = vals[-3:]
    return statistics.median(top)


def traffic(fetch_csv, write_csv, copy_mib, kernels):
    fetch = _counter_rows(fetch_csv, "FETCH_SIZE")
    write = _counter_rows(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib * (1 << 20)
    f_scale = copy_bytes / _copy_value(fetch, copy_mib)
    w_scale = copy_bytes / _copy_value(write, copy_mib)
    out = {}
    for k in kernels:
        fv = [v for n, vs in fetch.items() if short_name(n).split("<")[0] == k for v in vs]
        wv = [v for n, vs in write.items() if short_name(n).split("<")[0] == k for v in vs]
        if not fv or not wv:
            continue
        fb = statistics.mean(fv) * f_scale
        wb = statistics.mean(wv) * w_scale
        out[k] = {"fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                  "hbm_bytes_per_launch": round(fb + wb), "dispatches": len(fv),
                  "fetch_scale": f_scale, "write_scale": w_scale,
                  "source_sha": source_sha(KERNEL_SOURCES.get(k, ["ln.hip"]))}
    return out


def counters_markdown(paths, kernels, command):
    """Per-dispatch means of every counter in one or more `rocprofv3 --pmc` CSVs, one row per kernel (a
    kernel's dispatches averaged), one column per counter."""
    vals = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            k = short_name(r["Kernel_Name"]).split("<")[0]
            if k not in kernels:
                continue
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    names = sorted({c for v in vals.values() for c in v})
    out = [f"Command: `{command}`", "", "| kernel | " + " | ".join(names) + " |",
           "|---|" + "---:|" * len(names)]
    for k in kernels:
        if k not in vals:
            continue
        cells = [f"{statistics.mean(vals[k][c]):.4g}" if c in vals[k] else "" for c in names]
        out.append(f"| {k} | " + " | ".join(cells) + " |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--command", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--copy-mib", type=int, required=True)
    b.add_argument("--kernels", required=True)
    b.add_argument("--command", required=True)
    b.add_argument("--json")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernels", required=True)
    c.add_argument("--command", required=True)
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        sys.stdout.write(stats_markdown(args.csv, args.command))
        return
    if args.cmd == "counters":
        sys.stdout.write(counters_markdown(args.csv, args.kernels.split(","), args.command))
        return
    res = traffic(args.fetch_csv, args.write_csv, args.copy_mib, args.kernels.split(","))
    for k, v in res.items():
        v["command"] = args.command
    if args.json:
        old = {}
        if os.path.exists(args.json):
            with open(args.json) as f:
                old = json.load(f)
        old.update(res)
        with open(args.json, "w") as f:
            json.dump(old, f, indent=1, sort_keys=True)
            f.write("\n")
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
