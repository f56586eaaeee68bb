"""Turn rocprofv3 output into the short text summaries kept under profiles/.

    # a plain copy of known size, to scale the HBM byte counters
    python -m lsh_eviction_amd.profiling copy --mib 1024 --reps 4

    # kernel-trace statistics -> markdown
    python -m lsh_eviction_amd.profiling stats --csv <run_kernel_stats.csv> --cmd "<command>" --out <file.md>

    # FETCH_SIZE / WRITE_SIZE counter runs (decode and copy) -> bytes per launch
    python -m lsh_eviction_amd.profiling traffic --fetch <csv> --write <csv> --copy-fetch <csv> \
        --copy-write <csv> --copy-mib 1024 --kernel k_decode_fused --key long_128k/fused --out <json>

The counters are read from rocprofv3's `--output-format csv` files
(`*_counter_collection.csv`: one row per dispatch and counter).  FETCH_SIZE and
WRITE_SIZE count KiB moved between the L2 and memory; a copy of N bytes reads N
and writes N, so the copy's readings give the factor by which each counter
maps to bytes on this part.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _code_only(text: str) -> str:
    """C++ source without comments and with runs of whitespace collapsed, so that
    an edit of a comment does not count as a change of the kernel."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif text[i] in "\"'":
            q, j = text[i], i + 1
            while j < n and text[j] != q:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the code (comments and whitespace aside) of the decode kernels;
    counter readings taken on other code are stale."""
    h = hashlib.sha256()
    for f in ("k_decode.hip", "hkv_device.h"):
        with open(os.path.join(ROOT, "lsh_eviction_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    base = name.split("(")[0]
    if "<" in base:
        head, _, args = base.partition("<")
        base = head.split("::")[-1].split(" ")[-1] + "<" + args
    else:
        base = base.split("::")[-1].split(" ")[-1]
    return base if len(base) <= 72 else base[:69] + "..."


def per_dispatch(path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter of a counter-collection csv."""
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            if row.get("Counter_Name") != counter:
                continue
            acc[row["Kernel_Name"]][row.get("Dispatch_Id") or row.get("Correlation_Id")] += float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in acc.items()}


def _pick(per: dict, needle: str):
    hits = [(k, v) for k, v in per.items() if needle in k]
    if not hits:
        raise SystemExit(f"no dispatch of a kernel matching {needle!r}; kernels: {sorted(per)[:8]}")
    k, v = max(hits, key=lambda kv: len(kv[1]))
    return k, v


def _mean(v):
    return sum(v) / len(v)


def cmd_copy(args):
    import torch
    n = args.mib << 20
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {args.mib} MiB {args.reps} times", flush=True)


def cmd_stats(args):
    rows = list(csv.DictReader(open(args.csv, newline="")))
    lines = ["# rocprofv3 kernel statistics", "", f"Command: `{args.cmd}`", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = _short(r["Name"])
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    if args.note:
        lines += ["", args.note]
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as fh:
        fh.write(text)
    print(text)


def cmd_traffic(args):
    copy_bytes = args.copy_mib << 20
    cf = per_dispatch(args.copy_fetch, "FETCH_SIZE")
    cw = per_dispatch(args.copy_write, "WRITE_SIZE")
    ckf, cvf = _pick(cf, "copy")
    ckw, cvw = _pick(cw, "copy")
    f_fetch = _mean(cvf) * 1024.0 / copy_bytes     # counter bytes per byte read
    f_write = _mean(cvw) * 1024.0 / copy_bytes
    kf, vf = _pick(per_dispatch(args.fetch, "FETCH_SIZE"), args.kernel)
    kw, vw = _pick(per_dispatch(args.write, "WRITE_SIZE"), args.kernel)
    read_b = _mean(vf) * 1024.0 / f_fetch
    write_b = _mean(vw) * 1024.0 / f_write
    rec = {
        "kernel": _short(kf), "kernel_hash": kernel_source_hash(),
        "bytes_per_launch": round(read_b + write_b),
        "read_bytes": round(read_b), "write_bytes": round(write_b),
        "fetch_kib_raw": round(_mean(vf), 1), "write_kib_raw": round(_mean(vw), 1),
        "dispatches": [len(vf), len(vw)],
        "copy_kernel": _short(ckf), "copy_bytes": copy_bytes,
        "copy_fetch_factor": round(f_fetch, 4), "copy_write_factor": round(f_write, 4),
    }
    data = {}
    if os.path.exists(args.out):
        data = json.load(open(args.out))
    data[args.key] = rec
    with open(args.out, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(rec, indent=1))
    if args.md:
        write_traffic_md(args, rec)


def write_traffic_md(args, rec):
    """Markdown summary of one traffic record, with the commands that made it."""
    d = os.path.dirname
    runs = [("FETCH_SIZE", d(args.fetch), "bench"), ("WRITE_SIZE", d(args.write), "bench"),
            ("FETCH_SIZE", d(args.copy_fetch), "copy"), ("WRITE_SIZE", d(args.copy_write), "copy")]
    lines = [f"# HBM traffic of {args.kernel}, {args.key} (counter runs)", "", "Commands (each a run of its own):", ""]
    for ctr, outdir, what in runs:
        prog = (f"python -u bench.py {args.bench_args}" if what == "bench" else
                f"python -u -m lsh_eviction_amd.profiling copy --mib {args.copy_mib} --reps 4")
        lines.append(f"    rocprofv3 --pmc {ctr} --output-format csv -d {outdir} -o run -- {prog}")
    lines.append(f"    python -m lsh_eviction_amd.profiling traffic --fetch {args.fetch} --write {args.write} \\")
    lines.append(f"        --copy-fetch {args.copy_fetch} --copy-write {args.copy_write} --copy-mib {args.copy_mib} \\")
    lines.append(f"        --kernel {args.kernel} --key {args.key} --out {args.out} --md {args.md}"
                 + (f" --alg-bytes {args.alg_bytes}" if args.alg_bytes else ""))
    lines += ["", f"Calibration: a {args.copy_mib} MiB device copy (`{rec['copy_kernel']}`) reads and writes "
              f"{args.copy_mib} MiB per dispatch; its FETCH_SIZE reading gives {rec['copy_fetch_factor']} counter "
              f"bytes per byte read and its WRITE_SIZE reading {rec['copy_write_factor']} per byte written.", "",
              f"| per launch ({rec['dispatches'][0]} dispatches) | raw counter (KiB) | scaled bytes |", "|---|---:|---:|",
              f"| read (FETCH_SIZE) | {rec['fetch_kib_raw']} | {rec['read_bytes']:,} |",
              f"| write (WRITE_SIZE) | {rec['write_kib_raw']} | {rec['write_bytes']:,} |",
              f"| **total** | | **{rec['bytes_per_launch']:,}** |"]
    if args.alg_bytes:
        lines += ["", f"Algorithmic bytes per launch: {args.alg_bytes:,}; measured traffic is "
                  f"{rec['bytes_per_launch'] / args.alg_bytes:.3f}x that."]
    lines += ["", f"Kernel source hash when measured (of the code with comments and whitespace set aside): "
              f"`{rec['kernel_hash']}` (bench.py reports this traffic only while the code still has that hash)."]
    with open(args.md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def all_counters(path: str):
    """{counter: {kernel name: [value per dispatch]}} of a counter-collection csv."""
    acc = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            disp = row.get("Dispatch_Id") or row.get("Correlation_Id")
            acc[row["Counter_Name"]][row["Kernel_Name"]][disp] += float(row["Counter_Value"])
    return {c: {k: list(v.values()) for k, v in per.items()} for c, per in acc.items()}


def cmd_counters(args):
    """Mean per dispatch of every counter in the given csv files, for each
    kernel matching one of the needles; one markdown table."""
    needles = args.kernels.split(",")
    table = collections.OrderedDict()   # counter -> {needle: (mean, dispatches)}
    names = {}
    for path in args.csv:
        for ctr, per in all_counters(path).items():
            for nd in needles:
                hits = [(k, v) for k, v in per.items() if nd in k]
                if not hits:
                    continue
                k, v = max(hits, key=lambda kv: len(kv[1]))
                names[nd] = _short(k)
                table.setdefault(ctr, {})[nd] = (_mean(v), len(v))
    lines = [f"# {args.title}", "", "Commands (each a run of its own, the counters of one pass after --pmc):", ""]
    lines += [f"    {c}" for c in args.cmd]
    lines += ["", "Mean per dispatch (rocprofv3 sums a counter over its hardware instances unless its name says "
              "otherwise; derived counters are rocprofv3's own expressions).", ""]
    lines.append("| counter | " + " | ".join(f"`{names.get(nd, nd)}`" for nd in needles) + " |")
    lines.append("|---|" + "---:|" * len(needles))
    for ctr, per in table.items():
        cells = []
        for nd in needles:
            if nd in per:
                m, n = per[nd]
                cells.append(f"{m:,.4g} ({n})" if abs(m) < 1e4 else f"{m:,.0f} ({n})")
            else:
                cells.append("")
        lines.append(f"| {ctr} | " + " | ".join(cells) + " |")
    lines += ["", "(n) = dispatches averaged."]
    if args.note:
        lines += ["", args.note]
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text)
    print(text)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    a = sub.add_parser("copy")
    a.add_argument("--mib", type=int, default=1024)
    a.add_argument("--reps", type=int, default=4)
    a = sub.add_parser("stats")
    a.add_argument("--csv", required=True)
    a.add_argument("--cmd", required=True)
    a.add_argument("--out", required=True)
    a.add_argument("--note", default="")
    a = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write", "kernel", "key", "out"):
        a.add_argument("--" + k.replace("_", "-"), required=True, dest=k)
    a.add_argument("--copy-mib", type=int, default=1024)
    a.add_argument("--md", default="")
    a.add_argument("--alg-bytes", type=int, default=0)
    a.add_argument("--bench-args", default="--steps 20 --warmup 2 --no-cpu")
    a = sub.add_parser("counters")
    a.add_argument("--csv", nargs="+", required=True)
    a.add_argument("--kernels", required=True, help="comma-separated substrings of kernel names")
    a.add_argument("--cmd", nargs="+", default=[])
    a.add_argument("--title", default="rocprofv3 counters")
    a.add_argument("--out", default="")
    a.add_argument("--note", default="")
    args = ap.parse_args(argv)
    {"copy": cmd_copy, "stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[args.mode](args)


if __name__ == "__main__":
    main(sys.argv[1:])
