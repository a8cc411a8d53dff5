"""Summaries of rocprofv3 output (CSV format) for the measurement record.

Two summaries are produced from ``rocprofv3 --output-format csv`` runs:

* kernel time: ``stats`` reads ``*_kernel_stats.csv`` (``--kernel-trace
  --stats``) and writes a markdown table of calls / average / min / max
  duration per kernel;
* HBM traffic: ``traffic`` reads the ``*_counter_collection.csv`` of one
  ``--pmc FETCH_SIZE`` run and one ``--pmc WRITE_SIZE`` run of the benchmark,
  plus the same two counters for a plain copy kernel of known size, and
  writes per-launch HBM bytes for each kernel, scaled by the copy's
  known/measured ratio. The result carries a digest of the kernel sources so
  that the benchmark can tell whether the counters still describe the
  current kernels.

    python -m permute_ep_layout_amd.profiling stats --dir D --cmd "..." --out F.md
    python -m permute_ep_layout_amd.profiling traffic --fetch D1 --write D2 \\
        --copy-fetch D3 --copy-write D4 --copy-bytes B --workload dsv3 --out F.md
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ("permute_ep_layout_amd/csrc/epl_kernels.h", "permute_ep_layout_amd/csrc/epl.hip")
TRAFFIC_MARK = "traffic-json:"

# short names of the library's kernels, matched against demangled names
SHORT = (("ep_dispatch_decode_kernel", "dispatch_decode"),
         ("ep_layout_scan_kernel", "layout_scan"), ("ep_layout_kernel", "layout"),
         ("ep_scan_kernel", "scan"),
         ("ep_ll_scatter_kernel", "ll_scatter"), ("ep_ll_decode_kernel", "ll_decode"),
         ("ep_scatter_kernel", "scatter"), ("ep_combine_kernel", "combine"),
         ("ep_expert_scale_kernel", "expert"),
         # the benchmark's write-piece probes (bench_probe/stream_probe.hip)
         ("pieces_kernel<true, true>", "pieces_nt_xcd"),
         ("pieces_kernel<true, false>", "pieces_nt_inorder"),
         ("pieces_kernel<false, true>", "pieces_wb_xcd"),
         ("pieces_kernel<false, false>", "pieces_wb_inorder"))


def _code_only(text: str) -> str:
    """C/C++ source without comments and with whitespace runs collapsed, so
    that editing a comment does not make the counters look stale."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] == '"':                       # string literal, kept whole
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def source_digest(root: str = ROOT) -> str:
    """Digest of the kernel sources' code (comments and layout ignored)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def short_name(kernel_name: str) -> str:
    for key, short in SHORT:
        if key in kernel_name:
            return short
    return kernel_name.split("(")[0][:60]


def unique_short(counts: dict) -> dict:
    """{full name: short name} for {full name: launches}. Where instances of
    one template share a short name, the most-launched keeps it and the
    others get their template arguments appended (``scatter<7>``)."""
    out, taken = {}, set()
    for name in sorted(counts, key=lambda n: -counts[n]):
        short = short_name(name)
        if short in taken:
            head = name.split("(")[0]
            short += head[head.find("<"):] if "<" in head else f"#{len(taken)}"
        taken.add(short)
        out[name] = short
    return out


def _one(pattern: str, d: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return hits[0]


def kernel_stats(d: str):
    rows = list(csv.DictReader(open(_one("*kernel_stats.csv", d))))
    names = unique_short({r["Name"]: int(r["Calls"]) for r in rows})
    out = []
    for r in rows:
        out.append(dict(name=r["Name"], short=names[r["Name"]], calls=int(r["Calls"]),
                        avg_us=float(r["AverageNs"]) / 1e3, min_us=float(r["MinNs"]) / 1e3,
                        max_us=float(r["MaxNs"]) / 1e3))
    return out


def counter_per_dispatch(d: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter of a --pmc run."""
    path = _one("*counter_collection.csv", d)
    per = {}
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id")))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def write_stats(d: str, cmd: str, out: str, title: str):
    st = kernel_stats(d)
    lines = [f"# {title}", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | avg (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in st:
        lines.append(f"| `{r['short']}` | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} |")
    lines += ["", "Full kernel names:", ""] + [f"- `{r['short']}`: `{r['name']}`" for r in st]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def write_traffic(fetch: str, write: str, copy_fetch: str, copy_write: str, copy_bytes: int,
                  workload: str, out: str, cmds: dict):
    f_k = counter_per_dispatch(fetch, "FETCH_SIZE")
    w_k = counter_per_dispatch(write, "WRITE_SIZE")
    cf = counter_per_dispatch(copy_fetch, "FETCH_SIZE")
    cw = counter_per_dispatch(copy_write, "WRITE_SIZE")

    def biggest(d):   # the copy kernel: the one with the largest per-dispatch reading
        name = max(d, key=lambda n: statistics.median(d[n]))
        return name, statistics.median(d[name])

    cname, cfetch_kib = biggest(cf)
    _, cwrite_kib = biggest(cw)
    rf = copy_bytes / (cfetch_kib * 1024.0)
    rw = copy_bytes / (cwrite_kib * 1024.0)
    result = {"workload": workload, "source_digest": source_digest(),
              "copy_kernel": cname, "copy_bytes": copy_bytes,
              "copy_fetch_factor": rf, "copy_write_factor": rw, "kernels": {}}
    lines = [f"# HBM traffic per launch, {workload} workload", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 --pmc runs of the",
             "benchmark, each scaled by known/measured bytes of a plain copy kernel of "
             f"{copy_bytes} bytes (fetch factor {rf:.4f}, write factor {rw:.4f}).", "",
             "Commands:", ""]
    for k, c in cmds.items():
        lines += [f"- {k}: `{c}`"]
    lines += ["", "| kernel | dispatches | FETCH (MB) | WRITE (MB) | HBM bytes (MB, scaled) |",
              "|---|---|---|---|---|"]
    names = unique_short({n: len(f_k.get(n, w_k.get(n, []))) for n in set(f_k) | set(w_k)})
    for name in sorted(names, key=lambda n: names[n]):
        short = names[name]
        if short_name(name) not in dict(SHORT).values():
            continue
        fk = statistics.median(f_k.get(name, [0.0]))
        wk = statistics.median(w_k.get(name, [0.0]))
        nbytes = fk * 1024.0 * rf + wk * 1024.0 * rw
        result["kernels"][short] = {"fetch_kib": fk, "write_kib": wk,
                                    "bytes_per_launch": nbytes,
                                    "dispatches": len(f_k.get(name, []))}
        lines.append(f"| `{short}` | {len(f_k.get(name, []))} | {fk * 1024 / 1e6:.1f} | "
                     f"{wk * 1024 / 1e6:.1f} | {nbytes / 1e6:.1f} |")
    lines += ["", f"<!-- {TRAFFIC_MARK} {json.dumps(result)} -->"]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return result


def write_counters(d: str, cmd: str, out: str, title: str, all_kernels: bool = False):
    """Median per dispatch of every counter of one --pmc run, per kernel (the
    library's kernels, or every kernel of the run with `all_kernels`)."""
    path = _one("*counter_collection.csv", d)
    per = {}
    for r in csv.DictReader(open(path)):
        key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id")), r["Counter_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    launches = {}
    for (name, disp, _) in per:
        launches.setdefault(name, set()).add(disp)
    names = unique_short({n: len(d) for n, d in launches.items()})
    table = {}
    for (name, _, counter), v in per.items():
        table.setdefault(names[name], {}).setdefault(counter, []).append(v)
    counters = sorted({c for k in table.values() for c in k})
    lines = [f"# {title}", "", "Command:", "", "```", cmd, "```", "",
             "Median per dispatch (summed over the device's counter instances).", "",
             "| kernel | " + " | ".join(counters) + " |",
             "|---|" + "---|" * len(counters)]
    for k in sorted(table):
        if not all_kernels and k.split("<")[0] not in dict(SHORT).values():
            continue
        vals = [statistics.median(table[k][c]) if c in table[k] else float("nan") for c in counters]
        lines.append(f"| `{k}` | " + " | ".join(f"{v:.0f}" for v in vals) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_traffic(path: str):
    try:
        text = open(path).read()
    except OSError:
        return None
    i = text.find(TRAFFIC_MARK)
    if i < 0:
        return None
    j = text.find("-->", i)
    return json.loads(text[i + len(TRAFFIC_MARK):j].strip())


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("--dir", required=True)
    a.add_argument("--cmd", required=True)
    a.add_argument("--title", default="Kernel time (rocprofv3 --kernel-trace --stats)")
    a.add_argument("--out", required=True)
    b = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy-fetch", "copy-write"):
        b.add_argument(f"--{k}", required=True)
        b.add_argument(f"--{k}-cmd", default="")
    c = sub.add_parser("counters")
    c.add_argument("--dir", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--title", default="Counters (rocprofv3 --pmc)")
    c.add_argument("--out", required=True)
    c.add_argument("--all-kernels", action="store_true")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--out", required=True)
    args = ap.parse_args()
    if args.what == "stats":
        write_stats(args.dir, args.cmd, args.out, args.title)
    elif args.what == "counters":
        write_counters(args.dir, args.cmd, args.out, args.title, args.all_kernels)
    else:
        cmds = {"fetch": args.fetch_cmd, "write": args.write_cmd,
                "copy fetch": args.copy_fetch_cmd, "copy write": args.copy_write_cmd}
        print(json.dumps(write_traffic(args.fetch, args.write, args.copy_fetch, args.copy_write,
                                       args.copy_bytes, args.workload, args.out, cmds)))


if __name__ == "__main__":
    main()
