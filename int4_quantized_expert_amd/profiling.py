"""HBM traffic of the library's kernels from rocprofv3 counter passes.

Two `rocprofv3 --pmc` passes over the same benchmark command, one reading
FETCH_SIZE and one reading WRITE_SIZE (KiB per dispatch), are turned into
bytes per launch.  Each counter is scaled by what it reads for a plain device
copy of known size run in the same process (bench.py --copy-probe): on gfx950
FETCH_SIZE reads about half of the bytes a copy moves, WRITE_SIZE all of them.

The summary is a small markdown file with one JSON block.  It carries a digest
of the kernel sources, so a reader can tell whether the counters still describe
the code as it stands (bench.py reports `traffic` only when they do).

    python -m int4_quantized_expert_amd.profiling traffic --fetch F.csv --write W.csv \\
        --copy-bytes 268435456 --workload 80b_stack_decode --tokens 1 --out profiles/X.md \\
        --command "the rocprofv3 command lines"
    python -m int4_quantized_expert_amd.profiling kernels --stats S.csv --title "..." \\
        --out profiles/Y.md --command "the rocprofv3 command line"
    python -m int4_quantized_expert_amd.profiling counters --pmc A.csv B.csv --title "..." \\
        --out profiles/Z.md --command "the rocprofv3 command lines"

The `counters` form summarises SQ counter passes (any counters, any number of
passes) per library kernel: the mean per dispatch of each counter, the kernel's
register, LDS and scratch use as the profiler recorded them, and the shares of
wave time that the SQ_WAIT_* and SQ_ACTIVE_INST_* counters give (all of them
count in the same 4-cycle units, so their ratios to SQ_WAVE_CYCLES are shares).
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def source_digest() -> str:
    """sha256 over the kernel sources, the public headers and the build flags."""
    h = hashlib.sha256()
    inc = os.path.join(ROOT, "include")
    files = [os.path.join(PKG, "build.py")] + [os.path.join(inc, f) for f in sorted(os.listdir(inc)) if f.endswith(".h")]
    csrc = os.path.join(PKG, "csrc")
    files += [os.path.join(csrc, f) for f in sorted(os.listdir(csrc)) if f.endswith((".hip", ".h"))]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _unmangle(name: str) -> str | None:
    """`_ZN3moe12_GLOBAL__N_19k_combineILi1EDF16_EEv...` -> `k_combine<1, _Float16>`.

    rocprofv3 leaves some template kernels mangled; only the forms the library
    uses are read (integer, bool, float and _Float16 template arguments).
    """
    m = re.match(r"_ZN3moe(?:12_GLOBAL__N_1)?(\d+)", name)
    if not m:
        return None
    n = int(m.group(1))
    ident, rest = name[m.end():m.end() + n], name[m.end() + n:]
    if not rest.startswith("I"):
        return ident
    args, pos = [], 1
    while pos < len(rest) and rest[pos] != "E":
        t = re.match(r"L[ib](-?\d+)E|DF16_|f", rest[pos:])
        if not t:
            return ident
        args.append(t.group(1) if t.group(1) is not None else ("_Float16" if t.group(0) == "DF16_" else "float"))
        pos += t.end()
    return f"{ident}<{', '.join(args)}>"


def is_library_kernel(name: str) -> bool:
    return name.startswith(("void moe::", "moe::", "_ZN3moe"))


def short_name(kernel: str) -> str:
    """`void moe::(anonymous namespace)::k_decode_a<4, 1, 1>(moe::FusedArgs)` -> `k_decode_a<4, 1, 1>`."""
    un = _unmangle(kernel)
    if un is not None:
        return un
    name = re.sub(r"^void ", "", kernel.replace("(anonymous namespace)::", "")).strip()
    m = re.match(r"[\w:]*?(\w+(?:<[^()]*>)?)\s*(?:\(|$)", name)
    return m.group(1) if m else name


def read_counter(path: str) -> dict[str, list[float]]:
    per = defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def traffic_table(fetch_csv: str, write_csv: str, copy_bytes: int) -> dict:
    f, w = read_counter(fetch_csv), read_counter(write_csv)
    if COPY_KERNEL not in f or COPY_KERNEL not in w:
        raise ValueError(f"no {COPY_KERNEL} dispatch in the counter files (run with --copy-probe)")
    kib = copy_bytes / 1024.0
    f_scale, w_scale = max(f[COPY_KERNEL]) / kib, max(w[COPY_KERNEL]) / kib
    rows = {}
    for name in f:
        if not is_library_kernel(name) or name not in w:
            continue
        fk = sum(f[name]) / len(f[name])
        wk = sum(w[name]) / len(w[name])
        rows[short_name(name)] = {
            "dispatches": len(f[name]),
            "fetch_kib": round(fk, 2),
            "write_kib": round(wk, 2),
            "read_bytes": round(fk * 1024 / f_scale),
            "write_bytes": round(wk * 1024 / w_scale),
            "traffic_bytes": round(fk * 1024 / f_scale + wk * 1024 / w_scale),
        }
    return {"fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5), "kernels": rows}


def write_summary(out: str, table: dict, workload: str, tokens: int, command: str) -> None:
    blob = {"workload": workload, "tokens": tokens, "source_digest": source_digest(), **table}
    lines = [f"# HBM traffic per launch: {workload}, T={tokens}\n\n",
             "Commands (from the repository root; rocprofv3 run from /tmp with TMPDIR=/tmp):\n\n",
             "```\n" + command.strip() + "\n```\n\n",
             f"Scaling by a {COPY_KERNEL} of known size in the same process: FETCH_SIZE reads "
             f"{table['fetch_scale']} x the bytes copied, WRITE_SIZE {table['write_scale']} x.\n\n",
             "| Kernel | Dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | Read bytes | Written bytes |\n",
             "|---|---|---|---|---|---|\n"]
    for k, r in table["kernels"].items():
        lines.append(f"| {k} | {r['dispatches']} | {r['fetch_kib']} | {r['write_kib']} | {r['read_bytes']} | "
                     f"{r['write_bytes']} |\n")
    lines.append("\n```json\n" + json.dumps(blob, indent=1) + "\n```\n")
    with open(out, "w") as fh:
        fh.writelines(lines)


def load_traffic(profiles_dir: str, workload: str, tokens: int) -> dict | None:
    """The counter table for this workload if one matches the current sources, else None."""
    if not os.path.isdir(profiles_dir):
        return None
    digest = source_digest()
    for f in sorted(os.listdir(profiles_dir)):
        if not f.endswith(".md"):
            continue
        with open(os.path.join(profiles_dir, f)) as fh:
            text = fh.read()
        m = re.search(r"```json\n(.*?)\n```", text, re.S)
        if not m:
            continue
        try:
            blob = json.loads(m.group(1))
        except json.JSONDecodeError:
            continue
        if blob.get("workload") == workload and blob.get("tokens") == tokens and blob.get("source_digest") == digest:
            return blob
    return None


def traffic_of(blob: dict | None, kernel: str) -> int | None:
    """Bytes per launch of `kernel` (a short name, or its stem before any
    template arguments or description) in a counter table, if exactly one
    entry matches."""
    if blob is None:
        return None
    rows = blob["kernels"]
    if kernel in rows:
        return rows[kernel]["traffic_bytes"]
    stem = kernel.split(" ")[0].split("<")[0]
    hits = [r for name, r in rows.items() if name.split("<")[0] == stem]
    return hits[0]["traffic_bytes"] if len(hits) == 1 else None


def kernel_stats(stats_csv: str) -> list[dict]:
    """Rows of a rocprofv3 --stats kernel summary (durations in microseconds)."""
    rows = []
    with open(stats_csv) as fh:
        for r in csv.DictReader(fh):
            rows.append({"kernel": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3, "share": float(r["Percentage"])})
    return rows


def write_kernel_summary(out: str, rows: list[dict], title: str, command: str, notes: str) -> None:
    lines = [f"# {title}\n\n",
             "Command (from the repository root; rocprofv3 run from /tmp with TMPDIR=/tmp):\n\n",
             "```\n" + command.strip() + "\n```\n\n"]
    if notes:
        lines.append(notes.strip() + "\n\n")
    lines += ["| Kernel | Calls | Avg us | Min us | Max us | Share |\n", "|---|---|---|---|---|---|\n"]
    for r in rows:
        lines.append(f"| {r['kernel']} | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | {r['max_us']:.2f} | "
                     f"{r['share']:.1f}% |\n")
    with open(out, "w") as fh:
        fh.writelines(lines)


SHARES = (("SQ_WAIT_ANY", "waiting on anything"),
          ("SQ_WAIT_INST_ANY", "waiting on an issued instruction's result (s_waitcnt)"),
          ("SQ_ACTIVE_INST_VALU", "issuing VALU instructions"),
          ("SQ_ACTIVE_INST_VMEM", "issuing vector memory instructions"),
          ("SQ_ACTIVE_INST_LDS", "issuing LDS instructions"),
          ("SQ_ACTIVE_INST_SCA", "issuing scalar instructions"),
          ("SQ_WAIT_INST_LDS", "waiting on LDS results"))


def counter_table(paths: list[str]) -> dict:
    """Per library kernel: mean per dispatch of every counter in the passes,
    and the launch resources the profiler recorded with them."""
    vals: dict = defaultdict(lambda: defaultdict(list))
    res: dict = {}
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                if not is_library_kernel(name):
                    continue
                k = short_name(name)
                vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
                res[k] = {f: int(float(r[f])) for f in ("Grid_Size", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size",
                                                       "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count") if f in r}
    out = {}
    for k, per in vals.items():
        means = {c: sum(v) / len(v) for c, v in per.items()}
        row = {"dispatches": max(len(v) for v in per.values()), "resources": res[k],
               "counters": {c: round(m, 1) for c, m in sorted(means.items())}, "shares": {}}
        wc = means.get("SQ_WAVE_CYCLES")
        if wc:
            for c, _ in SHARES:
                if c in means:
                    row["shares"][c] = round(means[c] / wc, 4)
        out[k] = row
    return out


def write_counter_summary(out: str, table: dict, title: str, command: str, notes: str) -> None:
    lines = [f"# {title}\n\n",
             "Commands (from the repository root; rocprofv3 run from /tmp with TMPDIR=/tmp):\n\n",
             "```\n" + command.strip() + "\n```\n\n"]
    if notes:
        lines.append(notes.strip() + "\n\n")
    for k, row in table.items():
        r = row["resources"]
        lines.append(f"## {k}\n\n{row['dispatches']} dispatches; grid {r.get('Grid_Size')} work-items in groups of "
                     f"{r.get('Workgroup_Size')}; {r.get('VGPR_Count')} VGPRs + {r.get('Accum_VGPR_Count')} AGPRs, "
                     f"{r.get('SGPR_Count')} SGPRs, {r.get('LDS_Block_Size')} B LDS and {r.get('Scratch_Size')} B "
                     f"scratch per work-item as recorded.\n\n")
        if row["shares"]:
            lines += ["| Share of wave time | Counter / SQ_WAVE_CYCLES |\n", "|---|---|\n"]
            for c, what in SHARES:
                if c in row["shares"]:
                    lines.append(f"| {what} | {row['shares'][c]:.3f} ({c}) |\n")
            lines.append("\n")
        lines += ["| Counter | Mean per dispatch |\n", "|---|---|\n"]
        for c, v in row["counters"].items():
            lines.append(f"| {c} | {v:.1f} |\n")
        lines.append("\n")
    with open(out, "w") as fh:
        fh.writelines(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what")
    t = sub.add_parser("traffic", help="FETCH_SIZE / WRITE_SIZE passes -> bytes per launch")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, default=256 << 20)
    t.add_argument("--workload", required=True)
    t.add_argument("--tokens", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--command", required=True)
    k = sub.add_parser("kernels", help="rocprofv3 --stats kernel summary -> markdown table")
    k.add_argument("--stats", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--out", required=True)
    k.add_argument("--command", required=True)
    k.add_argument("--notes", default="")
    c = sub.add_parser("counters", help="SQ counter passes -> per-kernel means and shares of wave time")
    c.add_argument("--pmc", required=True, nargs="+")
    c.add_argument("--title", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--notes", default="")
    a = ap.parse_args()
    if a.what == "counters":
        write_counter_summary(a.out, counter_table(a.pmc), a.title, a.command, a.notes)
    elif a.what == "kernels":
        write_kernel_summary(a.out, kernel_stats(a.stats), a.title, a.command, a.notes)
    else:
        write_summary(a.out, traffic_table(a.fetch, a.write, a.copy_bytes), a.workload, a.tokens, a.command)


if __name__ == "__main__":
    main()
