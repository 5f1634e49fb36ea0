"""Summaries of rocprofv3 result databases, as the short text kept under
profiles/.

Kernel trace (per-kernel launch count and average / min / max duration):

    python rocprof_summary.py <db or dir> [title] [command]

Other counters of chosen kernels, averaged per dispatch, with the matrix
cores' busy fraction:

    python rocprof_summary.py --pmc --db <run> [--db <run>] --kernels a,b \
        --title ... --command ...

HBM byte counters (FETCH_SIZE / WRITE_SIZE, KiB per dispatch) of chosen
kernels, scaled by what the same counter reads for a plain device copy of
known size in the same run (the copy bench.py makes with
--calibrate-copy-mb), with the SHA-1 of the kernels' source so a reader can
tell whether the figures still describe the code:

    python rocprof_summary.py --counters \
        --db <fetch run> --db <write run> --copy-bytes N --kernels a,b \
        --source <file> --title ... --command ... --command ...
"""
import argparse
import glob
import hashlib
import os
import sqlite3
import sys


def _find_db(path):
    if os.path.isdir(path):
        found = glob.glob(os.path.join(path, "**", "*.db"), recursive=True)
        if not found:
            raise FileNotFoundError(f"no .db under {path}")
        return found[0]
    return path


def summarize(db, title="", command=""):
    c = sqlite3.connect(_find_db(db))
    rows = c.execute("select name, count(*), avg(end-start), min(end-start), max(end-start), "
                     "sum(end-start) from kernels group by name order by sum(end-start) desc"
                     ).fetchall()
    out = [f"# {title}".rstrip(), ""]
    if command:
        out += ["command:", "", "    " + command, ""]
    out.append("| kernel | launches | avg us | min us | max us | total us |")
    out.append("|---|---|---|---|---|---|")
    for name, cnt, avg, mn, mx, tot in rows:
        out.append(f"| {_short(name)} | {cnt} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | "
                   f"{mx / 1e3:.2f} | {tot / 1e3:.1f} |")
    return "\n".join(out) + "\n"


def counter_table(dbs):
    """{(kernel, counter): [values per dispatch]} over the given databases."""
    agg = {}
    for db in dbs:
        c = sqlite3.connect(_find_db(db))
        for name, cname, v in c.execute(
                "select kernel_name, counter_name, value from counters_collection"):
            agg.setdefault((_short(name), cname), []).append(v)
    return agg


def copy_factors(agg, copy_bytes):
    """Known bytes / counted bytes of the largest plain copy, per counter."""
    f = {}
    for (k, cname), vals in agg.items():
        if k.startswith("__amd_rocclr_copyBuffer") and cname in ("FETCH_SIZE", "WRITE_SIZE"):
            big = max(vals)
            if big > 0:
                f[cname] = copy_bytes / (big * 1024.0)
    return f


def counters_report(dbs, copy_bytes, kernels, source, title, commands):
    agg = counter_table(dbs)
    fac = copy_factors(agg, copy_bytes)
    out = [f"# {title}", ""]
    out += ["commands:", ""] + ["    " + c for c in commands] + [""]
    out.append(f"calibration: plain copy of {copy_bytes} bytes; factor = known bytes / "
               "counted bytes: " + ", ".join(f"{k} x{v:.3f}" for k, v in sorted(fac.items())))
    out += ["", "| kernel | counter | dispatches | avg KiB | scaled MB per dispatch |",
            "|---|---|---|---|---|"]
    per_launch = 0.0
    for (k, cname), vals in sorted(agg.items()):
        if not any(k.startswith(p) for p in kernels):
            continue
        avg = sum(vals) / len(vals)
        scaled = avg * 1024 * fac[cname] if cname in fac else None
        out.append(f"| {k} | {cname} | {len(vals)} | {avg:.1f} | "
                   f"{'' if scaled is None else f'{scaled / 1e6:.2f}'} |")
        if scaled is not None:
            per_launch += scaled
    sha = hashlib.sha1(open(source, "rb").read()).hexdigest()
    out += ["", f"traffic_bytes_per_launch: {per_launch:.0f}",
            f"source: {os.path.relpath(source, os.path.dirname(os.path.abspath(__file__)))}",
            f"source_sha1: {sha}"]
    return "\n".join(out) + "\n"


def pmc_report(dbs, kernels, title, commands, simds=1024, xcds=8):
    """Per-kernel averages of every counter in the given runs, and for the
    matrix-core counters the busy fraction: SQ_VALU_MFMA_BUSY_CYCLES over
    (SIMDs x GRBM_GUI_ACTIVE / XCDs), GRBM_GUI_ACTIVE being summed over the
    XCDs (MI355X: 256 CUs x 4 SIMDs, 8 XCDs)."""
    agg = counter_table(dbs)
    out = [f"# {title}", ""]
    out += ["commands:", ""] + ["    " + c for c in commands] + [""]
    out += ["| kernel | counter | dispatches | average per dispatch |", "|---|---|---|---|"]
    per = {}
    for (k, cname), vals in sorted(agg.items()):
        if not any(k.startswith(p) for p in kernels):
            continue
        avg = sum(vals) / len(vals)
        per.setdefault(k, {})[cname] = avg
        out.append(f"| {k} | {cname} | {len(vals)} | {avg:.4g} |")
    out.append("")
    for k, c in sorted(per.items()):
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "GRBM_GUI_ACTIVE" in c and c["GRBM_GUI_ACTIVE"] > 0:
            cyc = c["GRBM_GUI_ACTIVE"] / xcds
            out.append(f"- {k}: {cyc:.4g} cycles per XCD; matrix cores busy "
                       f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / (simds * cyc):.3f} of the SIMD cycles")
            if c.get("SQ_INSTS_MFMA"):
                out.append(f"  ({c['SQ_VALU_MFMA_BUSY_CYCLES'] / c['SQ_INSTS_MFMA']:.1f} busy "
                           f"cycles per MFMA instruction; {c.get('SQ_INSTS_VALU', 0) / c['SQ_INSTS_MFMA']:.2f}"
                           " VALU instructions per MFMA)")
    return "\n".join(out) + "\n"


def read_traffic(path, source):
    """traffic_bytes_per_launch from a counters summary, or None when the
    summary is missing or was taken on another version of `source`."""
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    kv = dict(l.split(": ", 1) for l in lines if ": " in l and not l.startswith("|"))
    try:
        sha = hashlib.sha1(open(source, "rb").read()).hexdigest()
    except OSError:
        return None
    if kv.get("source_sha1") != sha or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


def _short(name):
    short = name.replace("(anonymous namespace)::", "")
    if short.startswith("void "):
        short = short[5:]
    depth = 0
    for i, ch in enumerate(short):
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            return short[:i]
    return short


def main(argv):
    if argv and argv[0] == "--counters":
        ap = argparse.ArgumentParser()
        ap.add_argument("--db", action="append", required=True)
        ap.add_argument("--copy-bytes", type=int, required=True)
        ap.add_argument("--kernels", required=True)
        ap.add_argument("--source", required=True)
        ap.add_argument("--title", default="")
        ap.add_argument("--command", action="append", default=[])
        a = ap.parse_args(argv[1:])
        print(counters_report(a.db, a.copy_bytes, a.kernels.split(","), a.source, a.title,
                              a.command), end="")
        return 0
    if argv and argv[0] == "--pmc":
        ap = argparse.ArgumentParser()
        ap.add_argument("--db", action="append", required=True)
        ap.add_argument("--kernels", required=True)
        ap.add_argument("--title", default="")
        ap.add_argument("--command", action="append", default=[])
        a = ap.parse_args(argv[1:])
        print(pmc_report(a.db, a.kernels.split(","), a.title, a.command), end="")
        return 0
    print(summarize(argv[0], *(argv[1:3])), end="")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
