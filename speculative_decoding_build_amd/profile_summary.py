"""Summarise a rocprofv3 kernel-trace database (per-kernel launch count and
average / min / max duration) as the text kept under profiles/.

    python -m speculative_decoding_build_amd.profile_summary <results.db> [title] [command]
"""
import glob
import os
import sqlite3
import sys


def summarize(db, title="", command=""):
    c = sqlite3.connect(db)
    rows = c.execute("select name, count(*), avg(end-start), min(end-start), max(end-start), "
                     "sum(end-start) from kernels group by name order by sum(end-start) desc"
                     ).fetchall()
    out = [f"# {title}".rstrip(), ""]
    if command:
        out += ["command:", "", "    " + command, ""]
    out.append("| kernel | launches | avg us | min us | max us | total us |")
    out.append("|---|---|---|---|---|---|")
    for name, cnt, avg, mn, mx, tot in rows:
        short = _short(name)
        out.append(f"| {short} | {cnt} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | "
                   f"{tot / 1e3:.1f} |")
    return "\n".join(out) + "\n"


def counters(db, copy_bytes=0):
    """Per-kernel average of every counter in a rocprofv3 --pmc database.
    With ``copy_bytes`` (the size of the plain copy the run made), byte
    counters (FETCH_SIZE, WRITE_SIZE, in KiB) are also reported scaled by the
    factor that maps the copy kernel's reading onto its known size."""
    c = sqlite3.connect(db)
    rows = c.execute("select kernel_name, counter_name, value, grid_size from counters_collection"
                     ).fetchall()
    agg = {}
    for name, cname, v, g in rows:
        agg.setdefault((_short(name), cname), []).append((v, g))
    factor = {}
    if copy_bytes:
        for (k, cname), vals in agg.items():
            if k.startswith("__amd_rocclr_copyBuffer") and cname in ("FETCH_SIZE", "WRITE_SIZE"):
                big = max(v for v, _ in vals)
                factor[cname] = copy_bytes / (big * 1024.0) if big > 0 else None
    out = []
    for (k, cname), vals in sorted(agg.items()):
        avg = sum(v for v, _ in vals) / len(vals)
        line = f"| {k} | {cname} | {len(vals)} | {avg:.1f} |"
        if cname in factor and factor[cname]:
            line += f" {avg * 1024 * factor[cname] / 1e6:.1f} MB (x{factor[cname]:.3f}) |"
        else:
            line += " |"
        out.append(line)
    return factor, out


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


if __name__ == "__main__":
    if sys.argv[1] == "--counters":
        path = sys.argv[2]
        if os.path.isdir(path):
            path = glob.glob(os.path.join(path, "**", "*.db"), recursive=True)[0]
        copy_bytes = int(sys.argv[3]) if len(sys.argv) > 3 else 0
        f, lines = counters(path, copy_bytes)
        print("| kernel | counter | dispatches | average | scaled |")
        print("|---|---|---|---|---|")
        print("\n".join(lines))
        if f:
            print("\nscale factors (known copy bytes / counter bytes):", f)
        sys.exit(0)
    path = sys.argv[1]
    if os.path.isdir(path):
        path = glob.glob(os.path.join(path, "**", "*.db"), recursive=True)[0]
    print(summarize(path, *(sys.argv[2:4])))
