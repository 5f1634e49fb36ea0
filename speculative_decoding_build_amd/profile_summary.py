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
        short = name.replace("(anonymous namespace)::", "")
        if short.startswith("void "):
            short = short[5:]
        depth = 0
        for i, ch in enumerate(short):          # cut at the argument list
            depth += ch == "<"
            depth -= ch == ">"
            if ch == "(" and depth == 0:
                short = short[:i]
                break
        out.append(f"| {short} | {cnt} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | "
                   f"{tot / 1e3:.1f} |")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    path = sys.argv[1]
    if os.path.isdir(path):
        path = glob.glob(os.path.join(path, "**", "*.db"), recursive=True)[0]
    print(summarize(path, *(sys.argv[2:4])))
