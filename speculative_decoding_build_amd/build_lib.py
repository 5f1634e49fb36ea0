"""Builds libspecmi.so (the C-ABI library) from csrc/*.hip for gfx950.

    python speculative_decoding_build_amd/build_lib.py

Run as a script (the package itself refuses to import before the library
exists).  Each source compiles to an object of its own (in parallel), then
one link makes the shared library.
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libspecmi.so")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]
# Per-source flags (none at present).
EXTRA = {}


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _filter(stderr):
    return "\n".join(l for l in (stderr or "").splitlines() if "packed-fp32-ops" not in l)


def build(verbose=False) -> str:
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    with tempfile.TemporaryDirectory() as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, f"--offload-arch={ARCH}"] + COMMON + \
                EXTRA.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            return obj, res

        jobs = max(1, min(len(srcs), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(compile_one, srcs))
        for (obj, res), src in zip(results, srcs):
            err = _filter(res.stderr)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)} "
                                   f"({res.returncode}):\n{err}")
            if err.strip() and verbose:
                print(err, file=sys.stderr)
        out = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out] + \
            [obj for obj, _ in results]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{_filter(res.stderr)}")
        os.replace(out, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
