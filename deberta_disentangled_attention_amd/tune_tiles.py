"""Wave-count sweep of the forward's tiles (16-bit types): builds one library
per candidate, times bench.py's workloads with each, and records the kernel
times as JSON lines (resumable: entries already in the file are skipped).

    # on the build machine: compile the candidates
    python -m deberta_disentangled_attention_amd.tune_tiles build
    # on the GPU: time them (appends to OUT)
    python -m deberta_disentangled_attention_amd.tune_tiles run OUT [workload ...]
    # summarise OUT as a markdown table
    python -m deberta_disentangled_attention_amd.tune_tiles table OUT

A candidate fixes 32 NW queries per workgroup for every length
(-DDATTN_NW_D32 / D64 / D128); the kernel supports NW = 2, 4 at d = 32,
2, 4, 8 at d = 64 and 4, 8 at d = 128 (16-bit types). The in-tree build's
dispatch is the product; these libraries exist only to measure.
"""

from __future__ import annotations

import json
import os
import subprocess
import sys

from . import build as B

ROOT = os.path.dirname(B.PKG_DIR)
OUT_DIR = os.path.join(B.PKG_DIR, "tune_bin")
CANDIDATES = {
    "nw2": ["-DDATTN_NW_D32=2", "-DDATTN_NW_D64=2", "-DDATTN_NW_D128=4"],
    "nw4": ["-DDATTN_NW_D32=4", "-DDATTN_NW_D64=4", "-DDATTN_NW_D128=4"],
    "nw8": ["-DDATTN_NW_D32=4", "-DDATTN_NW_D64=8", "-DDATTN_NW_D128=8"],
}
WORKLOADS = ["c2", "c3", "c3p", "c4", "c4l2048", "c4l4096", "c5d32", "c5d128"]


def lib_path(name: str) -> str:
    return os.path.join(OUT_DIR, f"libdattn_{name}.so")


def build_all() -> None:
    os.makedirs(OUT_DIR, exist_ok=True)
    for name, flags in CANDIDATES.items():
        B.build(verbose=False, out=lib_path(name), extra=flags)
        print("built", lib_path(name), flush=True)


def run(out: str, workloads) -> None:
    done = set()
    if os.path.exists(out):
        for line in open(out):
            r = json.loads(line)
            done.add((r["candidate"], r["workload"]))
    for w in workloads:
        for name in CANDIDATES:
            if (name, w) in done:
                continue
            env = dict(os.environ, DATTN_LIB=lib_path(name))
            cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", w, "--steps", "30",
                   "--warmup", "5", "--no-cpu-baseline"]
            res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=300)
            if res.returncode != 0:
                raise RuntimeError(f"{name} {w}: {res.stderr[-2000:]}")
            r = json.loads(res.stdout.strip().splitlines()[-1])
            rec = {"candidate": name, "workload": w, "kernel_avg_ms": r["roofline"]["kernel_avg_ms"],
                   "kernel_median_ms": r["roofline"]["kernel_median_ms"], "frac": r["roofline"]["frac"]}
            with open(out, "a") as f:
                f.write(json.dumps(rec) + "\n")
            print(json.dumps(rec), flush=True)


def table(out: str) -> str:
    rows = [json.loads(l) for l in open(out)]
    ws = [w for w in WORKLOADS if any(r["workload"] == w for r in rows)]
    lines = ["| workload | " + " | ".join(CANDIDATES) + " | fastest |", "|---" * (len(CANDIDATES) + 2) + "|"]
    for w in ws:
        t = {r["candidate"]: r["kernel_median_ms"] for r in rows if r["workload"] == w}
        best = min(t, key=t.get)
        lines.append(f"| {w} | " + " | ".join(f"{t.get(c, float('nan')):.4f}" for c in CANDIDATES) + f" | {best} |")
    return "\n".join(lines)


if __name__ == "__main__":
    if len(sys.argv) < 2 or sys.argv[1] not in ("build", "run", "table"):
        raise SystemExit(__doc__)
    if sys.argv[1] == "build":
        build_all()
    elif sys.argv[1] == "run":
        run(sys.argv[2], sys.argv[3:] or WORKLOADS)
    else:
        print(table(sys.argv[2]))
