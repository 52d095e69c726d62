"""Build (here) and run (on the GPU) the standalone microbenchmarks.

    python -m deberta_disentangled_attention_amd.microbench.run build
    python -m deberta_disentangled_attention_amd.microbench.run run
"""

import os
import subprocess
import sys

from .. import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "bin")
PROGRAMS = ["mfma_valu", "lds_read"]


def build() -> None:
    os.makedirs(BIN, exist_ok=True)
    for p in PROGRAMS:
        cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-O3", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-w", "-o", os.path.join(BIN, p), os.path.join(HERE, p + ".hip")]
        subprocess.run(cmd, check=True)
        print("built", os.path.join(BIN, p))


def run() -> None:
    for p in PROGRAMS:
        print(f"## {p}\n", flush=True)
        subprocess.run([os.path.join(BIN, p)], check=True)
        print(flush=True)


if __name__ == "__main__":
    if len(sys.argv) != 2 or sys.argv[1] not in ("build", "run"):
        raise SystemExit(__doc__)
    build() if sys.argv[1] == "build" else run()
