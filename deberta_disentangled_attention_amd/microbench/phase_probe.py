"""Where a forward workgroup spends its time: cycles per wave in the
prologue (from the work item's start to its first tile: mask or sequence
search, Q row, relative-table thresholds and window), in the general (band)
tiles and in the far tiles, and inside the general tiles the split between
the tile start (load wait and barrier), the score products (C2C, the band
products E and F and their diagonal gathers; both halves) and the softmax with
P.V (both halves).

It builds a separate library from a copy of the kernel sources with
s_memtime reads inserted at the phase boundaries; that library's *_lse
forward writes, for each wave, the accumulated cycle counts into the lse
rows of the wave's queries (row 32w + k holds counter k % 8) instead of the
log-sum-exp. The product library is not touched.

    python -m deberta_disentangled_attention_amd.microbench.phase_probe build
    python -m deberta_disentangled_attention_amd.microbench.phase_probe run c4 c4l2048 c2

With --split (on both commands, its own library) two counters change meaning:
the far-step count becomes the general tiles' wait for their loads alone
(before the barrier), and the prologue becomes the P2C block of the general
tiles (its products, next-row fetches and diagonal sums), both in cycles per
general tile.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from .. import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
SRC_DIR = os.path.join(HERE, "bin", "phase_src")
LIB = os.path.join(HERE, "bin", "libdattn_phase.so")
SPLIT = "--split" in sys.argv
if SPLIT:
    SRC_DIR = os.path.join(HERE, "bin", "phase_split_src")
    LIB = os.path.join(HERE, "bin", "libdattn_phase_split.so")
ROOT = os.path.dirname(B.PKG_DIR)

COUNTERS = ["general tiles, all", "far tiles, all", "general tiles (count)", "far steps (count)",
            "general: start (wait, barrier, loads issue)", "general: score products",
            "general: softmax + P.V", "prologue"]
if SPLIT:
    COUNTERS[3] = "general: load wait only"
    COUNTERS[7] = "general: P2C block"


def _sub(text: str, anchor: str, new: str) -> str:
    if text.count(anchor) != 1:
        raise RuntimeError(f"instrumentation anchor not found exactly once: {anchor[:60]!r}")
    return text.replace(anchor, new)


def instrument(src: str) -> str:
    stamp = "__builtin_amdgcn_s_memtime()"
    src = _sub(src, "  constexpr int NT = C::NT;\n", f"  constexpr int NT = C::NT;\n  const uint64_t pe_ = {stamp};\n")
    src = _sub(src, "  const int key_end = min(ext, first_bad);  // keys below this need no mask test",
               "  const int key_end = min(ext, first_bad);  // keys below this need no mask test\n"
               "  float pc_[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};\n  uint64_t pg0_ = 0, pt_ = 0, pf0_ = 0;")
    src = _sub(src, "    if (first_general >= 0) {\n      if (tw_ok) phase1g(std::true_type{});",
               f"    pg0_ = {stamp};\n    pc_[7] = (float)(pg0_ - pe_);\n    if (first_general >= 0) {{\n      if (tw_ok) phase1g(std::true_type{{}});")
    src = _sub(src, "    const int nfar = FL + max(tm - FR, 0);\n    if (nfar > 0) {\n      const float tl2",
               f"    pf0_ = {stamp};\n    pc_[0] += (float)(pf0_ - pg0_);\n"
               "    const int nfar = FL + max(tm - FR, 0);\n    pc_[3] += (float)nfar;\n"
               "    if (nfar > 0) {\n      const float tl2")
    src = _sub(src, "  // ---- phase 2 (fp32): far tiles, double-buffered through registers --------",
               f"  if constexpr (ES == 2) pc_[1] += (float)({stamp} - pf0_);\n"
               "  // ---- phase 2 (fp32): far tiles, double-buffered through registers --------")
    src = _sub(src, "        wait_vm<0>();\n        __syncthreads();  // tile t in its slot; the other slot is free\n",
               f"        pt_ = {stamp};\n"
               "        wait_vm<0>();\n        __syncthreads();  // tile t in its slot; the other slot is free\n")
    src = _sub(src, "        half(std::integral_constant<int, 0>{});\n",
               f"        {{ const uint64_t tt_ = {stamp}; pc_[4] += (float)(tt_ - pt_); pt_ = tt_; }}\n"
               "        half(std::integral_constant<int, 0>{});\n")
    src = _sub(src, "        half(std::integral_constant<int, 1>{});\n",
               "        half(std::integral_constant<int, 1>{});\n        pc_[2] += 1.f;\n")
    src = _sub(src, "          mask_keys(kb, acc);\n          softmax_pv_half(acc, kb, m.a_off, vop_slot(vs));\n",
               f"          {{ const uint64_t tt_ = {stamp}; pc_[5] += (float)(tt_ - pt_); pt_ = tt_; }}\n"
               "          mask_keys(kb, acc);\n          softmax_pv_half(acc, kb, m.a_off, vop_slot(vs));\n"
               f"          {{ const uint64_t tt_ = {stamp}; pc_[6] += (float)(tt_ - pt_); pt_ = tt_; }}\n")
    src = _sub(src, "      p.lse[(base + qi) * p.H + head] = row_ok ? (m_run + log2f(l_tot)) * 0.6931471805599453f : NEG_INF;",
               "      { const int kk_ = li & 7; float v_ = 0.f;\n"
               "#pragma unroll\n        for (int z_ = 0; z_ < 8; ++z_) if (kk_ == z_) v_ = pc_[z_];\n"
               "        p.lse[(base + qi) * p.H + head] = v_; }")
    if SPLIT:
        src = _sub(src, "    pc_[3] += (float)nfar;\n", "")
        src = _sub(src, "    pc_[7] = (float)(pg0_ - pe_);\n", "")
        src = _sub(src, "        wait_vm<0>();\n        __syncthreads();  // tile t in its slot",
                   f"        wait_vm<0>();\n        {{ const uint64_t tw_ = {stamp}; pc_[3] += (float)(tw_ - pt_); }}\n"
                   "        __syncthreads();  // tile t in its slot")
        src = _sub(src, "          if (fb) {\n            if constexpr (F16) {",
                   f"          const uint64_t tf_ = {stamp};\n          if (fb) {{\n            if constexpr (F16) {{")
        src = _sub(src, "          if (eb) {\n            const f32x16_t e0",
                   f"          pc_[7] += (float)({stamp} - tf_);\n          if (eb) {{\n            const f32x16_t e0")
    return src


def build() -> str:
    shutil.rmtree(SRC_DIR, ignore_errors=True)
    shutil.copytree(B.CSRC, SRC_DIR)
    api = os.path.join(SRC_DIR, "dattn_api.hip")
    text = open(api).read().replace('#include "../../include/dattn.h"', '#include "dattn.h"')
    open(api, "w").write(text)
    fwd = os.path.join(SRC_DIR, "dattn_fwd.hip")
    text = instrument(open(fwd).read())
    open(fwd, "w").write(text)
    flags = [f"--offload-arch={B.ARCH}", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-w", f"-I{os.path.join(ROOT, 'include')}"]
    objs = [os.path.join(SRC_DIR, s + ".o") for s in B.SOURCES]

    def cc(pair):
        s, o = pair
        subprocess.run([B.hipcc(), *flags, *B.source_flags(s), "-c", "-o", o, os.path.join(SRC_DIR, s)], check=True)

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(cc, zip(B.SOURCES, objs)))
    subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", LIB, *objs], check=True)
    for o in objs:
        os.remove(o)
    print("built", LIB)
    return LIB


def run(workloads) -> None:
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    import bench
    import deberta_disentangled_attention_amd as dd

    # this package was imported before any setting could take effect: point
    # the binding at the probe library before its first call loads one
    if dd._lib_handle is not None:
        raise RuntimeError("the product library is already loaded")
    dd.LIB_PATH = LIB

    print("| workload | " + " | ".join(COUNTERS) + " |")
    print("|---|" + "---:|" * len(COUNTERS))
    for name in workloads:
        w = bench.build_workload(name)
        tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w.dtype]
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(tdt).cuda()
        q, k, v, qr, kr = dev(w.q), dev(w.k), dev(w.v), dev(w.qr), dev(w.kr)
        relmax = w.max_seqlen if w.packed else w.L
        table = dd.rel_bucket(relmax, w.position_buckets, w.max_relative_positions, device="cuda")
        for _ in range(3):
            if w.packed:
                cu = torch.from_numpy(w.cu_seqlens).cuda()
                _, lse = dd.dattn_fwd_varlen(q, k, v, qr, kr, table, relmax, cu, w.max_seqlen, w.H, w.d,
                                             flags=w.flags, lse=True)
            else:
                mask = None if w.mask is None else torch.from_numpy(w.mask).cuda()
                _, lse = dd.dattn_fwd_padded(q, k, v, qr, kr, table, relmax, mask, w.H, w.d,
                                             flags=w.flags, lse=True)
        torch.cuda.synchronize()
        L = lse.float().cpu().numpy().reshape(-1, w.H)
        # counter c of a wave sits in its rows 8g + c; waves with no general
        # tile (count 0) are left out of the per-tile averages
        c = [L[i::8].reshape(-1) for i in range(8)]
        n = np.minimum.reduce([len(x) for x in c])
        c = [x[:n] for x in c]
        # waves of query tiles with no valid query return before the
        # counters are written (their rows hold -inf): left out
        ok = np.all(np.isfinite(np.stack(c)), axis=0)
        c = [x[ok] for x in c]
        live = c[2] > 0
        per_g = lambda x: float(np.mean(x[live] / c[2][live])) if live.any() else 0.0
        vals = [np.mean(c[0]), np.mean(c[1]), np.mean(c[2]), np.mean(c[3]), per_g(c[4]), per_g(c[5]),
                per_g(c[6]), np.mean(c[7])]
        if SPLIT:
            vals[3], vals[7] = per_g(c[3]), per_g(c[7])
        print(f"| {name} | " + " | ".join(f"{x:.0f}" if i not in (2, 3) else f"{x:.1f}"
                                            for i, x in enumerate(vals)) + " |", flush=True)
    print("\nTotals and the prologue are cycles per wave (s_memtime); the three general-tile parts are"
          " cycles per general tile.")


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if a != "--split"]
    if not args or args[0] not in ("build", "run"):
        raise SystemExit(__doc__)
    if args[0] == "build":
        build()
    else:
        run(args[1:] or ["c4"])
