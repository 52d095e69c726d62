#!/usr/bin/env python3
"""Benchmark of the disentangled-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4]
    python bench.py --pack [--workload c3]     # padded vs device-packed
    python bench.py --relproj [--workload c2]  # qr/kr projection of that shape

A step is one pass of the whole hot path over one batch of synthetic input:
the relative-row table (rel_bucket) and the fused forward
(dattn_fwd_varlen / dattn_fwd_padded), both through the C ABI. Inputs are
resident in HBM before the timed region. The default workload is the
long-context packed case: 16 sequences of 8192 tokens (131072 tokens),
12 heads of 64, bf16, DeBERTa-v2 log buckets 256/512.

Output: one JSON line with the metric (effective TFLOP/s, counting 6*d per
valid (query, key) pair and head), tokens/s, the roofline object of the
dominant kernel (the fused forward; its average duration from HIP events
recorded on the launch stream around each launch) and the CPU oracle timed
on a bounded sample of the same workload.

--pack times, for a padded workload with a mask, the padded forward beside
the packed route: dattn_pack_index on the mask, dattn_pack_rows of the
fused QKV rows, the packed forward, and dattn_unpack_rows of the output.
The metadata and the packed activations are built once per batch and reused
by every layer, so the line reports the per-layer forward times and the
per-batch packing cost separately.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s + tokens/s, disentangled attn fwd, bf16 d=64, % MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}   # MI355X dense MFMA
HBM_GBS = 8000.0
KERNEL_SOURCES = ["deberta_disentangled_attention_amd/csrc/dattn_fwd.hip",
                  "deberta_disentangled_attention_amd/csrc/dattn_fwd_d128.hip",
                  "deberta_disentangled_attention_amd/csrc/dattn_device.h",
                  "deberta_disentangled_attention_amd/build.py"]   # its flags shape the kernel too
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dattn_fwd_c4_bf16_traffic.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def build_workload(name: str):
    import workloads
    table = {
        "c4": lambda: workloads.c4_long_packed_bf16(),
        "c4l2048": lambda: workloads.c4_long_packed_bf16(nseq=64, seqlen=2048),
        "c4l4096": lambda: workloads.c4_long_packed_bf16(nseq=32, seqlen=4096),
        "c2": lambda: workloads.c2_v3base_bf16(),
        "c3": lambda: workloads.c3_v2xlarge_fp16(),
        "c3p": lambda: workloads.c3_v2xlarge_fp16(packed=True),
        "c5d32": lambda: workloads.c5_sweep(32, "bf16"),
        "c5d128": lambda: workloads.c5_sweep(128, "bf16"),
        "c5f32": lambda: workloads.c5_sweep(128, "fp32"),
        "c1": lambda: workloads.c1_tiny_fp32(),
    }
    if name not in table:
        raise SystemExit(f"unknown workload {name}; choose from {sorted(table)}")
    return table[name]()


def algorithmic_bytes(w) -> float:
    """HBM bytes the forward must move at least: Q, K, V read and O written
    once per valid token and head (4 d esize), qr and kr read once per head
    (2 n_rel d esize), and for the padded layout the zero rows of the
    output, the mask and the relative-row table."""
    import workloads
    es = workloads.ESIZE[w.dtype]
    b = 4.0 * w.d * es * w.H * w.total_tokens
    if w.flags:
        b += 2.0 * w.n_rel * w.d * es * w.H
        b += 4.0 * (2 * (w.max_seqlen if w.packed else w.L) - 1)
    if not w.packed:
        b += (w.B * w.L - w.total_tokens) * w.H * w.d * es
        if w.mask is not None:
            b += w.B * w.L
    return b


def describe(w) -> str:
    lay = "packed" if w.packed else "padded+mask" if w.mask is not None else "padded"
    bucket = (f"log buckets {w.position_buckets}/{w.max_relative_positions}"
              if w.position_buckets > 0 else f"identity span {w.max_relative_positions}")
    return (f"{w.name}: {lay}, B={w.B}, L={w.L}, H={w.H}, d={w.d}, {w.dtype}, {bucket}, "
            f"{w.total_tokens} valid tokens")


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample, worker processes)
# ---------------------------------------------------------------------------

def _oracle_unit(args):
    from threadpoolctl import threadpool_limits
    import oracle.attention as oa
    (Qh, Kh, Vh, QRh, KRh, T, relmax, flags, d) = args
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oa.unit_forward(Qh, Kh, Vh, QRh, KRh, T, relmax, None, flags, oa.default_scale(d, flags))
        return time.perf_counter() - t0


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, max_units: int) -> dict:
    import multiprocessing as mp
    import numpy as np
    import oracle
    host_cores = len(os.sched_getaffinity(0))
    cores = min(host_cores, max_units)
    relmax = w.max_seqlen if w.packed else w.L
    T = oracle.rel_index_table(relmax, w.position_buckets, w.max_relative_positions)
    cu = w.cu_seqlens
    rng = np.random.default_rng(7)
    order = rng.permutation(w.B * w.H)[:cores]
    jobs, flop = [], 0.0
    for u in order:
        b, h = divmod(int(u), w.H)
        n = int(w.lens[b])
        sl = slice(int(cu[b]), int(cu[b + 1])) if w.packed else slice(0, n)
        src = (lambda x: x[sl]) if w.packed else (lambda x: x[b, sl])
        col = slice(h * w.d, (h + 1) * w.d)
        jobs.append((src(w.q)[:, col].astype(np.float64), src(w.k)[:, col].astype(np.float64),
                     src(w.v)[:, col].astype(np.float64), w.qr[:, col].astype(np.float64),
                     w.kr[:, col].astype(np.float64), T, relmax, w.flags, w.d))
        flop += (6 if w.flags else 4) * w.d * float(n) ** 2
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(processes=cores) as pool:
        pool.map(_oracle_unit, jobs, chunksize=1)
    wall = time.perf_counter() - t0
    return {"value": flop / wall / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(jobs)} of the {w.B * w.H} whole (sequence, head) units of "
                      f"{describe(w).split(':')[0]} ({int(w.lens.max())} tokens each at most), "
                      f"float64 numpy oracle, one single-threaded worker process per unit on "
                      f"{cores} of the {host_cores} host cores available; wall {wall:.2f} s",
            "wall_s": wall, "host_cores": host_cores, "cpu_model": cpu_model(),
            "units_timed": len(jobs), "units_total": w.B * w.H}


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def load_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None          # counters were taken on another version of the kernel
    return rec.get("traffic_bytes_per_launch")


# ---------------------------------------------------------------------------
# HBM traffic of the forward from rocprofv3 counters
# ---------------------------------------------------------------------------

COPY_PROBE_BYTES = 1 << 30


def copy_probe():
    """Three launches of a plain elementwise copy of 1 GiB (read 1 GiB,
    write 1 GiB), for calibrating FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(f"copy probe: {COPY_PROBE_BYTES} bytes read and written per launch, 3 launches")


def _counter_per_dispatch(csv_path, counter, kernel_substr):
    import csv
    import collections
    by = collections.defaultdict(float)
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and kernel_substr in row["Kernel_Name"]:
                by[int(row["Dispatch_Id"])] += float(row["Counter_Value"])
    if not by:
        raise SystemExit(f"{csv_path}: no {counter} rows for kernels matching {kernel_substr!r}")
    vals = list(by.values())
    return sum(vals) / len(vals), len(vals)


def write_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """Combine four rocprofv3 --pmc runs into the traffic record bench.py
    reports: forward FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
    divided by the same counter's reading per byte of the copy probe."""
    kf, nf = _counter_per_dispatch(fetch_csv, "FETCH_SIZE", "dattn_fwd_kernel")
    kw, nw = _counter_per_dispatch(write_csv, "WRITE_SIZE", "dattn_fwd_kernel")
    cf, _ = _counter_per_dispatch(copy_fetch_csv, "FETCH_SIZE", "MulFunctor")
    cw, _ = _counter_per_dispatch(copy_write_csv, "WRITE_SIZE", "MulFunctor")
    f_fetch = cf * 1024.0 / COPY_PROBE_BYTES
    f_write = cw * 1024.0 / COPY_PROBE_BYTES
    traffic = kf * 1024.0 / f_fetch + kw * 1024.0 / f_write
    rec = {
        "kernel": "dattn_fwd_kernel (16 x 8192 packed bf16, H=12, d=64)",
        "kernel_source_sha256": kernel_source_hash(),
        "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw,
        "dispatches": [nf, nw],
        "copy_probe_bytes": COPY_PROBE_BYTES,
        "copy_fetch_kib": cf, "copy_write_kib": cw,
        "calibration_fetch": f_fetch, "calibration_write": f_write,
        "traffic_bytes_per_launch": traffic,
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def _timed(fn, steps, warmup):
    """Average ms of fn() from HIP events on torch's current stream (the
    stream the binding launches on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def bench_pack(args):
    import numpy as np
    import torch
    import deberta_disentangled_attention_amd as dd

    w = build_workload(args.workload)
    if w.packed or w.mask is None:
        raise SystemExit("--pack needs a padded workload with a mask (c2, c3)")
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(tdt).cuda()
    hd = w.H * w.d
    qkv = torch.cat([dev(w.q), dev(w.k), dev(w.v)], dim=-1)        # fused [B, L, 3*H*d]
    qr, kr = dev(w.qr), dev(w.kr)
    mask = torch.from_numpy(np.ascontiguousarray(w.mask, np.uint8)).cuda()
    table = dd.rel_bucket(w.L, w.position_buckets, w.max_relative_positions, device="cuda")
    out_pad = torch.empty((w.B, w.L, hd), dtype=tdt, device="cuda")
    cu, tr, rp, mx = dd.pack_index(mask)
    total, max_len = int(cu[-1].item()), int(mx.item())   # host metadata, read once per batch
    packed = torch.empty((total, 3 * hd), dtype=tdt, device="cuda")
    out_pk = torch.empty((total, hd), dtype=tdt, device="cuda")
    back = torch.empty((w.B, w.L, hd), dtype=tdt, device="cuda")
    q, k, v = qkv[..., :hd], qkv[..., hd:2 * hd], qkv[..., 2 * hd:]
    pq, pk, pv = packed[:, :hd], packed[:, hd:2 * hd], packed[:, 2 * hd:]

    def padded():
        dd.dattn_fwd_padded(q, k, v, qr, kr, table, w.L, mask, w.H, w.d, flags=w.flags,
                            out=out_pad)

    def index():
        dd.lib().dattn_pack_index(mask.data_ptr(), w.B, w.L, cu.data_ptr(), tr.data_ptr(),
                                  rp.data_ptr(), mx.data_ptr(), dd._stream(mask))

    def pack():
        dd.pack_rows(qkv, tr, out=packed)

    def attn():
        dd.dattn_fwd_varlen(pq, pk, pv, qr, kr, table, w.L, cu, max_len, w.H, w.d,
                            flags=w.flags, out=out_pk)

    def unpack():
        dd.unpack_rows(out_pk, rp, w.B, w.L, out=back)

    S, W = args.steps, args.warmup
    t_pad, t_idx, t_pack, t_attn, t_unpack = (_timed(f, S, W)
                                              for f in (padded, index, pack, attn, unpack))
    # the whole route once more, back to back, and a check that it agrees
    t_route = _timed(lambda: (index(), pack(), attn(), unpack()), S, W)
    same = bool(torch.equal(back, out_pad))
    es = qkv.element_size()
    pack_bytes = total * 3 * hd * es * 2 + w.B * w.L * 4
    unpack_bytes = (total + w.B * w.L) * hd * es + w.B * w.L * 4
    fixed = t_idx + t_pack + t_unpack
    gain = t_pad - t_attn
    res = {
        "metric": "padded vs device-packed forward (ms)",
        "workload": describe(w), "dtype": w.dtype, "nseq": w.B, "seq_len": w.L,
        "total_tokens": total, "max_seqlen": max_len,
        "padding_fraction": round(1.0 - total / (w.B * w.L), 4),
        "steps": S, "warmup": W,
        "padded_fwd_ms": round(t_pad, 4),
        "packed_fwd_ms": round(t_attn, 4),
        "pack_index_ms": round(t_idx, 4),
        "pack_rows_qkv_ms": round(t_pack, 4),
        "unpack_rows_ms": round(t_unpack, 4),
        "packed_route_ms": round(t_route, 4),
        "route_equals_padded": same,
        "pack_rows_GBps": round(pack_bytes / (t_pack * 1e-3) / 1e9, 1),
        "unpack_rows_GBps": round(unpack_bytes / (t_unpack * 1e-3) / 1e9, 1),
        "layers_to_amortise_packing": (round(fixed / gain, 3) if gain > 0 else None),
    }
    print(json.dumps(res), flush=True)


def bench_relproj(args):
    """Time dattn_rel_proj on the workload's table shape: E [n_rel, H*d],
    weights [H*d, H*d], both tables in one launch."""
    import torch
    import deberta_disentangled_attention_amd as dd
    import workloads

    w = build_workload(args.workload)
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    hd = w.H * w.d
    E, Wq, Wk, bq, bk = workloads.projection_inputs(0, w.n_rel, hd, hd, w.dtype)
    dev = lambda x: torch.from_numpy(x).to(tdt).cuda()
    E, Wq, Wk, bq, bk = dev(E), dev(Wq), dev(Wk), dev(bq), dev(bk)
    qr = torch.empty((w.n_rel, hd), dtype=tdt, device="cuda")
    kr = torch.empty_like(qr)
    ms = _timed(lambda: dd.rel_proj(E, Wq, Wk, bq, bk, qr=qr, kr=kr), args.steps, args.warmup)
    flop = 2 * 2.0 * w.n_rel * hd * hd
    byts = (w.n_rel * hd + 2 * hd * hd + 2 * hd + 2 * w.n_rel * hd) * E.element_size()
    peak = PEAK_TFLOPS[w.dtype]
    print(json.dumps({
        "metric": "relative-table projection (qr and kr, one launch)",
        "workload": describe(w), "dtype": w.dtype, "n_rel": w.n_rel, "hidden": hd, "out": hd,
        "steps": args.steps, "warmup": args.warmup, "ms": round(ms, 5),
        "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 2), "pct_mfma_peak": round(100 * flop / (ms * 1e-3) / 1e12 / peak, 2),
        "GBps_min_bytes": round(byts / (ms * 1e-3) / 1e9, 1),
    }), flush=True)


def bench_bwd(args):
    """Time the backward (every launch of one dattn_bwd_* call) on the
    workload, from the forward's output and log-sum-exp computed once.
    Credited work is 2.5x the forward's effective flop: the five
    L x L x d products of an attention backward (S and dP recomputed, dV,
    dQ, dK) against the forward's two."""
    import numpy as np
    import torch
    import deberta_disentangled_attention_amd as dd

    w = build_workload(args.workload)
    if args.flags is not None:
        w.flags = args.flags
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(tdt).cuda()
    q, k, v, qr, kr = dev(w.q), dev(w.k), dev(w.v), dev(w.qr), dev(w.kr)
    relmax = w.max_seqlen if w.packed else w.L
    table = dd.rel_bucket(relmax, w.position_buckets, w.max_relative_positions, device="cuda")
    band = (dd.rel_bucket_band(relmax, w.position_buckets, w.max_relative_positions)
            if w.flags else 1)
    gen = torch.Generator(device="cpu").manual_seed(12345)
    if w.packed:
        cu = torch.from_numpy(w.cu_seqlens).cuda()
        out, lse = dd.dattn_fwd_varlen(q, k, v, qr, kr, table, relmax, cu, w.max_seqlen, w.H,
                                       w.d, flags=w.flags, lse=True)
        dout = torch.randn(out.shape, generator=gen).to(tdt).cuda()
        need = dd.bwd_workspace_size(w.total_tokens, w.B, w.H, w.d, tdt, band)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

        def bwd():
            return dd.dattn_bwd_varlen(q, k, v, out, dout, lse, qr, kr, table, relmax, band, cu,
                                       w.max_seqlen, w.H, w.d, flags=w.flags, workspace=ws)
    else:
        mask = None if w.mask is None else torch.from_numpy(w.mask).cuda()
        out, lse = dd.dattn_fwd_padded(q, k, v, qr, kr, table, relmax, mask, w.H, w.d,
                                       flags=w.flags, lse=True)
        dout = torch.randn(out.shape, generator=gen).to(tdt).cuda()
        need = dd.bwd_workspace_size(w.B * w.L, w.B, w.H, w.d, tdt, band)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

        def bwd():
            return dd.dattn_bwd_padded(q, k, v, out, dout, lse, qr, kr, table, relmax, band, mask,
                                       w.H, w.d, flags=w.flags, workspace=ws)

    for _ in range(args.warmup):
        bwd()
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    for a, b in events:
        a.record()
        bwd()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in events)
    avg = sum(ms) / len(ms)
    flop = 2.5 * w.effective_flop()
    peak = PEAK_TFLOPS[w.dtype]
    print(json.dumps({
        "metric": "disentangled attention backward (dq, dk, dv, dqr, dkr), effective TFLOP/s",
        "workload": describe(w), "dtype": w.dtype, "flags": w.flags, "band": band,
        "steps": args.steps, "warmup": args.warmup,
        "ms_avg": round(avg, 4), "ms_median": round(ms[len(ms) // 2], 4),
        "ms_min": round(ms[0], 4), "ms_max": round(ms[-1], 4),
        "effective_flop": flop, "TFLOPs": round(flop / (avg * 1e-3) / 1e12, 2),
        "pct_mfma_peak": round(100 * flop / (avg * 1e-3) / 1e12 / peak, 2),
        "tokens_per_s": round(w.total_tokens / (avg * 1e-3), 1),
        "workspace_bytes": int(need),
    }), flush=True)


def bench_fast_f32(args):
    """Time the fast fp32 forward (fp32 in and out, products on the fp16
    MFMA) against the strict fp32 forward on an fp32 workload; each timing
    covers every launch of one call (the fast mode's operand conversion,
    the fp16 kernel and the output widening)."""
    import numpy as np
    import torch
    import deberta_disentangled_attention_amd as dd

    w = build_workload(args.workload)
    if w.dtype != "fp32" or w.packed:
        raise SystemExit("--fast-f32 needs a padded fp32 workload (c1, c5f32)")
    if args.flags is not None:
        w.flags = args.flags
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    q, k, v, qr, kr = dev(w.q), dev(w.k), dev(w.v), dev(w.qr), dev(w.kr)
    table = dd.rel_bucket(w.L, w.position_buckets, w.max_relative_positions, device="cuda")
    mask = None if w.mask is None else torch.from_numpy(w.mask).cuda()
    out = torch.empty((w.B, w.L, w.H * w.d), dtype=torch.float32, device="cuda")
    need = dd.f32fast_workspace_size(w.B * w.L, w.n_rel if w.flags else 0, w.H, w.d)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def fast():
        dd.dattn_fwd_padded_f32fast(q, k, v, qr, kr, table, w.L, mask, w.H, w.d, flags=w.flags,
                                    out=out, workspace=ws)

    def strict():
        dd.dattn_fwd_padded(q, k, v, qr, kr, table, w.L, mask, w.H, w.d, flags=w.flags, out=out)

    t_fast = _timed(fast, args.steps, args.warmup)
    t_strict = _timed(strict, args.steps, args.warmup)
    flop = w.effective_flop()
    print(json.dumps({
        "metric": "fast fp32 forward (fp16 MFMA) vs strict fp32 forward",
        "workload": describe(w), "flags": w.flags, "steps": args.steps, "warmup": args.warmup,
        "fast_ms": round(t_fast, 4), "strict_ms": round(t_strict, 4),
        "speedup": round(t_strict / t_fast, 2),
        "fast_TFLOPs": round(flop / (t_fast * 1e-3) / 1e12, 2),
        "fast_pct_fp16_mfma_peak": round(100 * flop / (t_fast * 1e-3) / 1e12 / PEAK_TFLOPS["fp16"], 2),
        "strict_TFLOPs": round(flop / (t_strict * 1e-3) / 1e12, 2),
        "strict_pct_fp32_mfma_peak": round(100 * flop / (t_strict * 1e-3) / 1e12 / PEAK_TFLOPS["fp32"], 2),
        "workspace_bytes": int(need),
    }), flush=True)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--write-traffic":
        write_traffic(*sys.argv[2:6])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--copy-probe":
        copy_probe()
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=16)
    ap.add_argument("--flags", type=int, default=None,
                    help="override the position terms (0 none, 1 C2P, 2 P2C, 3 both)")
    ap.add_argument("--pack", action="store_true",
                    help="padded forward vs the device-packed route on a padded workload")
    ap.add_argument("--relproj", action="store_true",
                    help="time the qr/kr projection of the workload's table shape")
    ap.add_argument("--fast-f32", action="store_true",
                    help="fast fp32 mode (fp16 MFMA) against strict fp32 on an fp32 workload")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward on the workload (forward output and lse computed once)")
    ap.add_argument("--flush-l2", action="store_true",
                    help="overwrite a 512 MiB buffer before every step (outside the kernel's "
                         "events) so inputs are not served from L2 / Infinity Cache")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import deberta_disentangled_attention_amd as dd
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dd.lib()
    if args.relproj:
        if args.workload == "c4":
            args.workload = "c2"
        bench_relproj(args)
        return
    if args.bwd:
        bench_bwd(args)
        return
    if args.fast_f32:
        if args.workload == "c4":
            args.workload = "c5f32"
        bench_fast_f32(args)
        return
    if args.pack:
        if args.workload == "c4":
            args.workload = "c3"
        bench_pack(args)
        return
    w = build_workload(args.workload)
    if args.flags is not None:
        w.flags = args.flags
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(tdt).cuda()
    q, k, v, qr, kr = dev(w.q), dev(w.k), dev(w.v), dev(w.qr), dev(w.kr)
    relmax = w.max_seqlen if w.packed else w.L
    table = torch.empty(2 * relmax - 1, dtype=torch.int32, device="cuda")
    if w.packed:
        cu = torch.from_numpy(w.cu_seqlens).cuda()
        out = torch.empty((w.total_tokens, w.H * w.d), dtype=tdt, device="cuda")
    else:
        mask = None if w.mask is None else torch.from_numpy(w.mask).cuda()
        out = torch.empty((w.B, w.L, w.H * w.d), dtype=tdt, device="cuda")
    torch.cuda.synchronize()
    base_mem = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()

    def fwd():
        if w.packed:
            dd.dattn_fwd_varlen(q, k, v, qr, kr, table, relmax, cu, w.max_seqlen, w.H, w.d,
                                flags=w.flags, out=out)
        else:
            dd.dattn_fwd_padded(q, k, v, qr, kr, table, relmax, mask, w.H, w.d,
                                flags=w.flags, out=out)

    flush_buf = (torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
                 if args.flush_l2 else None)

    def step(ev=None):
        if flush_buf is not None:
            flush_buf.fill_(1)
        dd.rel_bucket(relmax, w.position_buckets, w.max_relative_positions, out=table)
        if ev is not None:
            ev[0].record()
        fwd()
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(args.steps):
        step(events[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    kern_ms = [a.elapsed_time(b) for a, b in events]
    peak_extra = torch.cuda.max_memory_allocated() - base_mem
    if flush_buf is not None:
        peak_extra -= flush_buf.numel()
    srt = sorted(kern_ms)

    def pct(p):
        # nearest-rank percentile of the per-launch kernel times
        return srt[min(len(srt) - 1, max(0, int(math.ceil(p / 100.0 * len(srt))) - 1))]

    flop = w.effective_flop()
    ms_per_step = total_ms / args.steps
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (kern_avg_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = load_traffic() if (args.workload == "c4" and w.flags == 3) else None
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded numpy PCG64 inputs of the workload's shape; no dataset, no weights)",
        "config": {"workload": describe(w), "nseq": w.B, "seq_len": w.L, "heads": w.H,
                   "head_dim": w.d, "total_tokens": w.total_tokens,
                   "layout": "packed" if w.packed else "padded",
                   "position_buckets": w.position_buckets,
                   "max_relative_positions": w.max_relative_positions,
                   "flags": w.flags, "parallelism": "single GPU"},
        "tokens_per_s": round(w.total_tokens / (ms_per_step * 1e-3), 1),
        "pct_mfma_peak": round(100.0 * value / peak, 2),
        "effective_flop_per_step": flop,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "kernel": "dattn_fwd_kernel", "kernel_avg_ms": round(kern_avg_ms, 4),
                     "kernel_median_ms": round(pct(50), 4),
                     "kernel_p10_ms": round(pct(10), 4), "kernel_p90_ms": round(pct(90), 4),
                     "kernel_min_ms": round(min(kern_ms), 4),
                     "kernel_max_ms": round(max(kern_ms), 4),
                     "median_frac": round(flop / (pct(50) * 1e-3) / 1e12 / peak, 4),
                     "hbm_GBps_algorithmic": round(algorithmic_bytes(w) / (kern_avg_ms * 1e-3) / 1e9, 1),
                     "l2_flushed": bool(args.flush_l2)},
        "device_memory": {"peak_extra_bytes_during_steps": int(peak_extra),
                          "relative_table_bytes": int(table.numel() * 4)},
        "host_wall_s_timed_region": round(wall, 4),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_units)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
