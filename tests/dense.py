"""Dense oracle checks of large GPU outputs.

At the benchmark sizes the float64 oracle cannot compute every output row
of every (sequence, head) unit in a test's time, so the large-shape parity
tests check, for EVERY unit:
  * one row drawn at random from every 32-query group (one wave's queries),
  * the first and last row of every 128-query tile (one workgroup),
and a few whole units in full. A wrong workgroup mapping, tile slot or ring
slot therefore shows up wherever it lands. The oracle runs in worker
processes (numpy only, one BLAS thread each); they never touch the GPU.
"""

from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

GROUP = 32     # queries of one wave
TILE = 128     # queries of one workgroup
CHUNK = 1024   # rows per oracle call when a unit is checked in full


def covering_rows(n: int, rng: np.random.Generator, group: int = GROUP,
                  tile: int = TILE) -> np.ndarray:
    """Sorted rows of an n-row sequence: one random row per `group` rows and
    the first and last row of every `tile` rows."""
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    g0 = np.arange(0, n, group)
    r = np.minimum(g0 + rng.integers(0, group, size=len(g0)), n - 1)
    t0 = np.arange(0, n, tile)
    return np.unique(np.concatenate([r, t0, np.minimum(t0 + tile - 1, n - 1)])).astype(np.int64)


def _job(args):
    """One oracle call on one unit's single-head slices (runs in a worker)."""
    from threadpoolctl import threadpool_limits
    import oracle
    from oracle import backward as BW
    kind, key, qh, kh, vh, qrh, krh, T, relmax, rows, valid, flags, scale = args
    d = qh.shape[1]
    with threadpool_limits(limits=1):
        if kind == "out":
            val = oracle.dattn_rows(qh, kh, vh, qrh, krh, T, relmax, 0, d, rows, valid=valid,
                                    flags=flags, scale=scale)
        else:
            val = BW.lse_rows(qh, kh, qrh, krh, T, relmax, 0, d, rows, valid=valid,
                              flags=flags, scale=scale)
    return key, rows, val


def unit_jobs(kind: str, w, T: np.ndarray, relmax: int, units: Iterable[Tuple[int, int]],
              full_units: Sequence[Tuple[int, int]] = (), seed: int = 0,
              flags: Optional[int] = None, scale: float = 0.0) -> list:
    """Oracle jobs ('out' or 'lse') for the given (sequence, head) units of a
    workload: covering rows of each unit, and every row of `full_units`
    (in chunks). Packed workloads index sequences through cu_seqlens."""
    flags = w.flags if flags is None else flags
    d = w.d
    cu = w.cu_seqlens
    jobs = []
    full = set(full_units)
    for (b, h) in units:
        n = int(w.lens[b])
        if n == 0:
            continue
        if w.packed:
            sl = slice(int(cu[b]), int(cu[b + 1]))
            qs, ks, vs = w.q[sl], w.k[sl], w.v[sl]
            valid = None
        else:
            qs, ks, vs = w.q[b, :n], w.k[b, :n], w.v[b, :n]
            valid = None if w.mask is None else w.mask[b, :n]
            if w.mask is not None and not np.all(w.mask[b, n:] == 0):
                raise ValueError("dense checks take right-padded masks")
        col = slice(h * d, (h + 1) * d)
        arrs = [np.ascontiguousarray(x[:, col]) for x in (qs, ks, vs, w.qr, w.kr)]
        if (b, h) in full:
            row_sets = [np.arange(s, min(s + CHUNK, n), dtype=np.int64) for s in range(0, n, CHUNK)]
        else:
            rng = np.random.default_rng([seed, b, h])
            row_sets = [covering_rows(n, rng)]
        for rows in row_sets:
            jobs.append((kind, (b, h), *arrs, T, relmax, rows, valid, flags, scale))
    return jobs


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_jobs(jobs: list) -> List[tuple]:
    """Run oracle jobs in spawned worker processes; results in job order."""
    if not jobs:
        return []
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=workers(), mp_context=ctx) as ex:
        return list(ex.map(_job, jobs, chunksize=1))
