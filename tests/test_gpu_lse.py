"""GPU parity of the forwards' row log-sum-exp (dattn_fwd_*_lse) against the
oracle (oracle.backward.lse_rows).

Bar, absolute: 1e-5 (fp32), 5e-3 (fp16), 1e-2 (bf16). lse is the log of the
row sum of exponentials, so a change of every score by at most e moves it by
at most e. The scores carry the products of inputs in the element type
accumulated in fp32 and, on far tiles, the operand
(q_i + qr[row]) * scale * log2(e) rounded once (relative 2^-9 bf16, 2^-11
fp16). For the 16-bit types the row sum is
taken from the exponentials after they are rounded to the element type (the
same P the P.V product reads), each term off by at most that relative
amount, which moves the log of the sum by at most 2^-9 (bf16) or 2^-11
(fp16). Rows without a valid key must be -inf, and the output must be
bit-identical to the forward without lse.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads
from oracle import backward as BW
from tests import dense
from tests import helpers as H

pytestmark = pytest.mark.gpu

LSE_TOL = {"fp32": 1e-5, "fp16": 5e-3, "bf16": 1e-2}


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check(got, want, dtype, tag):
    assert np.array_equal(np.isneginf(got), np.isneginf(want)), f"{tag}: -inf rows differ"
    fin = np.isfinite(want)
    err = float(np.abs(got[fin] - want[fin]).max()) if fin.any() else 0.0
    assert err <= LSE_TOL[dtype], f"{tag}: lse err {err:.3e}"
    return err


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("flags", [3, 0])
def test_lse_padded(dtype, d, flags):
    import torch
    import deberta_disentangled_attention_amd as dd
    rng = np.random.default_rng(d + flags)
    for L, kind in ((300, "random"), (700, "right")):
        lens = np.array([L, int(rng.integers(1, L))])
        w = workloads.make_workload(f"lse_{dtype}_{d}_{L}", dtype=dtype, B=2, L=L, H=2, d=d,
                                    position_buckets=16, max_relative_positions=64, lens=lens,
                                    seed=L + d, flags=flags)
        if kind == "random":
            m = (rng.random((2, L)) < 0.7).astype(np.uint8)
            m[0, :3] = 0
            w.mask = m
        _say(f"lse padded {dtype} d={d} flags={flags} L={L} {kind}")
        out0 = H.run_padded(w)
        T = H.gpu_table(w.L, w.position_buckets, w.max_relative_positions)
        mask = torch.from_numpy(np.ascontiguousarray(w.mask, np.uint8)).cuda()
        out, lse = dd.dattn_fwd_padded(H.dev(w.q, dtype), H.dev(w.k, dtype), H.dev(w.v, dtype),
                                       H.dev(w.qr, dtype), H.dev(w.kr, dtype), T, w.L, mask,
                                       w.H, w.d, flags=flags, lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out, out0)
        got = lse.cpu().numpy().reshape(w.B, w.L, w.H).astype(np.float64)
        Tn = np.asarray(T.cpu().numpy(), dtype=np.int64)
        for b in range(w.B):
            for h in range(w.H):
                want = BW.lse_rows(w.q[b], w.k[b], w.qr, w.kr, Tn, w.L, h, d, np.arange(L),
                                   valid=w.mask[b], flags=flags)
                _check(got[b, :, h], want, dtype, f"b={b} h={h}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_lse_varlen(dtype):
    import torch
    import deberta_disentangled_attention_amd as dd
    lens = np.array([1, 130, 0, 700, 64, 255])
    w = workloads.make_workload(f"lse_varlen_{dtype}", dtype=dtype, B=len(lens), L=700, H=2,
                                d=64, position_buckets=16, max_relative_positions=64,
                                lens=lens, seed=7, packed=True)
    _say(f"lse varlen {dtype}")
    T = H.gpu_table(w.max_seqlen, w.position_buckets, w.max_relative_positions)
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    args = (H.dev(w.q, dtype), H.dev(w.k, dtype), H.dev(w.v, dtype), H.dev(w.qr, dtype),
            H.dev(w.kr, dtype), T, w.max_seqlen, cu, w.max_seqlen, w.H, w.d)
    out0 = dd.dattn_fwd_varlen(*args)
    out, lse = dd.dattn_fwd_varlen(*args, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out0)
    got = lse.cpu().numpy().astype(np.float64)
    Tn = np.asarray(T.cpu().numpy(), dtype=np.int64)
    cuh = w.cu_seqlens
    for b in range(len(lens)):
        lo, hi = int(cuh[b]), int(cuh[b + 1])
        if hi == lo:
            continue
        for h in range(w.H):
            want = BW.lse_rows(w.q[lo:hi], w.k[lo:hi], w.qr, w.kr, Tn, w.max_seqlen, h, 64,
                               np.arange(hi - lo))
            _check(got[lo:hi, h], want, dtype, f"seq {b} h={h}")


def test_lse_long_packed_dense():
    """The benchmark workload (16 x 8192 packed bf16) in its launch
    configuration: covering rows of every (sequence, head) unit (every
    workgroup and wave) and one whole unit."""
    w = workloads.c4_long_packed_bf16()
    out0 = H.run_varlen(w)
    out, lse = H.run_varlen(w, lse=True)
    import torch
    assert torch.equal(out, out0)
    got = lse.cpu().numpy().astype(np.float64)
    T = oracle.rel_index_table(w.max_seqlen, w.position_buckets, w.max_relative_positions)
    cu = w.cu_seqlens
    units = [(b, h) for b in range(w.B) for h in range(w.H)]
    jobs = dense.unit_jobs("lse", w, T, w.max_seqlen, units, full_units=[(7, 3)], seed=6)
    worst, nrows = 0.0, 0
    for (b, h), rows, want in dense.run_jobs(jobs):
        worst = max(worst, _check(got[int(cu[b]) + rows, h], want, w.dtype, f"c4 seq {b} h={h}"))
        nrows += len(rows)
    _say(f"c4 dense lse: {nrows} rows checked, max err {worst:.3e}")
