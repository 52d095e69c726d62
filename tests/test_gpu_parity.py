"""GPU parity: the HIP path against the float64 oracle, element by element.

Bars: relative-row tables bit-exact; outputs within max-abs 1e-5 (fp32),
5e-3 (fp16), 1.5e-2 (bf16) on valid rows; padded rows exactly zero.
Small shapes span several 128-query x 64-key tiles plus ragged tails; the
five named configurations are checked in full where the oracle is fast and
on sampled rows (computed one by one by the oracle) where it is not.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads
from tests import dense
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# relative-row table
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("max_len,P,M", [
    (128, 0, 64), (512, 256, 512), (8192, 256, 512), (1, 256, 512), (100, 8, 20),
    (300, 16, 64), (4096, 64, 300), (2000, 2, 9), (777, 0, 5), (3000, 4, 7),
    (1500, 32, 129), (6000, 512, 1024),
])
def test_rel_bucket_bit_exact(max_len, P, M):
    _say(f"rel_bucket max_len={max_len} P={P} M={M}")
    got = H.gpu_table(max_len, P, M).cpu().numpy()
    want = oracle.rel_index_table(max_len, P, M)
    assert got.dtype == np.int32
    assert np.array_equal(got.astype(np.int64), want)


# bucket parameters: even and odd P, M just above P/2 to 2^31-1 (arguments that
# come within 1e-10 of an integer without reaching it at P=16 and P=32 with
# M = 2^31-1, exact integer arguments at P=32, M=129 and P=4, M=7)
SWEEP = [(P, M) for P in (2, 3, 4, 5, 8, 9, 16, 17, 32, 64, 100, 256, 257, 512)
         for M in sorted({P // 2 + 2, P, P + 1, 2 * P + 7, 129, 512, 1000, 65535, 2 ** 31 - 1})
         if M - 1 > P // 2]


LONG = [(16, 2 ** 31 - 1), (32, 2 ** 31 - 1), (32, 129), (4, 7), (256, 512), (512, 2 ** 31 - 1),
        (1024, 4096), (4096, 70000)]


def test_rel_bucket_sweep_bit_exact():
    """Every (P, M) of SWEEP at max_len 600, and the LONG sets (which hold
    the near-integer and exact-integer distances) at max_len 9000."""
    n = 0
    for max_len, sets in ((600, SWEEP), (9000, LONG)):
        for P, M in sets:
            got = H.gpu_table(max_len, P, M).cpu().numpy().astype(np.int64)
            want = oracle.rel_index_table(max_len, P, M)
            assert np.array_equal(got, want), (max_len, P, M, np.nonzero(got != want)[0][:5])
            n += 1
    _say(f"rel_bucket sweep: {n} (max_len, P, M) sets bit-exact")


# ---------------------------------------------------------------------------
# small shapes: every dtype, head dim, flag set and layout
# ---------------------------------------------------------------------------

def small_case(dtype, d, L, B=2, Hh=2, P=16, M=64, seed=0, mask_kind="right"):
    rng = np.random.default_rng(seed)
    if mask_kind == "right":
        lens = np.array([L] + list(rng.integers(1, L + 1, size=B - 1)))
    else:
        lens = np.full(B, L)
    w = workloads.make_workload(f"small_{dtype}_{d}_{L}", dtype=dtype, B=B, L=L, H=Hh, d=d,
                                position_buckets=P, max_relative_positions=M, lens=lens,
                                seed=seed)
    if mask_kind == "random":
        m = (rng.random((B, L)) < 0.75).astype(np.uint8)
        m[:, 0] = 1
        w.mask = m
    elif mask_kind == "none":
        w.mask = None
    return w


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("flags", [3, 1, 2, 0])
def test_small_padded(dtype, d, flags):
    for L, kind in ((37, "right"), (300, "random"), (700, "right")):
        w = small_case(dtype, d, L, seed=L + d + flags, mask_kind=kind)
        _say(f"padded {dtype} d={d} flags={flags} L={L} mask={kind}")
        got = H.host(H.run_padded(w, flags=flags))
        want = H.oracle_padded(w, flags=flags)
        H.assert_padded_close(got, want, H.valid_rows_padded(w), dtype, f"{w.name} f{flags}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_small_varlen(dtype, d):
    lens = np.array([1, 130, 0, 700, 64, 255])
    w = workloads.make_workload(f"varlen_{dtype}_{d}", dtype=dtype, B=len(lens), L=700, H=2,
                                d=d, position_buckets=16, max_relative_positions=64,
                                lens=lens, seed=d, packed=True)
    _say(f"varlen {dtype} d={d}")
    got = H.host(H.run_varlen(w))
    want = H.oracle_varlen(w)
    assert np.all(np.isfinite(got))
    err = float(np.abs(got - want).max())
    assert err <= H.TOL[dtype], err


def test_identity_bucket_and_explicit_scale():
    w = workloads.make_workload("ident", dtype="fp32", B=2, L=333, H=3, d=64,
                                position_buckets=0, max_relative_positions=40, seed=5,
                                lens=np.array([333, 200]))
    got = H.host(H.run_padded(w, scale=0.05))
    want = H.oracle_padded(w, scale=0.05)
    H.assert_padded_close(got, want, H.valid_rows_padded(w), "fp32", "ident")


def test_rel_max_len_larger_than_L():
    w = small_case("bf16", 64, 200, seed=9)
    got = H.host(H.run_padded(w, rel_max_len=1000))
    want = H.oracle_padded(w, rel_max_len=1000)
    H.assert_padded_close(got, want, H.valid_rows_padded(w), "bf16", "relmax")


# ---------------------------------------------------------------------------
# the named configurations
# ---------------------------------------------------------------------------

def test_c1_tiny_fp32():
    w = workloads.c1_tiny_fp32()
    got = H.host(H.run_padded(w))
    want = H.oracle_padded(w)
    worst = H.assert_padded_close(got, want, H.valid_rows_padded(w), "fp32", "c1")
    _say(f"c1 max abs err {worst:.3e}")


def test_c2_v3base_bf16():
    w = workloads.c2_v3base_bf16()
    got = H.host(H.run_padded(w))
    want = H.oracle_padded(w)
    worst = H.assert_padded_close(got, want, H.valid_rows_padded(w), "bf16", "c2")
    _say(f"c2 max abs err {worst:.3e}")


def test_c3_padded_and_packed():
    w = workloads.c3_v2xlarge_fp16()
    wp = workloads.c3_v2xlarge_fp16(packed=True)
    got = H.host(H.run_padded(w))
    want = H.oracle_padded(w)
    worst = H.assert_padded_close(got, want, H.valid_rows_padded(w), "fp16", "c3")
    gotp = H.host(H.run_varlen(wp, rel_max_len=w.L))
    wantp = H.oracle_varlen(wp, rel_max_len=w.L)
    errp = float(np.abs(gotp - wantp).max())
    assert errp <= H.TOL["fp16"]
    # packed equals padded on the valid rows (same kernel arithmetic)
    assert np.array_equal(gotp, workloads.pack(got, w.lens))
    _say(f"c3 max abs err padded {worst:.3e} packed {errp:.3e}")


def _dense_compare(jobs, got_fn, tol, tag):
    """Run the oracle jobs and compare each with the GPU rows got_fn(b, h,
    rows); returns the worst error and the number of rows checked."""
    worst, nrows = 0.0, 0
    for (b, h), rows, want in dense.run_jobs(jobs):
        got = got_fn(b, h, rows)
        assert np.all(np.isfinite(got)), f"{tag}: non-finite output in unit {(b, h)}"
        err = float(np.abs(got - want).max())
        assert err <= tol, f"{tag}: unit {(b, h)} max abs err {err:.3e} > {tol:.1e}"
        worst = max(worst, err)
        nrows += len(rows)
    return worst, nrows


def test_c4_long_packed_dense():
    """The benchmark workload (16 x 8192 packed bf16, H=12) in the launch
    configuration the benchmark times: covering rows of every (sequence,
    head) unit -- every 128-query workgroup and every wave -- and two whole
    units."""
    w = workloads.c4_long_packed_bf16()
    out = H.host(H.run_varlen(w))
    assert np.all(np.isfinite(out))
    T = oracle.rel_index_table(w.max_seqlen, w.position_buckets, w.max_relative_positions)
    cu = w.cu_seqlens
    units = [(b, h) for b in range(w.B) for h in range(w.H)]
    jobs = dense.unit_jobs("out", w, T, w.max_seqlen, units, full_units=[(0, 0), (15, 11)],
                           seed=4)
    worst, nrows = _dense_compare(
        jobs, lambda b, h, rows: out[int(cu[b]) + rows, h * w.d:(h + 1) * w.d],
        H.TOL[w.dtype], "c4")
    _say(f"c4 dense: {len(units)} units, {nrows} rows checked, max abs err {worst:.3e}")


@pytest.mark.parametrize("d,dtype", [(32, "bf16"), (128, "bf16"), (128, "fp32")])
@pytest.mark.parametrize("flags", [3, 0])
def test_c5_sweep_dense(d, dtype, flags):
    """Covering rows of every unit and one whole unit; the strict fp32
    L=1024 case in full."""
    w = workloads.c5_sweep(d, dtype, flags)
    out = H.host(H.run_padded(w))
    assert np.all(np.isfinite(out))
    T = oracle.rel_index_table(w.L, w.position_buckets, w.max_relative_positions)
    units = [(b, h) for b in range(w.B) for h in range(w.H)]
    full = units if dtype == "fp32" else [(1, 7)]
    jobs = dense.unit_jobs("out", w, T, w.L, units, full_units=full, seed=5)
    worst, nrows = _dense_compare(
        jobs, lambda b, h, rows: out[b, rows, h * w.d:(h + 1) * w.d], H.TOL[w.dtype],
        f"c5 d={d} {dtype} f{flags}")
    _say(f"c5 d={d} {dtype} flags={flags}: {nrows} rows checked, max abs err {worst:.3e}")
