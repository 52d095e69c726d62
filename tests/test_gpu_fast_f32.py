"""GPU parity of the fast fp32 forward (dattn_fwd_padded_f32fast /
dattn_fwd_varlen_f32fast) against the float64 oracle on the unrounded fp32
inputs.

The mode rounds every operand once to fp16 (TF32's 10-bit mantissa) and
runs the fp16 forward, so its bar is the fp16 forward's: max abs error
5e-3 on N(0,1) inputs. The oracle sees the fp32 values, so the operand
rounding itself (2^-12 relative per element) is part of the measured error.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads
from tests import dense
from tests import helpers as H

pytestmark = pytest.mark.gpu

FAST_TOL = H.TOL["fp16"]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _dev32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def run_fast_padded(w, flags=None):
    import torch
    import deberta_disentangled_attention_amd as dd
    flags = w.flags if flags is None else flags
    T = H.gpu_table(w.L, w.position_buckets, w.max_relative_positions)
    mask = None if w.mask is None else torch.from_numpy(np.ascontiguousarray(w.mask, np.uint8)).cuda()
    out = dd.dattn_fwd_padded_f32fast(_dev32(w.q), _dev32(w.k), _dev32(w.v), _dev32(w.qr),
                                      _dev32(w.kr), T, w.L, mask, w.H, w.d, flags=flags)
    torch.cuda.synchronize()
    return H.host(out)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("flags", [3, 0])
def test_fast_f32_small_padded(d, flags):
    rng = np.random.default_rng(d + flags)
    for L, kind in ((37, "right"), (300, "random"), (700, "right")):
        lens = np.array([L, int(rng.integers(1, L + 1))])
        w = workloads.make_workload(f"fast_{d}_{L}", dtype="fp32", B=2, L=L, H=2, d=d,
                                    position_buckets=16, max_relative_positions=64, lens=lens,
                                    seed=L + d, flags=flags)
        if kind == "random":
            m = (rng.random((2, L)) < 0.75).astype(np.uint8)
            m[:, 0] = 1
            w.mask = m
        got = run_fast_padded(w)
        want = H.oracle_padded(w)
        valid = H.valid_rows_padded(w)
        err = float(np.abs(got[valid] - want[valid]).max())
        _say(f"fast f32 padded d={d} flags={flags} L={L} {kind}: {err:.2e}")
        assert np.all(np.isfinite(got))
        assert err <= FAST_TOL, err
        assert np.all(got[~valid] == 0.0)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_fast_f32_varlen(d):
    import torch
    import deberta_disentangled_attention_amd as dd
    lens = np.array([1, 130, 0, 700, 64, 255])
    w = workloads.make_workload(f"fastv_{d}", dtype="fp32", B=len(lens), L=700, H=2, d=d,
                                position_buckets=16, max_relative_positions=64, lens=lens,
                                seed=d, packed=True)
    T = H.gpu_table(w.max_seqlen, w.position_buckets, w.max_relative_positions)
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    got = H.host(dd.dattn_fwd_varlen_f32fast(_dev32(w.q), _dev32(w.k), _dev32(w.v), _dev32(w.qr),
                                             _dev32(w.kr), T, w.max_seqlen, cu, w.max_seqlen, w.H,
                                             w.d, flags=w.flags))
    want = H.oracle_varlen(w)
    err = float(np.abs(got - want).max())
    _say(f"fast f32 varlen d={d}: {err:.2e}")
    assert np.all(np.isfinite(got)) and err <= FAST_TOL, err


@pytest.mark.parametrize("flags", [3, 0])
def test_fast_f32_c5_shape_dense(flags):
    """The strict-fp32 sweep shape (4 x 1024, H=16, d=128) in the fast mode:
    covering rows of every unit and one whole unit."""
    w = workloads.c5_sweep(128, "fp32", flags)
    out = run_fast_padded(w)
    assert np.all(np.isfinite(out))
    T = oracle.rel_index_table(w.L, w.position_buckets, w.max_relative_positions)
    units = [(b, h) for b in range(w.B) for h in range(w.H)]
    jobs = dense.unit_jobs("out", w, T, w.L, units, full_units=[(2, 5)], seed=6)
    worst, nrows = 0.0, 0
    for (b, h), rows, want in dense.run_jobs(jobs):
        got = out[b, rows, h * w.d:(h + 1) * w.d]
        err = float(np.abs(got - want).max())
        assert err <= FAST_TOL, f"unit {(b, h)}: {err:.3e}"
        worst, nrows = max(worst, err), nrows + len(rows)
    _say(f"fast f32 c5 flags={flags}: {nrows} rows, max abs err {worst:.3e}")


def test_fast_f32_without_tables():
    """flags = 0: no tables at all (NULL qr, kr, rel_idx); textbook attention."""
    import torch
    import deberta_disentangled_attention_amd as dd
    w = workloads.make_workload("fast_plain", dtype="fp32", B=1, L=77, H=3, d=64,
                                position_buckets=16, max_relative_positions=64,
                                lens=np.array([77]), seed=9, flags=0)
    got = H.host(dd.dattn_fwd_padded_f32fast(_dev32(w.q), _dev32(w.k), _dev32(w.v), None, None,
                                             None, 77, None, w.H, w.d, flags=0))
    want = H.oracle_padded(w, flags=0)
    assert float(np.abs(got - want).max()) <= FAST_TOL
