"""GPU parity of the backward (dattn_bwd_padded / dattn_bwd_varlen) against
the float64 oracle (oracle.backward), and its determinism.

The forward is run on the GPU with its log-sum-exp (as in training); the
backward reads that output and lse. Bar: per gradient, max |got - want| <=
tol * max |want| (errors relative to the gradient's own scale) with tol =
1e-5 (fp32), 4e-3 (fp16), 2e-2 (bf16), about ten rounding units of the
element type (2^-11 for fp16, 2^-9 for bf16): the 16-bit paths round P and
dS to the element type before the MFMA products (as the forward rounds P),
store the dS of band pairs in the element type, and the forward's output
(for D_i = dout_i . out_i) is itself rounded; everything accumulates in
fp32. Measured worst cases on the small shapes: 1.3e-6, 9e-4, 5.9e-3.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads
from oracle import backward as BW
from tests import helpers as H

pytestmark = pytest.mark.gpu

BWD_TOL = {"fp32": 1e-5, "fp16": 4e-3, "bf16": 2e-2}
NAMES = ("dq", "dk", "dv", "dqr", "dkr")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _dout(w, seed):
    rng = np.random.default_rng(seed)
    shape = w.q.shape
    return workloads.round_to(rng.standard_normal(shape).astype(np.float32), w.dtype)


def _compare(got, want, dtype, tag, flags):
    errs = {}
    for name in NAMES:
        g, ww = got[name], want[name]
        if name in ("dqr", "dkr") and not flags:
            continue
        scale = max(float(np.abs(ww).max()), 1e-30)
        err = float(np.abs(g - ww).max()) / scale
        errs[name] = err
        assert np.all(np.isfinite(g)), f"{tag} {name}: non-finite"
        assert err <= BWD_TOL[dtype], f"{tag} {name}: rel err {err:.3e} > {BWD_TOL[dtype]:.1e}"
    return errs


def run_bwd_padded(w, flags, dout, band=None, rel_max_len=None):
    import torch
    import deberta_disentangled_attention_amd as dd
    rel_max_len = rel_max_len or w.L
    dt = w.dtype
    Tg = H.gpu_table(rel_max_len, w.position_buckets, w.max_relative_positions)
    mask = None if w.mask is None else torch.from_numpy(np.ascontiguousarray(w.mask, np.uint8)).cuda()
    q, k, v = H.dev(w.q, dt), H.dev(w.k, dt), H.dev(w.v, dt)
    qr, kr = H.dev(w.qr, dt), H.dev(w.kr, dt)
    out, lse = dd.dattn_fwd_padded(q, k, v, qr, kr, Tg, rel_max_len, mask, w.H, w.d, flags=flags,
                                   lse=True)
    if band is None:
        band = dd.rel_bucket_band(rel_max_len, w.position_buckets, w.max_relative_positions)
    g = dd.dattn_bwd_padded(q, k, v, out, H.dev(dout, dt), lse, qr, kr, Tg, rel_max_len, band, mask,
                            w.H, w.d, flags=flags)
    torch.cuda.synchronize()
    res = {}
    for name, t in zip(NAMES, g):
        res[name] = None if t is None else H.host(t)
    for name in ("dq", "dk", "dv"):
        res[name] = res[name].reshape(w.B, w.L, w.H * w.d)
    return res, g


def oracle_bwd_padded(w, flags, dout, rel_max_len=None):
    rel_max_len = rel_max_len or w.L
    T = oracle.rel_index_table(rel_max_len, w.position_buckets, w.max_relative_positions)
    return BW.dattn_padded_bwd(w.q, w.k, w.v, w.qr, w.kr, T, rel_max_len, w.mask, w.H, w.d,
                               dout, flags)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("flags", [3, 1, 2, 0])
def test_bwd_small_padded(dtype, d, flags):
    rng = np.random.default_rng(d + 7 * flags)
    for L, kind in ((37, "right"), (300, "random"), (200, "right")):
        lens = np.array([L, int(rng.integers(1, L + 1))])
        w = workloads.make_workload(f"bwd_{dtype}_{d}_{L}", dtype=dtype, B=2, L=L, H=2, d=d,
                                    position_buckets=16, max_relative_positions=64, lens=lens,
                                    seed=L + d + flags, flags=flags)
        if kind == "random":
            m = (rng.random((2, L)) < 0.75).astype(np.uint8)
            m[:, 0] = 1
            w.mask = m
        dout = _dout(w, L)
        _say(f"bwd padded {dtype} d={d} flags={flags} L={L} {kind}")
        got, _ = run_bwd_padded(w, flags, dout)
        want = oracle_bwd_padded(w, flags, dout)
        errs = _compare(got, want, dtype, f"{w.name} f{flags}", flags)
        _say("   " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def run_bwd_varlen(w, flags, dout, band=None, rel_max_len=None):
    import torch
    import deberta_disentangled_attention_amd as dd
    rel_max_len = rel_max_len or max(w.max_seqlen, 1)
    dt = w.dtype
    Tg = H.gpu_table(rel_max_len, w.position_buckets, w.max_relative_positions)
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    q, k, v = H.dev(w.q, dt), H.dev(w.k, dt), H.dev(w.v, dt)
    qr, kr = H.dev(w.qr, dt), H.dev(w.kr, dt)
    out, lse = dd.dattn_fwd_varlen(q, k, v, qr, kr, Tg, rel_max_len, cu, w.max_seqlen, w.H, w.d,
                                   flags=flags, lse=True)
    if band is None:
        band = dd.rel_bucket_band(rel_max_len, w.position_buckets, w.max_relative_positions)
    g = dd.dattn_bwd_varlen(q, k, v, out, H.dev(dout, dt), lse, qr, kr, Tg, rel_max_len, band, cu,
                            w.max_seqlen, w.H, w.d, flags=flags)
    torch.cuda.synchronize()
    return {name: (None if t is None else H.host(t)) for name, t in zip(NAMES, g)}, g


def oracle_bwd_varlen(w, flags, dout, rel_max_len=None):
    rel_max_len = rel_max_len or max(w.max_seqlen, 1)
    T = oracle.rel_index_table(rel_max_len, w.position_buckets, w.max_relative_positions)
    return BW.dattn_varlen_bwd(w.q, w.k, w.v, w.qr, w.kr, T, rel_max_len, w.cu_seqlens, w.H, w.d,
                               dout, flags)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("flags", [3, 0])
def test_bwd_varlen(dtype, flags):
    lens = np.array([1, 130, 0, 700, 64, 255])
    w = workloads.make_workload(f"bwd_varlen_{dtype}", dtype=dtype, B=len(lens), L=700, H=2, d=64,
                                position_buckets=16, max_relative_positions=64, lens=lens,
                                seed=11, packed=True, flags=flags)
    dout = _dout(w, 3)
    _say(f"bwd varlen {dtype} flags={flags}")
    got, _ = run_bwd_varlen(w, flags, dout)
    want = oracle_bwd_varlen(w, flags, dout)
    errs = _compare(got, want, dtype, f"varlen {dtype}", flags)
    _say("   " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bwd_band_bounds(dtype):
    """The largest band (rel_max_len: no distance assumed saturated) and
    rel_max_len > L give the oracle's gradients too."""
    w = workloads.make_workload("bwd_band", dtype=dtype, B=2, L=333, H=2, d=64,
                                position_buckets=32, max_relative_positions=96,
                                lens=np.array([333, 201]), seed=5)
    dout = _dout(w, 9)
    want = oracle_bwd_padded(w, 3, dout, rel_max_len=500)
    for band in (None, 500):
        got, _ = run_bwd_padded(w, 3, dout, band=band, rel_max_len=500)
        errs = _compare(got, want, dtype, f"band {band}", 3)
        _say(f"bwd {dtype} band={band}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_bwd_c2_shape_and_determinism():
    """The v3-base shape (16 x 512 bf16, H=12, lengths 256..512, projected
    tables) against the oracle; a second call is bit-identical."""
    import torch
    w = workloads.c2_v3base_bf16()
    dout = _dout(w, 21)
    got, g1 = run_bwd_padded(w, 3, dout)
    want = oracle_bwd_padded(w, 3, dout)
    errs = _compare(got, want, "bf16", "c2", 3)
    _say("c2 bwd: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    _, g2 = run_bwd_padded(w, 3, dout)
    for name, a, b in zip(NAMES, g1, g2):
        assert torch.equal(a, b), f"{name} differs between two calls"


@pytest.mark.parametrize("layout", ["padded", "varlen"])
def test_bwd_workspace_prefilled_with_nan(layout):
    """The backward clears nothing globally: every workspace cell it reads is
    written first in the same call. A workspace full of NaN bytes must give
    the oracle's gradients (a read of an unwritten cell would spread NaN)."""
    import torch
    import deberta_disentangled_attention_amd as dd
    dt = "bf16"
    if layout == "padded":
        w = workloads.make_workload("nanws_p", dtype=dt, B=3, L=300, H=2, d=64, position_buckets=16,
                                    max_relative_positions=64, lens=np.array([300, 123, 7]), seed=21)
        rng = np.random.default_rng(5)
        m = (rng.random((3, 300)) < 0.8).astype(np.uint8)
        m[:, 0] = 1
        m[1, 123:] = 0
        m[2, 7:] = 0
        w.mask = m
    else:
        w = workloads.make_workload("nanws_v", dtype=dt, B=5, L=333, H=2, d=64, position_buckets=16,
                                    max_relative_positions=64, lens=np.array([5, 333, 0, 61, 200]),
                                    seed=22, packed=True)
    dout = _dout(w, 9)
    rel = w.L if layout == "padded" else w.max_seqlen
    band = dd.rel_bucket_band(rel, w.position_buckets, w.max_relative_positions)
    rows = w.B * w.L if layout == "padded" else w.total_tokens
    need = dd.bwd_workspace_size(rows, w.B, w.H, w.d, torch.bfloat16, band)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN in every format
    Tg = H.gpu_table(rel, w.position_buckets, w.max_relative_positions)
    q, k, v = H.dev(w.q, dt), H.dev(w.k, dt), H.dev(w.v, dt)
    qr, kr = H.dev(w.qr, dt), H.dev(w.kr, dt)
    if layout == "padded":
        mask = torch.from_numpy(np.ascontiguousarray(w.mask, np.uint8)).cuda()
        out, lse = dd.dattn_fwd_padded(q, k, v, qr, kr, Tg, rel, mask, w.H, w.d, lse=True)
        g = dd.dattn_bwd_padded(q, k, v, out, H.dev(dout, dt), lse, qr, kr, Tg, rel, band, mask,
                                w.H, w.d, workspace=ws)
        want = oracle_bwd_padded(w, 3, dout)
    else:
        cu = torch.from_numpy(w.cu_seqlens).cuda()
        out, lse = dd.dattn_fwd_varlen(q, k, v, qr, kr, Tg, rel, cu, w.max_seqlen, w.H, w.d, lse=True)
        g = dd.dattn_bwd_varlen(q, k, v, out, H.dev(dout, dt), lse, qr, kr, Tg, rel, band, cu,
                                w.max_seqlen, w.H, w.d, workspace=ws)
        want = oracle_bwd_varlen(w, 3, dout)
    torch.cuda.synchronize()
    got = {name: H.host(t) for name, t in zip(NAMES, g)}
    if layout == "padded":
        for name in ("dq", "dk", "dv"):
            got[name] = got[name].reshape(w.B, w.L, w.H * w.d)
    errs = _compare(got, want, dt, f"nan workspace {layout}", 3)
    _say(f"nan-prefilled workspace {layout}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_bwd_long_sequences_real_buckets(dtype):
    """DeBERTa's 256/512 buckets (band 512) on sequences long enough that
    every block range occurs: workgroups whose keys lie all beyond the band
    below, band blocks, all beyond above; packed with an odd offset."""
    lens = np.array([1500, 2100, 3])
    w = workloads.make_workload(f"bwd_long_{dtype}", dtype=dtype, B=len(lens), L=2100, H=2, d=64,
                                position_buckets=256, max_relative_positions=512, lens=lens,
                                seed=31, packed=True, qkv_scale=0.125)
    dout = _dout(w, 13)
    _say(f"bwd long sequences {dtype}")
    got, _ = run_bwd_varlen(w, 3, dout)
    want = oracle_bwd_varlen(w, 3, dout)
    errs = _compare(got, want, dtype, f"long {dtype}", 3)
    _say("   " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bwd_masked_rows_and_single_tokens(dtype):
    """A fully masked batch row (log-sum-exp -inf: zero gradients), a row
    whose only valid token is the last one, and a one-token packed
    sequence next to an empty one."""
    w = workloads.make_workload(f"bwd_edge_{dtype}", dtype=dtype, B=3, L=65, H=2, d=32,
                                position_buckets=16, max_relative_positions=64,
                                lens=np.array([65, 65, 65]), seed=3)
    m = np.ones((3, 65), np.uint8)
    m[1, :] = 0
    m[2, :64] = 0
    w.mask = m
    dout = _dout(w, 4)
    got, _ = run_bwd_padded(w, 3, dout)
    want = oracle_bwd_padded(w, 3, dout)
    errs = _compare(got, want, dtype, f"edge padded {dtype}", 3)
    for name in ("dq", "dk", "dv"):
        assert np.all(got[name][1] == 0.0), f"{name}: fully masked row not zero"
        assert np.all(got[name][2][:64] == 0.0), f"{name}: masked positions not zero"
    wv = workloads.make_workload(f"bwd_edge_v_{dtype}", dtype=dtype, B=3, L=40, H=2, d=32,
                                 position_buckets=16, max_relative_positions=64,
                                 lens=np.array([1, 0, 40]), seed=5, packed=True)
    dv_ = _dout(wv, 6)
    gotv, _ = run_bwd_varlen(wv, 3, dv_)
    wantv = oracle_bwd_varlen(wv, 3, dv_)
    errs.update({k + "_v": v for k, v in _compare(gotv, wantv, dtype, f"edge varlen {dtype}", 3).items()})
    _say(f"bwd edges {dtype}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
