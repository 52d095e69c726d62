"""GPU edge cases of the forward: determinism, poisoned padding and masked
keys, degenerate shapes, strided (fused QKV) inputs, complete output writes,
non-default streams and the O(L) device-memory property."""

import sys

import numpy as np
import pytest

import oracle
import workloads
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _small(dtype="bf16", B=3, L=333, Hh=2, d=64, lens=None, seed=0, P=16, M=64):
    lens = np.array([L, 150, 17][:B]) if lens is None else np.asarray(lens)
    return workloads.make_workload("edge", dtype=dtype, B=B, L=L, H=Hh, d=d,
                                   position_buckets=P, max_relative_positions=M,
                                   lens=lens, seed=seed)


def test_deterministic_bitwise():
    w = workloads.c2_v3base_bf16()
    a = H.host(H.run_padded(w))
    b = H.host(H.run_padded(w))
    assert np.array_equal(a, b)
    wp = workloads.c3_v2xlarge_fp16(packed=True)
    a = H.host(H.run_varlen(wp, rel_max_len=512))
    b = H.host(H.run_varlen(wp, rel_max_len=512))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_poisoned_padding_rows(dtype):
    """NaN in every padded position of Q, K and V leaves valid rows
    bit-identical and padded rows zero."""
    w = _small(dtype)
    clean = H.host(H.run_padded(w))
    valid = H.valid_rows_padded(w)
    for name in ("q", "k", "v"):
        x = getattr(w, name).copy()
        x[~valid] = np.nan
        setattr(w, name, x)
    dirty = H.host(H.run_padded(w))
    assert np.array_equal(clean[valid], dirty[valid])
    assert np.all(dirty[~valid] == 0.0)


@pytest.mark.parametrize("poison", [1e4, np.nan])
def test_poisoned_masked_keys_inside_extent(poison):
    """A non-prefix mask: masked keys inside the extent hold huge or NaN K/V
    values; valid outputs must not change and must match the oracle."""
    w = _small("fp16", seed=3)
    rng = np.random.default_rng(5)
    m = (rng.random((w.B, w.L)) < 0.6).astype(np.uint8)
    m[:, 0] = 1
    m[0, w.L - 1] = 1        # extent reaches the end in batch row 0
    w.mask = m
    clean = H.host(H.run_padded(w))
    want = H.oracle_padded(w)
    H.assert_padded_close(clean, want, m.astype(bool), "fp16", "masked")
    bad = ~m.astype(bool)
    for name in ("k", "v"):
        x = getattr(w, name).copy()
        x[bad] = poison
        setattr(w, name, x)
    dirty = H.host(H.run_padded(w))
    assert np.array_equal(clean[m.astype(bool)], dirty[m.astype(bool)])


def test_fully_masked_batch_row_and_length_one():
    w = _small("bf16", B=3, L=200, lens=[200, 0, 1])
    w.mask = workloads.right_pad_mask(w.lens, w.L)
    got = H.host(H.run_padded(w))
    want = H.oracle_padded(w)
    H.assert_padded_close(got, want, w.mask.astype(bool), "bf16", "fullmask")
    assert np.all(got[1] == 0.0)
    # length one: the only key is the query itself, output = v_0 (after rounding)
    assert np.max(np.abs(got[2, 0] - w.v[2, 0])) <= 1.5e-2


def test_single_token_problem():
    w = workloads.make_workload("one", dtype="fp32", B=1, L=1, H=1, d=32,
                                position_buckets=256, max_relative_positions=512, seed=1)
    got = H.host(H.run_padded(w))
    assert np.max(np.abs(got - w.v)) <= 1e-6


def test_varlen_degenerate_lengths():
    for lens in ([0, 0, 5, 0], [1], [0, 1, 0, 1], [2000, 0, 3]):
        lens = np.array(lens)
        w = workloads.make_workload("vl", dtype="bf16", B=len(lens), L=int(lens.max()), H=3,
                                    d=64, position_buckets=256, max_relative_positions=512,
                                    lens=lens, seed=int(lens.sum()), packed=True)
        _say(f"varlen lens {lens.tolist()}")
        got = H.host(H.run_varlen(w))
        want = H.oracle_varlen(w)
        assert np.all(np.isfinite(got))
        assert float(np.abs(got - want).max(initial=0.0)) <= 1.5e-2


def test_fused_qkv_strides_padded_and_packed():
    """Q, K, V as column views of one [tokens, 3*H*d] buffer (row stride 3*H*d)."""
    import torch
    import deberta_disentangled_attention_amd as dd
    w = _small("bf16", B=2, L=300, lens=[300, 211], Hh=4, d=32)
    hd = w.H * w.d
    fused = np.concatenate([w.q, w.k, w.v], axis=-1)
    buf = H.dev(fused, "bf16")
    q, k, v = buf[..., :hd], buf[..., hd:2 * hd], buf[..., 2 * hd:]
    got = H.host(H.run_padded(w, q=q, k=k, v=v))
    want = H.oracle_padded(w)
    H.assert_padded_close(got, want, H.valid_rows_padded(w), "bf16", "fused padded")
    wp = workloads.to_packed(w)
    fp = np.concatenate([wp.q, wp.k, wp.v], axis=-1)
    pbuf = H.dev(fp, "bf16")
    T = H.gpu_table(w.L, w.position_buckets, w.max_relative_positions)
    cu = torch.from_numpy(wp.cu_seqlens).cuda()
    out = dd.dattn_fwd_varlen(pbuf[:, :hd], pbuf[:, hd:2 * hd], pbuf[:, 2 * hd:],
                              H.dev(wp.qr, "bf16"), H.dev(wp.kr, "bf16"), T, w.L, cu,
                              wp.max_seqlen, w.H, w.d)
    torch.cuda.synchronize()
    assert np.array_equal(H.host(out), workloads.pack(got, w.lens))


def test_output_fully_written_and_stream():
    """The output buffer is pre-filled with NaN; every element is written.
    The call runs on a non-default stream."""
    import torch
    import deberta_disentangled_attention_amd as dd
    w = _small("fp16", B=3, L=270, lens=[270, 1, 129])
    T = H.gpu_table(w.L, w.position_buckets, w.max_relative_positions)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = torch.full((w.B, w.L, w.H * w.d), float("nan"), dtype=torch.float16, device="cuda")
        m = torch.from_numpy(w.mask).cuda()
        dd.dattn_fwd_padded(H.dev(w.q, "fp16"), H.dev(w.k, "fp16"), H.dev(w.v, "fp16"),
                            H.dev(w.qr, "fp16"), H.dev(w.kr, "fp16"), T, w.L, m, w.H, w.d,
                            out=out)
    s.synchronize()
    got = H.host(out)
    assert np.all(np.isfinite(got))
    want = H.oracle_padded(w)
    H.assert_padded_close(got, want, H.valid_rows_padded(w), "fp16", "stream")


def test_long_context_memory_is_o_of_l():
    """16 x 8192 packed bf16: the call allocates nothing, so the peak device
    allocation during it equals the inputs, outputs and the 64 KB table; a
    materialised bf16 [B, H, L, L] would be 25.8 GB."""
    import torch
    import deberta_disentangled_attention_amd as dd
    w = workloads.c4_long_packed_bf16()
    q, k, v = H.dev(w.q, "bf16"), H.dev(w.k, "bf16"), H.dev(w.v, "bf16")
    qr, kr = H.dev(w.qr, "bf16"), H.dev(w.kr, "bf16")
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    T = H.gpu_table(w.max_seqlen, w.position_buckets, w.max_relative_positions)
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    dd.dattn_fwd_varlen(q, k, v, qr, kr, T, w.max_seqlen, cu, w.max_seqlen, w.H, w.d, out=out)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() - base == 0
    assert np.all(np.isfinite(H.host(out[:4096])))


def test_max_length_padded_sampled():
    """L = 8192 in the padded layout with a ragged valid length."""
    w = workloads.make_workload("maxlen", dtype="bf16", B=1, L=8192, H=2, d=64,
                                position_buckets=256, max_relative_positions=512,
                                lens=np.array([8000]), seed=11)
    out = H.host(H.run_padded(w))
    T = oracle.rel_index_table(8192, 256, 512)
    rows = np.array([0, 1, 511, 512, 4000, 7998, 7999])
    for h in range(w.H):
        want = oracle.dattn_rows(w.q[0], w.k[0], w.v[0], w.qr, w.kr, T, 8192, h, w.d, rows,
                                 valid=w.mask[0])
        assert np.max(np.abs(out[0, rows, h * w.d:(h + 1) * w.d] - want)) <= 1.5e-2
    assert np.all(out[0, 8000:] == 0.0)


def test_many_short_sequences_varlen():
    """300 packed sequences of 1..40 tokens: exercises the tile-slot search
    over many sequences."""
    rng = np.random.default_rng(3)
    lens = rng.integers(1, 41, size=300)
    w = workloads.make_workload("many", dtype="bf16", B=len(lens), L=int(lens.max()), H=2, d=64,
                                position_buckets=256, max_relative_positions=512, lens=lens,
                                seed=4, packed=True)
    got = H.host(H.run_varlen(w, rel_max_len=64))
    want = H.oracle_varlen(w, rel_max_len=64)
    assert float(np.abs(got - want).max()) <= 1.5e-2


@pytest.mark.parametrize("nseq", [255, 256, 257, 511, 513, 1500])
def test_varlen_sequence_counts_around_search_strides(nseq):
    """Tile slots are mapped to sequences by a parallel search whose stride
    changes at multiples of the workgroup size; sweep across those edges."""
    rng = np.random.default_rng(nseq)
    lens = rng.integers(0, 24, size=nseq)
    lens[-1] = max(int(lens[-1]), 1)
    w = workloads.make_workload("counts", dtype="fp16", B=nseq, L=int(lens.max()), H=1, d=32,
                                position_buckets=8, max_relative_positions=20, lens=lens,
                                seed=nseq, packed=True)
    got = H.host(H.run_varlen(w, rel_max_len=32))
    want = H.oracle_varlen(w, rel_max_len=32)
    assert float(np.abs(got - want).max()) <= 5e-3


@pytest.mark.parametrize("L", [129, 200, 257, 300, 385, 513, 640, 1000])
def test_table_saturation_thresholds_across_lengths(L):
    """Small log buckets saturate early, so most tiles take the constant
    path; the saturation search runs over tables of 2L-1 entries."""
    for P, M in ((8, 20), (4, 7), (0, 24)):
        w = workloads.make_workload("sat", dtype="fp32", B=1, L=L, H=1, d=64,
                                    position_buckets=P, max_relative_positions=M, seed=L + P)
        got = H.host(H.run_padded(w))
        want = H.oracle_padded(w)
        H.assert_padded_close(got, want, H.valid_rows_padded(w), "fp32", f"sat L={L} P={P}")


# ---------------------------------------------------------------------------
# relative tables: windows too wide to stage, out-of-range rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("P,M,L", [(0, 1100, 2500), (512, 2048, 3000)])
def test_wide_table_window_reads_table_from_memory(dtype, P, M, L):
    """Tables whose non-saturated window spans more than the 2048 entries a
    workgroup stages in LDS (identity span 1100; log buckets 512/2048):
    band terms then read the table from device memory. Full check, padded
    and packed."""
    lens = np.array([L, L - 611])
    w = workloads.make_workload(f"wide_{P}_{M}", dtype=dtype, B=2, L=L, H=1, d=64,
                                position_buckets=P, max_relative_positions=M, lens=lens,
                                seed=L + P)
    T = oracle.rel_index_table(L, P, M)
    lo = int(np.argmax(T != T[0])) - 1
    hi = int(np.argmax(T == T[-1]))
    assert hi - lo + 1 > 2048, (lo, hi)        # the window the kernel cannot stage
    _say(f"wide table {dtype} P={P} M={M} L={L}")
    got = H.host(H.run_padded(w))
    want = H.oracle_padded(w)
    worst = H.assert_padded_close(got, want, H.valid_rows_padded(w), dtype, "wide padded")
    wp = workloads.to_packed(w)
    gotp = H.host(H.run_varlen(wp, rel_max_len=L))
    errp = float(np.abs(gotp - workloads.pack(want, w.lens)).max())
    assert errp <= H.TOL[dtype], errp
    _say(f"   max abs err padded {worst:.3e} packed {errp:.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_out_of_range_table_rows_read_edge_rows(dtype):
    """A non-decreasing table whose entries run from -75 to 74 with only 40
    rows in qr / kr: rows below 0 read row 0, rows from 40 on read row 39
    (the oracle's clamp_rows reading)."""
    L = 300
    w = workloads.make_workload("clamp", dtype=dtype, B=2, L=L, H=2, d=64, position_buckets=20,
                                max_relative_positions=64, lens=np.array([L, 123]), seed=17)
    w.qr, w.kr = w.qr[:40].copy(), w.kr[:40].copy()
    T = (np.arange(-(L - 1), L) // 4).astype(np.int32)
    assert T.min() < 0 and T.max() >= 40
    got = H.host(H.run_padded(w, table=T))
    want = oracle.dattn_padded(w.q, w.k, w.v, w.qr, w.kr, T, L, w.mask, w.H, w.d,
                               clamp_rows=True)
    worst = H.assert_padded_close(got, want, H.valid_rows_padded(w), dtype, "clamp padded")
    wp = workloads.to_packed(w)
    gotp = H.host(H.run_varlen(wp, rel_max_len=L, table=T))
    errp = float(np.abs(gotp - workloads.pack(want, w.lens)).max())
    assert errp <= H.TOL[dtype], errp
    _say(f"clamp {dtype}: max abs err padded {worst:.3e} packed {errp:.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [32, 64])
def test_short_packed_tile_dispatch(dtype, d):
    """Packed batches whose bound max_seqlen is at most 128 run 64-query tiles;
    the same batch under a larger bound runs the 128-query tiles. Both
    against the oracle, with the boundary lengths 127/128 present."""
    import torch
    import deberta_disentangled_attention_amd as dd
    rng = np.random.default_rng(d)
    lens = np.concatenate([rng.integers(1, 129, size=40), [128, 127, 1, 0, 64, 65]])
    w = workloads.make_workload("short", dtype=dtype, B=len(lens), L=128, H=3, d=d,
                                position_buckets=32, max_relative_positions=128, lens=lens,
                                seed=d + 1, packed=True)
    want = H.oracle_varlen(w, rel_max_len=128)
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    args = [H.dev(x, dtype) for x in (w.q, w.k, w.v, w.qr, w.kr)]
    for bound in (128, 4096):
        # the table must cover the bound; its entries depend on the distance only
        T = H.gpu_table(bound, w.position_buckets, w.max_relative_positions)
        got = H.host(dd.dattn_fwd_varlen(*args, T, bound, cu, bound, w.H, w.d, flags=w.flags))
        err = float(np.abs(got - want).max())
        print(f"short packed {dtype} d={d} bound={bound}: {err:.2e}", file=sys.stderr, flush=True)
        assert err <= H.TOL[dtype], (bound, err)


# Keys whose scores jump by more than 8 (base-2 units) from one far tile to a
# later one make the far loop raise its softmax offset in the middle of a run
# (left of the queries and right of them): the cold path forms the tile's
# scores again from global memory, rescales the accumulators that already
# hold the previous tile's P.V, and the loop restarts with a new bias block.
# Spike keys carry q.k of 40 to 490 against queries along one axis, at least
# 90 apart (more than 9 base-2 units at the default scale), so the largest
# spike dominates every row and no two keys compete: the rounding of the far
# tiles' scaled operand then stays well inside the bar. In key order the
# spikes rise and fall, so runs see raises and tiles that need none.
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("packed", [False, True])
def test_far_offset_raises_mid_run(dtype, packed):
    L, Hh, d = 2048, 2, 64
    w = workloads.make_workload("raise", dtype=dtype, B=1, L=L, H=Hh, d=d, position_buckets=256,
                                max_relative_positions=512, seed=41, packed=packed, with_mask=False)
    rng = np.random.default_rng(42)
    q = 0.1 * rng.standard_normal(w.q.shape)
    k = 0.1 * rng.standard_normal(w.k.shape)
    for h in range(Hh):
        q[..., h * d] += 2.0                                    # every query along axis 0
    spikes = {90: 65.0, 600: 20.0, 1000: 155.0, 1400: 110.0, 1830: 245.0, 1990: 200.0}
    for pos, c in spikes.items():
        for h in range(Hh):
            k[..., pos, h * d] += c
    w.q = workloads.round_to(q, dtype)
    w.k = workloads.round_to(k, dtype)
    w.qr = workloads.round_to(0.05 * rng.standard_normal(w.qr.shape), dtype)
    w.kr = workloads.round_to(0.05 * rng.standard_normal(w.kr.shape), dtype)
    if packed:
        got = H.host(H.run_varlen(w))
        want = H.oracle_varlen(w)
        err = float(np.abs(got - want).max())
    else:
        got = H.host(H.run_padded(w))
        want = H.oracle_padded(w)
        err = float(np.abs(got - want).max())
    _say(f"far offset raises {dtype} packed={packed}: max abs err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= H.TOL[dtype], err


def test_mask_scan_batches_and_alignment():
    """The padded extent scan reads the mask in batches (2048 positions a
    batch by 4-byte words, 512 by bytes when the row length or the pointer is
    not word-aligned): the last valid position and the first padded one lie
    past the first batch here, in both forms, and the same mask at an odd
    address (byte form) gives the word form's output bit for bit."""
    import torch
    for L, dtype in ((2600, "bf16"), (1001, "fp16")):
        w = workloads.make_workload(f"scan{L}", dtype=dtype, B=2, L=L, H=1, d=64,
                                    position_buckets=256, max_relative_positions=512,
                                    lens=np.array([L, L]), seed=11)
        m = np.zeros((2, L), np.uint8)
        m[0, :L - 200] = 1
        m[0, L - 700] = 0                # first padded position past the first batch
        m[1, :5] = 1
        m[1, L - 10] = 1                 # last valid position past the first batch
        w.mask = m
        _say(f"mask scan L={L} {dtype}")
        got = H.host(H.run_padded(w))
        want = H.oracle_padded(w)
        H.assert_padded_close(got, want, m.astype(bool), dtype, f"mask scan L={L}")
        big = torch.zeros(2 * L + 1, dtype=torch.uint8, device="cuda")
        big[1:] = torch.from_numpy(m.reshape(-1)).cuda()
        odd = big[1:].view(2, L)
        assert odd.data_ptr() % 4 != 0
        got_odd = H.host(H.run_padded(w, mask=odd))
        assert np.array_equal(got, got_odd)
