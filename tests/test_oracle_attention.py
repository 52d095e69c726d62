"""Pins for the oracle's attention forward (CPU only).

Each test ties the oracle to something other than its own code:
  * a pure-Python triple-loop brute force on tiny inputs,
  * torch's scaled_dot_product_attention for the cases that reduce to it,
  * inputs built so that the score matrix spells out which relative row
    each position term reads (catches a swapped sign, index or table),
  * the hand-derived example in tests/golden/worked_example_l2.json,
  * invariants: softmax rows sum to one, masked keys carry no weight,
    padded queries give zero, packed equals padded, position terms depend
    only on i - j.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa
from oracle import bucket

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force(q, k, v, qr, kr, T, Lmax, mask, H, d, flags, scale):
    """Scalar loops, one score at a time, straight from the definition."""
    B, L, _ = q.shape
    tau = scale if scale > 0 else 1.0 / math.sqrt(d * (1 + bin(flags).count("1")))
    out = [[[0.0] * (H * d) for _ in range(L)] for _ in range(B)]
    for b in range(B):
        m = [1] * L if mask is None else [int(x) for x in mask[b]]
        for h in range(H):
            c = h * d
            for i in range(L):
                if not m[i]:
                    continue
                sc = []
                for j in range(L):
                    if not m[j]:
                        continue
                    s = 0.0
                    for t in range(d):
                        s += float(q[b, i, c + t]) * float(k[b, j, c + t])
                    if flags & 1:
                        row = int(T[i - j + Lmax - 1])
                        for t in range(d):
                            s += float(q[b, i, c + t]) * float(kr[row, c + t])
                    if flags & 2:
                        row = int(T[j - i + Lmax - 1])
                        for t in range(d):
                            s += float(k[b, j, c + t]) * float(qr[row, c + t])
                    sc.append((j, s * tau))
                mx = max(s for _, s in sc)
                w = [(j, math.exp(s - mx)) for j, s in sc]
                Z = sum(x for _, x in w)
                for t in range(d):
                    out[b][i][c + t] = sum(x * float(v[b, j, c + t]) for j, x in w) / Z
    return np.array(out)


def rand_case(seed, B, L, H, d, P, M, masked=True):
    rng = np.random.default_rng(seed)
    s = bucket.span(P, M)
    q = rng.standard_normal((B, L, H * d))
    k = rng.standard_normal((B, L, H * d))
    v = rng.standard_normal((B, L, H * d))
    qr = rng.standard_normal((2 * s, H * d))
    kr = rng.standard_normal((2 * s, H * d))
    mask = None
    if masked:
        mask = (rng.random((B, L)) < 0.7).astype(np.uint8)
        mask[:, 0] = 1
    return q, k, v, qr, kr, mask


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("P,M,L", [(8, 20, 24), (0, 5, 13), (4, 7, 17)])
def test_brute_force_matches(flags, P, M, L):
    B, H, d = 2, 2, 3
    q, k, v, qr, kr, mask = rand_case(7 + flags + L, B, L, H, d, P, M)
    Lmax = L + 3
    T = bucket.rel_index_table(Lmax, P, M)
    got = oracle.dattn_padded(q, k, v, qr, kr, T, Lmax, mask, H, d, flags)
    want = brute_force(q, k, v, qr, kr, T, Lmax, mask, H, d, flags, 0.0)
    assert np.max(np.abs(got - want)) < 1e-12


def test_brute_force_explicit_scale():
    q, k, v, qr, kr, mask = rand_case(3, 1, 9, 1, 4, 8, 20)
    T = bucket.rel_index_table(9, 8, 20)
    got = oracle.dattn_padded(q, k, v, qr, kr, T, 9, mask, 1, 4, 3, scale=0.37)
    want = brute_force(q, k, v, qr, kr, T, 9, mask, 1, 4, 3, 0.37)
    assert np.max(np.abs(got - want)) < 1e-12


def _sdpa(qh, kh, vh, valid, scale):
    qt = torch.from_numpy(qh)[None, None]
    kt = torch.from_numpy(kh)[None, None]
    vt = torch.from_numpy(vh)[None, None]
    am = torch.from_numpy(valid.astype(bool))[None, None, None, :].expand(1, 1, qh.shape[0], kh.shape[0])
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("d", [8, 32])
def test_flags0_is_standard_attention(d):
    B, L, H = 2, 40, 3
    q, k, v, qr, kr, mask = rand_case(11, B, L, H, d, 16, 64)
    T = bucket.rel_index_table(L, 16, 64)
    got = oracle.dattn_padded(q, k, v, qr, kr, T, L, mask, H, d, flags=0)
    for b in range(B):
        valid = mask[b].astype(bool)
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            want = _sdpa(q[b, :, sl], k[b, :, sl], v[b, :, sl], mask[b], 1.0 / math.sqrt(d))
            assert np.max(np.abs(got[b][valid][:, sl] - want[valid])) < 1e-12
            assert np.all(got[b][~valid][:, sl] == 0.0)


def test_zero_relative_tables_is_attention_at_sqrt3d():
    B, L, H, d = 1, 33, 2, 16
    q, k, v, qr, kr, mask = rand_case(12, B, L, H, d, 8, 20, masked=False)
    qr[:] = 0.0
    kr[:] = 0.0
    T = bucket.rel_index_table(L, 8, 20)
    got = oracle.dattn_padded(q, k, v, qr, kr, T, L, None, H, d, flags=3)
    for h in range(H):
        sl = slice(h * d, (h + 1) * d)
        want = _sdpa(q[0, :, sl], k[0, :, sl], v[0, :, sl], np.ones(L), 1.0 / math.sqrt(3 * d))
        assert np.max(np.abs(got[0, :, sl] - want)) < 1e-12


@pytest.mark.parametrize("P,M,L,Lmax", [(8, 20, 30, 30), (16, 40, 50, 64), (0, 6, 20, 25)])
def test_c2p_reads_kr_at_row_of_i_minus_j(P, M, L, Lmax):
    """q_i = e_0 for every i, k = 0, kr[row] = row * e_0 and qr = garbage:
    then S_ij / tau must be exactly T(i - j)."""
    d = 4
    s = bucket.span(P, M)
    T = bucket.rel_index_table(Lmax, P, M)
    Q = np.zeros((L, d)); Q[:, 0] = 1.0
    K = np.zeros((L, d))
    KR = np.zeros((2 * s, d)); KR[:, 0] = np.arange(2 * s)
    QR = np.full((2 * s, d), -1000.0)
    S = oa.unit_scores(Q, K, QR, KR, T, Lmax, flags=3, tau=1.0)
    i, j = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    assert np.array_equal(S, T[i - j + Lmax - 1].astype(np.float64))


@pytest.mark.parametrize("P,M,L,Lmax", [(8, 20, 30, 30), (16, 40, 50, 64), (0, 6, 20, 25)])
def test_p2c_reads_qr_at_row_of_j_minus_i(P, M, L, Lmax):
    """k_j = e_0 for every j, q = 0, qr[row] = row * e_0, kr = garbage:
    then S_ij / tau must be exactly T(j - i)."""
    d = 4
    s = bucket.span(P, M)
    T = bucket.rel_index_table(Lmax, P, M)
    Q = np.zeros((L, d))
    K = np.zeros((L, d)); K[:, 0] = 1.0
    QR = np.zeros((2 * s, d)); QR[:, 0] = np.arange(2 * s)
    KR = np.full((2 * s, d), -1000.0)
    S = oa.unit_scores(Q, K, QR, KR, T, Lmax, flags=3, tau=1.0)
    i, j = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    assert np.array_equal(S, T[j - i + Lmax - 1].astype(np.float64))


def test_position_terms_depend_only_on_distance():
    """With identical query rows the C2P matrix is Toeplitz; with identical
    key rows the P2C matrix is Toeplitz."""
    rng = np.random.default_rng(5)
    L, d, P, M = 40, 8, 16, 40
    T = bucket.rel_index_table(L, P, M)
    QR = rng.standard_normal((32, d))
    KR = rng.standard_normal((32, d))
    Q = np.tile(rng.standard_normal(d), (L, 1))
    K0 = np.zeros((L, d))
    S = oa.unit_scores(Q, K0, QR, KR, T, L, flags=1, tau=1.0)
    for off in range(-L + 1, L):
        assert np.ptp(np.diagonal(S, offset=off)) == 0.0
    K = np.tile(rng.standard_normal(d), (L, 1))
    S = oa.unit_scores(np.zeros((L, d)), K, QR, KR, T, L, flags=2, tau=1.0)
    for off in range(-L + 1, L):
        assert np.ptp(np.diagonal(S, offset=off)) == 0.0


def _golden():
    with open(os.path.join(GOLDEN, "worked_example_l2.json")) as f:
        return json.load(f)


def test_golden_worked_example():
    g = _golden()
    q = np.array(g["q"]).reshape(1, 2, 1)
    k = np.array(g["k"]).reshape(1, 2, 1)
    v = np.array(g["v"]).reshape(1, 2, 1)
    qr = np.array(g["qr"]).reshape(2, 1)
    kr = np.array(g["kr"]).reshape(2, 1)
    T = bucket.rel_index_table(2, g["position_buckets"], g["max_relative_positions"])
    assert T.tolist() == g["table"]["T"]
    S = oa.unit_scores(q[0], k[0], qr, kr, T, 2, flags=3, tau=1.0)
    assert S.tolist() == g["unscaled_scores"]["values"]
    S1 = oa.unit_scores(q[0], k[0], qr, kr, T, 2, flags=1, tau=1.0)
    assert S1.tolist() == g["c2p_only"]["values"]
    S2 = oa.unit_scores(q[0], k[0], qr, kr, T, 2, flags=2, tau=1.0)
    assert S2.tolist() == g["p2c_only"]["values"]
    out = oracle.dattn_padded(q, k, v, qr, kr, T, 2, None, 1, 1, flags=3)
    tau = 1 / math.sqrt(3)
    assert abs(out[0, 0, 0] - (20 - 10 / (1 + math.exp(-5 * tau)))) < 1e-13
    assert abs(out[0, 1, 0] - (20 - 10 / (1 + math.exp(-8 * tau)))) < 1e-13
    out = oracle.dattn_padded(q, k, v, qr, kr, T, 2, np.array([g["masked"]["mask"]], np.uint8), 1, 1, flags=3)
    assert out[0, :, 0].tolist() == g["masked"]["O"]
    out = oracle.dattn_padded(q, k, v, qr, kr, T, 2, None, 1, 1, flags=1)
    t2 = 1 / math.sqrt(2)
    assert abs(out[0, 0, 0] - (10 + 10 * math.exp(t2) / (1 + math.exp(t2)))) < 1e-13
    assert abs(out[0, 1, 0] - (10 + 10 * math.exp(-4 * t2) / (1 + math.exp(-4 * t2)))) < 1e-13


def test_rows_sum_to_one_and_masked_keys_carry_no_weight():
    B, L, H, d = 3, 37, 2, 8
    q, k, v, qr, kr, mask = rand_case(21, B, L, H, d, 16, 64)
    T = bucket.rel_index_table(L, 16, 64)
    ones = np.ones_like(v)
    out = oracle.dattn_padded(q, k, ones, qr, kr, T, L, mask, H, d)
    valid = mask.astype(bool)
    assert np.max(np.abs(out[valid] - 1.0)) < 1e-13
    assert np.all(out[~valid] == 0.0)
    base = oracle.dattn_padded(q, k, v, qr, kr, T, L, mask, H, d)
    k2, v2 = k.copy(), v.copy()
    k2[~valid] = 1e6
    v2[~valid] = np.nan
    pert = oracle.dattn_padded(q, k2, v2, qr, kr, T, L, mask, H, d)
    assert np.array_equal(base[valid], pert[valid])


def test_packed_equals_padded():
    rng = np.random.default_rng(8)
    lens = np.array([5, 0, 19, 1, 12])
    B, L, H, d = len(lens), 20, 2, 6
    q, k, v, qr, kr, _ = rand_case(9, B, L, H, d, 8, 20, masked=False)
    mask = (np.arange(L)[None] < lens[:, None]).astype(np.uint8)
    T = bucket.rel_index_table(L, 8, 20)
    pad = oracle.dattn_padded(q, k, v, qr, kr, T, L, mask, H, d)
    cat = lambda x: np.concatenate([x[b, :n] for b, n in enumerate(lens)])
    cu = np.concatenate([[0], np.cumsum(lens)])
    packed = oracle.dattn_varlen(cat(q), cat(k), cat(v), qr, kr, T, L, cu, H, d)
    assert np.array_equal(packed, cat(pad))
    assert rng is not None


def test_rows_helper_equals_full_unit():
    B, L, H, d = 1, 50, 2, 8
    q, k, v, qr, kr, mask = rand_case(4, B, L, H, d, 16, 64)
    T = bucket.rel_index_table(64, 16, 64)
    full = oracle.dattn_padded(q, k, v, qr, kr, T, 64, mask, H, d)
    rows = [0, 3, 17, 49]
    for h in range(H):
        got = oracle.dattn_rows(q[0], k[0], v[0], qr, kr, T, 64, h, d, rows, valid=mask[0])
        assert np.array_equal(got, full[0, rows, h * d:(h + 1) * d])


def test_table_checks():
    q, k, v, qr, kr, _ = rand_case(1, 1, 10, 1, 4, 8, 20, masked=False)
    T = bucket.rel_index_table(8, 8, 20)
    with pytest.raises(ValueError):
        oracle.dattn_padded(q, k, v, qr, kr, T, 8, None, 1, 4)   # rel_max_len < L


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_clamp_rows_equals_tables_extended_by_their_edge_rows(flags):
    """clamp_rows (a row index below 0 reads row 0, one at or above n_rel
    reads row n_rel - 1) pinned against a different construction: the same
    table shifted into range over qr / kr extended by copies of their first
    and last rows; and also against the brute force."""
    L, H, d, n_rel, pad = 11, 2, 4, 6, 9
    q, k, v, _, _, mask = rand_case(21, 2, L, H, d, 3, 5)
    rng = np.random.default_rng(3)
    qr = rng.standard_normal((n_rel, H * d))
    kr = rng.standard_normal((n_rel, H * d))
    T = np.arange(-(L - 1), L) // 2 + 1            # -4 .. 6: both ends outside [0, 6)
    assert T.min() < 0 and T.max() >= n_rel
    with pytest.raises(ValueError):
        oracle.dattn_padded(q, k, v, qr, kr, T, L, mask, H, d, flags)
    got = oracle.dattn_padded(q, k, v, qr, kr, T, L, mask, H, d, flags, clamp_rows=True)
    ext = lambda x: np.concatenate([np.repeat(x[:1], pad, 0), x, np.repeat(x[-1:], pad, 0)])
    want = oracle.dattn_padded(q, k, v, ext(qr), ext(kr), T + pad, L, mask, H, d, flags)
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    Tc = np.minimum(np.maximum(T, 0), n_rel - 1)
    brute = brute_force(q, k, v, qr, kr, Tc, L, mask, H, d, flags, 0.0)
    assert np.allclose(got, brute, rtol=0, atol=1e-12)
