"""Pins of the packing oracle (oracle/pack.py), on the CPU.

The oracle's packing follows the definition of DisentangledFlash's packed
unpadded inference (README, "Packed unpadded inference"): valid rows in
order, int32 cumulative lengths, padded outputs restored with zero rows.
The pages print no worked example, so the pins are: small examples worked
out by hand from that definition, a pure-Python brute force with explicit
counters, the right-padded special case against the generator's own
concatenation helpers, and round-trip / inverse-map invariants.
"""

import numpy as np
import pytest

import workloads
from oracle import pack as P


def brute(mask):
    """Explicit loops and counters, no numpy reductions."""
    B, L = len(mask), len(mask[0]) if len(mask) else 0
    cu = [0]
    token_rows, row_to_packed = [], [-1] * (B * L)
    for b in range(B):
        n = 0
        for l in range(L):
            if mask[b][l]:
                row_to_packed[b * L + l] = len(token_rows)
                token_rows.append(b * L + l)
                n += 1
        cu.append(cu[-1] + n)
    token_rows += [-1] * (B * L - len(token_rows))
    return cu, token_rows, row_to_packed


def test_hand_example_holes():
    # row 0 right padded, row 1 with holes, row 2 full (worked by hand)
    m = np.array([[1, 1, 0, 0], [0, 1, 0, 1], [1, 1, 1, 1]], np.uint8)
    cu, tr, rp = P.pack_index(m, 3, 4)
    assert cu.tolist() == [0, 2, 4, 8]
    assert tr.tolist() == [0, 1, 5, 7, 8, 9, 10, 11, -1, -1, -1, -1]
    assert rp.tolist() == [0, 1, -1, -1, -1, 2, -1, 3, 4, 5, 6, 7]
    x = np.arange(12 * 2).reshape(12, 2)
    assert P.pack_rows(x, tr, 8).tolist() == [[0, 1], [2, 3], [10, 11], [14, 15],
                                             [16, 17], [18, 19], [20, 21], [22, 23]]


def test_hand_example_empty_row():
    m = np.array([[0, 0, 0], [1, 0, 1]], np.uint8)
    cu, tr, rp = P.pack_index(m, 2, 3)
    assert cu.tolist() == [0, 0, 2]
    assert tr.tolist() == [3, 5, -1, -1, -1, -1]
    assert rp.tolist() == [-1, -1, -1, 0, -1, 1]
    y = np.array([[7.0], [9.0]])
    assert P.unpack_rows(y, rp).ravel().tolist() == [0, 0, 0, 7, 0, 9]


def test_no_mask_is_identity():
    cu, tr, rp = P.pack_index(None, 3, 5)
    assert cu.tolist() == [0, 5, 10, 15]
    assert tr.tolist() == list(range(15))
    assert rp.tolist() == list(range(15))


@pytest.mark.parametrize("seed", range(6))
def test_brute_force(seed):
    rng = np.random.default_rng(seed)
    B, L = int(rng.integers(1, 7)), int(rng.integers(1, 9))
    m = (rng.random((B, L)) < rng.random()).astype(np.uint8) * rng.integers(1, 255, (B, L)).astype(np.uint8)
    cu, tr, rp = P.pack_index(m, B, L)
    bcu, btr, brp = brute(m.tolist())
    assert cu.tolist() == bcu and tr.tolist() == btr and rp.tolist() == brp


@pytest.mark.parametrize("seed", range(4))
def test_right_padded_matches_concatenation(seed):
    rng = np.random.default_rng(seed + 10)
    B, L, W = 5, 40, 3
    lens = rng.integers(0, L + 1, size=B)
    m = workloads.right_pad_mask(lens, L)
    x = rng.standard_normal((B, L, W))
    cu, tr, rp = P.pack_index(m, B, L)
    assert cu.tolist() == [0] + np.cumsum(lens).tolist()
    packed = P.pack_rows(x.reshape(B * L, W), tr, int(cu[-1]))
    assert np.array_equal(packed, workloads.pack(x, lens))
    back = P.unpack_rows(packed, rp).reshape(B, L, W)
    assert np.array_equal(back, workloads.unpack(packed, lens, L))


@pytest.mark.parametrize("seed", range(4))
def test_round_trip_and_inverse(seed):
    rng = np.random.default_rng(seed + 20)
    B, L, W = 7, 33, 4
    m = (rng.random((B, L)) < 0.4).astype(np.uint8)
    cu, tr, rp = P.pack_index(m, B, L)
    total = int(cu[-1])
    assert np.all(np.diff(cu) == m.sum(axis=1))
    assert np.all(np.diff(tr[:total]) > 0) and np.all(tr[total:] == -1)
    assert np.array_equal(rp[tr[:total]], np.arange(total))
    assert np.array_equal(rp >= 0, m.reshape(-1) != 0)
    x = rng.standard_normal((B * L, W))
    y = P.pack_rows(x, tr, total)
    assert np.array_equal(P.unpack_rows(y, rp), x * m.reshape(-1, 1))
    assert np.array_equal(P.pack_rows(P.unpack_rows(y, rp), tr, total), y)
