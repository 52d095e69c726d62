"""Pins of the relative-table projection oracle (oracle/relproj.py), on the CPU.

A hand-worked integer example, a pure-Python brute force, the identity and
zero maps, linearity in the embeddings, and agreement with the generator's
own construction of the projected tables (R times an [in, out] matrix),
which fixes the nn.Linear weight layout ([out, in]).
"""

import numpy as np
import pytest

import workloads
from oracle import relproj as P


def test_hand_example():
    E = np.array([[1, 2, 3], [0, -1, 4]])
    Wq = np.array([[1, 0, 0], [0, 1, 1]])          # outputs: e0, e1 + e2
    Wk = np.array([[2, 0, -1], [1, 1, 1]])         # outputs: 2 e0 - e2, e0 + e1 + e2
    bq = np.array([10, 20])
    qr, kr = P.rel_proj(E, Wq, Wk, bq, None)
    assert qr.tolist() == [[11, 25], [10, 23]]
    assert kr.tolist() == [[-1, 6], [-4, 3]]


def brute(E, W, b):
    n, h = len(E), len(E[0])
    o = len(W)
    out = [[0.0] * o for _ in range(n)]
    for r in range(n):
        for c in range(o):
            acc = 0.0 if b is None else float(b[c])
            for i in range(h):
                acc += float(E[r][i]) * float(W[c][i])
            out[r][c] = acc
    return out


@pytest.mark.parametrize("seed", range(4))
def test_brute_force(seed):
    rng = np.random.default_rng(seed)
    n, h, o = int(rng.integers(1, 6)), int(rng.integers(1, 7)), int(rng.integers(1, 6))
    E = rng.integers(-4, 5, (n, h))
    Wq, Wk = rng.integers(-3, 4, (o, h)), rng.integers(-3, 4, (o, h))
    bq = rng.integers(-5, 6, o)
    qr, kr = P.rel_proj(E, Wq, Wk, bq, None)
    assert qr.tolist() == brute(E.tolist(), Wq.tolist(), bq.tolist())
    assert kr.tolist() == brute(E.tolist(), Wk.tolist(), None)


def test_identity_and_zero_maps():
    rng = np.random.default_rng(7)
    E = rng.standard_normal((9, 6))
    b = rng.standard_normal(6)
    qr, kr = P.rel_proj(E, np.eye(6), np.zeros((6, 6)), b, b)
    assert np.array_equal(qr, E + b)
    assert np.array_equal(kr, np.broadcast_to(b, (9, 6)))


def test_linear_in_the_embeddings():
    rng = np.random.default_rng(8)
    E1, E2 = rng.integers(-8, 9, (5, 12)), rng.integers(-8, 9, (5, 12))
    Wq, Wk = rng.integers(-8, 9, (7, 12)), rng.integers(-8, 9, (7, 12))
    a1, k1 = P.rel_proj(3 * E1 - 2 * E2, Wq, Wk)
    a2, k2 = P.rel_proj(E1, Wq, Wk)
    a3, k3 = P.rel_proj(E2, Wq, Wk)
    assert np.array_equal(a1, 3 * a2 - 2 * a3) and np.array_equal(k1, 3 * k2 - 2 * k3)


def test_layout_matches_the_generator():
    """workloads.relative_tables draws R, then [in, out] matrices, and forms
    R @ W: the oracle's [out, in] weights are their transposes."""
    H, d, n_rel = 2, 8, 10
    hidden = H * d
    rng = np.random.Generator(np.random.PCG64(5))
    qr_w, kr_w = workloads.relative_tables(rng, n_rel, H, d, "fp32")
    rng = np.random.Generator(np.random.PCG64(5))
    R = rng.standard_normal(size=(n_rel, hidden)) * 0.02
    s = 1.0 / (0.02 * np.sqrt(hidden))
    Wq = rng.standard_normal(size=(hidden, hidden)) * s
    Wk = rng.standard_normal(size=(hidden, hidden)) * s
    qr, kr = P.rel_proj(R, Wq.T, Wk.T)
    assert np.allclose(qr.astype(np.float32), qr_w, rtol=0, atol=1e-6)
    assert np.allclose(kr.astype(np.float32), kr_w, rtol=0, atol=1e-6)


def test_abs_bound_dominates():
    rng = np.random.default_rng(9)
    E, W = rng.standard_normal((4, 5)), rng.standard_normal((3, 5))
    y, _ = P.rel_proj(E, W, W)
    assert np.all(np.abs(y) <= P.abs_bound(E, W) + 1e-12)
