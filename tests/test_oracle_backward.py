"""Pins of the backward oracle (oracle/backward.py), on the CPU.

The gradients are tied to things other than their own formulas: central
finite differences of the forward oracle, torch's autograd (float64, CPU)
through a forward written here independently with torch ops, the one-token
closed form, the row identity sum_j dS_ij = 0 (checked through dQ of a
problem whose keys are all equal), and masks.
"""

import numpy as np
import pytest

import oracle
from oracle import backward as BW


def tiny(seed, B=2, L=6, H=2, d=4, P=4, M=6, mask=True):
    rng = np.random.default_rng(seed)
    q, k, v, dout = (rng.standard_normal((B, L, H * d)) for _ in range(4))
    T = oracle.rel_index_table(L, P, M)
    n_rel = 2 * P
    qr, kr = (rng.standard_normal((n_rel, H * d)) for _ in range(2))
    m = None
    if mask:
        m = np.ones((B, L), dtype=np.uint8)
        m[1, 4:] = 0
        m[0, 2] = 0
    return q, k, v, qr, kr, T, m, dout


def loss(q, k, v, qr, kr, T, L, m, H, d, dout, flags):
    out = oracle.dattn_padded(q, k, v, qr, kr, T, L, m, H, d, flags, 0.0)
    return float(np.sum(out * dout))


@pytest.mark.parametrize("flags", [3, 1, 2, 0])
def test_finite_differences(flags):
    q, k, v, qr, kr, T, m, dout = tiny(flags + 1)
    B, L, HD = q.shape
    H, d = 2, 4
    g = BW.dattn_padded_bwd(q, k, v, qr, kr, T, L, m, H, d, dout, flags)
    eps = 1e-6
    for name, arr in (("dq", q), ("dk", k), ("dv", v), ("dqr", qr), ("dkr", kr)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss(q, k, v, qr, kr, T, L, m, H, d, dout, flags)
            arr[idx] = old - eps
            lm = loss(q, k, v, qr, kr, T, L, m, H, d, dout, flags)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        err = np.abs(num - g[name]).max()
        assert err < 1e-7 * max(1.0, np.abs(num).max()), (name, err)


@pytest.mark.parametrize("flags", [3, 1, 2])
def test_torch_autograd(flags):
    torch = pytest.importorskip("torch")
    q, k, v, qr, kr, T, m, dout = tiny(10 + flags, L=9, P=4, M=8)
    B, L, HD = q.shape
    H, d = 2, 4
    g = BW.dattn_padded_bwd(q, k, v, qr, kr, T, L, m, H, d, dout, flags)
    tau = oracle.default_scale(d, flags)
    tq, tk, tv, tqr, tkr = (torch.tensor(x, dtype=torch.float64, requires_grad=True)
                            for x in (q, k, v, qr, kr))
    Tt = torch.tensor(T, dtype=torch.long)
    ii = torch.arange(L)[:, None]
    jj = torch.arange(L)[None, :]
    c_idx = Tt[ii - jj + L - 1]          # row of kr for query i, key j
    p_idx = Tt[jj - ii + L - 1]          # row of qr for query i, key j
    mt = torch.tensor(m, dtype=torch.bool)
    total = 0.0
    for b in range(B):
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            Q, K, V = tq[b, :, sl], tk[b, :, sl], tv[b, :, sl]
            S = Q @ K.T
            if flags & 1:
                S = S + (Q[:, None, :] * tkr[:, sl][c_idx]).sum(-1)
            if flags & 2:
                S = S + (K[None, :, :] * tqr[:, sl][p_idx]).sum(-1)
            S = S * tau
            valid = mt[b]
            S = S.masked_fill(~valid[None, :], float("-inf"))
            A = torch.softmax(S, dim=-1)
            A = torch.where(valid[:, None], A, torch.zeros_like(A))
            O = A @ V
            total = total + (O * torch.tensor(dout[b, :, sl])).sum()
    total.backward()
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv), ("dqr", tqr), ("dkr", tkr)):
        # a table the enabled terms never read gets no gradient
        want = t.grad.numpy() if t.grad is not None else np.zeros_like(g[name])
        assert np.allclose(want, g[name], rtol=1e-10, atol=1e-12), name


def test_one_token_closed_form():
    """A single valid token: its softmax weight is 1 whatever the score, so
    dS = 0 (no gradient reaches q, k, qr, kr) and dV = dO."""
    q, k, v, qr, kr, T, _, dout = tiny(3, B=1, L=1, P=4, M=6, mask=False)
    T = oracle.rel_index_table(1, 4, 6)
    g = BW.dattn_padded_bwd(q, k, v, qr, kr, T, 1, None, 2, 4, dout, 3)
    for name in ("dq", "dk", "dqr", "dkr"):
        assert np.all(g[name] == 0), name
    assert np.array_equal(g["dv"], dout)


def test_masks_and_lse():
    q, k, v, qr, kr, T, m, dout = tiny(4)
    g = BW.dattn_padded_bwd(q, k, v, qr, kr, T, 6, m, 2, 4, dout, 3)
    pad = m == 0
    # padded queries: no gradient; padded keys: no dK, dV; lse -inf
    assert np.all(g["dq"][pad] == 0) and np.all(g["dk"][pad] == 0) and np.all(g["dv"][pad] == 0)
    assert np.all(np.isneginf(g["lse"][pad])) and np.all(np.isfinite(g["lse"][~pad]))
    # lse reproduces the forward: O = sum_j exp(S_ij - lse_i) v_j
    b, h, d = 0, 1, 4
    S = oracle.attention.unit_scores(q[b][:, 4:], k[b][:, 4:], qr[:, 4:], kr[:, 4:], T, 6, 3,
                                     oracle.default_scale(d, 3))
    valid = m[b].astype(bool)
    rows = np.nonzero(valid)[0]
    Wt = np.exp(S[rows] - g["lse"][b, rows, h][:, None]) * valid[None, :]
    out = oracle.dattn_padded(q, k, v, qr, kr, T, 6, m, 2, 4)
    assert np.allclose(Wt @ v[b][:, 4:], out[b][rows][:, 4:], atol=1e-12)


def test_rows_of_ds_sum_to_zero():
    """With every key equal, dQ_i = tau k sum_j dS_ij (no position terms),
    which the softmax makes zero."""
    rng = np.random.default_rng(5)
    L, d = 7, 4
    q = rng.standard_normal((1, L, d))
    k = np.broadcast_to(rng.standard_normal(d), (1, L, d)).copy()
    v = rng.standard_normal((1, L, d))
    dout = rng.standard_normal((1, L, d))
    T = oracle.rel_index_table(L, 4, 6)
    qr = kr = np.zeros((8, d))
    g = BW.dattn_padded_bwd(q, k, v, qr, kr, T, L, None, 1, d, dout, 0)
    assert np.abs(g["dq"]).max() < 1e-12


def test_varlen_equals_padded():
    q, k, v, qr, kr, T, _, dout = tiny(6, B=3, L=5, mask=False)
    lens = np.array([5, 2, 4])
    import workloads
    mask = workloads.right_pad_mask(lens, 5)
    gp = BW.dattn_padded_bwd(q, k, v, qr, kr, T, 5, mask, 2, 4, dout, 3)
    cu = np.concatenate([[0], np.cumsum(lens)])
    pk = lambda x: workloads.pack(x, lens)
    gv = BW.dattn_varlen_bwd(pk(q), pk(k), pk(v), qr, kr, T, 5, cu, 2, 4, pk(dout), 3)
    for name in ("dq", "dk", "dv"):
        assert np.allclose(gv[name], pk(gp[name]), atol=1e-13), name
    for name in ("dqr", "dkr"):
        assert np.allclose(gv[name], gp[name], atol=1e-12), name


def test_lse_rows_matches_unit_backward():
    q, k, v, qr, kr, T, m, dout = tiny(7)
    g = BW.dattn_padded_bwd(q, k, v, qr, kr, T, 6, m, 2, 4, dout, 3)
    for b in range(2):
        for h in range(2):
            got = BW.lse_rows(q[b], k[b], qr, kr, T, 6, h, 4, np.arange(6), valid=m[b])
            want = g["lse"][b, :, h]
            assert np.array_equal(np.isneginf(got), np.isneginf(want))
            fin = np.isfinite(want)
            assert np.allclose(got[fin], want[fin], rtol=0, atol=1e-12)
