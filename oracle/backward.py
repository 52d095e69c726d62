"""Gradients of the disentangled-attention forward, plain float64 on the CPU.

TEST INFRASTRUCTURE: only tests, the smoke entry and the benchmark's CPU
baseline may import this module. The product path never does.

What it computes. The pages' forward is inference-only: DisentangledFlash
falls back to the reference implementation in training mode (README,
"Status"), and the kernels-community layer declares no backward while its
author works on one (discussion #31, "Packaging and validation"). The
gradients here are those of the forward oracle (oracle.attention), written
out by the chain rule for one (sequence, head) unit:

    S_ij  = tau ( q_i.k_j + [C2P] q_i.kr[T(i-j)] + [P2C] k_j.qr[T(j-i)] )
    A     = softmax of each valid row over the valid keys, O = A V
    dV    = A^T dO
    dA_ij = dO_i . v_j
    D_i   = sum_j A_ij dA_ij            (equals dO_i . O_i)
    dS_ij = A_ij (dA_ij - D_i)          (zero for padded rows and keys)
    dQ_i  = tau sum_j dS_ij (k_j + [C2P] kr[T(i-j)])
    dK_j  = tau sum_i dS_ij (q_i + [P2C] qr[T(j-i)])
    dkr_r = tau sum over pairs with T(i-j) = r of dS_ij q_i      [C2P]
    dqr_r = tau sum over pairs with T(j-i) = r of dS_ij k_j      [P2C]

dkr and dqr collect every sequence of the batch (the relative tables are
shared). The statistic a backward kernel reads from the forward is also
returned: lse_i = log sum_j exp(S_ij) over the valid keys (natural log) for
valid rows, -inf for padded rows.

Pins: central finite differences of the forward oracle, torch's autograd on
the CPU (float64) of an independently written forward, the row identity
sum_j dS_ij = 0, masks, and the one-token closed form.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import C2P, P2C, _check_table, _head, default_scale, unit_scores


def unit_backward(Qh, Kh, Vh, QRh, KRh, T, rel_max_len: int, valid, flags: int, tau: float,
                  dOh):
    """Gradients of one (sequence, head) unit, all float64:
    (dQ [L, d], dK [L, d], dV [L, d], dQR [n_rel, d], dKR [n_rel, d], lse [L])."""
    L, d = Kh.shape
    n_rel = QRh.shape[0]
    valid = np.ones(L, dtype=bool) if valid is None else np.asarray(valid).astype(bool)
    S = unit_scores(Qh, Kh, QRh, KRh, T, rel_max_len, flags, tau)
    keymask = np.broadcast_to(valid[None, :], (L, L))
    pairmask = keymask & valid[:, None]
    Sm = np.where(pairmask, S, -np.inf)
    # rows with no valid pair (padded queries) take no part
    live = pairmask.any(axis=1)
    mx = np.where(live, np.max(np.where(pairmask, S, -np.inf), axis=1, initial=-np.inf), 0.0)
    E = np.where(pairmask, np.exp(Sm - mx[:, None]), 0.0)
    Z = E.sum(axis=1)
    A = np.where(live[:, None], E / np.where(Z > 0, Z, 1.0)[:, None], 0.0)
    lse = np.where(live, mx + np.log(np.where(Z > 0, Z, 1.0)), -np.inf)

    dO = np.asarray(dOh, dtype=np.float64)
    dV = A.T @ dO
    dA = dO @ Vh.T
    D = np.sum(A * dA, axis=1)
    dS = A * (dA - D[:, None])

    dQ = tau * (dS @ Kh)
    dK = tau * (dS.T @ Qh)
    dQR = np.zeros((n_rel, d))
    dKR = np.zeros((n_rel, d))
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    if flags & C2P:
        # G[i, r] = sum of dS_ij over the keys j with T(i - j) = r
        idx = T[i - j + (rel_max_len - 1)]
        G = np.zeros((L, n_rel))
        np.add.at(G, (np.broadcast_to(i, (L, L)), idx), dS)
        dQ += tau * (G @ KRh)
        dKR += tau * (G.T @ Qh)
    if flags & P2C:
        # Hm[j, r] = sum of dS_ij over the queries i with T(j - i) = r
        idx = T[j - i + (rel_max_len - 1)]
        Hm = np.zeros((L, n_rel))
        np.add.at(Hm, (np.broadcast_to(j, (L, L)), idx), dS)
        dK += tau * (Hm @ QRh)
        dQR += tau * (Hm.T @ Kh)
    return dQ, dK, dV, dQR, dKR, lse


def _grads(shape_tokens, H, d, n_rel):
    z = lambda *s: np.zeros(s, dtype=np.float64)
    return {"dq": z(*shape_tokens, H * d), "dk": z(*shape_tokens, H * d),
            "dv": z(*shape_tokens, H * d), "dqr": z(n_rel, H * d), "dkr": z(n_rel, H * d),
            "lse": z(*shape_tokens, H)}


def dattn_padded_bwd(q, k, v, qr, kr, rel_idx, rel_max_len: int, mask, H: int, d: int,
                     dout, flags: int = 3, scale: float = 0.0) -> dict:
    """Padded layout: q, k, v, dout [B, L, H*d]; mask [B, L] or None.
    Returns float64 arrays dq, dk, dv [B, L, H*d], dqr, dkr [n_rel, H*d] and
    lse [B, L, H]."""
    B, L, _ = q.shape
    n_rel = qr.shape[0]
    T = _check_table(rel_idx, rel_max_len, L, n_rel)
    tau = scale if scale > 0 else default_scale(d, flags)
    g = _grads((B, L), H, d, n_rel)
    for b in range(B):
        valid = None if mask is None else mask[b]
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            dQ, dK, dV, dQR, dKR, lse = unit_backward(
                _head(q[b], h, d), _head(k[b], h, d), _head(v[b], h, d), _head(qr, h, d),
                _head(kr, h, d), T, rel_max_len, valid, flags, tau, _head(dout[b], h, d))
            g["dq"][b, :, sl] = dQ
            g["dk"][b, :, sl] = dK
            g["dv"][b, :, sl] = dV
            g["dqr"][:, sl] += dQR
            g["dkr"][:, sl] += dKR
            g["lse"][b, :, h] = lse
    return g


def dattn_varlen_bwd(q, k, v, qr, kr, rel_idx, rel_max_len: int, cu_seqlens, H: int, d: int,
                     dout, flags: int = 3, scale: float = 0.0) -> dict:
    """Packed layout: q, k, v, dout [total_tokens, H*d]; every token valid.
    Returns dq, dk, dv [total_tokens, H*d], dqr, dkr [n_rel, H*d] and lse
    [total_tokens, H]."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n_rel = qr.shape[0]
    max_len = int(np.max(np.diff(cu))) if len(cu) > 1 else 0
    T = _check_table(rel_idx, rel_max_len, max_len, n_rel)
    tau = scale if scale > 0 else default_scale(d, flags)
    g = _grads((q.shape[0],), H, d, n_rel)
    for b in range(len(cu) - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi <= lo:
            continue
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            dQ, dK, dV, dQR, dKR, lse = unit_backward(
                _head(q[lo:hi], h, d), _head(k[lo:hi], h, d), _head(v[lo:hi], h, d),
                _head(qr, h, d), _head(kr, h, d), T, rel_max_len, None, flags, tau,
                _head(dout[lo:hi], h, d))
            g["dq"][lo:hi, sl] = dQ
            g["dk"][lo:hi, sl] = dK
            g["dv"][lo:hi, sl] = dV
            g["dqr"][:, sl] += dQR
            g["dkr"][:, sl] += dKR
            g["lse"][lo:hi, h] = lse
    return g


def lse_rows(q_seq, k_seq, qr, kr, rel_idx, rel_max_len: int, h: int, d: int, rows,
             valid=None, flags: int = 3, scale: float = 0.0) -> np.ndarray:
    """Row log-sum-exp (natural log) of selected rows of one (sequence,
    head) unit, -inf for rows with no valid key or a padded query; for
    checking sampled rows where the whole unit is too slow."""
    L = k_seq.shape[0]
    T = _check_table(rel_idx, rel_max_len, L, qr.shape[0])
    tau = scale if scale > 0 else default_scale(d, flags)
    rows = np.asarray(rows, dtype=np.int64)
    S = unit_scores(_head(q_seq, h, d), _head(k_seq, h, d), _head(qr, h, d), _head(kr, h, d),
                    T, rel_max_len, flags, tau, rows)
    keys = np.ones(L, dtype=bool) if valid is None else np.asarray(valid).astype(bool)
    out = np.full(len(rows), -np.inf)
    if keys.any():
        Sv = S[:, keys]
        mx = Sv.max(axis=1)
        out = mx + np.log(np.exp(Sv - mx[:, None]).sum(axis=1))
        if valid is not None:
            out = np.where(keys[rows], out, -np.inf)
    return out
