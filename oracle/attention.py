"""Disentangled-attention forward, plain float64 on the CPU.

TEST INFRASTRUCTURE: only tests, the smoke entry and the benchmark's CPU
baseline may import this module. The product path never does.

What it computes. DisentangledFlash (README, "Status"; kernels-community
discussion #31, "Motivation") computes exact bidirectional DeBERTa-v2/v3
attention: the content-to-content score plus content-to-position (C2P) and
position-to-content (P2C) terms, evaluated without an approximation and
without materialising [B, H, L, L] on the GPU. This oracle does materialise
the score matrix, one (sequence, head) unit at a time:

    S_ij = tau * ( q_i . k_j
                   + [C2P] q_i . kr[T(i - j)]
                   + [P2C] k_j . qr[T(j - i)] )
    tau  = 1 / sqrt(d * (1 + number of position terms enabled)) by default
    A    = softmax over the valid keys of row i (exact exclusion of the
           others), O_i = sum_j A_ij v_j

T is the relative-row table (oracle.bucket.rel_index_table), indexed by the
signed distance; qr and kr are the per-head projections of the relative
embedding table, [n_rel, H*d]. The pages print none of these formulas; they
are the DeBERTa-v2/v3 definitions the README's "Attribution" section points
to, with the readings listed beside the build's design notes.

Masks (README "Status": factorised 2-D padding masks). A [B, L] valid vector
m gives the 2-D mask m_i * m_j: a valid query row takes its softmax over the
valid keys only; a row with m_i = 0 has every weight zero, so its output is
zero. Positions are the padded-row indices.

Packed layout (README, "Packed unpadded inference"; fold-attention README,
packed self-attention with int32 cumulative lengths): sequence b occupies
rows cu[b] .. cu[b+1]-1 of a [total_tokens, H*d] array and its positions
restart at zero. Packed and padded are the same mathematics (discussion #31:
same kernel, same math, different layout).

Everything is computed in float64 from the working-dtype values (which the
callers pass already rounded, as float32 or float64 arrays).
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

C2P = 1
P2C = 2


def default_scale(d: int, flags: int) -> float:
    """tau = 1/sqrt(d * (1 + #position terms)): DeBERTa's scale factor,
    which is 1/sqrt(d) (standard attention) when both terms are off."""
    n_terms = (1 if flags & C2P else 0) + (1 if flags & P2C else 0)
    return 1.0 / math.sqrt(d * (1 + n_terms))


def _head(x: np.ndarray, h: int, d: int) -> np.ndarray:
    return np.asarray(x[..., h * d:(h + 1) * d], dtype=np.float64)


def unit_scores(Qh: np.ndarray, Kh: np.ndarray, QRh: np.ndarray, KRh: np.ndarray,
                T: np.ndarray, rel_max_len: int, flags: int, tau: float,
                rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Scaled score matrix S (float64) of one (sequence, head) unit.

    Qh, Kh: [L, d]; QRh, KRh: [n_rel, d]; T: relative-row table for
    distances -(rel_max_len-1) .. rel_max_len-1. `rows` restricts the
    result to those query rows (same definition, fewer rows).
    """
    L = Kh.shape[0]
    qi = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    kj = np.arange(L)
    Qs = Qh[qi]
    S = Qs @ Kh.T                                           # content-to-content
    if flags & C2P:
        # C2P: row i, column j uses kr at the row for distance i - j
        c2p_all = Qs @ KRh.T                                # [rows, n_rel]
        idx = T[qi[:, None] - kj[None, :] + (rel_max_len - 1)]
        S = S + np.take_along_axis(c2p_all, idx, axis=1)
    if flags & P2C:
        # P2C: row i, column j uses qr at the row for distance j - i,
        # multiplied with the key k_j
        p2c_all = Kh @ QRh.T                                # [L keys, n_rel]
        idx = T[kj[None, :] - qi[:, None] + (rel_max_len - 1)]
        S = S + p2c_all[kj[None, :], idx]
    return S * tau


def masked_softmax_apply(S: np.ndarray, Vh: np.ndarray, row_valid: np.ndarray,
                         key_valid: np.ndarray) -> np.ndarray:
    """O = softmax(S restricted to valid keys) V for valid rows; 0 otherwise."""
    out = np.zeros((S.shape[0], Vh.shape[1]), dtype=np.float64)
    keys = np.nonzero(key_valid)[0]
    rows = np.nonzero(row_valid)[0]
    if len(keys) == 0 or len(rows) == 0:
        return out
    Sv = S[np.ix_(rows, keys)]
    Sv = Sv - Sv.max(axis=1, keepdims=True)
    E = np.exp(Sv)
    A = E / E.sum(axis=1, keepdims=True)
    out[rows] = A @ Vh[keys]
    return out


def unit_forward(Qh, Kh, Vh, QRh, KRh, T, rel_max_len, valid, flags, tau,
                 rows=None) -> np.ndarray:
    """Output rows of one (sequence, head) unit; `valid` is the [L] mask."""
    L = Kh.shape[0]
    valid = np.ones(L, dtype=bool) if valid is None else np.asarray(valid).astype(bool)
    S = unit_scores(Qh, Kh, QRh, KRh, T, rel_max_len, flags, tau, rows)
    row_ids = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    return masked_softmax_apply(S, Vh, valid[row_ids], valid)


def _check_table(T: np.ndarray, rel_max_len: int, L: int, n_rel: int,
                 clamp_rows: bool = False) -> np.ndarray:
    """The relative-row table as int64. Rows outside [0, n_rel) are an error,
    or, with clamp_rows, read as the nearest edge row (the library's
    contract for such tables: a row index below 0 reads row 0, one at or
    above n_rel reads row n_rel - 1)."""
    T = np.asarray(T, dtype=np.int64)
    if rel_max_len < L:
        raise ValueError("rel_max_len must cover the sequence length")
    if T.shape[0] != 2 * rel_max_len - 1:
        raise ValueError("table must have 2*rel_max_len-1 entries")
    if clamp_rows:
        return np.clip(T, 0, n_rel - 1)
    if T.min(initial=0) < 0 or T.max(initial=0) >= n_rel:
        raise ValueError("table rows outside the relative tables")
    return T


def dattn_padded(q, k, v, qr, kr, rel_idx, rel_max_len: int, mask, H: int, d: int,
                 flags: int = 3, scale: float = 0.0, clamp_rows: bool = False) -> np.ndarray:
    """Padded layout. q, k, v: [B, L, H*d]; qr, kr: [n_rel, H*d]; mask:
    [B, L] (1 = valid) or None. Returns float64 [B, L, H*d]. clamp_rows:
    see _check_table."""
    B, L, _ = q.shape
    T = _check_table(rel_idx, rel_max_len, L, qr.shape[0], clamp_rows)
    tau = scale if scale > 0 else default_scale(d, flags)
    out = np.zeros((B, L, H * d), dtype=np.float64)
    for b in range(B):
        valid = None if mask is None else mask[b]
        for h in range(H):
            out[b, :, h * d:(h + 1) * d] = unit_forward(
                _head(q[b], h, d), _head(k[b], h, d), _head(v[b], h, d),
                _head(qr, h, d), _head(kr, h, d), T, rel_max_len, valid, flags, tau)
    return out


def dattn_varlen(q, k, v, qr, kr, rel_idx, rel_max_len: int, cu_seqlens, H: int,
                 d: int, flags: int = 3, scale: float = 0.0,
                 clamp_rows: bool = False) -> np.ndarray:
    """Packed layout. q, k, v: [total_tokens, H*d]; cu_seqlens: [nseq+1].
    Each sequence is one padded row of its own length with every token
    valid. Returns float64 [total_tokens, H*d]."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    max_len = int(np.max(np.diff(cu))) if len(cu) > 1 else 0
    T = _check_table(rel_idx, rel_max_len, max_len, qr.shape[0], clamp_rows)
    tau = scale if scale > 0 else default_scale(d, flags)
    out = np.zeros((q.shape[0], H * d), dtype=np.float64)
    for b in range(len(cu) - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        if hi <= lo:
            continue
        for h in range(H):
            out[lo:hi, h * d:(h + 1) * d] = unit_forward(
                _head(q[lo:hi], h, d), _head(k[lo:hi], h, d), _head(v[lo:hi], h, d),
                _head(qr, h, d), _head(kr, h, d), T, rel_max_len, None, flags, tau)
    return out


def dattn_rows(q_seq, k_seq, v_seq, qr, kr, rel_idx, rel_max_len: int, h: int,
               d: int, rows: Sequence[int], valid=None, flags: int = 3,
               scale: float = 0.0) -> np.ndarray:
    """Selected output rows of one (sequence, head) unit, for checking
    sampled outputs at sizes where the whole unit is too slow.
    q_seq, k_seq, v_seq: [L, H*d] of one sequence. Returns [len(rows), d]."""
    L = k_seq.shape[0]
    T = _check_table(rel_idx, rel_max_len, L, qr.shape[0])
    tau = scale if scale > 0 else default_scale(d, flags)
    return unit_forward(_head(q_seq, h, d), _head(k_seq, h, d), _head(v_seq, h, d),
                        _head(qr, h, d), _head(kr, h, d), T, rel_max_len, valid,
                        flags, tau, rows=np.asarray(rows, dtype=np.int64))
